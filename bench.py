"""Benchmark of the compressed decode-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-table] [--no-cpu-baseline] [--reps R] [--copy-probe MiB]

One step = one decode step of one layer: quantize-append of the new token for
every (batch, KV head), fused split-K decode attention over the whole
compressed cache, split merge with the single inverse rotation.  The layer
caches are held as R distinct replicas (R * cache bytes >= 1 GiB, four times
the 256 MB Infinity Cache; at most 64 replicas, so the 135 KB single-head
cache stays cache-resident) and step i uses replica i mod R, as consecutive
layers of a model would, so every step reads its cache from HBM.

The headline workload (default two_tier: batch 16, 16 heads, d 128, context
16384, fp16 near tier of 10% plus fp8 keys / 4-bit values: 947 MB, the largest
configuration) gives `value` (algorithmic bytes of a step / step time) and
`roofline` (the attention kernel alone: algorithmic bytes / its average launch
duration).  `configs` carries the same measurements for every configuration
(single_head_fp32, llama7b_layer, long_context, bitwidth_sweep at 2, 3 and 4
bits, decode_buffer, two_tier), so one run times them all.

Timing: every timed region is a replay of a captured HIP graph between one
pair of HIP events on the launch stream (no host launch overhead inside), R
timed replays after one untimed one; reported as the mean over all launches
and the median of the per-replay means.  Inputs are drawn on the device
(workloads.generate_device: the seeded recipe of the parity inputs) and are
resident in HBM before any timed region.  cpu_baseline = the CPU oracle on a
bounded sample of the headline workload, on this host's cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "packed-KV decode-attention HBM GB/s (% of peak) + quantize-append tokens/s"
TABLE = ("single_head_fp32", "llama7b_layer", "long_context", "bitwidth_sweep@b2", "bitwidth_sweep@b3",
         "bitwidth_sweep@b4", "decode_buffer", "two_tier")
MAX_REPLICAS = 64
# key side streams measured beside the table (llama7b_layer shapes): the
# outlier stream beside 4-bit codes, and the QJL sketch beside 3-bit keys
# (the page's 68-byte key) and 4-bit values
SIDE_TABLE = (("llama7b_layer+outliers", dict(outliers=8), 4), ("llama7b_layer@k3+qjl", dict(qjl=True), 3))


def cache_bytes(wl: W.Workload, outliers: int = 0, qjl: bool = False) -> dict:
    """Algorithmic bytes of the decode read and of one appended token (a key
    outlier stream adds its int8 codes and fp32 scale per token, a QJL sketch
    its d/8 sign bytes and fp16 residual norm)."""
    d = wl.head_dim
    kb = wl.k_bits
    krow = d * kb // 8
    vrow = d * wl.v_bits // 8
    pairs = wl.batch * wl.kv_heads
    far = wl.far_len
    knorm = 0 if kb == 8 else 2
    per_tok = krow + knorm + vrow + 2 + (outliers + 4 if outliers else 0) + (d // 8 + 2 if qjl else 0)
    near = wl.near_len * 2 * d * 2
    qb = wl.batch * wl.q_heads * d * (4 if wl.dtype == "f32" else 2)
    ob = wl.batch * wl.q_heads * d * 4
    in_b = 4 if wl.dtype == "f32" else 2
    append_tok = pairs * (2 * d * in_b + per_tok)
    return {"cache": pairs * (far * per_tok + near), "q": qb, "out": ob, "append_token": append_tok,
            "per_token_head": per_tok}


def workload(name: str) -> W.Workload:
    base, _, bits = name.partition("@b")
    wl = W.WORKLOADS[base]
    return wl.with_bits(int(bits)) if bits else wl


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="decode steps per timed graph replay")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=5, help="timed replays per measurement (median reported)")
    ap.add_argument("--workload", default="two_tier", choices=sorted(W.WORKLOADS) + [t for t in TABLE if "@" in t])
    ap.add_argument("--bits", type=int, default=None, help="override code bits (bitwidth_sweep)")
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--near-splits", type=int, default=None, help="near-tier splits (caches with a near tier)")
    ap.add_argument("--no-table", action="store_true", help="measure the headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gate", action="store_true",
                    help="score-gated attention with spike flags (kvq_decode_attention_gated): gate reference "
                         "= the query's own log-sum-exp from an ungated pass, spike threshold 4 below it")
    ap.add_argument("--outliers", type=int, default=0, choices=(0, 8),
                    help="key outlier stream with this many channels, calibrated on the first 256 tokens")
    ap.add_argument("--qjl", action="store_true",
                    help="QJL residual sketch on the keys (m = head_dim rows of a seeded Gaussian projection)")
    ap.add_argument("--k-bits", type=int, default=None, choices=(2, 3, 4),
                    help="override the key code bits only (e.g. 3 with --qjl: 3-bit codes plus the 1-bit sketch)")
    ap.add_argument("--query-scale", type=float, default=1.0,
                    help="multiply the decode query (a larger scale gives a more peaked softmax)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (HBM counter calibration)")
    return ap.parse_args(argv)


def copy_rate(mib: int = 1024, reps: int = 5) -> dict:
    """Achievable HBM rate on this machine: a plain device-to-device copy of
    `mib` MiB (torch's blit kernel), median of `reps` timed copies, as bytes
    read plus bytes written per second."""
    import torch
    n = mib * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    t = float(np.median(ts))
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_read": n, "bytes_written": n, "us": round(t * 1e6, 1), "GBps": round(2 * n / t / 1e9, 1)}


def copy_probe(mib: int):
    import torch
    n = mib * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}))


KERNEL_SOURCES = {
    "attend_pair_kernel": ("kvq_attend_pair.hip", "kvq_pair.h"),
    "attend_wide_kernel": ("kvq_attend_wide.hip", "kvq_pair.h"),
    "attend_mfma_kernel": ("kvq_attend_mfma.hip",),
    "attend_kernel": ("kvq_attend.hip",),
}


def kernel_source_sha(kernel: str = "attend_pair_kernel") -> str:
    """Hash of the sources a traffic figure depends on: the kernel's own
    files (for a two-launch name, both kernels') and the headers every
    attention kernel includes, so a figure taken on other code is not reused."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "compressed_decode_attention_randomized_amd", "csrc")
    files = []
    for k in kernel.split("+"):
        files += [f for f in KERNEL_SOURCES.get(k, ()) if f not in files]
    for name in files + ["kvq_lane.h", "kvq_internal.h"]:
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def read_traffic(workload: str, kernel_sha: str):
    """HBM bytes per attention launch from the committed counter summary, or
    None if it is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload.replace('@', '_').replace('+', '_')}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_sha:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _graph_time(fn, n_calls: int, reps: int):
    """Capture n_calls calls of fn(i) as one HIP graph; replay it once
    untimed, then `reps` times between event pairs on the current stream.
    Returns the per-call times (ms) of each replay."""
    import torch
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_calls):
            fn(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / n_calls)
    del graph
    return out


def _stats_us(per_call_ms):
    a = np.asarray(per_call_ms) * 1e3
    return {"avg_us": round(float(a.mean()), 3), "median_us": round(float(np.median(a)), 3),
            "min_us": round(float(a.min()), 3), "max_us": round(float(a.max()), 3)}


ARITH = {
    "attend_pair_kernel": "fp16 hi/lo operand pairs on v_mfma_f32_16x16x32_f16, fp32 accumulation",
    "attend_wide_kernel": "fp16 hi/lo operand pairs on v_mfma_f32_16x16x32_f16, fp32 accumulation",
    "attend_mfma_kernel": "fp16 hi/lo operand pairs on v_mfma_f32_16x16x32_f16, fp32 accumulation",
    "attend_kernel": "fp32 VALU FMAs (fp8 keys converted to fp32 in hardware), fp32 accumulation",
}


def measure(wl: W.Workload, args, dev, steps: int, reps: int, want_inputs: bool = False) -> dict:
    """Decode step, attention alone, bulk append and one-token append for one
    workload (see the module docstring)."""
    import torch
    import compressed_decode_attention_randomized_amd as kvq

    by = cache_bytes(wl, args.outliers, args.qjl)
    inp = W.generate_device(wl, dev)
    if wl.near_fraction:
        kn, vn = inp.tier("near")
        kf, vf = inp.tier("far")
        near_splits = wl.near_split_count
    else:
        kf, vf, kn, vn, near_splits = inp.k, inp.v, None, None, 0
    T = kf.shape[2]
    fmt = {2: kvq.KVQ_LM2, 3: kvq.KVQ_LM3, 4: kvq.KVQ_LM4, 8: kvq.KVQ_FP8_E4M3}
    q_dev = inp.q
    if args.query_scale != 1.0:
        q_dev = (q_dev.float() * args.query_scale).to(q_dev.dtype)
    R = min(MAX_REPLICAS, max(1, math.ceil((1 << 30) / by["cache"])))
    proj_t = None
    if args.qjl:
        proj_t = torch.from_numpy(np.ascontiguousarray(W.qjl_projection(wl.head_dim).T)).to(dev)
    caches = []
    for r in range(R):
        c = kvq.KVCache.allocate(wl.batch, wl.kv_heads, wl.head_dim, T, fmt[wl.k_bits], fmt[wl.v_bits],
                                 seed=W.SIGN_SEED, device=dev,
                                 near_k=None if kn is None else (kn if r == 0 else kn.clone()),
                                 near_v=None if vn is None else (vn if r == 0 else vn.clone()),
                                 outliers=args.outliers, qjl_proj_t=proj_t)
        if args.outliers:
            c.calibrate(kf[:, :, :min(256, T)].contiguous())
        caches.append(c)
    stream = torch.cuda.current_stream()

    # ---- bulk quantize-append of the whole context into every replica ----
    for c in caches[:2]:
        c.append(kf, vf, 0)
    torch.cuda.synchronize()
    app = []
    for _ in range(max(1, min(reps, 3))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for c in caches:
            c.append(kf, vf, 0)
        e1.record(stream)
        torch.cuda.synchronize()
        app.append(e0.elapsed_time(e1) / R)
    append_ms = float(np.median(app))
    append_bytes = wl.batch * wl.kv_heads * T * (2 * wl.head_dim * (4 if wl.dtype == "f32" else 2)
                                                + by["per_token_head"])

    # ---- decode steps ----
    k_new, v_new = kf[:, :, -1:].contiguous(), vf[:, :, -1:].contiguous()
    S = wl.splits
    bufs = [c.partial_buffers(wl.q_heads, S, near_splits) for c in caches[:2]]
    out = torch.empty((wl.batch, wl.q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    gate_kw = {}
    if args.gate:
        # the references a decode loop would carry over from its previous step
        lse = torch.empty((wl.batch, wl.q_heads), dtype=torch.float32, device=dev)
        caches[0].decode(q_dev, T, S, near_splits, lse=lse)
        gate_kw = {"gate_ref": lse, "spike_ref": lse - 4.0,
                   "spike_bits": torch.zeros((wl.batch, wl.q_heads, (T + 31) // 32), dtype=torch.int32, device=dev)}

    def attend(i):
        c = caches[i % R]
        po, pml = bufs[i % 2]
        c.attend(q_dev, T, S, near_splits, po, pml, **gate_kw)

    def step(i):
        c = caches[i % R]
        po, pml = bufs[i % 2]
        c.append(k_new, v_new, T - 1)
        if args.gate:
            gate_kw["spike_bits"].zero_()
        c.attend(q_dev, T, S, near_splits, po, pml, **gate_kw)
        c.merge(po, pml, S, near_splits, out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    step_ms = _graph_time(step, steps, reps)
    att_ms = _graph_time(attend, steps, reps)
    app1_ms = _graph_time(lambda i: caches[i % R].append(k_new, v_new, T - 1), steps, reps)

    att_bytes = by["cache"] + by["q"] + by["out"]
    step_bytes = att_bytes + by["append_token"]
    att = _stats_us(att_ms)
    st = _stats_us(step_ms)
    kernel = "attend_kernel" if args.gate else caches[0].attention_kernel(wl.q_heads, S, near_splits)
    achieved = att_bytes / (att["avg_us"] / 1e6) / 1e9
    traffic = read_traffic(wl.name, kernel_source_sha(kernel))
    res = {
        "workload": wl.name, "kernel": kernel, "arith": ARITH.get(kernel.split("+")[0], ""),
        "batch": wl.batch, "q_heads": wl.q_heads, "kv_heads": wl.kv_heads, "head_dim": wl.head_dim,
        "seq_len": wl.seq_len, "k_bits": wl.k_bits, "v_bits": wl.v_bits, "near_len": wl.near_len,
        "splits": S, "near_splits": near_splits, "layer_replicas": R,
        "attn_bytes_per_launch": att_bytes, "attn": att,
        "attn_GBps": round(achieved, 1), "attn_frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic_bytes_per_launch": traffic,
        "traffic_ratio": None if traffic is None else round(traffic / att_bytes, 4),
        "step_bytes": step_bytes, "step": st,
        "step_GBps": round(step_bytes / (st["avg_us"] / 1e6) / 1e9, 1),
        "append_tokens_per_s": round(wl.batch * T / (append_ms / 1e3), 1),
        "append_GBps": round(append_bytes / (append_ms / 1e3) / 1e9, 1),
        "append_frac": round(append_bytes / (append_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "append_us": round(append_ms * 1e3, 2),
        "append_step_us": _stats_us(app1_ms)["avg_us"],
    }
    if args.gate:
        # a gated launch skips the value rows of gated tokens: its rate is
        # quoted against the ungated algorithmic bytes (an effective rate)
        res["bytes_basis"] = "ungated"
    if want_inputs:
        res["_inputs"] = (inp, kf, vf, kn, vn)
    del caches, bufs
    return res


def cpu_baseline(wl: W.Workload, inputs, seconds: float = 12.0) -> dict:
    """The oracle as it stands on a bounded sample: (b, KV head) pairs of the
    same workload (their rows copied from the device inputs), taken one at a
    time until `seconds` of work have run.  Quantize-append of the pair's T
    tokens (keys and values) and decode attention of its G query heads are
    timed separately."""
    from threadpoolctl import threadpool_info
    from oracle import kvq_oracle as O
    inp, kf_d, vf_d, kn_d, vn_d = inputs
    d, G = wl.head_dim, wl.group
    s = O.rademacher_signs(W.SIGN_SEED, d)
    O.codebook(wl.v_bits, d)
    if wl.k_bits != 8:
        O.codebook(wl.k_bits, d)
    pairs = [(b, h) for b in range(wl.batch) for h in range(wl.kv_heads)]
    rng = np.random.default_rng(0)
    rng.shuffle(pairs)
    by = cache_bytes(wl)
    t_quant = t_att = 0.0
    n_pairs = 0
    att_times = []
    for b, h in pairs:
        kf, vf = kf_d[b, h].cpu().numpy(), vf_d[b, h].cpu().numpy()
        if kn_d is not None:
            kn, vn = kn_d[b, h].cpu().numpy(), vn_d[b, h].cpu().numpy()
        q = inp.q[b:b + 1, h * G:(h + 1) * G].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        if wl.k_bits == 8:
            kc, _ = O.quantize_fp8(kf, s)
            kn16 = None
        else:
            kc, kn16, _ = O.quantize_lm(kf, s, wl.k_bits)
        vc, vn16, _ = O.quantize_lm(vf, s, wl.v_bits)
        kp = kc if wl.k_bits == 8 else O.pack(kc, wl.k_bits)
        vp = O.pack(vc, wl.v_bits)
        t1 = time.perf_counter()
        k_rot = O.e4m3_decode(kp) if wl.k_bits == 8 else O.dequantize_lm(O.unpack(kp, wl.k_bits, d), kn16, wl.k_bits)
        v_rot = O.dequantize_lm(O.unpack(vp, wl.v_bits, d), vn16, wl.v_bits)
        if kn_d is not None:
            O.two_tier_attention(q, kn[None, None].astype(np.float64), vn[None, None].astype(np.float64),
                                 k_rot[None, None], v_rot[None, None], s)
        else:
            O.attention(q, k_rot[None, None], v_rot[None, None], s)
        t2 = time.perf_counter()
        t_quant += t1 - t0
        t_att += t2 - t1
        att_times.append(t2 - t1)
        n_pairs += 1
        if t_quant + t_att >= seconds:
            break
    pair_bytes = by["cache"] / (wl.batch * wl.kv_heads)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    cpu_model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": round(n_pairs * pair_bytes / t_att / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "cpu_model": cpu_model,
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{n_pairs} of {wl.batch * wl.kv_heads} (batch, kv-head) pairs of {wl.name}: "
                  f"oracle dequantize+attention over {wl.seq_len} tokens x {G} query heads each "
                  f"(value), oracle quantize of the same pairs' keys and values (append_tokens_per_s)",
        "append_tokens_per_s": round(n_pairs * wl.seq_len / t_quant, 2),
        "seconds": round(t_quant + t_att, 2),
        # each pair is one repetition of the same work; the first warms up
        "pair_median_value": round(pair_bytes / float(np.median(att_times[1:] or att_times)) / 1e9, 4),
        "pair_reps": len(att_times[1:] or att_times),
    }


def main(argv=None) -> int:
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: libkvq has no multi-GPU path "
              f"(requested --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        return 2
    import torch
    import compressed_decode_attention_randomized_amd as kvq

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return 0
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    kvq.load()
    dev = torch.device("cuda")
    wl = workload(args.workload)
    if args.bits:
        wl = wl.with_bits(args.bits)
    if args.k_bits:
        wl = dataclasses.replace(wl, k_bits=args.k_bits, name=f"{wl.name.split('@')[0]}@k{args.k_bits}")
    if args.splits:
        wl = wl.scaled(splits=args.splits)
    if args.near_splits:
        wl = wl.scaled(near_splits=args.near_splits)
    if args.qjl and wl.k_bits == 8:
        print("--qjl needs Lloyd-Max keys", file=sys.stderr)
        return 2
    if args.outliers or args.qjl:
        wl = dataclasses.replace(wl, name=wl.name + ("+outliers" if args.outliers else "") + ("+qjl" if args.qjl else ""))
    variant = args.gate or args.outliers or args.qjl or args.k_bits or args.query_scale != 1.0
    table = []
    if not args.no_table and not variant:
        plain = argparse.Namespace(**{**vars(args), "gate": False, "outliers": 0, "qjl": False,
                                      "query_scale": 1.0})
        for name in TABLE:
            if name == wl.name:
                continue
            print(f"# table: {name}", file=sys.stderr, flush=True)
            r = measure(workload(name), plain, dev, steps=min(args.steps, 100), reps=args.reps)
            table.append(r)
            torch.cuda.empty_cache()
        for label, kw, kbits in SIDE_TABLE:
            print(f"# table: {label}", file=sys.stderr, flush=True)
            side = argparse.Namespace(**{**vars(plain), **kw})
            base = workload("llama7b_layer")
            swl = dataclasses.replace(base, k_bits=kbits, name=label)
            r = measure(swl, side, dev, steps=min(args.steps, 100), reps=args.reps)
            r["workload"] = label
            table.append(r)
            torch.cuda.empty_cache()
    print(f"# headline: {wl.name}: cache {cache_bytes(wl, args.outliers, args.qjl)['cache'] / 1e6:.1f} MB",
          file=sys.stderr, flush=True)
    head = measure(wl, args, dev, steps=args.steps, reps=args.reps, want_inputs=not args.no_cpu_baseline)
    inputs = head.pop("_inputs", None)
    table.append({k: v for k, v in head.items()})
    table.sort(key=lambda r: TABLE.index(r["workload"]) if r["workload"] in TABLE else len(TABLE))
    att = head["attn"]
    result = {
        "metric": METRIC,
        "value": head["step_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step"]["avg_us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if head["kernel"].split("+")[0] == "attend_kernel" else "f16x2-f32acc",
        "arith": head["arith"],
        "data": "synthetic (seeded device draws of the workload recipe)",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.q_heads, "kv_heads": wl.kv_heads,
                   "head_dim": wl.head_dim, "seq_len": wl.seq_len, "k_bits": wl.k_bits, "v_bits": wl.v_bits,
                   "near_len": wl.near_len, "splits": head["splits"], "near_splits": head["near_splits"],
                   "layer_replicas": head["layer_replicas"], "launch": "hip_graph", "reps": args.reps,
                   "gated": bool(args.gate), "query_scale": args.query_scale, "outliers": args.outliers,
                   "qjl": bool(args.qjl), "step_bytes": head["step_bytes"]},
        "step_median_us": head["step"]["median_us"],
        "pct_of_hbm_peak": round(100 * head["step_GBps"] / HBM_PEAK_GBS, 2),
        "append_tokens_per_s": head["append_tokens_per_s"],
        "append_GBps": head["append_GBps"],
        "append_step_us": head["append_step_us"],
        "roofline": {"bound": "hbm", "achieved": head["attn_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["attn_frac"], "traffic": head["traffic_bytes_per_launch"],
                     "kernel": head["kernel"], "bytes_per_launch": head["attn_bytes_per_launch"],
                     "avg_us": att["avg_us"], "median_us": att["median_us"], "min_us": att["min_us"],
                     "max_us": att["max_us"]},
        "configs": table,
        "copy_probe": copy_rate(),
    }
    if args.gate:
        result["roofline"]["bytes_basis"] = "ungated"
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inputs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
