"""Benchmark of the compressed decode-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--copy-probe MiB]

One step = one decode step of one layer: quantize-append of the new token for
every (batch, KV head), fused split-K decode attention over the whole
compressed cache, split merge with the single inverse rotation.  The layer
caches are held as R distinct replicas (R * cache bytes >= 1 GiB, four times
the 256 MB Infinity Cache) and step i uses replica i mod R, as consecutive
layers of a model would, so every step reads its cache from HBM.

Printed: one JSON line.  value = algorithmic bytes of a step (packed codes and
norms of the whole cache, the query, the output, the new token in and its
codes out) / measured step time.  roofline = the attention kernel alone:
algorithmic bytes / its average launch duration, from HIP events on the stream
it runs on around a run of back-to-back launches (per-launch event pairs,
which add their own overhead, are reported beside it).  cpu_baseline = the CPU oracle on a bounded sample of the same
workload, on this host's cores.
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


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b_layer", choices=sorted(W.WORKLOADS))
    ap.add_argument("--bits", type=int, default=None, help="override code bits (bitwidth_sweep)")
    ap.add_argument("--splits", type=int, default=None)
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


def read_traffic(workload: str, kernel_sha: str):
    """HBM bytes per attention launch from the committed counter summary, or
    None if it is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload.replace('@', '_')}_hbm_traffic.txt")
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


KERNEL_SOURCES = {
    "attend_pair_kernel": ("kvq_attend_pair.hip", "kvq_pair.h"),
    "attend_wide_kernel": ("kvq_attend_wide.hip", "kvq_pair.h"),
    "attend_mfma_kernel": ("kvq_attend_mfma.hip",),
    "attend_kernel": ("kvq_attend.hip",),
}


def kernel_source_sha(kernel: str = "attend_pair_kernel") -> str:
    """Hash of the sources a traffic figure depends on: the kernel's own file
    and the headers every attention kernel includes, so a figure taken on
    other code is not reused."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "compressed_decode_attention_randomized_amd", "csrc")
    for name in KERNEL_SOURCES.get(kernel, ()) + ("kvq_lane.h", "kvq_internal.h"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def cpu_baseline(wl: W.Workload, inp: W.Inputs, seconds: float = 12.0) -> dict:
    """The oracle as it stands on a bounded sample: (b, KV head) pairs of the
    same workload, taken one at a time until `seconds` of decode work have
    run.  Quantize-append of the pair's T tokens (keys and values) and decode
    attention of its G query heads are timed separately."""
    from threadpoolctl import threadpool_info
    from oracle import kvq_oracle as O
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
    for b, h in pairs:
        if wl.near_fraction:
            idx_n, idx_f = inp.near_idx[b, h], inp.far_idx[b, h]
            kn, vn = inp.k[b, h, idx_n], inp.v[b, h, idx_n]
            kf, vf = inp.k[b, h, idx_f], inp.v[b, h, idx_f]
        else:
            kf, vf = inp.k[b, h], inp.v[b, h]
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
        q = inp.q[b:b + 1, h * G:(h + 1) * G].astype(np.float64)
        if wl.near_fraction:
            O.two_tier_attention(q, kn[None, None].astype(np.float64), vn[None, None].astype(np.float64),
                                 k_rot[None, None], v_rot[None, None], s)
        else:
            O.attention(q, k_rot[None, None], v_rot[None, None], s)
        t2 = time.perf_counter()
        t_quant += t1 - t0
        t_att += t2 - t1
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
    wl = W.WORKLOADS[args.workload]
    if args.bits:
        wl = wl.with_bits(args.bits)
    if args.k_bits:
        wl = dataclasses.replace(wl, k_bits=args.k_bits, name=f"{wl.name.split('@')[0]}@k{args.k_bits}")
    if args.splits:
        wl = wl.scaled(splits=args.splits)
    if args.qjl and wl.k_bits == 8:
        print("--qjl needs Lloyd-Max keys", file=sys.stderr)
        return 2
    dev = torch.device("cuda")
    by = cache_bytes(wl, args.outliers, args.qjl)
    print(f"# workload {wl.name}: cache {by['cache'] / 1e6:.1f} MB", file=sys.stderr, flush=True)

    inp = W.generate(wl)
    if wl.near_fraction:
        kn, vn = inp.tier("near")
        kf, vf = inp.tier("far")
        near_splits = wl.near_split_count
    else:
        kf, vf, kn, vn, near_splits = inp.k, inp.v, None, None, 0
    T = kf.shape[2]
    fmt = {2: kvq.KVQ_LM2, 3: kvq.KVQ_LM3, 4: kvq.KVQ_LM4, 8: kvq.KVQ_FP8_E4M3}
    k_dev = torch.from_numpy(np.ascontiguousarray(kf)).to(dev)
    v_dev = torch.from_numpy(np.ascontiguousarray(vf)).to(dev)
    q_dev = torch.from_numpy(inp.q).to(dev)
    if args.query_scale != 1.0:
        q_dev = (q_dev.float() * args.query_scale).to(q_dev.dtype)
    kn_dev = None if kn is None else torch.from_numpy(np.ascontiguousarray(kn)).to(dev)
    vn_dev = None if vn is None else torch.from_numpy(np.ascontiguousarray(vn)).to(dev)
    R = max(1, math.ceil((1 << 30) / by["cache"]))
    proj_t = None
    if args.qjl:
        proj_t = torch.from_numpy(np.ascontiguousarray(W.qjl_projection(wl.head_dim).T)).to(dev)
    caches = []
    for r in range(R):
        c = kvq.KVCache.allocate(wl.batch, wl.kv_heads, wl.head_dim, T, fmt[wl.k_bits], fmt[wl.v_bits],
                                 seed=W.SIGN_SEED, device=dev,
                                 near_k=None if kn_dev is None else kn_dev.clone(),
                                 near_v=None if vn_dev is None else vn_dev.clone(), outliers=args.outliers,
                                 qjl_proj_t=proj_t)
        if args.outliers:
            c.calibrate(k_dev[:, :, :min(256, T)].contiguous())
        caches.append(c)
    stream = torch.cuda.current_stream()

    # ---- bulk quantize-append of the whole context, per replica ----
    for c in caches[:2]:
        c.append(k_dev, v_dev, 0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for c in caches:
        c.append(k_dev, v_dev, 0)
    e1.record(stream)
    torch.cuda.synchronize()
    append_ms = e0.elapsed_time(e1) / R
    append_tok_s = wl.batch * T / (append_ms / 1e3)
    append_bytes = wl.batch * wl.kv_heads * T * (2 * wl.head_dim * (4 if wl.dtype == "f32" else 2)
                                                + by["per_token_head"])

    # ---- decode steps ----
    knew_np, vnew_np = W.new_token(wl)
    k_new = torch.from_numpy(knew_np).to(dev)
    v_new = torch.from_numpy(vnew_np).to(dev)
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

    def attend(c, po, pml):
        c.attend(q_dev, T, S, near_splits, po, pml, **gate_kw)

    def step(i):
        c = caches[i % R]
        po, pml = bufs[i % 2]
        c.append(k_new, v_new, T - 1)
        if args.gate:
            gate_kw["spike_bits"].zero_()
        attend(c, po, pml)
        c.merge(po, pml, S, near_splits, out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The K timed steps are one HIP graph (captured after the warm-up, then
    # replayed once untimed): the timed region is GPU work, not the host's
    # per-launch overhead.  The library records no memsets, so the graph
    # holds only the kernels.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # ---- the attention kernel alone: n_att back-to-back launches between one
    # event pair (average launch duration), then one event pair per launch ----
    n_att = max(50, min(args.steps, 400))
    for i in range(5):
        attend(caches[i % R], *bufs[0])
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n_att):
        attend(caches[i % R], *bufs[0])
    e1.record(stream)
    torch.cuda.synchronize()
    att_avg = e0.elapsed_time(e1) / n_att
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_att)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        attend(caches[i % R], *bufs[0])
        b.record(stream)
    torch.cuda.synchronize()
    att_ms = [a.elapsed_time(b) for a, b in evs]

    # ---- the one-token decode-step append alone: n_att back-to-back appends
    # replayed from a HIP graph (a Python launch would outlast the kernel) ----
    g_app = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_app):
        for i in range(n_att):
            caches[i % R].append(k_new, v_new, T - 1)
    g_app.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    g_app.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    append_step_us = e0.elapsed_time(e1) / n_att * 1e3

    att_bytes = by["cache"] + by["q"] + by["out"]
    step_bytes = att_bytes + by["append_token"]
    achieved = att_bytes / (att_avg / 1e3) / 1e9
    kernel = "attend_kernel" if args.gate else caches[0].attention_kernel(wl.q_heads, near_splits)
    traffic = read_traffic(wl.name, kernel_source_sha(kernel))
    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_step / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.q_heads, "kv_heads": wl.kv_heads,
                   "head_dim": wl.head_dim, "seq_len": wl.seq_len, "k_bits": wl.k_bits, "v_bits": wl.v_bits,
                   "splits": S, "near_splits": near_splits, "layer_replicas": R, "launch": "hip_graph",
                   "gated": bool(args.gate), "query_scale": args.query_scale, "outliers": args.outliers,
                   "qjl": bool(args.qjl), "step_bytes": step_bytes},
        "pct_of_hbm_peak": round(100 * step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
        "append_tokens_per_s": round(append_tok_s, 1),
        "append_GBps": round(append_bytes / (append_ms / 1e3) / 1e9, 2),
        "append_step_us": round(append_step_us, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": kernel, "bytes_per_launch": att_bytes,
                     "avg_us": round(att_avg * 1e3, 3),
                     "event_pair_avg_us": round(float(np.mean(att_ms)) * 1e3, 3),
                     "event_pair_min_us": round(min(att_ms) * 1e3, 3)},
        "copy_probe": copy_rate(),
    }
    if args.gate:
        # a gated launch skips the value rows of gated tokens: its rate is
        # quoted against the ungated algorithmic bytes (an effective rate)
        result["roofline"]["bytes_basis"] = "ungated"
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inp)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
