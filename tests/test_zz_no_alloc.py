"""kvq_decode_noalloc (the decode call for callers that cannot allocate: split
partials in the library's fixed device scratch) against kvq_decode (the same
kernels with a caller workspace), through the C ABI: identical outputs and
log-sum-exps on two calls in a row, the second with a smaller input, for a
plain cache and one with a near tier, plus the oracle bar on the first."""
import ctypes
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import compressed_decode_attention_randomized_amd as kvq  # noqa: E402
import workloads as W  # noqa: E402
from oracle import kvq_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.load()
    return torch.device("cuda")


def _t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _case(dev, wl):
    inp = W.generate(wl)
    if wl.near_fraction:
        kn, vn = inp.tier("near")
        kf, vf = inp.tier("far")
        SN = wl.near_split_count
    else:
        kf, vf, kn, vn, SN = inp.k, inp.v, None, None, 0
    T = kf.shape[2]
    fmt = {4: kvq.KVQ_LM4, 8: kvq.KVQ_FP8_E4M3}
    cache = kvq.KVCache.allocate(wl.batch, wl.kv_heads, wl.head_dim, T, fmt[wl.k_bits], fmt[wl.v_bits],
                                 seed=W.SIGN_SEED, device=dev, near_k=None if kn is None else _t(kn, dev),
                                 near_v=None if vn is None else _t(vn, dev))
    cache.append(_t(kf, dev), _t(vf, dev), 0)
    return inp, cache, T, SN, kn, vn


def _call(lib, fn, cache, q, T, S, SN, out, lse, ws=None):
    cs = cache.struct()
    stream = torch.cuda.current_stream().cuda_stream
    if ws is None:
        return lib.kvq_decode_noalloc(ctypes.byref(cs), q.data_ptr(), kvq.KVQ_F16, q.shape[1], T, S, SN,
                                      out.data_ptr(), lse.data_ptr(), stream)
    return lib.kvq_decode(ctypes.byref(cs), q.data_ptr(), kvq.KVQ_F16, q.shape[1], T, S, SN, ws.data_ptr(),
                          ws.numel(), out.data_ptr(), lse.data_ptr(), stream)


@pytest.mark.parametrize("name,big,small", [
    ("llama7b_layer", dict(batch=4, seq_len=3000, splits=8), dict(batch=2, seq_len=777, splits=5)),
    ("two_tier", dict(batch=4, q_heads=8, kv_heads=8, seq_len=2500, splits=6, near_splits=2),
     dict(batch=1, q_heads=4, kv_heads=4, seq_len=900, splits=3, near_splits=1)),
])
def test_noalloc_equals_workspace_decode(dev, name, big, small):
    lib = kvq.load()
    for i, kw in enumerate((big, small)):
        wl = W.WORKLOADS[name].scaled(**kw)
        inp, cache, T, SN, kn, vn = _case(dev, wl)
        q = _t(inp.q, dev)
        B, Hq, d = wl.batch, wl.q_heads, wl.head_dim
        n = lib.kvq_decode_workspace_bytes(B, Hq, wl.splits, SN, d)
        assert n > 0
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        o_ws = torch.full((B, Hq, d), float("nan"), device=dev)
        l_ws = torch.full((B, Hq), float("nan"), device=dev)
        o_na = torch.full((B, Hq, d), float("nan"), device=dev)
        l_na = torch.full((B, Hq), float("nan"), device=dev)
        assert _call(lib, "kvq_decode", cache, q, T, wl.splits, SN, o_ws, l_ws, ws) == kvq.KVQ_OK
        assert _call(lib, "kvq_decode_noalloc", cache, q, T, wl.splits, SN, o_na, l_na) == kvq.KVQ_OK, \
            lib.kvq_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na), f"call {i}: outputs differ"
        if i == 0:
            s = O.rademacher_signs(W.SIGN_SEED, d)
            kp = cache.k_codes[:, :, :T].cpu().numpy()
            vp = cache.v_codes[:, :, :T].cpu().numpy()
            k_rot = O.e4m3_decode(kp) if wl.k_bits == 8 else O.dequantize_lm(
                O.unpack(kp, 4, d), cache.k_norms[:, :, :T].cpu().numpy().view(np.uint16), 4)
            v_rot = O.dequantize_lm(O.unpack(vp, 4, d), cache.v_norms[:, :, :T].cpu().numpy().view(np.uint16), 4)
            q64 = inp.q.astype(np.float64)
            ref = O.attention(q64, k_rot, v_rot, s) if kn is None else \
                O.two_tier_attention(q64, kn.astype(np.float64), vn.astype(np.float64), k_rot, v_rot, s)
            got = o_na.cpu().numpy()
            assert np.abs(got - ref).max() <= 2e-3
            rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
            assert rel.max() <= 1e-3
