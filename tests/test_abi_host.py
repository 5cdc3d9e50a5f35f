"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, its host-side setup calls agree with the oracle, and host-side
validation rejects bad arguments before any launch (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_decode_attention_randomized_amd as kvq
from oracle import kvq_oracle as O
from tests.conftest import ROOT


def _header_functions():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", src)))


def test_library_loads_and_exports_header_symbols():
    lib = kvq.load()
    names = _header_functions()
    assert "kvq_quantize_append" in names and "kvq_decode_attention" in names and "kvq_merge" in names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(kvq.EXPORTED) == names


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_lloyd_max_table_bit_identical_to_oracle(bits, d):
    got = kvq.lloyd_max(bits, d)
    if bits == 1:
        want = (O.lloyd_max_gaussian(2)[0] / np.sqrt(d)).astype(np.float32)
    else:
        want, _ = O.codebook(bits, d)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("seed", [0, 1, 42, 2**63 + 5])
def test_signs_match_oracle(seed):
    assert np.array_equal(kvq.make_signs(seed, 256), O.rademacher_signs(seed, 256))


def test_row_bytes():
    assert kvq.row_bytes(kvq.KVQ_LM4, 128) == 64
    assert kvq.row_bytes(kvq.KVQ_LM3, 128) == 48
    assert kvq.row_bytes(kvq.KVQ_LM2, 256) == 64
    assert kvq.row_bytes(kvq.KVQ_FP8_E4M3, 128) == 128
    assert kvq.row_bytes(7, 128) == 0 and kvq.row_bytes(kvq.KVQ_LM4, 96) == 0


def _fake_cache(**over):
    """A cache struct whose device pointers are never dereferenced (every
    call below fails validation before any launch)."""
    base = dict(batch=2, kv_heads=2, head_dim=128, capacity=64, k_format=4, v_format=4,
                k_codes=0x1000, k_norms=0x2000, v_codes=0x3000, v_norms=0x4000, signs=0x5000,
                k_centroids=0x6000, v_centroids=0x7000, near_k=0, near_v=0, near_len=0, outlier_count=0,
                outlier_idx=0, outlier_codes=0, outlier_scales=0, qjl_dim=0, qjl_proj=0, qjl_signs=0, qjl_norms=0)
    base.update(over)
    return kvq.CacheStruct(**base)


def _append(cs, k=0x8000, v=0x9000, dtype=1, start=0, n=1):
    return kvq.load().kvq_quantize_append(ctypes.byref(cs) if cs is not None else None, k, v, dtype, start, n, None)


def _attend(cs, q=0x8000, qd=1, hq=4, T=8, S=2, SN=0, po=0xA000, pml=0xB000):
    return kvq.load().kvq_decode_attention(ctypes.byref(cs) if cs is not None else None, q, qd, hq, T, S, SN,
                                           po, pml, None)


def _gated(cs, gate=0xE000, spike=0, bits=0, T=8, **kw):
    return kvq.load().kvq_decode_attention_gated(ctypes.byref(cs), 0x8000, 1, 4, T, 2, 0, gate, spike, bits,
                                                 0xA000, 0xB000, None)


def test_gated_attention_validation():
    """The gated call's own argument checks (host only: every case fails
    before a launch)."""
    cs = _fake_cache()
    assert _gated(cs, gate=0, spike=0) == kvq.KVQ_EINVAL                   # neither reference
    assert _gated(cs, gate=0, spike=0xE000, bits=0) == kvq.KVQ_EINVAL      # spike_ref without flag words
    assert _gated(cs, gate=0xE000, spike=0, bits=0xF000) == kvq.KVQ_EINVAL # flag words without spike_ref
    assert _gated(cs, gate=0xE002) == kvq.KVQ_EINVAL                       # misaligned reference
    assert _gated(cs, gate=0, spike=0xE000, bits=0xF001) == kvq.KVQ_EINVAL # misaligned flag words
    assert _gated(cs, T=1000) == kvq.KVQ_ERANGE                             # the plain call's checks come first


def test_calibration_validation():
    lib = kvq.load()
    cs = _fake_cache()
    cal = lambda keys=0x8000, dt=1, n=4, out=0x9000: lib.kvq_calibrate_outliers(ctypes.byref(cs), keys, dt, n, out, None)
    assert cal(n=0) == kvq.KVQ_EINVAL
    assert cal(keys=0) == kvq.KVQ_EINVAL and cal(out=0) == kvq.KVQ_EINVAL
    assert cal(keys=0x8008) == kvq.KVQ_EINVAL and cal(out=0x9004) == kvq.KVQ_EINVAL
    assert cal(dt=7) == kvq.KVQ_EINVAL


def test_append_validation():
    assert _append(None) == kvq.KVQ_EINVAL
    assert _append(_fake_cache(), start=60, n=5) == kvq.KVQ_ERANGE
    assert _append(_fake_cache(), start=-1) == kvq.KVQ_ERANGE
    assert _append(_fake_cache(), dtype=5) == kvq.KVQ_EINVAL
    assert _append(_fake_cache(), k=0) == kvq.KVQ_EINVAL
    assert _append(_fake_cache(), k=0x8001) == kvq.KVQ_EINVAL           # misaligned input
    assert _append(_fake_cache(k_codes=0x1004)) == kvq.KVQ_EINVAL        # misaligned codes
    assert _append(_fake_cache(head_dim=96)) == kvq.KVQ_EUNSUPPORTED
    assert _append(_fake_cache(v_format=8)) == kvq.KVQ_EINVAL
    assert _append(_fake_cache(k_norms=0)) == kvq.KVQ_EINVAL
    assert _append(_fake_cache(outlier_count=4)) == kvq.KVQ_EUNSUPPORTED                 # 0 or 8 only
    assert _append(_fake_cache(outlier_count=8)) == kvq.KVQ_EINVAL                       # buffers missing
    assert _append(_fake_cache(outlier_count=8, outlier_idx=0xC000, outlier_codes=0xD000,
                               outlier_scales=0xE004)) == kvq.KVQ_EINVAL                 # misaligned scales
    assert _append(_fake_cache(outlier_count=8, k_format=8, k_norms=0, outlier_idx=0xC000,
                               outlier_codes=0xD000, outlier_scales=0xE000)) == kvq.KVQ_EUNSUPPORTED
    qjl = dict(qjl_dim=128, qjl_proj=0xC000, qjl_signs=0xD000, qjl_norms=0xE000)
    assert _append(_fake_cache(**{**qjl, "qjl_dim": 64})) == kvq.KVQ_EUNSUPPORTED        # m = head_dim only
    assert _append(_fake_cache(**{**qjl, "qjl_signs": 0})) == kvq.KVQ_EINVAL              # buffers missing
    assert _append(_fake_cache(**{**qjl, "qjl_norms": 0xE002})) == kvq.KVQ_EINVAL         # misaligned norms
    assert _append(_fake_cache(**qjl, k_format=8, k_norms=0)) == kvq.KVQ_EUNSUPPORTED     # Lloyd-Max keys only
    assert _append(_fake_cache(**qjl, outlier_count=8, outlier_idx=0xC000, outlier_codes=0xD000,
                               outlier_scales=0xE000)) == kvq.KVQ_EUNSUPPORTED          # one side stream at a time
    assert _gated(_fake_cache(**qjl)) == kvq.KVQ_EUNSUPPORTED
    assert _append(_fake_cache(), n=0) == kvq.KVQ_OK                     # nothing to do, no launch
    assert "capacity" in kvq.load().kvq_last_error().decode() or True


def test_attend_and_merge_validation():
    assert _attend(None) == kvq.KVQ_EINVAL
    assert _attend(_fake_cache(), hq=3) == kvq.KVQ_EINVAL                # not a multiple of kv_heads
    assert _attend(_fake_cache(), T=65) == kvq.KVQ_ERANGE
    assert _attend(_fake_cache(), S=0) == kvq.KVQ_EINVAL
    assert _attend(_fake_cache(), SN=1) == kvq.KVQ_EINVAL                # no near tier
    assert _attend(_fake_cache(near_len=4, near_k=0xC000, near_v=0xD000), SN=0) == kvq.KVQ_EINVAL
    assert _attend(_fake_cache(), q=0) == kvq.KVQ_EINVAL
    assert _attend(_fake_cache(), qd=7) == kvq.KVQ_EINVAL
    msg = kvq.load().kvq_last_error().decode()
    assert "q_dtype" in msg
    lib = kvq.load()
    cs = _fake_cache()
    assert lib.kvq_merge(ctypes.byref(cs), 0, 0xB000, 4, 2, 0, 0xC000, 0, None) == kvq.KVQ_EINVAL
    assert lib.kvq_merge(ctypes.byref(cs), 0xA000, 0xB000, 4, 0, 0, 0xC000, 0, None) == kvq.KVQ_EINVAL
    assert lib.kvq_merge(None, 0xA000, 0xB000, 4, 2, 0, 0xC000, 0, None) == kvq.KVQ_EINVAL
    assert lib.kvq_merge(ctypes.byref(cs), 0xA004, 0xB000, 4, 2, 0, 0xC000, 0, None) == kvq.KVQ_EINVAL
    assert _attend(_fake_cache(), po=0xA004) == kvq.KVQ_EINVAL           # misaligned partials


def test_attention_kernel_choice():
    """The kernel kvq_decode_attention dispatches to (no launch involved)."""
    lib = kvq.load()

    def name(hq=4, SN=0, S=4, **over):
        r = lib.kvq_decode_attention_kernel(ctypes.byref(_fake_cache(**over)), hq, S, SN)
        return None if r is None else r.decode()

    assert name() == "attend_pair_kernel"                                # 4-bit K and V, d=128, G=2
    assert name(hq=2) == "attend_pair_kernel"                            # G=1
    assert name(hq=32) is None                                           # G=16: above every kernel's groups
    assert name(head_dim=256) == "attend_wide_kernel"                     # 4-bit, d=256, G <= 8
    assert name(head_dim=256, hq=16) == "attend_wide_kernel"             # G=8
    assert name(head_dim=256, k_format=2, v_format=2) == "attend_wide_kernel"
    assert name(head_dim=256, k_format=3, v_format=3, hq=16) == "attend_wide_kernel"   # 3-bit, d=256, G=8
    assert name(head_dim=256, k_format=3, v_format=3, hq=2) == "attend_kernel"         # 3-bit at G=1: VALU kernel
    assert name(head_dim=256, k_format=3, v_format=4) == "attend_kernel"  # mixed widths: VALU kernel
    assert name(k_format=2, v_format=2) == "attend_mfma_kernel"
    assert name(k_format=3, v_format=3) is None                           # 3-bit values at d=128, G=2: not built
    assert name(head_dim=64) == "attend_kernel"
    assert name(k_format=8, k_norms=0, near_len=4, near_k=0xC000, near_v=0xD000, SN=1) == "attend_kernel"
    # 4-bit codes at d=128 beside an fp16 near tier: both tiers in one pair-table launch while the
    # near splits are at most the far splits and the far splits fit one work-group per compute unit
    near = dict(near_len=4, near_k=0xC000, near_v=0xD000)
    assert name(**near, SN=1) == "attend_pair_kernel"
    assert name(**near, SN=4, S=4) == "attend_pair_kernel"
    assert name(**near, SN=5, S=4) == "attend_pair_kernel+attend_kernel"     # more near than far splits
    assert name(**near, SN=1, S=65) == "attend_pair_kernel+attend_kernel"    # 4 pairs x 65 splits > 256 CUs
    assert name(**near, SN=1, S=64) == "attend_pair_kernel"
    # near splits on the VALU kernel, far splits on the d=256 pair-table kernel
    assert name(head_dim=256, near_len=4, near_k=0xC000, near_v=0xD000, SN=1) == "attend_wide_kernel+attend_kernel"
    assert name(S=0) is None
    assert name(hq=2, k_format=3, v_format=3, near_len=4, near_k=0xC000, near_v=0xD000, SN=1) == "attend_kernel"
    qjl = dict(qjl_dim=128, qjl_proj=0xC000, qjl_signs=0xD000, qjl_norms=0xE000)
    assert name(**qjl) == "attend_kernel"                                 # the QJL sketch beside 4-bit keys: VALU kernel
    assert name(**qjl, k_format=3, v_format=4) == "attend_wide_kernel"    # the page's 68-byte key, G=2
    assert name(**qjl, k_format=3, v_format=4, hq=2) == "attend_kernel"   # G=1
    out = dict(outlier_count=8, outlier_idx=0xC000, outlier_codes=0xD000, outlier_scales=0xE000)
    assert name(**out) == "attend_wide_kernel"                            # outlier stream, 4-bit, d=128, G=2
    assert name(**out, hq=16) == "attend_wide_kernel"                     # G=8
    assert name(**out, head_dim=256) == "attend_kernel"
    assert name(**out, k_format=3, v_format=3, hq=2) == "attend_kernel"
    assert name(**out, near_len=4, near_k=0xC000, near_v=0xD000, SN=1) == "attend_kernel"
    assert name(k_format=3, v_format=4, hq=8) == "attend_wide_kernel"     # 3-bit keys beside 4-bit values, G=4
    assert name(k_format=3, v_format=4, hq=16) == "attend_wide_kernel"    # G=8
    assert name(k_format=3, v_format=4, hq=2) == "attend_kernel"          # G=1: VALU kernel
    assert name(k_format=3, v_format=3, hq=4) is None                     # 3-bit values at d=128: G=1 only
    assert name(k_format=3, v_format=3, hq=2) == "attend_kernel"
    assert name(hq=3) is None and name(head_dim=96) is None


def test_status_strings():
    lib = kvq.load()
    for s in range(5):
        assert lib.kvq_status_string(s)
    assert lib.kvq_partials_floats(2, 4, 3, 128) == 2 * 4 * 3 * 128


def test_noalloc_size_limit_and_workspace_validation():
    """kvq_decode_noalloc refuses partials larger than its fixed scratch
    (16 MiB) before any launch; kvq_decode refuses a missing or small
    workspace; the workspace size follows the partials' layout."""
    lib = kvq.load()
    cs = _fake_cache(batch=64, kv_heads=64)
    assert lib.kvq_decode_workspace_bytes(64, 64, 64, 0, 128) > 16 << 20
    r = lib.kvq_decode_noalloc(ctypes.byref(cs), 0x8000, 1, 64, 32, 64, 0, 0xC000, 0, None)
    assert r == kvq.KVQ_ERANGE and "fixed scratch" in lib.kvq_last_error().decode()
    cs = _fake_cache()
    assert lib.kvq_decode_workspace_bytes(2, 4, 3, 1, 128) == 2 * 4 * 4 * 128 * 4 + 2 * 4 * 4 * 2 * 4
    n = lib.kvq_decode_workspace_bytes(2, 4, 3, 0, 128)
    # both refused on the host (one byte short; NULL), so no launch is attempted
    assert lib.kvq_decode(ctypes.byref(cs), 0x8000, 1, 4, 32, 3, 0, 0xA000, n - 1, 0xC000, 0, None) == kvq.KVQ_EINVAL
    assert lib.kvq_decode(ctypes.byref(cs), 0x8000, 1, 4, 32, 3, 0, 0, n, 0xC000, 0, None) == kvq.KVQ_EINVAL
    assert lib.kvq_decode_workspace_bytes(2, 4, 0, 0, 128) == 0
