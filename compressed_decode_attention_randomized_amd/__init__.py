"""Thin Python binding of libkvq (rotation-based KV-cache quantization and
decode attention on the compressed cache, MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
libkvq.so, reached through its C ABI (include/kvq.h).  PyTorch supplies
device memory and the current HIP stream.  There is no fallback: if the
library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ERANGE, KVQ_EHIP = range(5)
KVQ_F32, KVQ_F16 = 0, 1
KVQ_LM2, KVQ_LM3, KVQ_LM4, KVQ_FP8_E4M3 = 2, 3, 4, 8

EXPORTED = ("kvq_row_bytes", "kvq_lloyd_max", "kvq_make_signs", "kvq_quantize_append",
            "kvq_decode_attention", "kvq_decode_attention_gated", "kvq_decode_attention_kernel", "kvq_merge",
            "kvq_calibrate_outliers", "kvq_decode", "kvq_decode_workspace_bytes", "kvq_decode_noalloc",
            "kvq_partials_floats",
            "kvq_status_string", "kvq_last_error")


class KVQError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn} -> status {status}: {detail}")
        self.status = status


class CacheStruct(ctypes.Structure):
    """Mirror of `kvq_cache` in include/kvq.h."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32), ("k_format", ctypes.c_int32), ("v_format", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p), ("k_norms", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_norms", ctypes.c_void_p),
        ("signs", ctypes.c_void_p), ("k_centroids", ctypes.c_void_p), ("v_centroids", ctypes.c_void_p),
        ("near_k", ctypes.c_void_p), ("near_v", ctypes.c_void_p),
        ("near_len", ctypes.c_int32), ("outlier_count", ctypes.c_int32),
        ("outlier_idx", ctypes.c_void_p), ("outlier_codes", ctypes.c_void_p), ("outlier_scales", ctypes.c_void_p),
        ("qjl_dim", ctypes.c_int32), ("qjl_proj", ctypes.c_void_p), ("qjl_signs", ctypes.c_void_p),
        ("qjl_norms", ctypes.c_void_p),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvq.so (built by `python -m compressed_decode_attention_randomized_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libkvq.so not found at {path}; build it with "
                          "`python -m compressed_decode_attention_randomized_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    CP = ctypes.POINTER(CacheStruct)
    sig = {
        "kvq_row_bytes": (SZ, [I32, I32]),
        "kvq_lloyd_max": (I32, [I32, I32, P]),
        "kvq_make_signs": (I32, [U64, I32, P]),
        "kvq_quantize_append": (I32, [CP, P, P, I32, I32, I32, P]),
        "kvq_decode_attention": (I32, [CP, P, I32, I32, I32, I32, I32, P, P, P]),
        "kvq_decode_attention_gated": (I32, [CP, P, I32, I32, I32, I32, I32, P, P, P, P, P, P]),
        "kvq_calibrate_outliers": (I32, [CP, P, I32, I32, P, P]),
        "kvq_decode_attention_kernel": (ctypes.c_char_p, [CP, I32, I32, I32]),
        "kvq_merge": (I32, [CP, P, P, I32, I32, I32, P, P, P]),
        "kvq_partials_floats": (SZ, [I32, I32, I32, I32]),
        "kvq_decode": (I32, [CP, P, I32, I32, I32, I32, I32, P, SZ, P, P, P]),
        "kvq_decode_workspace_bytes": (SZ, [I32, I32, I32, I32, I32]),
        "kvq_decode_noalloc": (I32, [CP, P, I32, I32, I32, I32, I32, P, P, P]),
        "kvq_status_string": (ctypes.c_char_p, [I32]),
        "kvq_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _check(status: int, fn: str):
    if status != KVQ_OK:
        lib = load()
        raise KVQError(status, fn, lib.kvq_last_error().decode() or lib.kvq_status_string(status).decode())


# ---------------------------------------------------------------------------
# host-side setup calls
# ---------------------------------------------------------------------------

def row_bytes(fmt: int, head_dim: int) -> int:
    return int(load().kvq_row_bytes(fmt, head_dim))


def lloyd_max(bits: int, head_dim: int):
    """float32 centroid table (numpy, ascending) from kvq_lloyd_max."""
    import numpy as np
    out = np.zeros(1 << bits, dtype=np.float32)
    _check(load().kvq_lloyd_max(bits, head_dim, out.ctypes.data), "kvq_lloyd_max")
    return out


def make_signs(seed: int, head_dim: int):
    """int8 +-1 sign vector (numpy) from kvq_make_signs."""
    import numpy as np
    out = np.zeros(head_dim, dtype=np.int8)
    _check(load().kvq_make_signs(seed, head_dim, out.ctypes.data), "kvq_make_signs")
    return out


# ---------------------------------------------------------------------------
# device cache
# ---------------------------------------------------------------------------

def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return KVQ_F16
    if t.dtype == torch.float32:
        return KVQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use float16 or float32")


def _need(t, name: str, shape, dtype=None):
    """t must be a contiguous device tensor of this shape (and dtype, if given):
    the kernels index these buffers by the shape alone, so a wrong shape or
    element size would make them read or write past the allocation."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class KVCache:
    """One layer's compressed cache in device memory (torch tensors), plus the
    ctypes view of it handed to libkvq."""
    batch: int
    kv_heads: int
    head_dim: int
    capacity: int
    k_format: int
    v_format: int
    k_codes: object
    k_norms: object
    v_codes: object
    v_norms: object
    signs: object
    k_centroids: object
    v_centroids: object
    near_k: object = None
    near_v: object = None
    outlier_idx: object = None       # key outlier stream: [B, Hkv, 8] int32, codes [B, Hkv, cap, 8] int8,
    outlier_codes: object = None     # scales [B, Hkv, cap] float32 (None: stream off)
    outlier_scales: object = None
    qjl_proj: object = None          # QJL sketch: S^T [d, d] float32, sign bytes [B, Hkv, cap, d/8] uint8,
    qjl_signs: object = None         # residual norms [B, Hkv, cap] float16 (None: sketch off)
    qjl_norms: object = None

    @classmethod
    def allocate(cls, batch, kv_heads, head_dim, capacity, k_format=KVQ_LM4, v_format=KVQ_LM4,
                 seed=42, device="cuda", near_k=None, near_v=None, outliers: int = 0, qjl_proj_t=None):
        """outliers: 0, or 8 for the key outlier stream (its channels are
        chosen by calibrate()).  qjl_proj_t: the QJL projection transposed,
        [head_dim, head_dim] float32 on the device (element (j, i) is
        S[i][j]), or None for no sketch."""
        import torch
        kr, vr = row_bytes(k_format, head_dim), row_bytes(v_format, head_dim)
        if not kr or not vr:
            raise ValueError("unsupported head_dim/format")
        dev = torch.device(device)
        capacity = (capacity + 15) // 16 * 16          # the ABI wants a multiple of 16
        k_codes = torch.zeros((batch, kv_heads, capacity, kr), dtype=torch.uint8, device=dev)
        v_codes = torch.zeros((batch, kv_heads, capacity, vr), dtype=torch.uint8, device=dev)
        k_norms = torch.zeros((batch, kv_heads, capacity), dtype=torch.float16, device=dev)
        v_norms = torch.zeros((batch, kv_heads, capacity), dtype=torch.float16, device=dev)
        signs = torch.from_numpy(make_signs(seed, head_dim)).to(dev)
        kc = torch.from_numpy(lloyd_max(k_format, head_dim)).to(dev) if k_format != KVQ_FP8_E4M3 else \
            torch.zeros(16, dtype=torch.float32, device=dev)
        vc = torch.from_numpy(lloyd_max(v_format, head_dim)).to(dev)
        oi = oc = osc = None
        if outliers:
            oi = torch.zeros((batch, kv_heads, outliers), dtype=torch.int32, device=dev)
            oc = torch.zeros((batch, kv_heads, capacity, outliers), dtype=torch.int8, device=dev)
            osc = torch.zeros((batch, kv_heads, capacity), dtype=torch.float32, device=dev)
        zs = zn = None
        if qjl_proj_t is not None:
            _need(qjl_proj_t, "qjl_proj_t", (head_dim, head_dim))
            if qjl_proj_t.dtype != torch.float32:
                raise ValueError("qjl_proj_t must be float32")
            zs = torch.zeros((batch, kv_heads, capacity, head_dim // 8), dtype=torch.uint8, device=dev)
            zn = torch.zeros((batch, kv_heads, capacity), dtype=torch.float16, device=dev)
        return cls(batch, kv_heads, head_dim, capacity, k_format, v_format, k_codes, k_norms, v_codes,
                   v_norms, signs, kc, vc, near_k, near_v, oi, oc, osc, qjl_proj_t, zs, zn)

    @property
    def near_len(self) -> int:
        return 0 if self.near_k is None else int(self.near_k.shape[2])

    def struct(self) -> CacheStruct:
        p = lambda t: 0 if t is None else t.data_ptr()
        if self.near_k is not None:
            import torch
            _need(self.near_k, "near_k", (self.batch, self.kv_heads, self.near_len, self.head_dim), torch.float16)
            _need(self.near_v, "near_v", (self.batch, self.kv_heads, self.near_len, self.head_dim), torch.float16)
        return CacheStruct(self.batch, self.kv_heads, self.head_dim, self.capacity, self.k_format,
                           self.v_format, p(self.k_codes), p(self.k_norms), p(self.v_codes), p(self.v_norms),
                           p(self.signs), p(self.k_centroids), p(self.v_centroids), p(self.near_k),
                           p(self.near_v), self.near_len,
                           0 if self.outlier_idx is None else int(self.outlier_idx.shape[-1]),
                           p(self.outlier_idx), p(self.outlier_codes), p(self.outlier_scales),
                           0 if self.qjl_proj is None else self.head_dim, p(self.qjl_proj), p(self.qjl_signs),
                           p(self.qjl_norms))

    # -- kvq_quantize_append --------------------------------------------------
    def append(self, k, v, start_pos: int):
        n_new = int(k.shape[2])
        shape = (self.batch, self.kv_heads, n_new, self.head_dim)
        _need(k, "k", shape)
        _need(v, "v", shape)
        if k.dtype != v.dtype:
            raise TypeError("k and v must share a dtype")
        cs = self.struct()
        _check(load().kvq_quantize_append(ctypes.byref(cs), k.data_ptr(), v.data_ptr(), _dtype_code(k),
                                          start_pos, n_new, _stream_handle(k.device)), "kvq_quantize_append")

    # -- kvq_calibrate_outliers -----------------------------------------------
    def calibrate(self, k_calib):
        """Pick the key outlier channels from calibration keys [B, Hkv, N, d]
        (the context's first tokens) into outlier_idx."""
        if self.outlier_idx is None:
            raise ValueError("the cache has no outlier stream (allocate with outliers=8)")
        n = int(k_calib.shape[2])
        _need(k_calib, "k_calib", (self.batch, self.kv_heads, n, self.head_dim))
        cs = self.struct()
        _check(load().kvq_calibrate_outliers(ctypes.byref(cs), k_calib.data_ptr(), _dtype_code(k_calib), n,
                                             self.outlier_idx.data_ptr(), _stream_handle(k_calib.device)),
               "kvq_calibrate_outliers")

    # -- kvq_decode_attention -------------------------------------------------
    def partial_buffers(self, q_heads: int, num_splits: int, num_near_splits: int = 0):
        import torch
        S = num_splits + num_near_splits
        dev = self.k_codes.device
        return (torch.empty((self.batch, q_heads, S, self.head_dim), dtype=torch.float32, device=dev),
                torch.empty((self.batch, q_heads, S, 2), dtype=torch.float32, device=dev))

    def attend(self, q, seq_len: int, num_splits: int, num_near_splits: int = 0, part_o=None, part_ml=None,
               gate_ref=None, spike_ref=None, spike_bits=None):
        """kvq_decode_attention, or kvq_decode_attention_gated when a gate or
        spike reference ([B, Hq] float32) is given (spike_bits: [B, Hq,
        ceil(seq_len/32)] int32, zeroed by the caller)."""
        q_heads = int(q.shape[1])
        _need(q, "q", (self.batch, q_heads, self.head_dim))
        if part_o is None:
            part_o, part_ml = self.partial_buffers(q_heads, num_splits, num_near_splits)
        import torch
        S = num_splits + num_near_splits
        _need(part_o, "part_o", (self.batch, q_heads, S, self.head_dim), torch.float32)
        _need(part_ml, "part_ml", (self.batch, q_heads, S, 2), torch.float32)
        cs = self.struct()
        if gate_ref is None and spike_ref is None:
            _check(load().kvq_decode_attention(ctypes.byref(cs), q.data_ptr(), _dtype_code(q), q_heads, seq_len,
                                               num_splits, num_near_splits, part_o.data_ptr(), part_ml.data_ptr(),
                                               _stream_handle(q.device)), "kvq_decode_attention")
            return part_o, part_ml
        for name, ref in (("gate_ref", gate_ref), ("spike_ref", spike_ref)):
            if ref is not None:
                _need(ref, name, (self.batch, q_heads))
                if ref.dtype != torch.float32:
                    raise TypeError(f"{name} must be float32")
        if spike_bits is not None:
            _need(spike_bits, "spike_bits", (self.batch, q_heads, (seq_len + 31) // 32))
            if spike_bits.dtype != torch.int32:
                raise TypeError("spike_bits must be int32 (the bits of uint32 words)")
        p = lambda t: 0 if t is None else t.data_ptr()
        _check(load().kvq_decode_attention_gated(ctypes.byref(cs), q.data_ptr(), _dtype_code(q), q_heads, seq_len,
                                                 num_splits, num_near_splits, p(gate_ref), p(spike_ref),
                                                 p(spike_bits), part_o.data_ptr(), part_ml.data_ptr(),
                                                 _stream_handle(q.device)), "kvq_decode_attention_gated")
        return part_o, part_ml

    # -- kvq_merge ------------------------------------------------------------
    def merge(self, part_o, part_ml, num_splits: int, num_near_splits: int = 0, out=None, lse=None):
        import torch
        B, Hq, S, d = part_o.shape
        if B != self.batch or d != self.head_dim or S != num_splits + num_near_splits:
            raise ValueError(f"part_o has shape {tuple(part_o.shape)}, expected "
                             f"({self.batch}, Hq, {num_splits + num_near_splits}, {self.head_dim})")
        _need(part_o, "part_o", (B, Hq, S, d), torch.float32)
        _need(part_ml, "part_ml", (B, Hq, S, 2), torch.float32)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=part_o.device)
        _need(out, "out", (B, Hq, d), torch.float32)
        if lse is not None:
            _need(lse, "lse", (B, Hq), torch.float32)
        cs = self.struct()
        _check(load().kvq_merge(ctypes.byref(cs), part_o.data_ptr(), part_ml.data_ptr(), Hq, num_splits,
                                num_near_splits, out.data_ptr(), 0 if lse is None else lse.data_ptr(),
                                _stream_handle(part_o.device)), "kvq_merge")
        return out

    def attention_kernel(self, q_heads: int, num_splits: int, num_near_splits: int = 0) -> str:
        """Name of the kernel kvq_decode_attention launches for this cache."""
        cs = self.struct()
        name = load().kvq_decode_attention_kernel(ctypes.byref(cs), q_heads, num_splits, num_near_splits)
        if not name:
            raise KVQError(KVQ_EINVAL, "kvq_decode_attention_kernel", load().kvq_last_error().decode())
        return name.decode()

    def decode(self, q, seq_len: int, num_splits: int, num_near_splits: int = 0, lse=None):
        po, pml = self.attend(q, seq_len, num_splits, num_near_splits)
        return self.merge(po, pml, num_splits, num_near_splits, lse=lse)

    def workspace(self, q_heads: int, num_splits: int, num_near_splits: int = 0):
        """A device workspace for decode_ws (uint8, kvq_decode_workspace_bytes)."""
        import torch
        n = int(load().kvq_decode_workspace_bytes(self.batch, q_heads, num_splits, num_near_splits, self.head_dim))
        if not n:
            raise ValueError("invalid decode shape")
        return torch.empty(n, dtype=torch.uint8, device=self.k_codes.device)

    def decode_ws(self, q, seq_len: int, num_splits: int, num_near_splits: int = 0, workspace=None, out=None,
                  lse=None, noalloc: bool = False):
        """kvq_decode (split partials in `workspace`, from workspace() if None),
        or kvq_decode_noalloc (the library's fixed device scratch) when noalloc."""
        import torch
        q_heads = int(q.shape[1])
        _need(q, "q", (self.batch, q_heads, self.head_dim))
        if out is None:
            out = torch.empty((self.batch, q_heads, self.head_dim), dtype=torch.float32, device=q.device)
        _need(out, "out", (self.batch, q_heads, self.head_dim), torch.float32)
        if lse is not None:
            _need(lse, "lse", (self.batch, q_heads), torch.float32)
        cs = self.struct()
        lp = 0 if lse is None else lse.data_ptr()
        if noalloc:
            _check(load().kvq_decode_noalloc(ctypes.byref(cs), q.data_ptr(), _dtype_code(q), q_heads, seq_len,
                                             num_splits, num_near_splits, out.data_ptr(), lp,
                                             _stream_handle(q.device)), "kvq_decode_noalloc")
            return out
        if workspace is None:
            workspace = self.workspace(q_heads, num_splits, num_near_splits)
        if not (workspace.is_cuda and workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous device tensor")
        nbytes = workspace.numel() * workspace.element_size()
        _check(load().kvq_decode(ctypes.byref(cs), q.data_ptr(), _dtype_code(q), q_heads, seq_len, num_splits,
                                 num_near_splits, workspace.data_ptr(), nbytes, out.data_ptr(), lp,
                                 _stream_handle(q.device)), "kvq_decode")
        return out
