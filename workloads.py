"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module holds shapes and random draws only.  It contains none of the
method's arithmetic (no rotation, no norms, no codebook, no attention), so
both sides of every parity test receive identical inputs without either side
importing the other.

Five workloads, named by what they are, and one more for the fp16 decode
buffer:

  single_head_fp32   1 head, d=128, batch 1, context 1024, fp32 K/V ~N(0,1),
                     2 key channels scaled x20
  llama7b_layer      batch 8, 32 query / 8 KV heads (GQA 4), d=128,
                     context 8192, fp16 K/V ~N(0,1), 4 key channels/head x20
  long_context       batch 1, 32/8 heads, d=128, context 32768, fp16 K/V with
                     per-head lognormal(0,1) channel scales on K and on V,
                     32 split-K partitions
  bitwidth_sweep     batch 32, 16/16 heads, d=256, context 4096, fp16 K/V,
                     8 key channels/head x10, 2/3/4-bit codes
  two_tier           batch 16, 16/16 heads, d=128, context 16384, fp16 K/V;
                     10% of tokens (per batch entry and head) kept in fp16 as
                     the near tier, chosen as the top 10% of a seeded random
                     per-token score; the rest is the far tier (fp8 keys,
                     4-bit values)
  decode_buffer      llama7b_layer's shapes and draws; the 256 most recent
                     tokens stay fp16 (near tier, original domain), the rest
                     is 4-bit

Recipe (all draws from numpy PCG64, ``default_rng(1000 + index)``):
  1. K drawn N(0,1) in float32, shape [B, Hkv, T, d]; then V the same.
  2. Outlier channels: for each KV head, ``rng.choice(d, n, replace=False)``
     channel indices; those key channels are multiplied by the scale for every
     batch entry and token.
  3. Lognormal variant: per KV head, per channel, one lognormal(0, sigma)
     factor for K and an independent one for V.
  4. The decode query is drawn after K and V, N(0,1), shape [B, Hq, d].
  5. Everything is cast to the storage dtype with round-to-nearest-even.
  6. two_tier only: a per-(b, h, t) uniform score is drawn last; the near tier
     is the floor(0.1*T) tokens with the highest score (ties to the lower
     index), in ascending token order; the far tier is the rest, in order.
     decode_buffer draws no score: its near tier is the last 256 positions.
  7. QJL projection (keys with a residual sketch): its own generator,
     ``default_rng(QJL_SEED + d)``, an [m, d] float32 N(0,1) matrix, m = d;
     the library takes it transposed ([d, m]).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SIGN_SEED = 42
QJL_SEED = 4242


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    seq_len: int
    k_bits: int            # 2/3/4 Lloyd-Max bits; 8 means fp8-E4M3 keys (far tier)
    v_bits: int
    dtype: str             # "f32" or "f16"
    splits: int            # split-K partitions used by the timed launch
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    lognormal_sigma: float = 0.0
    near_fraction: float = 0.0
    # near tier = the most recent near_len tokens (an fp16 decode buffer)
    # instead of the seeded score mask
    near_recent: bool = False
    near_splits: int = 0   # near-tier split-K partitions (0: one per 8 far splits, at least 1)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def near_len(self) -> int:
        return int(np.floor(self.near_fraction * self.seq_len)) if self.near_fraction else 0

    @property
    def near_split_count(self) -> int:
        if not self.near_fraction:
            return 0
        return self.near_splits or max(1, self.splits // 8)

    @property
    def far_len(self) -> int:
        return self.seq_len - self.near_len

    def with_bits(self, bits: int) -> "Workload":
        return dataclasses.replace(self, k_bits=bits, v_bits=bits,
                                   name=f"{self.name.split('@')[0]}@b{bits}")

    def scaled(self, **kw) -> "Workload":
        """Same recipe at other sizes (used for small parity cases)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "single_head_fp32": Workload("single_head_fp32", 1, batch=1, q_heads=1, kv_heads=1,
                                 head_dim=128, seq_len=1024, k_bits=4, v_bits=4, dtype="f32",
                                 splits=8, outlier_channels=2, outlier_scale=20.0),
    "llama7b_layer": Workload("llama7b_layer", 2, batch=8, q_heads=32, kv_heads=8,
                              head_dim=128, seq_len=8192, k_bits=4, v_bits=4, dtype="f16",
                              splits=4, outlier_channels=4, outlier_scale=20.0),
    "long_context": Workload("long_context", 3, batch=1, q_heads=32, kv_heads=8,
                             head_dim=128, seq_len=32768, k_bits=4, v_bits=4, dtype="f16",
                             splits=32, lognormal_sigma=1.0),
    "bitwidth_sweep": Workload("bitwidth_sweep", 4, batch=32, q_heads=16, kv_heads=16,
                               head_dim=256, seq_len=4096, k_bits=4, v_bits=4, dtype="f16",
                               splits=2, outlier_channels=8, outlier_scale=10.0),
    "two_tier": Workload("two_tier", 5, batch=16, q_heads=16, kv_heads=16, head_dim=128,
                         seq_len=16384, k_bits=8, v_bits=4, dtype="f16", splits=18,
                         near_fraction=0.1, near_splits=5),
    # the llama7b_layer cache with its 256 most recent tokens kept in fp16 (a
    # decode buffer scored in the same pass through the near-tier path)
    "decode_buffer": Workload("decode_buffer", 6, batch=8, q_heads=32, kv_heads=8,
                              head_dim=128, seq_len=8192, k_bits=4, v_bits=4, dtype="f16",
                              splits=4, outlier_channels=4, outlier_scale=20.0,
                              near_fraction=256 / 8192, near_recent=True, near_splits=4),
}


@dataclasses.dataclass
class Inputs:
    wl: Workload
    k: np.ndarray                      # [B, Hkv, T, d]  storage dtype, all T tokens
    v: np.ndarray
    q: np.ndarray                      # [B, Hq, d]
    near_idx: Optional[np.ndarray] = None   # [B, Hkv, near_len] int64 (two_tier)
    far_idx: Optional[np.ndarray] = None    # [B, Hkv, far_len] int64

    def tier(self, which: str):
        """(k, v) of the near or far tier, [B, Hkv, n, d], in token order."""
        idx = self.near_idx if which == "near" else self.far_idx
        take = lambda a: np.take_along_axis(a, idx[..., None], axis=2)
        return take(self.k), take(self.v)


def _np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16}[dtype]


def generate(wl: Workload, seed_offset: int = 0) -> Inputs:
    """Draw one workload's K, V and decode query (see the module recipe)."""
    rng = np.random.default_rng(1000 + wl.index + seed_offset)
    shape = (wl.batch, wl.kv_heads, wl.seq_len, wl.head_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if wl.outlier_channels:
        for h in range(wl.kv_heads):
            ch = rng.choice(wl.head_dim, wl.outlier_channels, replace=False)
            k[:, h, :, ch] *= np.float32(wl.outlier_scale)
    if wl.lognormal_sigma:
        sk = rng.lognormal(0.0, wl.lognormal_sigma, size=(wl.kv_heads, wl.head_dim)).astype(np.float32)
        sv = rng.lognormal(0.0, wl.lognormal_sigma, size=(wl.kv_heads, wl.head_dim)).astype(np.float32)
        k *= sk[None, :, None, :]
        v *= sv[None, :, None, :]
    q = rng.standard_normal((wl.batch, wl.q_heads, wl.head_dim), dtype=np.float32)
    dt = _np_dtype(wl.dtype)
    out = Inputs(wl, k.astype(dt), v.astype(dt), q.astype(dt))
    del k, v
    if wl.near_fraction and wl.near_recent:
        pos = np.arange(wl.seq_len, dtype=np.int64)
        grid = (wl.batch, wl.kv_heads)
        out.near_idx = np.broadcast_to(pos[wl.far_len:], grid + (wl.near_len,)).copy()
        out.far_idx = np.broadcast_to(pos[:wl.far_len], grid + (wl.far_len,)).copy()
    elif wl.near_fraction:
        score = rng.random((wl.batch, wl.kv_heads, wl.seq_len))
        order = np.argsort(-score, axis=-1, kind="stable")
        near = np.sort(order[..., : wl.near_len], axis=-1)
        far = np.sort(order[..., wl.near_len:], axis=-1)
        out.near_idx, out.far_idx = near.astype(np.int64), far.astype(np.int64)
    return out


def new_token(wl: Workload, step: int = 0):
    """One decode step's new key/value ([B, Hkv, 1, d]) with the workload's statistics."""
    rng = np.random.default_rng(5000 + 97 * wl.index + step)
    shape = (wl.batch, wl.kv_heads, 1, wl.head_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    dt = _np_dtype(wl.dtype)
    return k.astype(dt), v.astype(dt)


def qjl_projection(d: int) -> np.ndarray:
    """The Gaussian projection S [m, d] (m = d) of the QJL residual sketch."""
    return np.random.default_rng(QJL_SEED + d).standard_normal((d, d), dtype=np.float32)


@dataclasses.dataclass
class DeviceInputs:
    """Device-resident draws of one workload (torch tensors): the same
    shapes, dtypes, distributions and structure as `generate`, drawn from a
    seeded torch generator on the device instead of numpy on the host, for
    runs where host generation of the larger configurations would dominate
    (the benchmark).  Not bit-identical to `generate`."""
    wl: Workload
    k: object                      # [B, Hkv, T, d] storage dtype
    v: object
    q: object                      # [B, Hq, d]
    near_idx: object = None        # [B, Hkv, near_len] int64
    far_idx: object = None         # [B, Hkv, far_len] int64

    def tier(self, which: str):
        import torch
        idx = self.near_idx if which == "near" else self.far_idx
        g = idx[..., None].expand(-1, -1, -1, self.wl.head_dim)
        return torch.gather(self.k, 2, g).contiguous(), torch.gather(self.v, 2, g).contiguous()


def generate_device(wl: Workload, device, seed_offset: int = 0) -> DeviceInputs:
    """The module recipe, steps 1-6, with torch's generator on `device`
    (seed 1000 + index + seed_offset)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(1000 + wl.index + seed_offset)
    B, Hkv, T, d = wl.batch, wl.kv_heads, wl.seq_len, wl.head_dim
    dt = {"f32": torch.float32, "f16": torch.float16}[wl.dtype]

    k = torch.randn((B, Hkv, T, d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((B, Hkv, T, d), generator=g, device=device, dtype=torch.float32)
    if wl.outlier_channels:
        for h in range(Hkv):
            ch = torch.randperm(d, generator=g, device=device)[: wl.outlier_channels]
            k[:, h, :, ch] *= wl.outlier_scale
    if wl.lognormal_sigma:
        sk = torch.exp(wl.lognormal_sigma * torch.randn((Hkv, d), generator=g, device=device))
        sv = torch.exp(wl.lognormal_sigma * torch.randn((Hkv, d), generator=g, device=device))
        k *= sk[None, :, None, :]
        v *= sv[None, :, None, :]
    k, v = k.to(dt), v.to(dt)
    q = torch.randn((B, wl.q_heads, d), generator=g, device=device, dtype=torch.float32).to(dt)
    out = DeviceInputs(wl, k, v, q)
    if wl.near_fraction and wl.near_recent:
        pos = torch.arange(T, device=device, dtype=torch.int64)
        out.near_idx = pos[wl.far_len:].expand(B, Hkv, -1).contiguous()
        out.far_idx = pos[:wl.far_len].expand(B, Hkv, -1).contiguous()
    elif wl.near_fraction:
        score = torch.rand((B, Hkv, T), generator=g, device=device, dtype=torch.float64)
        order = torch.argsort(-score, dim=-1, stable=True)
        out.near_idx = torch.sort(order[..., : wl.near_len], dim=-1).values
        out.far_idx = torch.sort(order[..., wl.near_len:], dim=-1).values
    return out
