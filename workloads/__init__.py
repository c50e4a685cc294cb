"""Seeded synthetic inputs for paged-KV decode attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the fp64 oracle and the HIP path can be fed from
it without sharing code.

Shapes follow the statement of the problem in AstrAI commit d565d44
("csrc/kernels/attn_paged_decode.cu", commit notes on the paged decode
kernels): q[B, q_len, Hq, D] bf16; k_cache, v_cache[num_pages, page_size, Hkv,
D] bf16; block_table[B, max_pages] int32; kv_lens[B] int32; an optional
additive fp32 mask [B, kv_len] (2D) or [B, q_len, kv_len] (3D).

Recipe (all draws from one CPU ``torch.Generator`` per case, in this order):
kv_lens -> page permutation -> q -> k -> v -> key outliers -> mask.
Values are fp32 ``randn`` rounded to bf16 (round-to-nearest-even).  The page
pool holds exactly sum_b ceil(L_b / P) pages plus ``spare_pages``; pages are
assigned to sequences in the order of a random permutation of the pool.
Unused block-table entries are -1.  With ``poison`` the slots no sequence
uses (tails of last pages, spare pages) hold bf16 NaN, so a kernel that reads
them produces NaN.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BF16_NAN = 0x7FC0
CAUSAL_LAST = -2   # causal_offset: each sequence's query tokens are its last keys


@dataclasses.dataclass
class Workload:
    """One paged decode problem, host side (numpy)."""
    name: str
    B: int
    q_len: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    q: np.ndarray            # uint16 bf16 bits [B, q_len, Hq, D]
    k_cache: np.ndarray      # uint16 bf16 bits [num_pages, P, Hkv, D]
    v_cache: np.ndarray      # uint16 bf16 bits [num_pages, P, Hkv, D]
    block_table: np.ndarray  # int32 [B, max_pages]
    kv_lens: np.ndarray      # int32 [B]
    scale: float             # fp32 value
    causal_offset: int = -1
    causal_offsets: Optional[np.ndarray] = None   # int32 [B] or None
    mask: Optional[np.ndarray] = None             # float32, 2D [B, S] or 3D [B, q_len, S]
    num_splits: int = 0
    seed: int = 0
    # Varlen batches: sequence b carries q_lens[b] <= q_len query tokens, the
    # first q_lens[b] of q[b] (the rest are padding, never read).
    q_lens: Optional[np.ndarray] = None           # int32 [B] or None

    @property
    def total_tokens(self) -> int:
        return int(self.q_lens.sum()) if self.q_lens is not None else self.B * self.q_len

    def packed_q(self) -> tuple[np.ndarray, np.ndarray]:
        """(q [T, Hq, D] with sequence b's tokens at rows cu[b] .. cu[b+1]-1,
        cu int32 [B + 1]) for a varlen batch."""
        n = self.q_lens if self.q_lens is not None else np.full(self.B, self.q_len, dtype=np.int32)
        cu = np.zeros(self.B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(n)
        q = np.concatenate([self.q[b, :int(n[b])] for b in range(self.B)], axis=0) if self.B else \
            self.q.reshape(0, self.Hq, self.D)
        return np.ascontiguousarray(q.reshape(-1, self.Hq, self.D)), cu

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_lens.max()) if self.B else 0

    @property
    def mask_strides(self) -> tuple[int, int]:
        """(stride_b, stride_q) of the mask in elements; (0, 0) without one."""
        if self.mask is None:
            return 0, 0
        if self.mask.ndim == 2:
            return int(self.mask.shape[1]), 0
        return int(self.mask.shape[1] * self.mask.shape[2]), int(self.mask.shape[2])

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one call reads: sum_b L_b * Hkv * D * 2 * 2."""
        return int(self.kv_lens.astype(np.int64).sum()) * self.Hkv * self.D * 4

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def to_contiguous(w: Workload, layout: str = "blhd", capacity: Optional[int] = None):
    """The workload's K/V as contiguous caches (no page table): key j of
    sequence b at row j of sequence b's region.  layout "blhd": [B, capacity,
    Hkv, D]; "bhld": [B, Hkv, capacity, D].  capacity defaults to the longest
    sequence; rows at or past kv_lens[b] hold bf16 NaN (never to be read).
    Returns (k, v) as uint16 bf16 bits."""
    cap = int(capacity) if capacity is not None else max(1, w.max_kv_len)
    P = w.page_size
    k = np.full((w.B, cap, w.Hkv, w.D), BF16_NAN, dtype=np.uint16)
    v = np.full((w.B, cap, w.Hkv, w.D), BF16_NAN, dtype=np.uint16)
    for b in range(w.B):
        L = int(w.kv_lens[b])
        for j0 in range(0, L, P):
            n = min(P, L - j0)
            pg = int(w.block_table[b, j0 // P])
            k[b, j0:j0 + n] = w.k_cache[pg, :n]
            v[b, j0:j0 + n] = w.v_cache[pg, :n]
    if layout == "bhld":
        k = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
        v = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    elif layout != "blhd":
        raise ValueError(layout)
    return k, v


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def build(name: str, *, B: int, q_len: int, Hq: int, Hkv: int, D: int,
          page_size: int, kv_lens, seed: int, scale: Optional[float] = None,
          spare_pages: int = 0, causal: str = "off", mask: str = "none",
          mask_p: float = 0.1, outlier_p: float = 0.0, outlier_mult: float = 8.0,
          poison: bool = True, max_pages_per_seq: Optional[int] = None,
          gen: Optional[torch.Generator] = None) -> Workload:
    """Lay out one problem.  ``kv_lens`` is a sequence of ints, or a callable
    ``f(generator) -> sequence`` drawn first from the case generator.

    causal: "off" (offset -1), "last" (per-sequence offsets L_b - q_len), or an
    int (one offset for the whole batch).
    mask: "none", "2d" or "3d" (Bernoulli(mask_p) entries are -inf, else 0).
    """
    g = gen if gen is not None else torch.Generator().manual_seed(seed)
    lens = kv_lens(g) if callable(kv_lens) else kv_lens
    lens = np.asarray(lens, dtype=np.int64).reshape(B)
    pages_per = [(int(L) + page_size - 1) // page_size for L in lens]
    used = int(sum(pages_per))
    num_pages = used + spare_pages
    perm = torch.randperm(max(num_pages, 1), generator=g).numpy()[:num_pages]
    mp = max_pages_per_seq if max_pages_per_seq is not None else max(max(pages_per, default=0), 1)
    bt = np.full((B, mp), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        for p in range(pages_per[b]):
            bt[b, p] = perm[cursor]
            cursor += 1

    q = _bf16_bits(torch.randn(B, q_len, Hq, D, generator=g))
    shape = (max(num_pages, 1), page_size, Hkv, D)
    kf = torch.randn(*shape, generator=g)
    vf = torch.randn(*shape, generator=g)
    if outlier_p > 0:
        sel = torch.rand(shape[:3], generator=g) < outlier_p
        kf[sel] *= outlier_mult
    k = _bf16_bits(kf)
    del kf
    v = _bf16_bits(vf)
    del vf
    if num_pages == 0:
        k = k[:0]
        v = v[:0]

    max_len = int(lens.max()) if B else 0
    m = None
    if mask in ("2d", "3d"):
        cols = max(max_len, 1)
        shp = (B, cols) if mask == "2d" else (B, q_len, cols)
        drop = torch.rand(shp, generator=g) < mask_p
        m = torch.zeros(shp, dtype=torch.float32)
        m[drop] = float("-inf")
        m = m.numpy()
    elif mask != "none":
        raise ValueError(mask)

    if poison:
        # slots no sequence uses: tails of each last page, and spare pages
        owned = np.zeros(num_pages, dtype=bool)
        for b in range(B):
            for p in range(pages_per[b]):
                pg = bt[b, p]
                owned[pg] = True
                lo = int(lens[b]) - p * page_size
                if lo < page_size:
                    k[pg, lo:] = BF16_NAN
                    v[pg, lo:] = BF16_NAN
        k[~owned] = BF16_NAN
        v[~owned] = BF16_NAN

    co = -1
    cos = None
    if causal == "last":
        cos = (lens - q_len).clip(min=0).astype(np.int32)
    elif causal != "off":
        co = int(causal)
    sc = np.float32(scale if scale is not None else 1.0 / math.sqrt(D))
    return Workload(name=name, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=D,
                    page_size=page_size, q=q, k_cache=k, v_cache=v,
                    block_table=bt, kv_lens=lens.astype(np.int32), scale=float(sc),
                    causal_offset=co, causal_offsets=cos, mask=m, seed=seed)


# ---- the five decode shapes ------------------------------------------------

def tiny(seed: int = 1010) -> Workload:
    """B=2, q_len=1, Hq=8, Hkv=2, D=64, page 32, kv_lens {37, 100}, 8 physical
    pages (6 used, 2 spare), no mask, causal off."""
    return build("tiny", B=2, q_len=1, Hq=8, Hkv=2, D=64, page_size=32,
                 kv_lens=[37, 100], seed=seed, spare_pages=2)


def decode_1b(seed: int = 1020, B: int = 8, max_len: int = 2048) -> Workload:
    """1B-model decode shape: B=8, Hq=24, Hkv=4 (G=6), D=64, page 32,
    kv_lens uniform on [128, max_len]."""
    lo = min(128, max_len)
    return build("decode_1b", B=B, q_len=1, Hq=24, Hkv=4, D=64, page_size=32,
                 kv_lens=lambda g: torch.randint(lo, max_len + 1, (B,), generator=g).tolist(),
                 seed=seed)


def sweep(D: int, Hq: int, seed: Optional[int] = None, B: int = 16, L: int = 4096,
          Hkv: int = 8, mask: str = "2d") -> Workload:
    """Head-dim/GQA sweep: B=16, kv_len 4096, page 32, Hkv 8, 10% -inf mask."""
    if seed is None:
        seed = 1030 + 100 * D + Hq
    return build(f"sweep_d{D}_h{Hq}", B=B, q_len=1, Hq=Hq, Hkv=Hkv, D=D,
                 page_size=32, kv_lens=[L] * B, seed=seed, mask=mask)


def long_ctx(seed: int = 1040, B: int = 4, L: int = 32768) -> Workload:
    """Long-context split-KV: B=4, Hq=32, Hkv=8, D=128, page 64, kv_len 32768,
    1% of K vectors scaled by 8."""
    return build("long_ctx", B=B, q_len=1, Hq=32, Hkv=8, D=128, page_size=64,
                 kv_lens=[L] * B, seed=seed, outlier_p=0.01)


def lognormal_lens(B: int, median: float = 1024.0, sigma: float = 1.0,
                   lo: int = 32, hi: int = 8192):
    def draw(g: torch.Generator):
        z = torch.randn(B, generator=g, dtype=torch.float64)
        L = torch.exp(math.log(median) + sigma * z).round().clamp(lo, hi)
        return L.to(torch.int64).tolist()
    return draw


def ragged(seed: int = 1050, B: int = 256, hi: int = 8192) -> Workload:
    """Large ragged batch: B=256, q_len=4, Hq=64, Hkv=8, D=128, page 32,
    kv_lens lognormal (median 1024, sigma 1) clipped to [32, hi], causal
    offsets L_b - 4 per sequence."""
    return build("ragged", B=B, q_len=4, Hq=64, Hkv=8, D=128, page_size=32,
                 kv_lens=lognormal_lens(B, hi=hi), seed=seed, causal="last")


def mixed(seed: int = 1060, B: int = 32, max_q: int = 64, hi: int = 8192) -> Workload:
    """Chunked prefill mixed with decode in one batch: B=32, Hq=32, Hkv=8,
    D=128, page 32; kv_lens lognormal (median 2048, sigma 0.75) clipped to
    [max_q, hi]; then (drawn last) each sequence carries a prefill chunk of
    U[8, max_q] query tokens with probability 1/4, else one decode token; each
    sequence's tokens are its last keys (causal_offset CAUSAL_LAST)."""
    g = torch.Generator().manual_seed(seed)
    w = build("mixed", B=B, q_len=max_q, Hq=32, Hkv=8, D=128, page_size=32,
              kv_lens=lognormal_lens(B, median=2048.0, sigma=0.75, lo=max_q, hi=hi), seed=seed, gen=g)
    chunk = torch.rand(B, generator=g) < 0.25
    n = torch.randint(8, max_q + 1, (B,), generator=g)
    q_lens = torch.where(chunk, n, torch.ones_like(n)).to(torch.int32).numpy()
    return w.replace(q_lens=q_lens, causal_offset=CAUSAL_LAST)


def prefill(seed: int = 1070, B: int = 4, chunk: int = 512, L: int = 4096) -> Workload:
    """Chunked prefill: B=4 sequences of L=4096 keys whose last 512 are a new
    chunk of query tokens (causal_offset CAUSAL_LAST), Hq=32, Hkv=8, D=128,
    page 32."""
    w = build("prefill", B=B, q_len=chunk, Hq=32, Hkv=8, D=128, page_size=32, kv_lens=[L] * B, seed=seed)
    return w.replace(causal_offset=CAUSAL_LAST)


def varlen(name: str, *, q_lens, seed: int, **kw) -> Workload:
    """``build`` with q_len = max(q_lens) (at least 1) and per-sequence query
    token counts q_lens (drawn from nothing: given); causal "lastv" sets
    causal_offset CAUSAL_LAST, the other causal modes are build's."""
    q_lens = np.asarray(q_lens, dtype=np.int32)
    causal = kw.pop("causal", "off")
    ql = max(1, int(q_lens.max()) if q_lens.size else 1)
    w = build(name, q_len=ql, seed=seed, causal="off" if causal == "lastv" else causal, **kw)
    if causal == "lastv":
        w = w.replace(causal_offset=CAUSAL_LAST)
    return w.replace(q_lens=q_lens)


CONFIGS = {
    "tiny": tiny,
    "decode_1b": decode_1b,
    "long_ctx": long_ctx,
    "ragged": ragged,
    "mixed": mixed,
    "prefill": prefill,
}
