"""fp64 CPU oracle for paged-KV decode attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and the
two share no code.

Two independent implementations of the same definition live here:

* ``decode`` / ``partial`` / ``combine`` -- ctypes wrappers over
  ``pkv_oracle.c`` (fp64, OpenMP over output rows, serial over keys);
* ``bruteforce_decode`` -- numpy, tiny inputs only: gather every sequence's
  pages into contiguous K/V, repeat kv heads up to the query heads, build the
  full score tensor with a separate visibility matrix, then a naive softmax
  and a dense matmul with V.

Operation (AstrAI commit d565d44, "csrc/kernels/attn_paged_decode.cu", commit
notes on the paged split-KV decode kernels): every query row (b, i, h)
attends over the keys of sequence b addressed through its page table; GQA
head sharing; optional additive mask; unified causal_offset (-1 = off, c >= 0
= absolute position of query token 0, so token i sees keys j <= c + i);
split-KV partials merged by a log-sum-exp combine.

``decode_varlen`` covers batches whose sequences carry different numbers of
query tokens (chunked prefill and decode together, as in the same commit
notes: prefill and decode kernels over one paged cache), one sequence at a
time by the definition above, and the causal mode in which each sequence's
tokens are its last keys.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile pkv_oracle.c with gcc (-O2, OpenMP) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        common = [I, I, I, I, I, I, I, I, P, P, P, P, P, ctypes.c_float, I, P, P, I64, I64]
        lib.pkv_oracle_decode.argtypes = common + [P, I]
        lib.pkv_oracle_decode.restype = I
        lib.pkv_oracle_partial.argtypes = common + [I, I, P, P, P, I]
        lib.pkv_oracle_partial.restype = I
        lib.pkv_oracle_combine.argtypes = [I64, I, I, P, P, P, P]
        lib.pkv_oracle_combine.restype = I
        lib.pkv_oracle_max_threads.argtypes = []
        lib.pkv_oracle_max_threads.restype = I
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


CAUSAL_LAST = -2


def _common_args(w):
    if getattr(w, "q_lens", None) is not None or w.causal_offset < -1:
        raise ValueError("varlen batches and causal_offset CAUSAL_LAST go through decode_varlen")
    q = np.ascontiguousarray(w.q, dtype=np.uint16)
    k = np.ascontiguousarray(w.k_cache, dtype=np.uint16)
    v = np.ascontiguousarray(w.v_cache, dtype=np.uint16)
    bt = np.ascontiguousarray(w.block_table, dtype=np.int32)
    kl = np.ascontiguousarray(w.kv_lens, dtype=np.int32)
    co = None if w.causal_offsets is None else np.ascontiguousarray(w.causal_offsets, dtype=np.int32)
    mk = None if w.mask is None else np.ascontiguousarray(w.mask, dtype=np.float32)
    msb, msq = w.mask_strides
    keep = (q, k, v, bt, kl, co, mk)
    args = [w.B, w.q_len, w.Hq, w.Hkv, w.D, w.page_size, w.num_pages,
            w.max_pages_per_seq, _ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(kl),
            ctypes.c_float(w.scale), w.causal_offset, _ptr(co), _ptr(mk), msb, msq]
    return keep, args


def decode(w, threads: int = 0) -> np.ndarray:
    """fp64 output [B, q_len, Hq, D] of the full decode (all visible keys)."""
    lib = _load()
    keep, args = _common_args(w)
    out = np.zeros((w.B, w.q_len, w.Hq, w.D), dtype=np.float64)
    rc = lib.pkv_oracle_decode(*args, _ptr(out), threads)
    if rc:
        raise RuntimeError(f"pkv_oracle_decode failed: {rc}")
    del keep
    return out


def partial(w, j_begin: int, j_end: int, threads: int = 0):
    """Split partial over keys [j_begin, j_end): (o, m, l) with o normalised,
    m the max score (natural log units), l = sum exp(s - m)."""
    lib = _load()
    keep, args = _common_args(w)
    o = np.zeros((w.B, w.q_len, w.Hq, w.D), dtype=np.float64)
    m = np.zeros((w.B, w.q_len, w.Hq), dtype=np.float64)
    l = np.zeros((w.B, w.q_len, w.Hq), dtype=np.float64)
    rc = lib.pkv_oracle_partial(*args, j_begin, j_end, _ptr(o), _ptr(m), _ptr(l), threads)
    if rc:
        raise RuntimeError(f"pkv_oracle_partial failed: {rc}")
    del keep
    return o, m, l


def combine(o_part: np.ndarray, m_part: np.ndarray, l_part: np.ndarray) -> np.ndarray:
    """Log-sum-exp merge.  o_part [rows, S, D], m/l [rows, S] -> [rows, D]."""
    lib = _load()
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    m_part = np.ascontiguousarray(m_part, dtype=np.float64)
    l_part = np.ascontiguousarray(l_part, dtype=np.float64)
    rows, S, D = o_part.shape
    out = np.zeros((rows, D), dtype=np.float64)
    rc = lib.pkv_oracle_combine(rows, S, D, _ptr(o_part), _ptr(m_part), _ptr(l_part), _ptr(out))
    if rc:
        raise RuntimeError(f"pkv_oracle_combine failed: {rc}")
    return out


def decode_contiguous(w, k: np.ndarray, v: np.ndarray, layout: str = "blhd", threads: int = 0) -> np.ndarray:
    """fp64 output for contiguous K/V (AstrAI paged-decode commit notes: a
    contiguous and a paged K/V addressing policy for the same decode, and the
    "bhld"/"blhd" layouts): key j of sequence b is row j of sequence b's
    region, k / v [B, cap, Hkv, D] ("blhd") or [B, Hkv, cap, D] ("bhld").
    That is the paged definition with one page of cap keys per sequence and
    page b holding sequence b, which is how it is evaluated here; the other
    fields of `w` (q, kv_lens, mask, causal offsets, scale) are used as given."""
    if layout == "bhld":
        k = k.transpose(0, 2, 1, 3)
        v = v.transpose(0, 2, 1, 3)
    elif layout != "blhd":
        raise ValueError(layout)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    B, cap = k.shape[0], k.shape[1]
    bt = np.arange(B, dtype=np.int32).reshape(B, 1)
    return decode(w.replace(k_cache=k, v_cache=v, block_table=bt, page_size=cap), threads)


def decode_varlen(w, threads: int = 0) -> np.ndarray:
    """fp64 output [T, Hq, D] of a batch whose sequence b carries n_b query
    tokens (w.q_lens, or q_len each when None; its tokens are w.q[b, :n_b]),
    rows in sequence order (T = sum n_b).

    Reading: each sequence is an independent decode problem with q_len = n_b,
    evaluated here by the fixed-length definition one sequence at a time.
    With causal_offset CAUSAL_LAST token i of sequence b sits at position
    L_b - n_b + i and sees keys j <= L_b - n_b + i; a token at a negative
    position (only when n_b > L_b) sees no key and its row is zero, as for
    any row with no visible key.  A per-sequence causal_offsets[b] or a fixed
    causal_offset >= 0 is the position of the sequence's token 0, as for the
    fixed-length batch."""
    n_all = w.q_lens if w.q_lens is not None else np.full(w.B, w.q_len, dtype=np.int32)
    outs = []
    for b in range(w.B):
        n = int(n_all[b])
        if n == 0:
            continue
        L = int(w.kv_lens[b])
        lead = 0
        if w.causal_offsets is not None:
            co = int(w.causal_offsets[b])
        elif w.causal_offset == CAUSAL_LAST:
            co = L - n
            if co < 0:
                lead, co = -co, 0
        else:
            co = int(w.causal_offset)
        out = np.zeros((n, w.Hq, w.D), dtype=np.float64)
        if lead < n:
            m = None
            if w.mask is not None:
                m = w.mask[b:b + 1] if w.mask.ndim == 2 else w.mask[b:b + 1, lead:n]
            sub = w.replace(B=1, q_len=n - lead, q=w.q[b:b + 1, lead:n], block_table=w.block_table[b:b + 1],
                            kv_lens=w.kv_lens[b:b + 1], causal_offset=co, causal_offsets=None, mask=m,
                            q_lens=None)
            out[lead:] = decode(sub, threads)[0]
        outs.append(out)
    if not outs:
        return np.zeros((0, w.Hq, w.D), dtype=np.float64)
    return np.concatenate(outs, axis=0)


def max_threads() -> int:
    return int(_load().pkv_oracle_max_threads())


# ---------------------------------------------------------------------------
# Brute force (numpy, fp64): a separate code path for tiny inputs.

def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bruteforce_varlen(w) -> np.ndarray:
    """Varlen brute force, token by token: [T, Hq, D].  Each query token is
    given its absolute position explicitly (CAUSAL_LAST: L_b - n_b + i), its
    visible keys are listed, and a naive softmax over them weights V."""
    G = w.Hq // w.Hkv
    P = w.page_size
    n_all = w.q_lens if w.q_lens is not None else np.full(w.B, w.q_len, dtype=np.int32)
    q = bf16_bits_to_f64(w.q)
    rows = []
    for b in range(w.B):
        n, L = int(n_all[b]), int(w.kv_lens[b])
        keys = [(int(w.block_table[b, j // P]), j % P) for j in range(L)]
        for i in range(n):
            if w.causal_offsets is not None:
                pos = int(w.causal_offsets[b]) + i if w.causal_offsets[b] >= 0 else None
            elif w.causal_offset == CAUSAL_LAST:
                pos = L - n + i
            else:
                pos = w.causal_offset + i if w.causal_offset >= 0 else None
            row = np.zeros((w.Hq, w.D))
            for h in range(w.Hq):
                kh = h // G
                s, vs = [], []
                for j, (pg, sl) in enumerate(keys):
                    if pos is not None and j > pos:
                        continue
                    sc = float(np.dot(q[b, i, h], bf16_bits_to_f64(w.k_cache[pg, sl, kh]))) * float(np.float32(w.scale))
                    if w.mask is not None:
                        sc += float(w.mask[b, j] if w.mask.ndim == 2 else w.mask[b, i, j])
                    if np.isfinite(sc):
                        s.append(sc)
                        vs.append(bf16_bits_to_f64(w.v_cache[pg, sl, kh]))
                if s:
                    e = np.exp(np.array(s) - max(s))
                    row[h] = (e / e.sum()) @ np.array(vs)
            rows.append(row)
    return np.array(rows).reshape(-1, w.Hq, w.D)


def bruteforce_decode(w) -> np.ndarray:
    """Gather -> repeat heads -> full scores + visibility -> naive softmax -> matmul."""
    B, ql, Hq, Hkv, D, P = w.B, w.q_len, w.Hq, w.Hkv, w.D, w.page_size
    G = Hq // Hkv
    q = bf16_bits_to_f64(w.q)                     # [B, ql, Hq, D]
    out = np.zeros((B, ql, Hq, D))
    for b in range(B):
        L = int(w.kv_lens[b])
        if L == 0:
            continue
        npg = (L + P - 1) // P
        pages = [int(w.block_table[b, p]) for p in range(npg)]
        Kc = np.concatenate([bf16_bits_to_f64(w.k_cache[pg]) for pg in pages], axis=0)[:L]
        Vc = np.concatenate([bf16_bits_to_f64(w.v_cache[pg]) for pg in pages], axis=0)[:L]
        # repeat kv heads so query head h sees kv head h // G
        Kr = np.repeat(Kc, G, axis=1)             # [L, Hq, D]
        Vr = np.repeat(Vc, G, axis=1)
        scores = np.einsum("ihd,jhd->hij", q[b], Kr) * float(np.float32(w.scale))  # [Hq, ql, L]
        if w.mask is not None:
            mrow = w.mask[b, :L] if w.mask.ndim == 2 else w.mask[b, :, :L]
            scores = scores + np.asarray(mrow, dtype=np.float64)
        visible = np.ones((ql, L), dtype=bool)
        c = int(w.causal_offsets[b]) if w.causal_offsets is not None else int(w.causal_offset)
        if c >= 0:
            for i in range(ql):
                visible[i, c + i + 1:] = False
        visible = np.broadcast_to(visible, scores.shape) & np.isfinite(scores)
        for h in range(Hq):
            for i in range(ql):
                sel = visible[h, i]
                if not sel.any():
                    continue
                s = scores[h, i, sel]
                e = np.exp(s - s.max())
                p = e / e.sum()
                out[b, i, h] = p @ Vr[sel, h, :]
    return out
