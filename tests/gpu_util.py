"""Helpers shared by the GPU tests: move a host workload to the device, call
the library through its C ABI, and compare against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_split_amd as pkv

FP32_TOL = 2e-3       # max |out_f32 - ref|
BF16_TOL = 1e-2       # max |out_bf16 - ref|, ref the unrounded fp64 value


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensors(w, device="cuda:0"):
    d = torch.device(device)

    def t(a, dtype):
        return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).to(d)

    return dict(
        q=t(w.q.view(np.int16), torch.bfloat16),
        k=t(w.k_cache.view(np.int16), torch.bfloat16),
        v=t(w.v_cache.view(np.int16), torch.bfloat16),
        bt=t(w.block_table, torch.int32),
        kl=t(w.kv_lens, torch.int32),
        co=None if w.causal_offsets is None else t(w.causal_offsets, torch.int32),
        mask=None if w.mask is None else t(w.mask, torch.float32),
    )


def problem(w, num_splits=0, heads_per_block=0):
    msb, msq = w.mask_strides
    return pkv.make_problem(batch=w.B, q_len=w.q_len, num_q_heads=w.Hq, num_kv_heads=w.Hkv,
                            head_dim=w.D, page_size=w.page_size, num_pages=w.num_pages,
                            max_pages_per_seq=w.max_pages_per_seq, max_kv_len=w.max_kv_len,
                            scale=w.scale, causal_offset=w.causal_offset, num_splits=num_splits,
                            mask_stride_b=msb, mask_stride_q=msq, heads_per_block=heads_per_block)


def paired(w, heads_per_block=0) -> bool:
    """Whether the library's paged plan pairs kv heads (pkv_plan_info.paired_heads):
    the [B, Hkv, L, D] contiguous layout never does, so its bits match the paged
    call's only when this is False."""
    return bool(pkv.plan(problem(w, heads_per_block=heads_per_block)).paired_heads)


def run(w, d=None, num_splits=0, stream=None, sync=True, heads_per_block=0):
    """Call pkv_paged_decode; return (out_bf16 bits uint16, out_f32 float32) as numpy."""
    if d is None:
        d = dev_tensors(w)
    p = problem(w, num_splits, heads_per_block)
    out = torch.empty(tuple(d["q"].shape), dtype=torch.bfloat16, device=d["q"].device)
    out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device=d["q"].device)
    pkv.paged_decode(d["q"], d["k"], d["v"], d["bt"], d["kl"], scale=w.scale,
                     causal_offset=w.causal_offset, causal_offsets=d["co"], mask=d["mask"],
                     out=out, out_f32=out32, stream=stream, problem=p)
    if sync:
        torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy()


def run_contiguous(w, layout, num_splits=0, heads_per_block=0, capacity=None, sync=True):
    """pkv_contiguous_decode on the workload's keys laid out contiguously
    (workloads.to_contiguous); returns (out_bf16 bits, out_f32, k, v) with the
    host K/V arrays used."""
    k, v = __import__("workloads").to_contiguous(w, layout, capacity)
    d = dev_tensors(w)
    dev = d["q"].device
    kt = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).to(dev)
    vt = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev)
    out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device=dev)
    out = pkv.contiguous_decode(d["q"], kt, vt, d["kl"], layout=layout, scale=w.scale,
                                causal_offset=w.causal_offset, causal_offsets=d["co"], mask=d["mask"],
                                num_splits=num_splits, max_kv_len=w.max_kv_len,
                                heads_per_block=heads_per_block, out_f32=out32)
    if sync:
        torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy(), k, v


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (independent host version)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bound(ref: np.ndarray) -> np.ndarray:
    """Per-element bf16 bound: 1e-2, or half a bf16 ulp of ref plus the fp32
    bound where bf16 quantisation alone exceeds 1e-2 (|ref| >= 4)."""
    mag = np.abs(ref)
    e = np.floor(np.log2(np.maximum(mag, 1e-30)))
    half_ulp = np.exp2(e - 8)
    return np.maximum(BF16_TOL, half_ulp + FP32_TOL)


def check(out16: np.ndarray, out32: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    """Assert the tolerances; return the measured errors."""
    got16 = bf16_bits_to_f64(out16)
    got32 = out32.astype(np.float64)
    assert np.isfinite(got32).all(), f"{what}: non-finite fp32 output"
    e32 = np.abs(got32 - ref)
    e16 = np.abs(got16 - ref)
    err32 = float(e32.max()) if e32.size else 0.0
    err16 = float(e16.max()) if e16.size else 0.0
    assert err32 <= FP32_TOL, f"{what}: fp32 max err {err32} at {np.unravel_index(e32.argmax(), e32.shape)}"
    bound = bf16_bound(ref)
    bad = e16 > bound
    assert not bad.any(), f"{what}: bf16 err {err16} beyond bound at {np.argwhere(bad)[:5]}"
    assert np.array_equal(out16, rne_bf16(out32)), f"{what}: out_bf16 != RNE(out_f32)"
    relaxed = int((e16 > BF16_TOL).sum())
    return dict(err32=err32, err16=err16, relaxed=relaxed)


def sub_batch(w, seqs):
    """The same problem restricted to sequences `seqs` (pools shared), for
    sampled oracle checks at full size."""
    seqs = np.asarray(seqs)
    return w.replace(
        B=len(seqs), q=w.q[seqs].copy(), block_table=w.block_table[seqs].copy(),
        kv_lens=w.kv_lens[seqs].copy(),
        causal_offsets=None if w.causal_offsets is None else w.causal_offsets[seqs].copy(),
        mask=None if w.mask is None else w.mask[seqs].copy())


def run_varlen(w, num_splits=0, heads_per_block=0, sync=True):
    """pkv_paged_decode_varlen on the workload's packed tokens (w.q_lens, or
    q_len per sequence); returns (out_bf16 bits [T, Hq, D], out_f32)."""
    d = dev_tensors(w)
    dev = d["q"].device
    qp, cu = w.packed_q()
    q = torch.from_numpy(qp.view(np.int16)).view(torch.bfloat16).to(dev)
    cu_t = torch.from_numpy(cu).to(dev)
    out32 = torch.empty(tuple(q.shape), dtype=torch.float32, device=dev)
    out = pkv.paged_decode_varlen(q, d["k"], d["v"], d["bt"], d["kl"], cu_t, max_q_len=w.q_len, scale=w.scale,
                                  causal_offset=w.causal_offset, causal_offsets=d["co"], mask=d["mask"],
                                  num_splits=num_splits, max_kv_len=w.max_kv_len,
                                  heads_per_block=heads_per_block, out_f32=out32)
    if sync:
        torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy()
