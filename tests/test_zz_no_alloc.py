"""pkv_paged_decode_noalloc (the static split workspace) against
pkv_paged_decode with a caller-allocated workspace: the same bits on every
shape family, on calls in a row whose sizes shrink and grow again (the static
buffer keeps each call's contents; every call must start from clean merge
counters)."""
import numpy as np
import pytest
import torch

import paged_kv_split_amd as pkv
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import dev_tensors, note, problem, run  # noqa: E402


def run_noalloc(w, num_splits=0, heads_per_block=0):
    d = dev_tensors(w)
    p = problem(w, num_splits, heads_per_block)
    out = torch.empty(tuple(d["q"].shape), dtype=torch.bfloat16, device=d["q"].device)
    out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device=d["q"].device)
    P = pkv._ptr
    st = pkv.paged_decode_noalloc_raw(p, P(d["q"]), P(d["k"]), P(d["v"]), P(d["bt"]), P(d["kl"]), P(d["co"]),
                                      P(d["mask"]), P(out), P(out32), int(torch.cuda.current_stream().cuda_stream))
    assert st == pkv.PKV_OK, pkv.status_string(st)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy()


def same_bits(w, splits=0):
    p = problem(w, splits)
    pl = pkv.plan(p)
    note(f"noalloc {w.name} B={w.B} q_len={w.q_len} Hq={w.Hq} Hkv={w.Hkv} D={w.D} splits={pl.splits} "
         f"in-kernel merge={pl.merge_in_kernel} kernels={pl.kernels}")
    a16, a32 = run_noalloc(w, splits)
    r16, r32 = run(w, num_splits=splits)
    assert np.array_equal(a16, r16)
    assert np.array_equal(a32.view(np.uint32), r32.view(np.uint32))
    return pl


def test_noalloc_calls_in_a_row_match_the_workspace_entry_point():
    big = workloads.build("na_big", B=8, q_len=2, Hq=32, Hkv=8, D=128, page_size=32,
                          kv_lens=[4000, 17, 2048, 900, 1, 3000, 333, 1500], seed=5001, causal="last", mask="2d")
    small = workloads.build("na_small", B=3, q_len=1, Hq=8, Hkv=2, D=64, page_size=16,
                            kv_lens=[700, 2100, 5], seed=5002)
    pls = [same_bits(big, 6), same_bits(small, 3), same_bits(big, 6), same_bits(small, 0)]
    assert pls[0].merge_in_kernel and pls[1].merge_in_kernel and pls[0].splits == 6


def test_noalloc_shape_families():
    cases = [
        workloads.tiny(),                                                    # one split: no workspace used
        workloads.build("na_d32", B=4, q_len=1, Hq=8, Hkv=8, D=32, page_size=32, kv_lens=[4096, 100, 2000, 3],
                        seed=5003, mask="2d"),                               # vector kernel, grouped heads
        workloads.build("na_d256", B=2, q_len=3, Hq=16, Hkv=4, D=256, page_size=64, kv_lens=[3000, 800],
                        seed=5004, causal="last"),
        workloads.build("na_prefill", B=1, q_len=200, Hq=16, Hkv=2, D=64, page_size=32, kv_lens=[1500],
                        seed=5005).replace(causal_offset=workloads.CAUSAL_LAST),   # prefill-shaped kernel
        workloads.build("na_many", B=1100, q_len=1, Hq=32, Hkv=8, D=64, page_size=32,
                        kv_lens=[1 + (i * 37) % 300 for i in range(1100)], seed=5006),  # past the counters: combine kernel
    ]
    for w, S in zip(cases, (0, 0, 5, 3, 2)):
        same_bits(w, S)
    assert pkv.plan(problem(cases[-1], 2)).kernels == 2


def test_noalloc_refuses_more_than_its_buffer():
    w = workloads.build("na_over", B=64, q_len=4, Hq=64, Hkv=8, D=128, page_size=32, kv_lens=[64] * 64, seed=5007)
    p = problem(w, 8)
    d = dev_tensors(w)
    out = torch.empty(tuple(d["q"].shape), dtype=torch.bfloat16, device=d["q"].device)
    P = pkv._ptr
    st = pkv.paged_decode_noalloc_raw(p, P(d["q"]), P(d["k"]), P(d["v"]), P(d["bt"]), P(d["kl"]), 0, 0, P(out), 0,
                                      int(torch.cuda.current_stream().cuda_stream))
    assert st == pkv.PKV_ERR_SCRATCH
    # the buffer is still good for the next call
    same_bits(w.replace(name="na_after"), 7)
