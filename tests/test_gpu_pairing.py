"""GPU parity of head pairing: at head_dim 32 the library reads two adjacent
kv heads as one head of 64 columns (each query row's q zero outside its own
head's half, its output that half).  Every paired plan is checked against the
fp64 oracle, and against the unpaired plan of the same problem (forced one kv
head per workgroup) within the fp32 bound: a row's result is its own head's,
whatever the pairing."""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import check, note, paired, run, run_contiguous, run_varlen, sub_batch  # noqa: E402

CASES = [
    # one query head per kv head (vector kernel, two rows of 64 columns)
    dict(B=3, q_len=1, Hq=8, Hkv=8, D=32, page_size=32, kv_lens=[1, 300, 4097]),
    dict(B=2, q_len=1, Hq=16, Hkv=16, D=32, page_size=8, kv_lens=[1000, 33], mask="2d"),
    dict(B=2, q_len=1, Hq=2, Hkv=2, D=32, page_size=1, kv_lens=[77, 5]),
    # matrix-core kernel: 4, 8 and 16 rows per pair
    dict(B=3, q_len=1, Hq=16, Hkv=8, D=32, page_size=16, kv_lens=[70, 513, 1]),
    dict(B=2, q_len=1, Hq=32, Hkv=8, D=32, page_size=64, kv_lens=[3000, 129], mask="2d"),
    dict(B=3, q_len=1, Hq=64, Hkv=8, D=32, page_size=32, kv_lens=[2048, 77, 1000], mask="2d"),
    dict(B=2, q_len=2, Hq=32, Hkv=8, D=32, page_size=32, kv_lens=[900, 60], causal="last", mask="3d"),
    dict(B=2, q_len=4, Hq=4, Hkv=2, D=32, page_size=16, kv_lens=[500, 4], causal=1),
    dict(B=2, q_len=8, Hq=4, Hkv=4, D=32, page_size=32, kv_lens=[300, 20], causal="last"),
]


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_paired_against_oracle_and_unpaired(i, splits):
    w = workloads.build(f"pair{i}", seed=4100 + i, spare_pages=2, **CASES[i])
    assert paired(w), "the case should take head pairing"
    note(f"pairing case {i} {CASES[i]} splits={splits}")
    o16, o32 = run(w, num_splits=splits)
    ref = oracle.decode(w)
    check(o16, o32, ref, f"paired {i}")
    u16, u32 = run(w, num_splits=splits, heads_per_block=1)      # forced grouping: never paired
    check(u16, u32, ref, f"unpaired {i}")
    assert np.abs(o32.astype(np.float64) - u32).max() <= 2e-3


@pytest.mark.parametrize("i", [0, 4, 6])
def test_paired_blhd_equals_paged_and_bhld_matches_oracle(i):
    """[B, L, Hkv, D] holds a key's head slices side by side, so it pairs like the
    paged cache (same plan, same bits); [B, Hkv, L, D] does not pair."""
    w = workloads.build(f"pairc{i}", seed=4200 + i, **CASES[i])
    p16, p32 = run(w)
    c16, c32, _, _ = run_contiguous(w, "blhd")
    assert np.array_equal(c16, p16) and np.array_equal(c32.view(np.uint32), p32.view(np.uint32))
    h16, h32, k, v = run_contiguous(w, "bhld")
    check(h16, h32, oracle.decode_contiguous(w, k, v, "bhld"), "bhld")


def test_paired_varlen_and_per_sequence_offsets():
    """A varlen batch (its own token count per sequence, causal at each end) on a
    paired plan, against the oracle's varlen form."""
    w = workloads.varlen("pairvl", q_lens=[2, 1, 0, 2], seed=4300, B=4, Hq=32, Hkv=8, D=32, page_size=32,
                         kv_lens=[700, 64, 5, 2000], causal="lastv", mask="2d")
    note("pairing varlen")
    o16, o32 = run_varlen(w)
    check(o16, o32, oracle.decode_varlen(w).reshape(o32.shape), "paired varlen")


@pytest.mark.parametrize("Hq", [8, 32, 64])
def test_paired_sweep_full_size_every_sequence_sampled_heads(Hq):
    """The D = 32 sweep shapes (B = 16 x 4096 keys, 2D mask) at the bench's plan:
    four sequences, all their rows."""
    w = workloads.sweep(32, Hq)
    assert paired(w)
    out16, out32 = run(w)
    seqs = [0, 5, 10, 15]
    check(out16[seqs], out32[seqs], oracle.decode(sub_batch(w, seqs)), f"sweep d32 h{Hq}")


def test_odd_kv_heads_are_not_paired():
    w = workloads.build("pairodd", B=2, q_len=1, Hq=6, Hkv=3, D=32, page_size=32, kv_lens=[500, 31], seed=4400)
    assert not paired(w)
    o16, o32 = run(w)
    check(o16, o32, oracle.decode(w), "odd Hkv")
