"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Tolerances: max |out_f32 - ref| <= 2e-3, max |out_bf16 - ref| <= 1e-2 (half a
bf16 ulp + 2e-3 where |ref| >= 4, since bf16 rounding alone exceeds 1e-2
there), out_bf16 == RNE(out_f32) bit for bit.  Small cases are checked on every
output; the full-size decode shapes on every output where the oracle is quick
and on sampled sequences (all their rows) where it is not.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import check, note, run, sub_batch  # noqa: E402


def compare(w, num_splits=0, seqs=None, heads_per_block=0):
    note(f"case {w.name} B={w.B} q_len={w.q_len} Hq={w.Hq} Hkv={w.Hkv} D={w.D} P={w.page_size} "
         f"maxL={w.max_kv_len} splits={num_splits} heads_per_block={heads_per_block} seed={w.seed}")
    out16, out32 = run(w, num_splits=num_splits, heads_per_block=heads_per_block)
    if seqs is None:
        ref = oracle.decode(w)
        return check(out16, out32, ref, w.name)
    ref = oracle.decode(sub_batch(w, seqs))
    return check(out16[seqs], out32[seqs], ref, w.name)


# ---- the five decode shapes -------------------------------------------------

def test_tiny():
    compare(workloads.tiny())


@pytest.mark.parametrize("splits", [0, 1, 3, 8])
def test_tiny_forced_splits(splits):
    compare(workloads.tiny(), num_splits=splits)


def test_decode_1b_full():
    compare(workloads.decode_1b())


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("Hq", [8, 32, 64])
def test_sweep_full_size_sampled(D, Hq):
    w = workloads.sweep(D, Hq)
    compare(w, seqs=[0, 7, 15])


@pytest.mark.parametrize("splits", [0, 1, 64])
def test_long_ctx_full(splits):
    compare(workloads.long_ctx(), num_splits=splits)


def test_ragged_full_size_sampled():
    w = workloads.ragged()
    L = w.kv_lens
    seqs = sorted({int(L.argmax()), int(L.argmin()), 0, 1, 100, 255})
    compare(w, seqs=seqs)


# ---- smaller cases that span several tiles and a ragged tail -----------------

SMALL = [
    dict(B=3, q_len=1, Hq=8, Hkv=8, D=32, page_size=32, kv_lens=[1, 300, 517]),
    dict(B=3, q_len=1, Hq=32, Hkv=8, D=64, page_size=16, kv_lens=[65, 255, 0]),
    dict(B=2, q_len=1, Hq=64, Hkv=8, D=128, page_size=64, kv_lens=[700, 33]),
    dict(B=2, q_len=1, Hq=16, Hkv=2, D=256, page_size=32, kv_lens=[257, 130]),
    dict(B=4, q_len=1, Hq=24, Hkv=4, D=64, page_size=32, kv_lens=[128, 129, 2047, 5]),   # G=6
    dict(B=2, q_len=3, Hq=6, Hkv=2, D=128, page_size=8, kv_lens=[100, 41], causal="last"),  # R=9: one 16-row MFMA block
    dict(B=2, q_len=4, Hq=64, Hkv=8, D=128, page_size=32, kv_lens=[300, 64], causal="last"),  # R=32
    dict(B=2, q_len=2, Hq=4, Hkv=1, D=32, page_size=1, kv_lens=[77, 5], causal=70),
    dict(B=2, q_len=1, Hq=2, Hkv=2, D=64, page_size=256, kv_lens=[600, 1]),
    dict(B=3, q_len=2, Hq=8, Hkv=2, D=64, page_size=32, kv_lens=[200, 90, 13], mask="3d"),
    dict(B=3, q_len=1, Hq=16, Hkv=4, D=128, page_size=32, kv_lens=[400, 333, 1], mask="2d", mask_p=0.5),
    dict(B=2, q_len=1, Hq=8, Hkv=1, D=256, page_size=64, kv_lens=[1000, 999], outlier_p=0.05),
    # rows that fill matrix-core tiles (R = G * q_len > 8)
    dict(B=2, q_len=2, Hq=8, Hkv=1, D=64, page_size=16, kv_lens=[300, 17]),                   # R=16
    dict(B=2, q_len=3, Hq=16, Hkv=1, D=128, page_size=32, kv_lens=[333, 70], causal="last"),  # R=48
    dict(B=2, q_len=1, Hq=32, Hkv=2, D=256, page_size=32, kv_lens=[500, 64]),                 # R=16, D=256
    dict(B=2, q_len=4, Hq=16, Hkv=4, D=32, page_size=8, kv_lens=[200, 5], mask="3d", causal="last"),
    dict(B=1, q_len=2, Hq=64, Hkv=4, D=128, page_size=64, kv_lens=[777], mask="2d", mask_p=0.3),  # R=32
    dict(B=3, q_len=1, Hq=24, Hkv=2, D=64, page_size=32, kv_lens=[90, 1, 0], outlier_p=0.05),  # R=12
    # two rows per kv head (VALU kernel with two rows) and three (matrix-core, mostly padding)
    dict(B=3, q_len=1, Hq=16, Hkv=8, D=32, page_size=16, kv_lens=[70, 513, 1]),                # R=2
    dict(B=2, q_len=2, Hq=4, Hkv=4, D=256, page_size=32, kv_lens=[300, 9], causal="last"),     # R=2
    dict(B=2, q_len=1, Hq=12, Hkv=4, D=64, page_size=64, kv_lens=[1000, 257], mask="2d"),      # R=3
    # three and four rows per kv head at D = 256 (VALU kernel, four rows per workgroup)
    dict(B=3, q_len=1, Hq=32, Hkv=8, D=256, page_size=32, kv_lens=[700, 1, 2049], mask="2d"),  # R=4
    dict(B=2, q_len=3, Hq=2, Hkv=2, D=256, page_size=16, kv_lens=[300, 4], causal="last",
         mask="3d"),                                                                           # R=3
    dict(B=2, q_len=2, Hq=16, Hkv=8, D=256, page_size=1, kv_lens=[130, 77], causal=60),        # R=4
]


@pytest.mark.parametrize("i", range(len(SMALL)))
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_small_cases(i, splits):
    kw = dict(SMALL[i])
    w = workloads.build(f"small{i}", seed=2000 + i, spare_pages=3, **kw)
    compare(w, num_splits=splits)


@pytest.mark.parametrize("i,hpb", [(i, h) for i in range(len(SMALL)) for h in (1, 2, 4, 8)
                                   if SMALL[i]["Hkv"] % h == 0 and (h < 8 or SMALL[i]["D"] <= 64)])
@pytest.mark.parametrize("splits", [1, 5])
def test_small_cases_heads_per_block(i, hpb, splits):
    """Every kv-head grouping of a workgroup (one to four heads with one or
    more waves per head; four heads from three rows on, and eight heads, in
    the shared-tile kernel), each dividing the case's kv heads, on the same
    cases."""
    kw = dict(SMALL[i])
    w = workloads.build(f"small{i}", seed=2000 + i, spare_pages=3, **kw)
    compare(w, num_splits=splits, heads_per_block=hpb)


@pytest.mark.parametrize("hpb", [1, 2, 4])
def test_sweep_heads_per_block_sampled(hpb):
    """Full-size sweep shapes (VALU and matrix-core kernels) with each grouping."""
    for D, Hq in ((64, 8), (32, 16), (128, 64), (256, 32)):
        w = workloads.sweep(D, Hq)
        compare(w, seqs=[0, 15], heads_per_block=hpb)


# ---- the shared-tile kernel (4 or 8 kv heads per workgroup) ----------------
# Whole head-group rows of each key loaded by the workgroup into shared
# tiles of 16 to 64 keys: pages smaller than a tile (per-key page lookups),
# page size 1, 2D and 3D masks, causal limits, 16- and 32-row blocks, empty
# and one-key sequences, one row per kv head.
GROUP_CASES = [
    dict(B=3, q_len=1, Hq=64, Hkv=8, D=32, page_size=32, kv_lens=[4096, 77, 1000], mask="2d"),      # R=8
    dict(B=2, q_len=4, Hq=32, Hkv=8, D=64, page_size=8, kv_lens=[700, 33], causal="last", mask="3d",
         mask_p=0.2),                                                                                 # R=16
    dict(B=2, q_len=4, Hq=64, Hkv=8, D=128, page_size=16, kv_lens=[3000, 5], causal="last"),         # R=32
    dict(B=3, q_len=2, Hq=24, Hkv=8, D=64, page_size=64, kv_lens=[1500, 64, 0]),                    # R=6
    dict(B=2, q_len=1, Hq=8, Hkv=8, D=32, page_size=1, kv_lens=[300, 2]),                           # R=1
    dict(B=2, q_len=3, Hq=16, Hkv=4, D=128, page_size=32, kv_lens=[1000, 129], causal="last",
         mask="2d", mask_p=0.3),                                                                      # R=12
    dict(B=2, q_len=1, Hq=16, Hkv=8, D=64, page_size=16, kv_lens=[2049, 1], outlier_p=0.05),        # R=2
    dict(B=2, q_len=8, Hq=32, Hkv=8, D=32, page_size=32, kv_lens=[900, 60], causal="last",
         mask="2d", mask_p=0.1),                                                                      # R=32
]


@pytest.mark.parametrize("i,hpb", [(i, h) for i in range(len(GROUP_CASES)) for h in (4, 8)
                                   if GROUP_CASES[i]["Hkv"] % h == 0 and (h < 8 or GROUP_CASES[i]["D"] <= 64)
                                   and (h == 8 or GROUP_CASES[i]["Hq"] // GROUP_CASES[i]["Hkv"]
                                        * GROUP_CASES[i]["q_len"] > 2)])
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_shared_tile_cases(i, hpb, splits):
    import paged_kv_split_amd as pkv
    from gpu_util import problem
    kw = dict(GROUP_CASES[i])
    w = workloads.build(f"group{i}", seed=2400 + i, spare_pages=3, **kw)
    assert pkv.plan(problem(w, splits, hpb)).kernel == pkv.PKV_KERNEL_SHARED_TILE
    compare(w, num_splits=splits, heads_per_block=hpb)


@pytest.mark.parametrize("D,Hq,hpb", [(32, 8, 8), (32, 64, 8), (32, 32, 4), (64, 8, 8), (64, 64, 8), (64, 32, 4),
                                      (128, 64, 4), (128, 32, 4)])
def test_sweep_shared_tile_sampled(D, Hq, hpb):
    """Full-size sweep shapes in the shared-tile kernel."""
    compare(workloads.sweep(D, Hq), seqs=[0, 7, 15], heads_per_block=hpb)


def test_long_ctx_and_ragged_shared_tile_sampled():
    compare(workloads.long_ctx(), seqs=[0, 3], heads_per_block=4)
    compare(workloads.long_ctx(), num_splits=64, seqs=[1], heads_per_block=4)
    w = workloads.ragged()
    L = w.kv_lens
    compare(w, seqs=sorted({int(L.argmax()), int(L.argmin()), 0, 100, 255}), heads_per_block=4)


def test_all_masked_and_empty_rows_are_zero():
    w = workloads.build("masked", B=3, q_len=1, Hq=8, Hkv=2, D=64, page_size=32,
                        kv_lens=[50, 0, 90], seed=2100, mask="2d", mask_p=0.0)
    w.mask[2, :] = -np.inf
    for s in (1, 4):
        out16, out32 = run(w, num_splits=s)
        assert not out32[1:].any() and not out16[1:].any()
        check(out16, out32, oracle.decode(w), "masked")


# ---- the score scale at its edges -------------------------------------------
# A negative scale (the kernels negate q and use |scale|), a zero scale (every
# visible key weighs the same: the rows are plain means of V) and a large
# one (near one-hot rows), on each kernel family, with and without a mask and
# causal limits.
SCALE_CASES = [
    lambda: workloads.build("scale_valu", B=3, q_len=1, Hq=8, Hkv=8, D=64, page_size=32,
                            kv_lens=[700, 33, 1500], seed=2201),
    lambda: workloads.build("scale_mfma", B=3, q_len=2, Hq=32, Hkv=8, D=128, page_size=16,
                            kv_lens=[1200, 5, 640], seed=2202, causal="last"),
    lambda: workloads.build("scale_mfma_mask", B=2, q_len=1, Hq=16, Hkv=2, D=64, page_size=32,
                            kv_lens=[900, 77], seed=2203, mask="3d", mask_p=0.2),
    lambda: workloads.build("scale_prefill", B=2, q_len=128, Hq=16, Hkv=4, D=64, page_size=32,
                            kv_lens=[900, 300], seed=2204).replace(causal_offset=workloads.CAUSAL_LAST),
]


@pytest.mark.parametrize("i", range(len(SCALE_CASES)))
@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.6])
@pytest.mark.parametrize("splits", [1, 3])
def test_negative_zero_and_large_scale(i, scale, splits):
    w = SCALE_CASES[i]().replace(scale=scale)
    note(f"scale {w.name} scale={scale} splits={splits}")
    out16, out32 = run(w, num_splits=splits)
    ref = oracle.decode_varlen(w).reshape(out32.shape) if w.causal_offset == workloads.CAUSAL_LAST \
        else oracle.decode(w)
    check(out16, out32, ref, f"{w.name} scale={scale}")


# ---- the documented limits ---------------------------------------------------
# PKV_MAX_SPLITS splits (most of them past a sequence's end or a few keys
# long), and pages of 4096 keys (the largest page size: one page-table entry
# covers more keys than a split), on each kernel family.
LIMIT_CASES = [
    lambda: workloads.build("max_splits_valu", B=3, q_len=1, Hq=8, Hkv=8, D=64, page_size=16,
                            kv_lens=[5000, 17, 1300], seed=2301),
    lambda: workloads.build("max_splits_mfma", B=2, q_len=2, Hq=32, Hkv=8, D=128, page_size=32,
                            kv_lens=[4100, 300], seed=2302, causal="last", mask="2d", mask_p=0.1),
    lambda: workloads.build("page4096_valu", B=3, q_len=1, Hq=16, Hkv=16, D=32, page_size=4096,
                            kv_lens=[9000, 4096, 1], seed=2303, spare_pages=1),
    lambda: workloads.build("page4096_mfma", B=2, q_len=4, Hq=16, Hkv=2, D=256, page_size=4096,
                            kv_lens=[8193, 600], seed=2304, causal="last"),
    lambda: workloads.build("page4096_prefill", B=1, q_len=160, Hq=8, Hkv=1, D=64, page_size=4096,
                            kv_lens=[5000], seed=2305).replace(causal_offset=workloads.CAUSAL_LAST),
]


@pytest.mark.parametrize("i", range(len(LIMIT_CASES)))
@pytest.mark.parametrize("splits", [0, 256])
def test_documented_limits(i, splits):
    import paged_kv_split_amd as pkv
    assert pkv.PKV_MAX_SPLITS == 256
    w = LIMIT_CASES[i]()
    note(f"limits {w.name} splits={splits}")
    out16, out32 = run(w, num_splits=splits)
    ref = oracle.decode_varlen(w).reshape(out32.shape) if w.causal_offset == workloads.CAUSAL_LAST \
        else oracle.decode(w)
    check(out16, out32, ref, f"{w.name} splits={splits}")
