"""GPU parity of the prefill-shaped matrix-core kernel (from 128 packed rows
per kv head at D <= 128: four waves of 32 rows sharing each 64-key K/V tile)
against the fp64 oracle: chunks of query tokens over paged K/V, causal at the
end of the sequence or at a fixed position, 2D/3D masks, forced splits with
the in-kernel merge and with the separate combine kernel, pages smaller than
a 16-key tile, more keys than one page-table window, contiguous K/V, and
varlen batches."""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import check, note, problem, run, run_contiguous, run_varlen  # noqa: E402

LAST = workloads.CAUSAL_LAST


def _kernel(w, splits=0, hpb=0):
    import paged_kv_split_amd as pkv
    return pkv.kernel_family(problem(w, splits, hpb))


def compare(w, splits=0, hpb=0, expect="split_prefill_mfma"):
    note(f"prefill {w.name} B={w.B} q_len={w.q_len} Hq={w.Hq} Hkv={w.Hkv} D={w.D} P={w.page_size} "
         f"L={w.kv_lens.tolist()[:6]} causal={w.causal_offset} mask={None if w.mask is None else w.mask.ndim} "
         f"splits={splits} hpb={hpb} seed={w.seed}")
    assert _kernel(w, splits, hpb) == expect
    o16, o32 = run(w, num_splits=splits, heads_per_block=hpb)
    ref = oracle.decode_varlen(w).reshape(o32.shape) if w.causal_offset == LAST else oracle.decode(w)
    return check(o16, o32, ref, f"prefill {w.name}")


# (B, q_len, Hq, Hkv, D, page, kv_lens, extra build args)
CASES = [
    (1, 128, 8, 1, 128, 32, [128], dict(causal="lastv")),                       # whole-sequence causal prefill
    (2, 200, 16, 4, 64, 16, [900, 200], dict(causal="lastv")),                  # ragged rows (800 = 6.25 blocks)
    (3, 64, 16, 2, 32, 32, [5000, 64, 1111], dict(causal="lastv", mask="3d", mask_p=0.2)),
    (2, 130, 32, 8, 128, 64, [3000, 141], dict(mask="2d", mask_p=0.3)),       # causal off, 2D mask
    (2, 129, 64, 16, 64, 8, [700, 300], dict(causal=100)),                      # page 8 (< 16-key tile), fixed offset
    (1, 128, 32, 8, 128, 16, [17000], dict(causal="lastv")),                    # two page-table windows
    (4, 130, 4, 1, 64, 32, [129, 130, 1000, 2], dict(causal="lastv", mask="2d", mask_p=0.1)),  # fewer keys than tokens
]


def _build(i, q_len_override=None):
    B, ql, Hq, Hkv, D, P, lens, kw = CASES[i]
    kw = dict(kw)
    causal = kw.pop("causal", "off")
    w = workloads.build(f"prefill{i}", B=B, q_len=ql, Hq=Hq, Hkv=Hkv, D=D, page_size=P, kv_lens=lens,
                        seed=4000 + i, spare_pages=2, causal="off" if causal == "lastv" else causal, **kw)
    if causal == "lastv":
        w = w.replace(causal_offset=LAST)
    return w


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_prefill_cases(i, splits):
    compare(_build(i), splits)


def test_forced_heads_per_block_takes_the_decode_kernel():
    w = _build(1)
    compare(w, 2, hpb=2, expect="split_decode_mfma")


def test_prefill_with_separate_combine():
    """More (sequence, kv head, 128-row block) units than arrival counters:
    the forced splits go through the combine kernel."""
    import paged_kv_split_amd as pkv
    w = workloads.build("prefill_comb", B=40, q_len=512, Hq=32, Hkv=8, D=64, page_size=32,
                        kv_lens=list(range(500, 500 + 40 * 7, 7)), seed=4100).replace(causal_offset=LAST)
    pl = pkv.plan(problem(w, 2))
    assert pl.rows_per_block == 128 and pl.units == 40 * 8 * 16 and pl.merge_in_kernel == 0 and pl.kernels == 2
    compare(w, 2)


@pytest.mark.parametrize("layout", ["blhd", "bhld"])
def test_prefill_contiguous(layout):
    w = _build(2)
    note(f"prefill contiguous {layout}")
    o16, o32, k, v = run_contiguous(w, layout, num_splits=2)
    check(o16, o32, oracle.decode_varlen(w).reshape(o32.shape), f"prefill contiguous {layout}")


def test_varlen_prefill_chunks():
    """A varlen batch bounded at 64 tokens with G = 8 (512 rows): decode
    tokens, prefill chunks and an empty sequence through the prefill kernel."""
    w = workloads.varlen("vprefill", q_lens=[64, 1, 0, 37, 1, 16], kv_lens=[3000, 500, 10, 37, 2049, 900], B=6,
                         Hq=32, Hkv=4, D=128, page_size=32, seed=4200, causal="lastv")
    import paged_kv_split_amd as pkv
    for splits in (0, 1, 4):
        assert pkv.plan_varlen(problem(w, splits), w.total_tokens).rows_per_block == 128
        note(f"varlen prefill splits={splits}")
        o16, o32 = run_varlen(w, num_splits=splits)
        check(o16, o32, oracle.decode_varlen(w), "varlen prefill")


@pytest.mark.parametrize("splits", [0, 3])
def test_varlen_prefill_with_3d_mask_and_single_sequence(splits):
    """Varlen through the prefill-shaped kernel with a 3D mask (indexed by
    the token within its sequence), and a batch of one sequence whose chunk
    is shorter than the bound."""
    w = workloads.varlen("vpmask", q_lens=[70, 1, 128, 0], kv_lens=[700, 64, 1500, 9], B=4, Hq=32, Hkv=8, D=64,
                         page_size=16, seed=4300, causal="lastv", mask="3d", mask_p=0.15)
    import paged_kv_split_amd as pkv
    assert pkv.plan_varlen(problem(w, splits), w.total_tokens).rows_per_block == 128
    note(f"varlen prefill 3d mask splits={splits}")
    o16, o32 = run_varlen(w, num_splits=splits)
    check(o16, o32, oracle.decode_varlen(w), "varlen prefill 3d mask")
    w1 = workloads.varlen("vp1", q_lens=[300], kv_lens=[2500], B=1, Hq=16, Hkv=2, D=128, page_size=32, seed=4301,
                          causal="lastv")
    w1 = w1.replace(q_len=512, q=np.concatenate([w1.q, np.zeros((1, 212, 16, 128), np.uint16)], axis=1))
    assert pkv.plan_varlen(problem(w1, splits), w1.total_tokens).rows_per_block == 128
    note(f"varlen prefill single sequence splits={splits}")
    o16, o32 = run_varlen(w1, num_splits=splits)
    check(o16, o32, oracle.decode_varlen(w1), "varlen prefill single sequence")


@pytest.mark.parametrize("splits", [0, 1, 8])
def test_whole_sequence_causal_prefill_of_2048_tokens(splits):
    """A 2048-token sequence prefilled whole (causal, G = 8: 16384 rows, 128
    row blocks of one kv head): the triangle of visible keys spans every
    position from 1 to 2048 keys, each row block's causal skip differs, and
    the (pair, row block) list is dealt over the eight XCDs."""
    w = workloads.build("long_prefill", B=1, q_len=2048, Hq=8, Hkv=1, D=64, page_size=64, kv_lens=[2048],
                        seed=4400).replace(causal_offset=LAST)
    compare(w, splits)


def test_prefill_workload_at_full_size_every_row():
    """The benchmark's prefill workload as timed (4 sequences of 4096 keys
    whose last 512 are a chunk of query tokens, Hq = 32, Hkv = 8, D = 128,
    the library's own split count and grouping): every row of every sequence
    against the oracle."""
    w = workloads.prefill()
    errs = compare(w)
    note(f"prefill workload: max err fp32 {errs['err32']:.3e} bf16 {errs['err16']:.3e}")
