"""GPU parity on seeded random problems: each case draws its shape and its
options together (head dim, GQA ratio, page size, batch, query tokens,
lengths including empty and one-key sequences, causal mode, mask, forced
splits and kv-head grouping, fixed-length or varlen), so combinations that
the hand-picked cases do not list are compared with the fp64 oracle too;
fixed-length cases also run over a contiguous copy of their keys, which must
give the same bits.
The draws are fixed by the case seed; sizes keep the oracle to a fraction of
a second per case."""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import check, note, paired, run, run_contiguous, run_varlen  # noqa: E402

N_CASES = 160


def draw_case(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([32, 64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    page = int(rng.choice([1, 4, 16, 32, 64, 256]))
    B = int(rng.integers(1, 9))
    varlen = bool(rng.random() < 0.4)
    q_len = int(rng.choice([1, 1, 2, 4, 9, 40, 130]))
    top = int(rng.choice([64, 700, 3000]))
    lens = rng.integers(0, top + 1, size=B)
    lens[rng.random(B) < 0.15] = 1
    if D == 256 and page == 256:
        page = 64
    causal = str(rng.choice(["off", "last", "fixed"]))
    mask = str(rng.choice(["none", "none", "2d", "3d"]))
    splits = int(rng.choice([0, 0, 1, 3, 16]))
    hpb = int(rng.choice([0, 0, 1, 2, 4]))
    if hpb and Hkv % hpb:
        hpb = 0
    kw = dict(B=B, Hq=Hkv * G, Hkv=Hkv, D=D, page_size=page, kv_lens=lens.tolist(), seed=9000 + seed,
              spare_pages=int(rng.integers(0, 3)), mask=mask, mask_p=0.15)
    if varlen:
        q_lens = rng.integers(0, q_len + 1, size=B)
        w = workloads.varlen(f"rand{seed}", q_lens=q_lens, causal="lastv" if causal != "off" else "off", **kw)
    else:
        c = {"off": "off", "last": "last", "fixed": int(rng.integers(0, 50))}[causal]
        w = workloads.build(f"rand{seed}", q_len=q_len, causal=c, **kw)
    return w, splits, hpb, varlen


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_problem(seed):
    w, splits, hpb, varlen = draw_case(seed)
    note(f"random seed={seed} B={w.B} q_len={w.q_len} Hq={w.Hq} Hkv={w.Hkv} D={w.D} P={w.page_size} "
         f"L={w.kv_lens.tolist()} q_lens={None if w.q_lens is None else w.q_lens.tolist()} "
         f"causal={w.causal_offset}/{w.causal_offsets is not None} mask={None if w.mask is None else w.mask.ndim} "
         f"splits={splits} hpb={hpb}")
    if varlen:
        o16, o32 = run_varlen(w, num_splits=splits, heads_per_block=hpb)
        ref = oracle.decode_varlen(w)
    else:
        o16, o32 = run(w, num_splits=splits, heads_per_block=hpb)
        ref = oracle.decode(w)
    check(o16, o32, ref.reshape(o32.shape), f"random seed={seed}")
    if not varlen:
        # the same keys in a contiguous cache: the same plan, the same bits (bhld never pairs kv
        # heads: with a paired paged plan it runs another plan, checked against the oracle)
        layout = ("blhd", "bhld")[seed % 2]
        c16, c32, _, _ = run_contiguous(w, layout, num_splits=splits, heads_per_block=hpb)
        if layout == "bhld" and paired(w, hpb):
            check(c16, c32, ref.reshape(c32.shape), f"random seed={seed} bhld")
        else:
            assert np.array_equal(c16, o16), f"contiguous {layout} bf16 differs"
            assert np.array_equal(c32.view(np.uint32), o32.view(np.uint32)), f"contiguous {layout} fp32 differs"
