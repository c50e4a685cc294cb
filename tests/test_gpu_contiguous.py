"""GPU parity of pkv_contiguous_decode (contiguous K/V in the "blhd" and
"bhld" layouts) against the fp64 oracle's contiguous form, and bit-identity
with pkv_paged_decode on the same logical keys: the two differ only in how a
key's address is found, not in any arithmetic."""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import check, note, paired, run, run_contiguous, sub_batch  # noqa: E402
from test_gpu_parity import SMALL  # noqa: E402


def compare_contiguous(w, layout, num_splits=0, heads_per_block=0, capacity=None, seqs=None, paged_too=True):
    note(f"contiguous {layout} {w.name} B={w.B} q_len={w.q_len} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
         f"maxL={w.max_kv_len} splits={num_splits} hpb={heads_per_block} capacity={capacity} seed={w.seed}")
    o16, o32, k, v = run_contiguous(w, layout, num_splits, heads_per_block, capacity)
    if seqs is None:
        ref = oracle.decode_contiguous(w, k, v, layout)
        check(o16, o32, ref, f"contiguous {layout} {w.name}")
    else:
        sw = sub_batch(w, seqs)
        ref = oracle.decode_contiguous(sw, k[seqs], v[seqs], layout)
        check(o16[seqs], o32[seqs], ref, f"contiguous {layout} {w.name}")
    if paged_too and not (layout == "bhld" and paired(w, heads_per_block)):
        # the same plan as the paged call, the same bits (head pairing, at D = 32, applies to the
        # paged and blhd layouts only: bhld then runs another plan, checked against the oracle above)
        p16, p32 = run(w, num_splits=num_splits, heads_per_block=heads_per_block)
        assert np.array_equal(o16, p16)
        assert np.array_equal(o32.view(np.uint32), p32.view(np.uint32))


@pytest.mark.parametrize("layout", ["blhd", "bhld"])
@pytest.mark.parametrize("i", range(len(SMALL)))
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_small_cases_contiguous(layout, i, splits):
    kw = dict(SMALL[i])
    w = workloads.build(f"small{i}", seed=2000 + i, spare_pages=3, **kw)
    compare_contiguous(w, layout, num_splits=splits)


@pytest.mark.parametrize("layout", ["blhd", "bhld"])
def test_capacity_beyond_the_longest_sequence(layout):
    """Rows past kv_lens[b] (NaN here, up to the cache capacity) are never read."""
    w = workloads.build("cap", B=3, q_len=2, Hq=16, Hkv=4, D=128, page_size=32, kv_lens=[700, 1, 300],
                        seed=2400, mask="2d", causal="last")
    compare_contiguous(w, layout, capacity=1000, paged_too=False)
    compare_contiguous(w, layout, num_splits=3, capacity=1000, paged_too=False)


@pytest.mark.parametrize("layout", ["blhd", "bhld"])
@pytest.mark.parametrize("hpb", [1, 2, 4])
def test_heads_per_block_contiguous(layout, hpb):
    w = workloads.build("hpbc", B=3, q_len=1, Hq=8, Hkv=8, D=64, page_size=32, kv_lens=[900, 33, 2047], seed=2410)
    compare_contiguous(w, layout, num_splits=4, heads_per_block=hpb)


@pytest.mark.parametrize("layout", ["blhd", "bhld"])
def test_decode_shapes_contiguous(layout):
    """The decode shapes at full size (sampled sequences where the oracle is slow)."""
    compare_contiguous(workloads.decode_1b(), layout)
    compare_contiguous(workloads.sweep(128, 32), layout, seqs=[0, 15])
    compare_contiguous(workloads.long_ctx(), layout, seqs=[0, 3])
