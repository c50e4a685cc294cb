"""Properties of the launch plan over random problems (host arithmetic only,
no GPU): every plan pkv_plan / pkv_plan_varlen returns is one the kernels
can run, the split count covers the longest sequence, the in-kernel merge is
taken only when its counters fit the workspace head, the workspace sizes
follow the documented layout, and a varlen batch that holds every token is
planned exactly as the fixed-length batch."""
import math

from hypothesis import given, settings, strategies as st

import paged_kv_split_amd as pkv

CUS = 256


@st.composite
def problems(draw):
    hkv = draw(st.sampled_from([1, 2, 4, 8, 16]))
    g = draw(st.sampled_from([1, 2, 3, 4, 6, 8, 16]))
    d = draw(st.sampled_from([32, 64, 128, 256]))
    page = draw(st.sampled_from([1, 8, 16, 32, 64, 256, 4096]))
    batch = draw(st.integers(1, 300))
    q_len = draw(st.sampled_from([1, 1, 2, 4, 16, 64, 200, 512]))
    max_len = draw(st.integers(1, 40000))
    pages_per_seq = max(1, math.ceil(max_len / page))
    causal = draw(st.sampled_from([-1, -1, 0, 17, pkv.PKV_CAUSAL_LAST]))
    splits = draw(st.sampled_from([0, 0, 0, 1, 2, 7, 64, 256]))
    hpb = draw(st.sampled_from([0, 0, 0, 1, 2, 4, 8]))
    if hpb and hkv % hpb or (hpb == 8 and d > 64):
        hpb = 0
    return pkv.make_problem(batch=batch, q_len=q_len, num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d,
                            page_size=page, num_pages=batch * pages_per_seq, max_pages_per_seq=pages_per_seq,
                            max_kv_len=max_len, scale=0.1, causal_offset=causal, num_splits=splits,
                            heads_per_block=hpb)


def _check_plan(p, pl):
    assert 1 <= pl.splits <= pkv.PKV_MAX_SPLITS
    if p.num_splits:
        assert pl.splits == p.num_splits
    assert pl.heads_per_block in (1, 2, 4, 8) and p.num_kv_heads % pl.heads_per_block == 0
    if p.heads_per_block:
        assert pl.heads_per_block == p.heads_per_block
    assert pl.rows_per_block in (1, 2, 4, 16, 32, 128)
    rows = (p.num_q_heads // p.num_kv_heads) * p.q_len
    hd, hpb = p.head_dim, pl.heads_per_block
    # head pairing: only at D = 32, an even kv head count, automatic grouping and at most 8 rows
    # per kv head; the launch is that of Hkv / 2 heads of 64 columns with twice the rows
    assert pl.paired_heads == (p.head_dim == 32 and p.num_kv_heads % 2 == 0 and p.heads_per_block == 0
                               and 2 * rows <= 16)
    if pl.paired_heads:
        assert hpb % 2 == 0
        rows, hd, hpb = 2 * rows, 64, hpb // 2
    assert pl.matrix_core == (1 if pl.rows_per_block >= 16 else 0)
    if pl.rows_per_block == 128:
        assert rows >= 128 and hd <= 128 and hpb == 1
    # the kernel follows from the rows, head dim and grouping
    if pl.rows_per_block == 128:
        assert pl.kernel == pkv.PKV_KERNEL_PREFILL
    elif hpb == 8 or (hpb == 4 and rows > 2 and hd <= 128):
        assert pl.kernel == pkv.PKV_KERNEL_SHARED_TILE and pl.rows_per_block in (16, 32)
        assert hpb < 8 or hd <= 64
    else:
        # the vector kernel up to 2 rows, at head_dim 256 up to 4 (four rows per workgroup)
        vector = rows <= 2 or (hd == 256 and rows <= 4)
        assert pl.kernel == (pkv.PKV_KERNEL_VECTOR if vector else pkv.PKV_KERNEL_MATRIX)
        if vector:
            assert pl.rows_per_block == (1 if rows <= 1 else 2 if rows <= 2 else 4)
    assert pl.workgroups == pl.units * pl.splits
    assert pl.merge_in_kernel in (0, 1) and pl.kernels in (1, 2)
    if pl.merge_in_kernel:
        assert pl.splits > 1 and pl.units <= pkv.PKV_MAX_FUSED_UNITS
    if pl.splits > 1 and not pl.merge_in_kernel:
        assert pl.kernels == 2
    # the splits cover the longest sequence
    assert pl.splits * math.ceil(p.max_kv_len / pl.splits) >= p.max_kv_len


@settings(max_examples=400, deadline=None, derandomize=True)
@given(problems())
def test_every_plan_is_runnable(p):
    pl = pkv.plan(p, CUS)
    _check_plan(p, pl)
    assert pkv.num_splits(p, CUS) == pl.splits
    ob, mb = pkv.workspace_bytes(p, pl.splits)
    rows = p.batch * p.q_len * p.num_q_heads
    if pl.splits > 1:
        assert ob == rows * pl.splits * p.head_dim * 4
        assert mb == pkv.PKV_COUNTER_BYTES + rows * pl.splits * 2 * 4
    else:
        assert (ob, mb) == (0, 0)


@settings(max_examples=300, deadline=None, derandomize=True)
@given(problems(), st.floats(0.0, 1.0))
def test_every_varlen_plan_is_runnable(p, frac):
    total = p.batch * p.q_len
    tokens = int(round(frac * total))
    pl = pkv.plan_varlen(p, tokens, CUS)
    _check_plan(p, pl)
    if tokens == total:
        # every token present: the plan of the fixed-length batch, field for field
        fx = pkv.plan(p, CUS)
        assert [getattr(pl, f) for f, _ in pkv.PlanInfo._fields_] == \
            [getattr(fx, f) for f, _ in pkv.PlanInfo._fields_]


@settings(max_examples=200, deadline=None, derandomize=True)
@given(problems())
def test_varlen_plan_with_every_token_is_the_fixed_plan(p):
    """A varlen batch holding all B * q_len tokens is planned exactly as the
    fixed-length batch (so the two entry points give it the same bits)."""
    fx = pkv.plan(p, CUS)
    vl = pkv.plan_varlen(p, p.batch * p.q_len, CUS)
    assert [getattr(vl, f) for f, _ in pkv.PlanInfo._fields_] == [getattr(fx, f) for f, _ in pkv.PlanInfo._fields_]
