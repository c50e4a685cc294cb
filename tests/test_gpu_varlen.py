"""GPU parity of pkv_paged_decode_varlen (sequences with different numbers of
query tokens: chunked prefill and decode in one batch) against the fp64
oracle's varlen form, and bit-identity with pkv_paged_decode where the two
describe the same problem."""
import numpy as np
import pytest

import oracle
import paged_kv_split_amd as pkv
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import check, note, problem, run, run_varlen  # noqa: E402

LAST = workloads.CAUSAL_LAST

# (q_lens, kv_lens, build args): VALU (G * max_q <= 2) and matrix-core
# families, several tiles and row blocks, ragged tails, empty sequences,
# sequences with fewer keys than tokens, masks, GQA groups.
CASES = [
    ([1, 2, 0, 2], [37, 300, 50, 2], dict(Hq=8, Hkv=8, D=64, page_size=32, causal="lastv")),
    ([1, 1, 1], [1000, 1, 4097], dict(Hq=16, Hkv=16, D=128, page_size=16, causal="lastv", mask="2d")),
    ([5, 1, 17, 0, 3], [600, 77, 2050, 9, 3], dict(Hq=32, Hkv=8, D=128, page_size=32, causal="lastv")),
    ([40, 1, 1, 33], [64, 900, 5000, 40], dict(Hq=16, Hkv=2, D=64, page_size=64, causal="lastv",
                                               mask="3d", mask_p=0.2)),
    ([7, 2, 1], [3, 1500, 700], dict(Hq=24, Hkv=4, D=64, page_size=32, causal="lastv")),   # 7 tokens, 3 keys
    ([3, 9, 1, 4], [129, 1030, 31, 800], dict(Hq=8, Hkv=2, D=256, page_size=16, causal="lastv")),
    ([2, 6, 1], [200, 400, 3000], dict(Hq=4, Hkv=1, D=32, page_size=32)),                  # causal off
    ([4, 1, 12], [500, 100, 2000], dict(Hq=32, Hkv=8, D=128, page_size=32, causal=20)),
    ([16, 16, 1, 16], [4000, 16, 2500, 700], dict(Hq=8, Hkv=1, D=128, page_size=32, causal="lastv",
                                                   mask="2d", mask_p=0.3)),
    ([2, 1, 0, 2], [900, 33, 5, 2], dict(Hq=16, Hkv=8, D=256, page_size=32, causal="lastv",
                                         mask="3d")),                                  # VALU, 4 rows
]


def compare_varlen(w, num_splits=0, heads_per_block=0):
    note(f"varlen {w.name} B={w.B} q_lens={w.q_lens.tolist() if w.q_lens is not None else w.q_len} "
         f"Hq={w.Hq} Hkv={w.Hkv} D={w.D} maxL={w.max_kv_len} causal={w.causal_offset} "
         f"mask={None if w.mask is None else w.mask.ndim} splits={num_splits} hpb={heads_per_block} seed={w.seed}")
    o16, o32 = run_varlen(w, num_splits, heads_per_block)
    ref = oracle.decode_varlen(w)
    assert o16.shape == ref.shape
    return check(o16, o32, ref, f"varlen {w.name}"), o16, o32


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("splits", [0, 1, 4])
def test_varlen_cases(i, splits):
    q_lens, lens, kw = CASES[i]
    w = workloads.varlen(f"varlen{i}", q_lens=q_lens, kv_lens=lens, B=len(q_lens), seed=3000 + i,
                         spare_pages=2, **kw)
    compare_varlen(w, num_splits=splits)


@pytest.mark.parametrize("hpb", [1, 2])
def test_varlen_heads_per_block(hpb):
    w = workloads.varlen("varlen_hpb", q_lens=[1, 3, 2], kv_lens=[1200, 90, 2600], B=3, Hq=16, Hkv=4, D=128,
                         page_size=32, seed=3100, causal="lastv")
    compare_varlen(w, num_splits=4, heads_per_block=hpb)


def test_mixed_prefill_and_decode_batch():
    """The mixed workload (a quarter of 32 sequences with prefill chunks of
    8..64 tokens, the rest one decode token) at full size, every row."""
    w = workloads.mixed()
    compare_varlen(w)


def test_equal_counts_are_the_fixed_batch_bit_for_bit():
    """Every sequence with q_len tokens: the varlen call and pkv_paged_decode
    give the same bits, with explicit per-sequence offsets and with
    CAUSAL_LAST through both entry points."""
    w = workloads.build("eq", B=5, q_len=3, Hq=32, Hkv=8, D=128, page_size=32, kv_lens=[3, 700, 2049, 64, 1300],
                        seed=3200, causal="last", mask="3d", mask_p=0.1)
    note("varlen equal counts: explicit offsets and CAUSAL_LAST")
    f16, f32 = run(w, num_splits=3)
    v16, v32 = run_varlen(w, num_splits=3)
    assert np.array_equal(v16.reshape(f16.shape), f16)
    assert np.array_equal(v32.reshape(f32.shape).view(np.uint32), f32.view(np.uint32))
    last = w.replace(causal_offsets=None, causal_offset=LAST)
    l16, l32 = run(last, num_splits=3)
    lv16, lv32 = run_varlen(last.replace(q_lens=np.full(5, 3, np.int32)), num_splits=3)
    assert np.array_equal(l16, f16) and np.array_equal(l32.view(np.uint32), f32.view(np.uint32))
    assert np.array_equal(lv16, v16) and np.array_equal(lv32.view(np.uint32), v32.view(np.uint32))


@pytest.mark.parametrize("shape", ["long_mha_d64", "gqa_causal_last"])
def test_equal_counts_auto_splits_bit_for_bit(shape):
    """Every sequence with q_len tokens and the split count and grouping left
    to the library: the varlen call follows pkv_paged_decode's plan (the
    first shape is one where a varlen-only key cap once gave 32 splits
    against 8) and gives the same bits."""
    if shape == "long_mha_d64":
        w = workloads.build("eq_auto_long", B=4, q_len=1, Hq=8, Hkv=8, D=64, page_size=32,
                            kv_lens=[32768] * 4, seed=3210)
    else:
        w = workloads.build("eq_auto_gqa", B=6, q_len=3, Hq=32, Hkv=8, D=128, page_size=32,
                            kv_lens=[5000, 37, 2049, 8000, 640, 3], seed=3211, causal="last", mask="2d")
    p = problem(w, 0)
    fx = pkv.plan(p)
    vl = pkv.plan_varlen(p, w.B * w.q_len)
    assert (vl.splits, vl.heads_per_block) == (fx.splits, fx.heads_per_block)
    note(f"varlen equal counts, auto splits: {shape} S={fx.splits} hpb={fx.heads_per_block}")
    f16, f32 = run(w)
    v16, v32 = run_varlen(w.replace(q_lens=np.full(w.B, w.q_len, np.int32)))
    assert np.array_equal(v16.reshape(f16.shape), f16)
    assert np.array_equal(v32.reshape(f32.shape).view(np.uint32), f32.view(np.uint32))


def test_causal_last_with_fewer_keys_than_tokens_fixed_entry():
    """pkv_paged_decode with causal_offset CAUSAL_LAST where some sequence is
    shorter than q_len: its leading rows see no key and are zero."""
    w = workloads.build("lastshort", B=3, q_len=6, Hq=8, Hkv=2, D=64, page_size=16, kv_lens=[2, 40, 6],
                        seed=3300).replace(causal_offset=LAST)
    note("fixed entry, CAUSAL_LAST, kv_lens [2, 40, 6], q_len 6")
    o16, o32 = run(w, num_splits=2)
    ref = oracle.decode_varlen(w).reshape(o32.shape)
    check(o16, o32, ref, "causal last fixed")
    assert (o32[0, :4] == 0).all()


def test_no_tokens_at_all_writes_nothing():
    import torch
    import paged_kv_split_amd as pkv
    w = workloads.varlen("none", q_lens=[0, 0], kv_lens=[30, 5], B=2, Hq=4, Hkv=2, D=64, page_size=16, seed=3400)
    note("varlen, zero tokens")
    d = torch.device("cuda:0")
    k = torch.from_numpy(w.k_cache.view(np.int16)).view(torch.bfloat16).to(d)
    bt = torch.from_numpy(w.block_table).to(d)
    kl = torch.from_numpy(w.kv_lens).to(d)
    cu = torch.zeros(3, dtype=torch.int32, device=d)
    q = torch.empty(0, 4, 64, dtype=torch.bfloat16, device=d)
    out = pkv.paged_decode_varlen(q, k, k, bt, kl, cu, max_q_len=1, scale=w.scale)
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 64)


def _plan(w, splits=0, hpb=0):
    import paged_kv_split_amd as pkv
    from gpu_util import problem
    return pkv.plan_varlen(problem(w, splits, hpb), w.total_tokens)


@pytest.mark.parametrize("splits", [0, 3])
def test_compact_row_blocks_over_64_sequences(splits):
    """150 sequences (the row-block search takes two rounds), most with one
    token: the grid holds floor(T * G / 32) + B row-block slots, not
    B * ceil(q_len * G / 32)."""
    import torch
    g = torch.Generator().manual_seed(3500)
    B = 150
    q_lens = torch.where(torch.rand(B, generator=g) < 0.2, torch.randint(0, 17, (B,), generator=g),
                         torch.ones(B, dtype=torch.int64)).tolist()
    lens = torch.randint(1, 600, (B,), generator=g).tolist()
    lens = [max(L, n) for L, n in zip(lens, q_lens)]
    w = workloads.varlen("compact150", q_lens=q_lens, kv_lens=lens, B=B, Hq=16, Hkv=2, D=64, page_size=16,
                         seed=3500, causal="lastv")
    pl = _plan(w, splits, 2)           # two kv heads per workgroup: the 32-row kernel
    assert pl.rows_per_block == 32
    assert pl.units == w.total_tokens * 8 // 32 + B
    compare_varlen(w, num_splits=splits, heads_per_block=2)
    pl = _plan(w, splits, 1)           # one: the 128-row prefill-shaped kernel (128 rows per sequence)
    assert pl.rows_per_block == 128 and pl.units == B * 2
    compare_varlen(w, num_splits=splits, heads_per_block=1)


def test_large_varlen_batch_with_separate_combine():
    """600 sequences (past the exact schedule's 256: one slot per (sequence,
    row block)) and more units than arrival counters: the splits go through
    the combine kernel, empty row blocks exit."""
    import torch
    g = torch.Generator().manual_seed(3600)
    B = 600
    q_lens = torch.where(torch.rand(B, generator=g) < 0.1, torch.randint(2, 9, (B,), generator=g),
                         torch.ones(B, dtype=torch.int64)).tolist()
    lens = torch.randint(8, 200, (B,), generator=g).tolist()
    w = workloads.varlen("varlen600", q_lens=q_lens, kv_lens=lens, B=B, Hq=64, Hkv=8, D=128, page_size=32,
                         seed=3600, causal="lastv")
    pl = _plan(w, 2, 1)
    assert pl.units == B * 2 * 8
    assert pl.merge_in_kernel == 0 and pl.kernels == 2
    compare_varlen(w, num_splits=2, heads_per_block=1)


def test_exact_schedule_with_separate_combine():
    """256 sequences (the exact schedule) with more units than arrival
    counters: every split of every row block gets a workgroup, and those
    past a row block's keys leave empty partials for the combine kernel."""
    import torch
    g = torch.Generator().manual_seed(3700)
    B = 256
    q_lens = torch.randint(0, 13, (B,), generator=g).tolist()
    lens = torch.randint(1, 100, (B,), generator=g).tolist()
    w = workloads.varlen("exact256", q_lens=q_lens, kv_lens=lens, B=B, Hq=128, Hkv=16, D=64, page_size=16,
                         seed=3700, causal="lastv")
    pl = _plan(w, 3, 1)
    nv = w.total_tokens * 8 // 32 + B
    assert nv < B * 3 and pl.units == nv * 16
    assert pl.merge_in_kernel == 0 and pl.kernels == 2
    compare_varlen(w, num_splits=3, heads_per_block=1)


def _dev_varlen(w):
    import torch
    from gpu_util import dev_tensors
    d = dev_tensors(w)
    qp, cu = w.packed_q()
    d["qp"] = torch.from_numpy(qp.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    d["cu"] = torch.from_numpy(cu).to("cuda:0")
    return d


def test_varlen_graph_capture_with_changing_token_counts():
    """A captured varlen call (exact schedule, in-kernel merge) replayed after
    q, kv_lens and the token counts change in place (same total): every
    replay equals an eager call on the same inputs, and the oracle."""
    import torch
    import paged_kv_split_amd as pkv
    w = workloads.varlen("vgraph", q_lens=[1, 9, 1, 6], kv_lens=[1500, 900, 3000, 400], B=4, Hq=32, Hkv=8, D=128,
                         page_size=32, seed=3800, causal="lastv")
    d = _dev_varlen(w)
    T = w.total_tokens
    p = problem_for_varlen(w, 4)
    o_part, ml_part = pkv.alloc_workspace(p, 4, "cuda:0")
    out = torch.empty(tuple(d["qp"].shape), dtype=torch.bfloat16, device="cuda:0")
    out32 = torch.empty(tuple(d["qp"].shape), dtype=torch.float32, device="cuda:0")

    def call(stream=None):
        pkv.paged_decode_varlen(d["qp"], d["k"], d["v"], d["bt"], d["kl"], d["cu"], max_q_len=w.q_len,
                                scale=w.scale, num_splits=4, max_kv_len=w.max_kv_len, out=out, out_f32=out32,
                                o_part=o_part, ml_part=ml_part, stream=stream)

    note("varlen graph capture")
    call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    counts = [[1, 9, 1, 6], [4, 4, 4, 5], [9, 0, 8, 0], [1, 1, 6, 9]]   # each at most the 9 the launch is sized for
    rng = np.random.default_rng(7)
    for rep, ql in enumerate(counts):
        assert sum(ql) == T
        lens = np.maximum(rng.integers(1, w.kv_lens + 1), np.array(ql)).astype(np.int32)
        wr = w.replace(q_lens=np.array(ql, np.int32), kv_lens=lens)
        qp, cu = wr.packed_q()
        d["qp"].copy_(torch.from_numpy(qp.view(np.int16)).view(torch.bfloat16).to("cuda:0"))
        d["cu"].copy_(torch.from_numpy(cu).to("cuda:0"))
        d["kl"].copy_(torch.from_numpy(lens).to("cuda:0"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        r32, r16 = out32.clone(), out.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(r32.view(torch.int32), out32.view(torch.int32)), f"replay {rep}"
        assert torch.equal(r16.view(torch.int16), out.view(torch.int16)), f"replay {rep}"
        check(r16.view(torch.int16).cpu().numpy().view(np.uint16), r32.cpu().numpy(), oracle.decode_varlen(wr),
              f"graph replay {rep}")


def problem_for_varlen(w, splits):
    from gpu_util import problem
    return problem(w, splits)


def test_one_workspace_across_varlen_fixed_and_prefill_calls():
    """The arrival counters of every call are left zero: varlen (exact
    schedule), fixed-length and prefill-shaped calls share one workspace in
    turn, each checked against the oracle."""
    import torch
    import paged_kv_split_amd as pkv
    from gpu_util import dev_tensors, problem
    wv = workloads.varlen("wsv", q_lens=[3, 1, 12, 1], kv_lens=[700, 2000, 900, 50], B=4, Hq=32, Hkv=8, D=128,
                          page_size=32, seed=3900, causal="lastv")
    wf = workloads.build("wsf", B=6, q_len=1, Hq=32, Hkv=8, D=128, page_size=32,
                         kv_lens=[3000, 100, 2000, 5, 900, 4096], seed=3901)
    wp = workloads.build("wsp", B=2, q_len=160, Hq=32, Hkv=8, D=128, page_size=32, kv_lens=[2000, 700],
                         seed=3902).replace(causal_offset=LAST)
    big = max(pkv.workspace_bytes(problem(x, 4), 4)[0] for x in (wv, wf, wp)), \
        max(pkv.workspace_bytes(problem(x, 4), 4)[1] for x in (wv, wf, wp))
    o_part = torch.empty(big[0] // 4, dtype=torch.float32, device="cuda:0")
    ml_part = torch.zeros(big[1] // 4, dtype=torch.float32, device="cuda:0")
    for rnd in range(2):
        note(f"shared workspace round {rnd}")
        d = _dev_varlen(wv)
        out32 = torch.empty(tuple(d["qp"].shape), dtype=torch.float32, device="cuda:0")
        o16 = pkv.paged_decode_varlen(d["qp"], d["k"], d["v"], d["bt"], d["kl"], d["cu"], max_q_len=wv.q_len,
                                      scale=wv.scale, num_splits=4, max_kv_len=wv.max_kv_len, out_f32=out32,
                                      o_part=o_part, ml_part=ml_part)
        torch.cuda.synchronize()
        check(o16.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy(), oracle.decode_varlen(wv),
              "shared workspace varlen")
        for x in (wf, wp):
            d = dev_tensors(x)
            p = problem(x, 4)
            out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device="cuda:0")
            o16 = pkv.paged_decode(d["q"], d["k"], d["v"], d["bt"], d["kl"], scale=x.scale,
                                   causal_offset=x.causal_offset, out_f32=out32, o_part=o_part, ml_part=ml_part,
                                   problem=p)
            torch.cuda.synchronize()
            ref = oracle.decode_varlen(x).reshape(out32.shape) if x.causal_offset == LAST else oracle.decode(x)
            check(o16.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy(), ref,
                  f"shared workspace {x.name}")
    head = ml_part[: pkv.PKV_COUNTER_BYTES // 4].view(torch.int32)
    assert int(head.abs().sum()) == 0


def test_varlen_calls_are_deterministic():
    w = workloads.mixed()
    note("varlen determinism")
    a16, a32 = run_varlen(w)
    b16, b32 = run_varlen(w)
    assert np.array_equal(a16, b16) and np.array_equal(a32.view(np.uint32), b32.view(np.uint32))
