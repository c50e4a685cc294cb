"""GPU invariants that need no oracle value: byte-identity under physical page
reshuffles and buffer moves, exact closed forms, poisoned unused memory,
agreement across split counts, graph capture, stream ordering, guard bands
around every output, and keys stored past element 2^32 of a cache."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_split_amd as pkv
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import check, dev_tensors, note, problem, run, sub_batch  # noqa: E402


def permute_pages(w, seed):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_pages)
    k = np.empty_like(w.k_cache)
    v = np.empty_like(w.v_cache)
    k[perm] = w.k_cache
    v[perm] = w.v_cache
    bt = np.where(w.block_table >= 0, perm[np.clip(w.block_table, 0, None)], -1).astype(np.int32)
    return w.replace(k_cache=k, v_cache=v, block_table=bt)


CASES = [
    lambda: workloads.tiny(),
    lambda: workloads.build("reshuffle_gqa", B=4, q_len=1, Hq=32, Hkv=8, D=128, page_size=32,
                            kv_lens=[1000, 513, 64, 1], seed=3001, mask="2d", spare_pages=5),
    lambda: workloads.build("reshuffle_causal", B=3, q_len=4, Hq=16, Hkv=2, D=64, page_size=16,
                            kv_lens=[300, 45, 128], seed=3002, causal="last"),
    lambda: workloads.build("reshuffle_d256", B=2, q_len=1, Hq=8, Hkv=8, D=256, page_size=64,
                            kv_lens=[700, 250], seed=3003),
    lambda: workloads.build("reshuffle_d32", B=2, q_len=1, Hq=64, Hkv=8, D=32, page_size=32,
                            kv_lens=[900, 31], seed=3004, mask="2d"),
]


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("splits", [1, 7])
def test_page_reshuffle_is_byte_identical(i, splits):
    w = CASES[i]()
    note(f"reshuffle {w.name} splits={splits}")
    a16, a32 = run(w, num_splits=splits)
    for seed in (1, 2):
        b16, b32 = run(permute_pages(w, seed), num_splits=splits)
        assert np.array_equal(a16, b16)
        assert np.array_equal(a32.view(np.uint32), b32.view(np.uint32))


def test_kv_len_one_returns_v_row_exactly():
    w = workloads.build("kv1", B=5, q_len=1, Hq=16, Hkv=4, D=128, page_size=32, kv_lens=[1] * 5,
                        seed=3010, spare_pages=4)
    for splits in (1, 4):
        note(f"kv_len=1 splits={splits}")
        out16, out32 = run(w, num_splits=splits)
        G = w.Hq // w.Hkv
        for b in range(w.B):
            pg = w.block_table[b, 0]
            for h in range(w.Hq):
                assert np.array_equal(out16[b, 0, h], w.v_cache[pg, 0, h // G])


def test_unused_block_table_entries_and_poison_never_read():
    w = workloads.build("poison", B=3, q_len=1, Hq=8, Hkv=2, D=64, page_size=32, kv_lens=[33, 100, 2],
                        seed=3020, spare_pages=6, max_pages_per_seq=8)
    ref16, ref32 = run(w, num_splits=1)
    bt = w.block_table.copy()
    bt[bt < 0] = np.iinfo(np.int32).max                     # would fault if dereferenced
    for splits in (1, 3):
        out16, out32 = run(w.replace(block_table=bt), num_splits=splits)
        assert np.isfinite(out32).all()
        check(out16, out32, oracle.decode(w), "poison")
    out16, out32 = run(w.replace(block_table=bt), num_splits=1)
    assert np.array_equal(out16, ref16)


def test_gqa_matches_mha_with_repeated_heads():
    w = workloads.build("gqa", B=2, q_len=1, Hq=32, Hkv=4, D=128, page_size=32, kv_lens=[700, 300],
                        seed=3030)
    G = w.Hq // w.Hkv
    mha = w.replace(Hkv=w.Hq, k_cache=np.repeat(w.k_cache, G, axis=2).copy(),
                    v_cache=np.repeat(w.v_cache, G, axis=2).copy())
    a16, a32 = run(w, num_splits=1)
    b16, b32 = run(mha, num_splits=1)
    assert np.abs(a32.astype(np.float64) - b32).max() <= 2e-3


@pytest.mark.parametrize("D", [64, 128])
def test_split_counts_agree(D):
    w = workloads.build("splits", B=2, q_len=1, Hq=16, Hkv=4, D=D, page_size=64, kv_lens=[4000, 1500],
                        seed=3040 + D, outlier_p=0.01)
    ref = oracle.decode(w)
    outs = {}
    for s in (1, 0, 2, 64, 256):
        note(f"splits {s}")
        outs[s] = run(w, num_splits=s)
        check(*outs[s], ref, f"S={s}")
    for s in (0, 2, 64, 256):
        assert np.abs(outs[s][1].astype(np.float64) - outs[1][1]).max() <= 2e-3


def test_zero_mask_is_byte_identical_to_no_mask():
    w = workloads.build("zmask", B=3, q_len=2, Hq=8, Hkv=2, D=128, page_size=32, kv_lens=[300, 77, 1],
                        seed=3050, mask="2d", mask_p=0.0)
    for s in (1, 3):
        a = run(w, num_splits=s)
        b = run(w.replace(mask=None), num_splits=s)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_causal_equals_truncated_single_token_calls():
    w = workloads.build("causal", B=3, q_len=4, Hq=8, Hkv=2, D=64, page_size=32, kv_lens=[300, 45, 4],
                        seed=3060, causal="last")
    out16, out32 = run(w, num_splits=1)
    for i in range(w.q_len):
        lens = np.minimum(w.kv_lens, w.causal_offsets + i + 1).astype(np.int32)
        wi = w.replace(q_len=1, q=w.q[:, i:i + 1].copy(), kv_lens=lens, causal_offsets=None)
        b16, b32 = run(wi, num_splits=1)
        assert np.abs(out32[:, i:i + 1].astype(np.float64) - b32).max() <= 2e-3


def test_replicas_at_other_addresses_are_byte_identical():
    w = workloads.build("replica", B=4, q_len=1, Hq=32, Hkv=8, D=128, page_size=32,
                        kv_lens=[2000, 100, 1, 900], seed=3070, mask="2d")
    d1 = dev_tensors(w)
    pad = torch.empty(12345 * 16, dtype=torch.uint8, device="cuda:0")   # shift later allocations
    d2 = dev_tensors(w)
    assert d1["k"].data_ptr() != d2["k"].data_ptr()
    for s in (1, 5):
        a = run(w, d1, num_splits=s)
        b = run(w, d2, num_splits=s)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    del pad


def test_repeated_calls_are_deterministic():
    w = workloads.ragged(B=32, hi=2048)
    d = dev_tensors(w)
    a = run(w, d)
    for _ in range(3):
        b = run(w, d)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


@pytest.mark.parametrize("D", [128, 32])   # D = 32: a head-paired plan
def test_graph_capture_replay_matches_eager(D):
    """Capture one call into a hipGraph with preallocated buffers, then replay
    after changing q and kv_lens in place; every replay must equal eager."""
    w = workloads.build("graph", B=4, q_len=1, Hq=32, Hkv=8, D=D, page_size=32,
                        kv_lens=[1500, 900, 64, 1000], seed=3080, mask="2d")
    d = dev_tensors(w)
    p = problem(w, num_splits=4)
    o_part, ml_part = pkv.alloc_workspace(p, 4, "cuda:0")
    out = torch.empty(tuple(d["q"].shape), dtype=torch.bfloat16, device="cuda:0")
    out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device="cuda:0")

    def call(stream=None):
        pkv.paged_decode(d["q"], d["k"], d["v"], d["bt"], d["kl"], scale=w.scale, mask=d["mask"],
                         out=out, out_f32=out32, o_part=o_part, ml_part=ml_part, problem=p, stream=stream)

    call()
    torch.cuda.synchronize()
    eager = out32.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for rep in range(4):
        if rep:
            newq = torch.randn(d["q"].shape, generator=torch.Generator().manual_seed(rep)).to(torch.bfloat16)
            d["q"].copy_(newq.to("cuda:0"))
            lens = rng.integers(1, w.kv_lens + 1).astype(np.int32)   # stay within each sequence's pages
            d["kl"].copy_(torch.from_numpy(lens).to("cuda:0"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replay = out32.clone()
        replay16 = out.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(replay.view(torch.int32), out32.view(torch.int32)), f"replay {rep}"
        assert torch.equal(replay16.view(torch.int16), out.view(torch.int16)), f"replay {rep}"
        if rep == 0:
            assert torch.equal(replay.view(torch.int32), eager.view(torch.int32))


def test_runs_on_the_given_stream_in_order():
    """Inputs are written by work queued on a side stream just before the call;
    a correct result shows the kernels ran on that stream after it."""
    w = workloads.build("stream", B=8, q_len=1, Hq=32, Hkv=8, D=128, page_size=32,
                        kv_lens=[2048] * 8, seed=3090)
    ref16, ref32 = run(w, num_splits=0)
    d = dev_tensors(w)
    real_q = d["q"].clone()
    d["q"].zero_()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    big = torch.empty(64 << 20, dtype=torch.float32, device="cuda:0")
    with torch.cuda.stream(s):
        for _ in range(20):
            big.mul_(1.0001)       # long-running work ahead of the copy
        d["q"].copy_(real_q)
    out16, out32 = run(w, d, num_splits=0, stream=s)
    assert np.array_equal(out16, ref16)


def test_wrapper_allocates_on_the_call_stream():
    """A call on a side stream that lets the wrapper allocate its output and
    split workspace: both are allocated with that stream current, so the
    workspace's zero fill runs on it ahead of the kernel.  The current stream
    is kept busy and holds a freed block of the workspace's size filled with
    non-zero counters; were the fill queued there (or that block handed to
    the side stream), the kernel would start on stale counters."""
    w = workloads.build("side_stream", B=8, q_len=1, Hq=32, Hkv=8, D=128, page_size=32,
                        kv_lens=[2048, 1900, 700, 2048, 33, 1500, 2048, 1024], seed=3091)
    p = problem(w, 0)
    S = pkv.num_splits_for(p)
    assert S > 1 and pkv.merges_in_kernel(p, S)
    ref16, _ = run(w, num_splits=S)
    d = dev_tensors(w)
    _, mb = pkv.workspace_bytes(problem(w, S), S)
    junk = torch.full((mb // 4,), 1.0, dtype=torch.float32, device="cuda:0")   # counters 0x3f800000
    del junk                                   # back to the current stream's pool
    big = torch.empty(64 << 20, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    note("side stream call with wrapper-allocated workspace")
    for _ in range(20):
        big.mul_(1.0001)                       # the current stream stays busy
    out = pkv.paged_decode(d["q"], d["k"], d["v"], d["bt"], d["kl"], scale=w.scale, num_splits=S,
                           max_kv_len=w.max_kv_len, stream=s)
    s.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    torch.cuda.synchronize()
    assert np.array_equal(got, ref16)


def test_concurrent_calls_on_two_streams():
    """The library keeps no state between calls: two problems, each with its
    own outputs and split workspace (in-kernel merge counters included), run
    interleaved on two streams at once give the bits each gives alone."""
    wa = workloads.build("conc_a", B=8, q_len=1, Hq=32, Hkv=8, D=128, page_size=32,
                         kv_lens=[3000, 17, 2048, 900, 1, 4096, 333, 1500], seed=3095)
    wb = workloads.build("conc_b", B=5, q_len=4, Hq=16, Hkv=2, D=64, page_size=16,
                         kv_lens=[700, 2100, 64, 5, 1300], seed=3096, causal="last", mask="2d")
    refs = [run(w, num_splits=s) for w, s in ((wa, 6), (wb, 5))]
    ws = [(wa, dev_tensors(wa), 6), (wb, dev_tensors(wb), 5)]
    outs = []
    for w, d, S in ws:
        p = problem(w, S)
        o_part, ml_part = pkv.alloc_workspace(p, S, d["q"].device)
        out = torch.empty(tuple(d["q"].shape), dtype=torch.bfloat16, device=d["q"].device)
        out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device=d["q"].device)
        outs.append((p, o_part, ml_part, out, out32))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    note("two streams, 20 interleaved calls each")
    for _ in range(20):
        for k, ((w, d, S), (p, o_part, ml_part, out, out32)) in enumerate(zip(ws, outs)):
            pkv.paged_decode(d["q"], d["k"], d["v"], d["bt"], d["kl"], scale=w.scale,
                             causal_offset=w.causal_offset, causal_offsets=d["co"], mask=d["mask"],
                             out=out, out_f32=out32, o_part=o_part, ml_part=ml_part, stream=streams[k],
                             problem=p)
    torch.cuda.synchronize()
    for (ref16, ref32), (p, o_part, ml_part, out, out32) in zip(refs, outs):
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), ref16)
        assert np.array_equal(out32.cpu().numpy().view(np.uint32), ref32.view(np.uint32))
        head = ml_part[:pkv.PKV_COUNTER_BYTES // 4]
        assert not head.any().item()   # every counter back at zero


def test_guard_bands_untouched():
    w = workloads.build("canary", B=3, q_len=2, Hq=8, Hkv=2, D=64, page_size=32, kv_lens=[500, 3, 200],
                        seed=3100, mask="2d", causal="last")
    d = dev_tensors(w)
    S = 6
    p = problem(w, num_splits=S)
    ob, mb = pkv.workspace_bytes(p, S)
    n = int(np.prod(d["q"].shape))
    G = 4096  # guard elements on each side
    sent32 = np.float32(-7.25)
    buf16 = torch.full((n + 2 * G,), 0x5A5A, dtype=torch.int16, device="cuda:0")
    buf32 = torch.full((n + 2 * G,), sent32, dtype=torch.float32, device="cuda:0")
    bufo = torch.full((ob // 4 + 2 * G,), sent32, dtype=torch.float32, device="cuda:0")
    bufm = torch.full((mb // 4 + 2 * G,), sent32, dtype=torch.float32, device="cuda:0")
    H = pkv.PKV_COUNTER_BYTES // 4
    bufm[G:G + H].zero_()          # the counter head starts at zero ...
    out = buf16[G:G + n].view(torch.bfloat16).view(d["q"].shape)
    out32 = buf32[G:G + n].view(d["q"].shape)
    pkv.paged_decode(d["q"], d["k"], d["v"], d["bt"], d["kl"], scale=w.scale, causal_offsets=d["co"],
                     mask=d["mask"], out=out, out_f32=out32, o_part=bufo[G:G + ob // 4],
                     ml_part=bufm[G:G + mb // 4], problem=p)
    torch.cuda.synchronize()
    for buf, val in ((buf16, 0x5A5A), (buf32, sent32), (bufo, sent32), (bufm, sent32)):
        h = buf.cpu().numpy()
        assert (h[:G] == val).all() and (h[-G:] == val).all()
    assert not bufm[G:G + H].any().item()   # ... and the call leaves it at zero
    check(out.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy(), oracle.decode(w), "canary")


def test_combine_entry_point_on_hand_made_partials():
    rows, S, D = 37, 5, 128
    rng = np.random.default_rng(7)
    o = rng.standard_normal((rows, S, D)).astype(np.float32)
    m = rng.standard_normal((rows, S)).astype(np.float32) * 3
    l = rng.uniform(0.5, 40, (rows, S)).astype(np.float32)
    l[3, :] = 0
    m[3, :] = -np.inf
    l[5, 2] = 0
    m[5, 2] = -np.inf
    ml = np.stack([m, l], axis=-1)
    ref = oracle.combine(o.astype(np.float64), m.astype(np.float64), l.astype(np.float64))
    od = torch.from_numpy(o).cuda()
    mld = torch.from_numpy(np.ascontiguousarray(ml)).cuda()
    out32 = torch.empty((rows, D), dtype=torch.float32, device="cuda:0")
    out = pkv.combine(od, mld, rows=rows, splits=S, head_dim=D, out_f32=out32)
    torch.cuda.synchronize()
    check(out.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy(), ref, "combine")
    assert not out32[3].any()


def _partials_then_combine(w, d, S):
    """The two-launch path: pkv_paged_decode_partials, then pkv_combine."""
    p = problem(w, num_splits=S)
    ob, mb = pkv.partials_bytes(p, S)
    o_part = torch.empty(ob // 4, dtype=torch.float32, device="cuda:0")
    ml_part = torch.empty(mb // 4, dtype=torch.float32, device="cuda:0")
    pkv.paged_decode_partials(d["q"], d["k"], d["v"], d["bt"], d["kl"], o_part=o_part, ml_part=ml_part,
                              problem=p, causal_offsets=d["co"], mask=d["mask"])
    rows = w.B * w.q_len * w.Hq
    out32 = torch.empty((rows, w.D), dtype=torch.float32, device="cuda:0")
    out = pkv.combine(o_part, ml_part, rows=rows, splits=S, head_dim=w.D, out_f32=out32)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), out32.cpu().numpy()


@pytest.mark.parametrize("shape", [
    dict(B=3, q_len=1, Hq=16, Hkv=8, D=128, page_size=32, kv_lens=[1500, 0, 333]),              # VALU, R=2
    dict(B=2, q_len=2, Hq=16, Hkv=2, D=64, page_size=16, kv_lens=[900, 77], causal="last"),      # MFMA, R=16
    dict(B=2, q_len=1, Hq=48, Hkv=1, D=256, page_size=64, kv_lens=[700, 1000], mask="2d"),        # MFMA, R=48
    dict(B=2, q_len=160, Hq=32, Hkv=8, D=64, page_size=32, kv_lens=[800, 300], causal="last"),   # prefill, R=640
    dict(B=3, q_len=1, Hq=8, Hkv=8, D=32, page_size=32, kv_lens=[1500, 0, 333]),                 # paired VALU
    dict(B=2, q_len=2, Hq=32, Hkv=8, D=32, page_size=16, kv_lens=[900, 77], causal="last",
         mask="2d"),                                                                              # paired MFMA
])
@pytest.mark.parametrize("S", [2, 7, 64])
def test_in_kernel_merge_equals_separate_combine(shape, S):
    """pkv_paged_decode (in-kernel merge by the last workgroup of each unit,
    or the combine kernel for larger grids) equals the split step followed by
    pkv_combine bit for bit: both merges run the same code in split order."""
    w = workloads.build("fusedeq", seed=3200 + S, **shape)
    d = dev_tensors(w)
    note(f"fusedeq S={S} in-kernel merge: {pkv.merges_in_kernel(problem(w, S), S)}")
    a16, a32 = run(w, d, num_splits=S)
    b16, b32 = _partials_then_combine(w, d, S)
    shp = a32.shape
    assert np.array_equal(a16, b16.reshape(shp))
    assert np.array_equal(a32.view(np.uint32), b32.reshape(shp).view(np.uint32))
    check(a16, a32, oracle.decode(w), "fused")


@pytest.mark.parametrize("hpb", [1, 0])
def test_many_units_use_the_combine_kernel(hpb):
    """More than PKV_MAX_FUSED_UNITS units with several splits: split kernel +
    combine kernel, with the (m, l) data after the counter head."""
    # matrix-core rows at D = 32: forced one kv head per workgroup, B * Hkv units; or head
    # pairing (automatic grouping), two pairs of kv heads per workgroup at three splits, 2 B units
    B = pkv.PKV_MAX_FUSED_UNITS // (8 if hpb else 2) + 9
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 150, B)
    w = workloads.build("manyunits", B=B, q_len=1, Hq=64, Hkv=8, D=32, page_size=16,
                        kv_lens=lens, seed=3300)
    info = pkv.plan(problem(w, num_splits=3, heads_per_block=hpb))
    assert info.paired_heads == (hpb == 0)
    assert info.units > pkv.PKV_MAX_FUSED_UNITS and not info.merge_in_kernel and info.kernels == 2
    out16, out32 = run(w, num_splits=3, heads_per_block=hpb)
    seqs = [0, 1, int(np.argmax(lens)), B // 2, B - 1]
    ref = oracle.decode(sub_batch(w, seqs))
    check(out16[seqs], out32[seqs], ref, "manyunits")


def test_one_workspace_serves_calls_of_any_shape():
    """A workspace cleared once serves a sequence of calls of different shapes
    and split counts (in-kernel merge and combine-kernel paths mixed); the
    counter head is zero after every call."""
    shapes = [
        dict(B=4, q_len=1, Hq=32, Hkv=8, D=128, page_size=32, kv_lens=[800, 20, 0, 1400]),
        dict(B=2400, q_len=1, Hq=64, Hkv=8, D=32, page_size=16, kv_lens=[70] * 2400),  # 4800 units (paired)
        dict(B=2, q_len=3, Hq=16, Hkv=2, D=64, page_size=8, kv_lens=[300, 41], causal="last"),
        dict(B=1, q_len=1, Hq=8, Hkv=1, D=32, page_size=64, kv_lens=[5000]),
    ]
    ws = [workloads.build(f"reuse{i}", seed=3400 + i, **kw) for i, kw in enumerate(shapes)]
    plans = [(w, S) for w in ws for S in (5, 2)]
    assert {pkv.plan(problem(w, num_splits=S)).merge_in_kernel for w, S in plans} == {0, 1}
    need_o = max(pkv.workspace_bytes(problem(w, num_splits=S), S)[0] for w, S in plans)
    need_m = max(pkv.workspace_bytes(problem(w, num_splits=S), S)[1] for w, S in plans)
    o_part = torch.empty(need_o // 4, dtype=torch.float32, device="cuda:0")
    ml_part = torch.empty(need_m // 4, dtype=torch.float32, device="cuda:0")
    ml_part.fill_(3.5)
    pkv.workspace_clear(ml_part)
    torch.cuda.synchronize()
    assert not ml_part.any().item()
    H = pkv.PKV_COUNTER_BYTES // 4
    for w, S in plans:
        note(f"reuse {w.name} B={w.B} S={S}")
        d = dev_tensors(w)
        p = problem(w, num_splits=S)
        out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device="cuda:0")
        out = pkv.paged_decode(d["q"], d["k"], d["v"], d["bt"], d["kl"], scale=w.scale,
                               causal_offsets=d["co"], mask=d["mask"], out_f32=out32,
                               o_part=o_part, ml_part=ml_part, problem=p)
        torch.cuda.synchronize()
        assert not ml_part[:H].any().item()
        seqs = list(range(min(w.B, 6)))
        ref = oracle.decode(sub_batch(w, seqs))
        check(out.view(torch.int16).cpu().numpy().view(np.uint16)[seqs], out32.cpu().numpy()[seqs], ref,
              w.name)


def test_both_merge_paths_are_exercised():
    """The shapes above cover both merge paths: in-kernel up to
    PKV_MAX_FUSED_UNITS units, the combine kernel beyond."""
    shapes = [(dict(B=3, q_len=1, Hq=32, Hkv=8, D=128, page_size=32, kv_lens=[1500, 0, 333]), 7),
              (dict(B=3, q_len=1, Hq=32, Hkv=8, D=128, page_size=32, kv_lens=[1500, 0, 333]), 64),
              (dict(B=2400, q_len=1, Hq=64, Hkv=8, D=32, page_size=16, kv_lens=[70] * 2400), 2)]
    flags = [pkv.merges_in_kernel(problem(workloads.build("paths", seed=1, **kw), S), S) for kw, S in shapes]
    assert flags == [True, True, False]


# Keys stored past 2^32 elements of a cache (8 GiB of bf16): page and sequence
# offsets are 64-bit products, so the same keys placed there give the same
# bytes as in a small cache.  One case per kernel family: the VALU kernel
# (one row per kv head), the 32-row matrix-core kernel and the prefill-shaped
# one (512 rows per kv head).
FAR = 1 << 32
FAR_CASES = [
    ("split_decode_valu", lambda: workloads.build("far_valu", B=3, q_len=1, Hq=8, Hkv=8, D=64, page_size=32,
                                                   kv_lens=[700, 33, 1500], seed=3101, mask="2d")),
    ("split_decode_mfma", lambda: workloads.build("far_mfma", B=3, q_len=1, Hq=32, Hkv=8, D=128, page_size=16,
                                                   kv_lens=[1200, 5, 640], seed=3102)),
    ("split_decode_mfma", lambda: workloads.build("far_paired", B=3, q_len=1, Hq=32, Hkv=8, D=32, page_size=16,
                                                   kv_lens=[1200, 5, 640], seed=3104, mask="2d")),   # head pairing
    ("split_prefill_mfma", lambda: workloads.build("far_prefill", B=2, q_len=128, Hq=16, Hkv=4, D=64, page_size=32,
                                                    kv_lens=[900, 300], seed=3103).replace(
                                                        causal_offset=workloads.CAUSAL_LAST)),
]


@pytest.mark.parametrize("i", range(len(FAR_CASES)))
def test_pages_past_4g_elements(i):
    family, make = FAR_CASES[i]
    w = make()
    stride = w.page_size * w.Hkv * w.D
    n = w.num_pages
    big = (FAR + stride - 1) // stride + n          # pages n .. big - 1 lie wholly past element 2^32
    assert (big - n) * stride >= FAR
    p_big = problem(w)
    p_big.num_pages = big
    assert pkv.kernel_family(p_big) == family
    note(f"far pages {w.name} num_pages={big} ({2 * big * stride * 2 / 2**30:.1f} GiB of K/V)")
    ref16, ref32 = run(w, num_splits=3)
    d = dev_tensors(w)
    shape = (big, w.page_size, w.Hkv, w.D)
    kb = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    vb = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    kb[big - n:] = d["k"]
    vb[big - n:] = d["v"]
    bt = torch.where(d["bt"] >= 0, d["bt"] + (big - n), d["bt"])
    p_big.num_splits = 3
    out = torch.empty(tuple(d["q"].shape), dtype=torch.bfloat16, device="cuda:0")
    out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device="cuda:0")
    pkv.paged_decode(d["q"], kb, vb, bt, d["kl"], scale=w.scale, causal_offset=w.causal_offset,
                     causal_offsets=d["co"], mask=d["mask"], out=out, out_f32=out32, problem=p_big)
    torch.cuda.synchronize()
    got16 = out.view(torch.int16).cpu().numpy().view(np.uint16)
    got32 = out32.cpu().numpy()
    del kb, vb
    torch.cuda.empty_cache()
    assert np.array_equal(got16, ref16)
    assert np.array_equal(got32.view(np.uint32), ref32.view(np.uint32))


@pytest.mark.parametrize("layout", ["blhd", "bhld"])
def test_contiguous_sequences_past_4g_elements(layout):
    w = workloads.build("far_contig", B=2, q_len=2, Hq=8, Hkv=2, D=64, page_size=32, kv_lens=[1000, 777],
                        seed=3104, causal="last")
    from gpu_util import run_contiguous
    ref16, ref32, k, v = run_contiguous(w, layout, num_splits=3)
    cap_small = k.shape[1] if layout == "blhd" else k.shape[2]
    # the last (sequence, head) region starts past element 2^32
    per_seq = FAR // (w.Hkv * w.D) + 1 if layout == "blhd" else FAR // (3 * w.D) + 1
    cap = max(per_seq, cap_small)
    last_region = (w.B - 1) * cap * w.Hkv * w.D if layout == "blhd" else (w.B * w.Hkv - 1) * cap * w.D
    assert last_region >= FAR
    note(f"far contiguous {layout} capacity={cap} ({2 * w.B * w.Hkv * cap * w.D * 2 / 2**30:.1f} GiB of K/V)")
    d = dev_tensors(w)
    ks = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    vs = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    shape = (w.B, cap, w.Hkv, w.D) if layout == "blhd" else (w.B, w.Hkv, cap, w.D)
    kb = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    vb = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    if layout == "blhd":
        kb[:, :cap_small] = ks
        vb[:, :cap_small] = vs
    else:
        kb[:, :, :cap_small] = ks
        vb[:, :, :cap_small] = vs
    out32 = torch.empty(tuple(d["q"].shape), dtype=torch.float32, device="cuda:0")
    out = pkv.contiguous_decode(d["q"], kb, vb, d["kl"], layout=layout, scale=w.scale,
                                causal_offset=w.causal_offset, causal_offsets=d["co"], mask=d["mask"],
                                num_splits=3, max_kv_len=w.max_kv_len, out_f32=out32)
    torch.cuda.synchronize()
    got16 = out.view(torch.int16).cpu().numpy().view(np.uint16)
    got32 = out32.cpu().numpy()
    del kb, vb
    torch.cuda.empty_cache()
    assert np.array_equal(got16, ref16)
    assert np.array_equal(got32.view(np.uint32), ref32.view(np.uint32))
