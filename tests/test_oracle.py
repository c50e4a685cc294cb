"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself: hand-worked examples
(tests/golden), closed forms, a separate brute-force implementation, and
invariants the operation must satisfy.  A plausible slip in the oracle (a
dropped scale, a wrong GQA head map, an off-by-one causal limit, a wrong page
index, a missing mask term, a wrong combine weight) fails at least one test
here; ``test_planted_mistakes_are_caught`` plants several of them on the CPU
to show it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def f32_to_bf16_bits(x) -> np.ndarray:
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    bits = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, np.asarray(x, dtype=np.float32)), "input not exact in bf16"
    return bits.copy()


def from_case(c) -> Workload:
    mask = None
    if c["mask"] is not None:
        mask = np.array([[float(v) for v in row] for row in c["mask"]], dtype=np.float32)
    return Workload(
        name=c["name"], B=c["B"], q_len=c["q_len"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"],
        page_size=c["page_size"], q=f32_to_bf16_bits(c["q"]),
        k_cache=f32_to_bf16_bits(c["k_pages"]), v_cache=f32_to_bf16_bits(c["v_pages"]),
        block_table=np.array(c["block_table"], dtype=np.int32),
        kv_lens=np.array(c["kv_lens"], dtype=np.int32), scale=float(np.float32(c["scale"])),
        causal_offset=c["causal_offset"], mask=mask)


CASES = json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_worked_examples(case):
    w = from_case(case)
    exp = np.array(case["expected"], dtype=np.float64)
    np.testing.assert_allclose(oracle.decode(w), exp, rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.bruteforce_decode(w), exp, rtol=0, atol=1e-15)


def small(seed, **kw):
    """Random tiny problem for brute-force comparison."""
    g = torch.Generator().manual_seed(seed)
    B = kw.pop("B", 3)
    lens = kw.pop("lens", None)
    if lens is None:
        lens = torch.randint(0, 70, (B,), generator=g).tolist()
    args = dict(B=B, q_len=2, Hq=4, Hkv=2, D=16, page_size=8)
    args.update(kw)
    return workloads.build("small", kv_lens=lens, seed=seed, spare_pages=2, **args)


BRUTE = [
    dict(),
    dict(q_len=1, Hq=8, Hkv=8, D=32),
    dict(q_len=3, Hq=6, Hkv=1, D=8, page_size=4),
    dict(q_len=4, Hq=4, Hkv=2, D=64, page_size=16, causal=5),
    dict(q_len=4, causal="last", mask="3d", mask_p=0.3),
    dict(mask="2d", mask_p=0.5),
    dict(q_len=2, Hq=12, Hkv=4, mask="2d", mask_p=0.95),     # many fully-masked rows
    dict(lens=[0, 1, 9], q_len=1),
    dict(D=128, page_size=32, lens=[33, 64, 65]),
]


@pytest.mark.parametrize("i", range(len(BRUTE)))
def test_oracle_matches_bruteforce(i):
    w = small(100 + i, **dict(BRUTE[i]))
    a = oracle.decode(w)
    b = oracle.bruteforce_decode(w)
    assert np.isfinite(a).all()
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_kv_len_one_returns_v_row_exactly():
    w = small(7, lens=[1, 1, 1], q_len=1, Hq=8, Hkv=2, D=32)
    out = oracle.decode(w)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        pg = w.block_table[b, 0]
        for h in range(w.Hq):
            v = oracle.bf16_bits_to_f64(w.v_cache[pg, 0, h // G])
            assert np.array_equal(out[b, 0, h], v)


def test_identical_keys_give_mean_of_v():
    w = small(8, lens=[5, 40, 17], q_len=1)
    w.k_cache[:] = w.k_cache[w.block_table[0, 0], 0, 0][None, None, None, :]
    out = oracle.decode(w)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(w.kv_lens[b])
        rows = [oracle.bf16_bits_to_f64(w.v_cache[w.block_table[b, j // w.page_size], j % w.page_size])
                for j in range(L)]
        mean = np.mean(np.stack(rows), axis=0)           # [Hkv, D]
        for h in range(w.Hq):
            np.testing.assert_allclose(out[b, 0, h], mean[h // G], rtol=0, atol=1e-13)


def test_scale_zero_gives_mean_of_v():
    w = small(9, lens=[3, 30, 64], q_len=1).replace(scale=0.0)
    out = oracle.decode(w)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(w.kv_lens[b])
        rows = [oracle.bf16_bits_to_f64(w.v_cache[w.block_table[b, j // w.page_size], j % w.page_size])
                for j in range(L)]
        mean = np.mean(np.stack(rows), axis=0)
        for h in range(w.Hq):
            np.testing.assert_allclose(out[b, 0, h], mean[h // G], rtol=0, atol=1e-13)


def test_empty_and_fully_masked_rows_are_zero():
    w = small(10, lens=[0, 12, 12], q_len=1, mask="2d", mask_p=0.0)
    w.mask[2, :] = -np.inf
    out = oracle.decode(w)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.array_equal(out[2], np.zeros_like(out[2]))
    assert np.abs(out[1]).sum() > 0


def test_gqa_equals_mha_with_repeated_kv_heads():
    w = small(11, lens=[20, 50, 9], Hq=8, Hkv=2, q_len=2)
    G = w.Hq // w.Hkv
    mha = w.replace(Hkv=w.Hq, k_cache=np.repeat(w.k_cache, G, axis=2).copy(),
                    v_cache=np.repeat(w.v_cache, G, axis=2).copy())
    assert np.array_equal(oracle.decode(w), oracle.decode(mha))


def permute_pages(w: Workload, seed: int) -> Workload:
    """Same logical content, physical pages shuffled (a new random slot for each)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_pages)          # old page p -> new slot perm[p]
    k = np.empty_like(w.k_cache)
    v = np.empty_like(w.v_cache)
    k[perm] = w.k_cache
    v[perm] = w.v_cache
    bt = np.where(w.block_table >= 0, perm[np.clip(w.block_table, 0, None)], -1).astype(np.int32)
    return w.replace(k_cache=k, v_cache=v, block_table=bt)


def test_page_permutation_is_byte_identical():
    w = small(12, lens=[31, 64, 70], mask="2d", causal=40)
    a = oracle.decode(w)
    b = oracle.decode(permute_pages(w, 1))
    assert np.array_equal(a, b)


def test_causal_equals_truncated_single_token_calls():
    w = small(13, lens=[30, 47, 64], q_len=4, causal="last")
    out = oracle.decode(w)
    for i in range(w.q_len):
        lens = np.minimum(w.kv_lens, w.causal_offsets + i + 1).astype(np.int32)
        wi = w.replace(q_len=1, q=w.q[:, i:i + 1].copy(), kv_lens=lens, causal_offsets=None,
                       causal_offset=-1)
        assert np.array_equal(out[:, i:i + 1], oracle.decode(wi))


def test_zero_mask_is_byte_identical_to_no_mask():
    w = small(14, lens=[11, 40, 64], mask="2d", mask_p=0.0)
    assert np.array_equal(oracle.decode(w), oracle.decode(w.replace(mask=None)))


def test_neg_inf_mask_equals_deleting_the_key():
    w = small(15, lens=[20, 20, 20], q_len=1, mask="2d", mask_p=0.0, page_size=4)
    j = 6
    w.mask[:, j] = -np.inf
    out = oracle.decode(w)
    # rebuild every sequence without key j: contiguous K/V, one key per page
    B, Hkv, D = w.B, w.Hkv, w.D
    keys, vals = [], []
    for b in range(B):
        for jj in range(int(w.kv_lens[b])):
            if jj == j:
                continue
            pg, sl = w.block_table[b, jj // w.page_size], jj % w.page_size
            keys.append(w.k_cache[pg, sl])
            vals.append(w.v_cache[pg, sl])
    n = len(keys)
    per = n // B
    bt = np.arange(n, dtype=np.int32).reshape(B, per)
    w2 = w.replace(page_size=1, k_cache=np.stack(keys)[:, None], v_cache=np.stack(vals)[:, None],
                   block_table=bt, kv_lens=np.full(B, per, dtype=np.int32), mask=None)
    np.testing.assert_allclose(out, oracle.decode(w2), rtol=0, atol=1e-13)


def test_constant_added_to_mask_leaves_output():
    w = small(16, lens=[33, 5, 64], mask="2d", mask_p=0.2)
    shifted = w.mask + np.float32(3.0)      # -inf stays -inf
    np.testing.assert_allclose(oracle.decode(w), oracle.decode(w.replace(mask=shifted)),
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("cuts", [[0, 64], [0, 7, 64], [0, 16, 32, 48, 64], [0, 1, 2, 3, 64, 64]])
def test_split_partials_combine_to_full(cuts):
    w = small(17, lens=[0, 33, 64], q_len=2, mask="2d", mask_p=0.3, causal="last")
    full = oracle.decode(w)
    parts = [oracle.partial(w, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    rows = w.B * w.q_len * w.Hq
    o = np.stack([p[0].reshape(rows, w.D) for p in parts], axis=1)
    m = np.stack([p[1].reshape(rows) for p in parts], axis=1)
    l = np.stack([p[2].reshape(rows) for p in parts], axis=1)
    merged = oracle.combine(o, m, l).reshape(full.shape)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-13)


def test_combine_closed_forms():
    D = 4
    o = np.array([[[1.0, 2, 3, 4], [5, 6, 7, 8]]])
    # equal (m, l): plain mean of the partials
    np.testing.assert_allclose(oracle.combine(o, np.array([[0.5, 0.5]]), np.array([[2.0, 2.0]])),
                               [[3.0, 4, 5, 6]], rtol=0, atol=1e-15)
    # weights l_s * exp(m_s - M): (1 * e^0, 1 * e^-1) -> e/(1+e), 1/(1+e)
    a, b = 0.7310585786300049, 0.2689414213699951
    np.testing.assert_allclose(oracle.combine(o, np.array([[1.0, 0.0]]), np.array([[1.0, 1.0]])),
                               [a * o[0, 0] + b * o[0, 1]], rtol=0, atol=1e-15)
    # empty partial (m=-inf, l=0) carries no weight; all empty -> 0
    np.testing.assert_allclose(oracle.combine(o, np.array([[-np.inf, 3.0]]), np.array([[0.0, 1.0]])),
                               o[:, 1], rtol=0, atol=0)
    assert np.array_equal(oracle.combine(o, np.array([[-np.inf, -np.inf]]), np.zeros((1, 2))),
                          np.zeros((1, D)))


def test_openmp_is_byte_identical_to_one_thread():
    w = small(18, B=6, lens=[5, 70, 64, 1, 33, 12], mask="2d", causal="last", q_len=3)
    assert np.array_equal(oracle.decode(w, threads=1), oracle.decode(w, threads=4))


def test_page_tails_and_spares_are_never_read():
    # workloads poisons every unused slot with NaN; the oracle output is finite
    w = small(19, lens=[9, 17, 63], q_len=2, mask="2d")
    assert np.isnan(oracle.bf16_bits_to_f64(w.k_cache)).any()
    assert np.isfinite(oracle.decode(w)).all()


def test_planted_mistakes_are_caught():
    """Each plausible slip, planted in a copy of the definition, breaks a pin."""
    w = small(20, lens=[9, 40, 64], q_len=2, Hq=8, Hkv=2, causal="last", mask="2d")
    good = oracle.bruteforce_decode(w)
    np.testing.assert_allclose(oracle.decode(w), good, rtol=0, atol=1e-12)
    G = w.Hq // w.Hkv
    # wrong GQA map (h % Hkv instead of h // G): differs from the repeat-interleave reading
    wrong = w.replace(k_cache=np.tile(w.k_cache, (1, 1, G, 1)), v_cache=np.tile(w.v_cache, (1, 1, G, 1)),
                      Hkv=w.Hq)
    assert not np.allclose(oracle.decode(wrong), good, atol=1e-6)
    # causal off by one (offset + 1)
    off = w.replace(causal_offsets=w.causal_offsets + 1)
    assert not np.allclose(oracle.decode(off), good, atol=1e-6)
    # dropped scale
    assert not np.allclose(oracle.decode(w.replace(scale=1.0)), good, atol=1e-6)
    # dropped mask
    assert not np.allclose(oracle.decode(w.replace(mask=None)), good, atol=1e-6)
    # wrong page (block-table rows swapped between two sequences of equal page count)
    bt = w.block_table.copy()
    bt[[1, 2]] = bt[[2, 1]]
    assert not np.allclose(oracle.decode(w.replace(block_table=bt, kv_lens=np.array([9, 64, 64], np.int32))),
                           oracle.bruteforce_decode(w.replace(kv_lens=np.array([9, 64, 64], np.int32))),
                           atol=1e-6)
    # combine with l dropped from the weight
    o = np.array([[[1.0], [3.0]]])
    m = np.array([[0.0, 0.0]])
    l = np.array([[1.0, 3.0]])
    assert abs(oracle.combine(o, m, l)[0, 0] - (1 * 1 + 3 * 3) / 4) < 1e-15
    assert abs(oracle.combine(o, m, l)[0, 0] - 2.0) > 0.4


def test_workload_shapes_and_page_tables():
    w = workloads.tiny()
    assert w.num_pages == 8 and w.max_pages_per_seq == 4
    used = w.block_table[w.block_table >= 0]
    assert sorted(used.tolist()) == sorted(set(used.tolist())) and len(used) == 6
    assert (w.block_table[0, 2:] == -1).all()
    assert w.q.shape == (2, 1, 8, 64) and w.k_cache.shape == (8, 32, 2, 64)
    r = workloads.ragged(B=64)
    assert r.kv_lens.min() >= 32 and r.kv_lens.max() <= 8192
    assert (r.causal_offsets == r.kv_lens - 4).all()
    assert r.num_pages == int(((r.kv_lens + 31) // 32).sum())
    s = workloads.sweep(32, 64, B=2, L=256)
    assert s.mask.shape == (2, 256) and 0.02 < np.isinf(s.mask).mean() < 0.25


@pytest.mark.parametrize("i", range(len(BRUTE)))
def test_contiguous_kv_matches_bruteforce_and_paged(i):
    """Contiguous K/V (both layouts, a capacity beyond the longest sequence
    whose extra rows are NaN): the same values as the brute-force path over
    the paged copy, and the same bits as the paged oracle."""
    w = small(200 + i, **dict(BRUTE[i]))
    paged = oracle.decode(w)
    brute = oracle.bruteforce_decode(w)
    for layout in ("blhd", "bhld"):
        k, v = workloads.to_contiguous(w, layout, capacity=max(1, w.max_kv_len) + 5)
        got = oracle.decode_contiguous(w, k, v, layout)
        assert np.isfinite(got).all()
        assert np.array_equal(got, paged)
        np.testing.assert_allclose(got, brute, rtol=0, atol=1e-12)


def test_contiguous_layouts_place_keys_as_documented():
    """to_contiguous puts key j of sequence b, kv head g at [b, j, g] (blhd)
    and [b, g, j] (bhld), and NaN past kv_lens[b]."""
    w = small(300, lens=[5, 0, 17], Hkv=2, Hq=4)
    kb, vb = workloads.to_contiguous(w, "blhd", capacity=20)
    kh, vh = workloads.to_contiguous(w, "bhld", capacity=20)
    P = w.page_size
    for b in range(w.B):
        L = int(w.kv_lens[b])
        for j in range(20):
            for g in range(w.Hkv):
                if j < L:
                    pg = int(w.block_table[b, j // P])
                    assert np.array_equal(kb[b, j, g], w.k_cache[pg, j % P, g])
                    assert np.array_equal(vh[b, g, j], w.v_cache[pg, j % P, g])
                else:
                    assert (kb[b, j, g] == workloads.BF16_NAN).all() and (vh[b, g, j] == workloads.BF16_NAN).all()


# ---- varlen batches (per-sequence query-token counts) ----------------------

VARLEN = [
    dict(q_lens=[1, 5, 0, 3], lens=[40, 9, 20, 3], causal="lastv"),             # last: n_b = L_b
    dict(q_lens=[4, 1, 2], lens=[2, 30, 0], causal="lastv"),                    # n > L: leading rows see nothing
    dict(q_lens=[3, 1, 6], lens=[50, 17, 64], causal="lastv", mask="3d", mask_p=0.3),
    dict(q_lens=[2, 2, 1], lens=[11, 64, 5], mask="2d", mask_p=0.4),            # causal off
    dict(q_lens=[5, 0, 1], lens=[33, 8, 70], causal=3),                         # one fixed position
    dict(q_lens=[1, 1, 1], lens=[7, 1, 40], causal="lastv", Hq=8, Hkv=1, D=32),
]


def varlen_small(seed, q_lens, lens, **kw):
    args = dict(B=len(q_lens), Hq=4, Hkv=2, D=16, page_size=8)
    args.update(kw)
    return workloads.varlen("varlen", q_lens=q_lens, kv_lens=lens, seed=seed, spare_pages=2, **args)


@pytest.mark.parametrize("i", range(len(VARLEN)))
def test_varlen_matches_token_by_token_bruteforce(i):
    w = varlen_small(400 + i, **dict(VARLEN[i]))
    a = oracle.decode_varlen(w)
    b = oracle.bruteforce_varlen(w)
    assert a.shape == (w.total_tokens, w.Hq, w.D)
    assert np.isfinite(a).all()
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_varlen_with_explicit_offsets_equals_the_fixed_batch():
    """Equal token counts and causal offsets L_b - q_len given per sequence:
    the varlen form is the fixed-length batch, bit for bit; and CAUSAL_LAST
    gives the same offsets."""
    w = small(410, B=4, lens=[9, 30, 64, 17], q_len=3, causal="last", mask="3d", mask_p=0.2)
    fixed = oracle.decode(w).reshape(-1, w.Hq, w.D)
    assert np.array_equal(oracle.decode_varlen(w), fixed)
    last = w.replace(causal_offsets=None, causal_offset=workloads.CAUSAL_LAST)
    assert np.array_equal(oracle.decode_varlen(last), fixed)
    assert np.array_equal(oracle.decode_varlen(last.replace(q_lens=np.full(4, 3, np.int32))), fixed)


def _sdpa_rows(w, b, n, L, is_causal):
    """torch's scaled_dot_product_attention in float64 on sequence b's keys
    (gathered through its page table, kv heads repeated to the query heads)."""
    P, G = w.page_size, w.Hq // w.Hkv
    idx = [(int(w.block_table[b, j // P]), j % P) for j in range(L)]
    K = np.stack([oracle.bf16_bits_to_f64(w.k_cache[pg, s]) for pg, s in idx])      # [L, Hkv, D]
    V = np.stack([oracle.bf16_bits_to_f64(w.v_cache[pg, s]) for pg, s in idx])
    q = torch.tensor(oracle.bf16_bits_to_f64(w.q[b, :n])).permute(1, 0, 2)          # [Hq, n, D]
    k = torch.tensor(K).repeat_interleave(G, dim=1).permute(1, 0, 2)
    v = torch.tensor(V).repeat_interleave(G, dim=1).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=is_causal,
                                                         scale=float(np.float32(w.scale)))
    return o.permute(1, 0, 2).numpy()


def test_causal_last_prefill_of_whole_sequence_is_textbook_causal_attention():
    """n_b = L_b with CAUSAL_LAST is causal self-attention over the sequence,
    which torch's scaled_dot_product_attention(is_causal=True) computes
    independently (its causal mask is aligned at token 0)."""
    w = varlen_small(420, q_lens=[12, 1, 7], lens=[12, 1, 7], causal="lastv", Hq=6, Hkv=2, D=32)
    got = oracle.decode_varlen(w)
    t = 0
    for b in range(w.B):
        n = int(w.q_lens[b])
        np.testing.assert_allclose(got[t:t + n], _sdpa_rows(w, b, n, n, True), rtol=0, atol=1e-12)
        t += n


def test_decode_token_with_causal_last_sees_every_key():
    """n_b = 1 with CAUSAL_LAST: the token is the last key, so it sees all L_b
    keys: non-causal attention of one query (torch's sdpa, float64)."""
    w = varlen_small(430, q_lens=[1, 1], lens=[37, 64], causal="lastv", Hq=4, Hkv=4, D=16)
    got = oracle.decode_varlen(w)
    for b in range(2):
        np.testing.assert_allclose(got[b:b + 1], _sdpa_rows(w, b, 1, int(w.kv_lens[b]), False), rtol=0,
                                   atol=1e-12)


def test_packed_q_and_mixed_workload():
    w = varlen_small(440, q_lens=[2, 0, 3], lens=[5, 6, 7])
    q, cu = w.packed_q()
    assert cu.tolist() == [0, 2, 2, 5] and q.shape == (5, 4, 16)
    assert np.array_equal(q[2:5], w.q[2, :3]) and np.array_equal(q[:2], w.q[0, :2])
    m = workloads.mixed()
    assert m.q_lens.max() <= m.q_len == 64 and m.q_lens.min() >= 1
    assert (m.kv_lens >= m.q_lens).all() and m.causal_offset == workloads.CAUSAL_LAST
    assert 0 < (m.q_lens > 1).sum() < m.B
    with pytest.raises(ValueError):
        oracle.decode(m)


def test_varlen_closed_forms():
    """Hand-checkable varlen cases (causal "last"): a token that sees one key
    returns that key's V row exactly; tokens whose visible keys are all equal
    return the exact mean of the visible V rows; a sequence with no tokens
    adds no rows; a token with no visible key (more tokens than keys) is 0."""
    P, D, Hkv, Hq = 4, 8, 1, 2
    rng = np.random.default_rng(11)
    kv = lambda n: f32_to_bf16_bits(np.round(rng.normal(size=(n, D)) * 4) / 4)
    # sequence 0: 2 keys, 2 tokens; sequence 1: no tokens; sequence 2: 3 keys, 1 token;
    # sequence 3: 1 key, 2 tokens (the first sees nothing)
    L = [2, 5, 3, 1]
    q_lens = [2, 0, 1, 2]
    pages = [[0], [1, 2], [3], [4]]
    k = np.zeros((5, P, Hkv, D), np.uint16)
    v = np.zeros((5, P, Hkv, D), np.uint16)
    same_key = kv(1)[0]
    for b, pg in enumerate(pages):
        for j in range(L[b]):
            k[pg[j // P], j % P, 0] = same_key
            v[pg[j // P], j % P, 0] = kv(1)[0]
    q = np.zeros((4, 2, Hq, D), np.uint16)
    q[:] = kv(1)[0]
    bt = np.full((4, 2), -1, np.int32)
    for b, pg in enumerate(pages):
        bt[b, :len(pg)] = pg
    w = Workload(name="closed", B=4, q_len=2, Hq=Hq, Hkv=Hkv, D=D, page_size=P, q=q, k_cache=k, v_cache=v,
                 block_table=bt, kv_lens=np.array(L, np.int32), scale=0.5, causal_offset=workloads.CAUSAL_LAST,
                 q_lens=np.array(q_lens, np.int32))
    out = oracle.decode_varlen(w)
    assert out.shape == (5, Hq, D)
    vrow = lambda b, j: oracle.bf16_bits_to_f64(v[pages[b][j // P], j % P, 0])
    for h in range(Hq):
        assert np.array_equal(out[0, h], vrow(0, 0))                           # token 0 of seq 0: key 0 only
        assert np.allclose(out[1, h], (vrow(0, 0) + vrow(0, 1)) / 2, atol=1e-15)  # token 1: keys 0, 1
        assert np.allclose(out[2, h], (vrow(2, 0) + vrow(2, 1) + vrow(2, 2)) / 3, atol=1e-15)
        assert (out[3, h] == 0).all()                                          # seq 3, token 0: position -1
        assert np.array_equal(out[4, h], vrow(3, 0))                           # seq 3, token 1: key 0
    np.testing.assert_allclose(oracle.bruteforce_varlen(w), out, rtol=0, atol=1e-15)
