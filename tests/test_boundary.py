"""The C-ABI boundary on the CPU: the library loads, exports every symbol that
include/pkv.h declares, rejects bad arguments with the documented status
before any HIP call, sizes workspace and splits by the documented
arithmetic, and links no allocation, copy or synchronisation routine."""
import ctypes
import os
import re
import subprocess

import pytest

import paged_kv_split_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    assert declared_functions() == sorted(pkv.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = pkv.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True, text=True).stdout
    defined = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in defined, name


def test_link_audit_no_alloc_copy_or_sync():
    out = subprocess.run(["nm", "-D", "--undefined-only", pkv.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1].split("@")[0] for l in out.splitlines() if l.strip()}
    banned = [s for s in syms if re.match(
        r"^hip(Malloc|Free|HostMalloc|HostFree|MallocAsync|FreeAsync|Memcpy|Memset|StreamSynchronize|"
        r"DeviceSynchronize|EventSynchronize|MallocManaged)", s) and not s.endswith("Async") or
        s in ("hipMemcpy", "hipMemset", "hipMalloc", "hipFree")]
    # async copies are banned too: the library only launches kernels
    banned += [s for s in syms if s.startswith(("hipMemcpy", "hipMemset", "hipMalloc", "hipFree"))]
    assert not banned, banned


def base_problem(**kw):
    args = dict(batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32, num_pages=8,
                max_pages_per_seq=4, max_kv_len=100, scale=0.125)
    args.update(kw)
    return pkv.make_problem(**args)


FAKE = 0x10000  # 64 KiB-aligned fake addresses: never dereferenced, checks fail first


def call(p, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, kl=FAKE, co=0, mask=0, o=0, ob=0, ml=0, mb=0, out=FAKE,
             out32=0)
    a.update(ptrs)
    return pkv.paged_decode_raw(p, a["q"], a["k"], a["v"], a["bt"], a["kl"], a["co"], a["mask"], a["o"],
                                a["ob"], a["ml"], a["mb"], a["out"], a["out32"], 0)


@pytest.mark.parametrize("field,value,status", [
    ("q_len", 0, pkv.PKV_ERR_SHAPE),
    ("num_q_heads", 0, pkv.PKV_ERR_SHAPE),
    ("num_kv_heads", 3, pkv.PKV_ERR_SHAPE),           # 8 % 3 != 0
    ("head_dim", 96, pkv.PKV_ERR_UNSUPPORTED),
    ("head_dim", 512, pkv.PKV_ERR_UNSUPPORTED),
    ("page_size", 48, pkv.PKV_ERR_UNSUPPORTED),
    ("page_size", 8192, pkv.PKV_ERR_UNSUPPORTED),
    ("page_size", 0, pkv.PKV_ERR_UNSUPPORTED),
    ("max_pages_per_seq", 0, pkv.PKV_ERR_SHAPE),
    ("max_kv_len", 129, pkv.PKV_ERR_SHAPE),           # > 4 pages * 32
    ("max_kv_len", -1, pkv.PKV_ERR_SHAPE),
    ("batch", -1, pkv.PKV_ERR_SHAPE),
    ("causal_offset", -3, pkv.PKV_ERR_SHAPE),
    ("num_splits", -1, pkv.PKV_ERR_SHAPE),
    ("num_splits", 257, pkv.PKV_ERR_UNSUPPORTED),
    ("scale", float("nan"), pkv.PKV_ERR_SHAPE),
    ("scale", float("inf"), pkv.PKV_ERR_SHAPE),
    ("mask_stride_b", -4, pkv.PKV_ERR_SHAPE),
    ("num_pages", -1, pkv.PKV_ERR_SHAPE),
])
def test_shape_errors(field, value, status):
    p = base_problem(**{field: value})
    assert call(p) == status
    s = ctypes.c_int(0)
    assert pkv.lib().pkv_num_splits(ctypes.byref(p), 256, ctypes.byref(s)) == status


@pytest.mark.parametrize("which", ["q", "k", "v", "bt", "kl", "out"])
def test_null_pointers(which):
    assert call(base_problem(num_splits=1), **{which: 0}) == pkv.PKV_ERR_NULL


@pytest.mark.parametrize("which,addr", [("q", FAKE + 8), ("k", FAKE + 2), ("v", FAKE + 4), ("out", FAKE + 2),
                                        ("out32", FAKE + 4), ("bt", FAKE + 2), ("kl", FAKE + 1),
                                        ("mask", FAKE + 2), ("co", FAKE + 3)])
def test_misaligned_pointers(which, addr):
    assert call(base_problem(num_splits=1), **{which: addr}) == pkv.PKV_ERR_ALIGN


def test_workspace_checks():
    p = base_problem(num_splits=4)
    ob, mb = pkv.workspace_bytes(p, 4)
    rows = 2 * 1 * 8
    # o_part [rows, S, D]; ml_part = the counter head, then (m, l) [rows, S, 2]
    assert ob == rows * 4 * 64 * 4 and mb == pkv.PKV_COUNTER_BYTES + rows * 4 * 2 * 4
    assert pkv.PKV_MAX_FUSED_UNITS == pkv.PKV_COUNTER_BYTES // 4
    assert call(p) == pkv.PKV_ERR_WORKSPACE
    assert call(p, o=FAKE, ob=ob, ml=FAKE, mb=mb - 1) == pkv.PKV_ERR_WORKSPACE
    assert call(p, o=FAKE, ob=ob - 4, ml=FAKE, mb=mb) == pkv.PKV_ERR_WORKSPACE
    assert call(p, o=FAKE + 8, ob=ob, ml=FAKE, mb=mb) == pkv.PKV_ERR_ALIGN
    assert call(p, o=FAKE, ob=ob, ml=FAKE + 4, mb=mb) == pkv.PKV_ERR_ALIGN
    assert call(p, o=FAKE, ob=ob, ml=FAKE + 8, mb=mb) == pkv.PKV_ERR_ALIGN
    assert pkv.workspace_bytes(p, 1) == (0, 0)
    with pytest.raises(pkv.PkvError):
        pkv.workspace_bytes(p, 0)
    with pytest.raises(pkv.PkvError):
        pkv.workspace_bytes(p, 257)


def test_batch_zero_is_a_noop_even_with_null_pointers():
    assert call(base_problem(batch=0), q=0, k=0, v=0, bt=0, kl=0, out=0) == pkv.PKV_OK


def test_forced_splits_are_returned_unchanged():
    for s in (1, 3, 64, 256):
        assert pkv.num_splits(base_problem(num_splits=s), 256) == s


def plan_of(p, cus=256):
    info = pkv.plan(p, cus)
    return info.splits, info.heads_per_block


def test_split_heuristic_shapes():
    """Heuristic: when units fill the chip, splits of at most max(1024, 64 R)
    keys; for few long sequences, splits that fill the chip, bounded by the key
    count and 64; kv heads grouped per workgroup only for 2..8 splits of a
    batch that does not fill the chip by itself."""
    # B=256, Hkv=8, R=32 (one 32-row workgroup per kv head): units fill the chip -> splits of
    # 64 * 32 = 2048 keys over max_kv_len 8192 -> 4, two heads per workgroup
    big = base_problem(batch=256, q_len=4, num_q_heads=64, num_kv_heads=8, head_dim=128,
                       max_pages_per_seq=256, max_kv_len=8192, num_pages=13000)
    assert plan_of(big) == (4, 2) and pkv.num_splits(big, 256) == 4
    # the same batch with short sequences: one split
    big_short = base_problem(batch=256, q_len=4, num_q_heads=64, num_kv_heads=8, head_dim=128,
                             max_pages_per_seq=64, max_kv_len=2048, num_pages=13000)
    assert plan_of(big_short) == (1, 1)
    # B=4, Hkv=8, G=4 (matrix-core rows, D=128) -> 32 units, 32768 keys -> one workgroup per CU
    long = base_problem(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
                        max_pages_per_seq=512, max_kv_len=32768, num_pages=2048)
    assert plan_of(long) == (8, 1)
    # one row per kv head (VALU kernel): grouping 4 or 2 heads would need 32 or 16 splits
    mha = base_problem(batch=4, num_q_heads=8, num_kv_heads=8, head_dim=64, page_size=64,
                       max_pages_per_seq=512, max_kv_len=32768, num_pages=2048)
    assert plan_of(mha) == (8, 1)
    # matrix-core rows (G=8) at D=64: two workgroups per CU, two heads each; at D=128 and 256: one
    # workgroup per CU (D=256: one head each, two splits); at D=32 head pairing: one pair (two kv
    # heads read as one of 64 columns, 16 rows) per workgroup, planned as D=64 with Hkv=4
    mf = {d: base_problem(batch=16, num_q_heads=64, num_kv_heads=8, head_dim=d, max_pages_per_seq=128,
                          max_kv_len=4096, num_pages=2048) for d in (32, 64, 128, 256)}
    info = pkv.plan(mf[32], 256)
    assert plan_of(mf[32]) == (8, 2) and info.paired_heads == 1
    assert info.rows_per_block == 16 and info.kernel == pkv.PKV_KERNEL_MATRIX and info.units == 16 * 4
    assert all(pkv.plan(mf[d], 256).paired_heads == 0 for d in (64, 128, 256))
    assert plan_of(mf[64]) == (8, 2)
    assert plan_of(mf[128]) == (4, 2)
    assert plan_of(mf[256]) == (2, 1)
    # B=8 decode (1B model): grouping would need 16+ splits -> one head per workgroup
    d1b = base_problem(batch=8, num_q_heads=24, num_kv_heads=4, head_dim=64, max_pages_per_seq=64,
                       max_kv_len=2048, num_pages=512)
    assert plan_of(d1b)[1] == 1
    # VALU kernel, B=16, Hkv=8: four heads per workgroup and 8 splits at D <= 128, one head at 256;
    # at D=32 two pairs per workgroup (the paired problem: two rows per head of 64 columns)
    for d, want in ((32, (8, 4)), (64, (8, 4)), (128, (8, 4)), (256, (2, 1))):
        v = base_problem(batch=16, num_q_heads=8, num_kv_heads=8, head_dim=d, max_pages_per_seq=128,
                         max_kv_len=4096, num_pages=2048)
        assert plan_of(v) == want, d
        info = pkv.plan(v, 256)
        assert info.paired_heads == (d == 32) and info.rows_per_block == (2 if d == 32 else 1)
    # more sequences: fewer splits; once the units fill the chip the splits hold at most
    # 1024 keys (one row per kv head)
    v64 = base_problem(batch=64, num_q_heads=8, num_kv_heads=8, head_dim=128, max_pages_per_seq=128,
                       max_kv_len=4096, num_pages=8192)
    assert plan_of(v64) == (2, 4)
    v256 = base_problem(batch=256, num_q_heads=8, num_kv_heads=8, head_dim=128, max_pages_per_seq=128,
                        max_kv_len=4096, num_pages=32768)
    assert plan_of(v256) == (4, 4)
    # short sequences cap the split count (two tiles per wave)
    short = base_problem(batch=1, num_q_heads=8, num_kv_heads=8, head_dim=128, max_pages_per_seq=4,
                         max_kv_len=100)
    assert plan_of(short) == (4, 4)
    short1 = base_problem(batch=1, num_q_heads=8, num_kv_heads=8, head_dim=128, max_pages_per_seq=4,
                          max_kv_len=100, heads_per_block=1)
    assert plan_of(short1) == (1, 1)
    # more CUs never means fewer splits
    assert pkv.num_splits(long, 512) >= pkv.num_splits(long, 256)
    # the heuristic never exceeds 64
    huge = base_problem(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=32, page_size=4096,
                        max_pages_per_seq=500, max_kv_len=2_000_000)
    assert plan_of(huge, 1024) == (64, 1)


def test_plan_report():
    """pkv_plan: forced values unchanged, units and workgroups consistent, the
    merge path and launch count as documented."""
    v = base_problem(batch=16, num_q_heads=8, num_kv_heads=8, head_dim=64, max_pages_per_seq=128,
                     max_kv_len=4096, num_pages=2048)
    info = pkv.plan(v, 256)
    assert (info.splits, info.heads_per_block, info.rows_per_block, info.matrix_core) == (8, 4, 1, 0)
    assert info.units == 16 * 2 and info.workgroups == info.units * 8
    assert info.merge_in_kernel == 1 and info.kernels == 1      # 256 workgroups <= 2 per CU
    forced = base_problem(batch=16, num_q_heads=8, num_kv_heads=8, head_dim=64, max_pages_per_seq=128,
                          max_kv_len=4096, num_pages=2048, num_splits=5, heads_per_block=2)
    info = pkv.plan(forced, 256)
    assert (info.splits, info.heads_per_block, info.units) == (5, 2, 16 * 4)
    one = base_problem(batch=16, num_q_heads=8, num_kv_heads=8, head_dim=64, max_pages_per_seq=128,
                       max_kv_len=4096, num_pages=2048, num_splits=1)
    info = pkv.plan(one, 256)
    assert (info.splits, info.heads_per_block, info.merge_in_kernel, info.kernels) == (1, 1, 0, 1)
    # many workgroups still merge in-kernel (units within the counter head)
    many = base_problem(batch=64, q_len=1, num_q_heads=64, num_kv_heads=8, head_dim=128, max_pages_per_seq=128,
                        max_kv_len=4096, num_pages=8192, num_splits=4)
    info = pkv.plan(many, 256)
    assert info.matrix_core == 1 and info.rows_per_block == 16 and info.heads_per_block == 2
    assert info.units == 64 * 4 and info.workgroups == 64 * 4 * 4
    assert info.merge_in_kernel == 1 and info.kernels == 1
    # more than PKV_MAX_FUSED_UNITS units never merge in-kernel
    lots = base_problem(batch=4096, num_q_heads=8, num_kv_heads=2, head_dim=64, max_pages_per_seq=4,
                        max_kv_len=100, num_pages=8, num_splits=2, heads_per_block=1)
    info = pkv.plan(lots, 100000)
    assert info.units > pkv.PKV_MAX_FUSED_UNITS and info.merge_in_kernel == 0 and info.kernels == 2
    empty = base_problem(batch=0)
    assert pkv.plan(empty, 256).kernels == 0
    with pytest.raises(pkv.PkvError):
        pkv.plan(base_problem(heads_per_block=4), 256)          # Hkv = 2


def test_heads_per_block_checks():
    assert call(base_problem(num_splits=1, heads_per_block=-1)) == pkv.PKV_ERR_SHAPE
    assert call(base_problem(num_splits=1, heads_per_block=3)) == pkv.PKV_ERR_UNSUPPORTED
    assert call(base_problem(num_splits=1, heads_per_block=16, num_kv_heads=8, num_q_heads=16)) == \
        pkv.PKV_ERR_UNSUPPORTED
    # eight kv heads per workgroup: the shared-tile kernel, head_dim <= 64 only
    assert call(base_problem(num_splits=1, heads_per_block=8, num_kv_heads=8, head_dim=128)) == \
        pkv.PKV_ERR_UNSUPPORTED
    assert call(base_problem(num_splits=1, heads_per_block=8, num_kv_heads=8)) == pkv.PKV_ERR_LAUNCH
    assert call(base_problem(num_splits=1, heads_per_block=4)) == pkv.PKV_ERR_SHAPE   # Hkv = 2
    # a valid forced grouping passes every host check (the launch then fails without a GPU)
    assert call(base_problem(num_splits=1, heads_per_block=2)) == pkv.PKV_ERR_LAUNCH


def test_combine_argument_checks():
    lib = pkv
    assert lib.combine_raw(4, 0, 64, FAKE, FAKE, FAKE, 0, 0) == pkv.PKV_ERR_SHAPE
    assert lib.combine_raw(-1, 2, 64, FAKE, FAKE, FAKE, 0, 0) == pkv.PKV_ERR_SHAPE
    assert lib.combine_raw(4, 2, 48, FAKE, FAKE, FAKE, 0, 0) == pkv.PKV_ERR_UNSUPPORTED
    assert lib.combine_raw(4, 300, 64, FAKE, FAKE, FAKE, 0, 0) == pkv.PKV_ERR_UNSUPPORTED
    assert lib.combine_raw(4, 2, 64, 0, FAKE, FAKE, 0, 0) == pkv.PKV_ERR_NULL
    assert lib.combine_raw(4, 2, 64, FAKE + 4, FAKE, FAKE, 0, 0) == pkv.PKV_ERR_ALIGN
    assert lib.combine_raw(0, 2, 64, 0, 0, 0, 0, 0) == pkv.PKV_OK


def test_status_strings_are_distinct():
    msgs = {pkv.status_string(s) for s in range(9)}
    assert len(msgs) == 9
    assert pkv.status_string(99) == "unknown status"


def test_problem_struct_layout():
    # the C struct: twelve 4-byte fields, two int64 strides, heads_per_block, tail padding
    assert ctypes.sizeof(pkv.Problem) == 72
    assert pkv.Problem.mask_stride_b.offset == 48
    assert pkv.Problem.heads_per_block.offset == 64
    assert ctypes.sizeof(pkv.PlanInfo) == 48      # ... kernels, kernel, tail padding to 8 bytes
    assert pkv.PlanInfo.units.offset == 16 and pkv.PlanInfo.merge_in_kernel.offset == 32
    assert pkv.PlanInfo.kernel.offset == 40


def test_workspace_clear_checks():
    assert pkv.workspace_clear_raw(0, 0, 0) == pkv.PKV_OK          # nothing to clear
    assert pkv.workspace_clear_raw(0, 64, 0) == pkv.PKV_ERR_NULL
    assert pkv.workspace_clear_raw(FAKE + 2, 64, 0) == pkv.PKV_ERR_ALIGN
    assert pkv.workspace_clear_raw(FAKE, 66, 0) == pkv.PKV_ERR_ALIGN


def test_grid_beyond_32bit_work_items_is_rejected():
    # 2^23 sequences x 2 kv heads = 2^24 workgroups of 256 threads: 2^32 work-items
    assert call(base_problem(batch=1 << 23, num_splits=1, heads_per_block=1)) == pkv.PKV_ERR_SHAPE
    assert pkv.combine_raw((1 << 25) * 2 + 8, 2, 64, FAKE, FAKE, FAKE, 0, 0) == pkv.PKV_ERR_SHAPE


def ccall(p, layout=pkv.PKV_KV_BLHD, capacity=128, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kl=FAKE, co=0, mask=0, o=0, ob=0, ml=0, mb=0, out=FAKE, out32=0)
    a.update(ptrs)
    return pkv.contiguous_decode_raw(p, layout, capacity, a["q"], a["k"], a["v"], a["kl"], a["co"], a["mask"],
                                     a["o"], a["ob"], a["ml"], a["mb"], a["out"], a["out32"], 0)


def test_contiguous_decode_checks():
    p = base_problem(num_splits=1, heads_per_block=1, max_kv_len=100)
    assert ccall(p, layout=0) == pkv.PKV_ERR_UNSUPPORTED
    assert ccall(p, layout=3) == pkv.PKV_ERR_UNSUPPORTED
    assert ccall(p, capacity=0) == pkv.PKV_ERR_SHAPE
    assert ccall(p, capacity=pkv.PKV_MAX_CONTIGUOUS_KEYS + 1) == pkv.PKV_ERR_SHAPE
    assert ccall(p, capacity=99) == pkv.PKV_ERR_SHAPE                     # max_kv_len > capacity
    for which in ("q", "k", "v", "kl", "out"):
        assert ccall(p, **{which: 0}) == pkv.PKV_ERR_NULL
    assert ccall(p, k=FAKE + 2) == pkv.PKV_ERR_ALIGN
    assert ccall(base_problem(batch=0)) == pkv.PKV_OK
    # the paged fields are ignored: a page size that pkv_paged_decode rejects is fine here
    odd = base_problem(num_splits=1, heads_per_block=1, page_size=48, num_pages=-1, max_kv_len=100)
    assert ccall(odd) == pkv.PKV_ERR_LAUNCH                              # passes every host check
    assert ccall(p, layout=pkv.PKV_KV_BHLD) == pkv.PKV_ERR_LAUNCH
    # several splits need the workspace, as for the paged entry point
    ps = base_problem(num_splits=4, heads_per_block=1, max_kv_len=100)
    assert ccall(ps) == pkv.PKV_ERR_WORKSPACE


def test_contiguous_problem_plans_like_the_entry_point():
    cp = pkv.contiguous_problem(batch=16, q_len=1, num_q_heads=8, num_kv_heads=8, head_dim=64, kv_capacity=4096)
    info = pkv.plan(cp, 256)
    assert (info.splits, info.heads_per_block) == (8, 4)
    assert pkv.workspace_bytes(cp, 8)[0] == 16 * 8 * 8 * 64 * 4


def test_kv_row_too_wide_is_rejected():
    assert call(base_problem(num_splits=1, num_q_heads=1 << 17, num_kv_heads=1 << 17, head_dim=256)) == \
        pkv.PKV_ERR_SHAPE


def call_varlen(p, cu=FAKE, total=2, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, kl=FAKE, co=0, mask=0, o=0, ob=0, ml=0, mb=0, out=FAKE,
             out32=0)
    a.update(ptrs)
    return pkv.paged_decode_varlen_raw(p, cu, total, a["q"], a["k"], a["v"], a["bt"], a["kl"], a["co"],
                                       a["mask"], a["o"], a["ob"], a["ml"], a["mb"], a["out"], a["out32"], 0)


def test_varlen_decode_checks():
    """Argument checks of pkv_paged_decode_varlen, all answered before any
    device work (no GPU here)."""
    p = base_problem(num_splits=1, q_len=4, causal_offset=pkv.PKV_CAUSAL_LAST)
    assert call_varlen(p, total=9) == pkv.PKV_ERR_SHAPE                 # > B * q_len = 8
    assert call_varlen(p, total=-1) == pkv.PKV_ERR_SHAPE
    assert call_varlen(p, total=0, cu=0, q=0, out=0) == pkv.PKV_OK      # no tokens: nothing to do
    assert call_varlen(base_problem(batch=0), total=0, cu=0) == pkv.PKV_OK
    assert call_varlen(p, cu=0) == pkv.PKV_ERR_NULL
    assert call_varlen(p, cu=FAKE + 2) == pkv.PKV_ERR_ALIGN
    assert call_varlen(p, q=0) == pkv.PKV_ERR_NULL
    assert call_varlen(p, q=FAKE + 8) == pkv.PKV_ERR_ALIGN
    assert call_varlen(base_problem(num_splits=1, causal_offset=-3)) == pkv.PKV_ERR_SHAPE
    assert call_varlen(base_problem(num_splits=4, q_len=4)) == pkv.PKV_ERR_WORKSPACE
    assert pkv.PKV_CAUSAL_LAST == -2


def test_plan_varlen():
    """pkv_plan_varlen sizes the grid for the rows the tokens fill: a batch of
    32 sequences bounded at 64 tokens (G = 4: 256 rows, 128-row blocks) that
    holds 273 tokens has about 41 row blocks with rows, ~27 rows each, so its
    sequences are split (5 splits of at most 1728 keys at 8192 keys); holding
    every token, it plans as pkv_plan does."""
    p = base_problem(batch=32, q_len=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=32,
                     num_pages=9000, max_pages_per_seq=256, max_kv_len=8192, causal_offset=pkv.PKV_CAUSAL_LAST)
    full = pkv.plan(p, 256)
    assert (full.splits, full.matrix_core, full.rows_per_block, full.units) == (1, 1, 128, 32 * 8 * 2)
    same = pkv.plan_varlen(p, 32 * 64, 256)
    assert [getattr(same, f) for f, _ in same._fields_] == [getattr(full, f) for f, _ in full._fields_]
    mixed = pkv.plan_varlen(p, 273, 256)
    assert mixed.splits == 5 and mixed.units == (273 * 4 // 128 + 32) * 8
    assert mixed.merge_in_kernel == 1 and mixed.kernels == 1
    assert pkv.plan_varlen(p, 0, 256).splits == 1
    with pytest.raises(pkv.PkvError):
        pkv.plan_varlen(p, 32 * 64 + 1, 256)
    with pytest.raises(pkv.PkvError):
        pkv.plan_varlen(p, -1, 256)


def test_grouping_needs_short_splits():
    """Two kv heads per workgroup would give 2 splits of 4096 keys for 32
    sequences of up to 8192 keys (D = 128, G = 4): the plan keeps one head per
    workgroup, which fills the chip with 8 splits of 1024 keys."""
    p = base_problem(batch=32, q_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=32,
                     num_pages=9000, max_pages_per_seq=256, max_kv_len=8192)
    pl = pkv.plan(p, 256)
    assert (pl.splits, pl.heads_per_block, pl.rows_per_block) == (8, 1, 16)
    p.heads_per_block = 2
    assert pkv.plan(p, 256).splits == 2


def call_noalloc(p, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, kl=FAKE, co=0, mask=0, out=FAKE, out32=0)
    a.update(ptrs)
    return pkv.paged_decode_noalloc_raw(p, a["q"], a["k"], a["v"], a["bt"], a["kl"], a["co"], a["mask"],
                                        a["out"], a["out32"], 0)


def test_noalloc_argument_checks():
    """pkv_paged_decode_noalloc checks its arguments as pkv_paged_decode does,
    before anything touches a device, and refuses a split workspace larger
    than its static buffer."""
    p = base_problem(num_splits=3)
    assert call_noalloc(p, q=0) == pkv.PKV_ERR_NULL
    assert call_noalloc(p, out=0) == pkv.PKV_ERR_NULL
    assert call_noalloc(p, k=FAKE + 2) == pkv.PKV_ERR_ALIGN
    assert call_noalloc(base_problem(q_len=0)) == pkv.PKV_ERR_SHAPE
    assert call_noalloc(base_problem(head_dim=48, num_splits=1)) == pkv.PKV_ERR_UNSUPPORTED
    assert call_noalloc(base_problem(batch=0), q=0, k=0, v=0, bt=0, kl=0, out=0) == pkv.PKV_OK
    # the limit: ml_part bytes rounded to 256, then o_part bytes
    big = base_problem(batch=64, q_len=4, num_q_heads=64, num_kv_heads=8, head_dim=128, num_pages=64 * 4,
                       max_pages_per_seq=4, max_kv_len=128)
    for S in (2, 4, 7, 8, 64):
        big.num_splits = S           # 8 MiB of o_part per split, plus (m, l) and the counters
        ob, mb = pkv.workspace_bytes(big, S)
        fits = (mb + 255) // 256 * 256 + ob <= pkv.PKV_NOALLOC_SCRATCH_BYTES
        assert fits == (S <= 7), S
        if not fits:
            assert call_noalloc(big) == pkv.PKV_ERR_SCRATCH
    # one split needs no workspace: no limit applies
    big.num_splits = 1
    assert call_noalloc(big, q=0) == pkv.PKV_ERR_NULL


def test_head_pairing_rule_and_workspace():
    """Head pairing (pkv_plan_info.paired_heads): only at head_dim 32 with an even
    kv head count, automatic grouping and at most 8 packed rows per kv head; the
    paired plan's split count is what pkv_num_splits reports; the workspace keeps
    the real 32 columns per output row."""
    cases = [
        (dict(head_dim=32, num_q_heads=8, num_kv_heads=8), True),                 # 1 row -> 2 paired rows
        (dict(head_dim=32, num_q_heads=64, num_kv_heads=8), True),                # 8 rows -> 16
        (dict(head_dim=32, num_q_heads=32, num_kv_heads=8, q_len=2), True),       # 8 rows
        (dict(head_dim=32, num_q_heads=32, num_kv_heads=8, q_len=3), False),      # 12 rows
        (dict(head_dim=32, num_q_heads=128, num_kv_heads=8), False),              # 16 rows
        (dict(head_dim=32, num_q_heads=6, num_kv_heads=3), False),                # odd kv heads
        (dict(head_dim=32, num_q_heads=8, num_kv_heads=8, heads_per_block=2), False),  # forced grouping
        (dict(head_dim=64, num_q_heads=8, num_kv_heads=8), False),
        (dict(head_dim=128, num_q_heads=32, num_kv_heads=8), False),
    ]
    for kw, want in cases:
        p = base_problem(batch=16, max_pages_per_seq=128, max_kv_len=4096, num_pages=2048, **kw)
        info = pkv.plan(p, 256)
        assert info.paired_heads == want, kw
        assert pkv.num_splits(p, 256) == info.splits
        if want:
            # heads_per_block counts real kv heads, two per pair; units count pairs
            assert info.heads_per_block % 2 == 0
            rows_per_pair = 2 * (kw["num_q_heads"] // kw["num_kv_heads"]) * kw.get("q_len", 1)
            assert info.rows_per_block == (2 if rows_per_pair == 2 else 16)
            assert info.units == 16 * (kw["num_kv_heads"] // info.heads_per_block)
        S = max(info.splits, 2)
        o, ml = pkv.workspace_bytes(p, S)
        rows = 16 * kw.get("q_len", 1) * kw["num_q_heads"]
        assert o == rows * S * kw["head_dim"] * 4
        assert ml == pkv.PKV_COUNTER_BYTES + rows * S * 2 * 4
