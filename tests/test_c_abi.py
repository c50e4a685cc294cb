"""The C ABI from a plain C99 program (tests/c_abi_probe.c, built here with
gcc against include/pkv.h and the shared library): the header compiles as C,
the structures have the layout the Python binding's ctypes view gives them,
the constants agree, and the host-only entry points answer a C caller as
they answer the binding.  No GPU is used."""
import ctypes
import os
import shutil
import subprocess

import pytest

import paged_kv_split_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.dirname(pkv.LIB_PATH)
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    if shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("gcc or the ROCm headers are not installed")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_probe")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "c_abi_probe.c"), "-o", exe,
           "-L", LIBDIR, "-lpkv", f"-Wl,-rpath,{LIBDIR}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=60).stdout
    lines = {}
    for ln in out.splitlines():
        key, _, rest = ln.partition(" ")
        if key in ("offset", "sizeof"):
            t, _, rest2 = rest.partition(" ")
            if key == "offset":
                f, _, rest2 = rest2.partition(" ")
                lines[(key, t, f)] = rest2.split()
            else:
                lines[(key, t)] = rest2.split()
        else:
            lines[key] = rest.split()
    return lines


def test_struct_layout_matches_the_binding(probe):
    for cname, ctype in (("pkv_problem", pkv.Problem), ("pkv_plan_info", pkv.PlanInfo)):
        assert int(probe[("sizeof", cname)][0]) == ctypes.sizeof(ctype), cname
        for name, ftype in ctype._fields_:
            off, size = map(int, probe[("offset", cname, name)])
            assert off == getattr(ctype, name).offset, (cname, name)
            assert size == ctypes.sizeof(ftype), (cname, name)


def test_constants_match_the_binding(probe):
    c = list(map(int, probe["const"]))
    assert c == [pkv.PKV_MAX_SPLITS, pkv.PKV_CAUSAL_LAST, pkv.PKV_COUNTER_BYTES, pkv.PKV_COUNTER_BYTES // 4,
                 pkv.PKV_KV_BLHD, pkv.PKV_KV_BHLD, 1 << 30]
    assert list(map(int, probe["status"])) == list(range(9))
    assert int(probe["scratch"][0]) == pkv.PKV_NOALLOC_SCRATCH_BYTES
    assert list(map(int, probe["kernels"])) == [pkv.PKV_KERNEL_VECTOR, pkv.PKV_KERNEL_MATRIX,
                                                pkv.PKV_KERNEL_SHARED_TILE, pkv.PKV_KERNEL_PREFILL]


def _decode_problem(**kw):
    args = dict(batch=8, q_len=1, num_q_heads=24, num_kv_heads=4, head_dim=64, page_size=32, num_pages=512,
                max_pages_per_seq=64, max_kv_len=2048, scale=0.125, causal_offset=-1)
    args.update(kw)
    return pkv.make_problem(**args)


def _plan_tuple(pl):
    return [pl.splits, pl.heads_per_block, pl.rows_per_block, pl.matrix_core, pl.units, pl.workgroups,
            pl.merge_in_kernel, pl.kernels, pl.kernel, pl.paired_heads]


def test_host_entry_points_answer_c_as_they_answer_python(probe):
    p = _decode_problem()
    assert list(map(int, probe["num_splits"])) == [0, pkv.num_splits(p, 256)]
    rc, *plan = map(int, probe["plan_decode"])
    assert rc == 0 and plan == _plan_tuple(pkv.plan(p, 256))
    v = _decode_problem(q_len=64, causal_offset=pkv.PKV_CAUSAL_LAST)
    rc, *plan = map(int, probe["plan_varlen"])
    assert rc == 0 and plan == _plan_tuple(pkv.plan_varlen(v, 100, 256))
    rc, ob, mb = map(int, probe["workspace"])
    assert rc == 0 and (ob, mb) == pkv.workspace_bytes(p, 6)


def test_argument_checks_from_c(probe):
    assert int(probe["err_null_problem"][0]) == 1
    assert int(probe["err_null_info"][0]) == 1
    assert int(probe["err_gqa"][0]) == 2
    assert int(probe["err_head_dim"][0]) == 3
    assert int(probe["err_page"][0]) == 3
    assert int(probe["err_splits"][0]) == 3
    assert int(probe["err_varlen_tokens"][0]) == 2
    assert " ".join(probe["status_string"])
