"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/sekv.h declares, and rejects bad arguments on the host before any HIP
call.  No compute call is made here."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

from compressed_kv_cache_sekv_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sekv.h")


@pytest.fixture(scope="module")
def L():
    from compressed_kv_cache_sekv_amd import lib as sl
    if not os.path.exists(sl.LIB_PATH):
        from compressed_kv_cache_sekv_amd import build
        build.build()
    return sl


def header_symbols():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:sekv_status|void|const char\*|int32_t)\s+(sekv_\w+)\s*\(", text, re.M))


def test_header_declares_the_boundary():
    syms = header_symbols()
    for name in ("sekv_build_index", "sekv_route", "sekv_decode_attend", "sekv_create", "sekv_index_import"):
        assert name in syms


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    syms = header_symbols()
    missing = [s for s in syms if not hasattr(lib, s)]
    assert not missing, missing
    assert set(L.EXPORTS) == syms


def test_max_spans_bound(L):
    lib = L.lib()
    for T, lmin in [(1, 8), (8, 8), (16, 8), (17, 8), (2048, 8), (131072, 8), (100, 1), (5, 3)]:
        assert lib.sekv_max_spans(T, lmin) == synth.max_spans(T, lmin)
    # brute force on tiny T: the most maximal runs of >= l_min separated by single anchors
    for T in range(1, 40):
        for lmin in (1, 2, 3, 8):
            best = max(k for k in range(T + 1) if k * lmin + max(k - 1, 0) <= T)
            assert lib.sekv_max_spans(T, lmin) == best
    assert lib.sekv_max_spans(0, 8) == 0 and lib.sekv_max_spans(10, 0) == 0


def _params(L, **kw):
    w = synth.WORKLOADS["llama8b_l1_32k"]
    p = L.build_params(w)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_validate_accepts_every_workload(L):
    for w in synth.WORKLOADS.values():
        assert L.validate_params(L.build_params(w)) == 0, w.name


@pytest.mark.parametrize("field,value,status", [
    ("Hkv", 7, 1), ("d", 96, 6), ("R", 256, 1), ("R", 48, 6), ("Hkv", 2, 6),
    ("l_min", 0, 1), ("oversample", 17, 1), ("power_iters", -1, 1), ("alpha_sp", float("nan"), 1),
    ("alpha_sp", float("inf"), 1), ("dprime", 0, 6), ("dprime", 65, 6), ("T", 0, 1), ("B", 0, 1), ("tier", 5, 1),
    ("ring_bytes", -1, 1), ("T", 2_000_000, 6),
])
def test_validate_rejects(L, field, value, status):
    assert L.validate_params(_params(L, **{field: value})) == status
    assert L.lib().sekv_last_error()


def test_null_arguments_fail_before_any_hip_call(L):
    lib = L.lib()
    p = _params(L)
    out = C.c_void_p()
    assert lib.sekv_build_index(None, C.byref(p), 1, 1, 1, 1, None, C.byref(out)) == 1
    assert lib.sekv_index_import(None, C.byref(p), None, C.byref(out)) == 1
    assert lib.sekv_route(None, None, 0, 1, 1, 1, 0, 1, None) == 1
    assert lib.sekv_route_pooled(None, None, 0, 1, 1, 1, 5, 1, None) == 1
    assert lib.sekv_decode_attend(None, None, 0, 1, 1, 1, 1, None) == 1
    assert lib.sekv_calibrate_tau(None, None, 0, 1, 1, 0.1, 1) == 1
    assert lib.sekv_rsvd_batched(None, 1, 1, 1, 1, 8, 128, 16, 8, 2, 0, 1, 1, 1) == 1
    assert lib.sekv_index_get_info(None, None) == 1
    assert lib.sekv_index_counts(None, None, None) == 1
    assert lib.sekv_validate_params(None) == 1
    assert b"null" in lib.sekv_last_error()
    lib.sekv_destroy(None)
    lib.sekv_index_free(None)


def test_mask_packing_roundtrip():
    from tests.sekv_cases import pack_mask, unpack_mask
    rng = np.random.default_rng(0)
    z = {(0, 0, 0): rng.random(130) < 0.3, (0, 0, 1): np.zeros(130, bool)}
    z[(0, 0, 1)][0] = True
    z[(0, 0, 1)][64] = True
    m = pack_mask(z, 1, 1, 2, 3)
    assert m[0, 0, 1, 0] == 1 and m[0, 0, 1, 1] == 1 and m[0, 0, 1, 2] == 0
    assert np.array_equal(unpack_mask(m[0, 0, 0], 130), z[(0, 0, 0)])


def test_struct_layouts_match_the_header(L, tmp_path):
    """The binding's ctypes structures against the C compiler's own layout of
    the header's structs (size and every member offset)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"sekv_build_params": L.BuildParams, "sekv_index_info": L.IndexInfo,
               "sekv_host_index": L.HostIndex, "sekv_host_index_out": L.HostIndexOut, "sekv_stats": L.Stats}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "sekv.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        cname, f, v = line.split()
        got[(cname, f)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "size")] == C.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
