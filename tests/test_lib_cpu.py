"""libl3 on a machine without a GPU: it loads, exports every entry point
include/l3.h declares, and its host-side argument checks return the
documented status codes (none of these calls reaches the GPU)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

LIB = os.path.join(ROOT, "static_token_routed_id_amd", "libl3.so")
HEADER = os.path.join(ROOT, "include", "l3.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(l3_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail("libl3.so is not built (python -m "
                    "static_token_routed_id_amd.build)")
    from static_token_routed_id_amd import _lib
    return _lib


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert "l3_plan" in names and "l3_forward" in names
    lib = ctypes.CDLL(LIB)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(L.EXPORTED) == set(names)


def test_status_strings(L):
    for code in range(-8, 1):
        assert L.l3_status_str(code)
    assert L.l3_stage_name(1) == "seg_fwd"
    assert L.l3_stage_name(99) is None


def test_workspace_size_checks(L):
    ok = L.make_desc(256, 1135, 64, 64, 32, L.L3_F32)
    p, s, c = L.l3_workspace_size(ok, 512)
    assert p > 512 * 4 * 5 and s >= 512 * (64 + 64 + 64) * 4 and c > 0
    p2, _, _ = L.l3_workspace_size(ok, 1024)
    assert p2 > p
    bad = [
        L.make_desc(256, 1135, 64, 64, 32, dtype=7),          # dtype
        L.make_desc(256, 1135, 64, 64, 32, y_dtype=3),        # y dtype
        L.make_desc(256, 1135, 96, 64, 32),                   # d % 64
        L.make_desc(256, 1135, 64, 64, 32, d_k=128),          # d_k != d
        L.make_desc(256, 1135, 64, 48, 32),                   # d_e % 64
        L.make_desc(256, 1135, 64, 64, 513),                  # k_max > 512
        L.make_desc(256, 1135, 64, 64, 0),                    # k_max < 1
        L.make_desc(0, 1135, 64, 64, 32),                     # vocab
        L.make_desc(256, 1135, 64, 64, 32, ln_eps=-1.0),      # eps
    ]
    want = [L.L3_ERR_DTYPE, L.L3_ERR_DTYPE] + [L.L3_ERR_SHAPE] * 7
    for dsc, code in zip(bad, want):
        with pytest.raises(L.L3Error) as e:
            L.l3_workspace_size(dsc, 16)
        assert e.value.status == code
    with pytest.raises(L.L3Error) as e:
        L.l3_workspace_size(ok, -1)
    assert e.value.status == L.L3_ERR_SHAPE


def test_plan_host_checks(L):
    lib = L.lib()
    dsc = L.make_desc(256, 1135, 64, 64, 32, L.L3_F32)
    out = ctypes.c_void_p()
    # NULL out pointer, NULL descriptor, NULL workspace, small workspace
    assert lib.l3_plan(ctypes.byref(dsc), None, 0, None, None, 0, None,
                       None) == L.L3_ERR_NULL
    assert lib.l3_plan(None, None, 0, None, None, 0, None,
                       ctypes.byref(out)) == L.L3_ERR_NULL
    assert lib.l3_plan(ctypes.byref(dsc), None, 0, None, None, 0, None,
                       ctypes.byref(out)) == L.L3_ERR_NULL
    buf = ctypes.create_string_buffer(64)
    p, _, _ = L.l3_workspace_size(dsc, 100)
    assert lib.l3_plan(ctypes.byref(dsc), None, 100, None, buf, 64, None,
                       ctypes.byref(out)) == L.L3_ERR_WORKSPACE
    assert lib.l3_plan(ctypes.byref(dsc), None, -3, None, buf, 64, None,
                       ctypes.byref(out)) == L.L3_ERR_SHAPE
    # workspaces must start on a 256-byte boundary
    raw = ctypes.create_string_buffer(p + 512)
    base = (ctypes.addressof(raw) + 255) // 256 * 256
    assert lib.l3_plan(ctypes.byref(dsc), None, 0, None,
                       ctypes.c_void_p(base + 16), p, None,
                       ctypes.byref(out)) == L.L3_ERR_WORKSPACE
    # an empty batch needs no device work: the handle is made, B = 0
    assert lib.l3_plan(ctypes.byref(dsc), None, 0, None, ctypes.c_void_p(base),
                       p, None, ctypes.byref(out)) == L.L3_OK
    assert lib.l3_plan_tokens(out) == 0
    # ids missing for a non-empty batch
    assert lib.l3_replan(out, None, 5, None, None) == L.L3_ERR_NULL
    # more tokens than the workspace holds
    assert lib.l3_replan(out, None, 10 ** 6, None, None) == L.L3_ERR_WORKSPACE
    # forward of an empty batch is a no-op
    assert lib.l3_forward(out, None, None, None, None, None, None, None, None,
                          None, 0, None, 0, None) == L.L3_OK
    assert lib.l3_forward(None, None, None, None, None, None, None, None,
                          None, None, 0, None, 0, None) == L.L3_ERR_NULL
    # staging: a NULL plan is refused; an empty batch has nothing to stage
    for fn in (lib.l3_stage_rows, lib.l3_stage_rows_dma):
        assert fn(None, None, None, None, None, 0, None) == L.L3_ERR_NULL
        assert fn(out, None, None, None, None, 0, None) == L.L3_OK
    lib.l3_plan_release(out)
    lib.l3_plan_release(None)
    assert lib.l3_plan_tokens(None) == -1


def test_read_probe_library():
    """The read probe bench.py times beside the gather (libl3probe.so, built
    with libl3.so) loads, exports its entry point and rejects a bad size or
    pattern on the host, before any launch."""
    path = os.path.join(ROOT, "static_token_routed_id_amd", "libl3probe.so")
    if not os.path.exists(path):
        pytest.fail("libl3probe.so is not built (python -m "
                    "static_token_routed_id_amd.build)")
    lib = ctypes.CDLL(path)
    f = lib.l3probe_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 1000, 0, 256, None, None) == -1     # not whole 64 KiB
    assert f(None, 0, 0, 256, None, None) == -1        # empty
    assert f(None, 65536, 0, 0, None, None) == -1      # no workgroups
    assert f(None, 65536, 5, 256, None, None) == -1    # no such pattern
