"""The C-ABI library loads and exports every function include/*.h declares.

CPU only: the library is loaded with ctypes but no compute entry point is
called. Also checks the host-side argument validation that fails before any
HIP call is made.
"""

import ctypes as C
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_moe_decode_amd", "libsmd.so")


def _declared():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text,
                             flags=re.M):
            name = m.group(1)
            if name not in ("if", "while", "for", "return", "sizeof"):
                names.add(name)
    return names


def test_header_declares_the_entry_points():
    names = _declared()
    for want in ("prerouter_forward", "moe_int4_decode", "lora_delta", "stage_experts",
                 "layer_step", "e0_create", "e0_destroy", "e0_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (run __graft_entry__.build())")
    lib = C.CDLL(LIB)
    missing = [n for n in sorted(_declared()) if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"


def test_binding_names_match_header():
    from sparse_moe_decode_amd import api
    names = _declared()
    assert set(api.EXPORTS) <= names
    for n in ("prerouter_forward", "moe_int4_decode", "lora_delta", "stage_experts",
              "layer_step"):
        assert callable(getattr(api, n))


def test_host_validation_rejects_bad_specs():
    from sparse_moe_decode_amd import api, synth
    lib = api._lib
    h = C.c_void_p()
    bad = dict(synth.dims("35b"), G=48)  # group not a multiple of 32
    assert lib.e0_create(C.byref(api.make_spec(bad)), 4, C.byref(h)) == -2
    bad = dict(synth.dims("35b"), K=9)
    assert lib.e0_create(C.byref(api.make_spec(bad)), 4, C.byref(h)) == -1
    bad = dict(synth.dims("8b"), topk_groups=0)
    assert lib.e0_create(C.byref(api.make_spec(bad)), 4, C.byref(h)) == -2
    assert b"sigmoid-group" in lib.e0_last_error()
    assert lib.e0_create(None, 4, C.byref(h)) == -1
    assert lib.e0_bundle_bytes(C.byref(api.make_spec(synth.dims("35b")))) == 1671168
    assert lib.e0_bundle_bytes(C.byref(api.make_spec(synth.dims("8b")))) == 1253376


def test_static_entry_point_checks_its_workspace_size_first():
    """moe_int4_decode_static validates the spec and the workspace it needs
    before any device call (the pointers below are never dereferenced)."""
    from sparse_moe_decode_amd import api, synth
    lib = api._lib
    ex = api.e0_experts()
    p = C.c_void_p(4096)
    spec = api.make_spec(synth.dims("35b"))
    assert lib.moe_int4_decode_static(C.byref(spec), C.byref(ex), None, None, p, p, p, 4000, p,
                                      None, None) == -2
    assert b"static workspace" in lib.e0_last_error()
    assert lib.moe_int4_decode_static(C.byref(spec), C.byref(ex), None, None, p, p, p, -1, p,
                                      None, None) == -1
    bad = api.make_spec(dict(synth.dims("35b"), K=9))
    assert lib.moe_int4_decode_static(C.byref(bad), C.byref(ex), None, None, p, p, p, 1, p,
                                      None, None) == -1
    assert lib.moe_int4_decode_static(None, C.byref(ex), None, None, p, p, p, 1, p, None,
                                      None) == -1
    assert lib.moe_int4_decode_static(C.byref(spec), C.byref(ex), None, None, p, p, p, 0, p,
                                      None, None) == 0
