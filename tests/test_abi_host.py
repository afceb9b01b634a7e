"""Host-only checks of the C ABI library: it loads, exports every function the
public header declares, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(spec_verify\w*)\s*\(", src)
    return sorted(set(names))


def _lib():
    import speculative_decoding_verification_temp_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        pytest.skip("library not built")
    return sv, sv.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("spec_verify_init", "spec_verify", "spec_verify_destroy"):
        assert n in names
    import speculative_decoding_verification_temp_amd as sv
    assert sorted(sv.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    sv, L = _lib()
    for n in _declared():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", sv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (spec_verify\w*)", out))
    assert set(_declared()) <= exported


def test_version_string():
    sv, L = _lib()
    assert b"gfx950" in L.spec_verify_version()


def test_host_side_argument_errors():
    sv, L = _lib()
    h = ctypes.c_void_p()
    assert L.spec_verify_init(None, 4, 4, 16, 1, 0.99) == sv.SV_EINVAL
    assert L.spec_verify_init(ctypes.byref(h), 4, 4, 16, 7, 0.99) == sv.SV_EUNSUPPORTED
    assert L.spec_verify_init(ctypes.byref(h), 0, 4, 16, 1, 0.99) == sv.SV_EINVAL
    assert L.spec_verify_init(ctypes.byref(h), 4, 0, 16, 1, 0.99) == sv.SV_EINVAL
    assert L.spec_verify_init(ctypes.byref(h), 4, 64, 16, 1, 0.99) == sv.SV_EINVAL
    assert L.spec_verify_init(ctypes.byref(h), 4, 4, 0, 1, 0.99) == sv.SV_EINVAL
    assert L.spec_verify_init(ctypes.byref(h), 4, 4, 16, 1, 1.5) == sv.SV_EINVAL
    assert L.spec_verify_init(ctypes.byref(h), 4, 4, 16, 1, float("nan")) == sv.SV_EINVAL
    assert h.value is None
    # NULL handle everywhere
    assert L.spec_verify(None, 1, None, None, None, None, 1.0, 0, 0.0, None, None, None,
                         None) == sv.SV_EINVAL
    assert L.spec_verify_destroy(None) == sv.SV_OK
    assert L.spec_verify_set_aux(None, None, None, None, None) == sv.SV_EINVAL
    assert L.spec_verify_get_ema(None, None, None, None) == sv.SV_EINVAL
    assert L.spec_verify_reset_ema(None, None) == sv.SV_EINVAL
    assert L.spec_verify_last_error(None) == b"null handle"


def test_noalloc_rejects_bad_arguments_before_the_device():
    """spec_verify_noalloc checks dtype, sizes and mode before it looks for a
    device, and leaves its message for spec_verify_last_error(NULL) on the
    calling thread only."""
    import threading
    sv, L = _lib()
    args = [None] * 4 + [1.0]
    outs = [None] * 4
    res = {}

    def run():
        res["dtype"] = L.spec_verify_noalloc(4, 4, 16, 7, *args, 0, 0.0, *outs)
        res["dtype_msg"] = L.spec_verify_last_error(None)
        res["B"] = L.spec_verify_noalloc(0, 4, 16, 1, *args, 0, 0.0, *outs)
        res["K"] = L.spec_verify_noalloc(4, 64, 16, 1, *args, 0, 0.0, *outs)
        res["V"] = L.spec_verify_noalloc(4, 4, 0, 1, *args, 0, 0.0, *outs)
        res["big"] = L.spec_verify_noalloc(4, 7, 1 << 28, 1, *args, 0, 0.0, *outs)
        res["mode"] = L.spec_verify_noalloc(4, 4, 16, 1, *args, 9, 0.0, *outs)
        res["mode_msg"] = L.spec_verify_last_error(None)

    t = threading.Thread(target=run)
    t.start()
    t.join()
    assert res["dtype"] == sv.SV_EUNSUPPORTED and b"dtype" in res["dtype_msg"]
    assert res["B"] == res["K"] == res["V"] == res["big"] == sv.SV_EINVAL
    assert res["mode"] == sv.SV_EINVAL and b"mode" in res["mode_msg"]
    assert L.spec_verify_last_error(None) == b"null handle"    # another thread's errors
