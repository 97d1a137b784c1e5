"""The C-ABI library loads, exports every function include/*.h declares, and rejects
bad arguments on the host.  No compute: runs without a GPU."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

import fp8_moe_ffn_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(moe_ffn_fp8_\w+)\s*\(", src))
    return names


def test_library_is_built_and_loads():
    assert os.path.exists(F.LIB_PATH), "run __graft_entry__.build() first"
    F.load()


def test_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_ffn_fp8_\w+)", out))
    assert names <= exported, names - exported
    assert names == set(F.SIGNATURES), "binding and header disagree"
    lib = F.load()
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings():
    assert F.status_string(F.OK) == "ok"
    for s in (F.ERR_INVALID_ARG, F.ERR_UNSUPPORTED, F.ERR_OUT_OF_MEMORY, F.ERR_HIP):
        assert F.status_string(s) not in ("ok", "unknown status")
    assert F.status_string(12345) == "unknown status"


@pytest.mark.parametrize("dims", [
    (100, 512, 4, 4),     # hidden not a multiple of 128
    (256, 500, 4, 4),     # inter not a multiple of 128
    (0, 512, 4, 4), (256, 0, 4, 4),
    (16384, 512, 0, 1),   # hidden too large
    (256, 512, -1, 4),    # negative experts
    (256, 512, 2000, 4),  # too many experts
    (256, 512, 4, 0),     # no tokens
    (256, 512, 4, (1 << 16) + 1),  # more tokens than a forward may take
])
def test_create_rejects_bad_dims(dims):
    lib = F.load()
    h = ctypes.c_void_p(1234)
    d = F.Dims(*dims)
    assert lib.moe_ffn_fp8_create(ctypes.byref(d), ctypes.byref(h)) == F.ERR_INVALID_ARG
    assert h.value is None  # *out cleared


@pytest.mark.parametrize("max_tokens", [16, 1000])
def test_create_rejects_sizes_beyond_the_lds_budget(max_tokens):
    """K = 8192 with 16 tokens per launch needs more LDS for the token codes than a CU
    has; a larger batch runs in launches of 16 tokens, so it is refused the same way."""
    lib = F.load()
    h = ctypes.c_void_p()
    d = F.Dims(8192, 512, 4, max_tokens)
    assert lib.moe_ffn_fp8_create(ctypes.byref(d), ctypes.byref(h)) == F.ERR_UNSUPPORTED


def test_null_arguments_rejected_before_device_work():
    lib = F.load()
    h = ctypes.c_void_p()
    assert lib.moe_ffn_fp8_create(None, ctypes.byref(h)) == F.ERR_INVALID_ARG
    d = F.Dims(256, 512, 4, 4)
    assert lib.moe_ffn_fp8_create(ctypes.byref(d), None) == F.ERR_INVALID_ARG
    assert lib.moe_ffn_fp8_forward(None, None, None, None, 1, None) == F.ERR_INVALID_ARG
    assert lib.moe_ffn_fp8_forward_debug(None, None, None, None, 1, None, None) == F.ERR_INVALID_ARG
    assert lib.moe_ffn_fp8_prepack_expert(None, 0, None, None, None, None, None) == F.ERR_INVALID_ARG
    assert lib.moe_ffn_fp8_unpack_expert(None, 0, None, None, None, None, None) == F.ERR_INVALID_ARG
    assert lib.moe_ffn_fp8_profile_begin(None) == F.ERR_INVALID_ARG
    assert lib.moe_ffn_fp8_profile_end(None, None, None) == F.ERR_INVALID_ARG
    assert lib.moe_ffn_fp8_e4m3_encode(None, None, -1, None) == F.ERR_INVALID_ARG
    assert lib.moe_ffn_fp8_e4m3_decode(None, None, 0, None) == F.OK  # n == 0: nothing to do
    assert lib.moe_ffn_fp8_destroy(None) == F.OK
    # host pointers are not device memory
    buf = (ctypes.c_float * 16)()
    out = (ctypes.c_uint8 * 16)()
    assert lib.moe_ffn_fp8_e4m3_encode(ctypes.cast(buf, ctypes.c_void_p),
                                       ctypes.cast(out, ctypes.c_void_p), 16, None) == F.ERR_INVALID_ARG
