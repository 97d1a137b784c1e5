"""The kernels' e4m3 / bf16 codec (fp8_moe_ffn_amd/csrc/codec.hpp), built for the host,
against the oracle.  Runs on the CPU; the same source is checked on the GPU by
tests/test_gpu_kernels.py."""

import ctypes
import os
import subprocess

import numpy as np
import pytest

from oracle import fp8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def codec(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("codec") / "libcodec_host.so")
    src = os.path.join(ROOT, "tests", "csrc", "codec_host.cpp")
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17", "-fPIC",
           "-shared", "-I", os.path.join(ROOT, "fp8_moe_ffn_amd", "csrc"), src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    lib = ctypes.CDLL(out)
    for f in ("host_encode", "host_encode_div", "host_decode", "host_bf16"):
        getattr(lib, f).restype = None
    return lib


def p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def enc(lib, v):
    v = np.ascontiguousarray(v, np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib.host_encode(p(v), p(out), ctypes.c_int64(v.size))
    return out


def enc_div(lib, v, s):
    v = np.ascontiguousarray(v, np.float32)
    s = np.ascontiguousarray(s, np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib.host_encode_div(p(v), p(s), p(out), ctypes.c_int64(v.size))
    return out


def test_decode_all_codes(codec):
    c = np.arange(256, dtype=np.uint8)
    out = np.zeros(256, np.float32)
    codec.host_decode(p(c), p(out), ctypes.c_int64(256))
    ref = fp8.e4m3_decode(c)
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(out[ok].astype(np.float64), ref[ok])
    assert np.array_equal(np.signbit(out[ok]), np.signbit(ref[ok]))


def test_encode_matches_oracle(codec):
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = (pos[:-1] + pos[1:]) / np.float32(2)
    rng = np.random.default_rng(1)
    v = np.concatenate([pos, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                        rng.uniform(-460, 460, 100000).astype(np.float32),
                        rng.uniform(-0.02, 0.02, 20000).astype(np.float32),
                        np.array([448, 463.9, 464, 1e6, np.inf, 0.0, -0.0, 1e-30, -1e-30], np.float32)])
    v = np.concatenate([v, -v])
    assert np.array_equal(enc(codec, v), fp8.e4m3_encode(v.astype(np.float64)))


def test_encode_of_quotient_rounds_once(codec):
    """e4m3(v / s) for float32 v, s must equal rounding the exact quotient, also when
    the float32 quotient lands on a midpoint between two codes."""
    rng = np.random.default_rng(2)
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    # scales as the step makes them: fp32(amax / 448) for bf16-like amax values
    s = (rng.uniform(0.5, 8.0, 40000).astype(np.float32) / np.float32(448)).astype(np.float32)
    target = rng.choice(mids, size=s.size) * rng.choice([-1.0, 1.0], size=s.size)
    v = (target * s.astype(np.float64)).astype(np.float32)  # v / s within an ulp of a midpoint
    v2 = rng.normal(0, 1, 40000).astype(np.float32)
    s2 = (np.abs(rng.normal(0, 1, 40000)).astype(np.float32) / np.float32(448)).astype(np.float32)
    v = np.concatenate([v, v2])
    s = np.concatenate([s, s2])
    ref = fp8.e4m3_encode(v.astype(np.float64) / s.astype(np.float64))
    got = enc_div(codec, v, s)
    assert np.array_equal(got, ref)
    # the midpoint cases really occur (the float32 quotient sits on a midpoint)
    q32 = v[:40000] / s[:40000]
    assert np.isin(np.abs(q32).astype(np.float64), mids).sum() > 100


def test_bf16_rounding(codec):
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.normal(0, 1, 100000), rng.normal(0, 1e4, 1000)]).astype(np.float32)
    # exact ties: a bf16 value plus half its spacing is a float32 value
    base = fp8.bf16_to_f64(rng.integers(0x3000, 0x5000, 1000).astype(np.uint16))
    ulp = np.ldexp(1.0, np.frexp(base)[1] - 8)
    v = np.concatenate([v, (base + ulp / 2).astype(np.float32)])
    out = np.zeros(v.shape, np.uint16)
    codec.host_bf16(p(v), p(out), ctypes.c_int64(v.size))
    assert np.array_equal(out, fp8.f64_to_bf16(v.astype(np.float64)))
