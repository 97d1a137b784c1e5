"""GPU checks of the library's building blocks through the C ABI: the e4m3 codec
against the oracle, the weight prepack as an exact permutation, and the streaming-read
probe."""

import numpy as np
import pytest
import torch

import fp8_moe_ffn_amd as F
import workloads as W
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu


def test_decode_all_codes(lib):
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    got = F.e4m3_decode(c).cpu().numpy().astype(np.float64)
    ref = ofp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_encode_matches_oracle(lib):
    pos = ofp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = (pos[:-1] + pos[1:]) / np.float32(2)
    rng = np.random.default_rng(0)
    v = np.concatenate([pos, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                        rng.uniform(-460, 460, 200000).astype(np.float32),
                        rng.uniform(-0.02, 0.02, 50000).astype(np.float32),
                        np.array([448, 463.9, 464, 1e6, np.inf, 0.0, -0.0], np.float32)])
    v = np.concatenate([v, -v])
    got = F.e4m3_encode(torch.from_numpy(v).cuda()).cpu().numpy()
    assert np.array_equal(got, ofp8.e4m3_encode(v.astype(np.float64)))


@pytest.mark.parametrize("scale", [np.float32(1.0), np.float32(3.1e-4) / np.float32(448), np.float32(0.75),
                                   np.float32(7.123456) / np.float32(448), np.float32(2.0 ** -20) * np.float32(1.7),
                                   # below 2**-96 the quantiser lifts scale and values by 2**64; the
                                   # last two are subnormal float32 scales (1 / s overflows)
                                   np.float32(2.0 ** -100) * np.float32(1.37), np.float32(2.0 ** -129) * np.float32(1.3),
                                   np.float32(2.0 ** -140) * np.float32(1.5)])
def test_quantize_is_the_exact_quotient_code(lib, scale):
    """The forward's quantiser: code of in / scale, rounded once from the exact quotient.
    Quotients are placed on every code, every rounding midpoint and a few float32 steps
    around each (where a product with the reciprocal could round across), plus random
    values over the whole range; the oracle encodes the float64 quotient."""
    s = np.float32(scale)
    pos = ofp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    targets = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2])
    v = (targets * np.float64(s)).astype(np.float32)
    near = [v]
    up, down = v.copy(), v.copy()
    for _ in range(6):
        up = np.nextafter(up, np.float32(np.inf))
        down = np.nextafter(down, np.float32(0))
        near += [up, down]
    rng = np.random.default_rng(int(s.view(np.uint32)))
    amax = np.float32(448) * s
    rand = rng.uniform(-1, 1, 400000).astype(np.float32) * amax
    vals = np.concatenate(near + [rand, np.array([0.0, -0.0, amax, -amax], np.float32)])
    vals = vals[np.abs(vals.astype(np.float64) / np.float64(s)) <= 448.0 * (1 + 2.0 ** -22)]
    vals = np.concatenate([vals, -vals])
    got = F.e4m3_quantize(torch.from_numpy(vals).cuda(), float(s)).cpu().numpy()
    ref = ofp8.e4m3_encode(vals.astype(np.float64) / np.float64(s))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (bad.size, vals[bad[:5]], got[bad[:5]], ref[bad[:5]])
    odd = vals[:1001]  # an odd count pairs the last element with itself
    assert np.array_equal(F.e4m3_quantize(torch.from_numpy(odd).cuda(), float(s)).cpu().numpy(),
                          ofp8.e4m3_encode(odd.astype(np.float64) / np.float64(s)))


@pytest.mark.parametrize("K,I", [(256, 512), (384, 640), (5120, 8192)])
def test_prepack_is_a_permutation(lib, K, I):
    m = F.MoeFFN(K, I, 1, 1)
    for slot in range(2):
        e = W.expert(3, slot, K, I, "cuda")
        m.prepack_expert(slot, e.w13, e.s13, e.w2, e.s2)
        back = W.Expert(torch.empty_like(e.w13), torch.empty_like(e.s13),
                        torch.empty_like(e.w2), torch.empty_like(e.s2))
        m.unpack_expert(slot, back.w13, back.s13, back.w2, back.s2)
        torch.cuda.synchronize()
        for a, b in zip((e.w13, e.s13, e.w2, e.s2), (back.w13, back.s13, back.w2, back.s2)):
            assert torch.equal(a, b)
    m.close()


@pytest.mark.parametrize("nbytes", [16, 160 * 1024, 3 * 160 * 1024 + 48, 64 << 20])
def test_stream_read_reads_every_word(lib, nbytes):
    """The ceiling probe reads every 16-byte word: with one word set so that the XOR of the
    buffer is the probe's fixed value (and everything else zero), it writes the sink, wherever
    that word sits (first chunk, a later chunk, the tail past the last whole chunk)."""
    magic = 0x9E3779B9
    words = nbytes // 4
    for pos in sorted({0, words // 2, words - 1}):
        buf = torch.zeros(words, dtype=torch.int32, device="cuda")
        buf[pos] = magic - (1 << 32)  # the bit pattern 0x9E3779B9 as int32
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        F.stream_read(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) & 0xFFFFFFFF == magic, (nbytes, pos)
    zero = torch.zeros(words, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    F.stream_read(zero, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
