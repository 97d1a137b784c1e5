"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Sizes: the tiny configuration (M=4, K=256, I=512, 4 experts + shared), ragged and
minimal shapes that leave partial k-step rounds and partial FC2 splits, batches above one
launch in both batch modes (grouped passes and chunked launches), the dense
shared expert at full Maverick size (K=5120, I=8192) for M = 1, 2, 4, 8, and the
routed step at full size (128 experts + shared, M=4, d = 1..4 distinct experts).
Acceptance checks are in tests/harness.py."""

import numpy as np
import pytest
import torch

import fp8_moe_ffn_amd as F
import workloads as W
from harness import Problem, check_all, check_codes, check_output, check_rel, chunked_active
from oracle import ffn as offn
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def modes_for(M):
    """Batch modes that run different kernels for M tokens: above GROUP_FROM, the grouped
    pass (the default) and, in the chunked mode, the decode kernels."""
    return [F.BATCH_GROUPED, F.BATCH_CHUNKED] if M > F.GROUP_FROM else [F.BATCH_GROUPED]


def test_tiny_config(lib):
    c = W.TINY
    say("case tiny", c)
    pr = Problem(c["seed"], c["M"], c["hidden"], c["inter"], c["num_experts"])
    s = check_all(pr.run_gpu(), pr.run_oracle(), c["num_experts"], pr.weights)
    say("tiny", s)


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_tiny_more_seeds(lib, seed):
    c = W.TINY
    pr = Problem(seed, c["M"], c["hidden"], c["inter"], c["num_experts"])
    check_all(pr.run_gpu(), pr.run_oracle(), c["num_experts"], pr.weights)


@pytest.mark.parametrize("M,K,I,E", [
    (1, 128, 128, 0),     # minimal sizes, one k-step, one partial FC2 split
    (3, 384, 640, 5),     # K: 3 k-steps (partial round); I: 5 k-steps (partial split)
    (16, 256, 1024, 3),   # max tokens, fewer experts than tokens
    (7, 1152, 1280, 9),   # odd everything
    (2, 640, 2176, 2),    # several FC2 splits plus a partial one
    (16, 256, 256, 160),  # more logits than one early load per thread covers
    (13, 128, 128, 1000), # near the largest expert count
])
def test_ragged_shapes(lib, M, K, I, E):
    say("case ragged", M, K, I, E)
    pr = Problem(10 + M, M, K, I, E)
    ref = pr.run_oracle()
    for mode in modes_for(M):  # above 8 tokens: the grouped pass and one decode launch
        pr.set_mode(mode)
        check_all(pr.run_gpu(), ref, E, pr.weights)


@pytest.mark.parametrize("mode", [F.BATCH_GROUPED, F.BATCH_CHUNKED], ids=["grouped", "chunked"])
@pytest.mark.parametrize("M,E", [(40, 6), (17, 3), (33, 0), (100, 1), (1030, 5)])
def test_batches_above_one_launch(lib, M, E, mode):
    """M above the 16 tokens one launch takes: grouped passes of up to 1024 tokens (every
    expert's rows in tiles of 16, the last partial; one expert for all 100 tokens; a
    second pass of 6 tokens at M = 1030), or consecutive launches of 16 in routed-expert
    order (more than one 1024-token tile of the ordering kernel): every output, code and
    scale against the oracle on the whole batch."""
    say("case batch", M, E, "grouped" if mode == F.BATCH_GROUPED else "chunked")
    pr = Problem(30 + M, M, 256, 512, E)
    pr.set_mode(mode)
    check_all(pr.run_gpu(), pr.run_oracle(), E, pr.weights)


@pytest.mark.parametrize("M,K,I,E", [
    (37, 384, 640, 5),     # K: 3 k-steps (waves without k-steps); I: a partial FC2 split
    (20, 1152, 1280, 9),   # odd everything; 9 k-steps over 8 waves
    (50, 128, 128, 0),     # minimal dense: one k-step, one partial split, 4 row tiles
    (300, 256, 1024, 3),   # about 100 tokens per expert: several row tiles per slot
    (1024, 256, 512, 1),   # the largest pass, one routed expert: 64 row tiles per slot
    (64, 1024, 2048, 200), # many experts, more slots than blocks' first items
])
def test_grouped_ragged_shapes(lib, M, K, I, E):
    """The grouped pass on shapes with partial k-step rounds, partial FC2 splits and
    many row tiles per expert, against the oracle."""
    say("case grouped ragged", M, K, I, E)
    pr = Problem(50 + M, M, K, I, E)
    check_all(pr.run_gpu(), pr.run_oracle(), E, pr.weights)


@pytest.mark.parametrize("M,K,I,E", [
    (4, 8192, 256, 2),      # the largest hidden size (8 k-steps per FC13 wave)
    (4, 128, 32768, 1),     # the largest intermediate size: 16 FC2 splits, the combine's long path
    (20, 128, 32768, 1),    # the same in a grouped pass
    (16, 128, 128, 1024),   # the largest expert count: a grouped pass, and one decode launch
    (40, 256, 256, 1024),   # ... a grouped pass with 40 slots
])
def test_maximum_sizes(lib, M, K, I, E):
    """The library's size limits (hidden 8192, intermediate 32768, 1024 experts) against the
    oracle, in every batch mode that runs different kernels for M tokens."""
    say("case maximum sizes", M, K, I, E)
    pr = Problem(70 + M, M, K, I, E)
    ref = pr.run_oracle()
    for mode in modes_for(M):
        pr.set_mode(mode)
        check_all(pr.run_gpu(), ref, E, pr.weights)


def test_grouped_equals_chunked_bitwise(lib):
    """Both batch modes do the same arithmetic in the same order (k-steps per wave, waves
    reduced in order, the same quantiser): a skewed batch gives the same bits either way."""
    M, K, I, E = 200, 1024, 2048, 16
    say("case grouped == chunked", M, K, I, E)
    targets = W.zipf_targets(3, M, E)
    pr = Problem(3, M, K, I, E, force=targets)
    g = pr.run_gpu()
    pr.set_mode(F.BATCH_CHUNKED)
    c = pr.run_gpu()
    for k in ("out", "xq", "s_x", "expert", "gate", "aq_shared", "s_a_shared", "aq_routed", "s_a_routed"):
        assert np.array_equal(np.asarray(g[k]).view(np.uint8), np.asarray(c[k]).view(np.uint8)), k


@pytest.mark.parametrize("M,K,I,E", [
    (300, 2048, 4096, 0),  # dense: a group of 256 tokens and a partial one of 44
    (128, 3072, 2048, 5),  # the smallest pass that runs wide, with routed experts beside it
])
def test_wide_shared_expert(lib, M, K, I, E):
    """A grouped pass of at least 128 tokens gives the shared expert's GEMMs to the kernels
    that split the tokens over the waves: the same bits as the decode kernels (chunked
    mode), and the oracle's bar on every output."""
    say("case wide shared expert", M, K, I, E)
    pr = Problem(90 + M, M, K, I, E)
    g = pr.run_gpu()
    check_all(g, pr.run_oracle(), E, pr.weights)
    pr.set_mode(F.BATCH_CHUNKED)
    c = pr.run_gpu()
    for k in ("out", "xq", "s_x", "expert", "gate", "aq_shared", "s_a_shared", "aq_routed", "s_a_routed"):
        assert np.array_equal(np.asarray(g[k]).view(np.uint8), np.asarray(c[k]).view(np.uint8)), k


@pytest.mark.timeout(900)
def test_throughput_batch_zipf_full_size(lib):
    """M = 256 tokens at Maverick size (K=5120, I=8192, 128 experts + shared) with
    Zipf(1.2) expert popularity, in one grouped pass: every output, code and scale of all
    256 tokens against the oracle, which computes the whole batch (each routed expert on
    its own tokens, so every row tile of the popular experts, the partial last ones
    included, is checked).  The chunked batch mode gives the same bits."""
    M, K, I, E = 256, W.HIDDEN, W.INTER, W.EXPERTS
    say("case zipf M=256 full size")
    targets = W.zipf_targets(0, M, E)
    pr = Problem(0, M, K, I, E, force=targets)
    gpu = pr.run_gpu()
    pr.set_mode(F.BATCH_CHUNKED)
    chk = pr.run_gpu()
    pr.set_mode(F.BATCH_GROUPED)
    for k in ("out", "xq", "s_x", "gate", "aq_shared", "aq_routed", "s_a_shared", "s_a_routed"):
        assert np.array_equal(np.asarray(gpu[k]).view(np.uint8), np.asarray(chk[k]).view(np.uint8)), k
    assert int(chk["num_active"][0]) == chunked_active(targets)
    assert gpu["expert"].tolist() == targets
    counts = np.bincount(targets, minlength=E)
    say("distinct experts", int((counts > 0).sum()), "top expert tokens", int(counts.max()),
        "experts with one token", int((counts == 1).sum()))
    # the oracle regenerates each expert's codes from its seed when it needs them
    weights = lambda slot: W.expert(pr.seed, slot, K, I, pr.gen_device).numpy()
    ref = oracle_ffn_forward(pr, weights)
    s = check_all(gpu, ref, E, weights, mode=F.BATCH_GROUPED, max_conditioned=0)
    say("zipf", s)


def oracle_ffn_forward(pr, weights):
    """The oracle's step on the problem's whole batch with the given weight source."""
    lg = W.bits(pr.logits) if pr.logits is not None else None
    return offn.forward(W.bits(pr.x), lg, weights, pr.E)


def test_activation_quotients_on_rounding_midpoints(lib):
    """Token 0's quotients x / s_x fall exactly on every e4m3 rounding midpoint (s_x is a
    power of two, so the kernel's reciprocal product is exact too and the ties must go
    to the even code); the quantiser's exact path decides them.  The codes must equal
    the oracle's bit for bit."""
    K, I, E, M = 512, 256, 3, 2
    pr = Problem(23, M, K, I, E)
    pos = ofp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    row = np.concatenate([[448.0], mids, -mids, pos[1:], -pos[1:]])
    row = np.resize(row, K) * 2.0 ** -3  # amax 56 -> s_x = 2**-3 exactly
    x = pr.x.clone()
    x[0] = torch.from_numpy(row.astype(np.float32)).to(torch.bfloat16).cuda()
    assert np.array_equal(ofp8.bf16_to_f64(W.bits(x[0:1].cpu()))[0], row)  # bf16-exact
    ref = pr.run_oracle(x)
    gpu = pr.run_gpu(x)
    assert ref["s_x"][0] == 2.0 ** -3
    assert np.array_equal(gpu["xq"], ref["xq"])
    check_all(gpu, ref, E, pr.weights)


@pytest.mark.parametrize("M", [5, 8])
def test_many_midpoints_over_the_early_chunks(lib, M):
    """At hidden 5120 and 5..8 tokens a lane quantises ten chunks of its token (eight
    held in registers, two staged in LDS).  Token 0 puts every quotient on a rounding
    midpoint (every lane marks every chunk for the exact path: ten passes of a full
    queue); token 1 does so for a random 30% of its elements (passes that fill part of
    the queue and stop at an index that would overflow it).  Codes bit for bit."""
    K, I, E = 5120, 256, 3
    pr = Problem(29 + M, M, K, I, E)
    pos = ofp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    dense = np.resize(np.concatenate([[448.0], mids, -mids]), K) * 2.0 ** -3
    rng = np.random.default_rng(M)
    sparse = rng.normal(0.0, 2.0, K).clip(-50.0, 50.0)
    pick = rng.random(K) < 0.3
    sparse[pick] = rng.choice(np.concatenate([mids, -mids]), int(pick.sum())) * 2.0 ** -3
    sparse[0] = 56.0  # amax 56 -> s_x = 2**-3 exactly
    x = pr.x.clone()
    for m, row in ((0, dense), (1, sparse)):
        x[m] = torch.from_numpy(row.astype(np.float32)).to(torch.bfloat16).cuda()
    ref = pr.run_oracle(x)
    gpu = pr.run_gpu(x)
    assert ref["s_x"][0] == ref["s_x"][1] == 2.0 ** -3
    assert np.array_equal(gpu["xq"], ref["xq"])
    check_all(gpu, ref, E, pr.weights)


@pytest.mark.parametrize("M", [4, 5, 8])
def test_ties_follow_the_rounding_of_the_scale(lib, M):
    """bf16 rows whose ideal ratios 448 x / amax fall exactly on rounding midpoints, over
    maxima whose scale fp32(amax / 448) rounds up, rounds down or is exact: the quotient
    x / s then lies just below, just above or on the midpoint, the same for the whole
    row.  Codes bit for bit against the oracle, which rounds the float64 quotient."""
    K, I, E = 5120, 256, 3
    pr = Problem(40 + M, M, K, I, E)
    pos = ofp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    amaxes = [4.125, 3.75, 2.625, 5.5, 3.3125, 0.171875, 7.0, 1.5]
    rng = np.random.default_rng(M)
    x = pr.x.clone()
    for m in range(M):
        am = amaxes[m % len(amaxes)]
        cand = mids * am / 448.0
        ties = cand[ofp8.bf16_to_f64(W.bits(torch.from_numpy(cand.astype(np.float32)).to(torch.bfloat16))) == cand]
        assert ties.size > 0
        row = rng.uniform(-am, am, K)
        pick = rng.random(K) < 0.3
        row[pick] = rng.choice(np.concatenate([ties, -ties]), int(pick.sum()))
        row[0] = am
        x[m] = torch.from_numpy(row.astype(np.float32)).to(torch.bfloat16).cuda()
    ref = pr.run_oracle(x)
    gpu = pr.run_gpu(x)
    assert np.array_equal(gpu["xq"], ref["xq"])
    check_all(gpu, ref, E, pr.weights)


@pytest.mark.parametrize("M", [4, 20])
def test_tiny_rows(lib, M):
    """Rows whose scales fall below the quantiser's lifted range (2**-96): token 0 is x
    times 2**-124, so s_x = fp32(amax / 448) is a subnormal float32 whose reciprocal
    overflows; token 2 is x times 2**-100 (a normal s_x below 2**-96); token 1 is scaled so
    that its intermediate's largest magnitude is near 2**-121, making both of its s_a
    subnormal (the intermediate scales as the square of x).  Activation codes and scales bit
    for bit, the rest to the usual bar, in one decode launch (M = 4) and a grouped pass
    (M = 20)."""
    K, I, E = 512, 1024, 3
    pr = Problem(90 + M, M, K, I, E)
    base = pr.run_oracle()
    amax_a = max(np.abs(base["a_shared"][1]).max(), np.abs(base["a_routed"][1]).max())
    k1 = int(round((np.log2(amax_a) + 121.0) / 2.0))
    x = pr.x.float()
    for m, k in ((0, 124), (1, k1), (2, 100)):
        x[m] = x[m] * 2.0 ** -k
    x = x.to(torch.bfloat16)
    ref = pr.run_oracle(x)
    gpu = pr.run_gpu(x)
    assert 0 < ref["s_x"][0] < 2.0 ** -126 and 2.0 ** -126 < ref["s_x"][2] < 2.0 ** -96
    assert 0 < ref["s_a_shared"][1] < 2.0 ** -126 and 0 < ref["s_a_routed"][1] < 2.0 ** -96
    say("tiny rows: s_x", ref["s_x"][:3], "s_a of token 1", ref["s_a_shared"][1], ref["s_a_routed"][1])
    s = check_all(gpu, ref, E, pr.weights, max_conditioned=1)
    say("tiny", s)
    assert np.isfinite(ofp8.bf16_to_f64(gpu["out"])).all()


def test_all_codes_in_weights_and_edge_activations(lib):
    """Weights cycle through every finite e4m3 code (subnormals, +-0, +-448); one
    token is all zero, one has a single nonzero element, one ties in the router."""
    K, I, E, M = 256, 256, 4, 4
    pr = Problem(21, M, K, I, E)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    rng = np.random.default_rng(0)
    for slot in range(E + 1):
        w13 = finite[rng.integers(0, finite.size, (K, 2 * I))]
        w2 = finite[rng.integers(0, finite.size, (I, K))]
        s13 = (rng.uniform(0.5, 2, 2 * I) / 448 / 16).astype(np.float32)
        s2 = (rng.uniform(0.5, 2, K) / 448 / 16).astype(np.float32)
        dev = [torch.from_numpy(a).cuda() for a in (w13, s13, w2, s2)]
        pr.ffn.prepack_expert(slot, *dev)
        pr._cpu[slot] = W.Expert(w13, s13, w2, s2)
    x = pr.x.clone()
    x[1] = 0
    x[2] = 0
    x[2, 17] = -3.0
    lg = pr.logits.clone()
    lg[3] = 0
    lg[3, 1] = 1.0
    lg[3, 2] = 1.0  # tie between experts 1 and 2 -> expert 1
    ref = pr.run_oracle(x, lg)
    gpu = pr.run_gpu(x, lg)
    assert ref["expert"][3] == 1
    check_all(gpu, ref, E, pr.weights)
    assert not gpu["xq"][1].any() and gpu["s_x"][1] == 0
    assert (ofp8.bf16_to_f64(gpu["out"][1]) == 0).all()


def test_empty_batch_is_a_noop(lib):
    pr = Problem(5, 2, 256, 512, 4)
    out = torch.full((2, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    st = pr.ffn.forward_raw(pr.x.data_ptr(), pr.logits.data_ptr(), out.data_ptr(), 0,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == F.OK and (out == 7.0).all()


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_dense_full_size(lib, M):
    """The shared-expert FFN at Maverick size (K=5120, I=8192), decode and verify shapes."""
    say("case dense full M =", M)
    pr = Problem(0, M, W.HIDDEN, W.INTER, 0)
    ref = pr.run_oracle()
    for mode in modes_for(M):
        pr.set_mode(mode)
        s = check_all(pr.run_gpu(), ref, 0, pr.weights, max_conditioned=0)
        say("dense", s)


# Shapes where a lane's share of x exceeds its early registers by one or two 16-byte
# chunks, so that the rest is loaded early into LDS: 5 or more tokens with 4096 < K <=
# 5120 (at most 4 tokens need a larger K than the library takes); at 16 tokens a
# wave's second token takes the late path.
STAGED_CASES = [(61, 8, 5120, 256, 3), (62, 5, 4608, 384, 0), (63, 6, 4224, 256, 2), (64, 16, 5120, 128, 2),
                (65, 7, 5120, 128, 6)]


@pytest.mark.parametrize("seed,M,K,I,E", STAGED_CASES)
def test_x_chunks_loaded_early_into_lds(lib, seed, M, K, I, E):
    """Every output, code and scale against the oracle, with and without the fused
    RMSNorm, where part of each lane's x goes through LDS."""
    say("case staged x", M, K, I, E)
    pr = Problem(seed, M, K, I, E)
    ref = pr.run_oracle()
    for mode in modes_for(M):
        pr.set_mode(mode)
        s = check_all(pr.run_gpu(), ref, E, pr.weights)
    norm = (W.norm_weight(seed, K).cuda(), 1e-5)
    s2 = check_all(pr.run_gpu(norm=norm), pr.run_oracle(norm=norm), E, pr.weights)
    say("staged", s, s2)


@pytest.fixture(scope="module")
def routed_full(lib):
    say("building 128-expert pool")
    c = W.ROUTED
    pr = Problem(c["seed"], c["M"], c["hidden"], c["inter"], c["num_experts"])
    return pr


@pytest.mark.parametrize("d", [1, 2, 3, 4])
def test_routed_full_size(routed_full, d):
    pr = routed_full
    targets = W.distinct_targets(pr.seed, d, pr.E, pr.M)
    lg = W.force_routing(pr.logits, targets)
    say("case routed full d =", d, targets)
    gpu = pr.run_gpu(logits=lg)
    ref = pr.run_oracle(logits=lg)
    assert int(gpu["num_active"][0]) == d
    s = check_all(gpu, ref, pr.E, pr.weights, max_conditioned=0)
    say("routed", d, s)


def test_routed_natural_logits(routed_full):
    pr = routed_full
    check_all(pr.run_gpu(), pr.run_oracle(), pr.E, pr.weights, max_conditioned=0)


@pytest.mark.parametrize("d", [1, 4])
def test_tensor_parallel_shard_full_size(lib, d):
    """One GPU's share of the step split 8 ways over the intermediate dimension: hidden
    5120, I / 8 = 1024 columns of every expert's gate and up projections (and the matching
    rows of the down projection), 128 routed experts + shared, 4 tokens on d distinct
    experts.  On one GPU the intermediate's scale spans the local share."""
    M, K, I, E = 4, W.HIDDEN, W.INTER // 8, W.EXPERTS
    say("case tp shard", M, K, I, E, "d =", d)
    targets = W.distinct_targets(0, d, E, M)
    pr = Problem(0, M, K, I, E, force=targets)
    gpu = pr.run_gpu()
    assert int(gpu["num_active"][0]) == d
    s = check_all(gpu, pr.run_oracle(), E, pr.weights, max_conditioned=0)
    say("tp shard", d, s)


def test_deterministic_and_batch_invariant(lib):
    pr = Problem(7, 4, 512, 1024, 6)
    first = pr.run_gpu()
    for _ in range(20):
        again = pr.run_gpu()
        for k in first:
            assert np.array_equal(first[k], again[k]), k
    for m in range(4):  # row m of the M=4 output equals an M=1 call on row m
        one = pr.run_gpu(pr.x[m:m + 1].contiguous(), pr.logits[m:m + 1].contiguous())
        assert np.array_equal(one["out"][0], first["out"][m])


@pytest.mark.parametrize("M", [4, 40])
def test_graph_capture_replays(lib, M):
    """A forward captured into a HIP graph replays to the eager result, with eager forwards
    in between: one decode launch (M = 4) and one grouped pass (M = 40, whose work counters
    and row maxima are cleared by its first kernel, not by a memset)."""
    pr = Problem(8, M, 512, 1024, 6)
    out = torch.empty((M, 512), dtype=torch.bfloat16, device="cuda")
    pr.ffn.forward(pr.x, pr.logits, out)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pr.ffn.forward(pr.x, pr.logits, out)
    torch.cuda.synchronize()
    for i in range(5):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        pr.ffn.forward(pr.x, pr.logits, torch.empty_like(out))  # eager work in between


def test_argument_errors_on_device(lib):
    pr = Problem(9, 2, 256, 512, 4)
    out = torch.empty((2, 256), dtype=torch.bfloat16, device="cuda")
    strm = torch.cuda.current_stream().cuda_stream
    f = pr.ffn.forward_raw
    assert f(pr.x.data_ptr(), pr.logits.data_ptr(), out.data_ptr(), 3, strm) == F.ERR_INVALID_ARG  # M > max
    assert f(pr.x.data_ptr(), pr.logits.data_ptr(), out.data_ptr(), -1, strm) == F.ERR_INVALID_ARG
    assert f(pr.x.data_ptr(), None, out.data_ptr(), 2, strm) == F.ERR_INVALID_ARG  # logits needed
    assert f(pr.x.data_ptr(), pr.logits.data_ptr(), pr.x.data_ptr(), 2, strm) == F.ERR_INVALID_ARG  # alias
    host = torch.empty((2, 256), dtype=torch.bfloat16)
    assert f(host.data_ptr(), pr.logits.data_ptr(), out.data_ptr(), 2, strm) == F.ERR_INVALID_ARG
    # a pointer near the end of its own hipMalloc allocation: the range check refuses it
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    raw = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(raw), ctypes.c_size_t(1 << 16)) == 0
    p_end = raw.value + (1 << 16) - 64  # 64 bytes left, a [2][256] bf16 input needs 1024
    lib_ = F.load()
    st = lib_.moe_ffn_fp8_forward(p_end, pr.logits.data_ptr(), pr.ffn.handle, out.data_ptr(), 2, strm)
    assert st == F.ERR_INVALID_ARG
    st = lib_.moe_ffn_fp8_forward(raw.value, pr.logits.data_ptr(), pr.ffn.handle, out.data_ptr(), 2, strm)
    assert st == F.OK  # the same allocation from its start is large enough
    torch.cuda.synchronize()
    assert hip.hipFree(raw) == 0
    # dense handle refuses logits
    dn = F.MoeFFN(256, 512, 0, 2)
    assert dn.forward_raw(pr.x.data_ptr(), pr.logits.data_ptr(), out.data_ptr(), 2, strm) == F.ERR_INVALID_ARG
    dn.close()
    torch.cuda.synchronize()


def _resolve_variant(variant, base):
    """'low' static scales: half the smallest dynamic scale of the plain step (float32),
    so that the largest values saturate."""
    v = dict(variant)
    if v.get("x_scale") == "low":
        v["x_scale"] = float(np.float32(base["s_x"].min() / 2))
    if v.get("a_scale") == "low":
        sa = np.concatenate([base["s_a_shared"], base["s_a_routed"][base["s_a_routed"] > 0]])
        v["a_scale"] = float(np.float32(sa.min() / 2))
    return v


VARIANTS = [dict(gate_on_input=1), dict(x_scale="low"), dict(a_scale="low"), dict(x_scale="low", a_scale="low"),
            dict(gate_on_input=1, x_scale="low", a_scale="low")]


@pytest.mark.parametrize("variant", VARIANTS, ids=["gate_on_input", "static_x", "static_a", "static_x_a", "all"])
def test_variant_readings(lib, variant):
    """The variant readings (gate on the routed expert's input; static calibrated
    scales that saturate the largest values) against the oracle's variants: every
    output, code and scale, a ragged shape and a batch above one launch."""
    for seed, M, K, I, E in [(41, 4, 256, 512, 4), (42, 13, 384, 640, 3), (43, 37, 256, 256, 5)]:
        say("case variant", variant, M, K, I, E)
        pr = Problem(seed, M, K, I, E)
        v = _resolve_variant(variant, pr.run_oracle())
        ref = pr.run_oracle(variant=v)
        gpu = pr.run_gpu(variant=v)
        s = check_all(gpu, ref, E, pr.weights, gate_on_input=bool(v.get("gate_on_input")), a_scale=v.get("a_scale"))
        if "x_scale" in v:
            assert (gpu["s_x"] == np.float32(v["x_scale"])).all() and (gpu["xq"] & 0x7F == 0x7E).any()
        if "a_scale" in v:
            assert (gpu["s_a_shared"] == np.float32(v["a_scale"])).all()
        say("variant", s)


@pytest.mark.parametrize("variant", [dict(gate_on_input=1), dict(x_scale="low", a_scale="low")],
                         ids=["gate_on_input", "static_x_a"])
def test_variant_readings_full_size(routed_full, variant):
    pr = routed_full
    targets = W.distinct_targets(pr.seed, 4, pr.E, pr.M)
    lg = W.force_routing(pr.logits, targets)
    v = _resolve_variant(variant, pr.run_oracle(logits=lg))
    say("case variant full size", v)
    gpu = pr.run_gpu(logits=lg, variant=v)
    ref = pr.run_oracle(logits=lg, variant=v)
    check_all(gpu, ref, pr.E, pr.weights, gate_on_input=bool(v.get("gate_on_input")), a_scale=v.get("a_scale"))


def test_variant_argument_errors(lib):
    pr = Problem(5, 2, 256, 512, 4)
    out = torch.empty((2, 256), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for bad, want in [(F.Variant(2, 0.0, 0.0), F.ERR_INVALID_ARG), (F.Variant(0, -1.0, 0.0), F.ERR_INVALID_ARG),
                      (F.Variant(0, 0.0, float("nan")), F.ERR_INVALID_ARG),
                      (F.Variant(0, float("inf"), 0.0), F.ERR_INVALID_ARG)]:
        st = pr.ffn.forward_variant_raw(pr.x.data_ptr(), pr.logits.data_ptr(), out.data_ptr(), 2, s, bad)
        assert st == want, (bad.gate_on_input, bad.x_scale, bad.a_scale, st)
    torch.cuda.synchronize()


RMS_CASES = [(51, 4, 256, 512, 4), (52, 13, 384, 640, 3), (53, 37, 256, 256, 5), (54, 8, 512, 256, 0),
             (55, 1, 128, 128, 1)]


@pytest.mark.parametrize("seed,M,K,I,E", RMS_CASES)
def test_fused_rmsnorm(lib, seed, M, K, I, E):
    """The step on rmsnorm(h) * w, the norm fused into the first kernel: every output,
    code and scale against the oracle (a ragged shape, a batch above one launch, the
    dense FFN, one token)."""
    say("case rmsnorm", M, K, I, E)
    pr = Problem(seed, M, K, I, E)
    norm = (W.norm_weight(seed, K).cuda(), 1e-5)
    s = check_all(pr.run_gpu(norm=norm), pr.run_oracle(norm=norm), E, pr.weights)
    say("rmsnorm", s)


def test_fused_rmsnorm_with_variants_and_a_scaled_input(lib):
    """The norm with the input gate and static scales, on a hidden state far from unit
    RMS (the norm's scale invariance carries the step)."""
    seed, M, K, I, E = 56, 6, 384, 512, 3
    pr = Problem(seed, M, K, I, E)
    h = (pr.x.float() * 37.0).to(torch.bfloat16)
    norm = (W.norm_weight(seed, K).cuda(), 1e-6)
    v = _resolve_variant(dict(gate_on_input=1, x_scale="low", a_scale="low"), pr.run_oracle(h, norm=norm))
    check_all(pr.run_gpu(h, variant=v, norm=norm), pr.run_oracle(h, variant=v, norm=norm), E, pr.weights,
              gate_on_input=True, a_scale=v["a_scale"])


def test_fused_rmsnorm_full_size(routed_full):
    pr = routed_full
    targets = W.distinct_targets(pr.seed, 4, pr.E, pr.M)
    lg = W.force_routing(pr.logits, targets)
    norm = (W.norm_weight(pr.seed, pr.K).cuda(), 1e-5)
    say("case rmsnorm full size")
    check_all(pr.run_gpu(logits=lg, norm=norm), pr.run_oracle(logits=lg, norm=norm), pr.E, pr.weights)


def test_fused_rmsnorm_argument_errors(lib):
    pr = Problem(5, 2, 256, 512, 4)
    out = torch.empty((2, 256), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    nw = W.norm_weight(5, 256).cuda()
    for w_ptr, eps, want in [(0, 1e-5, F.ERR_INVALID_ARG), (nw.data_ptr(), -1.0, F.ERR_INVALID_ARG),
                             (nw.data_ptr(), float("nan"), F.ERR_INVALID_ARG),
                             (nw.data_ptr() + 2, 1e-5, F.ERR_INVALID_ARG)]:
        st = pr.ffn.forward_rmsnorm_raw(pr.x.data_ptr(), w_ptr, eps, pr.logits.data_ptr(), out.data_ptr(), 2, s)
        assert st == want, (w_ptr, eps, st)
    torch.cuda.synchronize()
