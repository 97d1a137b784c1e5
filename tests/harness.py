"""Shared pieces of the GPU parity tests: build a seeded problem, run it through the
C ABI and through the oracle, and apply the acceptance checks.

Acceptance (written into the checks below):
* bf16 output: |gpu - ref| <= 1e-2 * |ref| + 1e-2 * rms(ref) element-wise, ref being
  the oracle's float64 result before rounding.  For a token whose re-quantised codes
  differ from the oracle's (allowed below: a float32 intermediate within rounding of an
  e4m3 midpoint may round the other way, and one such code moves the output by up to
  several tolerances at small I) and whose output misses that bar, ref is the oracle's
  FC2 and combine applied to the kernel's own codes and scales, which are checked on
  their own;
* likewise one stage earlier: for a token whose activation codes differ from the
  oracle's (allowed below; with the fused RMSNorm the kernel quantises float32 values
  that can sit within rounding of a midpoint), the intermediate, its codes and scales and
  the output are compared with the oracle's step from the kernel's own activation codes
  and scale (one flipped input code moves the intermediate by a few percent at small K,
  and a near-zero value can change sign);
* FP8 codes (activations and the re-quantised intermediate): |ord(gpu) - ord(ref)| <= 1
  and nonzero in at most 0.1% of the elements, ord(c) = +-(c & 0x7F);
* the activation codes and scales of every path that quantises the bf16 input itself
  (all but the fused RMSNorm, which quantises float32 normalised values): bit for bit,
  and s_x exactly fp32(amax / 448), since those paths decide every rounding exactly;
  then no token is conditioned on its activation codes;
* every output is first held to the oracle's own result; a token is conditioned on its
  re-quantised codes only when they differ and its output then misses the bar; such tokens
  are counted and capped per call (``max_conditioned``; by default max(1, M // 100), and 0
  where a test says so);
* routing (expert index, number of distinct experts): exact;
* gate, s_a: relative 1e-6.
"""

from __future__ import annotations

import numpy as np
import torch

import fp8_moe_ffn_amd as F
import workloads as W
from oracle import ffn as oracle_ffn
from oracle import fp8 as ofp8


class Problem:
    def __init__(self, seed, M, hidden, inter, num_experts, device="cuda", force=None,
                 gen_device=None, keep_sources=None):
        self.seed, self.M, self.K, self.I, self.E = seed, M, hidden, inter, num_experts
        gen_device = gen_device or ("cpu" if hidden * inter <= 4 << 20 else device)
        self.gen_device = gen_device
        self.x = W.activations(seed, M, hidden, gen_device).to(device)
        self.logits = (W.router_logits(seed, M, num_experts, gen_device, force=force).to(device)
                       if num_experts else None)
        if keep_sources is None:  # host copies only while they stay small
            keep_sources = (num_experts + 1) * 3 * hidden * inter < (1 << 30)
        self.ffn = F.MoeFFN(hidden, inter, num_experts, max(M, 1))
        self.mode = F.BATCH_GROUPED
        self._cpu = {}
        for slot in range(num_experts + 1):
            e = W.expert(seed, slot, hidden, inter, gen_device)
            dev = W.Expert(*(t.to(device) for t in (e.w13, e.s13, e.w2, e.s2)))
            self.ffn.prepack_expert(slot, dev.w13, dev.s13, dev.w2, dev.s2)
            if keep_sources:
                self._cpu[slot] = e.numpy()
        torch.cuda.synchronize()

    def weights(self, slot):
        if slot not in self._cpu:  # regenerate (same seed -> same codes)
            self._cpu[slot] = W.expert(self.seed, slot, self.K, self.I, self.gen_device).numpy()
        return self._cpu[slot]

    def set_mode(self, mode):
        self.ffn.set_batch_mode(mode)
        self.mode = mode

    def run_gpu(self, x=None, logits=None, variant=None, norm=None):
        """variant: a dict of moe_ffn_fp8_variant fields (None: the plain forward);
        norm: (norm weight bf16 tensor [K] on the device, eps) for the fused RMSNorm, x
        then being the hidden state."""
        x = self.x if x is None else x
        logits = self.logits if logits is None else logits
        M = x.shape[0]
        out = torch.empty((M, self.K), dtype=torch.bfloat16, device=x.device)
        dbg = F.debug_buffers(M, self.K, self.I, x.device)
        if norm is not None:
            v = variant or {}
            var = F.Variant(int(v.get("gate_on_input", 0)), float(v.get("x_scale") or 0.0),
                            float(v.get("a_scale") or 0.0))
            self.ffn.forward_rmsnorm(x, norm[0], norm[1], logits, out, var, dbg)
        elif variant is None:
            self.ffn.forward_debug(x, logits, out, dbg)
        else:
            self.ffn.forward_variant(x, logits, out, F.Variant(int(variant.get("gate_on_input", 0)),
                                                               float(variant.get("x_scale") or 0.0),
                                                               float(variant.get("a_scale") or 0.0)), dbg)
        torch.cuda.synchronize()
        r = {k: getattr(dbg, k).cpu().numpy() for k in
             ("xq", "s_x", "expert", "gate", "aq_shared", "s_a_shared", "aq_routed", "s_a_routed",
              "num_active")}
        assert int(dbg.sync_timeouts.item()) == 0, "a single launch gave up waiting for a phase"
        r["out"] = W.bits(out)
        # how a batch above one launch ran (the variants and the fused norm: always chunked)
        r["batch_mode"] = F.BATCH_CHUNKED if (variant is not None or norm is not None) else self.mode
        # the fused norm quantises float32 normalised values, which can sit within rounding
        # of a midpoint where the oracle's float64 ones do not; every other path is exact
        r["x_exact"] = norm is None
        return r

    def run_oracle(self, x=None, logits=None, variant=None, norm=None):
        x = self.x if x is None else x
        logits = self.logits if logits is None else logits
        lg = W.bits(logits) if logits is not None else None
        v = variant or {}
        return oracle_ffn.forward(W.bits(x), lg, self.weights, self.E,
                                  gate_on_input=bool(v.get("gate_on_input", 0)),
                                  x_scale=v.get("x_scale"), a_scale=v.get("a_scale"),
                                  norm_w_bits=W.bits(norm[0]) if norm is not None else None,
                                  norm_eps=norm[1] if norm is not None else 1e-5)


def ordv(c):
    c = np.asarray(c, np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def check_codes(got, ref, what, max_frac=1e-3):
    d = np.abs(ordv(got) - ordv(ref))
    assert d.max(initial=0) <= 1, f"{what}: a code differs by {d.max()}"
    frac = (d != 0).mean() if d.size else 0.0
    assert frac <= max_frac, f"{what}: {frac:.4%} of codes differ"
    return frac


def check_rel(got, ref, what, rtol=1e-6):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = np.abs(got - ref) > rtol * np.abs(ref)
    assert not bad.any(), f"{what}: {got[bad][:4]} vs {ref[bad][:4]}"


def rows_within_tolerance(out_bits, ref):
    """Per token: is every element of its bf16 output within the bar of check_output?"""
    got = ofp8.bf16_to_f64(out_bits)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    return np.all(np.abs(got - ref) <= 1e-2 * np.abs(ref) + 1e-2 * rms, axis=1)


def check_output(out_bits, ref, what="out"):
    got = ofp8.bf16_to_f64(out_bits)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    err = np.abs(got - ref)
    tol = 1e-2 * np.abs(ref) + 1e-2 * rms
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert np.all(err <= tol), f"{what}: max err/tol {np.max(err / np.maximum(tol, 1e-300)):.3f}"
    return float(np.max(err / np.maximum(tol, 1e-300))) if ref.size else 0.0


def chunked_active(experts, chunk=F.CHUNK):
    """Routed experts streamed by a forward that runs in launches of `chunk` tokens:
    the distinct experts of each chunk, summed.  A batch above one launch is taken in
    routed-expert order (ascending expert, then token), so its chunks are runs of that
    sorted sequence."""
    e = [int(v) for v in experts]
    if len(e) > chunk:
        e = sorted(e)
    return sum(len(set(e[i:i + chunk])) for i in range(0, len(e), chunk))


def grouped_active(experts, group=F.GROUP_MAX):
    """Routed experts streamed by a forward that runs grouped passes of `group`
    consecutive tokens: the distinct experts of each pass, summed."""
    e = [int(v) for v in experts]
    return sum(len(set(e[i:i + group])) for i in range(0, len(e), group))


def streamed_active(experts, mode=F.BATCH_GROUPED):
    """Routed experts a forward streams: one launch up to GROUP_FROM tokens, else by batch
    mode (the chunked mode: launches of up to CHUNK tokens)."""
    if len(experts) <= F.GROUP_FROM or mode == F.BATCH_CHUNKED:
        return chunked_active(experts)
    return grouped_active(experts)


def conditioned_ref(gpu, ref, weights, num_experts, rows, gate_on_input=False):
    """Float64 output of tokens `rows` from the kernel's re-quantised codes and scales:
    the oracle's FC2 of each expert and its combine, with the oracle's routing (the gate
    on the routed output unless it scaled the input)."""
    E = num_experts
    y = oracle_ffn.fc2(gpu["aq_shared"][rows], np.asarray(gpu["s_a_shared"], np.float64)[rows],
                       weights(E))
    if E:
        yr = np.zeros_like(y)
        ex = np.asarray(ref["expert"])[rows]
        for e in np.unique(ex):
            sel = np.nonzero(ex == e)[0]
            yr[sel] = oracle_ffn.fc2(gpu["aq_routed"][rows][sel],
                                     np.asarray(gpu["s_a_routed"], np.float64)[rows][sel], weights(int(e)))
        y = y + (yr if gate_on_input else np.asarray(ref["gate"])[rows][:, None] * yr)
    return y


def conditioned_step(gpu, ref, weights, num_experts, rows, gate_on_input=False, a_scale=None):
    """The oracle's step after the activation quantisation, for tokens `rows`, from the
    kernel's own activation codes and scales (routing and gates the oracle's)."""
    E = num_experts
    xq = np.asarray(gpu["xq"])[rows]
    sx = np.asarray(gpu["s_x"], np.float64)[rows]
    sh = oracle_ffn.expert_ffn(xq, sx, weights(E), a_scale)
    res = {"aq_shared": sh["aq"], "s_a_shared": sh["s_a"], "ref": sh["y"].copy()}
    if E:
        ex = np.asarray(ref["expert"])[rows]
        g = np.asarray(ref["gate"])[rows]
        aq_r = np.zeros_like(sh["aq"])
        sa_r = np.zeros(len(rows))
        y_r = np.zeros_like(sh["y"])
        for e in np.unique(ex):
            sel = np.nonzero(ex == e)[0]
            r = oracle_ffn.expert_ffn(xq[sel], sx[sel] * g[sel] if gate_on_input else sx[sel],
                                      weights(int(e)), a_scale)
            aq_r[sel], sa_r[sel], y_r[sel] = r["aq"], r["s_a"], r["y"]
        res.update({"aq_routed": aq_r, "s_a_routed": sa_r})
        res["ref"] = res["ref"] + (y_r if gate_on_input else g[:, None] * y_r)
    return res


def default_cap(M):
    """Tokens that may be conditioned on their re-quantised codes: a flip needs a float32
    intermediate within a few units in the last place of a rounding midpoint, about one
    value in 2**20 (fewer than 1 token in 100 at I = 8192 with a shared and a routed row
    each)."""
    return max(1, M // 100)


def check_all(gpu, ref, num_experts, weights, gate_on_input=False, a_scale=None, mode=None,
              x_exact=None, max_conditioned=None):
    """Every acceptance check; returns a small summary for printing.  `weights` maps an
    expert slot to its codes and scales (for tokens whose codes differ from the oracle's);
    gate_on_input and a_scale are the variant the step ran under; mode the batch mode
    (for the count of streamed experts; default: what run_gpu recorded).  x_exact: the
    activation codes and scales must equal the oracle's bit for bit (every path but the
    fused RMSNorm); max_conditioned: the cap on tokens conditioned on their re-quantised
    codes (default: default_cap(M))."""
    if mode is None:
        mode = gpu.get("batch_mode", F.BATCH_GROUPED)
    M = ref["out"].shape[0]
    if max_conditioned is None:
        max_conditioned = default_cap(M)
    if x_exact is None:
        x_exact = gpu.get("x_exact", True)
    s = {}
    if x_exact:
        got, want = np.asarray(gpu["xq"], np.uint8), np.asarray(ref["xq"], np.uint8)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"xq differs at {bad[:4].tolist()}: {got[tuple(bad[:4].T)]} vs {want[tuple(bad[:4].T)]}"
        sx_ref = np.asarray(ref["s_x"], np.float64).astype(np.float32)
        assert np.array_equal(np.asarray(gpu["s_x"], np.float32).view(np.uint32), sx_ref.view(np.uint32)), \
            f"s_x differs: {np.asarray(gpu['s_x'])[:4]} vs {sx_ref[:4]}"
    s["xq"] = check_codes(gpu["xq"], ref["xq"], "xq")
    check_rel(gpu["s_x"], ref["s_x"], "s_x")
    xdiff = (ordv(gpu["xq"]) != ordv(ref["xq"])).any(axis=1)
    s["tokens_x_conditioned"] = int(xdiff.sum())
    if xdiff.any():  # from here on, those tokens follow the kernel's own activation codes
        rows = np.nonzero(xdiff)[0]
        c = conditioned_step(gpu, ref, weights, num_experts, rows, gate_on_input, a_scale)
        ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
        for k, v in c.items():
            ref[k][rows] = v
    s["aq_shared"] = check_codes(gpu["aq_shared"], ref["aq_shared"], "aq_shared")
    check_rel(gpu["s_a_shared"], ref["s_a_shared"], "s_a_shared")
    if num_experts:
        assert gpu["expert"].tolist() == ref["expert"].tolist(), "routing differs"
        assert int(gpu["num_active"][0]) == streamed_active(ref["expert"], mode)
        check_rel(gpu["gate"], ref["gate"], "gate")
        s["aq_routed"] = check_codes(gpu["aq_routed"], ref["aq_routed"], "aq_routed")
        check_rel(gpu["s_a_routed"], ref["s_a_routed"], "s_a_routed")
    else:
        assert (gpu["expert"] == -1).all() and int(gpu["num_active"][0]) == 0
    differ = (ordv(gpu["aq_shared"]) != ordv(ref["aq_shared"])).any(axis=1)
    if num_experts:
        differ |= (ordv(gpu["aq_routed"]) != ordv(ref["aq_routed"])).any(axis=1)
    s["tokens_codes_differ"] = int(differ.sum())
    # every token's output against the oracle's own result first; only a token whose
    # re-quantised codes differ and whose output then misses the bar is compared with the
    # oracle's FC2 of the kernel's codes (at I = 8192 one code step moves an output by far
    # less than the tolerance; at small I it can move it by more)
    target = ref["ref"]
    miss = ~rows_within_tolerance(gpu["out"], target)
    assert not (miss & ~differ).any(), \
        f"tokens {np.nonzero(miss & ~differ)[0][:8].tolist()} miss the output bar with the oracle's own codes"
    if miss.any():
        rows = np.nonzero(miss)[0]
        target = target.copy()
        target[rows] = conditioned_ref(gpu, ref, weights, num_experts, rows, gate_on_input)
    s["tokens_conditioned"] = int(miss.sum())
    assert s["tokens_conditioned"] <= max_conditioned, \
        f"{s['tokens_conditioned']} tokens conditioned on their re-quantised codes (cap {max_conditioned})"
    s["out_err_over_tol"] = check_output(gpu["out"], target)
    s["M"] = M
    return s
