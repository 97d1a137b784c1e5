"""The FP8 MoE feed-forward step, evaluated in float64 on the CPU.

Test infrastructure (see ``oracle/__init__.py``): never imported by the product path.

Notation: M tokens, K hidden size, I intermediate size, E routed experts.  An
expert's weights are e4m3 codes with one float32 scale per output channel:

* ``w13`` codes ``[K][2I]``: columns ``[0, I)`` are the gate projection (FC1), columns
  ``[I, 2I)`` the up projection (FC3); ``s13`` float32 ``[2I]``.
* ``w2`` codes ``[I][K]`` (the down projection, FC2); ``s2`` float32 ``[K]``.

The pages name the fused FC13 + SwiGLU GEMM and the quantize step in front of a
GEMM (Blackwell 1,000 TPS/user blog, zh translation, section "CUDA kernel
optimisation and fusion", item "operator fusion"), FP8 GEMMs and MoE (same page,
its lead list), and nothing more.  Every further choice below is the plainest
reading of the pages that the rest of them supports, and says so where it is made.

Exactness: an e4m3 value is an integer multiple of 2**-9, so a product of two is a
multiple of 2**-18, and ``|sum| <= 448**2 * K < 2**31`` for K <= 8192.  The float64
sum therefore holds at most 49 significant bits and is exact in any order: BLAS may
do the contraction (``tests/test_oracle_ffn.py`` checks it against int64 sums).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence, Union

import numpy as np

from .fp8 import E4M3_MAX, bf16_to_f64, e4m3_decode, e4m3_encode, f64_to_bf16, fp32_round


@dataclass
class ExpertWeights:
    """e4m3 codes and float32 per-output-channel scales of one expert."""

    w13: np.ndarray  # uint8 [K][2I]
    s13: np.ndarray  # float32 [2I]
    w2: np.ndarray  # uint8 [I][K]
    s2: np.ndarray  # float32 [K]


def quantize_rows(v: np.ndarray):
    """Per-row dynamic FP8 quantisation of a float64 matrix ``v [R][C]``.

    ``s[r] = fp32(max_c |v[r, c]| / 448)`` (the float64 quotient rounded once to
    float32) and ``q[r, c] = e4m3(v[r, c] / s[r])`` with the quotient in float64.
    A row of zeros gets scale 0 and codes 0.  Returns ``(codes uint8, s float64)``
    where every ``s`` value is a float32 value.
    """
    v = np.asarray(v, dtype=np.float64)
    amax = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(v.shape[0])
    s = fp32_round(amax / E4M3_MAX)
    safe = np.where(s > 0, s, 1.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = e4m3_encode(v / safe[:, None])
    q[s == 0, :] = 0
    return q, s


def quantize_static(v: np.ndarray, s: float) -> np.ndarray:
    """Static FP8 quantisation with one calibrated scale for the whole tensor:
    ``q = e4m3(v / s)``, the quotient in float64, saturating at +-448 (``s > 0``).
    This is the variant reading of the activation scale that takes the quantize step
    with a scale fixed ahead of time instead of the per-token maximum."""
    assert s > 0
    return e4m3_encode(np.asarray(v, dtype=np.float64) / np.float64(s))


def rmsnorm(h: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row in float64: ``h / sqrt(mean_k h**2 + eps) * w``.

    The pages fuse the AllReduce with the RMSNorm that follows it and the quantize step
    into one kernel (Blackwell 1,000 TPS/user blog, zh translation, section "CUDA kernel
    optimisation and fusion", item "operator fusion"); here the norm feeds the
    per-token quantisation directly, from the unrounded value (never bf16), as the
    intermediate does."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=1, keepdims=True)
    return h / np.sqrt(ms + np.float64(eps)) * np.asarray(w, dtype=np.float64)[None, :]


def route_top1(logits: np.ndarray):
    """Top-1 routing with a sigmoid gate.

    ``e[m]`` is the lowest expert index among the largest logits of token m;
    ``gate[m] = 1 / (1 + exp(-logit[m, e[m]]))``.  No renormalisation.
    """
    logits = np.asarray(logits, dtype=np.float64)
    e = np.argmax(logits, axis=1)  # first index of the maximum
    top = logits[np.arange(logits.shape[0]), e]
    with np.errstate(over="ignore"):
        gate = 1.0 / (1.0 + np.exp(-top))
    return e.astype(np.int64), gate


def linear_fp8(q: np.ndarray, s_in: np.ndarray, w: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """``h[m, n] = s_in[m] * s_w[n] * sum_k dec(q[m, k]) * dec(w[k, n])``.

    The sum is exact (see the module docstring); the two scale products are
    rounded in float64.
    """
    acc = e4m3_decode(q) @ e4m3_decode(w)
    return acc * np.asarray(s_in, np.float64)[:, None] * np.asarray(s_w, np.float64)[None, :]


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """``silu(g) * u`` with ``silu(z) = z / (1 + exp(-z))``, no clamp and no beta."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def fc13_swiglu(xq, s_x, w: ExpertWeights) -> np.ndarray:
    """Fused gate/up GEMM followed by SwiGLU: returns float64 ``a [M][I]``."""
    h = linear_fp8(xq, s_x, w.w13, w.s13)
    inter = w.w13.shape[1] // 2
    return swiglu(h[:, :inter], h[:, inter:])


def fc2(aq, s_a, w: ExpertWeights) -> np.ndarray:
    """Down projection of the re-quantised intermediate: float64 ``y [M][K]``."""
    return linear_fp8(aq, s_a, w.w2, w.s2)


def expert_ffn(xq, s_x, w: ExpertWeights, a_scale: Optional[float] = None) -> dict:
    """One expert on the given token rows: FC13+SwiGLU, re-quantise (per row, or with
    the static ``a_scale``), FC2."""
    a = fc13_swiglu(xq, s_x, w)
    if a_scale is None:
        aq, s_a = quantize_rows(a)
    else:
        aq, s_a = quantize_static(a, a_scale), np.full(a.shape[0], np.float64(a_scale))
    y = fc2(aq, s_a, w)
    return {"a": a, "aq": aq, "s_a": s_a, "y": y}


WeightSource = Union[Sequence[ExpertWeights], Callable[[int], ExpertWeights]]


def _get(weights: WeightSource, slot: int) -> ExpertWeights:
    return weights(slot) if callable(weights) else weights[slot]


def forward(x_bits: np.ndarray, logits_bits: Optional[np.ndarray], weights: WeightSource,
            num_experts: int, gate_on_input: bool = False, x_scale: Optional[float] = None,
            a_scale: Optional[float] = None, norm_w_bits: Optional[np.ndarray] = None,
            norm_eps: float = 1e-5) -> dict:
    """The whole step.

    Variant readings (defaults: the readings of the step as built):
    ``gate_on_input``: the gate multiplies the token before the routed expert, and the
    output is ``y_shared + y_routed`` instead of the gate multiplying the routed output.
    The token reaches the FFN already quantised once (the pages fuse the quantize step
    into the AllReduce + RMSNorm kernel in front of it), so the gated input is
    ``gate[m] * s_x[m] * dec(xq[m])``: the same codes with the token's scale times the
    gate (float64 product here).
    ``x_scale`` / ``a_scale``: static calibrated scales (one per tensor) for the
    activation and the intermediate, instead of the per-token dynamic ones.
    ``norm_w_bits`` (bf16 bit patterns ``[K]``): the step takes ``x_bits`` as the hidden
    state h and computes on ``rmsnorm(h, norm_w, norm_eps)`` (the fused norm in front).

    ``x_bits`` bf16 bit patterns ``[M][K]``; ``logits_bits`` bf16 bit patterns
    ``[M][E]`` or None when ``num_experts == 0`` (plain dense FFN).  ``weights``
    maps a slot to its ``ExpertWeights``: slots ``0..E-1`` are the routed experts,
    slot ``E`` is the shared expert.

    Returns a dict with ``xq, s_x, expert, gate, a_shared, aq_shared, s_a_shared,
    a_routed, aq_routed, s_a_routed, y_shared, y_routed, ref`` (float64 output before
    rounding) and ``out`` (bf16 bit patterns).  ``*_routed`` row m belongs to the
    expert that token m was routed to; they are zero when E == 0.
    """
    x = bf16_to_f64(x_bits)
    if norm_w_bits is not None:
        x = rmsnorm(x, bf16_to_f64(norm_w_bits), norm_eps)
    m_tok, hidden = x.shape

    def quant_x(v):
        if x_scale is None:
            return quantize_rows(v)
        return quantize_static(v, x_scale), np.full(v.shape[0], np.float64(x_scale))

    xq, s_x = quant_x(x)

    shared = expert_ffn(xq, s_x, _get(weights, num_experts), a_scale)
    ref = shared["y"].copy()
    res = {
        "xq": xq, "s_x": s_x,
        "a_shared": shared["a"], "aq_shared": shared["aq"], "s_a_shared": shared["s_a"],
        "y_shared": shared["y"],
    }
    inter = shared["a"].shape[1]
    a_r = np.zeros((m_tok, inter))
    aq_r = np.zeros((m_tok, inter), dtype=np.uint8)
    s_a_r = np.zeros(m_tok)
    y_r = np.zeros((m_tok, hidden))
    if num_experts > 0:
        expert, gate = route_top1(bf16_to_f64(logits_bits))
        # each routed expert sees only the tokens routed to it
        for e in np.unique(expert):
            rows = np.nonzero(expert == e)[0]
            if gate_on_input:
                xq_e, s_e = xq[rows], s_x[rows] * gate[rows]
            else:
                xq_e, s_e = xq[rows], s_x[rows]
            r = expert_ffn(xq_e, s_e, _get(weights, int(e)), a_scale)
            a_r[rows], aq_r[rows], s_a_r[rows], y_r[rows] = r["a"], r["aq"], r["s_a"], r["y"]
        ref = ref + (y_r if gate_on_input else gate[:, None] * y_r)
    else:
        expert = np.full(m_tok, -1, dtype=np.int64)
        gate = np.zeros(m_tok)
    res.update({"expert": expert, "gate": gate, "a_routed": a_r, "aq_routed": aq_r,
                "s_a_routed": s_a_r, "y_routed": y_r, "ref": ref, "out": f64_to_bf16(ref)})
    return res
