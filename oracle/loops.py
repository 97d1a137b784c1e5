"""A second, loop-only evaluation of the step for tiny inputs.

Test infrastructure (see ``oracle/__init__.py``): never imported by the product path.

It computes the same definition as ``oracle.ffn.forward`` with independent code:

* e4m3 values come from the bit fields through ``math.ldexp`` (not a table);
* encoding is a linear search over all 127 non-negative finite codes for the
  smallest distance, ties going to the even code (not a midpoint search);
* sums are plain Python loops in the order k = 0, 1, ...;
* bf16 rounding uses exact rational arithmetic (``fractions.Fraction``) and
  Python's round-half-to-even ``round``.

Pure Python: use it only for sizes of a few hundred by a few hundred.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction


def dec(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m, -9)
    return s * math.ldexp(8 + m, e - 10)  # (1 + m/8) * 2**(e-7) = (8+m) * 2**(e-10)


def enc(v: float) -> int:
    a = abs(v)
    best, best_d = 0, math.inf
    for c in range(0x7F):  # 0x00 .. 0x7E, all non-negative finite codes
        d = abs(dec(c) - a)
        if d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    if a >= 448.0:
        best = 0x7E
    return best | (0x80 if math.copysign(1.0, v) < 0 else 0)


def to_f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16_bits_to_float(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (b & 0xFFFF) << 16))[0]


def float_to_bf16_bits(v: float) -> int:
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    _, e = math.frexp(v)  # |v| in [2**(e-1), 2**e)
    unit = Fraction(2) ** (e - 8)  # spacing of 8-significant-bit numbers in that binade
    r = round(Fraction(v) / unit) * unit  # Fraction round(): half to even
    return struct.unpack("<I", struct.pack("<f", float(r)))[0] >> 16


def quant_row(vals, static=None):
    if static is not None:  # one calibrated scale for the tensor; enc saturates
        return [enc(v / static) for v in vals], static
    amax = 0.0
    for v in vals:
        amax = max(amax, abs(v))
    s = to_f32(amax / 448.0)
    if s == 0.0:
        return [0] * len(vals), 0.0
    return [enc(v / s) for v in vals], s


def expert_rows(xq_rows, sx_rows, w13, s13, w2, s2, a_scale=None):
    """w13 [K][2I] and w2 [I][K] as nested lists of codes."""
    hidden = len(w13)
    inter = len(w13[0]) // 2
    out = []
    for xq, sx in zip(xq_rows, sx_rows):
        a = []
        for n in range(inter):
            g = 0.0
            u = 0.0
            for k in range(hidden):
                xv = dec(xq[k])
                g += xv * dec(w13[k][n])
                u += xv * dec(w13[k][inter + n])
            g = g * sx * s13[n]
            u = u * sx * s13[inter + n]
            sig = 1.0 / (1.0 + math.exp(-g)) if g > -700 else 0.0
            a.append(g * sig * u)
        aq, sa = quant_row(a, a_scale)
        y = []
        for k in range(hidden):
            acc = 0.0
            for j in range(inter):
                acc += dec(aq[j]) * dec(w2[j][k])
            y.append(acc * sa * s2[k])
        out.append({"a": a, "aq": aq, "s_a": sa, "y": y})
    return out


def forward(x_bits, logits_bits, weights, num_experts, gate_on_input=False, x_scale=None, a_scale=None,
            norm_w_bits=None, norm_eps=1e-5):
    """Same contract as ``oracle.ffn.forward`` (variants included) but with nested
    lists in and out.

    ``weights(slot)`` returns ``(w13, s13, w2, s2)`` as nested lists / lists.
    """
    x = [[bf16_bits_to_float(b) for b in row] for row in x_bits]
    if norm_w_bits is not None:  # RMSNorm: a plain sum of squares, divided by K
        nw = [bf16_bits_to_float(b) for b in norm_w_bits]
        normed = []
        for row in x:
            ss = 0.0
            for v in row:
                ss += v * v
            d = math.sqrt(ss / len(row) + norm_eps)
            normed.append([v / d * nw[k] for k, v in enumerate(row)])
        x = normed
    qs = [quant_row(row, x_scale) for row in x]
    xq = [q for q, _ in qs]
    sx = [s for _, s in qs]
    sh = expert_rows(xq, sx, *weights(num_experts), a_scale=a_scale)
    m_tok = len(x)
    expert = [-1] * m_tok
    gate = [0.0] * m_tok
    routed = [None] * m_tok
    if num_experts > 0:
        for m in range(m_tok):
            row = [bf16_bits_to_float(b) for b in logits_bits[m]]
            best = 0
            for e in range(1, len(row)):
                if row[e] > row[best]:
                    best = e
            expert[m] = best
            gate[m] = 1.0 / (1.0 + math.exp(-row[best]))
            if gate_on_input:  # the token's codes, its scale times the gate
                routed[m] = expert_rows([xq[m]], [sx[m] * gate[m]], *weights(best), a_scale=a_scale)[0]
            else:
                routed[m] = expert_rows([xq[m]], [sx[m]], *weights(best), a_scale=a_scale)[0]
    ref = []
    for m in range(m_tok):
        r = list(sh[m]["y"])
        if routed[m] is not None:
            g = 1.0 if gate_on_input else gate[m]
            r = [r[k] + g * routed[m]["y"][k] for k in range(len(r))]
        ref.append(r)
    out = [[float_to_bf16_bits(v) for v in row] for row in ref]
    return {"xq": xq, "s_x": sx, "expert": expert, "gate": gate,
            "aq_shared": [s["aq"] for s in sh], "s_a_shared": [s["s_a"] for s in sh],
            "aq_routed": [r["aq"] if r else None for r in routed],
            "s_a_routed": [r["s_a"] if r else 0.0 for r in routed],
            "ref": ref, "out": out}
