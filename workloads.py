"""Seeded synthetic inputs for the FP8 MoE feed-forward step.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.  It holds none of
the step's arithmetic: random numbers come from torch generators seeded through
``numpy.random.SeedSequence``, and the float -> e4m3 / bf16 conversions of the
inputs are torch's own casts (library routines).  Nothing here imports the oracle
or the HIP library.

Recipe (the pages print no shapes; Maverick-scale sizes: hidden K = 5120,
intermediate I = 8192, 128 routed experts plus one shared expert, top-1):

* weights of expert slot f (slots 0..E-1 routed, slot E shared), matrix t (13 or 2):
  ``w = 0.02 * N(0, 1)`` float32 from a generator seeded with ``(seed, f, t)``;
  one float32 scale per output channel ``s = amax / 448`` (float32 division, amax
  over the reduction axis); codes ``= e4m3(w / s)`` by torch's cast;
* activations ``x = bf16(N(0, 1))`` ``[M][K]``, seeded with ``(seed, 1001, M)``;
* router logits ``bf16(N(0, 1))`` ``[M][E]``, seeded with ``(seed, 1002, M)``;
  optional forcing of the routing (``force_experts``) raises the chosen expert's
  logit to ``bf16(rowmax + 1)`` so that it is the unique maximum;
* Zipf routing: ``perm = permutation(E)`` maps rank to expert, rank r drawn with
  probability proportional to ``r ** -s`` (s = 1.2), then the forcing above.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

HIDDEN = 5120
INTER = 8192
EXPERTS = 128


def _seed(*parts: int) -> int:
    st = np.random.SeedSequence([int(p) for p in parts]).generate_state(2, dtype=np.uint64)
    return int(st[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


@dataclass
class Expert:
    """One expert's codes and scales as torch tensors (all on one device)."""

    w13: torch.Tensor  # uint8 [K][2I]  columns [0,I) gate, [I,2I) up
    s13: torch.Tensor  # float32 [2I]
    w2: torch.Tensor  # uint8 [I][K]
    s2: torch.Tensor  # float32 [K]

    def numpy(self) -> "Expert":
        return Expert(*(t.cpu().numpy() for t in (self.w13, self.s13, self.w2, self.s2)))


def _quantized_matrix(rows: int, cols: int, gen: torch.Generator, device):
    w = torch.randn((rows, cols), generator=gen, device=device, dtype=torch.float32) * 0.02
    s = w.abs().amax(dim=0) / 448.0  # float32 division, per output column
    codes = (w / s).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), s.contiguous()


def expert(seed: int, slot: int, hidden: int, inter: int, device="cpu") -> Expert:
    w13, s13 = _quantized_matrix(hidden, 2 * inter, _gen(device, seed, slot, 13), device)
    w2, s2 = _quantized_matrix(inter, hidden, _gen(device, seed, slot, 2), device)
    return Expert(w13, s13, w2, s2)


def bf16_normal(rows: int, cols: int, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn((rows, cols), generator=gen, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def activations(seed: int, m: int, hidden: int, device="cpu") -> torch.Tensor:
    return bf16_normal(m, hidden, _gen(device, seed, 1001, m), device)


def norm_weight(seed: int, hidden: int, device="cpu") -> torch.Tensor:
    """RMSNorm weight [K] in bf16: 1 + 0.1 N(0, 1), the shape of a trained norm's gains."""
    g = _gen(device, seed, 1003, hidden)
    return (1.0 + 0.1 * torch.randn((hidden,), generator=g, device=device, dtype=torch.float32)).to(torch.bfloat16)


def force_routing(logits: torch.Tensor, experts_per_token) -> torch.Tensor:
    """Make ``experts_per_token[m]`` the unique largest logit of row m."""
    out = logits.clone()
    rowmax = logits.float().amax(dim=1)
    idx = torch.as_tensor(list(experts_per_token), device=logits.device, dtype=torch.long)
    rows = torch.arange(logits.shape[0], device=logits.device)
    out[rows, idx] = (rowmax + 1.0).to(torch.bfloat16)
    return out


def router_logits(seed: int, m: int, num_experts: int, device="cpu",
                  force: Optional[List[int]] = None) -> torch.Tensor:
    lg = bf16_normal(m, num_experts, _gen(device, seed, 1002, m), device)
    return force_routing(lg, force) if force is not None else lg


def distinct_targets(seed: int, d: int, num_experts: int, m: int) -> List[int]:
    """d distinct experts (seeded) and token m -> targets[m mod d]."""
    rng = np.random.Generator(np.random.PCG64(_seed(seed, 1003, d)))
    t = rng.choice(num_experts, size=d, replace=False)
    return [int(t[i % d]) for i in range(m)]


def zipf_targets(seed: int, m: int, num_experts: int, s: float = 1.2) -> List[int]:
    rng = np.random.Generator(np.random.PCG64(_seed(seed, 1004, m)))
    perm = rng.permutation(num_experts)
    p = np.arange(1, num_experts + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    rank = rng.choice(num_experts, size=m, p=p)
    return [int(perm[r]) for r in rank]


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (on the host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# Named configurations (sizes and seeds); see the module docstring for the recipe.
TINY = dict(M=4, hidden=256, inter=512, num_experts=4, seed=0)
DENSE = dict(hidden=HIDDEN, inter=INTER, num_experts=0, seed=0)  # M in 1, 2, 4, 8
ROUTED = dict(M=4, hidden=HIDDEN, inter=INTER, num_experts=EXPERTS, seed=0)  # d forced 1..4
ZIPF = dict(M=256, hidden=HIDDEN, inter=INTER, num_experts=EXPERTS, seed=0, zipf_s=1.2)
