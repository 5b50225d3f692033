"""Inputs whose next-layer pre combination cancels (test helper, no method
arithmetic).

The fused pass takes the RMSNorm of g = sum_i pre_i x'_i from the route
Gram matrix; these inputs make g a small remainder of large route terms.
The incoming coefficients are the identity post (res = I, post = 0), so
x' = x bit for bit, and x is built with x1 ~ -x0 and x3 ~ -x2.  The next
layer's pre weights are fixed through its bias: the pre block (columns 0..3)
of phi_next is zero and bias_next[0:4] = (b, b, b', b'), so pre'_0 = pre'_1
and pre'_2 = pre'_3.  Row kinds, by t % 6:

  0  exact:        x1 = -x0, x3 = -x2 (g = 0; the plain definition gives h = 0)
  1  near:         x1 = -x0 and x3 = -x2 with 16 elements each moved by
                   1 or 2 bf16 steps
  2  near x100:    kind 1 on a row scaled by 100
  3  partial:      x1 = bf16(-x0 + 0.1 n), x3 = bf16(-x2 + 0.1 n')
  4  moderate:     x1 = bf16(-x0 + 0.5 n), x3 = bf16(-x2 + 0.5 n') (well
                   above the kernels' recomputation threshold)
  5  independent:  the drawn routes unchanged
"""
from __future__ import annotations

import torch

from manifold_constrained_hyper_mhc_amd.synthetic import make_inputs

KINDS = 6
BIAS_PRE = (0.3, 0.3, -0.2, -0.2)


def _bf16(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


def _nudge(neg: torch.Tensor, gen: torch.Generator, k: int = 16) -> torch.Tensor:
    """Move k random elements of a bf16 row by 1 or 2 steps of its magnitude."""
    bits = neg.view(torch.int16).clone()
    C = bits.numel()
    idx = torch.randperm(C, generator=gen)[:k]
    d = torch.randint(1, 3, (k,), generator=gen, dtype=torch.int16)
    sgn = torch.where(torch.rand(k, generator=gen) < 0.5, -1, 1).to(torch.int16)
    bits[idx] = bits[idx] + d * sgn
    return bits.view(torch.bfloat16)


def cancel_inputs(T: int, C: int, seed: int = 0) -> dict:
    """CPU tensors of a fused call (see the module docstring); also returns
    ``kind`` [T] (the row kind of every token)."""
    inp = make_inputs(T, C, seed=seed, rows="normal", device="cpu")
    gen = torch.Generator().manual_seed(seed + 7919)
    x = inp["x"].clone()
    kind = torch.arange(T) % KINDS
    for t in range(T):
        k = int(kind[t])
        if k == 5:
            continue
        x0 = x[t, 0].float()
        x2 = x[t, 2].float()
        if k == 2:
            x0, x2 = x0 * 100.0, x2 * 100.0
        x0b, x2b = _bf16(x0), _bf16(x2)
        if k in (0, 1, 2):
            x1b, x3b = -x0b, -x2b
            if k in (1, 2):
                x1b, x3b = _nudge(x1b, gen), _nudge(x3b, gen)
        else:
            a = 0.1 if k == 3 else 0.5
            x1b = _bf16(-x0b.float() + a * torch.randn(C, generator=gen))
            x3b = _bf16(-x2b.float() + a * torch.randn(C, generator=gen))
        x[t, 0], x[t, 1], x[t, 2], x[t, 3] = x0b, x1b, x2b, x3b
    inp["x"] = x
    cf = torch.zeros((T, 24), dtype=torch.float32)
    cf[:, 0:4] = 0.5
    cf[:, 8:24] = torch.eye(4).reshape(16)
    inp["coeffs"] = cf
    inp["phi_next"] = inp["phi_next"].clone()
    inp["phi_next"][:, 0:4] = 0.0
    inp["bias_next"] = inp["bias_next"].clone()
    inp["bias_next"][0:4] = torch.tensor(BIAS_PRE, dtype=torch.float32)
    inp["kind"] = kind
    return inp
