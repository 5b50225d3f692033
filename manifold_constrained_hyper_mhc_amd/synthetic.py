"""Seeded synthetic inputs for the mHC hot path.

This module holds none of the method's arithmetic: it only draws random
tensors with the shapes and value distributions of the workloads and rounds
the streams to bf16.  Both the HIP library's tests/benchmark and the oracle's
tests take their inputs from here.

The pages' workloads are DeepSeek-V4/V4.1 decode and prefill with real
activations and weights ("[DSV4.1] Four BS=1 critical-path fixes for DSpark
decode", "Result"; "[SM80] Backport mHC fused post + int8 all-reduce",
"Test commands and results"); those are not available, and these draws
stand in for them.  Draw order inside one generator: x, y; phi, bias, gamma
(this layer); phi, bias, gamma (next layer); then the row modifiers.
"""

from __future__ import annotations

import dataclasses

import torch

from .params import Params  # noqa: F401  (re-exported for the tests)

N_ROUTES = 4
N_LOGITS = 24


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    C: int
    rows: str = "normal"   # "normal" | "outliers" | "decades"


# The five workload shapes: small oracle-sized case, decode, prefill with
# outlier tokens, MXFP8 over five magnitude decades, long prefill.
WORKLOADS = {
    "small": Workload("small", 16, 1024, "normal"),
    "decode": Workload("decode", 6, 7168, "normal"),
    "prefill": Workload("prefill", 8192, 7168, "outliers"),
    "mxfp8": Workload("mxfp8", 8192, 4096, "decades"),
    "long": Workload("long", 65536, 7168, "normal"),
}


def make_inputs(T: int, C: int, *, seed: int = 0, rows: str = "normal",
                device="cpu", phi_std: float = 0.02, bias_std: float = 0.1,
                gamma_std: float = 0.05, outlier_frac: float = 0.01,
                outlier_scale: float = 100.0) -> dict:
    """Draw one workload's tensors on ``device`` from ``torch.Generator(seed)``.

    x [T,4,C] and y [T,C] are N(0,1) rounded to bf16 (torch's cast rounds to
    nearest even).  phi [4C,24] ~ N(0, phi_std), bias [24] ~ N(0, bias_std),
    gamma [C] ~ 1 + N(0, gamma_std), all fp32, for this layer and the next.
    ``rows="outliers"`` multiplies a random 1% of rows of x and y (chosen
    without replacement) by 100 before rounding; ``rows="decades"`` multiplies
    every row by 10**U(-2, 3).
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    f32 = torch.float32
    x = torch.randn((T, N_ROUTES, C), generator=g, device=dev, dtype=f32)
    y = torch.randn((T, C), generator=g, device=dev, dtype=f32)
    out = {}
    for tag in ("", "_next"):
        out["phi" + tag] = torch.randn((N_ROUTES * C, N_LOGITS), generator=g, device=dev, dtype=f32) * phi_std
        out["bias" + tag] = torch.randn((N_LOGITS,), generator=g, device=dev, dtype=f32) * bias_std
        out["gamma" + tag] = 1.0 + torch.randn((C,), generator=g, device=dev, dtype=f32) * gamma_std
    row_scale = None
    if rows == "outliers":
        n_out = int(round(outlier_frac * T))
        idx = torch.randperm(T, generator=g, device=dev)[:n_out]
        row_scale = torch.ones((T,), device=dev, dtype=f32)
        row_scale[idx] = outlier_scale
        out["outlier_rows"] = torch.sort(idx).values
    elif rows == "decades":
        u = torch.rand((T,), generator=g, device=dev, dtype=f32)
        row_scale = torch.pow(torch.tensor(10.0, device=dev), u * 5.0 - 2.0)
    elif rows != "normal":
        raise ValueError(f"unknown row distribution {rows!r}")
    if row_scale is not None:
        x = x * row_scale[:, None, None]
        y = y * row_scale[:, None]
    out["x"] = x.to(torch.bfloat16)
    out["y"] = y.to(torch.bfloat16)
    del x, y
    return out


def make_int8_y(T: int, C: int, *, seed: int = 0, device="cpu", decades: tuple = (-3.0, 1.0)) -> dict:
    """An int8 sublayer output with per-token scales, drawn from
    ``torch.Generator(seed)``: y_q [T, C] int8 uniform over every code,
    [-128, 127], and y_scale [T] fp32 = 10**U(*decades) / 127 (full binary32
    mantissas, so the dequantised products round)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    y_q = torch.randint(-128, 128, (T, C), generator=g, device=dev, dtype=torch.int8)
    lo, hi = decades
    u = torch.rand((T,), generator=g, device=dev, dtype=torch.float64)
    y_scale = (torch.pow(10.0, lo + (hi - lo) * u) / 127.0).to(torch.float32)
    return {"y_q": y_q, "y_scale": y_scale}


def make_workload(name: str, *, seed: int = 0, device="cpu", T: int | None = None) -> dict:
    """Inputs of a named workload; ``T`` overrides the token count."""
    w = WORKLOADS[name]
    return make_inputs(w.T if T is None else T, w.C, seed=seed, rows=w.rows, device=device)
