"""Fused pre on cancelling routes, through the C ABI, against the oracle.

The fused pass forms sum_c g^2 of the pre as pre^T G pre from the route Gram
matrix; on the inputs of tests/_cancel.py (x1 ~ -x0, x3 ~ -x2, equal pre
weights per pair, unit and x100 rows, one exactly cancelling kind) that
quadratic form is a small difference of large fp32 terms.  The library lists
such tokens and recomputes their h directly; here every output is compared
with the oracle on every element, on both schedules, with and without the
MXFP8 epilogue, and the MXFP8 bytes with the oracle's encoding of the GPU's
own bf16 h on every block.
"""
import numpy as np
import pytest
import torch

import manifold_constrained_hyper_mhc_amd as mhc
import oracle as O
from manifold_constrained_hyper_mhc_amd.params import Params
from tests._cancel import cancel_inputs
from tests._compare import assert_bf16_close, assert_coeffs_close, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
P = Params()
KW = dict(hc_norm_eps=P.hc_norm_eps, hc_post_scale=P.hc_post_scale, sinkhorn_eps=P.sinkhorn_eps,
          sinkhorn_iters=P.sinkhorn_iters, rmsnorm_eps=P.rmsnorm_eps)


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mhc.lib()


def fix_count(ws):
    """Tokens the last fused call listed for the direct recomputation: the
    workspace's tagged count word (offset 16) when its tag is the launch epoch
    (offset 12)."""
    head = ws[:24].cpu().numpy()
    epoch = int(head[12:16].view(np.uint32)[0])
    word = int(head[16:24].view(np.uint64)[0])
    return (word & 0xFFFFFFFF) if (word >> 32) == epoch else 0


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("T,C,sched", [(37, 3072, "staged"), (520, 7168, "persistent"), (300, 7168, "staged"),
                                       (900, 4096, "persistent"), (1800, 2048, "persistent"),
                                       (12, 7168, "staged"), (16, 1024, "staged"), (30, 4096, "staged")])
def test_fused_on_cancelling_routes(T, C, sched, mx, monkeypatch):
    monkeypatch.setenv("MHC_SCHEDULE", sched)
    assert mhc.schedule(T, C) == sched
    inp = cancel_inputs(T, C, seed=T + C)
    d = {k: v.to(DEV) for k, v in inp.items()}
    ws = mhc.workspace(T, C, DEV, fresh=True)
    out = mhc.post_pre_fused(d["x"], d["y"], d["coeffs"], d["phi_next"], d["bias_next"], d["gamma_next"],
                             mxfp8=mx, ws=ws)
    torch.cuda.synchronize()
    mhc.check(ws)
    n_fix = fix_count(ws)
    ref = O.post_pre_fused(f64(inp["x"]), f64(inp["y"]), f64(inp["coeffs"]), f64(inp["phi_next"]),
                           f64(inp["bias_next"]), f64(inp["gamma_next"]), with_mxfp8=mx, **KW)
    assert torch.equal(out["x_out"], d["x"])
    assert_coeffs_close(f64(out["coeffs_next"]), ref["coeffs_next"], what="coeffs_next")
    h = f64(out["h"])
    assert np.all(np.isfinite(h))
    assert_bf16_close(h, ref["h"], what="h")
    kind = inp["kind"].numpy()
    assert not h[kind == 0].any(), "an exactly cancelling row must give h = 0"
    # the recomputation ran for the cancelling kinds (0-3) and not for the
    # moderate and independent ones
    assert int((kind <= 3).sum()) <= n_fix <= int((kind <= 4).sum()), n_fix
    if mx:
        q, s = O.mxfp8(h)
        assert np.array_equal(out["h_fp8"].cpu().numpy(), q)
        assert np.array_equal(out["h_scale"].cpu().numpy(), s)


def test_standalone_pre_on_cancelling_routes():
    T, C = 60, 7168
    inp = cancel_inputs(T, C, seed=4)
    cf = torch.zeros((T, 24), dtype=torch.float32)
    sig = torch.sigmoid(torch.tensor([0.3, 0.3, -0.2, -0.2], dtype=torch.float64)).float()
    cf[:, 0:4] = sig
    h = mhc.pre(inp["x"].to(DEV), cf.to(DEV), inp["gamma"].to(DEV))
    torch.cuda.synchronize()
    ref = O.pre(f64(inp["x"]), f64(cf)[:, 0:4], f64(inp["gamma"]), rmsnorm_eps=P.rmsnorm_eps)
    hg = f64(h)
    assert np.all(np.isfinite(hg))
    assert_bf16_close(hg, ref, what="h")
    assert not hg[inp["kind"].numpy() == 0].any()


def test_no_recomputation_on_the_benchmark_distributions():
    # independent N(0,1) routes with 1% outlier rows: nothing is listed, so the
    # recomputation kernel only reads the count
    from manifold_constrained_hyper_mhc_amd.synthetic import make_inputs
    T, C = 520, 7168
    inp = make_inputs(T, C, seed=2, rows="outliers", device=DEV)
    cf = torch.zeros((T, 24), dtype=torch.float32, device=DEV)
    cf[:, 0:8] = 0.5
    cf[:, 8:24] = torch.eye(4, device=DEV).reshape(16)  # x' = x + y / 2: independent routes
    ws = mhc.workspace(T, C, DEV, fresh=True)
    mhc.post_pre_fused(inp["x"], inp["y"], cf, inp["phi_next"], inp["bias_next"], inp["gamma_next"], ws=ws)
    torch.cuda.synchronize()
    assert fix_count(ws) == 0
