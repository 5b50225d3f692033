"""The decode-latency mode: a fused call with the Sinkhorn deferred, then
mhc_sinkhorn on a side stream, through the C ABI.

h needs only the pre weights, so the deferred call's h is complete at its
end; the res entries it leaves hold exp(logits) (the oracle's coefficients
with 0 Sinkhorn iterations); the side-stream mhc_sinkhorn then makes the
pair bitwise equal to one undeferred call, and both match the oracle.
"""
import numpy as np
import pytest
import torch

import manifold_constrained_hyper_mhc_amd as mhc
import oracle as O
from manifold_constrained_hyper_mhc_amd.params import Params
from manifold_constrained_hyper_mhc_amd.synthetic import make_inputs
from tests._compare import assert_coeffs_close, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
P = Params()
KW = dict(hc_norm_eps=P.hc_norm_eps, hc_post_scale=P.hc_post_scale, sinkhorn_eps=P.sinkhorn_eps)


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mhc.lib()


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("T,C,sched", [(6, 7168, "staged"), (16, 4096, "staged"), (64, 7168, "staged"),
                                       (520, 7168, "persistent")])
def test_deferred_sinkhorn_on_a_side_stream(T, C, sched, mx, monkeypatch):
    monkeypatch.setenv("MHC_SCHEDULE", sched)
    assert mhc.schedule(T, C) == sched
    inp = make_inputs(T, C, seed=T, rows="outliers", device="cpu")
    cf_in = O.f32_round(O.coeffs(f64(inp["x"]), f64(inp["phi"]), f64(inp["bias"]), sinkhorn_iters=20, **KW))
    inp["coeffs"] = torch.from_numpy(cf_in.astype(np.float32))
    d = {k: v.to(DEV) for k, v in inp.items()}
    ref = mhc.post_pre_fused(d["x"], d["y"], d["coeffs"], d["phi_next"], d["bias_next"], d["gamma_next"], mxfp8=mx)
    out = mhc.post_pre_fused(d["x"], d["y"], d["coeffs"], d["phi_next"], d["bias_next"], d["gamma_next"], mxfp8=mx,
                             defer_sinkhorn=True, ws=mhc.workspace(T, C, DEV, fresh=True))
    done = torch.cuda.Event()
    done.record()
    torch.cuda.synchronize()
    # before the Sinkhorn: res holds exp(logits), the oracle's 0-iteration coefficients
    pending = out["coeffs_next"].clone()
    x_out = f64(out["x_out"])
    o0 = O.coeffs(x_out, f64(inp["phi_next"]), f64(inp["bias_next"]), sinkhorn_iters=0, **KW)
    assert_coeffs_close(f64(pending), o0, what="deferred coefficients")
    for k in ("x_out", "h", "h_fp8", "h_scale"):
        if ref.get(k) is not None:
            assert torch.equal(out[k], ref[k]), k
    # the side stream finishes res, ordered after the fused call by an event
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        side.wait_event(done)
        mhc.sinkhorn(out["coeffs_next"], stream=side)
    side.synchronize()
    assert torch.equal(out["coeffs_next"], ref["coeffs_next"])
    o20 = O.coeffs(x_out, f64(inp["phi_next"]), f64(inp["bias_next"]), sinkhorn_iters=20, **KW)
    assert_coeffs_close(f64(out["coeffs_next"]), o20)


@pytest.mark.parametrize("iters", [0, 1, 7, 20])
def test_sinkhorn_entry_point(iters):
    # mhc_sinkhorn alone on given exp(logits): against the oracle's iterations
    T = 70
    g = torch.Generator().manual_seed(iters)
    logits = torch.randn((T, 16), generator=g, dtype=torch.float64) * 2.0
    cf = torch.zeros((T, 24), dtype=torch.float32)
    cf[:, 0:8] = 0.25
    cf[:, 8:] = torch.exp(logits).float()
    d = cf.to(DEV)
    mhc.sinkhorn(d, Params(sinkhorn_iters=iters))
    torch.cuda.synchronize()
    ref = O.sinkhorn(f64(cf[:, 8:]).reshape(T, 4, 4), iters, P.sinkhorn_eps).reshape(T, 16)
    assert torch.equal(d[:, 0:8].cpu(), cf[:, 0:8])
    assert_coeffs_close(f64(d[:, 8:]), ref, what="res")
