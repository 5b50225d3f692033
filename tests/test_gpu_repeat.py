"""Repeated full-size calls, bitwise: the exchange between workgroups under load.

The persistent kernel's workgroups exchange partial sums and q words through
memory: binary32 partial values released by tagged flags, tagged q words,
ring slots reused every few tiles, release words of the coefficients ring.
The sums are taken in a fixed order, so every call on the same inputs must
give the same bits; a value read before its release (a stale ring slot, a
flag seen before its values) would show up as a difference.  Each case runs
the benchmark's shapes many times in a row on one workspace, alternating with
a call of another shape (which leaves other tags and ring contents behind),
and compares every output with the first call's, bit for bit; the workspace
error word must stay clear.
"""
import numpy as np
import pytest
import torch

import manifold_constrained_hyper_mhc_amd as mhc
from manifold_constrained_hyper_mhc_amd.synthetic import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPS = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mhc.lib()


def _coeffs_in(T, C, seed):
    # incoming coefficients: a valid mix (rows of a doubly stochastic matrix
    # from the library's own coefficients of a stream; values only matter as
    # inputs here)
    g = torch.Generator(device="cpu").manual_seed(seed)
    cf = torch.rand((T, 24), generator=g, dtype=torch.float32)
    cf[:, 8:24] = cf[:, 8:24] / cf[:, 8:24].reshape(T, 4, 4).sum(-1, keepdim=True).repeat(1, 1, 4).reshape(T, 16)
    return cf.to(DEV)


def _assert_same(first, out, what, rep):
    for k, v in first.items():
        if v is None:
            continue
        assert torch.equal(v, out[k]), f"{what}: output {k} of call {rep} differs from the first call's"


@pytest.mark.parametrize("workload", ["prefill", "mxfp8"])
def test_fused_repeated_bitwise(workload):
    w = WORKLOADS[workload]
    mx = workload == "mxfp8"
    assert mhc.schedule(w.T, w.C) == "persistent"
    d = make_inputs(w.T, w.C, seed=5, rows=w.rows, device=DEV)
    cf = _coeffs_in(w.T, w.C, seed=6)
    small = make_inputs(300, w.C, seed=7, device=DEV)
    cf_small = _coeffs_in(300, w.C, seed=8)
    ws = mhc.workspace(w.T, w.C, DEV, fresh=True)
    pk = mhc.pack_phi(d["phi_next"])
    first = None
    for rep in range(REPS):
        out = mhc.post_pre_fused_prepacked(d["x"], d["y"], cf, pk, d["bias_next"], d["gamma_next"], mxfp8=mx, ws=ws)
        if rep % 4 == 3:
            # another shape in between: other tags and ring contents left behind
            mhc.post_pre_fused(small["x"], small["y"], cf_small, small["phi_next"], small["bias_next"],
                               small["gamma_next"], ws=ws)
        torch.cuda.synchronize()
        out = {k: (v.clone() if v is not None else None) for k, v in out.items()}
        if first is None:
            first = out
        else:
            _assert_same(first, out, workload, rep)
    mhc.check(ws)


def test_coefficients_repeated_bitwise():
    w = WORKLOADS["prefill"]
    d = make_inputs(w.T, w.C, seed=9, rows=w.rows, device=DEV)
    ws = mhc.workspace(w.T, w.C, DEV, fresh=True)
    first = None
    for rep in range(REPS):
        cf = mhc.coeffs(d["x"], d["phi"], d["bias"], ws=ws)
        torch.cuda.synchronize()
        if first is None:
            first = {"coeffs": cf.clone()}
        else:
            _assert_same(first, {"coeffs": cf}, "coefficients", rep)
    mhc.check(ws)


def test_broadcast_pre_repeated_bitwise():
    w = WORKLOADS["prefill"]
    d = make_inputs(w.T, w.C, seed=10, device=DEV)
    x0 = d["x"][:, 0, :].contiguous()
    ws = mhc.workspace(w.T, w.C, DEV, fresh=True)
    first = None
    for rep in range(REPS):
        cf, h = mhc.pre_broadcast(x0, d["phi"], d["bias"], d["gamma"], ws=ws)
        torch.cuda.synchronize()
        if first is None:
            first = {"coeffs": cf.clone(), "h": h.clone()}
        else:
            _assert_same(first, {"coeffs": cf, "h": h}, "broadcast pre", rep)
    mhc.check(ws)


@pytest.mark.parametrize("mx", [False, True])
def test_decode_repeated_bitwise(mx):
    # one-tile launches take their jobs by ticket, with the launch epoch in
    # the ticket's word; the last ticket advances the epoch and clears the
    # count.  Many calls in a row on one workspace, alternating with a
    # 32-token-tile call (staged) and a persistent one (which advance the
    # same epoch by other paths), and with coefficients-only one-tile calls
    # (fewer jobs per launch): every decode output bitwise equal to the
    # first call's, the error word clear.
    w = WORKLOADS["decode"]
    d = make_inputs(w.T, w.C, seed=11, device=DEV)
    cf = _coeffs_in(w.T, w.C, seed=12)
    mid = make_inputs(40, w.C, seed=13, device=DEV)
    cf_mid = _coeffs_in(40, w.C, seed=14)
    big = make_inputs(520, w.C, seed=15, device=DEV)
    cf_big = _coeffs_in(520, w.C, seed=16)
    ws = mhc.workspace(520, w.C, DEV, fresh=True)
    first = None
    for rep in range(REPS * 2):
        out = mhc.post_pre_fused(d["x"], d["y"], cf, d["phi_next"], d["bias_next"], d["gamma_next"], mxfp8=mx, ws=ws)
        cfo = mhc.coeffs(d["x"], d["phi"], d["bias"], ws=ws)
        if rep % 3 == 1:
            mhc.post_pre_fused(mid["x"], mid["y"], cf_mid, mid["phi_next"], mid["bias_next"], mid["gamma_next"], ws=ws)
        if rep % 5 == 2:
            mhc.post_pre_fused(big["x"], big["y"], cf_big, big["phi_next"], big["bias_next"], big["gamma_next"], ws=ws)
        torch.cuda.synchronize()
        out = {k: (v.clone() if v is not None else None) for k, v in out.items()}
        out["coeffs"] = cfo.clone()
        if first is None:
            first = out
        else:
            _assert_same(first, out, "decode", rep)
    mhc.check(ws)
    # the ticket count is back to zero after every one-tile launch
    head = ws[:16].cpu().numpy()
    assert int(head[8:12].view(np.uint32)[0]) == 0


def test_output_placement_does_not_change_results():
    # the binding places x_out and h off the alignment of x and y (a matter of
    # speed only): outputs in plain torch.empty buffers are bitwise the same
    w = WORKLOADS["prefill"]
    d = make_inputs(w.T, w.C, seed=17, rows=w.rows, device=DEV)
    cf = _coeffs_in(w.T, w.C, seed=18)
    placed = mhc.post_pre_fused(d["x"], d["y"], cf, d["phi_next"], d["bias_next"], d["gamma_next"])
    plain = {"x_out": torch.empty_like(d["x"]), "h": torch.empty_like(d["y"]),
             "coeffs_next": torch.empty((w.T, 24), dtype=torch.float32, device=DEV)}
    aligned = mhc.post_pre_fused(d["x"], d["y"], cf, d["phi_next"], d["bias_next"], d["gamma_next"], outs=plain)
    torch.cuda.synchronize()
    assert (placed["x_out"].data_ptr() - d["x"].data_ptr()) % 1024 == mhc.binding.PLACE_OFFSET
    for k in ("x_out", "h", "coeffs_next"):
        assert torch.equal(placed[k], aligned[k]), k
