"""HIP-graph capture of the library's calls.

The C ABI promises no allocation, synchronisation or per-stream state on the
call path, so a caller may capture its calls in a graph from the first call
on (the capture contract the [DSv4.1] Mega-mHC review asks of a fused mHC
kernel).  Each case captures one decode- or prefill-shaped step (projection
repack, fused post -> pre, the coefficients of the fused output) and replays
it several times, with the program's own eager work (clearing every output)
and a device synchronisation between the replays: every replay must
reproduce the eager step bit for bit, and the workspace error word must stay
0.  This is a consistency test of the HIP path with itself; parity with the
oracle is tested elsewhere.
"""
import pytest
import torch

import manifold_constrained_hyper_mhc_amd as mhc
from manifold_constrained_hyper_mhc_amd import binding
from manifold_constrained_hyper_mhc_amd.synthetic import make_inputs, make_int8_y

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (T, C, schedule, MXFP8): a decode step (one 16-token tile), prefill-shaped
# launches of both schedules with ragged last tiles, and the MXFP8 epilogue
CASES = [(6, 7168, "staged", False), (520, 7168, "persistent", False), (900, 4096, "persistent", True),
         (300, 7168, "staged", True)]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mhc.lib()


@pytest.mark.parametrize("T,C,sched,mx", CASES)
def test_graph_replays_match_eager(T, C, sched, mx, monkeypatch):
    monkeypatch.setenv("MHC_SCHEDULE", sched)
    d = make_inputs(T, C, seed=21, rows="outliers", device=DEV)
    ws = mhc.workspace(T, C, DEV, fresh=True)
    # incoming coefficients of the step: any valid rows will do
    cin = mhc.coeffs(d["x"], d["phi"], d["bias"], ws=ws)
    L = mhc.lib()
    packed = torch.empty(int(L.mhc_phi_packed_bytes(C)), dtype=torch.uint8, device=DEV)
    outs = {"x_out": torch.empty((T, 4, C), dtype=torch.bfloat16, device=DEV),
            "coeffs_next": torch.empty((T, 24), dtype=torch.float32, device=DEV),
            "h": torch.empty((T, C), dtype=torch.bfloat16, device=DEV)}
    if mx:
        outs["h_fp8"] = torch.empty((T, C), dtype=torch.uint8, device=DEV)
        outs["h_scale"] = torch.empty((T, C // 32), dtype=torch.uint8, device=DEV)
    cf2 = torch.empty((T, 24), dtype=torch.float32, device=DEV)

    def step():
        dev = torch.device(DEV)
        rc = L.mhc_pack_phi(binding._ptr(d["phi_next"]), C, binding._ptr(packed), binding._stream(dev))
        assert rc == 0, mhc.MhcError(rc, "mhc_pack_phi")
        mhc.post_pre_fused_prepacked(d["x"], d["y"], cin, packed, d["bias_next"], d["gamma_next"], mxfp8=mx,
                                     ws=ws, outs=outs)
        mhc.coeffs_prepacked(outs["x_out"], packed, d["bias_next"], out=cf2, ws=ws)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    ref["cf2"] = cf2.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for v in list(outs.values()) + [cf2]:
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = dict(outs, cf2=cf2)
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k} differs from the eager step"
    assert mhc.workspace_error(ws) == 0, "a bounded wait expired"


def test_graph_replays_int8_fused_and_broadcast_pre():
    # the int8-input fused pass and the broadcast first-layer pre, captured
    # together, replay bit for bit
    T, C = 520, 7168
    d = make_inputs(T, C, seed=23, rows="outliers", device=DEV)
    yq = make_int8_y(T, C, seed=4, device=DEV)
    ws = mhc.workspace(T, C, DEV, fresh=True)
    ws2 = mhc.workspace(T, C, DEV, fresh=True)
    cin = mhc.coeffs(d["x"], d["phi"], d["bias"], ws=ws)
    packed = mhc.pack_phi(d["phi_next"])
    x0 = d["x"][:, 0, :].contiguous()
    outs = {"x_out": torch.empty((T, 4, C), dtype=torch.bfloat16, device=DEV),
            "coeffs_next": torch.empty((T, 24), dtype=torch.float32, device=DEV),
            "h": torch.empty((T, C), dtype=torch.bfloat16, device=DEV)}
    cf0 = torch.empty((T, 24), dtype=torch.float32, device=DEV)
    h0 = torch.empty((T, C), dtype=torch.bfloat16, device=DEV)

    def step():
        mhc.post_int8_pre_fused(d["x"], yq["y_q"], yq["y_scale"], cin, None, d["bias_next"], d["gamma_next"],
                                ws=ws, outs=outs, phi_packed=packed)
        mhc.pre_broadcast(x0, None, d["bias_next"], d["gamma_next"], ws=ws2, coeffs_out=cf0, h_out=h0,
                          phi_packed=packed)

    step()
    torch.cuda.synchronize()
    got = dict(outs, cf0=cf0, h0=h0)
    ref = {k: v.clone() for k, v in got.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in got.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k} differs from the eager step"
    assert mhc.workspace_error(ws) == 0 and mhc.workspace_error(ws2) == 0, "a bounded wait expired"
