"""The fused pass on the library's static scratch (the entry point that
allocates nothing), through the C ABI, against the same pass with a
caller-owned workspace: bitwise the same outputs, on two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents),
and the oracle on the small case.  Also that every accepted shape fits the
scratch (the workspace is bounded), a prefill-sized call, and the ABI
constants.
"""
import ctypes

import numpy as np
import pytest
import torch

import manifold_constrained_hyper_mhc_amd as mhc
import oracle as O
from manifold_constrained_hyper_mhc_amd.params import Params
from manifold_constrained_hyper_mhc_amd.synthetic import make_inputs
from tests._compare import assert_bf16_close, assert_coeffs_close, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
P = Params()
KW = dict(hc_norm_eps=P.hc_norm_eps, hc_post_scale=P.hc_post_scale, sinkhorn_eps=P.sinkhorn_eps,
          sinkhorn_iters=P.sinkhorn_iters)


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mhc.lib()


def inputs(T, C, seed):
    inp = make_inputs(T, C, seed=seed, rows="outliers", device="cpu")
    cf = O.coeffs(f64(inp["x"]), f64(inp["phi"]), f64(inp["bias"]), **KW)
    inp["coeffs"] = torch.from_numpy(O.f32_round(cf).astype(np.float32))
    return inp


def test_static_scratch_matches_workspace_call():
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    # the second call is smaller: it meets the first call's words in the scratch
    for T, C, mx in [(520, 7168, True), (37, 3072, False)]:
        inp = inputs(T, C, seed=T)
        d = {k: v.to(DEV) for k, v in inp.items()}
        pk = mhc.pack_phi(d["phi_next"])
        ref = mhc.post_pre_fused_prepacked(d["x"], d["y"], d["coeffs"], pk, d["bias_next"], d["gamma_next"],
                                           mxfp8=mx, ws=mhc.workspace(T, C, DEV, fresh=True))
        out = mhc.post_pre_fused_prepacked_static(d["x"], d["y"], d["coeffs"], pk, d["bias_next"],
                                                  d["gamma_next"], mxfp8=mx, error_word=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, "a bounded wait expired"
        for k, v in ref.items():
            if v is not None:
                assert torch.equal(out[k], v), k
    # the small case against the oracle
    r = O.post_pre_fused(f64(inp["x"]), f64(inp["y"]), f64(inp["coeffs"]), f64(inp["phi_next"]),
                         f64(inp["bias_next"]), f64(inp["gamma_next"]), rmsnorm_eps=P.rmsnorm_eps, **KW)
    assert np.array_equal(f64(out["x_out"]), r["x_out"])
    assert_coeffs_close(f64(out["coeffs_next"]), r["coeffs_next"])
    assert_bf16_close(f64(out["h"]), r["h"])


def test_static_scratch_covers_every_shape():
    L = mhc.lib()
    assert L.mhc_abi_version() >= 4
    assert L.mhc_strerror(mhc.ERR_SCRATCH) != b"unknown status"
    # (that every accepted shape's plan fits the static scratch is checked
    # without a GPU in test_boundary.py)
    # a prefill-sized call on the scratch, bitwise the workspace call
    T, C = 8192, 4096
    d = make_inputs(T, C, seed=1, rows="decades", device=DEV)
    cf = torch.zeros((T, 24), dtype=torch.float32, device=DEV)
    cf[:, 0:8] = 0.5
    cf[:, 8:24] = torch.eye(4, device=DEV).reshape(16)
    pk = mhc.pack_phi(d["phi_next"])
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = mhc.post_pre_fused_prepacked_static(d["x"], d["y"], cf, pk, d["bias_next"], d["gamma_next"], mxfp8=True,
                                              error_word=err)
    ref = mhc.post_pre_fused_prepacked(d["x"], d["y"], cf, pk, d["bias_next"], d["gamma_next"], mxfp8=True,
                                       ws=mhc.workspace(T, C, DEV, fresh=True))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for k, v in ref.items():
        if v is not None:
            assert torch.equal(out[k], v), k
    # a NULL error word is refused before any HIP call
    p = mhc.binding.MhcParams.of(P)
    rc = L.mhc_post_pre_fused_prepacked_static(
        d["x"].data_ptr(), d["y"].data_ptr(), cf.data_ptr(), pk.data_ptr(), d["bias_next"].data_ptr(),
        d["gamma_next"].data_ptr(), 16, C, ctypes.byref(p), 0, out["x_out"].data_ptr(),
        out["coeffs_next"].data_ptr(), out["h"].data_ptr(), None, None, None, torch.cuda.current_stream().cuda_stream)
    assert rc == 1  # MHC_ERR_NULL
