"""MXFP8 scales in the MX matrix-core operand order (MHC_FLAG_MXFP8_MFMA_SCALES),
through the C ABI.

The bytes: bit-exact the oracle's layout (mxfp8_scales_mfma) of the oracle's
encoding of the GPU's own bf16 h, on both schedules, with the codes
unchanged.  The consumer: a GEMM on gfx950's v_mfma_scale_f32_16x16x128_f8f6f4
(tests/mx_consumer.hip) fed h_fp8 and these scale bytes reproduces
dequant(h) * dequant(B)^T computed on the CPU, and the linear bytes fed the
same way do not.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import manifold_constrained_hyper_mhc_amd as mhc
import oracle as O
from manifold_constrained_hyper_mhc_amd.synthetic import make_inputs, make_int8_y
from tests._compare import f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HELPER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmx_consumer.so")


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mhc.lib()


def coeffs_in(T):
    cf = torch.zeros((T, 24), dtype=torch.float32)
    cf[:, 4:8] = 0.7
    cf[:, 8:24] = torch.eye(4).reshape(16) * 0.9 + 0.025
    return cf


@pytest.mark.parametrize("T,C,sched", [(6, 7168, "staged"), (37, 3072, "staged"), (520, 7168, "persistent"),
                                       (300, 7168, "staged"), (900, 4096, "persistent"), (45, 16384, "staged")])
def test_mfma_scale_bytes(T, C, sched, monkeypatch):
    monkeypatch.setenv("MHC_SCHEDULE", sched)
    assert mhc.schedule(T, C) == sched
    d = make_inputs(T, C, seed=T, rows="decades", device=DEV)
    cf = coeffs_in(T).to(DEV)
    lin = mhc.post_pre_fused(d["x"], d["y"], cf, d["phi_next"], d["bias_next"], d["gamma_next"], mxfp8=True)
    mf = mhc.post_pre_fused(d["x"], d["y"], cf, d["phi_next"], d["bias_next"], d["gamma_next"], mxfp8="mfma")
    torch.cuda.synchronize()
    for k in ("x_out", "coeffs_next", "h", "h_fp8"):
        assert torch.equal(lin[k], mf[k]), k
    q, s = O.mxfp8(f64(lin["h"]))
    assert np.array_equal(lin["h_scale"].cpu().numpy(), s)
    assert np.array_equal(mf["h_fp8"].cpu().numpy(), q)
    assert np.array_equal(mf["h_scale"].cpu().numpy(), O.mxfp8_scales_mfma(s))


def test_mfma_scale_bytes_int8_and_static():
    # the int8-input fused pass and the static-scratch call take the flag too
    T, C = 77, 4096
    d = make_inputs(T, C, seed=3, rows="decades", device=DEV)
    yq = make_int8_y(T, C, seed=4, device=DEV)
    cf = coeffs_in(T).to(DEV)
    a = mhc.post_int8_pre_fused(d["x"], yq["y_q"], yq["y_scale"], cf, d["phi_next"], d["bias_next"],
                                d["gamma_next"], mxfp8="mfma")
    pk = mhc.pack_phi(d["phi_next"])
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    b = mhc.post_pre_fused_prepacked_static(d["x"], d["y"], cf, pk, d["bias_next"], d["gamma_next"], mxfp8="mfma",
                                            error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for out in (a, b):
        q, s = O.mxfp8(f64(out["h"]))
        assert np.array_equal(out["h_fp8"].cpu().numpy(), q)
        assert np.array_equal(out["h_scale"].cpu().numpy(), O.mxfp8_scales_mfma(s))


def dequant(codes, scale_lin):
    v = O.e4m3_decode(codes)
    e = scale_lin.astype(np.int64) - 127
    return (v.reshape(v.shape[0], -1, 32) * np.ldexp(1.0, e)[:, :, None]).reshape(v.shape)


def test_matrix_core_consumer():
    assert os.path.exists(HELPER), "tests/libmx_consumer.so is built by the package build"
    L = ctypes.CDLL(HELPER)
    L.mx_gemm.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2
    L.mx_gemm.restype = ctypes.c_int
    T, C, N = 40, 2048, 32
    d = make_inputs(T, C, seed=8, rows="decades", device=DEV)
    cf = coeffs_in(T).to(DEV)
    out = mhc.post_pre_fused(d["x"], d["y"], cf, d["phi_next"], d["bias_next"], d["gamma_next"], mxfp8="mfma")
    lin = mhc.post_pre_fused(d["x"], d["y"], cf, d["phi_next"], d["bias_next"], d["gamma_next"], mxfp8=True)
    torch.cuda.synchronize()
    M = (T + 15) // 16 * 16
    A = torch.zeros((M, C), dtype=torch.uint8, device=DEV)
    A[:T] = out["h_fp8"]
    rng = np.random.default_rng(9)
    Bc = rng.integers(0, 256, size=(N, C), dtype=np.uint8)
    Bc[(Bc & 0x7F) == 0x7F] = 0x38  # no NaN codes (0x38 = 1.0)
    Bs = rng.integers(120, 135, size=(N, C // 32), dtype=np.uint8)
    B = torch.from_numpy(Bc).to(DEV)
    Bsd = torch.from_numpy(Bs).to(DEV)
    stream = torch.cuda.current_stream().cuda_stream

    def gemm(scale_bytes):
        Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        assert L.mx_gemm(A.data_ptr(), scale_bytes.data_ptr(), B.data_ptr(), Bsd.data_ptr(), M, N, C,
                         Y.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        return f64(Y)[:T]

    s_lin = lin["h_scale"].cpu().numpy()
    Ad = dequant(out["h_fp8"].cpu().numpy(), s_lin)
    Bd = dequant(Bc, Bs)
    ref = Ad @ Bd.T
    # the instruction's own accumulation (measured within 3e-5 of
    # sum_k |a_k b_k|) is well inside this bound; a misplaced scale is off by
    # a factor of order one
    bound = np.abs(Ad) @ np.abs(Bd).T * 2.0 ** -12 + 1e-30
    Y = gemm(out["h_scale"])
    assert np.all(np.abs(Y - ref) <= bound), float(np.max(np.abs(Y - ref) / bound))
    # the linear bytes in the same place give other sums: the order matters
    wrong = torch.zeros_like(out["h_scale"])
    wrong[:s_lin.size] = lin["h_scale"].reshape(-1)
    Yw = gemm(wrong)
    assert not np.all(np.abs(Yw - ref) <= bound)
