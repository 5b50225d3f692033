"""The C ABI without a GPU: symbols, sizes and argument validation.

Every entry point validates its arguments before its first HIP call, so the
rejected calls below never touch a device.  The fake device addresses are
never dereferenced; these tests are skipped where a GPU is visible, so that
no call with a fake pointer can ever reach a launch.
"""
import ctypes
import os
import re

import pytest
import torch

import manifold_constrained_hyper_mhc_amd as mhc
from manifold_constrained_hyper_mhc_amd.binding import MhcParams

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")

OK, NULL, SHAPE, ALIGN, ALIAS, FLAGS, WORKSPACE, PARAM, HIP = range(9)

no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer validation tests run without a GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = mhc.lib()
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n


def test_schedule_query():
    """mhc_schedule validates like the other calls; without a usable device
    (or for a decode-sized T) it reports the staged kernel."""
    L = mhc.lib()
    out = ctypes.c_int(-7)
    assert L.mhc_schedule(16, 1000, ctypes.byref(out)) == 2 and out.value == -7  # MHC_ERR_SHAPE
    assert L.mhc_schedule(16, 1024, None) == 1  # MHC_ERR_NULL
    assert L.mhc_schedule(6, 7168, ctypes.byref(out)) == 0 and out.value == 0  # one tile: staged


def test_abi_version_and_strerror():
    L = mhc.lib()
    assert L.mhc_abi_version() == 6
    for code in range(11):
        assert L.mhc_strerror(code) != b"unknown status"
    assert L.mhc_strerror(99) == b"unknown status"


def test_sinkhorn_validation():
    L = mhc.lib()
    p = mhc.binding.MhcParams.of(P)
    assert L.mhc_sinkhorn(None, 0, ctypes.byref(p), None) == 0           # T = 0: no-op
    assert L.mhc_sinkhorn(None, 4, ctypes.byref(p), None) == 1           # MHC_ERR_NULL
    assert L.mhc_sinkhorn(fake(0, 4), 4, ctypes.byref(p), None) == 3     # MHC_ERR_ALIGN
    assert L.mhc_sinkhorn(fake(0), -1, ctypes.byref(p), None) == 2       # MHC_ERR_SHAPE
    bad = mhc.binding.MhcParams(1e-6, 1e-6, 2.0, 1e-6, -1)
    assert L.mhc_sinkhorn(fake(0), 4, ctypes.byref(bad), None) == 7      # MHC_ERR_PARAM
    assert L.mhc_workspace_bytes(16, 1024, 4) == L.mhc_workspace_bytes(16, 1024, 0) > 0  # flag accepted


def test_workspace_check_validation():
    # argument errors come back before any HIP call
    L = mhc.lib()
    assert L.mhc_workspace_check(None, None) == 6          # MHC_ERR_WORKSPACE
    assert L.mhc_workspace_check(fake(0, 16), None) == 6   # not 256-byte aligned


def test_sizes():
    L = mhc.lib()
    assert L.mhc_phi_packed_bytes(7168) == 4 * 7168 * 160
    assert L.mhc_phi_packed_bytes(1000) == 0          # not a multiple of 1024
    assert L.mhc_workspace_bytes(8192, 7168, 0) >= 4 * 7168 * 160
    assert L.mhc_workspace_bytes(8192, 7168, 2) == L.mhc_workspace_bytes(8192, 7168, 0)
    assert L.mhc_workspace_bytes(8192, 7168, 16) == 0  # unknown flag
    assert L.mhc_workspace_bytes(-1, 7168, 0) == 0
    w1, w2 = L.mhc_workspace_bytes(16, 1024, 0), L.mhc_workspace_bytes(17, 1024, 0)
    assert 0 < w1 <= w2
    assert L.mhc_workspace_bytes(0, 1024, 0) > 0
    assert L.mhc_workspace_bytes(1 << 20, 16384, 1) % 256 == 0 and L.mhc_workspace_bytes(1 << 20, 16384, 1) > 0
    # bounded: at most ~143 MiB for any accepted shape, and the size stops
    # growing with T beyond the staged launch budget
    for C in range(1024, 16385, 1024):
        assert L.mhc_workspace_bytes(1 << 20, C, 1) <= 144 << 20, C
        grow = L.mhc_workspace_bytes(1 << 20, C, 0) - L.mhc_workspace_bytes(1 << 16, C, 0)
        assert grow <= 4 * ((1 << 20) - (1 << 16)) + 256, C  # only the 4-byte list entries




# ---------------------------------------------------------------------------
# validation with fake device addresses (never dereferenced)
# ---------------------------------------------------------------------------
BASE = 0x7F0000000000
SPACING = 1 << 36


def fake(k, off=0):
    return ctypes.c_void_p(BASE + k * SPACING + off)


P = MhcParams(1e-6, 1e-6, 2.0, 1e-6, 20)


def post_call(L, T=16, C=1024, x=None, y=None, cf=None, out=None):
    return L.mhc_post(x or fake(0), y or fake(1), cf or fake(2), T, C, out or fake(3), None)


@no_gpu
def test_post_validation():
    L = mhc.lib()
    assert post_call(L, C=1000) == SHAPE
    assert post_call(L, C=0) == SHAPE
    assert post_call(L, T=-1) == SHAPE
    assert post_call(L, T=(1 << 20) + 1) == SHAPE
    assert post_call(L, C=16384 + 1024) == SHAPE
    assert L.mhc_post(None, fake(1), fake(2), 16, 1024, fake(3), None) == NULL
    assert L.mhc_post(fake(0), fake(1), fake(2), 16, 1024, None, None) == NULL
    assert post_call(L, y=fake(1, 8)) == ALIGN
    assert post_call(L, out=fake(0, 1024)) == ALIAS       # output inside x
    assert post_call(L, out=fake(1, 16)) == ALIAS         # output overlapping y
    # T == 0: nothing to do, pointers may be NULL
    assert L.mhc_post(None, None, None, 0, 1024, None, None) == OK


@no_gpu
def test_pre_validation():
    L = mhc.lib()
    bad = MhcParams(1e-6, float("nan"), 2.0, 1e-6, 20)
    assert L.mhc_pre(fake(0), fake(1), fake(2), 4, 1024, ctypes.byref(bad), fake(3), None) == PARAM
    neg = MhcParams(1e-6, -1.0, 2.0, 1e-6, 20)
    assert L.mhc_pre(fake(0), fake(1), fake(2), 4, 1024, ctypes.byref(neg), fake(3), None) == PARAM
    assert L.mhc_pre(fake(0), fake(1), fake(2), 4, 1024, None, fake(3), None) == NULL
    assert L.mhc_pre(fake(0), fake(1), fake(2), 4, 3000, ctypes.byref(P), fake(3), None) == SHAPE
    assert L.mhc_pre(fake(0), fake(1), fake(2), 4, 1024, ctypes.byref(P), fake(0, 4096), None) == ALIAS
    assert L.mhc_pre(fake(0), fake(1, 4), fake(2), 4, 1024, ctypes.byref(P), fake(3), None) == ALIGN
    assert L.mhc_pre(None, None, None, 0, 1024, ctypes.byref(P), None, None) == OK


@no_gpu
def test_pre_broadcast_validation():
    L = mhc.lib()
    ws_bytes = L.mhc_workspace_bytes(4, 1024, 0)

    def call(x0=None, T=4, C=1024, p=P, cf=None, h=None, ws=None, wsb=ws_bytes):
        return L.mhc_pre_broadcast(x0 or fake(0), T, C, fake(1), fake(2), fake(3),
                                   ctypes.byref(p) if p is not None else None, cf or fake(4), h or fake(5),
                                   ws or fake(6), wsb, None)
    assert call(p=None) == NULL
    assert call(C=3000) == SHAPE
    assert call(x0=fake(0, 8)) == ALIGN
    assert call(h=fake(0, 4096)) == ALIAS          # h inside x0 ([4][1024] bf16 = 8 KB)
    assert call(cf=fake(5, 16)) == ALIAS           # coeffs overlapping h
    assert call(wsb=16) == WORKSPACE
    bad = MhcParams(1e-6, 1e-6, 2.0, 1e-6, -1)
    assert call(p=bad) == PARAM
    assert L.mhc_pre_broadcast(None, 0, 1024, None, None, None, ctypes.byref(P), None, None, None, 0, None) == OK


@no_gpu
def test_post_int8_validation():
    L = mhc.lib()

    def call(T=16, C=1024, x=None, q=None, sc=None, cf=None, out=None):
        return L.mhc_post_int8(x or fake(0), q or fake(1), sc or fake(2), cf or fake(3), T, C, out or fake(4), None)
    assert call(C=1000) == SHAPE
    assert call(T=-1) == SHAPE
    assert L.mhc_post_int8(fake(0), None, fake(2), fake(3), 16, 1024, fake(4), None) == NULL
    assert L.mhc_post_int8(fake(0), fake(1), None, fake(3), 16, 1024, fake(4), None) == NULL
    assert call(sc=fake(2, 4)) == ALIGN
    assert call(q=fake(1, 8)) == ALIGN
    assert call(out=fake(1, 4096)) == ALIAS        # output overlapping the int8 codes
    assert call(out=fake(2, 0)) == ALIAS           # output overlapping the scales
    assert L.mhc_post_int8(None, None, None, None, 0, 1024, None, None) == OK


def fused_call(L, T=16, C=1024, flags=0, p=P, ws=None, ws_bytes=None, h=True, fp8=None, sc=None,
               x_out=None, cf_next=None, phi=None, gamma=None):
    if ws_bytes is None:
        ws_bytes = L.mhc_workspace_bytes(T, C, flags) if T >= 0 else 0
    return L.mhc_post_pre_fused(fake(0), fake(1), fake(2), phi or fake(3), fake(4), gamma or fake(5), T, C,
                                ctypes.byref(p) if p is not None else None, flags, x_out or fake(6),
                                cf_next or fake(7), fake(8) if h else None, fp8, sc, ws or fake(11),
                                ws_bytes, None)


@no_gpu
def test_fused_validation():
    L = mhc.lib()
    assert fused_call(L, C=1536) == SHAPE
    assert fused_call(L, flags=16) == FLAGS
    assert fused_call(L, flags=2 | 16) == FLAGS
    assert fused_call(L, flags=8) == FLAGS                          # matrix-core scale order without MXFP8
    assert fused_call(L, flags=2, fp8=fake(9)) == FLAGS             # fp8 output without the MXFP8 flag
    assert fused_call(L, fp8=fake(9)) == FLAGS                      # fp8 output without the flag
    assert fused_call(L, flags=1, fp8=fake(9)) == NULL              # flag without the scale output
    assert fused_call(L, h=False) == NULL                           # bf16 h required without the flag
    assert fused_call(L, p=None) == NULL
    assert fused_call(L, p=MhcParams(1e-6, 1e-6, float("inf"), 1e-6, 20)) == PARAM
    assert fused_call(L, p=MhcParams(1e-6, 1e-6, 2.0, 1e-6, -1)) == PARAM
    assert fused_call(L, p=MhcParams(1e-6, 1e-6, 2.0, 1e-6, 5000)) == PARAM
    assert fused_call(L, p=MhcParams(-1e-6, 1e-6, 2.0, 1e-6, 20)) == PARAM
    assert fused_call(L, ws_bytes=100) == WORKSPACE
    assert fused_call(L, ws=fake(11, 16)) == WORKSPACE             # not 256-byte aligned
    assert fused_call(L, x_out=fake(0, 2048)) == ALIAS
    assert fused_call(L, cf_next=fake(6, 32)) == ALIAS              # two outputs overlap
    assert fused_call(L, ws=fake(6, 0)) == ALIAS                    # workspace over an output
    assert fused_call(L, phi=fake(3, 4)) == ALIGN
    assert fused_call(L, T=0, h=False, flags=1) == OK


@no_gpu
def test_coeffs_validation():
    L = mhc.lib()
    ws_bytes = L.mhc_workspace_bytes(16, 1024, 0)

    def call(T=16, C=1024, x=None, phi=None, out=None, ws=None, wsb=ws_bytes, p=P):
        return L.mhc_coeffs(x or fake(0), T, C, phi or fake(1), fake(2), ctypes.byref(p), out or fake(3),
                            ws or fake(4), wsb, None)
    assert call(C=512) == SHAPE
    assert call(wsb=ws_bytes - 256) == WORKSPACE
    assert call(out=fake(0, 64)) == ALIAS
    assert call(x=fake(0, 2)) == ALIGN
    assert call(p=MhcParams(float("nan"), 1e-6, 2.0, 1e-6, 20)) == PARAM
    assert L.mhc_coeffs(fake(0), 16, 1024, None, fake(2), ctypes.byref(P), fake(3), fake(4), ws_bytes, None) == NULL
    assert call(T=0) == OK


@no_gpu
def test_pack_phi_validation():
    L = mhc.lib()
    assert L.mhc_pack_phi(None, 1024, fake(1), None) == NULL
    assert L.mhc_pack_phi(fake(0), 1000, fake(1), None) == SHAPE
    assert L.mhc_pack_phi(fake(0), 1024, fake(1, 16), None) == ALIGN
    assert L.mhc_pack_phi(fake(0), 1024, fake(0, 256), None) == ALIAS


@no_gpu
def test_hip_failure_is_an_error_code_without_a_gpu():
    # a valid call reaches the HIP runtime, which has no device here
    L = mhc.lib()
    assert L.mhc_workspace_init(fake(0), 4096, None) == HIP
    assert L.mhc_last_hip_error() != 0
    assert L.mhc_workspace_init(None, 4096, None) == WORKSPACE
    assert L.mhc_workspace_init(fake(0, 8), 4096, None) == WORKSPACE


def test_binding_rejects_bad_tensors_before_the_library():
    x = torch.zeros((2, 4, 1024), dtype=torch.float32)
    with pytest.raises((TypeError, ValueError)):
        mhc.post(x, torch.zeros((2, 1024), dtype=torch.bfloat16), torch.zeros((2, 24)))
    xb = torch.zeros((2, 4, 1024), dtype=torch.bfloat16)
    with pytest.raises(ValueError):      # CPU tensors are refused
        mhc.post(xb, torch.zeros((2, 1024), dtype=torch.bfloat16), torch.zeros((2, 24)))


@no_gpu
def test_static_scratch_plan_fits_every_shape():
    # The static entry point plans its staged launches for its 64 MiB array.
    # Every accepted shape gets past its scratch check (MHC_ERR_SCRATCH = 10)
    # to the next one, the error word's alignment (MHC_ERR_ALIGN = 3): a
    # misaligned error word ends the call there, before any HIP call, so the
    # tensors can be far-apart addresses that are never touched.
    L = mhc.lib()
    p = MhcParams(1e-6, 1e-6, 2.0, 1e-6, 20)

    def far(k, off=0):  # 1 TiB apart: the largest x (2^20 x 4 x 16384 bf16) is 128 GiB
        return ctypes.c_void_p(0x100000000000 + (k << 40) + off)

    for C in range(1024, 16385, 1024):
        for T in (1 << 20, 100000, 8192, 6):
            rc = L.mhc_post_pre_fused_prepacked_static(
                far(0), far(1), far(2), far(3), far(4), far(5), T, C, ctypes.byref(p), 1,
                far(6), far(7), far(8), far(9), far(10), far(11, 1), None)
            assert rc == ALIGN, (T, C, rc)


def test_output_placement():
    # the outputs the binding allocates start PLACE_OFFSET bytes past their
    # reference modulo 1 KiB, whatever the reference's own alignment
    from manifold_constrained_hyper_mhc_amd import binding
    assert binding.PLACE_OFFSET % 256 == 0 and 0 < binding.PLACE_OFFSET < 1024
    big = torch.empty(64 * 4 * 1024 + 2048, dtype=torch.bfloat16)
    for skip in (0, 128, 256, 384):
        ref = big[skip: skip + 64 * 4 * 1024].view(64, 4, 1024)
        for shape, dtype in (((64, 4, 1024), torch.bfloat16), ((64, 1024), torch.bfloat16)):
            t = binding._placed_empty(shape, dtype, torch.device("cpu"), ref)
            assert tuple(t.shape) == shape and t.is_contiguous()
            assert (t.data_ptr() - ref.data_ptr()) % 1024 == binding.PLACE_OFFSET
