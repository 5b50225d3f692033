"""The oracle's MX matrix-core scale layout (mxfp8_scales_mfma), pinned by a
lane-by-lane reconstruction from the operand description of
v_mfma_scale_f32_16x16x128_f8f6f4 (lane l: row l % 16 of a 16-row block,
32 K-values of block l / 16 of a 128-wide K-tile kt, scale from byte kt % 4
of the dword a consumer loads for K-tiles 4 (kt // 4) .. + 3), written
independently of the oracle's reshape.
"""
import numpy as np

import oracle as O


def lane_centric(scale, T, C):
    rows = (T + 15) // 16 * 16
    out = np.zeros(rows * C // 32, dtype=np.uint8)
    for rb in range(rows // 16):
        for kt in range(C // 128):
            for lane in range(64):
                token = 16 * rb + lane % 16
                channel0 = 128 * kt + 32 * (lane // 16)      # the 32 channels this lane holds
                dword = (rb * (C // 512) + kt // 4) * 64 + lane
                byte = 4 * dword + kt % 4                     # op_sel kt % 4
                out[byte] = scale[token, channel0 // 32] if token < T else 0
    return out


def test_layout_matches_the_operand_description():
    rng = np.random.default_rng(0)
    for T, C in [(1, 512), (16, 1024), (37, 3072), (70, 2048)]:
        s = rng.integers(0, 255, size=(T, C // 32), dtype=np.uint8)
        assert np.array_equal(O.mxfp8_scales_mfma(s), lane_centric(s, T, C)), (T, C)


def test_layout_is_a_permutation_with_zero_padding():
    rng = np.random.default_rng(1)
    T, C = 37, 4096
    s = rng.integers(1, 255, size=(T, C // 32), dtype=np.uint8)
    m = O.mxfp8_scales_mfma(s)
    assert m.size == 48 * C // 32
    assert np.array_equal(np.sort(m[m != 0]), np.sort(s.reshape(-1)))
    assert np.count_nonzero(m == 0) == (48 - T) * C // 32
