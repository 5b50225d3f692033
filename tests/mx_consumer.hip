// Test helper (not part of libmhc): a consumer of MXFP8 h in the MX
// matrix-core scale order, computing Y = dequant(A) * dequant(B)^T with the
// gfx950 instruction v_mfma_scale_f32_16x16x128_f8f6f4.  It shows that the
// scale bytes the library writes with MHC_FLAG_MXFP8_MFMA_SCALES are the
// operands that instruction takes.  Operand layout of the instruction (as
// measured on MI355X with a probe that placed data in one lane group and
// one half of its bytes at a time): lane l = 16 g + r holds row r; its
// bytes 0..15 are K = 16 g + 0..15 and its bytes 16..31 are
// K = 64 + 16 g + 0..15 of the 128-wide K-tile; its scale byte (op_sel
// kt % 4 of the dword at lane l of [row block][K-tile / 4][64][4]) applies
// to the 32-wide K-block g, K = 32 g .. 32 g + 31, of row r.
//
//   A: [M][K] e4m3 codes (h_fp8), a_scale: the matrix-core order
//   B: [N][K] e4m3 codes, b_scale: [N][K/32] linear bytes
//   Y: [M][N] fp32; one wave per 16 x 16 tile; M, N multiples of 16 and
//   K a multiple of 512 (the caller checks)
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int SEL>
__device__ __forceinline__ f32x4_t mx_step(i32x8_t a, i32x8_t b, f32x4_t c, int sa, int sb) {
  // cbsz = blgp = 0: both operands OCP e4m3
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, SEL, sa, 0, sb);
}

__global__ __launch_bounds__(64) void k_mx_gemm(const uint8_t* __restrict__ A, const uint32_t* __restrict__ a_scale,
                                                const uint8_t* __restrict__ B, const uint8_t* __restrict__ b_scale,
                                                int M, int N, int K, float* __restrict__ Y) {
  const int l = threadIdx.x;
  const int mt = blockIdx.x, nt = blockIdx.y;
  const int r = l & 15, kb = l >> 4;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int kt = 0; kt < K / 128; ++kt) {
    // bytes 0..15: K = 16 kb + 0..15; bytes 16..31: K = 64 + 16 kb + 0..15
    const uint8_t* ap = A + (int64_t)(16 * mt + r) * K + 128 * kt + 16 * kb;
    const uint8_t* bp = B + (int64_t)(16 * nt + r) * K + 128 * kt + 16 * kb;
    const i32x4_t a0 = *reinterpret_cast<const i32x4_t*>(ap), a1 = *reinterpret_cast<const i32x4_t*>(ap + 64);
    const i32x4_t b0 = *reinterpret_cast<const i32x4_t*>(bp), b1 = *reinterpret_cast<const i32x4_t*>(bp + 64);
    const i32x8_t av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const i32x8_t bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    const int sa = (int)a_scale[((int64_t)mt * (K / 512) + kt / 4) * 64 + l];
    const int sb = (int)b_scale[(int64_t)(16 * nt + r) * (K / 32) + 4 * kt + kb];
    switch (kt & 3) {
      case 0: acc = mx_step<0>(av, bv, acc, sa, sb); break;
      case 1: acc = mx_step<1>(av, bv, acc, sa, sb); break;
      case 2: acc = mx_step<2>(av, bv, acc, sa, sb); break;
      default: acc = mx_step<3>(av, bv, acc, sa, sb); break;
    }
  }
  // output: lane l holds column l % 16 of rows 4 (l / 16) + e
#pragma unroll
  for (int e = 0; e < 4; ++e) Y[(int64_t)(16 * mt + 4 * kb + e) * N + 16 * nt + r] = acc[e];
}

extern "C" int mx_gemm(const void* A, const void* a_scale, const void* B, const void* b_scale, int M, int N, int K,
                       float* Y, void* stream) {
  if (M <= 0 || N <= 0 || K <= 0 || M % 16 || N % 16 || K % 512) return 1;
  k_mx_gemm<<<dim3(M / 16, N / 16), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(A), static_cast<const uint32_t*>(a_scale), static_cast<const uint8_t*>(B),
      static_cast<const uint8_t*>(b_scale), M, N, K, Y);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
