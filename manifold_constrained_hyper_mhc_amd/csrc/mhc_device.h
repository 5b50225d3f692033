// Device helpers shared by the libmhc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mhc_internal.h"

namespace mhc {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  A uint32 holds two bf16 values, element 0 in the low half.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Round two floats to bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  bf16x2_t r = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// Unpack 8 bf16 (one 16-byte chunk) to floats.
__device__ __forceinline__ void unpack8(const u32x4_t v, float* f) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_lo(v[k]);
    f[2 * k + 1] = bf16_hi(v[k]);
  }
}

__device__ __forceinline__ u32x4_t pack8(const float* f) {
  u32x4_t v;
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = pack_bf16x2(f[2 * k], f[2 * k + 1]);
  return v;
}

// ---------------------------------------------------------------------------
// Memory: 16-byte loads and stores; streaming data uses non-temporal hints.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
// LAST_USE: a non-temporal load (the line is not read again); otherwise a
// plain load that leaves the line in the caches for a later reader.
template <bool LAST_USE>
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  if constexpr (LAST_USE) return ld16_stream(p);
  return ld16(p);
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ void st16_stream(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// ---------------------------------------------------------------------------
// Post: the fixed binary32 chain a = post_j * y; a = fma(res_ji, x_i, a),
// i = 0..3, then one bf16 rounding.  Written with explicit builtins so the
// compiler cannot contract or reorder it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float post_chain(float pw, float yv, const float* rj, float x0, float x1,
                                            float x2, float x3) {
  float a = pw * yv;  // an fma addend, so it cannot be contracted into anything
  a = __builtin_fmaf(rj[0], x0, a);
  a = __builtin_fmaf(rj[1], x1, a);
  a = __builtin_fmaf(rj[2], x2, a);
  a = __builtin_fmaf(rj[3], x3, a);
  return a;
}

// ---------------------------------------------------------------------------
// Coefficient finalisation of one token: RMS scale, logits, sigmoid
// pre/post, Sinkhorn on exp(logits) (rows, then columns, each divided by its
// sum + eps).  sums: d[24] followed by the sum of squares.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

__device__ inline void finalize_coeffs(const float* d, float ss, const float* bias, int C,
                                       const Scalars& sc, float* out) {
  const float r = 1.0f / sqrtf(ss / (float)(kRoutes * C) + sc.hc_norm_eps);
  float l[kCoeffs];
#pragma unroll
  for (int m = 0; m < kCoeffs; ++m) l[m] = r * d[m] + bias[m];
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = sigmoidf_(l[i]);
#pragma unroll
  for (int j = 0; j < 4; ++j) out[4 + j] = sc.hc_post_scale * sigmoidf_(l[4 + j]);
  float m[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) m[k] = expf(l[8 + k]);
  const float eps = sc.sinkhorn_eps;
  for (int it = 0; it < sc.sinkhorn_iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float s = ((m[4 * j] + m[4 * j + 1]) + m[4 * j + 2]) + m[4 * j + 3] + eps;
#pragma unroll
      for (int i = 0; i < 4; ++i) m[4 * j + i] = m[4 * j + i] / s;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = ((m[i] + m[4 + i]) + m[8 + i]) + m[12 + i] + eps;
#pragma unroll
      for (int j = 0; j < 4; ++j) m[4 * j + i] = m[4 * j + i] / s;
    }
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) out[8 + k] = m[k];
}

// sum_c g_c^2 for g = sum_i p_i x_i, from the route Gram matrix.
__device__ __forceinline__ float gram_quadratic(const float* G, const float* p) {
  float diag = p[0] * p[0] * G[0] + p[1] * p[1] * G[1] + p[2] * p[2] * G[2] + p[3] * p[3] * G[3];
  float off = p[0] * p[1] * G[4] + p[0] * p[2] * G[5] + p[0] * p[3] * G[6] + p[1] * p[2] * G[7] +
              p[1] * p[3] * G[8] + p[2] * p[3] * G[9];
  return diag + 2.0f * off;
}

// When the routes of the pre combination cancel, p^T G p is a small
// difference of large fp32 terms.  Each Gram entry carries an absolute error
// of at most n u sum_c |x_i x_j| <= n u sqrt(G_ii G_jj) (n fp32 additions on
// its longest path, at most ~170 for C <= 16384, u = 2^-24), so the error of
// p^T G p is bounded by about (n + 12) u B with
//   B = (sum_i |p_i| sqrt(G_ii))^2,
// i.e. ~1.1e-5 B.  A token with p^T G p <= B / 64 could carry a relative
// error above 1e-3 in its sum of squares; such a token is flagged and its
// pre is recomputed from x' directly (k_pre_fix).  Independent routes give
// p^T G p / B >= 1/4, so only strongly cancelling combinations are flagged.
constexpr float kCancelRatio = 1.0f / 64.0f;
__device__ __forceinline__ float gram_bound(const float* G, const float* p) {
  const float s = __builtin_fabsf(p[0]) * sqrtf(G[0]) + __builtin_fabsf(p[1]) * sqrtf(G[1]) +
                  __builtin_fabsf(p[2]) * sqrtf(G[2]) + __builtin_fabsf(p[3]) * sqrtf(G[3]);
  return s * s;
}
// The RMSNorm factor of the fused pre from the Gram matrix (the quadratic
// form clamped at 0, so that rounding never takes the square root of a
// negative number) and whether the token needs the direct recomputation.
__device__ __forceinline__ float gram_rms_factor(const float* G, const float* p, int C, float eps, bool& cancels) {
  const float gq = gram_quadratic(G, p);
  const float gb = gram_bound(G, p);
  cancels = gb > 0.0f && !(gq > kCancelRatio * gb);
  return 1.0f / sqrtf(__builtin_fmaxf(gq, 0.0f) / (float)C + eps);
}

// ---------------------------------------------------------------------------
// MXFP8: UE8M0 exponent of a block from the bits of its bf16 amax, and the
// OCP e4m3fn codes of the scaled values, round-to-nearest-even.
// amax = (1 + f/128) 2^E and 448 = 1.75 * 2^8, so the smallest e with
// amax <= 448 * 2^e is E - 8 when f <= 96 and E - 7 otherwise.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int mx_scale_exponent(float amax_bf16) {
  const uint32_t u = __float_as_uint(amax_bf16);
  const int ef = (int)((u >> 23) & 0xFF);
  if (ef == 0) return -127;  // zero or below 2^-126: the exponent clamps
  const int E = ef - 127;
  const int f = (int)((u >> 16) & 0x7F);
  int e = (f > 96) ? E - 7 : E - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Byte offset of the scale of token t's 32-channel block blk in h_scale:
// linear [T][C/32], or (mfma) the A-operand scale order of
// v_mfma_scale_f32_16x16x128_f8f6f4, [T/16][C/512][64 lanes][4 bytes] with
// lane 16 (blk % 4) + t % 16 and byte (blk / 4) % 4 of row block t / 16 and
// 512-channel group blk / 16.
__device__ __forceinline__ int64_t mx_scale_offset(int64_t t, int blk, int C, bool mfma) {
  if (!mfma) return t * (int64_t)(C >> 5) + blk;
  const int64_t lane = 16 * (blk & 3) + (t & 15);
  return ((((t >> 4) * (int64_t)(C >> 9) + (blk >> 4)) * 64 + lane) << 2) + ((blk >> 2) & 3);
}

// Four OCP e4m3fn codes of values with |v| <= 448, packed first value in the
// low byte, by the gfx950 converter (round to nearest even, subnormals kept):
// each pair is one v_cvt_pk_fp8_f32.  The codes are tested bit for bit
// against the oracle's encoder through the MXFP8 outputs.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------------------
// Wave reductions over lanes that differ in bits 4 and 5 (the four 16-lane
// groups of an MFMA operand).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sum_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ float max_groups(float v) {
  v = __builtin_fmaxf(v, __shfl_xor(v, 16));
  v = __builtin_fmaxf(v, __shfl_xor(v, 32));
  return v;
}

}  // namespace mhc
