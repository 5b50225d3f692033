// libmhc kernels for gfx950 (MI355X): wave64, MFMA 16x16x32 bf16, LDS.
//
// The path ([P1] "What this fixes"; [P2] review "Correctness findings";
// [P3] "What changed" item 3 — see include/mhc.h for the page titles):
//   post      x'_j = sum_i res_ji x_i + post_j y                     (k_post)
//   coeffs    RMS-scaled 24-wide projection of the flattened row,
//             sigmoid pre/post, Sinkhorn res                          (k_split, coeffs mode)
//   pre       h = RMSNorm(sum_i pre_i x_i) * gamma                    (k_pre)
//   fused     post -> coeffs' -> pre' with x' kept on chip            (k_split, fused modes)
#include "mhc_device.h"

namespace mhc {

// ===========================================================================
// Projection packing.  The flattened row index k = route*C + c runs over 4C
// rows of phi [4C][24].  Each fp32 element is split into three bf16 terms
// (hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi - mid); the sum is v
// exactly for |v| >= 2^-100), giving 72 columns, padded to 80 = five MFMA
// column blocks:
//   block 0: hi  of logits 0..15        block 3: hi  of 16..23 | mid of 16..23
//   block 1: mid of logits 0..15        block 4: lo  of 16..23 | zero
//   block 2: lo  of logits 0..15
// Packed layout: [k/32][block][lane 0..63][8 bf16]; lane l of a fragment
// holds rows k = 32q + 8*(l/16) + e, e = 0..7, of column 16*block + l%16,
// which is the B-operand layout of v_mfma_f32_16x16x32_bf16.
// ===========================================================================
__device__ __forceinline__ float bf16_round_f(float v) { return bf16_lo(pack_bf16x2(v, 0.0f)); }

__global__ __launch_bounds__(256) void k_pack_phi(const float* __restrict__ phi, int C,
                                                  u32x4_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(4 * C / 32) * kPackBlocks * kWave;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  const int64_t qb = idx >> 6;
  const int blk = (int)(qb % kPackBlocks);
  const int64_t q = qb / kPackBlocks;
  const int n16 = lane & 15, g = lane >> 4;
  int col, term;
  if (blk < 3) {
    col = n16;
    term = blk;
  } else if (blk == 3) {
    col = 16 + (n16 & 7);
    term = n16 < 8 ? 0 : 1;
  } else {
    col = n16 < 8 ? 16 + n16 : -1;
    term = 2;
  }
  float v[8];
  const int64_t k0 = q * 32 + g * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float p = col >= 0 ? phi[(k0 + e) * kCoeffs + col] : 0.0f;
    const float hi = bf16_round_f(p);
    const float r1 = p - hi;
    const float mid = bf16_round_f(r1);
    const float lo = bf16_round_f(r1 - mid);
    v[e] = term == 0 ? hi : (term == 1 ? mid : lo);
  }
  out[idx] = pack8(v);
}

// ===========================================================================
// Split-row kernel.
//
// Workgroup = 4 waves; blockIdx = tile * S + split.  The tile holds
// M = 16*RB tokens; the workgroup owns channels [split*CC, split*CC + CC) of
// all 4 routes, wave w the CW channels starting at split*CC + w*CW.
// Lane l serves token 16*r + l%16 of row block r and, in each 32-channel
// step, channels 8*(l/16) .. +8: this is the A-operand layout of the MFMA,
// so the bf16 stream chunk a lane loads (or the x' it computes) is its MFMA
// operand without any shuffle.
//
// Phase A  load x (and y, post/res), compute x' = post chain (bf16), store
//          x', accumulate the route Gram matrix (fused) or the sum of
//          squares (coeffs) and the 24 projections on the matrix cores.
// Reduce   fold hi+mid+lo, sum the 4 waves in LDS, write the tile's partial
//          [M][34] to the workspace and arrive on the tile counter.  The
//          last workgroup to arrive sums the S partials in split order
//          (deterministic), finalises the coefficients of the M tokens and,
//          in the fused modes, publishes pre'_i * r_h (the RMSNorm scale of
//          g = sum_i pre'_i x'_i, taken from the Gram matrix:
//          sum_c g_c^2 = pre'^T G pre') and raises the tile flag.
// Phase C  (fused) the other workgroups wait for the flag, then every
//          workgroup writes h = (sum_i q_i x'_i) * gamma from the x' still in
//          registers, as bf16 and/or MXFP8.
//
// Progress: workgroups are dispatched in blockIdx order, so a waiting
// workgroup's partners are either running or will be dispatched once earlier
// (complete) tiles retire.  The wait is bounded anyway; on expiry it sets the
// workspace error word and continues.
// ===========================================================================
constexpr uint32_t kSpinLimit = 1u << 24;

template <int MODE, int RB, int CW>
__global__ __launch_bounds__(256) void k_split(const SplitArgs a) {
  constexpr bool FUSED = MODE != kModeCoeffs;
  constexpr bool MX = MODE == kModeFusedMx;
  constexpr int W = 4, M = 16 * RB, NS = CW / 32, CC = W * CW;
  constexpr int NV = kPartVals;

  __shared__ float red[W][M][NV];
  __shared__ float fin[M][NV];
  __shared__ float qs[M][4];
  __shared__ uint32_t s_last, s_f0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int S = a.S;
  const int tile = (int)(blockIdx.x / S), split = (int)(blockIdx.x % S);
  const int64_t tok0 = (int64_t)tile * M;
  const int C = a.C;
  const int cw0 = split * CC + wave * CW;

  // ---------------- phase A: loads ----------------
  u32x4_t xf[RB][NS][4];
  u32x4_t yv[RB][NS];
  float pw[RB][4], rs[RB][16];
  bool valid[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int64_t t = tok0 + r * 16 + n16;
    valid[r] = t < a.T;
    const uint16_t* xr = a.x + (valid[r] ? t : 0) * (int64_t)(4 * C);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = cw0 + s * 32 + g * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xf[r][s][i] = valid[r] ? ld16_stream(xr + (int64_t)i * C + c) : u32x4_t{0, 0, 0, 0};
      if constexpr (FUSED)
        yv[r][s] = valid[r] ? ld16_stream(a.y + t * (int64_t)C + c) : u32x4_t{0, 0, 0, 0};
    }
    if constexpr (FUSED) {
      const float* cf = a.coeffs_in + (valid[r] ? t : 0) * kCoeffs + 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) pw[r][k] = valid[r] ? cf[k] : 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) rs[r][k] = valid[r] ? cf[4 + k] : 0.0f;
    }
  }

  // ---------------- phase A: post, statistics, projection ----------------
  constexpr int NG = FUSED ? kGram : 1;
  float st[RB][NG];
  f32x4_t acc[RB][kPackBlocks];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
#pragma unroll
    for (int k = 0; k < NG; ++k) st[r][k] = 0.0f;
#pragma unroll
    for (int b = 0; b < kPackBlocks; ++b) acc[r][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float xv[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) unpack8(xf[r][s][i], xv[i]);
      if constexpr (FUSED) {
        float yy[8];
        unpack8(yv[r][s], yy);
        float o[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            o[j][e] = post_chain(pw[r][j], yy[e], &rs[r][4 * j], xv[0][e], xv[1][e], xv[2][e], xv[3][e]);
#pragma unroll
        for (int j = 0; j < 4; ++j) xf[r][s][j] = pack8(o[j]);
        if (valid[r]) {
          const int64_t t = tok0 + r * 16 + n16;
          uint16_t* xo = a.x_out + t * (int64_t)(4 * C) + cw0 + s * 32 + g * 8;
#pragma unroll
          for (int j = 0; j < 4; ++j) st16_stream(xo + (int64_t)j * C, xf[r][s][j]);
        }
        // statistics of the bf16 x'
#pragma unroll
        for (int j = 0; j < 4; ++j) unpack8(xf[r][s][j], xv[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          st[r][0] = __builtin_fmaf(xv[0][e], xv[0][e], st[r][0]);
          st[r][1] = __builtin_fmaf(xv[1][e], xv[1][e], st[r][1]);
          st[r][2] = __builtin_fmaf(xv[2][e], xv[2][e], st[r][2]);
          st[r][3] = __builtin_fmaf(xv[3][e], xv[3][e], st[r][3]);
          st[r][4] = __builtin_fmaf(xv[0][e], xv[1][e], st[r][4]);
          st[r][5] = __builtin_fmaf(xv[0][e], xv[2][e], st[r][5]);
          st[r][6] = __builtin_fmaf(xv[0][e], xv[3][e], st[r][6]);
          st[r][7] = __builtin_fmaf(xv[1][e], xv[2][e], st[r][7]);
          st[r][8] = __builtin_fmaf(xv[1][e], xv[3][e], st[r][8]);
          st[r][9] = __builtin_fmaf(xv[2][e], xv[3][e], st[r][9]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) st[r][0] = __builtin_fmaf(xv[i][e], xv[i][e], st[r][0]);
      }
    }
    // projection: 4 routes x 5 column blocks per 32-channel step
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kstep = ((int64_t)j * C + cw0 + s * 32) >> 5;
      const u32x4_t* bp = reinterpret_cast<const u32x4_t*>(a.phi_packed) + kstep * (kPackBlocks * kWave) + lane;
      u32x4_t bfrag[kPackBlocks];
#pragma unroll
      for (int b = 0; b < kPackBlocks; ++b) bfrag[b] = bp[b * kWave];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xf[r][s][j]);
#pragma unroll
        for (int b = 0; b < kPackBlocks; ++b)
          acc[r][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bfrag[b]),
                                                             acc[r][b], 0, 0, 0);
      }
    }
  }

  // gamma for phase C, fetched while the reduction runs
  float gm[NS][8];
  if constexpr (FUSED) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float4* gp = reinterpret_cast<const float4*>(a.gamma + cw0 + s * 32 + g * 8);
      const float4 g0 = gp[0], g1 = gp[1];
      gm[s][0] = g0.x; gm[s][1] = g0.y; gm[s][2] = g0.z; gm[s][3] = g0.w;
      gm[s][4] = g1.x; gm[s][5] = g1.y; gm[s][6] = g1.z; gm[s][7] = g1.w;
    }
  }

  // ---------------- reduce within the workgroup ----------------
  // MFMA output: lane l holds column l%16 of rows 4*(l/16)+e, e = 0..3.
#pragma unroll
  for (int r = 0; r < RB; ++r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo16 = (acc[r][0][e] + acc[r][1][e]) + acc[r][2][e];
      const float v3 = acc[r][3][e], v4 = acc[r][4][e];
      const float mid = __shfl_xor(v3, 8);
      const int row = r * 16 + 4 * g + e;
      red[wave][row][n16] = lo16;
      if (n16 < 8) red[wave][row][16 + n16] = (v3 + mid) + v4;
    }
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float v = sum_groups(st[r][k]);
      if (g == 0) red[wave][r * 16 + n16][24 + k] = v;
    }
  }
  __syncthreads();
  float* flat_fin = &fin[0][0];
  const float* flat_red = &red[0][0][0];
  constexpr int NVU = FUSED ? NV : 25;  // values in use per token
  for (int idx = tid; idx < M * NV; idx += 256) {
    if (idx % NV >= NVU) continue;
    flat_fin[idx] = ((flat_red[idx] + flat_red[M * NV + idx]) + flat_red[2 * M * NV + idx]) +
                    flat_red[3 * M * NV + idx];
  }

  bool last = true;
  uint32_t f0 = 0;
  if (S > 1) {
    float* part = a.partials + (int64_t)blockIdx.x * (M * NV);
    for (int idx = tid; idx < M * NV; idx += 256) part[idx] = flat_fin[idx];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const uint32_t fl = __hip_atomic_load(&a.flag[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t old = __hip_atomic_fetch_add(&a.cnt[tile], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      s_f0 = fl;
      s_last = (old == (uint32_t)(S - 1)) ? 1u : 0u;
    }
    __syncthreads();
    last = s_last != 0;
    f0 = s_f0;
    if (last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const float* tp = a.partials + (int64_t)tile * S * (M * NV);
      for (int idx = tid; idx < M * NV; idx += 256) {
        if (idx % NV >= NVU) continue;
        float v = 0.0f;
        for (int sp = 0; sp < S; ++sp) v += tp[(int64_t)sp * (M * NV) + idx];
        flat_fin[idx] = v;
      }
    }
  }

  if (last) {
    __syncthreads();
    if (tid < M) {
      const int64_t t = tok0 + tid;
      float ss;
      if constexpr (FUSED)
        ss = ((fin[tid][24] + fin[tid][25]) + fin[tid][26]) + fin[tid][27];
      else
        ss = fin[tid][24];
      float out[kCoeffs];
      finalize_coeffs(&fin[tid][0], ss, a.bias, C, a.sc, out);
      if (t < a.T) {
        float4* co = reinterpret_cast<float4*>(a.coeffs_out + t * kCoeffs);
#pragma unroll
        for (int k = 0; k < 6; ++k) co[k] = make_float4(out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]);
      }
      if constexpr (FUSED) {
        const float q = gram_quadratic(&fin[tid][24], out);
        const float rh = 1.0f / sqrtf(q / (float)C + a.sc.rmsnorm_eps);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qs[tid][i] = out[i] * rh;
          if (S > 1) a.publish[((int64_t)tile * M + tid) * 4 + i] = out[i] * rh;
        }
      }
    }
    if (S > 1) {
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        __hip_atomic_store(&a.cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (FUSED)
          __hip_atomic_store(&a.flag[tile], f0 + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  } else {
    if constexpr (!FUSED) return;  // coeffs: only the last workgroup writes
    if (tid == 0) {
      uint32_t it = 0;
      while (__hip_atomic_load(&a.flag[tile], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == f0) {
        __builtin_amdgcn_s_sleep(2);
        if (++it > kSpinLimit) {
          __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int idx = tid; idx < M * 4; idx += 256) (&qs[0][0])[idx] = a.publish[(int64_t)tile * M * 4 + idx];
    __syncthreads();
  }

  // ---------------- phase C: h = (sum_i q_i x'_i) * gamma ----------------
  if constexpr (FUSED) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t t = tok0 + r * 16 + n16;
      const float q0 = qs[r * 16 + n16][0], q1 = qs[r * 16 + n16][1];
      const float q2 = qs[r * 16 + n16][2], q3 = qs[r * 16 + n16][3];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = cw0 + s * 32 + g * 8;
        float xv[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) unpack8(xf[r][s][i], xv[i]);
        float hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = q0 * xv[0][e];
          v = __builtin_fmaf(q1, xv[1][e], v);
          v = __builtin_fmaf(q2, xv[2][e], v);
          v = __builtin_fmaf(q3, xv[3][e], v);
          hv[e] = v * gm[s][e];
        }
        const u32x4_t hb = pack8(hv);
        if (a.h != nullptr && valid[r]) st16_stream(a.h + t * (int64_t)C + c, hb);
        if constexpr (MX) {
          float hr[8];
          unpack8(hb, hr);
          float amax = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(hr[e]));
          amax = max_groups(amax);
          const int ex = mx_scale_exponent(amax);
          const float scale = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-ex, ex <= 120
          uint32_t w0 = 0, w1 = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w0 |= e4m3_code(hr[e] * scale) << (8 * e);
            w1 |= e4m3_code(hr[4 + e] * scale) << (8 * e);
          }
          if (valid[r]) {
            *reinterpret_cast<u32x2_t*>(a.h_fp8 + t * (int64_t)C + c) = u32x2_t{w0, w1};
            if (g == 0) a.h_scale[t * (int64_t)(C / 32) + ((cw0 + s * 32) >> 5)] = (uint8_t)(ex + 127);
          }
        }
      }
    }
  }
}

// ===========================================================================
// Post (standalone): one thread per (token, 8 channels); consecutive threads
// read consecutive 16-byte chunks of each route.
// ===========================================================================
__global__ __launch_bounds__(256) void k_post(const uint16_t* __restrict__ x, const uint16_t* __restrict__ y,
                                              const float* __restrict__ cf, int64_t T, int C,
                                              uint16_t* __restrict__ x_out) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int G = C >> 3;
  const int64_t t = u / G;
  if (t >= T) return;
  const int c = (int)(u - t * G) * 8;
  const float* cp = cf + t * kCoeffs + 4;
  float pw[4], rs[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) pw[k] = cp[k];
#pragma unroll
  for (int k = 0; k < 16; ++k) rs[k] = cp[4 + k];
  const uint16_t* xr = x + t * (int64_t)(4 * C) + c;
  float xv[4][8], yy[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack8(ld16_stream(xr + (int64_t)i * C), xv[i]);
  unpack8(ld16_stream(y + t * (int64_t)C + c), yy);
  uint16_t* xo = x_out + t * (int64_t)(4 * C) + c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = post_chain(pw[j], yy[e], &rs[4 * j], xv[0][e], xv[1][e], xv[2][e], xv[3][e]);
    st16_stream(xo + (int64_t)j * C, pack8(o));
  }
}

// ===========================================================================
// Pre (standalone): one workgroup of 128 threads per token.  Thread k holds
// G 8-channel groups (channels 8*(j*128 + k)), so C = 1024*G; g stays in
// registers for the normalisation.  For C > 8192 the row is read twice.
// ===========================================================================
__device__ __forceinline__ float block128_sum(float v, float* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) sh[tid >> 6] = v;
  __syncthreads();
  return sh[0] + sh[1];
}

__device__ __forceinline__ void pre_group(const uint16_t* xr, int C, int c, const float* p, float* gv) {
  float xv[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack8(ld16_stream(xr + (int64_t)i * C + c), xv[i]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v = p[0] * xv[0][e];
    v = __builtin_fmaf(p[1], xv[1][e], v);
    v = __builtin_fmaf(p[2], xv[2][e], v);
    v = __builtin_fmaf(p[3], xv[3][e], v);
    gv[e] = v;
  }
}

__device__ __forceinline__ void pre_store(uint16_t* hr, const float* gamma, int c, const float* gv, float rh) {
  const float4* gp = reinterpret_cast<const float4*>(gamma + c);
  const float4 g0 = gp[0], g1 = gp[1];
  const float gmv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  float hv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) hv[e] = (gv[e] * rh) * gmv[e];
  st16_stream(hr + c, pack8(hv));
}

template <int G>
__global__ __launch_bounds__(128) void k_pre(const uint16_t* __restrict__ x, const float* __restrict__ cf,
                                             const float* __restrict__ gamma, int C, float eps,
                                             uint16_t* __restrict__ h) {
  __shared__ float sh[2];
  const int64_t t = blockIdx.x;
  const int k = threadIdx.x;
  const float4 pq = *reinterpret_cast<const float4*>(cf + t * kCoeffs);
  const float p[4] = {pq.x, pq.y, pq.z, pq.w};
  const uint16_t* xr = x + t * (int64_t)(4 * C);
  float gv[G][8];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    pre_group(xr, C, (j * 128 + k) * 8, p, gv[j]);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(gv[j][e], gv[j][e], ss);
  }
  ss = block128_sum(ss, sh);
  const float rh = 1.0f / sqrtf(ss / (float)C + eps);
  uint16_t* hr = h + t * (int64_t)C;
#pragma unroll
  for (int j = 0; j < G; ++j) pre_store(hr, gamma, (j * 128 + k) * 8, gv[j], rh);
}

__global__ __launch_bounds__(128) void k_pre_wide(const uint16_t* __restrict__ x, const float* __restrict__ cf,
                                                  const float* __restrict__ gamma, int C, float eps,
                                                  uint16_t* __restrict__ h) {
  __shared__ float sh[2];
  const int64_t t = blockIdx.x;
  const int k = threadIdx.x;
  const float4 pq = *reinterpret_cast<const float4*>(cf + t * kCoeffs);
  const float p[4] = {pq.x, pq.y, pq.z, pq.w};
  const uint16_t* xr = x + t * (int64_t)(4 * C);
  const int G = C >> 10;
  float ss = 0.0f;
  for (int j = 0; j < G; ++j) {
    float gv[8];
    pre_group(xr, C, (j * 128 + k) * 8, p, gv);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(gv[e], gv[e], ss);
  }
  ss = block128_sum(ss, sh);
  const float rh = 1.0f / sqrtf(ss / (float)C + eps);
  uint16_t* hr = h + t * (int64_t)C;
  for (int j = 0; j < G; ++j) {
    float gv[8];
    pre_group(xr, C, (j * 128 + k) * 8, p, gv);
    pre_store(hr, gamma, (j * 128 + k) * 8, gv, rh);
  }
}

__global__ void k_fill_zero(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ===========================================================================
// Launchers
// ===========================================================================
hipError_t launch_pack_phi(const float* phi, int C, void* out, hipStream_t s) {
  const int64_t total = (int64_t)(4 * C / 32) * kPackBlocks * kWave;
  const int64_t blocks = (total + 255) / 256;
  k_pack_phi<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(phi, C, reinterpret_cast<u32x4_t*>(out));
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_split_mode(const Plan& p, const SplitArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(p.tiles * p.s)), block(256);
  if (p.rb == 2 && p.cw == 64) {
    k_split<MODE, 2, 64><<<grid, block, 0, s>>>(a);
  } else if (p.rb == 1 && p.cw == 128) {
    k_split<MODE, 1, 128><<<grid, block, 0, s>>>(a);
  } else {
    return hipErrorInvalidConfiguration;
  }
  return hipGetLastError();
}

hipError_t launch_split(const Plan& plan, int mode, const SplitArgs& a, hipStream_t s) {
  switch (mode) {
    case kModeCoeffs: return launch_split_mode<kModeCoeffs>(plan, a, s);
    case kModeFused: return launch_split_mode<kModeFused>(plan, a, s);
    case kModeFusedMx: return launch_split_mode<kModeFusedMx>(plan, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_post(const uint16_t* x, const uint16_t* y, const float* cf, int64_t T, int C,
                       uint16_t* x_out, hipStream_t s) {
  const int64_t units = T * (C / 8);
  const int64_t blocks = (units + 255) / 256;
  k_post<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(x, y, cf, T, C, x_out);
  return hipGetLastError();
}

hipError_t launch_pre(const uint16_t* x, const float* cf, const float* gamma, int64_t T, int C,
                      float eps, uint16_t* h, hipStream_t s) {
  const dim3 grid((unsigned)T), block(128);
  switch (C >> 10) {
    case 1: k_pre<1><<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
    case 2: k_pre<2><<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
    case 3: k_pre<3><<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
    case 4: k_pre<4><<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
    case 5: k_pre<5><<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
    case 6: k_pre<6><<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
    case 7: k_pre<7><<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
    case 8: k_pre<8><<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
    default: k_pre_wide<<<grid, block, 0, s>>>(x, cf, gamma, C, eps, h); break;
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  k_fill_zero<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(reinterpret_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace mhc
