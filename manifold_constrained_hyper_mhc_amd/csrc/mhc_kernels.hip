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
// exactly for |v| >= 2^-100).  Five MFMA column blocks of 16 per 32 rows:
//   block 0: hi  of logits 0..15        block 3: hi  of 16..23 | mid of 16..23
//   block 1: mid of logits 0..15        block 4: lo  of 16..23 | zero
//   block 2: lo  of logits 0..15
// Blocks 0-2 accumulate into one MFMA accumulator (x'*hi + x'*mid + x'*lo:
// every product is exact, the sum is an fp32 accumulation) and blocks 3-4
// into a second one whose columns 0..7 hold hi+lo and 8..15 mid of logits
// 16..23.
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
// Workgroup = 4 waves; blockIdx = tile * S + split.  A tile holds
// M = 16*RB tokens; the workgroup owns channels [split*CC, split*CC + CC) of
// all 4 routes and wave w the CW channels from split*CC + w*CW.  Lane l
// serves token 16*r + l%16 of row block r (r < RB) and, in each 32-channel
// step, channels 8*(l/16) .. +8.  That is the A-operand layout of
// v_mfma_f32_16x16x32_bf16, so the bf16 chunk a lane loads (or the x' it
// computes) is its MFMA operand as is, and one projection fragment serves
// RB row blocks.
//
// Phase A  load x (and y; post/res staged in LDS), compute x' with the post
//          chain, round to bf16, store it and keep it in registers;
//          accumulate the route Gram matrix of x' (fused; its trace is the
//          sum of squares) or the sum of squares of x (coeffs), and the 24
//          projections on the matrix cores.
// Reduce   fold hi+mid+lo, sum the 4 waves in LDS and write the tile's
//          partial [M][34] to the workspace.  Barrier 1 over the tile's S
//          workgroups; then workgroup `split` reduces tokens
//          split, split+S, ... (split order, so the sums are deterministic),
//          finalises their coefficients with one wave per token (Sinkhorn on
//          16 lanes) and, in the fused modes, publishes pre'_i * r_h, where
//          r_h is the RMSNorm scale of g = sum_i pre'_i x'_i obtained from
//          the Gram matrix: sum_c g_c^2 = pre'^T G pre'.  Barrier 2 (fused).
// Phase C  (fused) h = (sum_i q_i x'_i) * gamma from the registers, as bf16
//          and/or MXFP8.
//
// Communication between workgroups uses agent-coherent 64-bit words that
// carry a value and a tag: (float bits) | (tag << 32).  The tag of a launch
// is the tile's epoch + 1, read when the workgroup starts; a reader polls
// the words it needs until their tags match, so no counter sits on the
// critical path and no cache write-back or invalidation is needed (agent
// scope accesses bypass the per-XCD caches, and an aligned 64-bit access is
// single-copy atomic, so a value is never seen with the wrong tag).  The
// last workgroup of a tile to leave (a counter off the critical path) bumps
// the epoch, so every launch uses a fresh tag and a zero-filled workspace
// is a valid start.  Every word a launch reads is written in that launch.
// Workgroups are dispatched in blockIdx order, so every workgroup a waiting
// one depends on is running or will run once earlier tiles retire; the waits
// are bounded anyway and set the workspace error word on expiry.
// ===========================================================================
constexpr uint32_t kSpinLimit = 1u << 22;
// Reduce-scatter bounds: a workgroup owns at most ceil(M/S) <= 8 tokens
// (M = 64, S >= 8) and gathers at most (M + S - 1) * 34 <= 18 * 256 words.
constexpr int kMaxTileTokensPerGroup = 8;
constexpr int kGatherPerThread = 18;

__device__ __forceinline__ void tagged_store(uint64_t* p, float v, uint32_t tag) {
  const uint64_t w = (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float tagged_value(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Wait until the word at p carries `tag`; returns its value.
__device__ __forceinline__ float tagged_wait(const uint64_t* p, uint32_t tag, uint32_t* err) {
  uint64_t w = tagged_load(p);
  uint32_t it = 0;
  while ((uint32_t)(w >> 32) != tag) {
    __builtin_amdgcn_s_sleep(1);
    if (++it > kSpinLimit) {
      __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    w = tagged_load(p);
  }
  return tagged_value(w);
}

// Coefficients of one token on one wave.  sums: 24 projections, then the
// Gram matrix (fused) or the sum of squares (coeffs).  Lanes 0..15 carry
// res[j][i] (j = lane/4, i = lane%4), lanes 16..23 pre/post.  Returns in
// every lane the value of coefficient `slot(lane)`; q gets pre_i * r_h.
template <bool FUSED>
__device__ __forceinline__ float finalize_wave(const float* sums, const float* bias, int C, const Scalars& sc,
                                               int lane, float* q) {
  const float ss = FUSED ? ((sums[24] + sums[25]) + sums[26]) + sums[27] : sums[24];
  const float r = 1.0f / sqrtf(ss / (float)(kRoutes * C) + sc.hc_norm_eps);
  const int li = lane < 16 ? 8 + lane : (lane < 24 ? lane - 16 : 0);
  const float l = r * sums[li] + bias[li];
  const float sg = 1.0f / (1.0f + expf(-l));
  const float pp = (lane >= 20 && lane < 24) ? sc.hc_post_scale * sg : sg;
  float v = expf(l);
  const float eps = sc.sinkhorn_eps;
  for (int it = 0; it < sc.sinkhorn_iters; ++it) {
    float rs = v + __shfl_xor(v, 1);
    rs += __shfl_xor(rs, 2);
    v = v / (rs + eps);
    float cs = v + __shfl_xor(v, 4);
    cs += __shfl_xor(cs, 8);
    v = v / (cs + eps);
  }
  if constexpr (FUSED) {
    const float p[4] = {__shfl(pp, 16), __shfl(pp, 17), __shfl(pp, 18), __shfl(pp, 19)};
    const float gq = gram_quadratic(sums + 24, p);
    const float rh = 1.0f / sqrtf(gq / (float)C + sc.rmsnorm_eps);
    q[0] = p[0] * rh;
    q[1] = p[1] * rh;
    q[2] = p[2] * rh;
    q[3] = p[3] * rh;
  }
  return lane < 16 ? v : pp;
}

template <int MODE, int RB, int CW>
__global__ __launch_bounds__(256, 2) void k_split(const SplitArgs a) {
  constexpr bool FUSED = MODE != kModeCoeffs;
  constexpr bool MX = MODE == kModeFusedMx;
  constexpr int W = 4, M = 16 * RB, NS = CW / 32, CC = W * CW;
  constexpr int NV = kPartVals;
  constexpr int NG = FUSED ? kGram : 1;

  __shared__ float red[W][M][NV];
  __shared__ float cfs[FUSED ? M : 1][20];
  __shared__ float fin[kMaxTileTokensPerGroup][NV];
  __shared__ float qs[FUSED ? M : 1][4];
  __shared__ uint32_t s_tag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int S = a.S;
  const int tile = (int)(blockIdx.x / S), split = (int)(blockIdx.x % S);
  const int64_t tok0 = (int64_t)tile * M;
  const int C = a.C;
  const int cw0 = split * CC + wave * CW;

  if (tid == 0)
    s_tag = __hip_atomic_load(a.epoch + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  // ---------------- phase A: loads ----------------
  if constexpr (FUSED) {
    for (int idx = tid; idx < M * 5; idx += 256) {
      const int m = idx / 5, k = idx % 5;
      const int64_t t = tok0 + m;
      const float4 v = t < a.T ? reinterpret_cast<const float4*>(a.coeffs_in + t * kCoeffs)[1 + k]
                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      cfs[m][4 * k] = v.x;
      cfs[m][4 * k + 1] = v.y;
      cfs[m][4 * k + 2] = v.z;
      cfs[m][4 * k + 3] = v.w;
    }
  }
  u32x4_t xf[RB][NS][4];
  u32x4_t yv[RB][NS];
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
  }
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
  __syncthreads();  // cfs, s_tag
  const uint32_t tag = s_tag;

  // ---------------- phase A: post and statistics ----------------
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    float st[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) st[k] = 0.0f;
    float pw[4], rs[16];
    if constexpr (FUSED) {
#pragma unroll
      for (int k = 0; k < 4; ++k) pw[k] = cfs[r * 16 + n16][k];
#pragma unroll
      for (int k = 0; k < 16; ++k) rs[k] = cfs[r * 16 + n16][4 + k];
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (FUSED) {
        // two channels at a time: unpack, post chain, round, statistics
        u32x4_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float xl[4] = {bf16_lo(xf[r][s][0][k]), bf16_lo(xf[r][s][1][k]), bf16_lo(xf[r][s][2][k]),
                               bf16_lo(xf[r][s][3][k])};
          const float xh[4] = {bf16_hi(xf[r][s][0][k]), bf16_hi(xf[r][s][1][k]), bf16_hi(xf[r][s][2][k]),
                               bf16_hi(xf[r][s][3][k])};
          const float yl = bf16_lo(yv[r][s][k]), yh = bf16_hi(yv[r][s][k]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[j][k] = pack_bf16x2(post_chain(pw[j], yl, &rs[4 * j], xl[0], xl[1], xl[2], xl[3]),
                                  post_chain(pw[j], yh, &rs[4 * j], xh[0], xh[1], xh[2], xh[3]));
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const float v0 = h2 ? bf16_hi(o[0][k]) : bf16_lo(o[0][k]);
            const float v1 = h2 ? bf16_hi(o[1][k]) : bf16_lo(o[1][k]);
            const float v2 = h2 ? bf16_hi(o[2][k]) : bf16_lo(o[2][k]);
            const float v3 = h2 ? bf16_hi(o[3][k]) : bf16_lo(o[3][k]);
            st[0] = __builtin_fmaf(v0, v0, st[0]);
            st[1] = __builtin_fmaf(v1, v1, st[1]);
            st[2] = __builtin_fmaf(v2, v2, st[2]);
            st[3] = __builtin_fmaf(v3, v3, st[3]);
            st[4] = __builtin_fmaf(v0, v1, st[4]);
            st[5] = __builtin_fmaf(v0, v2, st[5]);
            st[6] = __builtin_fmaf(v0, v3, st[6]);
            st[7] = __builtin_fmaf(v1, v2, st[7]);
            st[8] = __builtin_fmaf(v1, v3, st[8]);
            st[9] = __builtin_fmaf(v2, v3, st[9]);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) xf[r][s][j] = o[j];
        if (valid[r]) {
          const int64_t t = tok0 + r * 16 + n16;
          uint16_t* xo = a.x_out + t * (int64_t)(4 * C) + cw0 + s * 32 + g * 8;
#pragma unroll
          for (int j = 0; j < 4; ++j) st16_stream(xo + (int64_t)j * C, xf[r][s][j]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float vl = bf16_lo(xf[r][s][i][k]), vh = bf16_hi(xf[r][s][i][k]);
            st[0] = __builtin_fmaf(vl, vl, st[0]);
            st[0] = __builtin_fmaf(vh, vh, st[0]);
          }
      }
    }
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float v = sum_groups(st[k]);
      if (g == 0) red[wave][r * 16 + n16][24 + k] = v;
    }
  }

  // ---------------- phase A: projection on the matrix cores ----------------
  f32x4_t acc[RB][2];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    acc[r][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    acc[r][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_barrier(0);  // keep one route's fragments live at a time
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
          acc[r][b < 3 ? 0 : 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              av, __builtin_bit_cast(bf16x8_t, bfrag[b]), acc[r][b < 3 ? 0 : 1], 0, 0, 0);
      }
    }
  }
  // MFMA output: lane l holds column l%16 of rows 4*(l/16)+e, e = 0..3.
#pragma unroll
  for (int r = 0; r < RB; ++r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v1 = acc[r][1][e];
      const float mid = __shfl_xor(v1, 8);
      const int row = r * 16 + 4 * g + e;
      red[wave][row][n16] = acc[r][0][e];
      if (n16 < 8) red[wave][row][16 + n16] = v1 + mid;
    }
  }
  __syncthreads();

  // ---------------- tile partial -> workspace ----------------
  constexpr int NVU = FUSED ? NV : 25;
  uint64_t* part = a.partials + (int64_t)blockIdx.x * (M * NV);
  const float* flat_red = &red[0][0][0];
  for (int idx = tid; idx < M * NV; idx += 256) {
    if (idx % NV >= NVU) continue;
    tagged_store(part + idx, ((flat_red[idx] + flat_red[M * NV + idx]) + flat_red[2 * M * NV + idx]) +
                                 flat_red[3 * M * NV + idx], tag);
  }

  // ---------------- reduce-scatter: tokens split, split+S, ... ----------------
  // Token m of the tile is reduced by workgroup m % S, which owns
  // ntok <= ceil(M/S) tokens.  Their ntok x S x 34 tagged words are
  // gathered with every load in flight (<= kGatherPerThread per thread),
  // the stale ones re-polled together, staged in LDS (over the per-wave
  // partial buffer, no longer needed) and summed in split order.
  const uint64_t* tp = a.partials + (int64_t)tile * S * (M * NV);
  const int ntok = split < M ? (M - split + S - 1) / S : 0;
  if (ntok > 0) {
    float* stage = &red[0][0][0];
    const int nwords = ntok * S * NV;
    uint64_t w[kGatherPerThread];
#pragma unroll
    for (int q = 0; q < kGatherPerThread; ++q) {
      const int u = tid + 256 * q;
      const int v = u % NV, rr = u / NV;
      const int sp = rr % S, kk = rr / S;
      w[q] = (u < nwords && v < NVU) ? tagged_load(tp + ((int64_t)sp * M + split + kk * S) * NV + v)
                                     : ((uint64_t)tag << 32);
    }
    uint32_t it = 0;
    for (;;) {
      bool stale = false;
#pragma unroll
      for (int q = 0; q < kGatherPerThread; ++q) stale |= (uint32_t)(w[q] >> 32) != tag;
      if (!stale) break;
      __builtin_amdgcn_s_sleep(1);
      if (++it > kSpinLimit) {
        __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
#pragma unroll
      for (int q = 0; q < kGatherPerThread; ++q) {
        const int u = tid + 256 * q;
        const int v = u % NV, rr = u / NV;
        const int sp = rr % S, kk = rr / S;
        if ((uint32_t)(w[q] >> 32) != tag) w[q] = tagged_load(tp + ((int64_t)sp * M + split + kk * S) * NV + v);
      }
    }
#pragma unroll
    for (int q = 0; q < kGatherPerThread; ++q) {
      const int u = tid + 256 * q;
      if (u < nwords) stage[u] = tagged_value(w[q]);
    }
    __syncthreads();
    for (int pidx = tid; pidx < ntok * NV; pidx += 256) {
      const int kk = pidx / NV, v = pidx % NV;
      float acc = 0.0f;
      if (v < NVU)
        for (int sp = 0; sp < S; ++sp) acc += stage[(kk * S + sp) * NV + v];
      fin[kk][v] = acc;
    }
    __syncthreads();
    for (int k0 = 0; k0 < ntok; k0 += W) {
      const int kk = k0 + wave;
      if (kk < ntok) {
        const int m = split + kk * S;
        float q[4];
        const float cv = finalize_wave<FUSED>(fin[kk], a.bias, C, a.sc, lane, q);
        const int64_t t = tok0 + m;
        if (t < a.T && lane < 24) a.coeffs_out[t * kCoeffs + (lane < 16 ? 8 + lane : lane - 16)] = cv;
        if constexpr (FUSED) {
          if (lane < 4) tagged_store(a.publish + ((int64_t)tile * M + m) * 4 + lane, q[lane], tag);
        }
      }
    }
  }

  if constexpr (FUSED) {
    for (int idx = tid; idx < M * 4; idx += 256)
      (&qs[0][0])[idx] = tagged_wait(a.publish + (int64_t)tile * M * 4 + idx, tag, a.err);
  }
  // leave: the last workgroup of the tile moves the epoch on
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.dep + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)S - 1u) {
      __hip_atomic_store(a.dep + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.epoch + tile, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if constexpr (!FUSED) return;

  // ---------------- phase C: h = (sum_i q_i x'_i) * gamma ----------------
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
  if (p.rb == 4 && p.cw == 32) {
    k_split<MODE, 4, 32><<<grid, block, 0, s>>>(a);
  } else if (p.rb == 2 && p.cw == 64) {
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
