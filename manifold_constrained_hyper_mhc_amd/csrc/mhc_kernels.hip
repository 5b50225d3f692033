// libmhc kernels for gfx950 (MI355X): wave64, MFMA 16x16x32 bf16, LDS.
//
// The path ([P1] "What this fixes"; [P2] review "Correctness findings";
// [P3] "What changed" item 3 — see include/mhc.h for the page titles):
//   post      x'_j = sum_i res_ji x_i + post_j y                     (k_post; int8 y with
//             per-token scales: k_post<true>)
//   coeffs    RMS-scaled 24-wide projection of the flattened row,
//             sigmoid pre/post, Sinkhorn res                          (k_persist / k_split, coeffs mode)
//   pre       h = RMSNorm(sum_i pre_i x_i) * gamma                    (k_pre)
//   fused     post -> coeffs' -> pre' with x' kept on chip            (k_persist / k_split, fused modes)
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

// One thread per (32-row k-step, fragment lane): it reads its 8 rows of the
// two columns it serves (n16 for blocks 0-2, 16 + n16 % 8 for blocks 3-4)
// once and writes its lane of all five blocks.
__global__ __launch_bounds__(256) void k_pack_phi(const float* __restrict__ phi, int C,
                                                  u32x4_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(4 * C / 32) * kWave;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  const int64_t q = idx >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int64_t k0 = q * 32 + g * 8;
  float t[5][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float* row = phi + (k0 + e) * kCoeffs;
    float hi, mid, lo;
    // blocks 0-2: hi, mid, lo of logit n16
    {
      const float p = row[n16];
      hi = bf16_round_f(p);
      const float r1 = p - hi;
      mid = bf16_round_f(r1);
      lo = bf16_round_f(r1 - mid);
      t[0][e] = hi;
      t[1][e] = mid;
      t[2][e] = lo;
    }
    // blocks 3-4: [hi | mid] and [lo | 0] of logit 16 + n16 % 8
    {
      const float p = row[16 + (n16 & 7)];
      hi = bf16_round_f(p);
      const float r1 = p - hi;
      mid = bf16_round_f(r1);
      lo = bf16_round_f(r1 - mid);
      t[3][e] = n16 < 8 ? hi : mid;
      t[4][e] = n16 < 8 ? lo : 0.0f;
    }
  }
#pragma unroll
  for (int b = 0; b < kPackBlocks; ++b) out[(q * kPackBlocks + b) * kWave + lane] = pack8(t[b]);
}

// hi, mid and lo of one fp32 value (their sum is the value for |v| >= 2^-100)
__device__ __forceinline__ void split3(float v, float& hi, float& mid, float& lo) {
  hi = bf16_round_f(v);
  const float r1 = v - hi;
  mid = bf16_round_f(r1);
  lo = bf16_round_f(r1 - mid);
}

// The projection of a broadcast stream summed over its routes, packed like
// k_pack_phi packs a projection of C rows: Phi[c][m] = ((phi[c][m] +
// phi[C + c][m]) + phi[2C + c][m]) + phi[3C + c][m] in fp32.  PACKED: the
// route values come from the 4-route packed layout (hi + mid + lo, exact in
// fp32), so both inputs give the same bits.  One thread per (32-row k-step,
// fragment lane), as in k_pack_phi.
template <bool PACKED>
__global__ __launch_bounds__(256) void k_pack_phi_sum(const float* __restrict__ phi, const u32x4_t* __restrict__ pk,
                                                      int C, u32x4_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(C / 32) * kWave;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  const int64_t q = idx >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int lo16 = 16 * g + (n16 & 7);  // block 3/4 lane of logit 16 + n16 % 8 (hi/lo; mid at + 8)
  float va[8], vb[8];  // route sums of logit n16 and of logit 16 + n16 % 8, rows 32q + 8g + e
#pragma unroll
  for (int e = 0; e < 8; ++e) va[e] = vb[e] = 0.0f;
  // every load of the four routes first (one memory round trip), then the
  // sums in route order
  u32x4_t fr[PACKED ? 4 : 1][6];
  float pr[PACKED ? 1 : 4][2][8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (PACKED) {
      const u32x4_t* f = pk + ((int64_t)j * (C / 32) + q) * (kPackBlocks * kWave);
      fr[j][0] = f[0 * kWave + lane];
      fr[j][1] = f[1 * kWave + lane];
      fr[j][2] = f[2 * kWave + lane];
      fr[j][3] = f[3 * kWave + lo16];
      fr[j][4] = f[3 * kWave + lo16 + 8];
      fr[j][5] = f[4 * kWave + lo16];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float* row = phi + ((int64_t)j * C + q * 32 + g * 8 + e) * kCoeffs;
        pr[j][0][e] = row[n16];
        pr[j][1][e] = row[16 + (n16 & 7)];
      }
    }
  }
  // (keeps the compiler from moving the loads between the sums below)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float ra[8], rb[8];
    if constexpr (PACKED) {
      float h0[8], m0[8], l0[8], h1[8], m1[8], l1[8];
      unpack8(fr[j][0], h0);
      unpack8(fr[j][1], m0);
      unpack8(fr[j][2], l0);
      unpack8(fr[j][3], h1);
      unpack8(fr[j][4], m1);
      unpack8(fr[j][5], l1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ra[e] = (h0[e] + m0[e]) + l0[e];
        rb[e] = (h1[e] + m1[e]) + l1[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ra[e] = pr[j][0][e];
        rb[e] = pr[j][1][e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      va[e] = j == 0 ? ra[e] : va[e] + ra[e];
      vb[e] = j == 0 ? rb[e] : vb[e] + rb[e];
    }
  }
  float t[5][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float hi, mid, lo;
    split3(va[e], hi, mid, lo);
    t[0][e] = hi;
    t[1][e] = mid;
    t[2][e] = lo;
    split3(vb[e], hi, mid, lo);
    t[3][e] = n16 < 8 ? hi : mid;
    t[4][e] = n16 < 8 ? lo : 0.0f;
  }
#pragma unroll
  for (int b = 0; b < kPackBlocks; ++b) out[(q * kPackBlocks + b) * kWave + lane] = pack8(t[b]);
}

// ===========================================================================
// Split-row kernel (a staggered pipeline over tiles).
//
// A tile holds TM tokens.  A token's row is spread over S = C / 128
// "splits", each owning 128 channels of all 4 routes.  Workgroup
// (stage k, split s) does three jobs in this order, each on another tile:
//
//   A  tile k: lane tid serves the 8 channels 8*(tid%16) of tokens
//      16p + tid/16 (sixteen lanes cover one 256-byte row segment).  It
//      computes x' with the post chain, stores it, stages it in LDS and on
//      the matrix cores (wave w: the 32-channel step w) forms the 24
//      projections of the flattened row (A = x' rows of 16 tokens, B =
//      packed projection fragments, the three bf16 terms in one
//      accumulator) and the route Gram matrix G_ij = sum_c x'_i x'_j
//      (A = rows (token, route) of 4 tokens, D = A A^T; the trace of G is
//      the sum of squares).  The 4 waves' partials are summed in LDS and the
//      tile partial [TM][34] goes to the workspace as tagged words.
//   R  tile k - D1: workgroup s reduces tokens m with m % S == s: it gathers
//      their S partials, sums them in split order (deterministic),
//      finalises the coefficients on one wave per token (Sinkhorn on 16
//      lanes) and, in the fused modes, publishes q_i = pre'_i * r_h first
//      (before the Sinkhorn iterations, which q does not need), where r_h
//      is the RMSNorm scale of g = sum_i pre'_i x'_i from the Gram matrix:
//      sum_c g^2 = pre'^T G pre'.
//   C  (fused modes) tile k - D2: the pre step.  It reads x' of its 128
//      channels back from x_out when phase A of the same split ran on the
//      same XCD (their shared L2 holds the stores), and otherwise loads x
//      and y again and recomputes x' with the post chain, bit for bit what
//      A stored; it waits for the tile's published q_i and writes
//      h = (sum_i q_i x'_i) * gamma as bf16 and/or MXFP8 (a 32-channel
//      block is 4 neighbouring lanes).
//
// R consumes what A of stage k - D1 produced and C what R of stage
// k - (D2 - D1) produced, each at the same point of an older workgroup's
// life, so with delays of a few stages (more than the spread of
// workgroup progress) nothing waits in steady state, and the inputs that C
// reads again are still in the caches.  The grid has tiles + D2 (fused) or
// tiles + D1 stages of S workgroups; the last stages only do R and C.  Stages are dispatched in blockIdx
// order and a job depends only on lower stages, so progress never depends
// on a later workgroup; the waits are bounded anyway.
//
// LDS layout of x': row = 4*token + route, sixteen 16-byte chunks per row,
// chunk k stored at k ^ ((token + 4*route) & 15).  The coalesced writes,
// the projection reads (16 tokens, one route, one chunk) and the Gram reads
// (4 tokens x 4 routes, one chunk) then each touch 16 distinct chunk
// positions: no bank conflicts.
//
// blockIdx -> (stage, split): the S workgroups of a stage are consecutive;
// when S is a multiple of 8 the split is interleaved over blockIdx mod 8, so
// that with the round-robin dispatch of workgroups over the 8 XCDs each XCD
// reads only 1/8 of the packed projection (which then stays in its L2).
//
// Communication between workgroups uses 64-bit words that carry a value and
// a tag: (float bits) | (tag << 32).  The tag of a launch is the
// workspace's launch epoch + 1, read by every workgroup when it starts; a
// reader polls the words it needs until their tags match, so no counter
// sits on the critical path and no cache write-back or invalidation is
// needed (the words are written and read with system scope, which bypasses
// the per-XCD caches, and an aligned 64-bit access is single-copy atomic,
// so a value is never seen with a wrong tag).  Stale words of earlier launches carry older tags whatever the
// shapes of those launches were.  Off the critical path, the last of a
// tile's final consumers counts the tile as done, and the one completing the
// last tile advances the epoch and clears the counter, so the workspace
// (counters at fixed offsets) is ready for the next launch of any shape.
// ===========================================================================
constexpr uint32_t kSpinLimit = 1u << 22;
// Reduce-scatter bounds, checked by the host when it makes the plan: a
// workgroup owns ntok = ceil(TM/S) <= 7 tokens (ntok * 34 <= 256 partial
// words) and one thread sums a run of at most kRunMax splits of one word
// (the kernel is instantiated for runs of up to 8 and up to kRunMax).
constexpr int kMaxTileTokensPerGroup = 8;

// Tagged words are exchanged between workgroups on different XCDs, whose L2
// caches are not kept coherent with each other: stores and loads use system
// scope (sc0 sc1), which writes through to memory and reads from it, so a
// poll never spins on a stale line of its own L2.
__device__ __forceinline__ void tagged_store(uint64_t* p, float v, uint32_t tag) {
  const uint64_t w = (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// XCD (accelerator complex die) the calling wave runs on: hardware register
// XCC_ID, bits 3:0.
__device__ __forceinline__ uint32_t xcd_id() { return (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u; }

__device__ __forceinline__ uint64_t tagged_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float tagged_value(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Every exchanged word of a launch with tag L carries 2 L + (g % 2), where
// g is the generation of its ring slot (0 where the layout is not a ring),
// so words of different launches never share a tag (until 2^31 launches
// have wrapped the epoch), whichever layout each launch used.
__device__ __forceinline__ uint32_t ring_tag(uint32_t tag, uint32_t gen) { return 2u * tag + (gen & 1u); }

__device__ __forceinline__ void store_sys32(void* p, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t load_sys32(const void* p) {
  return __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
}

// Appends token t to the workspace list of tokens whose fused pre is
// recomputed directly (fix_flagged).  The count is a tagged word: a count
// left by an earlier launch (older tag) counts as zero, so no launch has to
// clear it.  The entry is written through to memory (system scope), where
// the launch's last workgroup reads it.
__device__ __forceinline__ void flag_for_fix(const SplitArgs& a, uint32_t tag, int64_t t) {
  uint64_t old = __hip_atomic_load(a.fix_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t idx;
  for (;;) {
    const bool cur = (uint32_t)(old >> 32) == tag;
    const uint64_t nw = cur ? old + 1u : (((uint64_t)tag << 32) | 1u);
    if (__hip_atomic_compare_exchange_strong(a.fix_word, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
      idx = cur ? (uint32_t)old : 0u;
      break;
    }
  }
  if ((int64_t)idx < a.T) store_sys32(a.fix_list + idx, (uint32_t)t);
}

// DPP lane moves inside rows of 16 lanes (no LDS traffic): quad_perm swaps
// within groups of 4 lanes, row_ror rotates the 16-lane row.
#define MHC_DPP(v, ctrl) __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, false))
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowRor4 = 0x124;   // row_ror:4
constexpr int kDppRowRor8 = 0x128;   // row_ror:8

// Coefficients of one token on one wave.  sums: 24 projections, then the
// Gram matrix (fused) or the sum of squares (coeffs).  Lanes 0..15 carry
// res[j][i] (j = lane/4, i = lane%4), lanes 16..23 pre/post.  Row sums of
// the 4x4 matrix are sums over lane ^ {1, 2}, column sums over the 16-lane
// row rotated by 4, 8, 12.  Each normalisation multiplies by the reciprocal
// of (sum + eps).  Returns in every lane the value of coefficient
// slot(lane).  In the fused modes publish(q, pre, cancels), q_i = pre_i * r_h,
// runs before the Sinkhorn iterations: the pre step needs only q, so it does
// not wait for them; `cancels` says that the token's pre must be recomputed
// directly (gram_rms_factor).  bias_lane: bias[wave_bias_index(lane)],
// loaded by the caller ahead of time.
__device__ __forceinline__ int wave_bias_index(int lane) { return lane < 16 ? 8 + lane : (lane < 24 ? lane - 16 : 0); }
template <bool FUSED, class Publish>
__device__ __forceinline__ float finalize_wave(const float* sums, float bias_lane, int C, const Scalars& sc,
                                               int lane, Publish&& publish) {
  const float ss = FUSED ? ((sums[24] + sums[25]) + sums[26]) + sums[27] : sums[24];
  const float r = 1.0f / sqrtf(ss / (float)(kRoutes * C) + sc.hc_norm_eps);
  const int li = wave_bias_index(lane);
  const float l = r * sums[li] + bias_lane;
  const float sg = 1.0f / (1.0f + expf(-l));
  const float pp = (lane >= 20 && lane < 24) ? sc.hc_post_scale * sg : sg;
  float v = expf(l);
  if constexpr (FUSED) {
    const float p[4] = {__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pp), 16)),
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pp), 17)),
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pp), 18)),
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pp), 19))};
    bool cancels;
    const float rh = gram_rms_factor(sums + 24, p, C, sc.rmsnorm_eps, cancels);
    const float q[4] = {p[0] * rh, p[1] * rh, p[2] * rh, p[3] * rh};
    publish(q, p, cancels);
  }
  const float eps = sc.sinkhorn_eps;
  for (int it = 0; it < sc.sinkhorn_iters; ++it) {
    float rs = v + MHC_DPP(v, kDppQuadSwap1);
    rs = rs + MHC_DPP(rs, kDppQuadSwap2);
    v = v * __builtin_amdgcn_rcpf(rs + eps);
    float cs = v + MHC_DPP(v, kDppRowRor8);
    cs = cs + MHC_DPP(cs, kDppRowRor4);
    v = v * __builtin_amdgcn_rcpf(cs + eps);
  }
  return lane < 16 ? v : pp;
}

// Coefficients of four tokens on one wave, one token per 16-lane row, with
// the arithmetic of finalize_wave: lane k of a row carries res[k/4][k%4]
// of the row's token and, for k < 8, its pre (k < 4) or post (4 <= k < 8)
// weight.  The Sinkhorn row and column sums are the same row-local DPP
// moves, so the four rows run side by side.  sums: this lane's token.
// publish(q, pre, cancels) of the fused modes runs before the Sinkhorn iterations.
// BC: the stream is one [T][4C] row x0 broadcast to the routes, split into
// pseudo-routes (sums[24..27] are its sum of squares in four parts), so
// g = psum x0 with psum = ((pre0 + pre1) + pre2) + pre3, sum g^2 =
// psum^2 ss, and every q word is psum r_h (no cancellation is possible).
// bias: the bias vector, or this lane's two entries of it loaded beforehand
// (LaneBias), so that the finalisation waits for no memory load.
struct LaneBias {
  float p, r;  // bias[lane % 8], bias[8 + lane % 16]
};
__device__ __forceinline__ float bias_pw(const float* b, int kp) { return b[kp]; }
__device__ __forceinline__ float bias_pw(const LaneBias& b, int) { return b.p; }
__device__ __forceinline__ float bias_res(const float* b, int k) { return b[8 + k]; }
__device__ __forceinline__ float bias_res(const LaneBias& b, int) { return b.r; }
template <bool FUSED, bool BC = false, class Bias, class Publish>
__device__ __forceinline__ void finalize_rows(const float* sums, const Bias& bias, int C, const Scalars& sc,
                                              int lane, float& res, float& pp, Publish&& publish) {
  const int k = lane & 15, kp = lane & 7;
  const float ss = FUSED ? ((sums[24] + sums[25]) + sums[26]) + sums[27] : sums[24];
  const float r = 1.0f / sqrtf(ss / (float)(kRoutes * C) + sc.hc_norm_eps);
  const float lp = r * sums[kp] + bias_pw(bias, kp);
  const float sg = 1.0f / (1.0f + expf(-lp));
  pp = kp >= 4 ? sc.hc_post_scale * sg : sg;
  if constexpr (FUSED) {
    const int row0 = lane & 48;
    const float p[4] = {__shfl(pp, row0), __shfl(pp, row0 + 1), __shfl(pp, row0 + 2), __shfl(pp, row0 + 3)};
    if constexpr (BC) {
      const float psum = ((p[0] + p[1]) + p[2]) + p[3];
      const float qb = psum / sqrtf(psum * psum * ss / (float)(kRoutes * C) + sc.rmsnorm_eps);
      const float q[4] = {qb, qb, qb, qb};
      publish(q, p, false);
    } else {
      bool cancels;
      const float rh = gram_rms_factor(sums + 24, p, C, sc.rmsnorm_eps, cancels);
      const float q[4] = {p[0] * rh, p[1] * rh, p[2] * rh, p[3] * rh};
      publish(q, p, cancels);
    }
  }
  const float l = r * sums[8 + k] + bias_res(bias, k);
  float v = expf(l);
  const float eps = sc.sinkhorn_eps;
  for (int it = 0; it < sc.sinkhorn_iters; ++it) {
    float rs = v + MHC_DPP(v, kDppQuadSwap1);
    rs = rs + MHC_DPP(rs, kDppQuadSwap2);
    v = v * __builtin_amdgcn_rcpf(rs + eps);
    float cs = v + MHC_DPP(v, kDppRowRor8);
    cs = cs + MHC_DPP(cs, kDppRowRor4);
    v = v * __builtin_amdgcn_rcpf(cs + eps);
  }
  res = v;
}

constexpr int kCC = 128;  // channels per workgroup

__device__ __forceinline__ int xs_offset(int token, int route, int chunk) {
  // 16-byte units
  return (token * 4 + route) * 16 + (chunk ^ ((token + 4 * route) & 15));
}

// Gram slot of (e, j), e <= j: 00,11,22,33 -> 0..3, 01,02,03,12,13,23 -> 4..9
__device__ __forceinline__ int gram_slot(int e, int j) {
  if (e == j) return e;
  return e == 0 ? 3 + j : (e == 1 ? 5 + j : 9);
}

// Per-lane stream registers of one tile: x (then x') of 4 routes and y for
// the tokens 16p + tid/16, p < TM/16.
template <int NP>
struct TileRegs {
  u32x4_t x[NP][4];
  u32x4_t y[NP];
};

// y of a token's 8 channels at cl: packed bf16, or (YQ) the 8 int8 codes in
// words 0-1 and the token's binary32 scale in word 2
template <bool YQ, bool LAST_USE>
__device__ __forceinline__ u32x4_t load_y8(const SplitArgs& a, int64_t t, int cl) {
  if constexpr (YQ) {
    const uint64_t v = *reinterpret_cast<const uint64_t*>(a.y_q + t * (int64_t)a.C + cl);
    return u32x4_t{(uint32_t)v, (uint32_t)(v >> 32), __float_as_uint(a.y_scale[t]), 0u};
  } else {
    return ld16<LAST_USE>(a.y + t * (int64_t)a.C + cl);
  }
}

// the two y values of channel pair q (0..3) of a load_y8 result
template <bool YQ>
__device__ __forceinline__ void y_pair(const u32x4_t& v, int q, float& lo, float& hi) {
  if constexpr (YQ) {
    const float sc = __uint_as_float(v[2]);
    const uint32_t w = v[q >> 1] >> (16 * (q & 1));
    lo = (float)(int8_t)(uint8_t)w * sc;
    hi = (float)(int8_t)(uint8_t)(w >> 8) * sc;
  } else {
    lo = bf16_lo(v[q]);
    hi = bf16_hi(v[q]);
  }
}

// g = ((p0 x0 + p1 x1) + p2 x2) + p3 x3 in binary64: the product of an fp32
// weight and a bf16 value is exact there, so routes that cancel exactly give
// exactly 0 and nearly cancelling ones keep their leading bits.
__device__ __forceinline__ double combine_f64(const double* p, float x0, float x1, float x2, float x3) {
  double g = p[0] * (double)x0;
  g = __builtin_fma(p[1], (double)x1, g);
  g = __builtin_fma(p[2], (double)x2, g);
  g = __builtin_fma(p[3], (double)x3, g);
  return g;
}

// x' of 8 channels of token t, all 4 routes, from the inputs: the post chain
// of post_tile, bit for bit what x_out holds.  pw, rs: the token's post and
// res coefficients.
template <bool YQ>
__device__ __forceinline__ void xprime8(const SplitArgs& a, int64_t t, int c, const float* pw, const float* rs,
                                        float (*xp)[8]) {
  u32x4_t xin[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xin[i] = ld16(a.x + t * a.xts + (int64_t)i * a.xrs + c);
  const u32x4_t yv = load_y8<YQ, false>(a, t, c);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float xl[4] = {bf16_lo(xin[0][q]), bf16_lo(xin[1][q]), bf16_lo(xin[2][q]), bf16_lo(xin[3][q])};
    const float xh[4] = {bf16_hi(xin[0][q]), bf16_hi(xin[1][q]), bf16_hi(xin[2][q]), bf16_hi(xin[3][q])};
    float yl, yh;
    y_pair<YQ>(yv, q, yl, yh);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t o = pack_bf16x2(post_chain(pw[j], yl, &rs[4 * j], xl[0], xl[1], xl[2], xl[3]),
                                     post_chain(pw[j], yh, &rs[4 * j], xh[0], xh[1], xh[2], xh[3]));
      xp[j][2 * q] = bf16_lo(o);
      xp[j][2 * q + 1] = bf16_hi(o);
    }
  }
}

// The direct pre of the tokens a fused launch listed because their route
// combination cancels (gram_rms_factor): run once the list is complete (and
// the listed tokens' pre weights, written through to memory before the
// tokens' q words): by the last workgroup of a staged launch (NT = 256), and
// of a persistent launch with the MXFP8 epilogue (NT = 512), or by the last
// reduce workgroup of any other persistent launch (NT = 512).  Per token: x' recomputed from x, y and the post
// coefficients (inputs only, so nothing another XCD wrote is read), g in
// binary64, sum_c g^2 in binary64, then h and its MXFP8 blocks written; the
// pre step left these tokens' rows unwritten (the sign of q0).  A launch
// with no listed token only reads the count.
// (COPY: a separate instantiation for a second caller, so that the
// compiler's inlining of the first does not depend on it)
template <bool YQ, bool MX, int NT, int COPY = 0>
__device__ void fix_flagged(const SplitArgs& a, uint32_t tag, double* red, uint32_t first = 0, uint32_t stride = 1) {
  const int tid = threadIdx.x;
  const uint64_t w = __hip_atomic_load(a.fix_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  uint32_t n = (uint32_t)(w >> 32) == tag ? (uint32_t)w : 0u;
  if ((int64_t)n > a.T) n = (uint32_t)a.T;
  const int C = a.C, nch = C >> 3;
  for (uint32_t k = first; k < n; k += stride) {
    const int64_t t = load_sys32(a.fix_list + k);
    double p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = (double)__uint_as_float(load_sys32(a.coeffs_out + t * kCoeffs + i));
    float pw[4], rs[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = a.coeffs_in[t * kCoeffs + 4 + i];
#pragma unroll
    for (int i = 0; i < 16; ++i) rs[i] = a.coeffs_in[t * kCoeffs + 8 + i];
    double ss = 0.0;
    for (int j = tid; j < nch; j += NT) {
      float xp[4][8];
      xprime8<YQ>(a, t, 8 * j, pw, rs, xp);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double g = combine_f64(p, xp[0][e], xp[1][e], xp[2][e], xp[3][e]);
        ss = __builtin_fma(g, g, ss);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    double tot = red[0];
#pragma unroll
    for (int wv = 1; wv < NT / 64; ++wv) tot += red[wv];
    const double rh = 1.0 / sqrt(tot / (double)C + (double)a.sc.rmsnorm_eps);
    for (int j = tid; j < nch; j += NT) {
      float xp[4][8];
      xprime8<YQ>(a, t, 8 * j, pw, rs, xp);
      const float4* gp = reinterpret_cast<const float4*>(a.gamma + 8 * j);
      const float4 g0 = gp[0], g1 = gp[1];
      const float gmv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      float hv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        hv[e] = (float)(combine_f64(p, xp[0][e], xp[1][e], xp[2][e], xp[3][e]) * rh * (double)gmv[e]);
      const u32x4_t hb = pack8(hv);
      if (a.h != nullptr) st16(a.h + t * (int64_t)C + 8 * j, hb);
      if constexpr (MX) {
        // a 32-channel block is the chunks 4b .. 4b+3: lanes tid ^ {1, 2}
        float hr[8];
        unpack8(hb, hr);
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(hr[e]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
        const int ex = mx_scale_exponent(amax);
        const float scale = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-ex, ex <= 120
        const uint32_t w0 = e4m3_pack4(hr[0] * scale, hr[1] * scale, hr[2] * scale, hr[3] * scale);
        const uint32_t w1 = e4m3_pack4(hr[4] * scale, hr[5] * scale, hr[6] * scale, hr[7] * scale);
        *reinterpret_cast<u32x2_t*>(a.h_fp8 + t * (int64_t)C + 8 * j) = u32x2_t{w0, w1};
        if ((j & 3) == 0) a.h_scale[mx_scale_offset(t, j >> 2, C, a.scale_mfma != 0)] = (uint8_t)(ex + 127);
      }
    }
    __syncthreads();  // red[] is reused by the next token
  }
}

template <bool WITH_Y, int TM, bool LAST_USE, bool YQ = false>
__device__ __forceinline__ void load_stream(const SplitArgs& a, int64_t tok0, int cl, int tr, TileRegs<TM / 16>& R) {
  constexpr int NP = TM / 16;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t t = tok0 + p * 16 + tr;
    const bool valid = t < a.T;
    const uint16_t* xp = a.x + (valid ? t : 0) * a.xts + cl;
#pragma unroll
    for (int i = 0; i < 4; ++i) R.x[p][i] = valid ? ld16<LAST_USE>(xp + (int64_t)i * a.xrs) : u32x4_t{0, 0, 0, 0};
    if constexpr (WITH_Y) R.y[p] = valid ? load_y8<YQ, LAST_USE>(a, t, cl) : u32x4_t{0, 0, 0, 0};
  }
}

// x' of a tile, read back from x_out (last use)
template <int TM>
__device__ __forceinline__ void load_xprime(const SplitArgs& a, int64_t tok0, int cl, int tr, TileRegs<TM / 16>& R) {
  constexpr int NP = TM / 16;
  const int C = a.C;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t t = tok0 + p * 16 + tr;
    const bool valid = t < a.T;
    const uint16_t* xp = a.x_out + (valid ? t : 0) * (int64_t)(4 * C) + cl;
#pragma unroll
    for (int i = 0; i < 4; ++i) R.x[p][i] = valid ? ld16_stream(xp + (int64_t)i * C) : u32x4_t{0, 0, 0, 0};
  }
}

// post / res of the tile's tokens: thread tid < TM*5 fetches one float4
// (token tid/5, part tid%5) into a register, stored to LDS [TM][20] later,
// so that the fetch does not delay the issue of other loads.
template <int TM>
__device__ __forceinline__ float4 fetch_post_coeffs(const SplitArgs& a, int64_t tok0, int tid) {
  const int64_t t = tok0 + tid / 5;
  if (tid >= TM * 5 || t >= a.T) return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  return reinterpret_cast<const float4*>(a.coeffs_in + t * kCoeffs)[1 + tid % 5];
}
template <int TM>
__device__ __forceinline__ void store_post_coeffs(float4 v, int tid, float (*cfs)[20]) {
  if (tid >= TM * 5) return;
  float* d = &cfs[tid / 5][4 * (tid % 5)];
  d[0] = v.x;
  d[1] = v.y;
  d[2] = v.z;
  d[3] = v.w;
}

// x' = post chain of (x, y) in place, for the lane's tokens
template <int TM, bool YQ>
__device__ __forceinline__ void post_tile(TileRegs<TM / 16>& R, const float (*cfs)[20], int tr) {
  constexpr int NP = TM / 16;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int m = p * 16 + tr;
    float pw[4], rs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) pw[q] = cfs[m][q];
#pragma unroll
    for (int q = 0; q < 16; ++q) rs[q] = cfs[m][4 + q];
    u32x4_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float xl[4] = {bf16_lo(R.x[p][0][q]), bf16_lo(R.x[p][1][q]), bf16_lo(R.x[p][2][q]), bf16_lo(R.x[p][3][q])};
      const float xh[4] = {bf16_hi(R.x[p][0][q]), bf16_hi(R.x[p][1][q]), bf16_hi(R.x[p][2][q]), bf16_hi(R.x[p][3][q])};
      float yl, yh;
      y_pair<YQ>(R.y[p], q, yl, yh);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j][q] = pack_bf16x2(post_chain(pw[j], yl, &rs[4 * j], xl[0], xl[1], xl[2], xl[3]),
                              post_chain(pw[j], yh, &rs[4 * j], xh[0], xh[1], xh[2], xh[3]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) R.x[p][j] = o[j];
  }
}

// Four workgroups per CU (<= 128 VGPRs, 4 x 39.5 KB of LDS) when the reduce
// runs are short; long runs (hidden sizes above 7168) need more registers,
// and so does a launch by tickets (a short, latency-bound call, whose
// projection fragments are in registers with its stream).
// TK: a launch of one tile (at most 32 tokens, latency-bound), whose
// workgroups take their jobs by ticket, in the order they start (see
// below); its pre step recomputes x' (the workgroup that stored it runs at
// the same time, so the read-back path would seldom apply), phase A then
// neither waits for its x' stores nor announces them, and its projection
// fragments are loaded with its stream.  (Launches of 2 to 4 tiles by
// tickets, every phase A first, measured slower than the staged pipeline:
// 17.7 vs 17.0 us at 64 tokens, 25.6 vs 19.5 us at 128.)
template <int MODE, int TM, int RUN, bool TK>
__global__ __launch_bounds__(256, RUN <= 8 && !TK ? 4 : 2) void k_split(const SplitArgs a) {
  constexpr bool FUSED = mode_fused(MODE);
  constexpr bool MX = mode_mx(MODE);
  constexpr bool YQ = mode_yq(MODE);
  constexpr int W = 4, NV = kPartVals, NP = TM / 16, RB = TM / 16, NQ = TM / 4;
  constexpr int NVU = FUSED ? NV : 25;
  constexpr bool ONE = TK;
  // partial words per token in the workspace: [tiles][S][TM][PW], dense, so
  // that every store instruction writes whole lines
  constexpr int PW = NVU;
  // LDS: x' (TM*4 rows x 256 B), later reused for the wave partials and the
  // reduce-scatter run sums
  constexpr int XS_BYTES = TM * 4 * 256;
  constexpr int RED_BYTES = W * TM * NV * 4;
  constexpr int LDS_BYTES = XS_BYTES > RED_BYTES ? XS_BYTES : RED_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  __shared__ float cfs_a[FUSED ? TM : 1][20];
  __shared__ float cfs_c[FUSED ? TM : 1][20];
  __shared__ float fin[kMaxTileTokensPerGroup][NV];
  __shared__ float qs[FUSED ? TM : 1][4];
  __shared__ uint32_t s_tag, s_xdirect, s_job;
  u32x4_t* xs = reinterpret_cast<u32x4_t*>(lds);
  float* red = reinterpret_cast<float*>(lds);   // [W][TM][NV]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S;
  const int tiles = (int)a.tiles;
  int split, tA, tR, tC;
  if constexpr (ONE) {
    // A launch's workgroups start on the XCDs one after another (about half
    // a microsecond apart), so a job bound to blockIdx may wait for the last
    // XCD.  Here each workgroup takes a ticket in the order it starts, with
    // the launch epoch in the same 64-bit word (ticket in the low half, epoch
    // in the high half): tickets [0, S) run phase A of split t, the next
    // min(S, TM) the reduce of the tokens split t - S owns, the last S (fused
    // modes) the pre step of split t - S - min(S, TM).  A job waits only for
    // jobs of lower tickets, which have started.  The last ticket advances
    // the epoch and clears the ticket: every workgroup has read the epoch.
    static_assert(kWsEpoch == kWsTicket + 4 && kWsTicket % 8 == 0, "ticket and epoch share a 64-bit word");
    if (tid == 0) {
      uint64_t* lw = reinterpret_cast<uint64_t*>(a.epoch - 1);
      const uint64_t old = __hip_atomic_fetch_add(lw, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t next = (uint32_t)(old >> 32) + 1u;
      s_tag = next;
      s_job = (uint32_t)old;
      if ((uint32_t)old == gridDim.x - 1u)
        __hip_atomic_store(lw, (uint64_t)next << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // s_job, s_tag
    const int job = (int)s_job, nR = S < TM ? S : TM;
    tA = job < S ? 0 : -1;
    tR = job >= S && job < S + nR ? 0 : -1;
    tC = FUSED && job >= S + nR ? 0 : -1;
    split = tA >= 0 ? job : (tR >= 0 ? job - S : job - S - nR);
  } else {
    int stage;
    if ((S & 7) == 0) {
      const int per = S >> 3, b = (int)blockIdx.x, j = b >> 3;
      stage = j / per;
      split = (b & 7) * per + j % per;
    } else {
      stage = (int)(blockIdx.x / S);
      split = (int)(blockIdx.x % S);
    }
    tA = stage < tiles ? stage : -1;
    tR = (stage - a.d1 >= 0 && stage - a.d1 < tiles) ? stage - a.d1 : -1;
    tC = (FUSED && stage - a.d2 >= 0 && stage - a.d2 < tiles) ? stage - a.d2 : -1;
  }
  const int C = a.C;
  const int c0 = split * a.cs;
  const int c8 = tid & 15, tr = tid >> 4;
  const int cl = c0 + c8 * 8;  // this lane's first channel in A and C
  const int n16 = lane & 15, g = lane >> 4;
  const int chunk = wave * 4 + g;  // MFMA: 32-channel step `wave`, 8 channels per lane group

  // ---- issue the loads that do not depend on this workgroup's own work ----
  // A's stream (x, y of tile tA), the post coefficients of tiles tA and tC,
  // and R's gather of the partials of tile tR (written by workgroups of stage
  // tR, D1 stages earlier, normally complete by now; stale words are polled
  // again when R runs).
  if (!ONE && tid == 0) s_tag = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  TileRegs<NP> ra;
  if (tA >= 0) load_stream<FUSED, TM, true, YQ>(a, (int64_t)tA * TM, cl, tr, ra);
  uint64_t own = 0;
  if (!ONE && tid == 0 && tC >= 0) own = tagged_load(a.owner + (int64_t)tC * S + split);
  float4 cfa = make_float4(0.0f, 0.0f, 0.0f, 0.0f), cfc = cfa;
  if constexpr (FUSED) {
    if (tA >= 0) cfa = fetch_post_coeffs<TM>(a, (int64_t)tA * TM, tid);
    if (tC >= 0) cfc = fetch_post_coeffs<TM>(a, (int64_t)tC * TM, tid);
  }
  // R: workgroup `split` owns tokens split + kk*S, kk < ntok.  Each of its
  // ntok*34 partial words is summed over the S splits by RT threads, thread
  // r taking the run of splits [r*L, r*L + L); the RT run sums are added in
  // run order, so the total is a fixed-order sum.
  const int ntok = split < TM ? (TM - split + S - 1) / S : 0;
  const bool doR = tR >= 0 && ntok > 0;
  const int npair = ntok * NV;
  const int RT = npair == 0 ? 1 : (256 / npair < 1 ? 1 : (256 / npair > 8 ? 8 : 256 / npair));
  const int L = (S + RT - 1) / RT;
  const int pidx = tid / RT, rr = tid % RT;
  const int kk = pidx / NV, v = pidx % NV;
  const bool active = doR && pidx < npair && v < NVU;
  const int sp0 = rr * L, n = active ? (S - sp0 < L ? (S - sp0 > 0 ? S - sp0 : 0) : L) : 0;
  const uint64_t* gbase =
      a.partials + ((int64_t)(doR ? tR : 0) * S * TM + (int64_t)sp0 * TM + split + kk * S) * PW + v;
  const int64_t gstride = (int64_t)TM * PW;
  uint64_t w[RUN];
#pragma unroll
  for (int q = 0; q < RUN; ++q) w[q] = q < n ? tagged_load(gbase + q * gstride) : 0;
  // this lane's bias entry for the finalisation (loaded now, off its path)
  const float bias_lane = doR ? a.bias[wave_bias_index(lane)] : 0.0f;
  if constexpr (FUSED) {
    store_post_coeffs<TM>(cfa, tid, cfs_a);
    store_post_coeffs<TM>(cfc, tid, cfs_c);
  }
  // The pre step of tile tC reads back the x' that phase A of the same split
  // stored, when that workgroup ran on this XCD (their shared L2 holds the
  // stores); otherwise it recomputes x' from x and y.
  if (tid == 0)
    s_xdirect = !ONE && tC >= 0 && !a.recompute_x && (uint32_t)(own >> 32) == ring_tag(s_tag, 0) &&
                __float_as_uint(tagged_value(own)) == xcd_id();
  __syncthreads();  // s_tag, cfs, s_xdirect
  const uint32_t tag = s_tag;
  const uint32_t wtag = ring_tag(tag, 0);  // the tag of this launch's exchanged words
  const bool xdirect = s_xdirect != 0;

  // ---------------- A: post, statistics and projection of tile tA ----------------
  if (tA >= 0) {
    const int64_t tok0 = (int64_t)tA * TM;
    // projection fragments of the wave's 32-channel step, all four routes
    u32x4_t bfrag[4][kPackBlocks];
    auto load_bfrag = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t kstep = ((int64_t)j * a.prs + c0 + wave * 32) >> 5;
        const u32x4_t* bp = reinterpret_cast<const u32x4_t*>(a.phi_packed) + kstep * (kPackBlocks * kWave) + lane;
#pragma unroll
        for (int b = 0; b < kPackBlocks; ++b) bfrag[j][b] = bp[b * kWave];
      }
    };
    if constexpr (ONE) load_bfrag();
    if constexpr (FUSED) post_tile<TM, YQ>(ra, cfs_a, tr);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int m = p * 16 + tr;
      if constexpr (FUSED) {
        if (tok0 + m < a.T) {
          uint16_t* xo = a.x_out + (tok0 + m) * (int64_t)(4 * C) + cl;
#pragma unroll
          for (int j = 0; j < 4; ++j) st16(xo + (int64_t)j * C, ra.x[p][j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) xs[xs_offset(m, j, c8)] = ra.x[p][j];
    }
    // (otherwise the fragments are loaded now, in flight together while
    // the workgroup meets at the barrier)
    if constexpr (!ONE) load_bfrag();
    __syncthreads();  // x' staged

    f32x4_t acc[RB][2];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      acc[r][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      acc[r][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xs[xs_offset(r * 16 + n16, j, chunk)]);
#pragma unroll
        for (int b = 0; b < kPackBlocks; ++b)
          acc[r][b < 3 ? 0 : 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              av, __builtin_bit_cast(bf16x8_t, bfrag[j][b]), acc[r][b < 3 ? 0 : 1], 0, 0, 0);
      }
    }
    // (after the projection, so that the fragments are dead: fewer registers)
    // Gram matrices: groups of 4 tokens; lane l reads row l%16 = (token 4q + (l%16)/4, route l%4)
    float gv[NQ][4];
#pragma unroll
    for (int qg = 0; qg < NQ; ++qg) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xs[xs_offset(4 * qg + (n16 >> 2), n16 & 3, chunk)]);
      const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, av, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) gv[qg][e] = d[e];
    }
    __syncthreads();  // LDS x' no longer needed: reuse it for the wave partials

    // MFMA output: lane l holds column l%16 of rows 4*(l/16)+e.
#pragma unroll
    for (int r = 0; r < RB; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v1 = acc[r][1][e];
        const float mid = MHC_DPP(v1, kDppRowRor8);  // lane ^ 8 (rotation by 8 of a 16-lane row)
        const int row = r * 16 + 4 * g + e;
        red[(wave * TM + row) * NV + n16] = acc[r][0][e];
        if (n16 < 8) red[(wave * TM + row) * NV + 16 + n16] = v1 + mid;
      }
    }
    // Gram: useful lanes have (l/16) == (l%16)/4: token 4q + l/16, column route j = l%4, rows e
    if ((n16 >> 2) == g) {
      const int jr = n16 & 3;
#pragma unroll
      for (int qg = 0; qg < NQ; ++qg) {
        const int row = 4 * qg + g;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e <= jr) red[(wave * TM + row) * NV + 24 + gram_slot(e, jr)] = gv[qg][e];
      }
    }
    if constexpr (FUSED && !ONE) {
      // every wave's x' stores have reached the L2 before the owner word
      // (stored after this barrier) announces them
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();

    uint64_t* part = a.partials + ((int64_t)tA * S + split) * (TM * PW);
    for (int idx = tid; idx < TM * NV; idx += 256) {
      const int vv = idx % NV;
      if (vv >= PW) continue;
      float sum = ((red[idx] + red[TM * NV + idx]) + red[2 * TM * NV + idx]) + red[3 * TM * NV + idx];
      if constexpr (!FUSED) {
        if (vv == 24) {  // coeffs: only the trace of the Gram matrix
          const int b = idx - 24;
          sum = 0.0f;
#pragma unroll
          for (int ww = 0; ww < W; ++ww)
            sum += ((red[ww * TM * NV + b + 24] + red[ww * TM * NV + b + 25]) + red[ww * TM * NV + b + 26]) +
                   red[ww * TM * NV + b + 27];
        }
      }
      tagged_store(part + (idx / NV) * PW + vv, sum, wtag);
    }
    __syncthreads();  // LDS free for R
    if (FUSED && !ONE && tid == 0) tagged_store(a.owner + (int64_t)tA * S + split, __uint_as_float(xcd_id()), wtag);
  }

  // the loads of C (inputs only) are in flight while R runs
  TileRegs<NP> rc;
  float gm[8];
  if (tC >= 0) {
    if (xdirect) {
      load_xprime<TM>(a, (int64_t)tC * TM, cl, tr, rc);
    } else {
      load_stream<true, TM, true, YQ>(a, (int64_t)tC * TM, cl, tr, rc);
    }
    const float4* gp = reinterpret_cast<const float4*>(a.gamma + cl);
    const float4 g0 = gp[0], g1 = gp[1];
    gm[0] = g0.x; gm[1] = g0.y; gm[2] = g0.z; gm[3] = g0.w;
    gm[4] = g1.x; gm[5] = g1.y; gm[6] = g1.z; gm[7] = g1.w;
  }

  // ---------------- R: reduce-scatter of tile tR ----------------
  if (doR) {
    const int64_t tok0 = (int64_t)tR * TM;
    float* runs = reinterpret_cast<float*>(lds);  // [npair][RT]
    uint32_t it = 0;
    for (;;) {
      bool stale = false;
#pragma unroll
      for (int q = 0; q < RUN; ++q) stale |= q < n && (uint32_t)(w[q] >> 32) != wtag;
      if (!stale) break;
      __builtin_amdgcn_s_sleep(1);
      if (++it > kSpinLimit) {
        __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
#pragma unroll
      for (int q = 0; q < RUN; ++q)
        if (q < n && (uint32_t)(w[q] >> 32) != wtag) w[q] = tagged_load(gbase + q * gstride);
    }
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < RUN; ++q)
      if (q < n) sum += tagged_value(w[q]);
    if (pidx < npair) runs[pidx * RT + rr] = sum;
    __syncthreads();
    for (int p2 = tid; p2 < npair; p2 += 256) {
      float t2 = 0.0f;
      for (int q = 0; q < RT; ++q) t2 += runs[p2 * RT + q];
      fin[p2 / NV][p2 % NV] = t2;
    }
    __syncthreads();
    for (int k0 = 0; k0 < ntok; k0 += W) {
      const int kq = k0 + wave;
      if (kq < ntok) {
        const int m = split + kq * S;
        uint64_t* const qdst = a.publish + ((int64_t)tR * TM + m) * 4 + (lane & 3);
        const int64_t t = tok0 + m;
        const float cv = finalize_wave<FUSED>(fin[kq], bias_lane, a.rms_c, a.sc, lane,
                                              [=](const float* q, const float* pw, bool cancels)
                                                  __attribute__((always_inline)) {
                                                // a cancelling token: listed (and its pre weights written
                                                // through) before its q words, whose sign bit on q0 tells
                                                // the pre step to leave its h to the recomputation
                                                if (cancels && t < a.T) {
                                                  if (lane < 4) store_sys32(a.coeffs_out + t * kCoeffs + lane,
                                                                            __float_as_uint(pw[lane & 3]));
                                                  if (lane == 0) flag_for_fix(a, tag, t);
                                                  __builtin_amdgcn_s_waitcnt(0);
                                                }
                                                const float qv = q[lane & 3];
                                                if (lane < 4) tagged_store(qdst, (lane == 0 && cancels) ? -qv : qv, wtag);
                                              });
        if (t < a.T && lane < 24) a.coeffs_out[t * kCoeffs + (lane < 16 ? 8 + lane : lane - 16)] = cv;
      }
    }
  }

  // ---------------- C: pre of tile tC ----------------
  if constexpr (FUSED) {
    if (tC >= 0) {
      const int64_t tok0 = (int64_t)tC * TM;
      // (one tile: x' first, so that only the pre itself follows the q words)
      if (ONE && !xdirect) post_tile<TM, YQ>(rc, cfs_c, tr);
      if (tid < TM * 4) {
        const uint64_t* qp = a.publish + tok0 * 4 + tid;
        uint64_t qw = tagged_load(qp);
        uint32_t it = 0;
        while ((uint32_t)(qw >> 32) != wtag) {
          __builtin_amdgcn_s_sleep(1);
          if (++it > kSpinLimit) {
            __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          qw = tagged_load(qp);
        }
        (&qs[0][0])[tid] = tagged_value(qw);
      }
      if (!ONE && !xdirect) post_tile<TM, YQ>(rc, cfs_c, tr);
      __syncthreads();  // qs
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int m = p * 16 + tr;
        const int64_t t = tok0 + m;
        const bool valid = t < a.T;
        const float q0 = qs[m][0], q1 = qs[m][1], q2 = qs[m][2], q3 = qs[m][3];
        // a negative q0 marks a token whose h the launch's last workgroup
        // recomputes directly (fix_flagged): its stores are left to that
        const bool keep = valid && !__builtin_signbit(q0);
        float xv[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) unpack8(rc.x[p][i], xv[i]);
        float hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float vv = q0 * xv[0][e];
          vv = __builtin_fmaf(q1, xv[1][e], vv);
          vv = __builtin_fmaf(q2, xv[2][e], vv);
          vv = __builtin_fmaf(q3, xv[3][e], vv);
          hv[e] = vv * gm[e];
        }
        const u32x4_t hb = pack8(hv);
        if (a.h != nullptr && keep) st16_stream(a.h + t * (int64_t)C + cl, hb);
        if constexpr (MX) {
          // a 32-channel block is the 4 lanes c8 = 4b .. 4b+3
          float hr[8];
          unpack8(hb, hr);
          float amax = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(hr[e]));
          amax = __builtin_fmaxf(amax, MHC_DPP(amax, kDppQuadSwap1));
          amax = __builtin_fmaxf(amax, MHC_DPP(amax, kDppQuadSwap2));
          const int ex = mx_scale_exponent(amax);
          const float scale = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-ex, ex <= 120
          const uint32_t w0 = e4m3_pack4(hr[0] * scale, hr[1] * scale, hr[2] * scale, hr[3] * scale);
          const uint32_t w1 = e4m3_pack4(hr[4] * scale, hr[5] * scale, hr[6] * scale, hr[7] * scale);
          if (keep) {
            *reinterpret_cast<u32x2_t*>(a.h_fp8 + t * (int64_t)C + cl) = u32x2_t{w0, w1};
            if ((c8 & 3) == 0) a.h_scale[mx_scale_offset(t, cl >> 5, C, a.scale_mfma != 0)] = (uint8_t)(ex + 127);
          } else if (!valid && a.scale_mfma && t < ((a.T + 15) & ~(int64_t)15) && (c8 & 3) == 0) {
            // a padding row of the last 16-row block: its h is all zero (x'
            // rows past T load as 0), so its scale byte is 0
            a.h_scale[mx_scale_offset(t, cl >> 5, C, true)] = (uint8_t)(ex + 127);
          }
        }
      }
    }
  }

  // ---------------- leave ----------------
  // The last of a tile's S final consumers (C in the fused modes, R in the
  // coeffs mode) counts the tile done; the one that completes the last tile
  // advances the launch epoch.
  // In the fused modes that workgroup then recomputes the pre of the tokens
  // whose route combination cancels (every tile's pre steps have run, so the
  // list is complete).
  // (By tickets: the epoch advanced with the last ticket, and the pre step
  // of split 0 recomputes the listed tokens as soon as its own rows are
  // out, having seen every token's q words, which follow their listing.)
  if constexpr (ONE) {
    if constexpr (FUSED) {
      if (tC >= 0 && split == 0) {
        __syncthreads();  // qs, LDS free
        fix_flagged<YQ, MX, 256>(a, tag, reinterpret_cast<double*>(lds));
      }
    }
    return;
  }
  const int tLeave = FUSED ? tC : tR;
  if (tLeave >= 0) {
    __syncthreads();
    if (tid == 0) {
      uint32_t last = 0;
      const uint32_t old = __hip_atomic_fetch_add(a.dep + tLeave, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == (uint32_t)S - 1u) {
        __hip_atomic_store(a.dep + tLeave, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t done = __hip_atomic_fetch_add(a.tiles_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == a.tiles - 1u) {
          __hip_atomic_store(a.tiles_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last = 1;
        }
      }
      s_xdirect = last;  // (no longer needed for its first use: reused as the flag)
    }
    if constexpr (FUSED) {
      __syncthreads();
      if (s_xdirect != 0) fix_flagged<YQ, MX, 256>(a, tag, reinterpret_cast<double*>(lds));
    }
  }
}

// ===========================================================================
// Persistent split-row kernel (fused modes and coeffs, long launches).
//
// One workgroup of 512 threads per CU, all resident at once:
//   * S*L "stream" workgroups: workgroup (split s, lane r) owns the 128
//     channels of split s and the tiles t = r, r + L, r + 2L, ...  Its slice
//     of the packed projection (72 KB: block 4 keeps only its 32 used lanes)
//     is copied to LDS once.  A tile's 32 tokens form two row blocks of 16;
//     the four waves of row block b (waves 4b .. 4b+3, one per SIMD) take
//     the four 32-channel steps of the split.  Every lane works in the
//     operand layout of v_mfma_f32_16x16x32_bf16: lane l holds token l%16
//     of its row block and channels 8*(l/16) .. +7 of its step, for all four
//     routes, so its x' registers are directly the A operands of the
//     projection (B = packed projection fragments from LDS) and of the Gram
//     products x'_a x'_b^T, whose diagonals are the route Gram entries.
//     Per tile and row block there are two phases:
//       P (vector ALU): partial sums of the previous tile, loads of the next
//         tile's y and coefficients, the pre step of tile t_{i-D} from x'
//         kept in registers since its own phase P, the post of tile t_i,
//         x' and h out;
//       M (matrix cores): asynchronous global->LDS copy of tile t_{i+2}'s x
//         slice, projection and Gram of tile t_i, fold of the four steps
//         through LDS, then the post coefficients and q words of the next
//         tile to LDS.
//     The two row blocks run half an iteration apart: while one runs P,
//     the other runs M, so each SIMD has one wave on its vector ALU and one
//     on its matrix core between the two barriers of an iteration.
//     The coefficients-only mode has neither post nor x' ring: its stream
//     workgroups keep x in registers three tiles ahead (whole-line loads,
//     turned into the operand layout through an LDS stage) and run both
//     row blocks in step.  The broadcast mode (kModeBcast) is the fused
//     pipeline without post on the pseudo-routes of a [T][C] input x0: x'
//     is x0, and the pre step writes the four pseudo-routes' channels of h.
//   * 32 to 64 "reduce" workgroups gather the S partial rows of 8 tokens at
//     a time (16 in the broadcast mode, a whole tile in the coefficients-only
//     mode), finalise their coefficients (four tokens per wave, one per
//     16-lane row) and publish q_i = pre'_i * r_h.
// Stream workgroups wait for q words published by reduce workgroups, which
// wait for partials of stream workgroups, so the launch needs all of its
// workgroups resident together (the host sizes L from the CU count; every
// wait is bounded and sets the workspace error word on expiry).  Nothing is
// read back from x_out: the pre step uses the x' registers, so the HBM
// traffic is the algorithmic one plus the partial and q words.
// ===========================================================================
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};
template <int N>
struct IntC {
  static constexpr int value = N;
};
constexpr int kPersistThreads = 512;
constexpr int kPersistTM = 32;
// Iterations between the post and the pre step of a tile: 7 (the x' of 7
// tiles held in registers, 251-256 VGPRs with no spill at two waves per
// SIMD), or 6 with the MXFP8 epilogue, which measured faster there.
constexpr int persist_depth(int mode) { return mode_mx(mode) ? 6 : 7; }
constexpr uint32_t kPersistSpinLimit = 1u << 18;
constexpr int kPersistMaxS = 64;  // splits per row the reduce threads can gather
constexpr int kCoeffsAhead = 3;   // coefficients-only pass: tiles of x held in registers ahead
// LDS projection fragments of one (route, 32-channel step): blocks 0-3 whole
// (64 lanes each) and the 32 lanes of block 4 whose column is < 8 (the rest
// of block 4 is zero), in 16-byte units.
constexpr int kPhiFrag = 4 * kWave + kWave / 2;
// 16-byte chunks of one row block's x slice: 16 tokens x 4 routes x 16
constexpr int kHalfChunks = 16 * 4 * 16;
// The fused passes keep their partial and q words in a ring of R = kRingK * L
// tiles (L stream workgroups per split): tile t uses slot t % R.  Stream
// workgroup lane r's tiles t = r + L i take slot r + L (i % kRingK), and the
// units of tiles t and t + R meet the same reduce workgroup (R is a multiple
// of 8 and a reduce workgroup owns every 32nd unit of 4 per tile).  The
// release flag and the q words of tile t carry the tag
// 2 * launch_tag + (t / R) % 2, so the flag or q word an older tile of the
// same slot left behind never passes as fresh (the partial values
// themselves carry no tag: they are read only after their flag).  Reuse is
// safe because of the q-word chain: a stream workgroup stores tile t_{i-1}'s
// partial values in phase P(i) only after it has seen the q words of tile
// t_{i-D-1}, which the reduce publishes after gathering every split's values
// of that tile; kRingK >= D + 1 then keeps a slot's old tile gathered before
// it is overwritten, and likewise its q words read before new ones land.
// The flag of tile t_{i-1} follows in phase P(i+1), so the old tile's flag
// has been read too.

// Whether a bounded wait of the launch has expired (read from memory; the
// polls look at it every 16th round only, so that a poll round costs one
// load latency).
__device__ __forceinline__ bool error_seen(uint32_t* err) {
  return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0u;
}

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Workgroup barrier for the persistent loop: waits for this wave's LDS
// operations, then s_barrier.  The text argument only keeps two otherwise
// identical barriers apart in the compiled code.
#define MHC_GROUP_BARRIER(where) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier ; " where ::: "memory")

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Asynchronous copy of 16 bytes per lane from global memory into LDS: lane l
// writes LDS bytes [base + 16 l, base + 16 l + 16), base uniform over the
// wave.  Written as inline assembly so that the compiler neither counts nor
// waits for it: callers wait with an explicit vmcnt, and the compiler's own
// waits for other loads only get more conservative from the uncounted ops.
// Non-temporal: every x line is read once, whole, by one wave.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
}

// The same copy with the default cache policy, for data that other
// workgroups of the XCD read too (the projection slice).
__device__ __forceinline__ void lds_dma16_shared(const void* src, uint32_t base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
}

// Buffer resource over [base, base + bytes): the hardware drops stores at
// offsets past the end, so a store to a row past T needs no branch (raw
// buffer, gfx9 resource word 3).
// cache-policy operand of a buffer load with system scope (sc0 sc1), which
// sees the system-scope stores of other workgroups
constexpr int kCachePolicySystem = 1 | 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// The persistent kernel's loads and stores of y, h and x_out use the default
// cache policy: a wave covers 64 bytes of each of 16 rows, half of a
// 128-byte line whose other half a neighbouring wave reads or writes.  With
// the non-temporal policy the halves leave the L2 separately (measured: 29%
// more bytes written to memory, and a slower pass).

template <int MODE>
__global__ __launch_bounds__(kPersistThreads, 1) void k_persist(const SplitArgs a) {
  constexpr bool FUSED = mode_fused(MODE);
  constexpr bool YQ = mode_yq(MODE);
  constexpr bool MX = mode_mx(MODE);
  constexpr bool BC = mode_bc(MODE);
  constexpr bool U16 = mode_u16(MODE);  // 16-token reduce units
  static_assert(!BC || (FUSED && !MX && !YQ), "the broadcast pass is the bf16 fused pipeline without post");
  static_assert(!U16 || (FUSED && !YQ && !MX), "16-token reduce units: the bf16 fused modes");
  constexpr int TM = kPersistTM, NV = kPartVals, D = persist_depth(MODE);
  static_assert(kRingK >= D + 1, "a ring slot is reused only after its tile was gathered");
  // LDS: projection slice [4 routes][4 steps][kPhiFrag] x 16 B; x slots
  // [2][row block][token][route][16 chunks] x 16 B (chunk c of token t at
  // position c ^ (t % 16), so that the 16 tokens a wave reads at once hit
  // distinct banks); wave partials; post coefficients; q words; gamma.
  // The partial values are [ring slot][S][TM][NV] binary32 words, or
  // [ring slot][S][TM][kCoeffsWords] in the coefficients-only mode, each
  // (slot, split, row block) released by one tagged flag: every store
  // instruction writes whole lines (a system-scope store that covers part
  // of a line measured several times slower per byte).
  __shared__ __attribute__((aligned(16))) u32x4_t phi_lds[16 * kPhiFrag + 1];
  // (the coefficients-only mode has one stage per row block instead of the
  // slot pairs: [1][row block][row][16 chunks], chunk c of token t at c ^ t)
  __shared__ __attribute__((aligned(16))) u32x4_t xslot[FUSED ? 2 : 1][2][kHalfChunks];
  // [wave][token of its row block][projection, Gram] | coefficients only:
  // [buffer][wave][token, word]
  __shared__ float red[FUSED ? 8 : 2][FUSED ? 16 : 8][FUSED ? NV : 16 * kCoeffsWords];
  __shared__ float cfs[FUSED ? TM : 1][20];
  __shared__ float qs[FUSED ? TM : 1][4];
  __shared__ float gam[FUSED ? (BC ? 4 * kCC : kCC) : 1];
  __shared__ uint32_t s_last;  // this workgroup left last
  float* finw = reinterpret_cast<float*>(&xslot[0][0][0]);  // reduce workgroups: [2][8][NV] or [TM][NV] sums

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, C = a.C, L = a.lanes;
  const int tiles = (int)a.tiles;
  const uint32_t tag = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const int nstream = S * L;

  if ((int)blockIdx.x >= nstream) {
    // ------------------------- reduce workgroup -------------------------
    // Work unit u = 8 tokens: tile u / 4, tokens 8 (u % 4) .. + 7 (one half
    // of a row block, whose partial words arrive together).  Reduce
    // workgroup j owns the units j, j + R, ... (R reduce workgroups).
    // Waves 2-7 gather: thread v < 8 NV sums value v of the unit (a
    // contiguous run in every split's [TM][NV] partial) over the S splits in
    // split order, in one pass, once the unit's release flags are in.  Waves
    // 0-1 finalise the previous unit meanwhile, four tokens per wave (one per
    // 16-lane row); the sums are double-buffered in LDS.  (The
    // coefficients-only mode takes whole tiles per round instead, its sums
    // as [TM][NV] in LDS.)
    const int j = (int)blockIdx.x - nstream;
    const int nred = (int)gridDim.x - nstream;
    const int nunits = tiles * (TM / 8);
    const int64_t pstride = (int64_t)TM * (FUSED ? NV : kCoeffsWords);  // one split's partial tile
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int v = tid - 128;  // gather thread's word
    const bool act = wv >= 2 && v < 8 * NV;
    uint32_t want = ring_tag(tag, 0);  // the tag the flags of the unit being gathered carry
    if constexpr (!FUSED) {
      // Coefficients only: nothing waits on the result but the end of the
      // launch, so whole tiles per round (all threads gather, then every
      // wave finalises four tokens) give more tokens per round.
      // The partial values live in a ring of cring tiles (coeffs_ring_tiles:
      // kCoeffsRingTilesWide at <= 16 splits, else kCoeffsRingTiles): tile t
      // in slot t % cring, generation t / cring.  The ring is a multiple of
      // the reduce workgroup count, so every tile of a slot is gathered here,
      // in order; once a tile's values are in, the slot's release word gets
      // its generation (the full number, in the value field), and stream
      // workgroups wait for it before refilling the slot.
      static_assert(kCoeffsRingTiles % 32 == 0 && kCoeffsRingTilesWide % 64 == 0, "one reduce workgroup per slot");
      // The partial values are plain binary32 words, released per (tile,
      // split, row block) by a tagged flag: every wave polls the 2 S flags
      // of a tile (lane k: split k, both row blocks), then loads the values
      // with system scope, after the flags.
      const float* pf = reinterpret_cast<const float*>(a.partials);
      auto tile_flags_in = [&](int t, auto kRing) __attribute__((always_inline)) {
        constexpr int cring = decltype(kRing)::value;
        const uint32_t wt = ring_tag(tag, (uint32_t)(t / cring));
        const uint64_t* fb = a.pflag + (int64_t)(t % cring) * S * 2;
        const uint64_t f0 = lane < S ? tagged_load(fb + 2 * lane) : 0;
        const uint64_t f1 = lane < S ? tagged_load(fb + 2 * lane + 1) : 0;
        return __builtin_amdgcn_ballot_w64(lane < S && ((uint32_t)(f0 >> 32) != wt || (uint32_t)(f1 >> 32) != wt)) == 0;
      };
      auto wait_tile = [&](int t, auto kRing) __attribute__((always_inline)) {
        if (!tile_flags_in(t, kRing)) {
          uint32_t it = 0;
          do {
            __builtin_amdgcn_s_sleep(1);
            if (++it > kPersistSpinLimit || ((it & 15u) == 0u && error_seen(a.err))) {
              __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          } while (!tile_flags_in(t, kRing));
        }
        // the value loads stay behind the flag loads they depend on
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      };
      // finalise tile t from the sums in LDS (every wave four tokens), then
      // the coefficients out
      auto finalize_tile = [&](int t) __attribute__((always_inline)) {
        const int ml = 4 * wv + (lane >> 4), kk = lane & 15;
        const int64_t tok = (int64_t)t * TM + ml;
        float res, pp;
        finalize_rows<false>(finw + ml * NV, a.bias, a.rms_c, a.sc, lane, res, pp,
                             [](const float*, const float*, bool) {});
        if (tok < a.T) {
          a.coeffs_out[tok * kCoeffs + 8 + kk] = res;
          if (kk < 8) a.coeffs_out[tok * kCoeffs + kk] = pp;
        }
      };
      if (S <= 16) {
        constexpr int cring = kCoeffsRingTilesWide;
        using Ring = IntC<kCoeffsRingTilesWide>;
        // Few splits (a broadcast stream on pseudo-routes): thread v takes
        // the words v and v + 512 of the tile's TM * 25, both in one round
        // of loads, and the next tile's loads are issued before this tile
        // is finalised, so the gather latency overlaps the finalisation.
        constexpr int NWT = TM * kCoeffsWords;  // 800
        float w0[16], w1[16];
        const bool has1 = tid + kPersistThreads < NWT;
        // the next tile's values, loaded once its flags are in (those of the
        // first tile are waited for here; later ones after a finalisation)
        auto issue = [&](int t) __attribute__((always_inline)) {
          wait_tile(t, Ring{});
          const float* base = pf + (int64_t)(t % cring) * S * pstride + tid;
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            w0[k] = k < S ? __uint_as_float(load_sys32(base + k * pstride)) : 0.0f;
            w1[k] = k < S && has1 ? __uint_as_float(load_sys32(base + k * pstride + kPersistThreads)) : 0.0f;
          }
        };
        auto settle = [&](int) __attribute__((always_inline)) {
          float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            s0 += k < S ? w0[k] : 0.0f;
            s1 += k < S ? w1[k] : 0.0f;
          }
          finw[(tid / kCoeffsWords) * NV + tid % kCoeffsWords] = s0;
          if (has1) {
            const int v1 = tid + kPersistThreads;
            finw[(v1 / kCoeffsWords) * NV + v1 % kCoeffsWords] = s1;
          }
        };
        if (j < tiles) issue(j);
        for (int t = j; t < tiles; t += nred) {
          settle(t);
          __syncthreads();  // the tile's sums (every gather load has returned)
          if (tid == 0)
            tagged_store(a.release + t % cring, __uint_as_float((uint32_t)(t / cring)),
                         ring_tag(tag, 0));
          if (t + nred < tiles) issue(t + nred);
          finalize_tile(t);
          __syncthreads();  // this tile's sums are read
        }
      } else
      for (int t = j; t < tiles; t += nred) {
        constexpr int cring = kCoeffsRingTiles;
        const int slot = t % cring;
        const uint32_t gen = (uint32_t)(t / cring);
        wait_tile(t, IntC<kCoeffsRingTiles>{});
        for (int w = tid; w < TM * kCoeffsWords; w += kPersistThreads) {
          const int wo = (w / kCoeffsWords) * NV + w % kCoeffsWords;  // (token, word) in the [TM][NV] sums
          const float* vb = pf + (int64_t)slot * S * pstride + w;
          float f[kPersistMaxS];
#pragma unroll
          for (int k = 0; k < kPersistMaxS; ++k) f[k] = k < S ? __uint_as_float(load_sys32(vb + k * pstride)) : 0.0f;
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < kPersistMaxS; ++k) acc += k < S ? f[k] : 0.0f;
          finw[wo] = acc;
        }
        __syncthreads();  // the tile's sums (every gather load has returned)
        if (tid == 0) tagged_store(a.release + slot, __uint_as_float(gen), ring_tag(tag, 0));
        finalize_tile(t);
        __syncthreads();  // this tile's sums are read
      }
    } else if constexpr (U16) {
      // 16-token units (the broadcast pass, and kModeUnit16 at few splits):
      // one row block, released by one flag per split.  Waves 4-7 gather
      // unit u + nred (thread v sums the words v and v + 256, and wave 4
      // also v + 512, of the unit's 16 NV over the S splits, with
      // system-scope buffer loads all issued before the first is waited
      // for; past the S splits the buffer's range check returns zeros) while
      // waves 0-3 finalise unit u, four tokens per wave.
      const int R = kRingK * L;
      const float* pf = reinterpret_cast<const float*>(a.partials);
      const int nunits = tiles * 2;
      const int v = tid - 256;
      auto flags_in = [&](const uint64_t* fb) __attribute__((always_inline)) {
        const uint64_t f = lane < S ? tagged_load(fb + 2 * lane) : 0;
        return __builtin_amdgcn_ballot_w64(lane < S && (uint32_t)(f >> 32) != want) == 0;
      };
      auto gather = [&](int u, float* fin, auto kMax) __attribute__((always_inline)) {
        constexpr int KM = decltype(kMax)::value;  // splits the loads cover (>= S)
        const int tu = u >> 1;
        want = ring_tag(tag, (uint32_t)(tu / R));
        const uint64_t* fb = a.pflag + (int64_t)(tu % R) * S * 2 + (u & 1);
        if (!flags_in(fb)) {
          uint32_t it = 0;
          do {
            __builtin_amdgcn_s_sleep(1);
            if (++it > kPersistSpinLimit || ((it & 15u) == 0u && error_seen(a.err))) {
              __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          } while (!flags_in(fb));
        }
        // the value loads stay behind the flag loads they depend on
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc(pf + (int64_t)(tu % R) * S * pstride + (u & 1) * 16 * NV, (uint32_t)(S * pstride * 4));
        float f0[KM], f1[KM];
#pragma unroll
        for (int k = 0; k < KM; ++k) {
          f0[k] = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)((k * pstride + v) * 4), 0, kCachePolicySystem));
          f1[k] = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)((k * pstride + v + 256) * 4), 0, kCachePolicySystem));
        }
        float s2 = 0.0f;
        if (wv == 4) {
          const bool has2 = v + 512 < 16 * NV;
          float f2[KM];
#pragma unroll
          for (int k = 0; k < KM; ++k)
            f2[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rs, has2 ? (uint32_t)((k * pstride + v + 512) * 4) : 0x7ffffff0u, 0, kCachePolicySystem));
#pragma unroll
          for (int k = 0; k < KM; ++k) s2 += f2[k];
          if (has2) fin[v + 512] = s2;
        }
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int k = 0; k < KM; ++k) {
          s0 += f0[k];
          s1 += f1[k];
        }
        fin[v] = s0;
        fin[v + 256] = s1;
      };
      auto gather_unit = [&](int u, float* fin) __attribute__((always_inline)) {
        if (S <= 16) {
          gather(u, fin, IntC<16>{});
        } else {
          gather(u, fin, IntC<kPersistMaxS / 2>{});
        }
      };
      if (j < nunits && wv >= 4) gather_unit(j, finw);
      const LaneBias lb = wv < 4 ? LaneBias{a.bias[lane & 7], a.bias[8 + (lane & 15)]} : LaneBias{0.0f, 0.0f};
      __syncthreads();
      int k = 0;
      for (int u = j; u < nunits; u += nred, ++k) {
        float* fin = finw + (k & 1) * (16 * NV);  // this unit's sums
        if (wv < 4) {
          // token 4 wave + r of the unit on lanes 16r .. 16r + 15
          const int ml = 4 * wv + (lane >> 4), kk = lane & 15;
          const int tu = u >> 1;
          const int64_t tok = (int64_t)tu * TM + (u & 1) * 16 + ml;
          const int64_t ptok = (int64_t)(tu % R) * TM + (u & 1) * 16 + ml;  // ring slot of the q words
          const uint32_t qtag = ring_tag(tag, (uint32_t)(tu / R));
          float res, pp;
          finalize_rows<true, BC>(fin + ml * NV, lb, BC ? a.rms_c : C, a.sc, lane, res, pp,
                                  [&](const float* q, const float* pw, bool cancels) __attribute__((always_inline)) {
                                    // (as in the 8-token units below: a cancelling token is
                                    // listed before its q words, whose sign bit on q0 marks it)
                                    if (cancels && tok < a.T) {
                                      if (kk < 4)
                                        store_sys32(a.coeffs_out + tok * kCoeffs + kk,
                                                    __float_as_uint(kk == 0 ? pw[0] : kk == 1 ? pw[1] : kk == 2 ? pw[2] : pw[3]));
                                      if (kk == 0) flag_for_fix(a, tag, tok);
                                      __builtin_amdgcn_s_waitcnt(0);
                                    }
                                    if (kk < 4)
                                      tagged_store(a.publish + ptok * 4 + kk,
                                                   kk == 0 ? (cancels ? -q[0] : q[0]) : kk == 1 ? q[1] : kk == 2 ? q[2] : q[3],
                                                   qtag);
                                  });
          if (tok < a.T) {
            a.coeffs_out[tok * kCoeffs + 8 + kk] = res;
            if (kk < 8) a.coeffs_out[tok * kCoeffs + kk] = pp;
          }
        } else if (u + nred < nunits) {
          gather_unit(u + nred, finw + ((k + 1) & 1) * (16 * NV));
        }
        __syncthreads();  // the next unit's sums are in; this unit's are read
      }
      // the last reduce workgroup recomputes the listed tokens (bf16 h; as
      // in the 8-token units below)
      if constexpr (!MX && !BC) {
        if (tid == 0) {
          uint32_t* rd = reinterpret_cast<uint32_t*>(a.fix_word + 1);
          uint32_t last = 0;
          const uint32_t done = __hip_atomic_fetch_add(rd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (done == (uint32_t)nred - 1u) {
            __hip_atomic_store(rd, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = 1;
          }
          s_last = last;
        }
        __syncthreads();
        if (s_last != 0) {
          const SplitArgs* ap = (const SplitArgs*)__builtin_amdgcn_kernarg_segment_ptr();
          asm volatile("" : "+s"(ap));
          fix_flagged<YQ, false, kPersistThreads, 1>(*ap, tag, reinterpret_cast<double*>(&red[0][0][0]));
        }
      }
    } else {
      // The fused pass's partial values are plain binary32 words, released
      // per (tile, split, row block) by a tagged flag that the stream
      // workgroup stores once the values are complete in memory: the wave
      // polls the S flags of a unit's row block (lane k: split k), then
      // loads the values with system scope, after the flags.
      const int R = kRingK * L;
      const float* pf = reinterpret_cast<const float*>(a.partials);
      auto flags_in = [&](const uint64_t* fb) __attribute__((always_inline)) {
        const uint64_t f = lane < S ? tagged_load(fb + 2 * lane) : 0;
        return __builtin_amdgcn_ballot_w64(lane < S && (uint32_t)(f >> 32) != want) == 0;
      };
      auto gather = [&](int u, float* fin) __attribute__((always_inline)) {
        const int tu = u >> 2;
        want = ring_tag(tag, (uint32_t)(tu / R));
        const uint64_t* fb = a.pflag + (int64_t)(tu % R) * S * 2 + ((u & 3) >> 1);
        if (!flags_in(fb)) {
          uint32_t it = 0;
          do {
            __builtin_amdgcn_s_sleep(1);
            // bounded: a wait that expires sets the error word, and every
            // other wait of the launch gives up as soon as it sees it
            if (++it > kPersistSpinLimit || ((it & 15u) == 0u && error_seen(a.err))) {
              __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          } while (!flags_in(fb));
        }
        // the value loads stay behind the flag loads they depend on
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const float* vb = pf + (int64_t)(tu % R) * S * pstride + (u & 3) * 8 * NV + (act ? v : 0);
        float f[kPersistMaxS];
#pragma unroll
        for (int k = 0; k < kPersistMaxS; ++k)
          f[k] = act && k < S ? __uint_as_float(load_sys32(vb + k * pstride)) : 0.0f;
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < kPersistMaxS; ++k) acc += k < S ? f[k] : 0.0f;
        if (v >= 0 && v < 8 * NV) fin[v] = act ? acc : 0.0f;
      };
      if (j < nunits && wv >= 2) gather(j, finw);
      // the finalising waves' bias entries, loaded once (so that no round's
      // finalisation waits for a memory load)
      const LaneBias lb = wv < 2 ? LaneBias{a.bias[lane & 7], a.bias[8 + (lane & 15)]} : LaneBias{0.0f, 0.0f};
      __syncthreads();
      int k = 0;
      for (int u = j; u < nunits; u += nred, ++k) {
        float* fin = finw + (k & 1) * (8 * NV);  // this unit's sums
        if (wv < 2) {
          // token 4 wave + r of the unit on lanes 16r .. 16r + 15
          const int ml = 4 * wv + (lane >> 4), kk = lane & 15;
          const int tu = u >> 2;
          const int64_t tok = (int64_t)tu * TM + (u & 3) * 8 + ml;
          const int64_t ptok = (int64_t)(tu % R) * TM + (u & 3) * 8 + ml;  // ring slot of the q words
          const uint32_t qtag = ring_tag(tag, (uint32_t)(tu / R));
          float res, pp;
          // every row of the tile is published ([R][TM][4] words): the
          // stream workgroups poll whole row blocks, padding rows included
          finalize_rows<FUSED>(fin + ml * NV, lb, C, a.sc, lane, res, pp,
                               [&](const float* q, const float* pw, bool cancels) __attribute__((always_inline)) {
                                 // a cancelling token: listed (and its pre weights written through)
                                 // before its q words, whose sign bit on q0 tells the pre step to
                                 // leave its h to the recomputation
                                 if (cancels && tok < a.T) {
                                   if (kk < 4)
                                     store_sys32(a.coeffs_out + tok * kCoeffs + kk,
                                                 __float_as_uint(kk == 0 ? pw[0] : kk == 1 ? pw[1] : kk == 2 ? pw[2] : pw[3]));
                                   if (kk == 0) flag_for_fix(a, tag, tok);
                                   __builtin_amdgcn_s_waitcnt(0);
                                 }
                                 if (kk < 4)
                                   tagged_store(a.publish + ptok * 4 + kk,
                                                kk == 0 ? (cancels ? -q[0] : q[0]) : kk == 1 ? q[1] : kk == 2 ? q[2] : q[3],
                                                qtag);
                               });
          if (tok < a.T) {
            a.coeffs_out[tok * kCoeffs + 8 + kk] = res;
            if (kk < 8) a.coeffs_out[tok * kCoeffs + kk] = pp;
          }
        } else if (u + nred < nunits) {
          gather(u + nred, finw + ((k + 1) & 1) * (8 * NV));
        }
        __syncthreads();  // the next unit's sums are in; this unit's are read
      }
      // The last reduce workgroup to finish recomputes the listed tokens
      // (bf16 modes; see the leave section for the MXFP8 ones): every token
      // has been finalised, so the list is complete, and the stream
      // workgroups, still running their last pre steps, leave the listed
      // tokens' rows alone.  The arguments are read through the
      // kernel-argument segment's address, made opaque (as in the leave
      // section), so that the main loop's registers do not change.
      if constexpr (!MX) {
        if (tid == 0) {
          uint32_t* rd = reinterpret_cast<uint32_t*>(a.fix_word + 1);
          static_assert(kWsRedDone == kWsFixWord + 8, "reduce-done counter after the fix word");
          uint32_t last = 0;
          const uint32_t done = __hip_atomic_fetch_add(rd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (done == (uint32_t)nred - 1u) {
            __hip_atomic_store(rd, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = 1;
          }
          s_last = last;
        }
        __syncthreads();
        if (s_last != 0) {
          const SplitArgs* ap = (const SplitArgs*)__builtin_amdgcn_kernarg_segment_ptr();
          asm volatile("" : "+s"(ap));
          fix_flagged<YQ, false, kPersistThreads>(*ap, tag, reinterpret_cast<double*>(&red[0][0][0]));
        }
      }
    }
  } else {
    // ------------------------- stream workgroup -------------------------
    const int split = (int)blockIdx.x % S, r = (int)blockIdx.x / S;
    const int c0 = split * a.cs;
    const int n16 = lane & 15, g = lane >> 4;
    // (wave index made provably uniform, so that branches on the row block
    // are scalar and buffer resources stay in scalar registers)
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int rb = wv >> 2, ks = wv & 3;  // row block (pipeline group), 32-channel step
    const int gt = tid & 255;                 // thread of the row block's group
    const int m = rb * 16 + n16;              // this lane's token in the tile
    const int ch = 32 * ks + 8 * g;           // this lane's first channel in the split
    const int cl = c0 + ch;
    const int xpos = (4 * ks + g) ^ n16;  // LDS position of this lane's chunk in a row
    const int niter = r < tiles ? (tiles - r + L - 1) / L : 0;

    // projection slice -> LDS: asynchronous global -> LDS copies, all of a
    // wave's in flight at once (lane l of copy k fills fragment
    // k * 512 + 64 wave + l), waited for together with the first tiles'
    // loads below; and one zero fragment for block 4's unused lanes
    {
      static_assert(16 * kPhiFrag % kPersistThreads == 0, "whole waves of fragments");
      const u32x4_t* pk = reinterpret_cast<const u32x4_t*>(a.phi_packed);
#pragma unroll
      for (int k = 0; k < 16 * kPhiFrag / kPersistThreads; ++k) {
        const int base = k * kPersistThreads + wv * kWave;
        const int idx = base + lane;
        const int jk = idx / kPhiFrag, o = idx % kPhiFrag;
        const int jr = jk >> 2, kq = jk & 3;
        const int64_t kstep = ((int64_t)jr * a.prs + c0 + kq * 32) >> 5;
        int b, ln;
        if (o < 4 * kWave) {
          b = o >> 6;
          ln = o & 63;
        } else {
          b = 4;
          ln = ((o - 4 * kWave) >> 3) * 16 + ((o - 4 * kWave) & 7);
        }
        lds_dma16_shared(pk + (kstep * kPackBlocks + b) * kWave + ln,
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_address(&phi_lds[base])));
      }
      if (tid == 0) phi_lds[16 * kPhiFrag] = u32x4_t{0, 0, 0, 0};
    }
    // gamma slice: loaded now, stored to LDS after the prologue's wait
    // (a compiler wait for it here would also wait for the copies above)
    // (broadcast: the 512 channels of the split's four pseudo-routes)
    const float gam_v = FUSED && (BC || tid < kCC) ? a.gamma[c0 + tid] : 0.0f;
    // block 4 fragment of this lane: its own column if < 8, else the zero fragment
    const int b4off = n16 < 8 ? 4 * kWave + g * 8 + n16 : -1;

    if constexpr (!FUSED) {
      // Coefficients only: no post and no x' ring, so x is loaded into
      // registers kCoeffsAhead tiles ahead, with loads the compiler counts
      // and waits for.  A wave instruction loads 4 rows x 256 bytes (whole
      // 128-byte lines; loading the MFMA operand layout directly reads 16
      // rows x 64 bytes per instruction, half lines, at two thirds of the
      // rate), and the tile goes through an LDS stage into the operand
      // layout.  Step i: tile t_i to the stage and the loads of t_{i+A};
      // barrier; the partial words of t_{i-1} (the four waves of the row
      // block added from LDS buffer (i - 1) & 1) and the projection of t_i
      // into buffer i & 1; barrier.  The loop is unrolled by A so that every
      // register buffer has a fixed index.
      constexpr int A = kCoeffsAhead, NW = kCoeffsWords;
      u32x4_t xq[A][4];
      u32x4_t* const stage = &xslot[0][rb][0];
      // chunk q = gt + 256 k of the row block's tile: row q / 16 (token
      // row / 4, route row % 4), 16-byte chunk q % 16 of the split's 256 bytes
      // (issued unconditionally, so that the compiler's wait counts never
      // merge paths with and without the loads: past the last tile every
      // lane reads the first 16 bytes of x, whose value is not used)
      auto load_x = [&](u32x4_t* dst, int i) __attribute__((always_inline)) {
        const bool ok = i < niter;
        const int64_t tok0 = (int64_t)(r + L * i) * TM + rb * 16;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int q = gt + 256 * k, row = q >> 4;
          const int64_t tok = tok0 + (row >> 2);
          const int64_t off = (tok < a.T ? tok : 0) * a.xts + (int64_t)(row & 3) * a.xrs + c0 + 8 * (q & 15);
          dst[k] = ld16_stream(a.x + (ok ? off : 0));
        }
      };
      auto stage_write = [&](const u32x4_t* src) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int q = gt + 256 * k, row = q >> 4;
          stage[row * 16 + ((q & 15) ^ (row >> 2))] = src[k];
        }
      };
      // partial values of tile t_i: 16 tokens x NW words of this row block
      // (ring slots [cring][S][TM][NW]: dense, whole lines per store).  A
      // slot that held an earlier tile (generation > 0) is refilled only
      // once its release word says that tile was gathered.  Two schedules
      // (one loop copy each, so that the compiler's wait counting follows
      // one of them):
      //   early flags (the 64-tile ring, >= 17 splits): the release word is
      //     loaded at the start of the step, before its x loads, and every
      //     fold first waits for all of the wave's memory operations but
      //     those x loads (the partial values stored in the step before
      //     among them), whose flag the next step stores at its start;
      //   late flags (the 512-tile ring at <= 16 splits: a broadcast
      //     stream's pseudo-routes, or C = 2048; a call seldom reuses a
      //     slot there): nothing waits in the
      //     fold unless the slot is reused (the release word is loaded
      //     there); the flag of tile t_{i-A-2} is stored after the first
      //     barrier of step i (see step).
      // (the ring: kCoeffsRingTilesWide tiles in the late schedule, which runs
      // at <= 16 splits, kCoeffsRingTiles in the early one; coeffs_ring_tiles)
      auto release_of = [&](int i) __attribute__((always_inline)) {
        return tagged_load(a.release + (r + L * i) % kCoeffsRingTiles);
      };
      auto fold = [&](int i, uint64_t rel, auto kLate) __attribute__((always_inline)) {
        constexpr bool LATE = decltype(kLate)::value;
        constexpr int cring = LATE ? kCoeffsRingTilesWide : kCoeffsRingTiles;
        const int t = r + L * i;
        const uint32_t gen = (uint32_t)(t / cring);
        float* part = reinterpret_cast<float*>(a.partials) + ((int64_t)(t % cring) * S + split) * (TM * NW) +
                      rb * 16 * NW;
        if constexpr (!LATE) {
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
          __builtin_amdgcn_sched_barrier(0);
        }
        if (gen > 0) {
          if constexpr (LATE) rel = tagged_load(a.release + t % cring);
          const uint32_t rtag = ring_tag(tag, 0);
          uint32_t it = 0;
          while ((uint32_t)(rel >> 32) != rtag || (uint32_t)rel < gen - 1u) {
            __builtin_amdgcn_s_sleep(1);
            if (++it > kPersistSpinLimit || ((it & 15u) == 0u && error_seen(a.err))) {
              __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            rel = tagged_load(a.release + t % cring);
          }
        }
        const float* rr = &red[i & 1][rb * 4][0];
        float sum[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int idx = min(gt + 256 * k, 16 * NW - 1);
          sum[k] = ((rr[idx] + rr[16 * NW + idx]) + rr[2 * 16 * NW + idx]) + rr[3 * 16 * NW + idx];
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int idx = gt + 256 * k;
          if (idx < 16 * NW) store_sys32(part + idx, __float_as_uint(sum[k]));
        }
      };
      // release flag of this row block's partial values of tile t_i
      auto flag = [&](int i, auto kLate) __attribute__((always_inline)) {
        constexpr int cring = decltype(kLate)::value ? kCoeffsRingTilesWide : kCoeffsRingTiles;
        const int t = r + L * i;
        if (gt == 0)
          tagged_store(a.pflag + ((int64_t)(t % cring) * S + split) * 2 + rb, 0.0f, ring_tag(tag, (uint32_t)(t / cring)));
      };
      // projection and sum of squares of tile t_i from the stage (rows past
      // T read token 0 and are zeroed) -> LDS buffer i & 1
      auto project = [&](int i) __attribute__((always_inline)) {
        const bool live = (int64_t)(r + L * i) * TM + m < a.T;
        u32x4_t xa[4];
#pragma unroll
        for (int jr = 0; jr < 4; ++jr) {
          const u32x4_t v = stage[(n16 * 4 + jr) * 16 + ((4 * ks + g) ^ n16)];
          xa[jr] = live ? v : u32x4_t{0, 0, 0, 0};
        }
        f32x4_t acc0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
#pragma unroll
        for (int jr = 0; jr < 4; ++jr) {
          const u32x4_t* bp = phi_lds + (jr * 4 + ks) * kPhiFrag;
          u32x4_t bf[kPackBlocks];
#pragma unroll
          for (int b = 0; b < 4; ++b) bf[b] = bp[b * kWave + lane];
          bf[4] = b4off >= 0 ? bp[b4off] : phi_lds[16 * kPhiFrag];
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xa[jr]);
#pragma unroll
          for (int b = 0; b < kPackBlocks; ++b) {
            if (b < 3) {
              acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bf[b]), acc0, 0, 0, 0);
            } else {
              acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bf[b]), acc1, 0, 0, 0);
            }
          }
        }
        // sum of squares: the diagonal of x_j x_j^T, token n in lane
        // n + 16 (n / 4), element n % 4
        f32x4_t gm[4];
#pragma unroll
        for (int jr = 0; jr < 4; ++jr)
          gm[jr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[jr]),
                                                          __builtin_bit_cast(bf16x8_t, xa[jr]),
                                                          f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        float gd[4];
#pragma unroll
        for (int jr = 0; jr < 4; ++jr) {
          float vv = gm[jr][0];
          vv = (n16 & 3) == 1 ? gm[jr][1] : vv;
          vv = (n16 & 3) == 2 ? gm[jr][2] : vv;
          gd[jr] = (n16 & 3) == 3 ? gm[jr][3] : vv;
        }
        float* rw = &red[i & 1][wave][0];  // [16 tokens][NW]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v1 = acc1[e];
          const float mid = MHC_DPP(v1, kDppRowRor8);  // lane ^ 8 (rotation by 8 of a 16-lane row)
          rw[(4 * g + e) * NW + n16] = acc0[e];
          if (n16 < 8) rw[(4 * g + e) * NW + 16 + n16] = v1 + mid;
        }
        if ((n16 >> 2) == g) rw[n16 * NW + 24] = ((gd[0] + gd[1]) + gd[2]) + gd[3];
      };
      // step i >= 1 (step 0 has no partial values to store)
      //   early flags: the flag of tile t_{i-3} (its values were stored in
      //     step i - 2 and complete at the wait of step i - 1's fold, before
      //     its last barrier); the release word of tile t_{i-1}'s slot; the
      //     x loads of tile t_{i+A}; barrier; the fold of t_{i-1}.
      //   late flags: the x loads of tile t_{i+A}; barrier; the flag of tile
      //     t_{i-A-2} (its values were issued in step i - A - 1, before the
      //     x loads of tile t_i, which every wave waited for in stage_write
      //     before that barrier, so they are complete in memory); the fold
      //     of t_{i-1}.
      auto step_early = [&](int i, u32x4_t* xb) __attribute__((always_inline)) {
        if (i >= 3) flag(i - 3, BoolC<false>{});
        const uint64_t rel = release_of(i - 1);
        __builtin_amdgcn_sched_barrier(0);
        stage_write(xb);
        load_x(xb, i + A);
        MHC_GROUP_BARRIER("coefficients, early flags: stage written");
        fold(i - 1, rel, BoolC<false>{});
        project(i);
        MHC_GROUP_BARRIER("coefficients, early flags: stage read");
      };
      auto step_late = [&](int i, u32x4_t* xb) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        stage_write(xb);
        load_x(xb, i + A);
        MHC_GROUP_BARRIER("coefficients, late flags: stage written");
        if (i >= A + 2) flag(i - A - 2, BoolC<true>{});
        fold(i - 1, 0, BoolC<true>{});
        project(i);
        MHC_GROUP_BARRIER("coefficients, late flags: stage read");
      };
      auto run = [&](auto kLate) __attribute__((always_inline)) {
        constexpr bool LATE = decltype(kLate)::value;
        // tile t_i is in xq[i % A]
        int i = 1;
        for (; i + A <= niter; i += A) {
#pragma unroll
          for (int k = 0; k < A; ++k) {
            if constexpr (LATE) {
              step_late(i + k, xq[(k + 1) % A]);
            } else {
              step_early(i + k, xq[(k + 1) % A]);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < A; ++k) {
          if (i + k < niter) {
            if constexpr (LATE) {
              step_late(i + k, xq[(k + 1) % A]);
            } else {
              step_early(i + k, xq[(k + 1) % A]);
            }
          }
        }
        fold(niter - 1, LATE ? (uint64_t)0 : release_of(niter - 1), kLate);
        // the last tiles' values are complete in every wave: their flags
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        constexpr int kTail = LATE ? A + 2 : 3;
        for (int k = niter >= kTail ? niter - kTail : 0; k < niter; ++k) flag(k, kLate);
      };
      if (niter > 0) {
#pragma unroll
        for (int k = 0; k < A; ++k) load_x(xq[k], k);
        // the projection copies (issued before these 4 A loads) have landed
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * A));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // the projection slice is in LDS
        stage_write(xq[0]);
        load_x(xq[0], A);
        MHC_GROUP_BARRIER("coefficients: first stage written");
        project(0);
        MHC_GROUP_BARRIER("coefficients: first stage read");
        if (S <= 16) {
          run(BoolC<true>{});
        } else {
          run(BoolC<false>{});
        }
      }
    } else {

    // x slice of this row block of tile t_i -> slot i%2: wave-instruction k
    // covers the four routes of token ks + 4k of the row block (1 KB of LDS,
    // 4 x 256 contiguous bytes of x).
    const uint32_t slot0 = lds_address(&xslot[0][rb][0]);
    constexpr uint32_t kSlotStride = 2u * kHalfChunks * 16u;  // bytes from xslot[0][b] to xslot[1][b]
    auto issue_x = [&](int i) __attribute__((always_inline)) {
      const int t = r + L * (i < niter ? i : 0);
      const uint32_t sb = slot0 + (uint32_t)(i & 1) * kSlotStride;
      const int jr = lane >> 4, p = lane & 15;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int q = ks + 4 * k;
        const int64_t tok = (int64_t)t * TM + rb * 16 + q;
        const int64_t tc = tok < a.T ? tok : 0;
        const uint16_t* src = BC ? a.x + tc * a.xts + (int64_t)jr * a.xrs + c0 + 8 * (p ^ q)
                                 : a.x + tc * (int64_t)(4 * C) + (int64_t)jr * C + c0 + 8 * (p ^ q);
        lds_dma16(src, __builtin_amdgcn_readfirstlane(sb + (uint32_t)q * 1024u));
      }
    };
    // y and post coefficients of this row block of tile t_i (registers)
    u32x4_t ny = u32x4_t{0, 0, 0, 0};
    float4 ncf = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    uint64_t nq = 0;
    auto issue_y = [&](int i) __attribute__((always_inline)) {
      if constexpr (BC) return;  // no post
      const int t = r + L * (i < niter ? i : 0);
      const int64_t tok = (int64_t)t * TM + m;
      const int64_t tc = tok < a.T ? tok : 0;
      if constexpr (YQ) {
        ny = load_y8<true, false>(a, tc, cl);
      } else {
        ny = *reinterpret_cast<const u32x4_t*>(a.y + tc * (int64_t)C + cl);
      }
      const int64_t ct = (int64_t)t * TM + rb * 16 + gt / 5;
      const bool cv = gt < 16 * 5 && ct < a.T;
      ncf = reinterpret_cast<const float4*>(a.coeffs_in + (cv ? ct : 0) * kCoeffs)[1 + (cv ? gt % 5 : 0)];
    };
    // q words (this row block) of the tile whose pre step runs in phase P of
    // iteration i
    auto issue_q = [&](int i) __attribute__((always_inline)) {
      const int ic = i - D;
      const int slot = ic >= 0 && ic < niter ? r + L * (ic % kRingK) : 0;
      nq = tagged_load(a.publish + ((int64_t)slot * TM + rb * 16) * 4 + (gt & 63));
    };

    u32x4_t ring[D][4];  // x' of the last D tiles (packed bf16, 4 routes)
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) ring[k][jr] = u32x4_t{0, 0, 0, 0};
    u32x4_t o[4];  // x' of the current tile, from phase P to phase M
#pragma unroll
    for (int jr = 0; jr < 4; ++jr) o[jr] = u32x4_t{0, 0, 0, 0};

    // Memory-operation order of one row block (vmcnt counts them in issue
    // order; the x slot copies are invisible to the compiler's counting):
    //   P(i): partial stores of tile t_{i-1} (up to 3), loads of tile t_{i+1}
    //         (FUSED: y, coefficients, q), h and x_out buffer stores
    //         (unconditional: rows past T are dropped by the bounds check)
    //   M(i): x slot copies of tile t_{i+2} (4, invisible), MFMAs, fold,
    //         explicit wait for all but those 4, then the next tile's post
    //         coefficients and q words to LDS.
    // The loads M(i) and P(i+1) consume are followed by at least 4 counted
    // stores before the copies, so a compiler wait for them never reaches
    // the copies, and the explicit wait leaves exactly the copies pending.

    // ---- phase P of tile t_i ----
    auto phaseP = [&](int i, auto kA, auto kC, auto kPrev) __attribute__((always_inline)) {
      constexpr bool doA = decltype(kA)::value;
      constexpr bool doC = FUSED && decltype(kC)::value;
      constexpr bool doPrev = decltype(kPrev)::value;
      const int t = r + L * i;
      // release of tile t_{i-2}'s partial values, stored in phase P(i-1):
      // every wave of the row block has since waited for all its memory
      // operations but the slot copies issued after them, and passed a
      // barrier, so those write-through stores are complete and the flag
      // cannot be seen before them
      if (i >= 2 && i <= niter + 1 && gt == 0) {
        const int ip = i - 2;
        tagged_store(a.pflag + ((int64_t)(r + L * (ip % kRingK)) * S + split) * 2 + rb, 0.0f,
                     ring_tag(tag, (uint32_t)(ip / kRingK)));
      }
      // partial row of tile t_{i-1}: this row block's 16 tokens x NV values,
      // the four 32-channel steps added in order
      if constexpr (doPrev) {
        // tile t_{i-1}, ring slot r + L ((i - 1) % kRingK)
        float* part = reinterpret_cast<float*>(a.partials) +
                      ((int64_t)(r + L * ((i - 1) % kRingK)) * S + split) * (TM * NV) + rb * 16 * NV;
        // all twelve LDS reads first, then the stores (values past the row
        // block are not stored)
        float sum[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const int idr = min(gt + k * 256, 16 * NV - 1);
          const int tm = idr / NV, vv = idr % NV;
          sum[k] = ((red[rb * 4][tm][vv] + red[rb * 4 + 1][tm][vv]) + red[rb * 4 + 2][tm][vv]) + red[rb * 4 + 3][tm][vv];
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const int idx = gt + k * 256;
          if (idx < 16 * NV) store_sys32(part + idx, __float_as_uint(sum[k]));
        }
      }
      const u32x4_t cy = ny;
      if constexpr (FUSED) {
        issue_y(i + 1);
        issue_q(i + 1);
      }
      // pre step of tile t_{i-D}
      if constexpr (doC && BC) {
        // broadcast: h of the split's four pseudo-routes, (q x') gamma at
        // channels c0 + 128 jr + ch (q = psum r_h, the same in all 4 words)
        const int64_t tokC0 = (int64_t)(r + L * (i - D)) * TM + rb * 16;
        const uint32_t nC = (uint32_t)max((int64_t)0, min((int64_t)16, a.T - tokC0));
        const float qb = qs[m][0];
        const __amdgpu_buffer_rsrc_t rhb = buffer_rsrc(a.h + tokC0 * C, nC * (uint32_t)(2 * C));
#pragma unroll
        for (int jr = 0; jr < 4; ++jr) {
          float hv[8];
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            hv[2 * qd] = (qb * bf16_lo(ring[0][jr][qd])) * gam[kCC * jr + ch + 2 * qd];
            hv[2 * qd + 1] = (qb * bf16_hi(ring[0][jr][qd])) * gam[kCC * jr + ch + 2 * qd + 1];
          }
          __builtin_amdgcn_raw_buffer_store_b128(pack8(hv), rhb, (n16 * C + cl + kCC * jr) * 2, 0, 0);
        }
      } else if constexpr (doC) {
        const int64_t tokC0 = (int64_t)(r + L * (i - D)) * TM + rb * 16;
        const uint32_t nC = (uint32_t)max((int64_t)0, min((int64_t)16, a.T - tokC0));
        const float q0 = qs[m][0], q1 = qs[m][1], q2 = qs[m][2], q3 = qs[m][3];
        // a negative q0 marks a token whose h the launch's last workgroup
        // recomputes directly (fix_flagged): its stores go past the end of
        // the buffer range, where the hardware drops them
        const uint32_t drop = __builtin_signbit(q0) ? 0x80000000u : 0u;
        float hv[8];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          float xl[4], xh[4];
#pragma unroll
          for (int jr = 0; jr < 4; ++jr) {
            xl[jr] = bf16_lo(ring[0][jr][qd]);
            xh[jr] = bf16_hi(ring[0][jr][qd]);
          }
          float vl = q0 * xl[0], vh = q0 * xh[0];
          vl = __builtin_fmaf(q1, xl[1], vl);
          vh = __builtin_fmaf(q1, xh[1], vh);
          vl = __builtin_fmaf(q2, xl[2], vl);
          vh = __builtin_fmaf(q2, xh[2], vh);
          vl = __builtin_fmaf(q3, xl[3], vl);
          vh = __builtin_fmaf(q3, xh[3], vh);
          hv[2 * qd] = vl * gam[ch + 2 * qd];
          hv[2 * qd + 1] = vh * gam[ch + 2 * qd + 1];
        }
        const u32x4_t hb = pack8(hv);
        if (!MX || a.h != nullptr)
          __builtin_amdgcn_raw_buffer_store_b128(hb, buffer_rsrc(a.h + tokC0 * C, nC * (uint32_t)(2 * C)),
                                                 ((n16 * C + cl) * 2) | drop, 0, 0);
        if constexpr (MX) {
          // a 32-channel block is the 4 lanes n16, n16 + 16, n16 + 32, n16 + 48
          float hr[8];
          unpack8(hb, hr);
          float amax = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(hr[e]));
          amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
          amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
          const int ex = mx_scale_exponent(amax);
          const float scale = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-ex, ex <= 120
          const uint32_t w0 = e4m3_pack4(hr[0] * scale, hr[1] * scale, hr[2] * scale, hr[3] * scale);
          const uint32_t w1 = e4m3_pack4(hr[4] * scale, hr[5] * scale, hr[6] * scale, hr[7] * scale);
          __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{w0, w1}, buffer_rsrc(a.h_fp8 + tokC0 * C, nC * (uint32_t)C),
                                                (n16 * C + cl) | drop, 0, 0);
          // the block's four lanes store the same scale byte; the
          // matrix-core order covers whole 16-row blocks (rows past T hold
          // h = 0, whose scale byte is 0), up to ceil(T/16)*16 rows
          const int blk = cl >> 5;
          const uint32_t nS = a.scale_mfma ? (tokC0 < a.T ? 16u : 0u) : nC;
          const uint32_t soff = a.scale_mfma ? (uint32_t)mx_scale_offset(n16, blk, C, true)
                                             : (uint32_t)(n16 * (C / 32) + blk);
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(ex + 127),
                                               buffer_rsrc(a.h_scale + tokC0 * (C / 32), nS * (uint32_t)(C / 32)),
                                               soff | drop, 0, 0);
        }
      }
      if constexpr (FUSED) {
        // shift the x' ring: slot 0 is consumed
#pragma unroll
        for (int k = 0; k + 1 < D; ++k)
#pragma unroll
          for (int jr = 0; jr < 4; ++jr) ring[k][jr] = ring[k + 1][jr];
      }
      // post of tile t_i: x (slot) and y -> x' in the MFMA A layout
      if constexpr (doA) {
        const int64_t tokA0 = (int64_t)t * TM + rb * 16;
        const uint32_t nA = (uint32_t)max((int64_t)0, min((int64_t)16, a.T - tokA0));
        const u32x4_t* sp = &xslot[i & 1][rb][0];
        u32x4_t xin[4];
#pragma unroll
        for (int jr = 0; jr < 4; ++jr) xin[jr] = sp[(n16 * 4 + jr) * 16 + xpos];
        if constexpr (FUSED && !BC) {
          float pw[4], rs[16];
#pragma unroll
          for (int k = 0; k < 4; ++k) pw[k] = cfs[m][k];
#pragma unroll
          for (int k = 0; k < 16; ++k) rs[k] = cfs[m][4 + k];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float xl[4] = {bf16_lo(xin[0][q]), bf16_lo(xin[1][q]), bf16_lo(xin[2][q]), bf16_lo(xin[3][q])};
            const float xh[4] = {bf16_hi(xin[0][q]), bf16_hi(xin[1][q]), bf16_hi(xin[2][q]), bf16_hi(xin[3][q])};
            float yl, yh;
            y_pair<YQ>(cy, q, yl, yh);
#pragma unroll
            for (int jr = 0; jr < 4; ++jr)
              o[jr][q] = pack_bf16x2(post_chain(pw[jr], yl, &rs[4 * jr], xl[0], xl[1], xl[2], xl[3]),
                                     post_chain(pw[jr], yh, &rs[4 * jr], xh[0], xh[1], xh[2], xh[3]));
          }
          const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x_out + tokA0 * (4 * C), nA * (uint32_t)(8 * C));
#pragma unroll
          for (int jr = 0; jr < 4; ++jr)
            __builtin_amdgcn_raw_buffer_store_b128(o[jr], rx, ((n16 * 4 + jr) * C + cl) * 2, 0, 0);
        } else {
#pragma unroll
          for (int jr = 0; jr < 4; ++jr) o[jr] = xin[jr];
        }
        if ((uint32_t)n16 >= nA) {
#pragma unroll
          for (int jr = 0; jr < 4; ++jr) o[jr] = u32x4_t{0, 0, 0, 0};
        }
        if constexpr (FUSED) {
#pragma unroll
          for (int jr = 0; jr < 4; ++jr) ring[D - 1][jr] = o[jr];
        }
      }
    };

    // ---- phase M of tile t_i: slot copy of t_{i+2}, projection, Gram, fold ----
    auto phaseM = [&](int i) __attribute__((always_inline)) {
      issue_x(i + 2);
      // projection: A = x' of route jr (16 tokens x 32 channels), B = the
      // five packed blocks of (route jr, step ks); blocks 0-2 accumulate
      // logits 0..15, blocks 3-4 logits 16..23 (hi+lo | mid)
      u32x4_t xa[4];
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) xa[jr] = FUSED ? ring[D - 1][jr] : o[jr];
      f32x4_t acc0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) {
        const u32x4_t* bp = phi_lds + (jr * 4 + ks) * kPhiFrag;
        u32x4_t bf[kPackBlocks];
#pragma unroll
        for (int b = 0; b < 4; ++b) bf[b] = bp[b * kWave + lane];
        bf[4] = b4off >= 0 ? bp[b4off] : phi_lds[16 * kPhiFrag];
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xa[jr]);
#pragma unroll
        for (int b = 0; b < kPackBlocks; ++b) {
          if (b < 3) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bf[b]), acc0, 0, 0, 0);
          } else {
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bf[b]), acc1, 0, 0, 0);
          }
        }
      }
      // Gram: D = x'_a x'_b^T over the 32 channels; its diagonal entry for
      // token n sits in lane n + 16*(n/4), element n%4 (picked with
      // selects after all products are issued: no branch waits on a result)
      const bool holds = (n16 >> 2) == g;
      constexpr int NG = FUSED ? 10 : 4;
      constexpr int ga[10] = {0, 1, 2, 3, 0, 0, 0, 1, 1, 2};
      constexpr int gb[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
      f32x4_t gm[NG];
#pragma unroll
      for (int s2 = 0; s2 < NG; ++s2)
        gm[s2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[ga[s2]]),
                                                        __builtin_bit_cast(bf16x8_t, xa[gb[s2]]),
                                                        f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      bool em[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) em[e] = (n16 & 3) == e;
      float gd[NG];
#pragma unroll
      for (int s2 = 0; s2 < NG; ++s2) {
        float vv = gm[s2][0];
        vv = em[1] ? gm[s2][1] : vv;
        vv = em[2] ? gm[s2][2] : vv;
        gd[s2] = em[3] ? gm[s2][3] : vv;
      }
      // MFMA output: lane l holds column l%16 of rows 4*(l/16)+e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v1 = acc1[e];
        const float mid = MHC_DPP(v1, kDppRowRor8);  // lane ^ 8 (rotation by 8 of a 16-lane row)
        red[wave][4 * g + e][n16] = acc0[e];
        if (n16 < 8) red[wave][4 * g + e][16 + n16] = v1 + mid;
      }
      if (holds) {
        if constexpr (FUSED) {
#pragma unroll
          for (int s2 = 0; s2 < 10; ++s2) red[wave][n16][24 + s2] = gd[s2];
        } else {
          red[wave][n16][24] = ((gd[0] + gd[1]) + gd[2]) + gd[3];
        }
      }
    };

    // ---- before phase P of tile t_i: its slot, post coefficients, q words ----
    // copied: whether this slot's phase M issued slot copies (left pending)
    auto prepP = [&](int i, auto kCopied) __attribute__((always_inline)) {
      constexpr bool copied = decltype(kCopied)::value;
      // Everything but the copies just issued has landed: the slot of t_i
      // (copied during the phase M before), the loads and stores of the last
      // phase P.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(copied ? 4 : 0));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (FUSED) {
        const int ti = r + L * i;
        const float4 ccf = ncf;
        if (!BC && gt < 16 * 5) {
          const bool ok = (int64_t)ti * TM + rb * 16 + gt / 5 < a.T;
          float* dd = &cfs[rb * 16 + gt / 5][4 * (gt % 5)];
          dd[0] = ok ? ccf.x : 0.0f;
          dd[1] = ok ? ccf.y : 0.0f;
          dd[2] = ok ? ccf.z : 0.0f;
          dd[3] = ok ? ccf.w : 0.0f;
        }
        // q words of the tile whose pre step runs in phase P(i)
        const int ic = i - D;
        if (ic >= 0 && ic < niter && gt < 64) {
          uint64_t qw = nq;
          const uint32_t qtag = ring_tag(tag, (uint32_t)(ic / kRingK));
          if ((uint32_t)(qw >> 32) != qtag) {
            const uint64_t* qp = a.publish + ((int64_t)(r + L * (ic % kRingK)) * TM + rb * 16) * 4 + gt;
            uint32_t it = 0;
            do {
              __builtin_amdgcn_s_sleep(1);
              if (++it > kPersistSpinLimit || ((it & 15u) == 0u && error_seen(a.err))) {
                __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
              }
              qw = tagged_load(qp);
            } while ((uint32_t)(qw >> 32) != qtag);
          }
          qs[rb * 16 + gt / 4][gt & 3] = tagged_value(qw);
        }
      }
    };

    using Yes = BoolC<true>;
    using No = BoolC<false>;
    // Iteration i: [row block 0: P(i) | row block 1: M(i-1)] barrier
    //              [row block 0: M(i) | row block 1: P(i)]   barrier
    // Phase P(i) has the post when i < niter, the pre step when
    // D <= i < niter + D, the previous tile's partials when 1 <= i <= niter;
    // phase M(i) runs for i < niter.
    if (niter > 0) {
      // prologue: this row block's x slices of the first two tiles, y,
      // coefficients and q of the first; nothing pending when the loop starts
      issue_x(0);
      if constexpr (FUSED) {
        issue_y(0);
        issue_q(0);
      }
      issue_x(1);
      // everything so far has landed: the projection copies, the slots, y
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __builtin_amdgcn_sched_barrier(0);
      if (FUSED && (BC || tid < kCC)) gam[tid] = gam_v;
      if (rb == 0) prepP(0, No{});
      __syncthreads();
      // step i: [row block 0: P(i)       | row block 1: M(i-1), prep P(i)]   barrier
      //         [row block 0: M(i), prep P(i+1) | row block 1: P(i)]         barrier
      // Each row block runs its own copy of the loop (the same barriers in
      // the same order), so that the compiler's wait counting follows one
      // row block's memory operations only: with one loop whose slots branch
      // on the row block, the two paths merge between the slots and phase M
      // would wait for the other path's loads and its own stores.  The
      // barriers are written out with a distinct text per place (LDS
      // operations drained, then s_barrier), so that the compiler cannot
      // merge the two loops back into one at a shared barrier call.
      auto stepA = [&](int i, auto kA, auto kC, auto kPrev, auto kMprev, auto kMcur) __attribute__((always_inline)) {
        constexpr bool mCur = decltype(kMcur)::value;  // phase M(i) runs
        phaseP(i, kA, kC, kPrev);
        MHC_GROUP_BARRIER("row block 0, slot 1");
        if constexpr (mCur) {
          phaseM(i);
          prepP(i + 1, Yes{});
        } else {
          prepP(i + 1, No{});
        }
        MHC_GROUP_BARRIER("row block 0, slot 2");
      };
      auto stepB = [&](int i, auto kA, auto kC, auto kPrev, auto kMprev, auto kMcur) __attribute__((always_inline)) {
        constexpr bool mPrev = decltype(kMprev)::value;  // phase M(i-1) runs
        if constexpr (mPrev) {
          phaseM(i - 1);
          prepP(i, Yes{});
        } else {
          prepP(i, No{});
        }
        MHC_GROUP_BARRIER("row block 1, slot 1");
        phaseP(i, kA, kC, kPrev);
        MHC_GROUP_BARRIER("row block 1, slot 2");
      };
      // Phase P(i) has the post when i < niter, the pre step when
      // D <= i < niter + D, the previous tile's partials when 1 <= i <= niter;
      // phase M(i) runs when i < niter.
      auto run = [&](auto step) __attribute__((always_inline)) {
        int i = 0;
        step(0, Yes{}, No{}, No{}, No{}, Yes{});
        ++i;
        const int pro = niter < D ? niter : D;
        for (; i < pro; ++i) step(i, Yes{}, No{}, Yes{}, Yes{}, Yes{});
        for (; i < niter; ++i) step(i, Yes{}, Yes{}, Yes{}, Yes{}, Yes{});
        // i = niter: the last tile's partials and row block 1's last phase M
        if (i < D) {
          step(i, No{}, No{}, Yes{}, Yes{}, No{});
        } else {
          step(i, No{}, Yes{}, Yes{}, Yes{}, No{});
        }
        ++i;
        for (; i < niter + D; ++i) {
          if (i >= D) {
            step(i, No{}, Yes{}, No{}, No{}, No{});
          } else {
            step(i, No{}, No{}, No{}, No{}, No{});  // (only the next phase P's preparation)
          }
        }
      };
      if (rb == 0) {
        run(stepA);
      } else {
        run(stepB);
      }
      // the last slot copies land before the workgroup's LDS is released
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __builtin_amdgcn_sched_barrier(0);
    }
    }
    // (a workgroup without tiles: its projection copies land before its LDS
    // is released)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- leave: the last workgroup to finish advances the launch epoch ----
  // In the MXFP8 modes it then recomputes the listed tokens (every reduce
  // workgroup has left, so the list is complete); the bf16 modes do that in
  // their last reduce workgroup (the tail here changed the main loop's
  // register allocation of those modes: prefill 268 -> 273 us).
  __syncthreads();
  if (tid == 0) {
    uint32_t last = 0;
    const uint32_t done = __hip_atomic_fetch_add(a.tiles_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1u) {
      __hip_atomic_store(a.tiles_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = 1;
    }
    s_last = last;
  }
  if constexpr (FUSED && MX) {
    __syncthreads();
    if (s_last != 0) {
      // The arguments are read here through the kernel-argument segment's
      // address (the kernel's one argument sits at its start), made opaque,
      // so that the compiler cannot hoist these loads to the kernel's entry:
      // hoisted, their scalar registers stay live through the main loop and
      // raise its spills.  (Taking the address of the argument itself
      // copies it to scratch memory, which slowed the whole kernel 1.66x.)
      const SplitArgs* ap = (const SplitArgs*)__builtin_amdgcn_kernarg_segment_ptr();
      asm volatile("" : "+s"(ap));
      fix_flagged<YQ, MX, kPersistThreads>(*ap, tag, reinterpret_cast<double*>(&red[0][0][0]));
    }
  }
}

// ===========================================================================
// Post (standalone): one thread per (token, 8 channels); consecutive threads
// read consecutive 16-byte chunks of each route.
// ===========================================================================
// YQ: y arrives as int8 codes [T][C] with one binary32 scale per token; its
// value is the binary32 product code * scale, which enters the chain in
// place of the bf16 y.
template <bool YQ>
__global__ __launch_bounds__(256) void k_post(const uint16_t* __restrict__ x, const void* __restrict__ y,
                                              const float* __restrict__ y_scale, const float* __restrict__ cf,
                                              int64_t T, int C, uint16_t* __restrict__ x_out) {
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
  if constexpr (YQ) {
    const uint64_t v = __builtin_nontemporal_load(
        reinterpret_cast<const uint64_t*>(static_cast<const int8_t*>(y) + t * (int64_t)C + c));
    const float sc = y_scale[t];
#pragma unroll
    for (int e = 0; e < 8; ++e) yy[e] = (float)(int8_t)(uint8_t)(v >> (8 * e)) * sc;
  } else {
    unpack8(ld16_stream(static_cast<const uint16_t*>(y) + t * (int64_t)C + c), yy);
  }
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


// g of 8 channels: the 4 routes combined in binary64 and kept as the nearest
// fp32 value.  B: a broadcast stream (route stride 0), whose routes are all
// x0: g = psum * x0 with psum = ((p0 + p1) + p2) + p3 in fp32 (no
// cancellation is possible, every pre weight being positive).
template <bool B>
__device__ __forceinline__ void pre_group(const uint16_t* xr, int64_t xrs, int c, const double* p, float psum,
                                          float* gv) {
  if constexpr (B) {
    float x0[8];
    unpack8(ld16_stream(xr + c), x0);
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[e] = psum * x0[e];
  } else {
    float xv[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack8(ld16_stream(xr + (int64_t)i * xrs + c), xv[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[e] = (float)combine_f64(p, xv[0][e], xv[1][e], xv[2][e], xv[3][e]);
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

template <int G, bool B>
__global__ __launch_bounds__(128) void k_pre(const uint16_t* __restrict__ x, int64_t xts, int64_t xrs,
                                             const float* __restrict__ cf, const float* __restrict__ gamma, int C,
                                             float eps, uint16_t* __restrict__ h) {
  __shared__ float sh[2];
  const int64_t t = blockIdx.x;
  const int k = threadIdx.x;
  const float4 pq = *reinterpret_cast<const float4*>(cf + t * kCoeffs);
  const double p[4] = {pq.x, pq.y, pq.z, pq.w};
  const float psum = ((pq.x + pq.y) + pq.z) + pq.w;
  const uint16_t* xr = x + t * xts;
  float gv[G][8];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    pre_group<B>(xr, xrs, (j * 128 + k) * 8, p, psum, gv[j]);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(gv[j][e], gv[j][e], ss);
  }
  ss = block128_sum(ss, sh);
  const float rh = 1.0f / sqrtf(ss / (float)C + eps);
  uint16_t* hr = h + t * (int64_t)C;
#pragma unroll
  for (int j = 0; j < G; ++j) pre_store(hr, gamma, (j * 128 + k) * 8, gv[j], rh);
}

template <bool B>
__global__ __launch_bounds__(128) void k_pre_wide(const uint16_t* __restrict__ x, int64_t xts, int64_t xrs,
                                                  const float* __restrict__ cf, const float* __restrict__ gamma,
                                                  int C, float eps, uint16_t* __restrict__ h) {
  __shared__ float sh[2];
  const int64_t t = blockIdx.x;
  const int k = threadIdx.x;
  const float4 pq = *reinterpret_cast<const float4*>(cf + t * kCoeffs);
  const double p[4] = {pq.x, pq.y, pq.z, pq.w};
  const float psum = ((pq.x + pq.y) + pq.z) + pq.w;
  const uint16_t* xr = x + t * xts;
  const int G = C >> 10;
  float ss = 0.0f;
  for (int j = 0; j < G; ++j) {
    float gv[8];
    pre_group<B>(xr, xrs, (j * 128 + k) * 8, p, psum, gv);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(gv[e], gv[e], ss);
  }
  ss = block128_sum(ss, sh);
  const float rh = 1.0f / sqrtf(ss / (float)C + eps);
  uint16_t* hr = h + t * (int64_t)C;
  for (int j = 0; j < G; ++j) {
    float gv[8];
    pre_group<B>(xr, xrs, (j * 128 + k) * 8, p, psum, gv);
    pre_store(hr, gamma, (j * 128 + k) * 8, gv, rh);
  }
}

// ===========================================================================
// Sinkhorn iterations on stored coefficients: the res entries coeffs[t][8..23]
// hold exp(logits) (a fused call with the Sinkhorn deferred) and get `iters`
// iterations in place, with the arithmetic of finalize_rows (one token per
// 16-lane row, row and column sums by the same DPP moves, each normalisation
// a multiplication by the hardware reciprocal of sum + eps), so the result is
// bitwise the one an undeferred call writes.
// ===========================================================================
__global__ __launch_bounds__(256) void k_sinkhorn(float* __restrict__ cf, int64_t T, float eps, int iters) {
  const int lane = threadIdx.x & 63;
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;  // 16 lanes per token
  const int k = lane & 15;
  float v = t < T ? cf[t * kCoeffs + 8 + k] : 1.0f;
  for (int it = 0; it < iters; ++it) {
    float rs = v + MHC_DPP(v, kDppQuadSwap1);
    rs = rs + MHC_DPP(rs, kDppQuadSwap2);
    v = v * __builtin_amdgcn_rcpf(rs + eps);
    float cs = v + MHC_DPP(v, kDppRowRor8);
    cs = cs + MHC_DPP(cs, kDppRowRor4);
    v = v * __builtin_amdgcn_rcpf(cs + eps);
  }
  if (t < T) cf[t * kCoeffs + 8 + k] = v;
}

__global__ void k_fill_zero(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ===========================================================================
// Launchers
// ===========================================================================
hipError_t launch_pack_phi(const float* phi, int C, void* out, hipStream_t s) {
  const int64_t total = (int64_t)(4 * C / 32) * kWave;
  const int64_t blocks = (total + 255) / 256;
  k_pack_phi<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(phi, C, reinterpret_cast<u32x4_t*>(out));
  return hipGetLastError();
}

hipError_t launch_pack_phi_sum(const float* phi, const void* packed, int C, void* out, hipStream_t s) {
  const int64_t total = (int64_t)(C / 32) * kWave;
  const int64_t blocks = (total + 255) / 256;
  u32x4_t* o = reinterpret_cast<u32x4_t*>(out);
  if (phi != nullptr) {
    k_pack_phi_sum<false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(phi, nullptr, C, o);
  } else {
    k_pack_phi_sum<true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(nullptr, reinterpret_cast<const u32x4_t*>(packed),
                                                                      C, o);
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_split_mode(const Plan& p, const SplitArgs& a, hipStream_t s) {
  const int64_t stages = p.tiles + (mode_fused(MODE) ? p.d2 : p.d1);
  // by tickets (one tile): S phase-A jobs, min(S, m) reduce jobs, S pre jobs
  const bool tk = p.tiles == 1;
  const int64_t nR = p.s < p.m ? p.s : p.m;
  const int64_t blocks = tk ? p.s + nR + (mode_fused(MODE) ? p.s : 0) : stages * p.s;
  const dim3 grid((unsigned)blocks), block(256);
  if ((p.m != 32 && p.m != 16) || p.cc != kCC || (p.m == 16 && !tk)) return hipErrorInvalidConfiguration;
  const bool short_runs = plan_run_len(p) <= 8;
  if (p.m == 16) {
    if (short_runs) k_split<MODE, 16, 8, true><<<grid, block, 0, s>>>(a);
    else k_split<MODE, 16, kRunMax, true><<<grid, block, 0, s>>>(a);
  } else if (tk) {
    if (short_runs) k_split<MODE, 32, 8, true><<<grid, block, 0, s>>>(a);
    else k_split<MODE, 32, kRunMax, true><<<grid, block, 0, s>>>(a);
  } else {
    if (short_runs) k_split<MODE, 32, 8, false><<<grid, block, 0, s>>>(a);
    else k_split<MODE, 32, kRunMax, false><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_persist_mode(const Plan& p, const SplitArgs& a, hipStream_t s) {
  // 32 to 64 reduce workgroups; the coefficients-only mode's rings are
  // whole multiples of its count (32, or 64 at <= 16 splits)
  if (p.reds < 32 || p.reds > 64) return hipErrorInvalidConfiguration;
  if (!mode_fused(MODE) && p.reds != 32 && !(p.reds == 64 && p.s <= 16)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(p.s * p.lanes + p.reds)), block(kPersistThreads);
  k_persist<MODE><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_split(const Plan& plan, int mode, const SplitArgs& a, hipStream_t s) {
  if (plan.lanes > 0) {
    switch (mode) {
      case kModeCoeffs: return launch_persist_mode<kModeCoeffs>(plan, a, s);
      case kModeFused: return launch_persist_mode<kModeFused>(plan, a, s);
      case kModeFusedMx: return launch_persist_mode<kModeFusedMx>(plan, a, s);
      case kModeFused | kModeYInt8: return launch_persist_mode<kModeFused | kModeYInt8>(plan, a, s);
      case kModeFusedMx | kModeYInt8: return launch_persist_mode<kModeFusedMx | kModeYInt8>(plan, a, s);
      // (16-token reduce units gather at most kPersistMaxS / 2 splits)
      case kModeFused | kModeBcast:
        if (plan.s > kPersistMaxS / 2) return hipErrorInvalidConfiguration;
        return launch_persist_mode<kModeFused | kModeBcast>(plan, a, s);
      case kModeFused | kModeUnit16:
        if (plan.s > kPersistMaxS / 2) return hipErrorInvalidConfiguration;
        return launch_persist_mode<kModeFused | kModeUnit16>(plan, a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (mode) {
    case kModeCoeffs: return launch_split_mode<kModeCoeffs>(plan, a, s);
    case kModeFused: return launch_split_mode<kModeFused>(plan, a, s);
    case kModeFusedMx: return launch_split_mode<kModeFusedMx>(plan, a, s);
    case kModeFused | kModeYInt8: return launch_split_mode<kModeFused | kModeYInt8>(plan, a, s);
    case kModeFusedMx | kModeYInt8: return launch_split_mode<kModeFusedMx | kModeYInt8>(plan, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_post(const uint16_t* x, const uint16_t* y, const float* cf, int64_t T, int C,
                       uint16_t* x_out, hipStream_t s) {
  const int64_t units = T * (C / 8);
  const int64_t blocks = (units + 255) / 256;
  k_post<false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(x, y, nullptr, cf, T, C, x_out);
  return hipGetLastError();
}

hipError_t launch_post_int8(const uint16_t* x, const int8_t* y_q, const float* y_scale, const float* cf, int64_t T,
                            int C, uint16_t* x_out, hipStream_t s) {
  const int64_t units = T * (C / 8);
  const int64_t blocks = (units + 255) / 256;
  k_post<true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(x, y_q, y_scale, cf, T, C, x_out);
  return hipGetLastError();
}

template <bool B>
static void launch_pre_b(const uint16_t* x, int64_t xts, int64_t xrs, const float* cf, const float* gamma,
                         int64_t T, int C, float eps, uint16_t* h, hipStream_t s) {
  const dim3 grid((unsigned)T), block(128);
  switch (C >> 10) {
    case 1: k_pre<1, B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
    case 2: k_pre<2, B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
    case 3: k_pre<3, B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
    case 4: k_pre<4, B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
    case 5: k_pre<5, B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
    case 6: k_pre<6, B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
    case 7: k_pre<7, B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
    case 8: k_pre<8, B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
    default: k_pre_wide<B><<<grid, block, 0, s>>>(x, xts, xrs, cf, gamma, C, eps, h); break;
  }
}

hipError_t launch_pre(const uint16_t* x, int64_t xts, int64_t xrs, const float* cf, const float* gamma, int64_t T,
                      int C, float eps, uint16_t* h, hipStream_t s) {
  if (xrs == 0) {
    launch_pre_b<true>(x, xts, xrs, cf, gamma, T, C, eps, h, s);
  } else {
    launch_pre_b<false>(x, xts, xrs, cf, gamma, T, C, eps, h, s);
  }
  return hipGetLastError();
}


hipError_t launch_sinkhorn(float* cf, int64_t T, float eps, int iters, hipStream_t s) {
  const int64_t blocks = (T * 16 + 255) / 256;
  if (blocks == 0) return hipSuccess;
  k_sinkhorn<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(cf, T, eps, iters);
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
