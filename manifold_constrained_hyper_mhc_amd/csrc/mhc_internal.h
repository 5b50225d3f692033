// Internal interface between the C ABI (mhc_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace mhc {

constexpr int kRoutes = 4;
constexpr int kCoeffs = 24;
constexpr int kWave = 64;
constexpr int kGram = 10;  // route Gram matrix entries (00,11,22,33,01,02,03,12,13,23)

struct Scalars {
  float hc_norm_eps, rmsnorm_eps, hc_post_scale, sinkhorn_eps;
  int sinkhorn_iters;
};

// The split-row kernel covers a tile of m tokens and cc channels of every
// route per workgroup; a token's row is spread over s = C / cc workgroups
// whose partial sums meet in the workspace.
struct Plan {
  int m = 32;      // tokens per tile
  int cc = 128;    // channels per workgroup
  int d1 = 1;      // stage delay of the reduce after a tile's phase A
  int d2 = 2;      // stage delay of the pre step (fused modes), > d1
  int s = 1;       // workgroups per row
  int lanes = 0;   // persistent kernel: stream workgroups per split (0: staged kernel)
  int reds = 32;   // persistent kernel: reduce workgroups (32 to 64; see choose_kernel)
  int64_t tiles = 0;
  int64_t chunk_tiles = 0;  // staged kernel: tiles per launch (a longer call is a sequence of launches)
  // workspace layout (byte offsets)
  size_t off_pub = 0, off_part = 0, off_own = 0, off_rel = 0, off_fix = 0, off_phi = 0, total = 0;
  size_t off_flag = 0;  // persistent passes: release flags, inside the partial region after the values
};

// Workspace bounds.  The persistent kernel keeps its exchanged words in
// rings (fused: kRingK * L tiles; coefficients only: coeffs_ring_tiles(S)
// tiles), with at most kMaxLaneSplits = L * S stream workgroups; the staged
// kernel runs a call as launches of at most chunk_tiles tiles, whose partial
// words take at most kStagedBudget bytes (kStagedBudgetStatic on the static
// scratch).  So a workspace holds about that budget + 4 bytes per token +
// the packed projection, whatever T is.  (Each staged launch pays its
// pipeline's fill and drain: the larger budget keeps a prefill-sized call in
// one launch up to C = 7168 and in three at C = 16384.)
constexpr int kRingK = 8;
// Coefficients-only ring: 64 tiles, or 512 at <= 16 splits (many stream
// lanes, whose release flags trail their values by A + 2 steps: the ring
// keeps at least 16 steps of every lane in flight).
constexpr int kCoeffsRingTiles = 64;
constexpr int kCoeffsRingTilesWide = 512;
inline int coeffs_ring_tiles(int s) { return s <= 16 ? kCoeffsRingTilesWide : kCoeffsRingTiles; }
constexpr int kMaxLaneSplits = 256;
constexpr size_t kStagedBudget = (size_t)128 << 20;
constexpr size_t kStagedBudgetStatic = (size_t)32 << 20;

constexpr int kPartVals = 24 + kGram;   // per token: projection + route Gram matrix
constexpr int kCoeffsWords = 25;        // per token, coefficients only: projection + sum of squares

// Workspace header at fixed offsets, whatever the shape of a call: the error
// word, the tiles-done counter, the ticket counter of a one-tile launch and
// the launch epoch (the low and high halves of one 64-bit word), the tagged
// count of tokens whose fused pre needs the direct recomputation, then one
// leave counter per possible tile (2^20 tokens / 32 tokens per tile).
constexpr size_t kWsErr = 0, kWsTilesDone = 4, kWsTicket = 8, kWsEpoch = 12, kWsFixWord = 16, kWsRedDone = 24;
constexpr size_t kWsDep = 256;
constexpr int64_t kMaxTiles = (int64_t)(1 << 20) / 32;
constexpr size_t kWsHeaderBytes = kWsDep + (size_t)kMaxTiles * 4;
constexpr int kPackBlocks = 5;          // 80 packed columns = 5 MFMA 16-column blocks
// Persistent kernel: at most this many workgroups (one per compute unit).
constexpr int kPersistMaxBlocks = 512;
constexpr size_t kPackBytesPerRow = 160;  // 80 bf16 per flattened row k

Plan make_plan(int64_t T, int64_t C, size_t staged_budget = kStagedBudget);
// The staged launch of a chunk of `tokens` tokens of a call planned as p.
Plan chunk_plan(const Plan& p, int64_t tokens);

// Reduce-scatter of the split kernel: a workgroup owns ntok = ceil(m/s)
// tokens of a tile; each of their ntok*34 partial words is summed over the
// s splits by r = clamp(256/(ntok*34), 1, 8) threads, each taking a run of
// plan_run_len() splits (at most kRunMax).
constexpr int kRunMax = 20;
inline int plan_run_len(const Plan& p) {
  const int64_t ntok = (p.m + p.s - 1) / p.s;
  const int64_t npair = ntok * kPartVals;
  int64_t r = npair > 0 ? 256 / npair : 1;
  r = r < 1 ? 1 : (r > 8 ? 8 : r);
  return (int)((p.s + r - 1) / r);
}
inline size_t phi_packed_bytes(int64_t C) { return (size_t)(4 * C) * kPackBytesPerRow; }

struct SplitArgs {
  const uint16_t* x;
  const uint16_t* y;
  const float* coeffs_in;
  const uint32_t* phi_packed;
  const float* bias;
  const float* gamma;
  uint16_t* x_out;
  float* coeffs_out;
  uint16_t* h;
  uint8_t* h_fp8;
  uint8_t* h_scale;
  uint64_t* partials;  // staged kernel: [tiles][S][M][34] tagged words ([..][25]: coefficients only);
                       // persistent kernel: [R][S][M][34] ([cring][S][M][25]) plain
                       // binary32 values, released by pflag
  uint64_t* pflag;     // persistent kernel: [ring slots][S][2 row blocks] tagged release flags
  uint32_t* epoch;     // launch epoch (fixed offset)
  uint32_t* tiles_done;  // tiles completed in this launch (fixed offset)
  uint32_t* dep;       // [kMaxTiles] workgroups of a tile that have left (fixed offset)
  uint64_t* publish;   // [tiles][M][4] tagged words
  uint64_t* owner;     // [tiles][S] tagged XCD id of the workgroup that ran phase A
  uint64_t* release;   // [cring] coefficients-only ring: generation of each slot's gathered tile
  uint64_t* fix_word;  // (launch tag << 32) | number of tokens in fix_list (fixed offset)
  uint32_t* fix_list;  // [T] tokens whose fused pre is recomputed directly (fix_flagged)
  uint32_t* err;
  const int8_t* y_q;      // int8 y [T][C] and its per-token scales [T] (fused modes with kModeYInt8)
  const float* y_scale;
  int64_t T;
  int64_t xts, xrs;    // element strides of x between tokens and between routes: 4C and C, or (a
                       // [T][C] stream broadcast to the routes, coefficients mode only) C and 0, or
                       // C and 128 for its pseudo-routes (see cs)
  int cs;              // channels per split in x's channel space: 128, or 512 for a broadcast stream
                       // split into 4 pseudo-routes of 128 consecutive channels
  int prs;             // rows of the packed projection between two routes: C, or 128 (pseudo-routes
                       // over a route-summed projection of C rows)
  int rms_c;           // the RMS scale divides the sum of squares by 4 rms_c: C, or C / 4 when the
                       // split rows cover each channel of a broadcast stream once instead of 4 times
  uint32_t tiles;
  int C;
  int S;
  int d1, d2;
  int lanes;           // persistent kernel: stream workgroups per split
  int recompute_x;     // the pre step never reads x_out back
  int scale_mfma;      // MXFP8 scale bytes in the MX matrix-core operand order (mx_scale_offset)
  Scalars sc;
};

// kModeYInt8 is a flag on the fused modes: y arrives as int8 codes with one
// binary32 scale per token.  kModeBcast is a flag on kModeFused (persistent
// kernel only): the coefficients and pre of a [T][C] stream broadcast to the
// 4 routes, on pseudo-routes, in one pass (no post, no x_out; x holds x0).
// kModeUnit16 is a flag on kModeFused (persistent kernel only, at most 32
// splits): the reduce workgroups take 16-token units, as the broadcast pass
// does.
enum SplitMode { kModeCoeffs = 0, kModeFused = 1, kModeFusedMx = 2, kModeYInt8 = 4, kModeBcast = 8, kModeUnit16 = 16 };
constexpr bool mode_fused(int m) { return (m & 3) == kModeFused || (m & 3) == kModeFusedMx; }
constexpr bool mode_mx(int m) { return (m & 3) == kModeFusedMx; }
constexpr bool mode_yq(int m) { return (m & kModeYInt8) != 0; }
constexpr bool mode_bc(int m) { return (m & kModeBcast) != 0; }
constexpr bool mode_u16(int m) { return (m & (kModeBcast | kModeUnit16)) != 0; }

hipError_t launch_pack_phi(const float* phi, int C, void* out, hipStream_t s);
// Packed route-summed projection of C rows, Phi[c] = ((phi[c] + phi[C+c]) +
// phi[2C+c]) + phi[3C+c], from fp32 phi or (phi == NULL) from the packed
// 4-route projection `packed`.
hipError_t launch_pack_phi_sum(const float* phi, const void* packed, int C, void* out, hipStream_t s);
hipError_t launch_split(const Plan& plan, int mode, const SplitArgs& a, hipStream_t s);
hipError_t launch_post(const uint16_t* x, const uint16_t* y, const float* cf, int64_t T, int C,
                       uint16_t* x_out, hipStream_t s);
hipError_t launch_post_int8(const uint16_t* x, const int8_t* y_q, const float* y_scale, const float* cf, int64_t T,
                            int C, uint16_t* x_out, hipStream_t s);
hipError_t launch_pre(const uint16_t* x, int64_t xts, int64_t xrs, const float* cf, const float* gamma, int64_t T,
                      int C, float rmsnorm_eps, uint16_t* h, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// `iters` Sinkhorn iterations in place on coeffs[t][8..23] (which hold exp(logits)).
hipError_t launch_sinkhorn(float* coeffs, int64_t T, float eps, int iters, hipStream_t s);
// After a persistent fused launch: the direct pre of the tokens it listed
// (the count is read on the device, so it is always launched).

}  // namespace mhc
