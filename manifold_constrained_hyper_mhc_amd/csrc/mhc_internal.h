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

// The split-row kernel covers a tile of M = 16*RB tokens and CC = 4*CW
// channels of every route per workgroup; a token's row is spread over
// S = C / CC workgroups whose partial sums meet in the workspace.
struct Plan {
  int rb = 4;      // 16-token MFMA row blocks per workgroup
  int cw = 32;     // channels per wave
  int m = 64;      // tokens per tile
  int cc = 128;    // channels per workgroup
  int s = 1;       // workgroups per row
  int64_t tiles = 0;
  // workspace layout (byte offsets)
  size_t off_err = 0, off_epoch = 0, off_dep = 0, off_pub = 0, off_part = 0, off_phi = 0, total = 0;
};

constexpr int kPartVals = 24 + kGram;   // per token: projection + route Gram matrix
constexpr int kPackBlocks = 5;          // 80 packed columns = 5 MFMA 16-column blocks
constexpr size_t kPackBytesPerRow = 160;  // 80 bf16 per flattened row k

Plan make_plan(int64_t T, int64_t C);
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
  uint64_t* partials;  // [tiles][S][M][34] tagged words
  uint32_t* epoch;     // [tiles]
  uint32_t* dep;       // [tiles]
  uint64_t* publish;   // [tiles][M][4] tagged words
  uint32_t* err;
  int64_t T;
  int C;
  int S;
  Scalars sc;
};

enum SplitMode { kModeCoeffs = 0, kModeFused = 1, kModeFusedMx = 2 };

hipError_t launch_pack_phi(const float* phi, int C, void* out, hipStream_t s);
hipError_t launch_split(const Plan& plan, int mode, const SplitArgs& a, hipStream_t s);
hipError_t launch_post(const uint16_t* x, const uint16_t* y, const float* cf, int64_t T, int C,
                       uint16_t* x_out, hipStream_t s);
hipError_t launch_pre(const uint16_t* x, const float* cf, const float* gamma, int64_t T, int C,
                      float rmsnorm_eps, uint16_t* h, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace mhc
