// Measurement aid (libmhc_bench.so, not part of libmhc): plain copies and
// reads of device memory that give the bandwidth ceilings the fused pass is
// compared with, on the same tensors.
//   kind 0: linear copy   src -> dst, 16 bytes per lane, 4 loads in flight
//   kind 1: linear read   of src (a per-thread xor is stored so the loads stay)
//   kind 2: piece copy    the access pattern of the persistent fused kernel:
//           src is `rows` rows of row_bytes; workgroup (split s, lane r) of
//           S * lanes moves the 256-byte piece s of the 128 rows of tiles
//           r, r + lanes, ... (8 loads of 16 bytes per thread in flight)
//   kind 3: piece read    kind 2 without the stores
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__global__ __launch_bounds__(256) void k_copy_linear(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                     int64_t n, int store, u32x4_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  u32x4_t acc = {0, 0, 0, 0};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
    u32x4_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = i + k * stride < n ? __builtin_nontemporal_load(src + i + k * stride) : acc;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (store) {
        if (i + k * stride < n) __builtin_nontemporal_store(v[k], dst + i + k * stride);
      } else {
        acc ^= v[k];
      }
    }
  }
  if (!store) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_copy_pieces(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                     int64_t rows, int64_t row_bytes, int S, int lanes, int store,
                                                     u32x4_t* __restrict__ sink) {
  const int s = (int)blockIdx.x % S, r = (int)blockIdx.x / S;
  const int tid = threadIdx.x;
  const int64_t tiles = (rows + 127) / 128;
  u32x4_t acc = {0, 0, 0, 0};
  for (int64_t t = r; t < tiles; t += lanes) {
    u32x4_t v[8];
    // 8 rounds of 16 rows x 256 bytes: thread tid takes 16-byte chunk tid % 16 of row round*16 + tid / 16
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = t * 128 + k * 16 + tid / 16;
      v[k] = row < rows ? *reinterpret_cast<const u32x4_t*>(src + row * row_bytes + 256 * s + 16 * (tid % 16)) : acc;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = t * 128 + k * 16 + tid / 16;
      if (store) {
        if (row < rows) *reinterpret_cast<u32x4_t*>(dst + row * row_bytes + 256 * s + 16 * (tid % 16)) = v[k];
      } else {
        acc ^= v[k];
      }
    }
  }
  if (!store) sink[(int64_t)blockIdx.x * 256 + tid] = acc;
}

// Piece copy with a piece width of PB bytes (256, 512, 1024 or 2048): src
// is `rows` rows of row_bytes; S = row_bytes / PB pieces per row; workgroup
// (piece s, lane r) of S * lanes copies piece s of the tiles of 32768 / PB
// rows r, r + lanes, ...: always 8 rounds of 16 bytes per thread per tile,
// so only the width of the contiguous run per row changes.
template <int PB>
__global__ __launch_bounds__(256) void k_copy_wide(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   int64_t rows, int64_t row_bytes, int S, int lanes) {
  constexpr int TPR = PB / 16, RPR = 256 / TPR, TR = 8 * RPR;
  const int s = (int)blockIdx.x % S, r = (int)blockIdx.x / S;
  const int tid = threadIdx.x;
  const int64_t tiles = (rows + TR - 1) / TR;
  const u32x4_t z = {0, 0, 0, 0};
  for (int64_t t = r; t < tiles; t += lanes) {
    u32x4_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = t * TR + k * RPR + tid / TPR;
      v[k] = row < rows ? *reinterpret_cast<const u32x4_t*>(src + row * row_bytes + (int64_t)PB * s + 16 * (tid % TPR))
                        : z;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = t * TR + k * RPR + tid / TPR;
      if (row < rows) *reinterpret_cast<u32x4_t*>(dst + row * row_bytes + (int64_t)PB * s + 16 * (tid % TPR)) = v[k];
    }
  }
}

// Piece copy of src to dst in pieces of piece_bytes with about `workgroups`
// workgroups (lanes = workgroups / (row_bytes / piece_bytes), at least 1).
// Returns 0, 1 for bad arguments (nothing launched), 2 if the launch failed.
extern "C" int bench_copy_pieces(const void* src, void* dst, int64_t rows, int64_t row_bytes, int piece_bytes,
                                 int workgroups, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (src == nullptr || dst == nullptr || rows <= 0 || workgroups <= 0) return 1;
  if (piece_bytes != 256 && piece_bytes != 512 && piece_bytes != 1024 && piece_bytes != 2048) return 1;
  if (row_bytes <= 0 || row_bytes % piece_bytes != 0) return 1;
  const int S = (int)(row_bytes / piece_bytes);
  const int lanes = workgroups / S > 0 ? workgroups / S : 1;
  if ((int64_t)S * lanes > 65536) return 1;
  const dim3 grid((unsigned)(S * lanes)), block(256);
  const auto* s8 = static_cast<const uint8_t*>(src);
  auto* d8 = static_cast<uint8_t*>(dst);
  switch (piece_bytes) {
    case 256: k_copy_wide<256><<<grid, block, 0, st>>>(s8, d8, rows, row_bytes, S, lanes); break;
    case 512: k_copy_wide<512><<<grid, block, 0, st>>>(s8, d8, rows, row_bytes, S, lanes); break;
    case 1024: k_copy_wide<1024><<<grid, block, 0, st>>>(s8, d8, rows, row_bytes, S, lanes); break;
    default: k_copy_wide<2048><<<grid, block, 0, st>>>(s8, d8, rows, row_bytes, S, lanes); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// sink: (kind 1, 3) a device buffer of grid * 256 * 16 bytes: 1024 * 4096
// bytes for kind 1, S * lanes * 4096 for kind 3.  Returns 0, or 1 for bad
// arguments (nothing launched), 2 if the launch failed.
extern "C" int bench_copy(int kind, const void* src, void* dst, int64_t rows, int64_t row_bytes, int lanes,
                          void* sink, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows <= 0 || row_bytes <= 0 || (row_bytes & 255) != 0 || src == nullptr) return 1;
  if ((kind == 0 || kind == 2) && dst == nullptr) return 1;
  if ((kind == 1 || kind == 3) && sink == nullptr) return 1;
  const int64_t n16 = rows * row_bytes / 16;
  if (kind == 0 || kind == 1) {
    k_copy_linear<<<1024, 256, 0, st>>>(static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16,
                                        kind == 0, static_cast<u32x4_t*>(sink));
  } else if (kind == 2 || kind == 3) {
    const int S = (int)(row_bytes / 256);
    if (lanes <= 0 || S * lanes > 4096) return 1;
    k_copy_pieces<<<S * lanes, 256, 0, st>>>(static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows,
                                             row_bytes, S, lanes, kind == 2, static_cast<u32x4_t*>(sink));
  } else {
    return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
