// The libmhc C ABI: argument validation, workspace layout and launches.
// Every check runs before the first HIP call, so a rejected call has no
// effect on the device (and the checks can be exercised without a GPU).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "mhc.h"
#include "mhc_internal.h"

// Workspace of mhc_post_pre_fused_prepacked_static, for callers that cannot
// allocate: one copy per GPU, held until the process ends.  Host code never
// uses this name as an address (on the host it is only a stand-in for the
// device symbol); it takes each device's address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MHC_STATIC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MHC_OK;
  g_last_hip_error = (int)e;
  return MHC_ERR_HIP;
}

struct Span {
  const void* p;
  size_t bytes;
};

bool overlaps(Span a, Span b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int64_t T, int64_t C) {
  if (T < 0 || T > MHC_MAX_TOKENS) return MHC_ERR_SHAPE;
  if (C <= 0 || C % 1024 != 0 || C > MHC_MAX_HIDDEN) return MHC_ERR_SHAPE;
  return MHC_OK;
}

int check_params(const mhc_params* p, bool needs_coeff_scalars) {
  if (p == nullptr) return MHC_ERR_NULL;
  auto ok_eps = [](float v) { return isfinite(v) && v >= 0.0f; };
  if (!ok_eps(p->rmsnorm_eps)) return MHC_ERR_PARAM;
  if (needs_coeff_scalars) {
    if (!ok_eps(p->hc_norm_eps) || !ok_eps(p->sinkhorn_eps)) return MHC_ERR_PARAM;
    if (!isfinite(p->hc_post_scale)) return MHC_ERR_PARAM;
    if (p->sinkhorn_iters < 0 || p->sinkhorn_iters > 1024) return MHC_ERR_PARAM;
  }
  return MHC_OK;
}

mhc::Scalars scalars(const mhc_params* p) {
  mhc::Scalars s;
  s.hc_norm_eps = p->hc_norm_eps;
  s.rmsnorm_eps = p->rmsnorm_eps;
  s.hc_post_scale = p->hc_post_scale;
  s.sinkhorn_eps = p->sinkhorn_eps;
  s.sinkhorn_iters = p->sinkhorn_iters;
  return s;
}

// All listed tensors non-null and 16-byte aligned; no output overlaps an
// input or another output.
int check_tensors(const Span* in, int nin, const Span* out, int nout) {
  for (int k = 0; k < nin; ++k)
    if (in[k].p == nullptr) return MHC_ERR_NULL;
  for (int k = 0; k < nout; ++k)
    if (out[k].p == nullptr) return MHC_ERR_NULL;
  for (int k = 0; k < nin; ++k)
    if (!aligned16(in[k].p)) return MHC_ERR_ALIGN;
  for (int k = 0; k < nout; ++k)
    if (!aligned16(out[k].p)) return MHC_ERR_ALIGN;
  for (int o = 0; o < nout; ++o) {
    for (int k = 0; k < nin; ++k)
      if (overlaps(out[o], in[k])) return MHC_ERR_ALIAS;
    for (int k = o + 1; k < nout; ++k)
      if (overlaps(out[o], out[k])) return MHC_ERR_ALIAS;
  }
  return MHC_OK;
}

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

// Bounds of the split kernel's reduce-scatter (ntok * 34 partial words per
// workgroup, runs of at most kRunMax splits per thread); the tile count must
// fit the fixed leave counters.
bool plan_fits(const mhc::Plan& p) {
  const int64_t ntok = (p.m + p.s - 1) / p.s;
  if (ntok > 8 || ntok * mhc::kPartVals > 256) return false;
  return mhc::plan_run_len(p) <= mhc::kRunMax && (p.m == 32 || p.m == 16) && p.tiles <= mhc::kMaxTiles;
}

// Persistent kernel: one 512-thread workgroup per CU, S*L stream workgroups
// plus 32 or 64 reduce workgroups, all resident.  It runs when 16 <= S <= 64
// (8 <= S for the coefficients of a broadcast stream) and each stream
// workgroup gets at least four tiles (two for a broadcast stream), unless the environment
// variable MHC_SCHEDULE is "staged" (read on every call); otherwise the
// staged kernel runs.
bool persistent_allowed() {
  const char* v = getenv("MHC_SCHEDULE");
  return v == nullptr || strcmp(v, "staged") != 0;
}

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// Which call a persistent launch serves: the fused pass (8-token reduce
// units, or 16-token units: kModeUnit16), the coefficients of a 4-route
// stream, those of a broadcast stream on pseudo-routes, or the one-pass
// coefficients and pre of a broadcast stream on pseudo-routes.
enum class Use { kFused, kFused16, kCoeffs, kCoeffsPseudo, kBcastFused };

// The persistent kernel takes 16 to 64 splits per row (8 to 64 for a
// broadcast stream on pseudo-routes); the fused pass and the coefficients
// of a 4-route stream take it for the same shapes.  Its reduce workgroups:
// 32, or 64 at <= 16 splits for the fused pass with 8-token units and the
// broadcast coefficients, and the CUs the stream lanes leave at 17-24
// splits for the fused pass; the one-pass broadcast pre takes 48 at <= 9
// splits, else 32.  At so few splits the stream workgroups' tiles
// are short, and the reduce workgroups, which take one unit at a time and
// wait for its flags and then its values, set the pace at 32; the
// coefficients of a 4-route stream run faster with the two extra stream
// lanes that 32 leave.
void choose_kernel(mhc::Plan& p, Use use = Use::kFused) {
  p.lanes = 0;
  if (!persistent_allowed()) return;
  const bool pseudo = use == Use::kCoeffsPseudo || use == Use::kBcastFused;
  if (p.m != 32 || p.s < (pseudo ? 8 : 16) || p.s > 64) return;
  const int cus = device_cus();
  // (the broadcast pass balances its stream lanes against its reduce
  // workgroups, T = 8192: at 8 splits 48 reduce workgroups gave 48-49 us
  // against 59 with 32 and 50 with 64; at 10 splits 32 and 48 both 58 us;
  // at 12-16 splits 32 was the fastest, 66 us against 75 with 48 at 14)
  const int reds = use == Use::kBcastFused ? (p.s <= 9 ? 48 : 32)
                                           : (p.s <= 16 && (use == Use::kFused || use == Use::kCoeffsPseudo) ? 64 : 32);
  // the lane count that decides the schedule: with 32 reduce workgroups
  // outside a broadcast stream, so that both calls take the same one
  int lanes = (cus - (pseudo ? reds : 32)) / p.s;
  // the workspace's rings hold kRingK tiles per stream workgroup lane
  if (lanes * p.s > mhc::kMaxLaneSplits) lanes = mhc::kMaxLaneSplits / p.s;
  // Enough tiles for the persistent kernel's fixed cost: four per stream
  // workgroup (two for the broadcast coefficients).  Below that the staged
  // kernel measured faster: at C = 7168 (4 lanes) up to 12 tiles (T = 384:
  // 33.0 vs 35.0 us fused), at C = 4096 (7 lanes) up to 24 (T = 768: 33.2 vs
  // 37.8 us), at C = 2048 (14 lanes) up to 64 (T = 2048: 39.4 vs 41.0 us);
  // above, the persistent one (T = 512 at C = 7168: 38.0 vs 39.8 us).
  // (the broadcast pre's one pass takes over from its two passes at two
  // tiles per stream workgroup: at C = 7168, T = 1536 29.7 against 34.5 us)
  if (lanes < 1 || p.tiles < (use == Use::kCoeffsPseudo || use == Use::kBcastFused ? 2 : 4) * (int64_t)lanes) return;
  lanes = std::min(lanes, (cus - reds) / p.s);
  if (lanes < 1 || p.s * lanes + reds > mhc::kPersistMaxBlocks) return;
  p.lanes = lanes;
  // the fused pass at 17-24 splits (9 to 13 stream lanes, whose tiles come
  // fast) also takes the CUs its stream lanes leave for more reduce
  // workgroups: C = 3072, T = 8192: 137-141 us with 40 against 150-153 with
  // 32; at 40-64 splits the same measured 2-4% slower
  p.reds = (use == Use::kFused || use == Use::kFused16) && p.s > 16 && p.s <= 24
               ? std::max(reds, std::min(64, cus - p.s * lanes))
               : reds;
}

int check_workspace(const void* ws, size_t bytes, const mhc::Plan& plan) {
  if (!plan_fits(plan)) return MHC_ERR_SHAPE;
  if (ws == nullptr) return MHC_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return MHC_ERR_WORKSPACE;
  if (bytes < plan.total) return MHC_ERR_WORKSPACE;
  return MHC_OK;
}

}  // namespace

namespace mhc {

// Stage delays of the reduce (d1) and the pre step (d2) behind a tile's
// phase A in a staged launch of `tiles` tiles: a few stages absorb the spread
// of workgroup progress; a short launch keeps them short so that its few
// tiles are not delayed.
static void set_delays(Plan& p, int64_t tiles) {
  if (tiles >= 64) {
    p.d1 = 12;
    p.d2 = 16;
  } else {
    p.d1 = 1;
    p.d2 = 2;
  }
}

// Tile shape: 32 tokens x 128 channels (of every route) per workgroup.
Plan make_plan(int64_t T, int64_t C, size_t staged_budget) {
  Plan p;
  p.m = T <= 16 ? 16 : 32;  // a decode-sized call takes one 16-token tile
  p.cc = 128;
  p.s = (int)(C / p.cc);
  p.tiles = (T + p.m - 1) / p.m;
  // staged launches: at most staged_budget bytes of partial words each
  const size_t tile_words = (size_t)p.s * p.m * kPartVals * sizeof(uint64_t);
  int64_t chunk = (int64_t)(staged_budget / tile_words);
  chunk = chunk < 16 ? 16 : (chunk > 256 ? 256 : chunk);
  p.chunk_tiles = p.tiles < chunk ? p.tiles : chunk;
  set_delays(p, p.chunk_tiles);
  // persistent rings (32-token tiles, at most 64 splits: where the
  // persistent kernel can run): fused kRingK tiles per lane, coefficients
  // only coeffs_ring_tiles(s)
  int64_t ring_f = 0, ring_c = 0;
  if (p.m == 32 && p.s <= 64) {
    ring_f = (int64_t)kRingK * (kMaxLaneSplits / p.s);
    ring_f = p.tiles < ring_f ? p.tiles : ring_f;
    const int64_t cr = coeffs_ring_tiles(p.s);
    ring_c = p.tiles < cr ? p.tiles : cr;
  }
  size_t part = (size_t)p.chunk_tiles * tile_words;
  // persistent passes: binary32 values in their ring, then one release flag
  // per (slot, split, row block), after the larger of the two rings' values
  const size_t vals_f = (size_t)ring_f * p.s * p.m * kPartVals * sizeof(float);
  const size_t vals_c = (size_t)ring_c * p.s * p.m * kCoeffsWords * sizeof(float);
  const size_t flag_rel = round256(vals_f > vals_c ? vals_f : vals_c);
  const int64_t ring_max = ring_f > ring_c ? ring_f : ring_c;
  const size_t part_r = flag_rel + (size_t)ring_max * p.s * 2 * sizeof(uint64_t);
  part = part > part_r ? part : part_r;
  const int64_t pub_tiles = p.chunk_tiles > ring_f ? p.chunk_tiles : ring_f;
  size_t off = kWsHeaderBytes;
  p.off_pub = off;
  off = round256(off + (size_t)pub_tiles * p.m * 4 * sizeof(uint64_t));
  p.off_part = off;
  p.off_flag = off + flag_rel;
  off = round256(off + part);
  p.off_own = off;
  off = round256(off + (size_t)p.chunk_tiles * p.s * sizeof(uint64_t));
  p.off_rel = off;
  off = round256(off + (size_t)kCoeffsRingTilesWide * sizeof(uint64_t));
  p.off_fix = off;
  off = round256(off + (size_t)T * sizeof(uint32_t));
  p.off_phi = off;
  off = round256(off + phi_packed_bytes(C));
  p.total = off;
  return p;
}

Plan chunk_plan(const Plan& p, int64_t tokens) {
  Plan c = p;
  c.lanes = 0;
  c.tiles = (tokens + p.m - 1) / p.m;
  c.chunk_tiles = c.tiles;
  set_delays(c, c.tiles);
  return c;
}

}  // namespace mhc

namespace {

mhc::SplitArgs split_args(const mhc::Plan& plan, void* ws, int64_t T, int64_t C, const mhc_params* p) {
  mhc::SplitArgs a;
  memset(&a, 0, sizeof(a));
  char* base = static_cast<char*>(ws);
  a.err = reinterpret_cast<uint32_t*>(base + mhc::kWsErr);
  a.epoch = reinterpret_cast<uint32_t*>(base + mhc::kWsEpoch);
  a.tiles_done = reinterpret_cast<uint32_t*>(base + mhc::kWsTilesDone);
  a.dep = reinterpret_cast<uint32_t*>(base + mhc::kWsDep);
  a.publish = reinterpret_cast<uint64_t*>(base + plan.off_pub);
  a.partials = reinterpret_cast<uint64_t*>(base + plan.off_part);
  a.pflag = reinterpret_cast<uint64_t*>(base + plan.off_flag);
  a.owner = reinterpret_cast<uint64_t*>(base + plan.off_own);
  a.release = reinterpret_cast<uint64_t*>(base + plan.off_rel);
  a.fix_word = reinterpret_cast<uint64_t*>(base + mhc::kWsFixWord);
  a.fix_list = reinterpret_cast<uint32_t*>(base + plan.off_fix);
  a.T = T;
  a.xts = 4 * C;
  a.xrs = C;
  a.cs = 128;
  a.prs = (int)C;
  a.rms_c = (int)C;
  a.tiles = (uint32_t)plan.tiles;
  a.C = (int)C;
  a.S = plan.s;
  a.d1 = plan.d1;
  a.d2 = plan.d2;
  a.lanes = plan.lanes;
  a.sc = scalars(p);
  return a;
}

// One coefficients or fused call: a single persistent launch, or staged
// launches of at most run.chunk_tiles tiles each, over consecutive tokens,
// every pointer offset to the chunk's first token.  Each fused launch
// recomputes the tokens it listed itself.
int run_split(const mhc::Plan& run, int mode, const mhc::SplitArgs& a, hipStream_t s) {
  int rc;
  if (run.lanes > 0) return hip_status(mhc::launch_split(run, mode, a, s));
  const int64_t chunk = run.chunk_tiles * run.m;
  for (int64_t t0 = 0; t0 < a.T; t0 += chunk) {
    const int64_t n = a.T - t0 < chunk ? a.T - t0 : chunk;
    const mhc::Plan pc = mhc::chunk_plan(run, n);
    mhc::SplitArgs c = a;
    c.T = n;
    c.tiles = (uint32_t)pc.tiles;
    c.d1 = pc.d1;
    c.d2 = pc.d2;
    const int64_t C = a.C;
    c.x = a.x + t0 * a.xts;
    if (a.y) c.y = a.y + t0 * C;
    if (a.y_q) c.y_q = a.y_q + t0 * C;
    if (a.y_scale) c.y_scale = a.y_scale + t0;
    if (a.coeffs_in) c.coeffs_in = a.coeffs_in + t0 * mhc::kCoeffs;
    if (a.x_out) c.x_out = a.x_out + t0 * 4 * C;
    c.coeffs_out = a.coeffs_out + t0 * mhc::kCoeffs;
    if (a.h) c.h = a.h + t0 * C;
    if (a.h_fp8) c.h_fp8 = a.h_fp8 + t0 * C;
    if (a.h_scale) c.h_scale = a.h_scale + t0 * (C / 32);
    if ((rc = hip_status(mhc::launch_split(pc, mode, c, s)))) return rc;
  }
  return MHC_OK;
}

// The coefficients of a [T][C] stream x0 standing for all 4 routes are
// computed on pseudo-routes: a split takes 512 consecutive channels of x0 as
// 4 routes of 128, against the projection summed over the routes (packed
// with launch_pack_phi_sum), so each channel is read and projected once.  Its
// plan is the plan of hidden size C / 4 (C / 512 splits).  Where that plan
// does not fit the staged kernel's reduce (C = 1024, or C = 2048 with
// 32-token tiles), the 4 routes are the same x0 read with route stride 0
// against the 4-route projection.
bool bcast_pseudo(const mhc::Plan& pb) { return plan_fits(pb); }

// Workspace bytes of every layout a call of T tokens and C channels can use.
size_t workspace_need(int64_t T, int64_t C) {
  const size_t a = mhc::make_plan(T, C).total;
  const mhc::Plan pb = mhc::make_plan(T, C / 4);
  return bcast_pseudo(pb) && pb.total > a ? pb.total : a;
}

// bcast: x is a [T][C] stream that stands for all 4 routes.
int coeffs_impl(const uint16_t* x, int64_t T, int64_t C, const float* phi, const void* phi_packed,
                const float* bias, const mhc_params* p, float* coeffs, void* ws, size_t ws_bytes,
                void* stream, bool bcast = false) {
  int rc = check_shape(T, C);
  if (rc) return rc;
  if ((rc = check_params(p, true))) return rc;
  if (T == 0) return MHC_OK;
  const size_t xb = (size_t)T * (bcast ? 1 : 4) * C * 2, cb = (size_t)T * 24 * 4;
  const Span phi_span = phi ? Span{phi, (size_t)4 * C * 24 * 4} : Span{phi_packed, mhc::phi_packed_bytes(C)};
  const Span in[] = {{x, xb}, phi_span, {bias, 96}};
  const Span out[] = {{coeffs, cb}};
  if ((rc = check_tensors(in, 3, out, 1))) return rc;
  mhc::Plan plan = mhc::make_plan(T, C);
  bool pseudo = false;
  if (bcast) {
    const mhc::Plan pb = mhc::make_plan(T, C / 4);
    if (bcast_pseudo(pb)) {
      plan = pb;
      pseudo = true;
    }
  }
  if ((rc = check_workspace(ws, ws_bytes, plan))) return rc;
  const Span wsp{ws, plan.total};
  if (overlaps(wsp, out[0])) return MHC_ERR_ALIAS;
  for (const Span& s : in)
    if (overlaps(wsp, s)) return MHC_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  mhc::Plan run = plan;
  choose_kernel(run, pseudo ? Use::kCoeffsPseudo : Use::kCoeffs);
  mhc::SplitArgs a = split_args(run, ws, T, C, p);
  const void* packed = phi_packed;
  void* dst = static_cast<char*>(ws) + plan.off_phi;
  if (pseudo) {
    if ((rc = hip_status(mhc::launch_pack_phi_sum(phi, phi_packed, (int)C, dst, s)))) return rc;
    packed = dst;
  } else if (phi != nullptr) {
    if ((rc = hip_status(mhc::launch_pack_phi(phi, (int)C, dst, s)))) return rc;
    packed = dst;
  }
  a.x = x;
  if (pseudo) {
    a.xts = C;
    a.xrs = 128;
    a.cs = 512;
    a.prs = 128;
    a.rms_c = (int)(C / 4);
  } else if (bcast) {
    a.xts = C;
    a.xrs = 0;
  }
  a.phi_packed = static_cast<const uint32_t*>(packed);
  a.bias = bias;
  a.coeffs_out = coeffs;
  return run_split(run, mhc::kModeCoeffs, a, s);
}

// Coefficients, then pre, of a [T][C] stream broadcast to the 4 routes:
// where the persistent schedule runs, one pass on pseudo-routes
// (kModeBcast: each stream workgroup keeps its x0 slices in registers until
// their q words arrive, so x0 is read once); otherwise the coefficients
// call, then a pre launch that reads x0 again.
int pre_broadcast_impl(const uint16_t* x0, int64_t T, int64_t C, const float* phi, const void* phi_packed,
                       const float* bias, const float* gamma, const mhc_params* p, float* coeffs, uint16_t* h,
                       void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(T, C);
  if (rc) return rc;
  if ((rc = check_params(p, true))) return rc;
  if (T == 0) return MHC_OK;
  const Span phi_span = phi ? Span{phi, (size_t)4 * C * 24 * 4} : Span{phi_packed, mhc::phi_packed_bytes(C)};
  const Span in[] = {{x0, (size_t)T * C * 2}, phi_span, {bias, 96}, {gamma, (size_t)C * 4}};
  const Span out[] = {{coeffs, (size_t)T * 24 * 4}, {h, (size_t)T * C * 2}};
  if ((rc = check_tensors(in, 4, out, 2))) return rc;
  if (ws != nullptr && overlaps(Span{ws, workspace_need(T, C)}, out[1])) return MHC_ERR_ALIAS;
  const mhc::Plan pb = mhc::make_plan(T, C / 4);
  if (bcast_pseudo(pb)) {
    mhc::Plan run = pb;
    choose_kernel(run, Use::kBcastFused);
    if (run.lanes > 0) {
      if ((rc = check_workspace(ws, ws_bytes, pb))) return rc;
      const Span wsp{ws, pb.total};
      for (const Span& o : out)
        if (overlaps(wsp, o)) return MHC_ERR_ALIAS;
      for (const Span& i : in)
        if (overlaps(wsp, i)) return MHC_ERR_ALIAS;
      hipStream_t s = static_cast<hipStream_t>(stream);
      void* dst = static_cast<char*>(ws) + pb.off_phi;
      if ((rc = hip_status(mhc::launch_pack_phi_sum(phi, phi_packed, (int)C, dst, s)))) return rc;
      mhc::SplitArgs a = split_args(run, ws, T, C, p);
      a.x = x0;
      a.xts = C;
      a.xrs = 128;
      a.cs = 512;
      a.prs = 128;
      a.rms_c = (int)(C / 4);
      a.phi_packed = static_cast<const uint32_t*>(dst);
      a.bias = bias;
      a.gamma = gamma;
      a.coeffs_out = coeffs;
      a.h = h;
      return hip_status(mhc::launch_split(run, mhc::kModeFused | mhc::kModeBcast, a, s));
    }
  }
  if ((rc = coeffs_impl(x0, T, C, phi, phi_packed, bias, p, coeffs, ws, ws_bytes, stream, true))) return rc;
  return hip_status(
      mhc::launch_pre(x0, C, 0, coeffs, gamma, T, (int)C, p->rmsnorm_eps, h, static_cast<hipStream_t>(stream)));
}

// The sublayer output of a fused call: bf16 [T][C], or int8 codes [T][C]
// with one fp32 scale per token.
struct YIn {
  const uint16_t* bf16;
  const int8_t* q;
  const float* scale;
};

// The device address of the static scratch on the current device, taken
// once per device with hipGetSymbolAddress; the first call on a device also
// enqueues a clear of the whole array on `s` (a kernel, no memset node).
int static_scratch(void** out, hipStream_t s) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  int rc = hip_status(hipGetDevice(&dev));
  if (rc) return rc;
  if (dev < 0 || dev >= 64) return MHC_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if ((rc = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))))) return rc;
    if (ptr == nullptr) return MHC_ERR_HIP;
    if ((rc = hip_status(mhc::launch_fill_zero(ptr, MHC_STATIC_SCRATCH_BYTES, s)))) return rc;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return MHC_OK;
}

// err_word: NULL for the workspace's own error word; otherwise (the static
// scratch variant) the caller's device word that a bounded wait which expires
// sets, and ws is ignored: the call runs on the static scratch.
int fused_impl(const YIn& y, const uint16_t* x, const float* coeffs, const float* phi,
               const void* phi_packed, const float* bias, const float* gamma, int64_t T, int64_t C,
               const mhc_params* p, unsigned flags, uint16_t* x_out, float* coeffs_next, uint16_t* h,
               uint8_t* h_fp8, uint8_t* h_scale, void* ws, size_t ws_bytes, void* stream,
               uint32_t* err_word = nullptr) {
  int rc = check_shape(T, C);
  if (rc) return rc;
  if ((rc = check_params(p, true))) return rc;
  if (flags & ~(MHC_FLAG_MXFP8 | MHC_FLAG_RECOMPUTE_X | MHC_FLAG_DEFER_SINKHORN | MHC_FLAG_MXFP8_MFMA_SCALES))
    return MHC_ERR_FLAGS;
  const bool mx = (flags & MHC_FLAG_MXFP8) != 0;
  const bool mfma_scales = (flags & MHC_FLAG_MXFP8_MFMA_SCALES) != 0;
  if (mfma_scales && !mx) return MHC_ERR_FLAGS;
  if (mx) {
    if (T > 0 && (h_fp8 == nullptr || h_scale == nullptr)) return MHC_ERR_NULL;
  } else if (h_fp8 != nullptr || h_scale != nullptr) {
    return MHC_ERR_FLAGS;
  }
  if (T == 0) return MHC_OK;
  if (!mx && h == nullptr) return MHC_ERR_NULL;
  const size_t xb = (size_t)T * 4 * C * 2, yb = (size_t)T * C * 2, cb = (size_t)T * 24 * 4;
  const Span phi_span = phi ? Span{phi, (size_t)4 * C * 24 * 4} : Span{phi_packed, mhc::phi_packed_bytes(C)};
  const bool yq = y.bf16 == nullptr;
  Span in[7] = {{x, xb}, {coeffs, cb}, phi_span, {bias, 96}, {gamma, (size_t)C * 4}};
  int nin = 5;
  if (yq) {
    in[nin++] = {y.q, (size_t)T * C};
    in[nin++] = {y.scale, (size_t)T * 4};
  } else {
    in[nin++] = {y.bf16, yb};
  }
  Span out[5];
  int nout = 0;
  out[nout++] = {x_out, xb};
  out[nout++] = {coeffs_next, cb};
  if (h) out[nout++] = {h, yb};
  if (mx) {
    // the matrix-core scale order covers whole 16-row blocks
    const int64_t scale_rows = mfma_scales ? (T + 15) / 16 * 16 : T;
    out[nout++] = {h_fp8, (size_t)T * C};
    out[nout++] = {h_scale, (size_t)scale_rows * (C / 32)};
  }
  if ((rc = check_tensors(in, nin, out, nout))) return rc;
  // (the static scratch: staged launches of at most kStagedBudgetStatic
  // bytes of partial words, so that every accepted shape fits)
  const mhc::Plan plan = mhc::make_plan(T, C, err_word != nullptr ? mhc::kStagedBudgetStatic : mhc::kStagedBudget);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (err_word != nullptr) {
    // static scratch: every check first, then the scratch's address
    if (!plan_fits(plan)) return MHC_ERR_SHAPE;
    if (plan.total > (size_t)MHC_STATIC_SCRATCH_BYTES) return MHC_ERR_SCRATCH;
    if (((uintptr_t)err_word & 3u) != 0) return MHC_ERR_ALIGN;
    const Span ew{err_word, sizeof(uint32_t)};
    for (int k = 0; k < nin; ++k)
      if (overlaps(ew, in[k])) return MHC_ERR_ALIAS;
    for (int k = 0; k < nout; ++k)
      if (overlaps(ew, out[k])) return MHC_ERR_ALIAS;
    if ((rc = static_scratch(&ws, s))) return rc;
  } else {
    if ((rc = check_workspace(ws, ws_bytes, plan))) return rc;
    const Span wsp{ws, plan.total};
    for (int k = 0; k < nin; ++k)
      if (overlaps(wsp, in[k])) return MHC_ERR_ALIAS;
    for (int k = 0; k < nout; ++k)
      if (overlaps(wsp, out[k])) return MHC_ERR_ALIAS;
  }

  mhc::Plan run = plan;
  choose_kernel(run, !yq && !mx && plan.s <= 32 ? Use::kFused16 : Use::kFused);
  mhc::SplitArgs a = split_args(run, ws, T, C, p);
  if (err_word != nullptr) a.err = err_word;
  const void* packed = phi_packed;
  if (phi != nullptr) {
    void* dst = static_cast<char*>(ws) + plan.off_phi;
    if ((rc = hip_status(mhc::launch_pack_phi(phi, (int)C, dst, s)))) return rc;
    packed = dst;
  }
  a.x = x;
  a.y = y.bf16;
  a.y_q = y.q;
  a.y_scale = y.scale;
  a.coeffs_in = coeffs;
  a.phi_packed = static_cast<const uint32_t*>(packed);
  a.bias = bias;
  a.gamma = gamma;
  a.x_out = x_out;
  a.coeffs_out = coeffs_next;
  a.h = h;
  a.h_fp8 = h_fp8;
  a.h_scale = h_scale;
  a.recompute_x = (flags & MHC_FLAG_RECOMPUTE_X) != 0;
  a.scale_mfma = mfma_scales ? 1 : 0;
  // deferred Sinkhorn: the res slots get exp(logits), mhc_sinkhorn finishes them
  if (flags & MHC_FLAG_DEFER_SINKHORN) a.sc.sinkhorn_iters = 0;
  // 16-token reduce units where the persistent kernel runs at <= 32 splits
  // (bf16 y and h): there the stream lanes' tiles come fast enough for the
  // reduce's throughput to matter
  const bool unit16 = run.lanes > 0 && run.s <= 32 && !yq && !mx;
  const int mode = (mx ? mhc::kModeFusedMx : mhc::kModeFused) | (yq ? mhc::kModeYInt8 : 0) |
                   (unit16 ? mhc::kModeUnit16 : 0);
  // (tokens whose route combination cancels get their pre recomputed directly)
  return run_split(run, mode, a, s);
}

}  // namespace

extern "C" {

int mhc_abi_version(void) { return MHC_ABI_VERSION; }

const char* mhc_strerror(int status) {
  switch (status) {
    case MHC_OK: return "success";
    case MHC_ERR_NULL: return "a required pointer is NULL";
    case MHC_ERR_SHAPE: return "T or C out of range (C must be a positive multiple of 1024)";
    case MHC_ERR_ALIGN: return "a tensor is not 16-byte aligned";
    case MHC_ERR_ALIAS: return "an output overlaps an input or another output";
    case MHC_ERR_FLAGS: return "unknown flag, or outputs inconsistent with the flags";
    case MHC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MHC_ERR_PARAM: return "a scalar parameter is out of range";
    case MHC_ERR_HIP: return "a HIP runtime call failed";
    case MHC_ERR_EXPIRED: return "a bounded wait of a call that used this workspace expired: its outputs are invalid";
    case MHC_ERR_SCRATCH:
      return "T and C need a larger workspace than the static scratch (MHC_STATIC_SCRATCH_BYTES) holds: "
             "use the call with a caller-owned workspace";
    default: return "unknown status";
  }
}

int mhc_last_hip_error(void) { return g_last_hip_error; }

size_t mhc_workspace_bytes(int64_t T, int64_t C, unsigned flags) {
  if (check_shape(T, C) != MHC_OK ||
      (flags & ~(MHC_FLAG_MXFP8 | MHC_FLAG_RECOMPUTE_X | MHC_FLAG_DEFER_SINKHORN | MHC_FLAG_MXFP8_MFMA_SCALES)))
    return 0;
  return workspace_need(T, C);
}

int mhc_schedule(int64_t T, int64_t C, int* schedule) {
  if (schedule == nullptr) return MHC_ERR_NULL;
  const int rc = check_shape(T, C);
  if (rc != MHC_OK) return rc;
  mhc::Plan p = mhc::make_plan(T, C);
  choose_kernel(p);
  *schedule = p.lanes > 0 ? MHC_SCHEDULE_PERSISTENT : MHC_SCHEDULE_STAGED;
  return MHC_OK;
}

int mhc_sinkhorn(float* coeffs, int64_t T, const mhc_params* p, void* stream) {
  if (T < 0 || T > MHC_MAX_TOKENS) return MHC_ERR_SHAPE;
  int rc = check_params(p, true);
  if (rc) return rc;
  if (T == 0) return MHC_OK;
  if (coeffs == nullptr) return MHC_ERR_NULL;
  if (!aligned16(coeffs)) return MHC_ERR_ALIGN;
  return hip_status(mhc::launch_sinkhorn(coeffs, T, p->sinkhorn_eps, p->sinkhorn_iters, static_cast<hipStream_t>(stream)));
}

int mhc_workspace_check(const void* workspace, void* stream) {
  if (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0) return MHC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  int rc = hip_status(hipMemcpyAsync(&word, static_cast<const char*>(workspace) + mhc::kWsErr, sizeof(word),
                                     hipMemcpyDeviceToHost, s));
  if (rc) return rc;
  if ((rc = hip_status(hipStreamSynchronize(s)))) return rc;
  return word != 0u ? MHC_ERR_EXPIRED : MHC_OK;
}

int mhc_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return MHC_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0 || (workspace_bytes & 3u) != 0) return MHC_ERR_WORKSPACE;
  return hip_status(mhc::launch_fill_zero(workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

size_t mhc_phi_packed_bytes(int64_t C) {
  if (check_shape(0, C) != MHC_OK) return 0;
  return mhc::phi_packed_bytes(C);
}

int mhc_pack_phi(const float* phi, int64_t C, void* phi_packed, void* stream) {
  int rc = check_shape(0, C);
  if (rc) return rc;
  if (phi == nullptr || phi_packed == nullptr) return MHC_ERR_NULL;
  if (!aligned16(phi) || ((uintptr_t)phi_packed & 255u) != 0) return MHC_ERR_ALIGN;
  if (overlaps(Span{phi, (size_t)4 * C * 24 * 4}, Span{phi_packed, mhc::phi_packed_bytes(C)})) return MHC_ERR_ALIAS;
  return hip_status(mhc::launch_pack_phi(phi, (int)C, phi_packed, static_cast<hipStream_t>(stream)));
}

int mhc_coeffs(const uint16_t* x, int64_t T, int64_t C, const float* phi, const float* bias,
               const mhc_params* p, float* coeffs, void* workspace, size_t workspace_bytes,
               void* stream) {
  return coeffs_impl(x, T, C, phi, nullptr, bias, p, coeffs, workspace, workspace_bytes, stream);
}

int mhc_coeffs_prepacked(const uint16_t* x, int64_t T, int64_t C, const void* phi_packed,
                         const float* bias, const mhc_params* p, float* coeffs, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return coeffs_impl(x, T, C, nullptr, phi_packed, bias, p, coeffs, workspace, workspace_bytes, stream);
}

int mhc_pre_broadcast(const uint16_t* x0, int64_t T, int64_t C, const float* phi, const float* bias,
                      const float* gamma, const mhc_params* p, float* coeffs, uint16_t* h, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return pre_broadcast_impl(x0, T, C, phi, nullptr, bias, gamma, p, coeffs, h, workspace, workspace_bytes, stream);
}

int mhc_pre_broadcast_prepacked(const uint16_t* x0, int64_t T, int64_t C, const void* phi_packed, const float* bias,
                                const float* gamma, const mhc_params* p, float* coeffs, uint16_t* h,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return pre_broadcast_impl(x0, T, C, nullptr, phi_packed, bias, gamma, p, coeffs, h, workspace, workspace_bytes,
                            stream);
}

int mhc_pre(const uint16_t* x, const float* coeffs, const float* gamma, int64_t T, int64_t C,
            const mhc_params* p, uint16_t* h, void* stream) {
  int rc = check_shape(T, C);
  if (rc) return rc;
  if ((rc = check_params(p, false))) return rc;
  if (T == 0) return MHC_OK;
  const Span in[] = {{x, (size_t)T * 4 * C * 2}, {coeffs, (size_t)T * 24 * 4}, {gamma, (size_t)C * 4}};
  const Span out[] = {{h, (size_t)T * C * 2}};
  if ((rc = check_tensors(in, 3, out, 1))) return rc;
  return hip_status(
      mhc::launch_pre(x, 4 * C, C, coeffs, gamma, T, (int)C, p->rmsnorm_eps, h, static_cast<hipStream_t>(stream)));
}

int mhc_post(const uint16_t* x, const uint16_t* y, const float* coeffs, int64_t T, int64_t C,
             uint16_t* x_out, void* stream) {
  int rc = check_shape(T, C);
  if (rc) return rc;
  if (T == 0) return MHC_OK;
  const size_t xb = (size_t)T * 4 * C * 2;
  const Span in[] = {{x, xb}, {y, (size_t)T * C * 2}, {coeffs, (size_t)T * 24 * 4}};
  const Span out[] = {{x_out, xb}};
  if ((rc = check_tensors(in, 3, out, 1))) return rc;
  return hip_status(mhc::launch_post(x, y, coeffs, T, (int)C, x_out, static_cast<hipStream_t>(stream)));
}

int mhc_post_int8(const uint16_t* x, const int8_t* y_q, const float* y_scale, const float* coeffs, int64_t T,
                  int64_t C, uint16_t* x_out, void* stream) {
  int rc = check_shape(T, C);
  if (rc) return rc;
  if (T == 0) return MHC_OK;
  const size_t xb = (size_t)T * 4 * C * 2;
  const Span in[] = {{x, xb}, {y_q, (size_t)T * C}, {y_scale, (size_t)T * 4}, {coeffs, (size_t)T * 24 * 4}};
  const Span out[] = {{x_out, xb}};
  if ((rc = check_tensors(in, 4, out, 1))) return rc;
  return hip_status(
      mhc::launch_post_int8(x, y_q, y_scale, coeffs, T, (int)C, x_out, static_cast<hipStream_t>(stream)));
}

int mhc_post_pre_fused(const uint16_t* x, const uint16_t* y, const float* coeffs,
                       const float* phi_next, const float* bias_next, const float* gamma_next,
                       int64_t T, int64_t C, const mhc_params* p, unsigned flags, uint16_t* x_out,
                       float* coeffs_next, uint16_t* h, uint8_t* h_fp8, uint8_t* h_scale,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return fused_impl(YIn{y, nullptr, nullptr}, x, coeffs, phi_next, nullptr, bias_next, gamma_next, T, C, p, flags, x_out,
                    coeffs_next, h, h_fp8, h_scale, workspace, workspace_bytes, stream);
}

int mhc_post_pre_fused_prepacked(const uint16_t* x, const uint16_t* y, const float* coeffs,
                                 const void* phi_next_packed, const float* bias_next,
                                 const float* gamma_next, int64_t T, int64_t C,
                                 const mhc_params* p, unsigned flags, uint16_t* x_out,
                                 float* coeffs_next, uint16_t* h, uint8_t* h_fp8,
                                 uint8_t* h_scale, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return fused_impl(YIn{y, nullptr, nullptr}, x, coeffs, nullptr, phi_next_packed, bias_next, gamma_next, T, C, p, flags,
                    x_out, coeffs_next, h, h_fp8, h_scale, workspace, workspace_bytes, stream);
}

int mhc_post_pre_fused_prepacked_static(const uint16_t* x, const uint16_t* y, const float* coeffs,
                                        const void* phi_next_packed, const float* bias_next, const float* gamma_next,
                                        int64_t T, int64_t C, const mhc_params* p, unsigned flags, uint16_t* x_out,
                                        float* coeffs_next, uint16_t* h, uint8_t* h_fp8, uint8_t* h_scale,
                                        uint32_t* error_word, void* stream) {
  if (T > 0 && error_word == nullptr) return MHC_ERR_NULL;
  return fused_impl(YIn{y, nullptr, nullptr}, x, coeffs, nullptr, phi_next_packed, bias_next, gamma_next, T, C, p, flags,
                    x_out, coeffs_next, h, h_fp8, h_scale, nullptr, 0, stream, error_word);
}

int mhc_post_int8_pre_fused(const uint16_t* x, const int8_t* y_q, const float* y_scale, const float* coeffs,
                            const float* phi_next, const float* bias_next, const float* gamma_next, int64_t T,
                            int64_t C, const mhc_params* p, unsigned flags, uint16_t* x_out, float* coeffs_next,
                            uint16_t* h, uint8_t* h_fp8, uint8_t* h_scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (T > 0 && (y_q == nullptr || y_scale == nullptr)) return MHC_ERR_NULL;
  return fused_impl(YIn{nullptr, y_q, y_scale}, x, coeffs, phi_next, nullptr, bias_next, gamma_next, T, C, p, flags,
                    x_out, coeffs_next, h, h_fp8, h_scale, workspace, workspace_bytes, stream);
}

int mhc_post_int8_pre_fused_prepacked(const uint16_t* x, const int8_t* y_q, const float* y_scale,
                                      const float* coeffs, const void* phi_next_packed, const float* bias_next,
                                      const float* gamma_next, int64_t T, int64_t C, const mhc_params* p,
                                      unsigned flags, uint16_t* x_out, float* coeffs_next, uint16_t* h,
                                      uint8_t* h_fp8, uint8_t* h_scale, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (T > 0 && (y_q == nullptr || y_scale == nullptr)) return MHC_ERR_NULL;
  return fused_impl(YIn{nullptr, y_q, y_scale}, x, coeffs, nullptr, phi_next_packed, bias_next, gamma_next, T, C, p,
                    flags, x_out, coeffs_next, h, h_fp8, h_scale, workspace, workspace_bytes, stream);
}

}  // extern "C"
