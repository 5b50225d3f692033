/*
 * libmhc — the mHC hyper-connection hot path on AMD Instinct MI355X (gfx950).
 *
 * mHC wraps every transformer sublayer with a residual stream of 4 routes
 * ("hc_mult = 4"; hidden size a multiple of 1024), per-token mixing
 * coefficients computed from the RMS-scaled, route-flattened row, a post
 * step that writes the sublayer output back into the stream, and a pre step
 * (combine + RMSNorm) that feeds the next sublayer.  Sources, by page and
 * section:
 *   [P1] "[SM80] Backport mHC fused post + int8 all-reduce; fixes #28, #29",
 *        "What this fixes": post with a fused sum of squares feeding the
 *        prenorm GEMM.
 *   [P2] "[DSv4.1] Integrate Mega-mHC from DeepGEMM", review "Correctness
 *        findings" (route count, hidden % 1024, token limit, scalar names,
 *        the capture contract) and the SM12x comment (the projection takes
 *        the flattened row of width hc_mult * hidden).
 *   [P3] "[DSV4.1] Four BS=1 critical-path fixes for DSpark decode",
 *        "What changed" item 3 and "Correctness" (combine+RMSNorm written in
 *        BF16, MXFP8 epilogue with UE8M0 scales, bitwise equal to the
 *        unfused pair); "Measured and deliberately left out" (per-token mHC
 *        statistics and Sinkhorn; the fused post->pre kernel at T = 6).
 *
 * Conventions for every entry point
 *   - Tensors are device pointers owned by the caller, row-major and
 *     contiguous, 16-byte aligned.  bf16 tensors are passed as raw bits
 *     (uint16_t).  Layouts:
 *       x, x_out  [T][4][C] bf16     residual stream, route-major rows
 *       y         [T][C]    bf16     sublayer output
 *       h         [T][C]    bf16     normalised pre output
 *       coeffs    [T][24]   fp32     {pre[4], post[4] (already times
 *                                     hc_post_scale), res[4][4] row-major,
 *                                     row j = output route}
 *       phi       [4*C][24] fp32     projection, row k = route*C + channel
 *       bias      [24] fp32, gamma [C] fp32
 *       h_fp8     [T][C]    uint8    OCP e4m3fn codes
 *       h_scale   [T][C/32] uint8    UE8M0 exponent bytes (bias 127),
 *                                     linear layout (or, with
 *                                     MHC_FLAG_MXFP8_MFMA_SCALES, the MX
 *                                     matrix-core operand order)
 *   - T is the token count, 0 <= T <= MHC_MAX_TOKENS; T == 0 validates the
 *     scalars and returns MHC_OK without touching memory (pointers may then
 *     be NULL).  C is the hidden size, a positive multiple of 1024 and at
 *     most MHC_MAX_HIDDEN.  The route count is fixed at 4.
 *   - Every argument is validated before any HIP call, so a rejected call
 *     has no effect on the device.  Outputs must not overlap inputs or each
 *     other.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     The library never allocates, frees or synchronises on the call path
 *     and keeps no per-stream state, so calls may be captured in a HIP
 *     graph from the first call on.  Errors of the device work itself
 *     surface at the caller's next synchronisation.
 *   - No exception crosses this interface.  Return values are mhc_status
 *     codes; mhc_strerror() names them and mhc_last_hip_error() gives the
 *     hipError_t behind the last MHC_ERR_HIP of the calling thread.
 */
#ifndef MHC_H_
#define MHC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: coefficients, pre, post, fused post -> pre, packing, workspace.
 * 2: adds mhc_pre_broadcast(_prepacked), mhc_post_int8 and
 *    mhc_post_int8_pre_fused(_prepacked); every version-1 call is unchanged.
 * 3: adds mhc_workspace_check and MHC_ERR_EXPIRED; fused calls recompute the
 *    pre of tokens whose route combination cancels (see mhc_post_pre_fused).
 * 4: adds mhc_post_pre_fused_prepacked_static and MHC_ERR_SCRATCH.
 * 5: adds MHC_FLAG_DEFER_SINKHORN and mhc_sinkhorn.
 * 6: adds MHC_FLAG_MXFP8_MFMA_SCALES. */
#define MHC_ABI_VERSION 6
#define MHC_NUM_ROUTES 4
#define MHC_NUM_COEFFS 24
#define MHC_MAX_TOKENS (1 << 20)  /* [P2] review: the kernel's token limit 2^20 */
#define MHC_MAX_HIDDEN 16384 /* keeps a row within 128 co-resident workgroups */
#define MHC_MXFP8_BLOCK 32
/* Size of the library's static scratch (one per GPU), the workspace of
 * mhc_post_pre_fused_prepacked_static. */
#define MHC_STATIC_SCRATCH_BYTES (64u << 20)

/* Scalars of the method, passed by name ([P2] review warns against a
 * positional float tail whose order differs between two paths). */
typedef struct mhc_params {
  float hc_norm_eps;    /* eps of the RMS scale of the flattened 4C row */
  float rmsnorm_eps;    /* eps of the RMSNorm in pre */
  float hc_post_scale;  /* post = hc_post_scale * sigmoid(logit) */
  float sinkhorn_eps;   /* each Sinkhorn normalisation divides by (sum + eps) */
  int32_t sinkhorn_iters; /* iterations of (rows, then columns); 0..1024 */
} mhc_params;

typedef enum mhc_status {
  MHC_OK = 0,
  MHC_ERR_NULL = 1,       /* a required pointer is NULL */
  MHC_ERR_SHAPE = 2,      /* T or C out of range, C % 1024 != 0 */
  MHC_ERR_ALIGN = 3,      /* a tensor is not 16-byte aligned */
  MHC_ERR_ALIAS = 4,      /* an output overlaps an input or another output */
  MHC_ERR_FLAGS = 5,      /* unknown flag, or outputs inconsistent with flags */
  MHC_ERR_WORKSPACE = 6,  /* workspace NULL, too small or misaligned */
  MHC_ERR_PARAM = 7,      /* a scalar is negative, not finite or out of range */
  MHC_ERR_HIP = 8,        /* a HIP runtime call failed (see mhc_last_hip_error) */
  MHC_ERR_EXPIRED = 9,    /* mhc_workspace_check: a bounded wait of a call that used the
                             workspace expired, so that call's outputs are invalid */
  MHC_ERR_SCRATCH = 10    /* the call needs more workspace than MHC_STATIC_SCRATCH_BYTES */
} mhc_status;

/* Flags of mhc_post_pre_fused. */
#define MHC_FLAG_MXFP8 1u /* also write h as MXFP8: e4m3fn codes + UE8M0 scale per 32 channels */
/* The pre step normally reads x_out back where the same XCD wrote it (its
 * L2 holds the lines) and recomputes x' from x and y elsewhere; with this
 * flag it always recomputes.  Results are bitwise identical either way. */
#define MHC_FLAG_RECOMPUTE_X 2u
/* Decode-latency mode ([P3] "Measured and deliberately left out": the mHC
 * statistics and Sinkhorn run on a side stream, off the critical path of
 * the next projection).  The fused call writes everything as usual except
 * coeffs_next[t][8..23], which it leaves holding exp(logits), the
 * Sinkhorn's input; h (which needs only the pre weights) is complete when
 * the call's work ends.  mhc_sinkhorn then finishes res in place, on any
 * stream ordered after the call (e.g. a side stream waiting on an event
 * recorded after it) and before anything reads res (the next post).  The
 * two calls together write bitwise what one call without the flag writes. */
#define MHC_FLAG_DEFER_SINKHORN 4u
/* With MHC_FLAG_MXFP8: write the UE8M0 scale bytes in the operand order of
 * the gfx950 MX-scaled matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4
 * that a consumer GEMM with h as its A matrix (rows = tokens, K = channels)
 * feeds them from, instead of the linear [T][C/32] layout ([P3]
 * "Correctness": the quantizer's scales are compared as the consumer's
 * swizzled scale block).  In that instruction lane l of a wave holds row
 * l % 16 and the 32 channels of K-block l / 16 of a 128-channel K-tile, i.e.
 * one MX block, and takes its scale from one byte (op_sel) of a 32-bit
 * register.  The layout is [ceil(T/16)][C/512][64][4] bytes: byte
 * ((rb * (C/512) + kg) * 64 + l) * 4 + b holds the scale of token
 * 16 rb + l % 16 and 32-channel block 16 kg + 4 b + l / 16, so one dword
 * per lane carries the scales of the 4 K-tiles 4 kg .. 4 kg + 3 (op_sel b).
 * h_scale then holds ceil(T/16) * 16 * C/32 bytes; the bytes of the rows
 * past T in the last 16-row block are written as those of all-zero blocks
 * (0).  The codes h_fp8 are unchanged. */
#define MHC_FLAG_MXFP8_MFMA_SCALES 8u

/* ---------------------------------------------------------------------------
 * Library information
 * ------------------------------------------------------------------------- */
int mhc_abi_version(void);
const char* mhc_strerror(int status);
/* hipError_t of the last failed HIP call made by this thread (0 if none). */
int mhc_last_hip_error(void);

/* ---------------------------------------------------------------------------
 * Workspace.  mhc_coeffs and mhc_post_pre_fused reduce each token's row
 * across several workgroups and need a caller-owned device workspace of
 * mhc_workspace_bytes(T, C, flags) bytes (256-byte aligned).  Its size is
 * bounded whatever T is: the partial sums live in rings reused as the tiles
 * pass, or a long call runs as several launches, so it holds at most
 * ~128 MiB of partial sums, 4 bytes per token (the list of tokens whose pre
 * is recomputed) and the packed projection (640 C bytes): at most ~143 MiB
 * (T = 2^20, C = 16384), ~130 MiB at T = 8192, C = 7168.  Before its
 * first use a workspace must be cleared with mhc_workspace_init (a kernel on
 * `stream`, no memset node).  Every call leaves it ready for the next one:
 * its counters are reset, and the words it wrote carry that call's launch
 * tag, which no later call accepts.  So it can be reused by any later call
 * with any T and C whose size it covers.  One
 * workspace must not be used by two calls that may run concurrently.
 * Its first 4 bytes are an error word (uint32): the kernels' waits on other
 * workgroups are bounded, and one that expires sets it nonzero, after which
 * that call's outputs are invalid.  Calls never clear it; mhc_workspace_init
 * does.  mhc_workspace_check reads it.  A caller that cannot rule out other
 * work occupying compute units while a persistent-schedule call runs (see
 * Schedule below: kernels on other streams, other processes on the GPU)
 * must check the word before it uses that call's outputs.
 *
 * Schedule.  When 16 <= C/128 <= 64 and T spans enough 32-token tiles
 * (four per stream workgroup), these two calls run a persistent kernel: one
 * 512-thread workgroup per compute unit, every one of which must be
 * resident at once; work that occupies compute units meanwhile delays it,
 * and if that outlasts its bounded waits they expire and set the error word.
 * Otherwise, or with the environment variable MHC_SCHEDULE=staged (read on
 * every call), a staged kernel runs whose workgroups wait only on work of
 * workgroups that started before them (lower-numbered ones, or in a launch
 * of one tile, lower tickets taken in the order of starting).  Results of the two schedules are equal to
 * within the stated tolerances; x_out is bitwise equal, and either
 * schedule's MXFP8 codes are the exact encoding of its own bf16 h.
 * ------------------------------------------------------------------------- */
size_t mhc_workspace_bytes(int64_t T, int64_t C, unsigned flags);
/* Reads the workspace's error word: enqueues a 4-byte device-to-host copy on
 * `stream` and synchronises with it (the only synchronising call of the
 * library; it is not for graph capture).  Returns MHC_OK when no bounded wait
 * of any call that used the workspace since its last mhc_workspace_init has
 * expired, MHC_ERR_EXPIRED when one has (those calls' outputs are invalid;
 * mhc_workspace_init clears the word), MHC_ERR_WORKSPACE for a NULL or
 * misaligned workspace, MHC_ERR_HIP if the copy or the synchronisation fails. */
int mhc_workspace_check(const void* workspace, void* stream);
/* Which kernel mhc_coeffs and mhc_post_pre_fused run for T tokens and
 * channel count C on the current device under the current MHC_SCHEDULE:
 * writes MHC_SCHEDULE_STAGED or MHC_SCHEDULE_PERSISTENT to *schedule.
 * Returns MHC_ERR_NULL or MHC_ERR_SHAPE (nothing written) on bad arguments.
 * Queries the device's compute-unit count (no launch, no allocation). */
enum { MHC_SCHEDULE_STAGED = 0, MHC_SCHEDULE_PERSISTENT = 1 };
int mhc_schedule(int64_t T, int64_t C, int* schedule);
int mhc_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Coefficients ([P1] "What this fixes": the sum of squares feeding the
 * prenorm GEMM; [P2] SM12x comment: the projection takes the flattened row;
 * [P3] "Measured and deliberately left out": mHC statistics and Sinkhorn).
 * Per token t:
 *   r      = 1 / sqrt(sum_{i,c} x[t][i][c]^2 / (4C) + hc_norm_eps)
 *   l[m]   = r * sum_{k} x_flat[t][k] * phi[k][m] + bias[m],  k = i*C + c
 *   pre    = sigmoid(l[0..3]); post = hc_post_scale * sigmoid(l[4..7])
 *   res    = sinkhorn_iters x (rows then columns, each divided by its
 *            sum + sinkhorn_eps) applied to exp(l[8..23]) as 4x4, row j =
 *            output route
 * Writes coeffs [T][24].  Uses the workspace (see above).
 * ------------------------------------------------------------------------- */
int mhc_coeffs(const uint16_t* x, int64_t T, int64_t C, const float* phi, const float* bias,
               const mhc_params* p, float* coeffs, void* workspace, size_t workspace_bytes,
               void* stream);

/* ---------------------------------------------------------------------------
 * Pre: combine + RMSNorm ([P3] "What changed" item 3: the combine+norm
 * output is written in BF16 and feeds the sublayer's first projection).
 *   g[c] = sum_i pre[t][i] * x[t][i][c]
 *   h[t][c] = bf16_rne(g[c] / sqrt(mean_c g^2 + rmsnorm_eps) * gamma[c])
 * pre is read from coeffs[t][0..3] (stride 24).
 * ------------------------------------------------------------------------- */
int mhc_pre(const uint16_t* x, const float* coeffs, const float* gamma, int64_t T, int64_t C,
            const mhc_params* p, uint16_t* h, void* stream);

/* ---------------------------------------------------------------------------
 * Pre of a broadcast input ([P2] review, SM12x comment: the first layer's
 * pre takes a (T, H) input that stands for every route, which the
 * route-flattened GEMM path cannot take as it is).  x0 [T][C] bf16 is the
 * stream of all 4 routes, x[t][i][c] = x0[t][c]; the call computes
 * mhc_coeffs and then mhc_pre of that stream, reading x0 (2C bytes per
 * token) instead of a [T][4][C] copy.  Writes coeffs [T][24] (pre, post,
 * res of this layer) and h [T][C] bf16.  Uses the workspace (see above);
 * the same bounds, alignment and aliasing rules as mhc_coeffs and mhc_pre.
 * From C = 3072 (or T <= 16 at C = 2048) the coefficients are computed on
 * pseudo-routes: a split takes 512 consecutive channels of x0 against the
 * projection summed over the routes and rounded to binary32, so they are
 * not bitwise those of mhc_coeffs on the explicit [T][4][C] copy; both
 * meet the same bounds against the plain definition.  Where the persistent
 * schedule runs (8 to 32 splits of 512 channels, so 4096 <= C, at least
 * two 32-token tiles per stream workgroup, MHC_SCHEDULE not "staged"), one
 * launch computes both, each workgroup holding its x0 slices in registers
 * until their coefficients are published (x0 is read once):
 * h = bf16_rne((q * x0[c]) * gamma[c])
 * with psum = ((pre0 + pre1) + pre2) + pre3 and q = psum / sqrt(psum^2 *
 * sum_c x0^2 / C + rmsnorm_eps), all binary32.  Otherwise a pre launch
 * (mhc_pre's arithmetic on g = psum * x0) follows the coefficients.
 * ------------------------------------------------------------------------- */
int mhc_pre_broadcast(const uint16_t* x0, int64_t T, int64_t C, const float* phi, const float* bias,
                      const float* gamma, const mhc_params* p, float* coeffs, uint16_t* h, void* workspace,
                      size_t workspace_bytes, void* stream);
int mhc_pre_broadcast_prepacked(const uint16_t* x0, int64_t T, int64_t C, const void* phi_packed, const float* bias,
                                const float* gamma, const mhc_params* p, float* coeffs, uint16_t* h,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Post ([P2] "Purpose"/review: the mHC post kernel).
 *   x_out[t][j][c] = bf16_rne(sum_i res[t][j][i] * x[t][i][c] + post[t][j] * y[t][c])
 * post and res are read from coeffs[t][4..23].  The value that is rounded is
 * the binary32 chain  a = post_j * y;  a = fma(res[j][i], x_i, a) for
 * i = 0..3  (a fixed order, so the bf16 result is reproducible).
 * ------------------------------------------------------------------------- */
int mhc_post(const uint16_t* x, const uint16_t* y, const float* coeffs, int64_t T, int64_t C,
             uint16_t* x_out, void* stream);

/* ---------------------------------------------------------------------------
 * Post of an int8 sublayer output ([P1] "What this fixes": the tensor-
 * parallel all-reduce of the sublayer output runs in int8 and hands the
 * post kernel the int8 values with one scale per token).
 *   y[t][c] = binary32(y_q[t][c] * y_scale[t])
 * then exactly mhc_post's chain with this y in place of the bf16 y:
 *   x_out[t][j][c] = bf16_rne(a),  a = post_j * y;  a = fma(res[j][i], x_i, a), i = 0..3.
 * y_q [T][C] int8 (two's complement, any value in [-128, 127]), y_scale
 * [T] fp32, both device memory owned by the caller and read only.  Same
 * shape, alignment (16 bytes for every pointer) and aliasing rules as
 * mhc_post; returns MHC_ERR_NULL / MHC_ERR_ALIGN / MHC_ERR_ALIAS /
 * MHC_ERR_SHAPE before any HIP call, MHC_ERR_HIP if the launch fails.
 * ------------------------------------------------------------------------- */
int mhc_post_int8(const uint16_t* x, const int8_t* y_q, const float* y_scale, const float* coeffs, int64_t T,
                  int64_t C, uint16_t* x_out, void* stream);

/* ---------------------------------------------------------------------------
 * Fused post -> next pre ([P2] "Purpose"/review: the fused post->pre kernel
 * and Mega-mHC; [P1]: the shared sum of squares; [P3] item 3: the MXFP8
 * epilogue).  In one pass over the stream:
 *   x_out       = mhc_post(x, y, coeffs)
 *   coeffs_next = mhc_coeffs(x_out; phi_next, bias_next)   (from the bf16 x_out)
 *   h           = mhc_pre(x_out, coeffs_next, gamma_next)
 * and with MHC_FLAG_MXFP8, per 32-channel block of the bf16 h: amax = max|h|,
 * e = the smallest integer with amax <= 448 * 2^e (clamped to [-127, 127],
 * -127 for an all-zero block), h_scale = e + 127, h_fp8 = e4m3fn_rne(h * 2^-e).
 * h may be NULL when MHC_FLAG_MXFP8 is set; h_fp8 and h_scale are required
 * with the flag and must be NULL without it.
 * The fused pass takes sum_c g^2 of the pre from the route Gram matrix
 * G_ij = sum_c x'_i x'_j as pre^T G pre, which shares the pass with the
 * coefficients ([P1] "What this fixes": the sum of squares fused into post).
 * Where the routes of g = sum_i pre_i x'_i cancel (pre^T G pre <= B / 64,
 * B = (sum_i |pre_i| sqrt(G_ii))^2), that difference of large fp32 terms is
 * not accurate enough; such tokens are listed in the workspace and their h
 * (and MXFP8 blocks) is recomputed after the pass, in binary64, from x'
 * recomputed from x, y and coeffs (the inputs), within the same launch: by
 * its last workgroup (staged launches, and persistent ones with MXFP8), or
 * by its last reduce workgroup (persistent launches without MXFP8).
 * An exactly cancelling combination (g = 0) gives h = 0.
 *
 * Placement (performance only).  A workgroup reads x and writes x_out at the
 * same offsets within their rows (and y and h).  When x_out starts at the
 * same address modulo 1 KiB as x, those reads and writes meet in the same
 * memory channels and the pass measured 3-4% slower on MI355X (prefill
 * T = 8192, C = 7168: 267 against 257 us); starting x_out 256, 512 or 768
 * bytes past x modulo 1 KiB (and h past y) avoids it.  The Python binding
 * allocates its outputs that way.
 * ------------------------------------------------------------------------- */
int mhc_post_pre_fused(const uint16_t* x, const uint16_t* y, const float* coeffs,
                       const float* phi_next, const float* bias_next, const float* gamma_next,
                       int64_t T, int64_t C, const mhc_params* p, unsigned flags,
                       uint16_t* x_out, float* coeffs_next, uint16_t* h, uint8_t* h_fp8,
                       uint8_t* h_scale, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The deferred Sinkhorn of MHC_FLAG_DEFER_SINKHORN: p->sinkhorn_iters
 * iterations (rows, then columns, each divided by sum + p->sinkhorn_eps) in
 * place on coeffs[t][8..23] (row-major 4x4, row j = output route) for
 * t < T; the other coefficient slots are not touched.  coeffs [T][24] fp32,
 * device memory owned by the caller, 16-byte aligned.  Validates like the
 * other calls (MHC_ERR_SHAPE, MHC_ERR_PARAM, MHC_ERR_NULL, MHC_ERR_ALIGN)
 * before its one launch on `stream`; T == 0 is a no-op.
 * ------------------------------------------------------------------------- */
int mhc_sinkhorn(float* coeffs, int64_t T, const mhc_params* p, void* stream);

/* ---------------------------------------------------------------------------
 * Pre-packed projection.  The two calls above first repack phi (fp32) into
 * the layout the matrix cores read: three bf16 terms per element (hi + mid +
 * lo == phi exactly for |phi| >= 2^-100), in 1 KiB fragments.  A caller
 * whose phi is a fixed weight can pack it once with mhc_pack_phi into a
 * buffer of mhc_phi_packed_bytes(C) bytes (256-byte aligned) and call the
 * _prepacked variants, which skip that step; results are bitwise identical.
 * ------------------------------------------------------------------------- */
size_t mhc_phi_packed_bytes(int64_t C);
int mhc_pack_phi(const float* phi, int64_t C, void* phi_packed, void* stream);
int mhc_coeffs_prepacked(const uint16_t* x, int64_t T, int64_t C, const void* phi_packed,
                         const float* bias, const mhc_params* p, float* coeffs, void* workspace,
                         size_t workspace_bytes, void* stream);
int mhc_post_pre_fused_prepacked(const uint16_t* x, const uint16_t* y, const float* coeffs,
                                 const void* phi_next_packed, const float* bias_next,
                                 const float* gamma_next, int64_t T, int64_t C,
                                 const mhc_params* p, unsigned flags, uint16_t* x_out,
                                 float* coeffs_next, uint16_t* h, uint8_t* h_fp8,
                                 uint8_t* h_scale, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ---------------------------------------------------------------------------
 * mhc_post_pre_fused_prepacked without a workspace argument, for callers that
 * cannot allocate device memory or size a workspace per call: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * call allocates and frees nothing; its workspace is a static device array of
 * MHC_STATIC_SCRATCH_BYTES in the library (one per GPU, zero at load, held
 * until the process ends).  The first call on a device takes the array's
 * address (hipGetSymbolAddress) and enqueues a clear of it on `stream` before
 * its own kernels; later calls reuse it as it was left, which the launch tags
 * make safe (see Workspace above).
 *   - Arguments, outputs, flags and results are those of
 *     mhc_post_pre_fused_prepacked (bitwise the same outputs).
 *   - Limit: the call plans its work for the array: a long staged call
 *     runs as launches of at most 32 MiB of partial sums (more launches than
 *     with a workspace of mhc_workspace_bytes), so that every T and C the
 *     library accepts fits (at most ~46 MiB); a shape that would not fit
 *     returns MHC_ERR_SCRATCH before any HIP call.
 *   - error_word: a caller-owned device uint32 (4-byte aligned, not overlapping
 *     any other argument), required when T > 0; a bounded wait that expires
 *     sets it nonzero and the call's outputs are then invalid.  The library
 *     never clears it.
 *   - Every call on a GPU shares that GPU's array: calls that may overlap in
 *     time on one GPU (two streams, two threads) race and must not be issued.
 * ------------------------------------------------------------------------- */
int mhc_post_pre_fused_prepacked_static(const uint16_t* x, const uint16_t* y, const float* coeffs,
                                        const void* phi_next_packed, const float* bias_next, const float* gamma_next,
                                        int64_t T, int64_t C, const mhc_params* p, unsigned flags, uint16_t* x_out,
                                        float* coeffs_next, uint16_t* h, uint8_t* h_fp8, uint8_t* h_scale,
                                        uint32_t* error_word, void* stream);

/* ---------------------------------------------------------------------------
 * Fused post -> next pre of an int8 sublayer output ([P1] "What this fixes":
 * the mHC post kernel fused with the int8 all-reduce handoff, int8 values
 * plus one scale per token).  Exactly mhc_post_pre_fused with x_out =
 * mhc_post_int8(x, y_q, y_scale, coeffs); every other argument, output,
 * flag, workspace and error rule is that of mhc_post_pre_fused.  y_q
 * [T][C] int8 and y_scale [T] fp32 are device memory owned by the caller,
 * read only, 16-byte aligned; MHC_ERR_NULL if either is NULL with T > 0.
 * ------------------------------------------------------------------------- */
int mhc_post_int8_pre_fused(const uint16_t* x, const int8_t* y_q, const float* y_scale, const float* coeffs,
                            const float* phi_next, const float* bias_next, const float* gamma_next, int64_t T,
                            int64_t C, const mhc_params* p, unsigned flags, uint16_t* x_out, float* coeffs_next,
                            uint16_t* h, uint8_t* h_fp8, uint8_t* h_scale, void* workspace, size_t workspace_bytes,
                            void* stream);
int mhc_post_int8_pre_fused_prepacked(const uint16_t* x, const int8_t* y_q, const float* y_scale,
                                      const float* coeffs, const void* phi_next_packed, const float* bias_next,
                                      const float* gamma_next, int64_t T, int64_t C, const mhc_params* p,
                                      unsigned flags, uint16_t* x_out, float* coeffs_next, uint16_t* h,
                                      uint8_t* h_fp8, uint8_t* h_scale, void* workspace, size_t workspace_bytes,
                                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H_ */
