/*
 * libw4a16 -- W4A16 linear layer for AMD Instinct MI355X (gfx950).
 *
 *   y[M, N] = x[M, K] . dequant(Wq)^T (+ bias[N])
 *
 * The operation is the one the page "[ROCm][Kernel] Add
 * HybridW4A16LinearKernel: Triton prefill + HIP skinny decode" describes in
 * its description: fp16/bf16 activations, 4-bit weights packed eight per
 * int32 in an [N, K/8] tensor shared by the decode and prefill paths,
 * symmetric uint4b8 (w = (q - 8) * s) or asymmetric uint4 (w = (q - zp) * s)
 * with one scale (and zero point) per row and group of 32, 64 or 128
 * consecutive k; small M goes to a skinny decode kernel, larger M to a
 * dequantising GEMM.  Zero points are packed int32 [N/8, G], eight rows per
 * word, as the page "Upstream sync 67/N: merge 382bbd5144
 * HybridW4A16LinearKernel (conflict)" states in the section "Upstream's Python
 * side is kept -- and it does NOT work here".
 *
 * Layout contract (all tensors contiguous, row-major):
 *   wq     int32  [N, K/8]  N * K/8 words.  Each word holds one 8-k slice of
 *                           a row: the weight at k = 8L + (0,2,4,6,1,3,5,7)[t]
 *                           of slice L sits in nibble t (bits 4t..4t+3).  A
 *                           row's words are in slice order except inside each
 *                           complete run of 16 words (128 k), stored as the 4x4
 *                           transpose: run word 4r+t holds slice 4t+r of the
 *                           run; a last, incomplete run stays in slice order.
 *                           Rows form tiles of 16.  A complete tile i occupies
 *                           words [16i*K/8, 16(i+1)*K/8): for each complete run
 *                           u, a block of 256 words at offset 256u whose word
 *                           4(16r + j) + e is run word 4r+e of the tile's row j;
 *                           after the blocks, the rows' incomplete runs, row
 *                           after row.  A last, incomplete tile (N % 16 != 0)
 *                           stores its rows one after another, K/8 words each.
 *                           w4a16_pack_weights / w4a16_unpack_weights convert.
 *                           Bits are unsigned (int32 or uint32 storage).
 *   zp     int32  [N/8, G]  nibble i of word (r, j) is the zero point of row 8r+i
 *                           and group j.  NULL selects symmetric uint4b8 (z = 8).
 *   scales act    [N, G]    G = K / group_size.
 *   x      act    [M, K]    y act [M, N]; bias act [N] or NULL.
 *   act is fp16 (W4A16_F16) or bf16 (W4A16_BF16), one dtype for x, scales,
 *   bias and y.
 *
 * Numerics: the library computes with the exact dequantised weights
 * (q - z) * s, accumulates in fp32, adds the bias in fp32 and rounds each
 * output once, to nearest-even, to the activation dtype.  w4a16_dequant
 * returns (q - z) * s rounded once, to nearest-even, to the activation dtype.
 * Range: with bf16, the prefill GEMM (the path taken above the decode
 * threshold) forms q * s as (q * 2^-9) * (s * 2^9), so it needs
 * |s| < 2^119 (s * 2^9 finite); a larger scale gives a non-finite output
 * there.  Every other path, and w4a16_dequant, takes any finite scale.
 *
 * Conventions shared by every entry point:
 *   - The caller owns every buffer.  The library keeps no pointer after a
 *     call returns and allocates no device memory in any call.
 *   - Device entry points are asynchronous on `stream` (a hipStream_t; NULL is
 *     the default stream).  They never synchronise and make no HIP call that
 *     is illegal during stream capture once a device has been initialised
 *     (the first call on a device queries its properties).
 *   - Errors are reported by the returned status and a thread-local message
 *     (w4a16_last_error); the library never aborts and never prints.
 *   - Only gfx950 is supported; other devices get W4A16_ERR_UNSUPPORTED.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 4

typedef enum w4a16_status {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1,  /* bad shape, group size, NULL pointer, aliasing */
  W4A16_ERR_UNSUPPORTED = 2,  /* device is not gfx950, or the case is outside the accept set */
  W4A16_ERR_ALIGNMENT = 3,    /* a pointer is not aligned as required */
  W4A16_ERR_DEVICE = 4,       /* a HIP runtime query failed */
  W4A16_ERR_LAUNCH = 5,       /* a kernel launch failed */
  W4A16_ERR_WORKSPACE = 6     /* workspace missing or smaller than w4a16_workspace_size */
} w4a16_status;

typedef enum w4a16_dtype { W4A16_F16 = 0, W4A16_BF16 = 1 } w4a16_dtype;

typedef enum w4a16_path {
  W4A16_PATH_AUTO = 0,  /* pick by M, N, K, group and dtype */
  W4A16_PATH_GEMV = 1,  /* skinny split-K decode kernel (M <= W4A16_GEMV_MAX_M) */
  W4A16_PATH_GEMM = 2   /* prefill MFMA GEMM (weights dequantised in registers) */
} w4a16_path;

/* Largest M the skinny decode kernel accepts (one MFMA tile of tokens; above
 * it the prefill GEMM is faster at every measured shape). */
#define W4A16_GEMV_MAX_M 16

/* ABI version of the loaded library (W4A16_ABI_VERSION it was built with). */
int w4a16_abi_version(void);

/* Re-reads the tuning environment variables (host only).  The library reads
 * them once, at the first call that needs them, so that a launch makes no
 * getenv call; a process that changes them afterwards (a sweep, a test) calls
 * this.  None of them is needed for correct results:
 *   W4A16_FORCE_PATH=gemv|gemm, W4A16_M_THRESHOLD=<m>  path selection
 *   W4A16_GEMM_TILE=mb,splits[,two_pass[,cb]]        prefill tile and K split
 *   W4A16_GEMV_KPW=<k>, W4A16_GEMV_SPLITS=<s>         decode k-steps per wave, K splits
 *   W4A16_GEMV_NO_WGSZ=1                              decode: per-wave scale loads
 *   W4A16_GEMV_NO_ONE=1                               decode: few tokens on the general kernel
 *   W4A16_LOG=1                                       one line per call on stderr
 * Must not run concurrently with other library calls. */
void w4a16_reload_tuning(void);

/* Message describing the last failing call on this thread ("" after success).
 * Valid until the next library call on the same thread. */
const char* w4a16_last_error(void);

/* ---------------------------------------------------------------- host ---
 * Host-side packing, run once per weight.  Buffers are host memory owned by
 * the caller.  q and zp values must lie in 0..15.
 *
 * w4a16_pack_weights:   q uint8 [N, K] -> wq int32 [N, K/8]; K % 8 == 0.
 * w4a16_unpack_weights: the inverse (every 32-bit word is valid input).
 * w4a16_pack_zeros:     z uint8 [N, G] -> zpk int32 [N/8, G]; N % 8 == 0.
 * w4a16_unpack_zeros:   the inverse.
 * Errors: W4A16_ERR_INVALID_ARG on NULL pointers, negative sizes, sizes not
 * divisible as stated, or a code above 15 (nothing is written then).
 */
w4a16_status w4a16_pack_weights(const uint8_t* q, int64_t N, int64_t K, int32_t* wq);
w4a16_status w4a16_unpack_weights(const int32_t* wq, int64_t N, int64_t K, uint8_t* q);
w4a16_status w4a16_pack_zeros(const uint8_t* z, int64_t N, int64_t G, int32_t* zpk);
w4a16_status w4a16_unpack_zeros(const int32_t* zpk, int64_t N, int64_t G, uint8_t* z);

/* Validates the arguments of w4a16_linear without touching any device.
 * The accept set is the one the page "Upstream sync 67/N: merge 382bbd5144
 * HybridW4A16LinearKernel (conflict)" re-tests in its reviewer's item 2: the
 * quantisation types (uint4b8 when zp == NULL, uint4 with zero points), the
 * activation dtypes fp16 / bf16, the group sizes and K divisibility.
 * Rules: group_size in {32, 64, 128} (the pages' accept set), or
 * group_size == K with K % 32 == 0 (per-channel: one scale and zero point per
 * row, scales [N, 1], zp [N/8, 1]); K >= group_size and K % group_size == 0; N >= 1; N % 8 == 0 when zp != NULL; M >= 0;
 * K <= 2^24 (W4A16_ERR_UNSUPPORTED above: the kernels use 32-bit offsets);
 * dtype is W4A16_F16 or W4A16_BF16; x, wq, scales, y non-NULL when M > 0;
 * x and wq 16-byte aligned, scales/bias/y 2-byte aligned, zp 4-byte aligned;
 * y must not overlap x, wq, scales, zp or bias. */
w4a16_status w4a16_check_args(const void* x, const int32_t* wq, const void* scales,
                              const int32_t* zp, const void* bias, const void* y,
                              int64_t M, int64_t N, int64_t K, int32_t group_size,
                              int32_t dtype);

/* The path W4A16_PATH_AUTO resolves to for this problem (host only).  The
 * page "[ROCm][Kernel] Add HybridW4A16LinearKernel: Triton prefill + HIP
 * skinny decode" (description) sends M <= 5 to its skinny decode kernel and
 * larger M to its prefill GEMM; that bound was tuned on RDNA.  Here it is
 * re-measured on MI355X: the decode kernel for M <= 8, except M <= 6 when
 * K > 16384 with 160 Mi weights (N * K) or more and groups of 64 or more; when
 * 4096 < K <= 16384 for M <= 12 below 32 Mi weights; when K <= 4096 for
 * M <= 16 below 20 Mi weights and M <= 9 above, except with N >= 14336
 * (M <= 8); the GEMM above.  Tuning overrides (environment, read
 * once; see w4a16_reload_tuning): W4A16_M_THRESHOLD=<m> moves the bound,
 * W4A16_FORCE_PATH=gemv|gemm forces one path. */
w4a16_path w4a16_select_path(int64_t M, int64_t N, int64_t K, int32_t group_size,
                             int32_t dtype, int32_t has_zp);

/* Workspace bytes w4a16_linear needs for this problem and path (AUTO allowed).
 * 0 means none; otherwise at least 64 KiB.  Layout: the first 64 KiB hold
 * per-tile completion counters (16384; a split layer with more output tiles
 * is run as several launches of at most 16384 tiles), the rest fp32 partial
 * sums of a K split.  The
 * workspace must be zero-filled before its first use; every completed call
 * leaves the counter region zero again (the partial sums are always written
 * before they are read), so one workspace serves later calls of any shape on
 * the same stream.  Calls that overlap in time must not share one. */
size_t w4a16_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size,
                            int32_t dtype, int32_t has_zp, int32_t path);

/* How w4a16_linear_path would run this problem on the current device (host
 * only; 256 CUs, MI355X's count, when no device is visible).  For logging,
 * tuning and tests; the numbers describe the launch, not the result.
 * Errors: W4A16_ERR_INVALID_ARG / W4A16_ERR_UNSUPPORTED as w4a16_check_args
 * for the sizes, group and dtype (M >= 1 here), W4A16_ERR_UNSUPPORTED for
 * W4A16_PATH_GEMV with M > W4A16_GEMV_MAX_M, W4A16_ERR_INVALID_ARG for a NULL
 * out or an unknown path. */
typedef struct w4a16_plan_info {
  int32_t path;            /* W4A16_PATH_GEMV or W4A16_PATH_GEMM (AUTO resolved) */
  int32_t tile_features;   /* output features (rows of wq) per output tile */
  int32_t tile_tokens;     /* tokens per output tile */
  int32_t splits;          /* K ranges per output tile (1: K is not split) */
  int64_t tiles;           /* output tiles */
  int64_t counter_tiles;   /* most output tiles of one launch that keep a
                              completion counter in the workspace (0: none) */
  int32_t launches;        /* kernel launches per call */
  int32_t waves;           /* waves per workgroup */
  int32_t two_pass;        /* 1: the K split is summed by a second kernel */
  int32_t kernel;          /* decode: 1 the few-token instance (M <= 4, and
                              M <= 8 where the general kernel splits K; K a
                              whole number of 128-k steps; group-wise scales;
                              it runs when scales and zero points are also
                              16-byte aligned), 0 the general decode kernel;
                              GEMM: 0 */
  uint64_t workspace_bytes; /* equals w4a16_workspace_size */
  /* GEMM tail launch (0 when there is none): the tiles past the last full
     round of workgroups (K unsplit) run as a second launch of tiles half as
     tall, tail_tile_tokens x tail_tile_features, tail_tiles of them (two per
     tile; halves wholly past M included, they exit at once) */
  int32_t tail_tile_tokens;
  int32_t tail_tile_features;
  int64_t tail_tiles;
} w4a16_plan_info;

w4a16_status w4a16_plan(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t dtype,
                        int32_t has_zp, int32_t path, w4a16_plan_info* out);

/* -------------------------------------------------------------- device ---
 * y = x . dequant(wq, scales, zp)^T (+ bias), on the current HIP device,
 * asynchronously on `stream`.  All pointers are device pointers.  M == 0 is a
 * no-op.  `workspace` may be NULL when w4a16_workspace_size(...) is 0.
 * Errors: any w4a16_check_args error; W4A16_ERR_UNSUPPORTED on a device that
 * is not gfx950; W4A16_ERR_WORKSPACE; W4A16_ERR_DEVICE; W4A16_ERR_LAUNCH. */
w4a16_status w4a16_linear(const void* x, const int32_t* wq, const void* scales,
                          const int32_t* zp, const void* bias, void* y,
                          int64_t M, int64_t N, int64_t K, int32_t group_size,
                          int32_t dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/* w4a16_linear with the path forced (tests and the dispatch sweep).
 * W4A16_PATH_GEMV with M > W4A16_GEMV_MAX_M is W4A16_ERR_UNSUPPORTED. */
w4a16_status w4a16_linear_path(const void* x, const int32_t* wq, const void* scales,
                               const int32_t* zp, const void* bias, void* y,
                               int64_t M, int64_t N, int64_t K, int32_t group_size,
                               int32_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream, int32_t path);

/* Allocation-free variant of w4a16_linear, for callers that cannot allocate
 * device memory or take a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, layout,
 * numerics and results as w4a16_linear with W4A16_PATH_AUTO, minus the
 * workspace: a K split keeps its completion counters and fp32 partial sums in
 * a scratch array of W4A16_NOALLOC_SCRATCH_BYTES that the library holds in
 * device memory, one per GPU, from module load until the process ends.  The
 * call itself allocates nothing.  Its first call on a device looks up that
 * device's array and clears its counters with a kernel on `stream`.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (other streams, other
 * threads) race and give wrong results; serialise them (one stream).
 * Errors: those of w4a16_linear except W4A16_ERR_WORKSPACE; and
 * W4A16_ERR_UNSUPPORTED when the problem needs more split-K workspace than
 * the array holds (w4a16_workspace_size above W4A16_NOALLOC_SCRATCH_BYTES). */
#define W4A16_NOALLOC_SCRATCH_BYTES (64u << 20)
w4a16_status w4a16_linear_noalloc(const void* x, const int32_t* wq, const void* scales,
                                  const int32_t* zp, const void* bias, void* y,
                                  int64_t M, int64_t N, int64_t K, int32_t group_size,
                                  int32_t dtype, void* stream);

/* Dequantised weights w[N, K] (activation dtype): (q - z) * s rounded once to
 * nearest-even.  Device pointers; same layout rules as w4a16_linear. */
w4a16_status w4a16_dequant(const int32_t* wq, const void* scales, const int32_t* zp,
                           void* w, int64_t N, int64_t K, int32_t group_size,
                           int32_t dtype, void* stream);

/* Expert-indexed decode (the fused-MoE skinny W4A16 GEMM the page "Upstream
 * sync 67/N: merge 382bbd5144 HybridW4A16LinearKernel (conflict)" lists in its
 * conflict table beside the linear kernel).  For token m and slot j of its
 * top-k experts, slot s = m * topk + j, expert e = topk_ids[m, j]:
 *   y[s, :] = topk_weights[m, j] * (x_row . dequant(W_e)^T + bias_e)
 * rounded once to the activation dtype; x_row = x[m] (x_per_slot == 0, x is
 * [M, K]) or x[s] (x_per_slot != 0, x is [M * topk, K]).
 *   wq     int32 [E, N, K/8]  expert e's [N, K/8] block in the wq layout above
 *   scales act   [E, N, G]    zp int32 [E, N/8, G] or NULL; bias act [E, N] or NULL
 *   topk_ids int32 [M, topk]  device; an id outside [0, E) gives a zero row
 *   topk_weights fp32 [M, topk] or NULL (1)
 *   y      act   [M * topk, N]
 * Groups as for w4a16_linear.  Every slot is one decode-kernel problem with
 * M = 1 and one K range, so no workspace is used; M * topk <= 65535 and one
 * expert's N*K/2 below 4 GiB.  Device pointers, caller-owned; asynchronous on
 * `stream`.  Alignment: x and wq 16 bytes; zp, topk_ids, topk_weights 4;
 * scales, bias, y 2.  y must not overlap any input.  Errors as w4a16_linear;
 * W4A16_ERR_UNSUPPORTED when K needs more than one workgroup per slot: with
 * N > 16 that is K above 15360, 13312 or 9216 for groups of 128, 64 or 32
 * (per-channel scales count as the largest of these dividing K), except that
 * groups of 64 and 128 also run K up to 16384 when K is a multiple of 256
 * (the single-token decode instance: at most 16 runs of 8 k-steps). */
w4a16_status w4a16_moe_linear(const void* x, const int32_t* wq, const void* scales,
                              const int32_t* zp, const void* bias, const int32_t* topk_ids,
                              const float* topk_weights, void* y, int64_t M, int64_t topk,
                              int64_t E, int64_t N, int64_t K, int32_t group_size,
                              int32_t dtype, int32_t x_per_slot, void* stream);

/* Dequantised prefill copy ("Converge the two W4A16 linear kernels onto the
 * upstream shell", "What this does": the optional dequantized prefill cache).
 * A caller that keeps w = w4a16_dequant(...) resident (N*K activation-dtype
 * values, four times the packed weights) can run prefill as a dense product:
 *   y[M, N] = x[M, K] . w[N, K]^T (+ bias[N])
 * on the matrix cores with fp32 accumulation, the bias added in fp32 before
 * one nearest-even rounding to the activation dtype.  It runs the prefill
 * GEMM's own kernel with the weight fragments loaded from w instead of
 * unpacked from codes, so its results match w4a16_linear's prefill path
 * (the same rounded weights) up to summation order.
 *   x, w: device pointers, contiguous row-major, 16-byte aligned; bias, y:
 *   2-byte aligned; y must not overlap x, w or bias.  K a multiple of 32 (as
 *   for the dequantised weights of any accepted layer); N*K*2 and M*K*2 below
 *   4 GiB.
 *   workspace: device memory of at least w4a16_dense_workspace_size bytes
 *   (0: none, NULL accepted), 256-byte aligned, zero-filled before its first
 *   use and then reusable as w4a16_linear's, not overlapping the other
 *   buffers.
 * Errors: the usual argument, alignment, size (W4A16_ERR_UNSUPPORTED) and
 * workspace codes. */
w4a16_status w4a16_linear_dense(const void* x, const void* w, const void* bias, void* y,
                                int64_t M, int64_t N, int64_t K, int32_t dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes w4a16_linear_dense needs: the split-K workspace of its
 * plan (completion counters and fp32 partial sums, laid out as
 * w4a16_workspace_size describes), 0 when K is not split.  has_bias does not
 * change it.  Host only. */
size_t w4a16_dense_workspace_size(int64_t M, int64_t N, int64_t K, int32_t dtype,
                                  int32_t has_bias);

/* The 4-bit codes q[N, K] (uint8, 0..15) unpacked on the device from wq. */
w4a16_status w4a16_unpack_device(const int32_t* wq, uint8_t* q, int64_t N, int64_t K,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
