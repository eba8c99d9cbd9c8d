// Internal interface between the host library (argument checks, device cache,
// dispatch) and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

struct LinearArgs {
  const void* x;
  const int32_t* wq;
  const void* scales;
  const int32_t* zp;  // NULL: symmetric
  const void* bias;   // may be NULL
  void* y;
  int64_t M, N, K;
  int group;  // the kernels' group: 32, 64 or 128 (a divisor of K for per-channel scales)
  int dtype;
  int sG;     // scale / zero-point row stride, in groups: K / group_size
  int gmul;   // 1, or 0 for per-channel scales (every group of a row reads column 0)
  bool dense = false;  // prefill GEMM only: wq points at act-dtype weights w[N, K]
};

// ---- tuning overrides ------------------------------------------------------
// Read from the environment once, at the first call that needs them (so a
// launch costs no getenv), and again on w4a16_reload_tuning().  None is
// needed for correctness; they serve sweeps, tests and experiments.
struct Tuning {
  int force_path;       // W4A16_FORCE_PATH: 0 none, 1 gemv, 2 gemm
  int m_threshold;      // W4A16_M_THRESHOLD: -1 for the measured default
  int gemm_tile[4];     // W4A16_GEMM_TILE "mb,splits[,two_pass[,cb]]"
  int gemm_tile_n;      //   fields given (0: not set)
  int gemv_kpw;         // W4A16_GEMV_KPW: 0 for the planner's choice
  int gemv_splits;      // W4A16_GEMV_SPLITS: 0 for the planner's choice
  bool gemv_no_wgsz;    // W4A16_GEMV_NO_WGSZ: per-wave scale loads only
  bool gemv_no_one;     // W4A16_GEMV_NO_ONE: single tokens on the general decode kernel
  bool log;             // W4A16_LOG: one line per call on stderr
};
const Tuning& tuning();
void reload_tuning();

// ---- workspace ---------------------------------------------------------------
// Both kernels that split K keep one completion counter per output tile at the
// start of the workspace and their fp32 partial sums after this fixed-size
// counter region.  The last workgroup of a tile resets its counter, so the
// region is zero again after every completed call; the partial sums are always
// written in full before they are read, so their stale contents never matter,
// whatever the shape of the previous call.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int64_t kMaxCounters = (int64_t)(kCounterBytes / sizeof(uint32_t));

// ---- skinny decode kernel ------------------------------------------------
// One workgroup owns 16 output rows (one MFMA column tile) and one K range
// ("split"); its waves take the 128-wide k-steps of that range in turn and
// are reduced through LDS.  With more than one split, each workgroup stores
// fp32 partial sums and the last one to finish a row tile adds them up in
// split order (counter in the workspace), so results are deterministic.
// A split layer with more row tiles than kMaxCounters is launched in chunks
// of at most kMaxCounters row tiles (the launches run one after another on
// the stream), so every launch's counters fit the counter region.
constexpr int kGemvRowsPerTile = 16;
constexpr int kGemvKStep = 128;       // k per wave step: 4 chunks of 32
constexpr int kGemvMaxWaves = 16;     // 1024 threads
constexpr int kGemvMaxM = 16;         // one MFMA row tile of tokens
constexpr int kGemvStepsPerWave = 8;
// decode, single token bf16 g128: the workgroup's scales (16 rows x 8 groups
// per wave, bf16) and packed zero points (2 row blocks x 8 groups per wave)
constexpr int kGemvWgSzBytes = kGemvMaxWaves * (16 * 8 * 2 + 2 * 8 * 4);
// K bound: per-lane byte offsets within a row tile, and products of a row
// index below 16 with K or a stride, stay in 24-bit / 32-bit arithmetic
constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int kGemvXSegsPerThread = 8;  // 16-byte x loads per thread when x is staged
// Dynamic LDS per decode workgroup (cross-wave reduction + staged x).  The
// kernel's LDS layout and the host's plan both size it with gemv_lds_bytes,
// and the plan splits K until it fits the budget.  gfx950 has 160 KiB of LDS
// per CU: with at most one row tile per CU a workgroup may take nearly all of
// it (a K split costs a partial-sum hand-off; 2.5 KiB are left for the
// kernel's static LDS: the workgroup scale-fetch array of the single-token
// instance and the split flag); with more tiles than CUs, 64 KiB, so that
// several workgroups are resident on a CU at once.
constexpr size_t kGemvLdsBudget = 160 * 1024 - kGemvWgSzBytes - 256;  // the most any plan uses
constexpr size_t kGemvLdsBudgetShared = 64 * 1024;  // more row tiles than CUs

struct GemvPlan {
  int tiles;             // ceil(N / 16)
  int ksteps;            // ceil(K / 128)
  int splits;            // K ranges per row tile
  int ksteps_per_split;
  int waves;             // waves per workgroup
  int kpw;               // k-steps per wave (upper bound)
  size_t lds_bytes;      // dynamic LDS of one workgroup
  // the few-token instance (gemv_one_kernel, M <= 8), when the shape allows
  // it: k-steps per wave (8 or 4; 0: not this shape), token rows, its waves
  // and LDS.  It runs when, in addition, the scales are group-wise and the
  // scale and zero-point tensors are 16-byte aligned (otherwise the general
  // kernel runs, with the fields above).
  int one_kpw = 0;
  int one_mt = 0;
  int one_waves = 0;     // waves per workgroup: runs per K range
  int one_splits = 1;    // K ranges (partial sums through the workspace when > 1)
  size_t one_lds_bytes = 0;
};

// LDS bytes of one wave's staging region (M <= 16 kernel): x [M][kpw*128 + 8]
// halves, scales [16][groups] halves, zero points [2][groups] words, then
// fp32 x partial sums (16 k each) and per-group x sums [groups][16].  The
// kernel recomputes it from M, kpw and the group, so host and device share it.
__host__ __device__ inline int gemv_wave_lds_bytes(int M, int kpw, int group) {
  const int kr = kpw * kGemvKStep;
  const int ngr = kr / group;
  int b = M * (kr + 8) * 2 + 16 * ngr * 2 + 2 * ngr * 4;
  b = (b + 15) / 16 * 16;
  b += M * (kr / 16) * 4 + ngr * 16 * 4;
  return (b + 15) / 16 * 16;
}
size_t gemv_lds_bytes(int waves, int64_t M, int kpw, int group);
// the few-token instance: per wave, 16 fp32 sums per token row and the run of
// x of each staged token (the MT rows, or the M tokens of an eight-row instance)
inline size_t gemv_one_lds_bytes(int waves, int kpw, int mt, int64_t M) {
  const size_t staged = mt == 8 ? (size_t)M : (size_t)mt;
  // (staged token rows 64 bytes apart beyond their x when there are several)
  return (size_t)waves * (16 * sizeof(float) * (size_t)mt + staged * (2 * (size_t)kpw * kGemvKStep + (mt > 1 ? 64 : 0)));
}
// token rows of the few-token instance for M tokens (0: not served)
inline int gemv_one_rows(int64_t M) { return M == 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : (M <= 8 ? 8 : 0))); }
GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int group, int dtype, int cu_count);
size_t gemv_workspace_bytes(const GemvPlan& p, int64_t M, int64_t N);
// Expert-indexed decode: slots = M * topk products of one token row with the
// expert topk_ids[slot]'s slice of [E, ...] stacks (see w4a16_moe_linear).
struct MoeArgs {
  const int32_t* ids;
  const float* weights;  // NULL: 1
  int64_t topk, experts, slots;
  bool x_per_slot;
};
constexpr int64_t kMaxGridZ = 65535;

hipError_t launch_gemv(const LinearArgs& a, const GemvPlan& p, void* workspace,
                       hipStream_t stream, const MoeArgs* moe = nullptr);
// whether launch_gemv runs the single-token instance for these arguments
bool gemv_one_runs(const LinearArgs& a, const GemvPlan& p, const MoeArgs* moe = nullptr);

// ---- prefill GEMM ----------------------------------------------------------
// A workgroup owns 32*mb tokens x 256 output features; `splits` K ranges of
// `steps_per_split` 128-k steps each; units = tiles * splits workgroups.
struct GemmPlan {
  int mb;                // tile height 32 * mb tokens
  int cb;                // tile width 128 * cb features (cb column blocks of 32 per wave)
  int splits;
  int steps_per_split;
  int tiles_n;
  int tiles;
  int units;
  // K split summed by a second kernel from plain fp32 partials (small M,
  // many splits) instead of by the tile's last workgroup
  bool two_pass;
  // tail launch (K unsplit): the tiles from tail_tile0 on, past the last
  // full round of workgroups, run as a second launch of tiles half as tall
  // (32 tail_mb tokens, two per tile) in one round; tail_units = 0: none.
  // units is then tail_tile0, the first launch's grid.
  int tail_mb, tail_tile0, tail_units;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int group, int dtype, bool asym, int cu_count,
                   bool dense = false);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int group, int dtype, bool asym,
                            int cu_count, bool dense = false);
hipError_t launch_gemm(const LinearArgs& a, void* workspace, int cu_count, hipStream_t stream);

// ---- elementwise -----------------------------------------------------------
hipError_t launch_dequant(const int32_t* wq, const void* scales, const int32_t* zp, int sG, int gmul, void* w,
                          int64_t N, int64_t K, int group, int dtype, hipStream_t stream);
hipError_t launch_unpack(const int32_t* wq, uint8_t* q, int64_t N, int64_t K,
                         hipStream_t stream);
// bytes (a multiple of 4) of device memory set to zero by a kernel
hipError_t launch_zero_words(void* p, size_t bytes, hipStream_t stream);

}  // namespace w4a16
