// Skinny split-K W4A16 decode kernel for gfx950 (M <= 16).
//
// The pages' decode path ("[ROCm][Kernel] Add HybridW4A16LinearKernel: Triton
// prefill + HIP skinny decode", description) is a split-K skinny GEMM for
// small M that dequantises with the exponent-OR trick.  These kernels keep the
// split-K idea and the trick, and re-plan the rest for CDNA4:
//
// * Work unit: 16 output rows (one MFMA column tile) x one 128-wide k-step,
//   i.e. one 128-k run of each row.  Lane (j = lane % 16, r = lane / 16)
//   issues one 16-byte non-temporal load per k-step, run words 4r..4r+3 of
//   row n0 + j; the runs are stored as a 4x4 word transpose, so register t
//   holds slice r of chunk t -- exactly the B operand layout of
//   v_mfma_f32_16x16x32 for chunk t, and every MFMA covers 32 k of one
//   quantisation group.  The weights of a complete 16-row tile are stored
//   tile-major, so the 64 lanes' pieces of one run are one contiguous 1 KiB
//   block: whole cache lines, and each load's bytes come back together.  (An
//   incomplete last run, stored in order, is transposed across the four
//   16-lane rows with permlane swaps instead.)
// * The scale is factored out of the dot product: per group the wave forms
//   sum_k x[m,k] * (q[n,k] - z[n,g]) in fp32 and adds s[n,g] times it to the
//   accumulator; nothing is rounded to the activation dtype before the output.
//   B is built by the AND-OR alone (magic + q, exact).  fp16 removes the
//   offset with one packed add per weight pair, (1024 + q) - (1024 + z), exact.
//   bf16 has no packed add on gfx950, so it keeps B = 128 + q and subtracts
//   (128 + z) * sum_k x[m,k] per group in fp32, the group sums of x being
//   formed once per workgroup while x is staged.
// * A workgroup owns one row tile and one K range.  Its waves take
//   contiguous runs of k-steps and issue every load up front, x and the
//   per-group scales and zero points first (staged in LDS, coalesced), then
//   the weights; each k-step waits only for its own weights, so the dot
//   products of early k-steps overlap the arrival of later ones.  Every CU
//   pays roughly the same issue time per load instruction whatever its size,
//   so the loads are few and wide: 1 KiB weight and x loads, and (single
//   token, bf16, groups of 128) one workgroup-wide fetch of the scales and
//   zero points instead of two small loads per wave.
// * The host splits K across workgroups only when a K range needs more than
//   16 waves or the LDS budget: the partial-sum hand-off costs more than idle
//   CUs.  So there is no limit on K * M (the pages' converged kernel likewise
//   streams the overflow from global, "[ROCm] Converge the two W4A16 linear
//   kernels onto the upstream shell", "What this does").
// * Waves are reduced through LDS in wave order; with several K ranges per
//   row tile the partial sums go through the workspace and the last workgroup
//   to arrive adds them in range order.  Results do not depend on scheduling.
//
// gemv_small_kernel serves M <= 16 (one MFMA row tile of tokens).  Above
// that the prefill GEMM is faster at every measured shape.  One token on
// most shapes runs gemv_one_kernel (further below), which keeps only x in
// LDS and finishes each group in the 16-lane row that owns it.
#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"


namespace w4a16 {

struct GemvParams {
  const uint16_t* x;
  const uint32_t* wq;
  const uint16_t* scales;
  const uint32_t* zp;
  const uint16_t* bias;
  uint16_t* y;
  float* partial;      // [splits][M][N] when splits > 1
  uint32_t* counters;  // [launch tiles] when splits > 1; zero between calls
  int tile_base;       // row tile of blockIdx.x == 0: a split layer with more row
                       // tiles than counters is launched in chunks of tiles
  int M, N, K, G;
  int sG, gmul;  // scale / zero-point index of (row n, group g): n * sG + g * gmul
  int nchunks;  // K / 32
  int ksteps;   // ceil(nchunks / 4)
  int ksteps_per_split;
  int splits;
  int kpw;      // k-steps per wave (contiguous runs)
  int waves;    // waves per workgroup
  // per-wave staging geometry (M <= 16 kernel): log2 of the 16-byte x
  // segments per row and of the groups in one wave's run of kpw k-steps, and
  // the bytes of one wave's LDS region
  int lg_xsegs_per_wave;
  int lg_groups_per_wave;
  int wave_lds_bytes;
  float yscale;  // multiplies each sum after the bias (1; an expert slot's router weight)
  // expert-indexed mode (moe_ids != NULL): workgroup z handles slot z, whose
  // expert moe_ids[z] selects slice e of the weight / scale / zp / bias stacks
  const int32_t* moe_ids;
  const float* moe_weights;  // [slots] or NULL
  int topk, experts, x_per_slot;
  size_t w_estride, s_estride, z_estride;  // words / halves / words per expert
  int slots;  // workgroups along z: 1, or the expert slots
};

// One 16-byte global->LDS load per active lane: lane l reads base + off and
// writes LDS bytes lds + 16 l .. lds + 16 l + 15 (lds wave-uniform).  M0
// holds the LDS address for the load (one wait state after it is written) and
// is given back its value afterwards.
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t off, unsigned char* lds) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds_addr), "v"(off), "s"(base) : "memory");
}

// The expert slot of this workgroup (expert-indexed mode): its expert's
// slices, its x row and output row.  False for an id outside [0, experts),
// whose row is zero.
__device__ __forceinline__ bool select_slot(GemvParams& p) {
  const int slot = blockIdx.z;
  const int e = p.moe_ids[slot];
  const size_t xrow = (size_t)(p.x_per_slot ? slot : slot / p.topk);
  p.y += (size_t)slot * p.N;
  if (e < 0 || e >= p.experts) return false;
  p.wq += (size_t)e * p.w_estride;
  p.scales += (size_t)e * p.s_estride;
  if (p.zp) p.zp += (size_t)e * p.z_estride;
  if (p.bias) p.bias += (size_t)e * p.N;
  p.x += xrow * p.K;
  if (p.moe_weights) p.yscale = p.moe_weights[slot];
  return true;
}

// Addresses of one lane's 16-byte weight pieces, run by run, for the row
// tile starting at row n0: lane (r, j) needs run words 4r..4r+3 of row
// n0 + j.  In a complete tile they are piece 16 r + j of the run's 1 KiB
// block; in a final incomplete tile, bytes 16 r of the row's 64-byte run.
// The incomplete last run (chunks 4R.. of K/32) is stored in slice order,
// T = 4 * tail chunks words per row; lanes past it read its last chunk.
// Every address is a wave-uniform base (scalar registers) plus a 32-bit
// per-lane byte offset, the form the loads take without vector address
// arithmetic.
struct WeightWalk {
  const char* base;   // wave-uniform: row n0 of the tile
  uint32_t lane_off;  // complete runs: base + ks * run_bytes + lane_off
  uint32_t run_bytes;
  uint32_t tail_off;  // the incomplete last run: base + tail_off
  int full_runs;
  __device__ __forceinline__ const char* at(int ks) const {
    const bool full = ks < full_runs;  // wave-uniform
    return base + (full ? (size_t)ks * run_bytes : 0) + (size_t)(full ? lane_off : tail_off);
  }
};

__device__ __forceinline__ WeightWalk weight_walk(const uint32_t* wq, int N, int K, int nchunks,
                                                  int n0, int j, int r) {
  WeightWalk w;
  const uint32_t row_bytes = (uint32_t)(K >> 1);
  const int full_runs = nchunks >> 2;
  const int tail_chunks = nchunks - 4 * full_runs;
  const uint32_t tail_piece = 16u * (uint32_t)max(0, min(r, tail_chunks - 1));
  w.full_runs = full_runs;
  w.base = reinterpret_cast<const char*>(wq) + (size_t)n0 * row_bytes;
  if (n0 + kGemvRowsPerTile <= N) {
    w.run_bytes = 1024u;
    w.lane_off = (uint32_t)(16 * r + j) * 16u;
    w.tail_off = (uint32_t)full_runs * 1024u + (uint32_t)j * (uint32_t)(16 * tail_chunks) + tail_piece;
  } else {
    const uint32_t dn = (uint32_t)(min(n0 + j, N - 1) - n0);
    w.run_bytes = 64u;
    w.lane_off = __umul24(dn, row_bytes) + 16u * (uint32_t)r;
    w.tail_off = __umul24(dn, row_bytes) + (uint32_t)full_runs * 64u + tail_piece;
  }
  return w;
}

// Store or hand over the reduced sums of one row tile: with one K range the
// output (+ bias, one rounding); otherwise the fp32 partial, and the last
// workgroup to finish the tile adds the partials in range order.
template <int DT>
__device__ __forceinline__ void finish_tile(const GemvParams& p, const float* red, int nwaves,
                                            int nel, int tile, int split, int* last_flag) {
  uint32_t* const counter = p.counters + (tile - p.tile_base);  // this launch's tiles
  for (int e = threadIdx.x; e < nel; e += blockDim.x) {
    const int mt = e >> 8;
    const int r = (e >> 6) & 3;
    const int l = e & 63;
    const int m = mt * 16 + 4 * (l >> 4) + r;
    const int nn = tile * kGemvRowsPerTile + (l & 15);
    if (m < p.M && nn < p.N) {
      float v = 0.f;
      for (int w = 0; w < nwaves; ++w) v += red[w * nel + e];
      if (p.splits == 1) {
        if (p.bias) v += act_to_f32<DT>(p.bias[nn]);
        p.y[(size_t)m * p.N + nn] = f32_to_act<DT>(v * p.yscale);
      } else {
        store_coherent(p.partial + ((size_t)split * p.M + m) * p.N + nn, v);
      }
    }
  }
  if (p.splits == 1) return;

  // every thread's partial sums have completed (stores count in vmcnt on
  // gfx950; the barrier itself does not wait for them), then one arrival
  wait_vm_all();
  __syncthreads();
  if (threadIdx.x == 0)
    *last_flag = (arrive(counter) == (uint32_t)(p.splits - 1));
  __syncthreads();
  if (!*last_flag) return;
  for (int e = threadIdx.x; e < 16 * p.M; e += blockDim.x) {
    const int m = e >> 4;
    const int nn = tile * kGemvRowsPerTile + (e & 15);
    if (nn < p.N) {
      float v = 0.f;
      for (int s = 0; s < p.splits; ++s) v += load_coherent(p.partial + ((size_t)s * p.M + m) * p.N + nn);
      if (p.bias) v += act_to_f32<DT>(p.bias[nn]);
      p.y[(size_t)m * p.N + nn] = f32_to_act<DT>(v * p.yscale);
    }
  }
  if (threadIdx.x == 0) reset_counter(counter);  // ready for the next call
}

// ---------------------------------------------------------------------------
// M <= 16
// ---------------------------------------------------------------------------
// Each wave stages only what it reads -- x, scales and zero points of its own
// run of k-steps -- in a private LDS region, so no wave waits for another
// before its dot products; the only barrier is the final cross-wave sum.
// All staging index maps are shifts and masks (the per-wave sizes are powers
// of two), keeping the vector-ALU work in front of the weight loads small.
// ONE: a single token (M == 1), whose sums are row 0 of each MFMA result
// (lanes 0..15, register 0); the other rows are then never updated.
// MOE: expert-indexed mode (a separate instance, so that the plain layer has
// no branch in front of its parameter loads and they arrive in one batch).
constexpr int small_waves_per_simd(int kpw, bool one, int gs, int xpt) {
  return kpw == 8 && xpt == 8 ? 4 : (kpw == 8 && !one && gs == 32 ? 6 : 7);
}

// WGSZ (single token, bf16, groups of 128, every wave a full run of 8 k-steps,
// one K range): the workgroup's scales and zero points are fetched once for
// all its waves, by a few 1 KiB global->LDS loads issued first, instead of two
// small loads per wave; every load instruction costs a CU about the same issue
// time whatever its size, and on the large layers that issue time paces the
// weight stream.  Each group's sum is kept in a register and scaled after the
// run, behind one workgroup barrier.
// At most 72 VGPRs (seven waves per SIMD, which runs the largest decode layers'
// workgroups in one round), 80 for the two-token g32 instance, which spills
// at 72; every instance fits without spilling.
// The leading scalar arguments are everything the loads in front of the run
// need; this file is compiled with kernel-argument preloading, so they arrive
// in SGPRs when the wave starts instead of after a scalar load from the
// argument segment (gfx950 preloads plain arguments, not the parameter
// struct).  The other fields that the loads need are derived from them.
template <int DT, int GS, bool ASYM, int KPW, int XPT, bool ONE, bool MOE, bool WGSZ>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(small_waves_per_simd(KPW, ONE, GS, XPT)))) void gemv_small_kernel(const uint16_t* a_x, const uint32_t* a_wq,
                                                          const uint16_t* a_scales, const uint32_t* a_zp,
                                                          int a_M, int a_N, int a_K, int a_sG, int a_gmul,
                                                          int a_kps, const GemvParams params) {
  constexpr int CPG = GS / 32;          // 32-k chunks per group (1, 2, 4)
  constexpr int SPT = (32 * KPW) / GS > 0 ? (32 * KPW) / GS : 1;  // scale loads per lane
  static_assert(!WGSZ || (ONE && DT == DT_BF16 && GS == 128 && KPW == 8), "WGSZ instance");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int last_flag;
  // WGSZ: the workgroup's scales [group piece][16 rows][8 groups] (bf16), then
  // its zero points [group quad][2 row blocks][4 groups] (packed words)
  __shared__ __attribute__((aligned(16))) unsigned char wgsz[WGSZ ? kGemvWgSzBytes : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  GemvParams p = params;
  p.x = a_x;
  p.wq = a_wq;
  p.scales = a_scales;
  p.zp = a_zp;
  p.M = a_M;
  p.N = a_N;
  p.K = a_K;
  p.sG = a_sG;
  p.gmul = a_gmul;
  p.ksteps_per_split = a_kps;
  // as the host sets them (the plan's k-steps per wave is KPW)
  p.G = a_K / GS;
  p.nchunks = a_K >> 5;
  p.ksteps = (p.nchunks + 3) >> 2;
  p.kpw = KPW;
  p.waves = (a_kps + KPW - 1) / KPW;
  p.lg_xsegs_per_wave = __builtin_ctz(KPW * (kGemvKStep / 8));
  p.lg_groups_per_wave = __builtin_ctz(KPW * kGemvKStep / GS > 0 ? KPW * kGemvKStep / GS : 1);
  p.wave_lds_bytes = gemv_wave_lds_bytes(a_M, KPW, GS);
  if constexpr (MOE) {
    if (!select_slot(p)) {
      // not an expert: a zero row (the whole workgroup leaves here)
      const int n = (blockIdx.x + p.tile_base) * kGemvRowsPerTile + tid;
      if (tid < kGemvRowsPerTile && n < p.N) p.y[n] = 0;
      return;
    }
  }
  // wave index as a wave-uniform (scalar) value, so the per-wave k-step
  // bookkeeping below stays in SGPRs and its branches are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = p.waves;
  const int col = lane & 15;   // MFMA column: output row within the tile
  const int row4 = lane >> 4;  // 16-lane row of the wave
  const int tile = blockIdx.x + p.tile_base;
  const int split = blockIdx.y;
  const int n0 = tile * kGemvRowsPerTile;

  const int ks_begin = split * p.ksteps_per_split;
  const int ks_end = min(p.ksteps, ks_begin + p.ksteps_per_split);
  const int kpw = p.kpw;                      // a power of two
  const int my_first = ks_begin + wave * kpw;
  const int my_steps = max(0, min(kpw, ks_end - my_first));
  const int kw0 = my_first * kGemvKStep;      // first k of this wave's run
  const int gw0 = kw0 / GS;                   // first group of this wave's run
  const int ngw = kpw * (kGemvKStep / GS);    // groups per wave run (power of two)
  const int lg_ngw = p.lg_groups_per_wave;
  const int xsegs_row = kpw * (kGemvKStep / 8);  // 16-byte x segments per row of the run
  const int lg_xsegs = p.lg_xsegs_per_wave;
  const int xstride = xsegs_row * 8 + 8;      // padded LDS row of x, in halves

  // LDS: the cross-wave sums, then one region per wave (gemv_lds_bytes)
  float* red = reinterpret_cast<float*>(smem);  // [nwaves][256]
  unsigned char* wreg = smem + (size_t)nwaves * 256 * sizeof(float) + (size_t)wave * p.wave_lds_bytes;
  uint16_t* xs = reinterpret_cast<uint16_t*>(wreg);   // [M][xstride]
  uint16_t* sl = xs + p.M * xstride;                  // [16][ngw]
  uint32_t* zl = reinterpret_cast<uint32_t*>(sl + 16 * ngw);  // [2][ngw]
  // bf16: 16-k partial sums of x, then x summed over each group, per token
  float* xpart = reinterpret_cast<float*>(
      wreg + ((((size_t)p.M * xstride + 16 * ngw) * sizeof(uint16_t) + 2 * ngw * sizeof(uint32_t) + 15) & ~(size_t)15));
  float* xsum = xpart + p.M * kpw * 8;  // [ngw][16]

  // ---- 1. loads: x, scales and zero points of this wave's run, then weights ----
  // (each a wave-uniform base plus a 32-bit per-lane byte offset)
  const int gwg = nwaves * ngw;  // WGSZ: groups of the workgroup's K range, 8 per wave
  if constexpr (WGSZ) {
    // 16-byte pieces straight to LDS: scale piece c * 16 + r is groups
    // 8c..8c+7 of row n0 + r (one piece per wave and row), zero-point piece
    // c * 2 + b is groups 4c..4c+3 of row block n0 / 8 + b
    const int gw0_wg = ks_begin * (kGemvKStep / GS);
    const int np_s = 2 * gwg, np_z = gwg / 2;
    const int wz = min((np_s + 63) >> 6, nwaves - 1);  // the wave that loads the zero points
    // (written as assembly, so the compiler does not take these LDS writes
    // for possible aliases of the x staging and wait for every later load
    // before it; they are the wave's oldest loads, so its own waits for later
    // loads cover them, and the run's end waits for them explicitly)
    if (64 * wave < np_s) {
      const int pc = 64 * wave + lane;
      if (pc < np_s) {
        const uint32_t off = 2u * (__umul24(min(pc & 15, p.N - 1 - n0), p.sG) + (uint32_t)(gw0_wg + 8 * (pc >> 4)));
        lds_dma16(reinterpret_cast<const char*>(p.scales + (size_t)n0 * p.sG), off, wgsz + 1024 * wave);
      }
    }
    if (ASYM && wave == wz && lane < np_z) {
      const uint32_t off = 4u * (__umul24(min(lane & 1, (p.N >> 3) - 1 - (n0 >> 3)), p.sG) + (uint32_t)(gw0_wg + 4 * (lane >> 1)));
      lds_dma16(reinterpret_cast<const char*>(p.zp + (size_t)(n0 >> 3) * p.sG), off, wgsz + 32 * gwg);
    }
  }
  const int xsegs = p.M * xsegs_row;
  const int xk0 = min(kw0, p.K - 8);  // k of the x base; lanes read k = min(kw0 + 8 seg, K - 8)
  const char* xbase = reinterpret_cast<const char*>(p.x + xk0);
  // (the per-lane products below take 24-bit operands: a row index below 16
  // times a stride or K below 2^24, and a group index times 0 or 1)
  u32x4 xr[XPT];  // only the loads that carry x are filled, and only they are staged
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    if (64 * j < xsegs) {  // wave-uniform: only the loads that carry x
      const int e = min(lane + 64 * j, xsegs - 1);
      const int m = e >> lg_xsegs;
      const int k = min(kw0 + ((e & (xsegs_row - 1)) << 3), p.K - 8);
      const uint32_t off = 2u * (__umul24(m, p.K) + (uint32_t)(k - xk0));
      xr[j] = *reinterpret_cast<const u32x4*>(xbase + off);
    }
  }
  // scales of the run: when each row's groups of the run are whole 16-byte
  // pieces of the scale tensor, one 16-byte load per lane (lane = row *
  // pieces per row + piece); otherwise one 2-byte load per scale
  const bool svec = ngw >= 8 && p.gmul == 1 && (p.sG & 7) == 0 && (gw0 & 7) == 0 &&
                    gw0 + ngw <= p.G && (reinterpret_cast<uintptr_t>(p.scales) & 15) == 0;
  // (srv and sr are filled only on their own branch and read only on it:
  // giving them a value on the other branch would make that branch write a
  // register with a load in flight on this one, and the compiler then waits
  // for every earlier load -- x -- before the weights are issued)
  u32x4 srv;
  uint32_t sr[SPT];
  uint32_t zr = 0u;
  if constexpr (!WGSZ) {
  const char* sbase = reinterpret_cast<const char*>(p.scales + (size_t)n0 * p.sG);  // row n0
  const int last_dr = p.N - 1 - n0;  // rows past N read row N - 1
  if (svec) {
    const int lg_ppr = lg_ngw - 3;
    const int e = min(lane, (16 << lg_ppr) - 1);
    const int r = e >> lg_ppr;
    const uint32_t off = 2u * (__umul24(min(r, last_dr), p.sG) + (uint32_t)(gw0 + 8 * (e & ((1 << lg_ppr) - 1))));
    srv = *reinterpret_cast<const u32x4*>(sbase + off);
  } else {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int e = min(lane + 64 * j, 16 * ngw - 1);
      const int r = e >> lg_ngw;
      const int g = min(gw0 + (e & (ngw - 1)), p.G - 1);
      const uint32_t off = 2u * (__umul24(min(r, last_dr), p.sG) + __umul24(g, p.gmul));
      sr[j] = *reinterpret_cast<const uint16_t*>(sbase + off);
    }
  }
  if constexpr (ASYM) {
    const int e = min(lane, 2 * ngw - 1);
    const int rr = e >> lg_ngw;
    const int g = min(gw0 + (e & (ngw - 1)), p.G - 1);
    const char* zbase = reinterpret_cast<const char*>(p.zp + (size_t)(n0 >> 3) * p.sG);
    const uint32_t off = 4u * (__umul24(min(rr, (p.N >> 3) - 1 - (n0 >> 3)), p.sG) + __umul24(g, p.gmul));
    zr = *reinterpret_cast<const uint32_t*>(zbase + off);
  }
  }
  __builtin_amdgcn_sched_barrier(0);
  // weights: a wave-uniform base per k-step plus one per-lane offset, so each
  // load needs no vector address arithmetic.  A complete row tile is stored
  // tile-major: run ks of its 16 rows is one contiguous 1 KiB block and this
  // lane's 16 bytes are its piece `lane` (r = row4, row = col).  The rows of
  // a final incomplete tile are stored one after another, 64 bytes per run.
  const WeightWalk ww = weight_walk(p.wq, p.N, p.K, p.nchunks, n0, col, row4);
  const int last_ks = ks_end - 1;
  u32x4 wv[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int ks = min(my_first + i, last_ks);
    wv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ww.at(ks)));
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. stage them in this wave's LDS region (read back by the same wave) ----
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int e = lane + 64 * j;
    if (e < xsegs) {
      const int m = e >> lg_xsegs;
      *reinterpret_cast<u32x4*>(xs + m * xstride + ((e & (xsegs_row - 1)) << 3)) = xr[j];
    }
  }
  if constexpr (!WGSZ) {
    if (svec) {
      // lane = row * (ngw / 8) + piece holds scales row * ngw + 8 * piece ...
      if (lane < 2 * ngw) *reinterpret_cast<u32x4*>(sl + 8 * lane) = srv;
    } else {
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int e = lane + 64 * j;
        if (e < 16 * ngw) sl[e] = (uint16_t)sr[j];
      }
    }
    if constexpr (ASYM) {
      if (lane < 2 * ngw) zl[lane] = zr;
    }
  }
  if constexpr (DT == DT_BF16) {
    // sum of x over every group of the run, per token (zero past M): the
    // magic offset and the zero point then cost one multiply-add per group,
    // (128 + z) * xsum, instead of an MFMA with -(128 + z) per chunk
    const int lg_parts = lg_xsegs - 1;  // kpw * 8 partials of 16 k per token
    for (int it = lane; it < (p.M << lg_parts); it += 64) {
      const uint16_t* src = xs + (it >> lg_parts) * xstride + ((it & ((1 << lg_parts) - 1)) << 4);
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(src);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(src + 8);
      // named components, not v[e] in a loop: see add_f16x2 on bit casts of
      // vector elements
      float sum = sum_bf16x2(v0.x, 0.f);
      sum = sum_bf16x2(v0.y, sum);
      sum = sum_bf16x2(v0.z, sum);
      sum = sum_bf16x2(v0.w, sum);
      sum = sum_bf16x2(v1.x, sum);
      sum = sum_bf16x2(v1.y, sum);
      sum = sum_bf16x2(v1.z, sum);
      sum = sum_bf16x2(v1.w, sum);
      xpart[it] = sum;
    }
    constexpr int PPG = GS / 16;  // partials per group
    for (int it = lane; it < 16 * ngw; it += 64) {
      const int g = it >> 4, tok = it & 15;
      float v = 0.f;
      if (tok < p.M) {
#pragma unroll
        for (int q = 0; q < PPG; ++q) v += xpart[(tok << lg_parts) + g * PPG + q];
      }
      xsum[it] = v;
    }
  }

  // ---- 3. dot products, one k-step at a time as its weights arrive ----
  const uint32_t mask_v = vgpr_const(0x000F000Fu);
  const uint16_t* xrow = xs + min(col, p.M - 1) * xstride + row4 * 8;  // rows >= M: any valid row
  const uint16_t* srow_l = sl + col * ngw;
  const uint32_t* zrow_l = zl + (col >> 3) * ngw;
  const int zshift = 4 * (col & 7);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  // one k-step (four 32-k chunks); FULL: all four chunks lie inside K
  auto kstep = [&](const u32x4 wraw, const int i, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const int c0 = (my_first + i) * 4;
    // a complete 128-k run is stored transposed, so register t already holds
    // this lane's slice of chunk t; an incomplete last run is stored in
    // order and is transposed across the 16-lane rows here
    u32x4 wt = wraw;
    if constexpr (!FULL) transpose_rows4(wt);
    // fp16: two chains by chunk parity.  bf16: one chain collecting both
    // x . (128 + q) and, from a second MFMA, x . (-(128 + z)).
    f32x4 ch[2];
    uint32_t nmz = neg_magic_pair<DT>(8u);
    u32x4 bcv = {nmz, nmz, nmz, nmz};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = c0 + t;
      if (!FULL && c >= p.nchunks) break;
      const int gl = i * (4 / CPG) + t / CPG;  // group within this wave's run
      if constexpr (ASYM) {
        if (t % CPG == 0) {
          nmz = neg_magic_pair<DT>((zrow_l[gl] >> zshift) & 0xFu);
          if constexpr (DT == DT_BF16) bcv = u32x4{nmz, nmz, nmz, nmz};
        }
      }
      const u32x4 a = *reinterpret_cast<const u32x4*>(xrow + i * kGemvKStep + t * 32);
      const bool fresh = (t % CPG) == 0;
      if constexpr (DT == DT_F16) {
        const u32x4 bq = qz_word_f16(wt[t], mask_v, nmz);  // q - z, exact
        const int u = (t % CPG) & 1;
        ch[u] = mfma16x16x32<DT>(a, bq, (t % CPG) < 2 ? f32x4{0.f, 0.f, 0.f, 0.f} : ch[u]);
      } else {
        const u32x4 bq = magic_word<DT>(wt[t], mask_v);     // 128 + q, exact
        ch[0] = mfma16x16x32<DT>(a, bq, fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : ch[0]);
        ch[0] = mfma16x16x32<DT>(a, bcv, ch[0]);
      }
      if (t % CPG == CPG - 1) {
        const float s = act_to_f32<DT>(srow_l[gl]);
        acc += s * ch[0];
        if constexpr (DT == DT_F16 && CPG > 1) acc += s * ch[1];
      }
    }
  };

  // (a WGSZ launch has only such waves: the host checks that K is a whole
  // number of 8-step runs of 128 and that there is one K range)
  if (WGSZ || (my_steps == KPW && (my_first + KPW) * 4 <= p.nchunks)) {
    // Common case: the wave's whole run is complete 128-k runs.  Branch-free
    // and software pipelined by 32-k chunks: the x fragment of chunk q + XD
    // is read from LDS while chunk q is multiplied (a ring of XD + 1
    // fragments, few registers, so that many waves stay resident).  bf16
    // multiplies x by 128 + q only; the offset and the zero point are
    // removed per group with the x sums.
    constexpr int XD = ONE ? 2 : 1;  // measured best on the decode layers
    constexpr int NQ = 4 * KPW;  // chunks of the run
    u32x4 xa[XD + 1];
    auto load_x = [&](int q) {
      return *reinterpret_cast<const u32x4*>(xrow + (q >> 2) * kGemvKStep + (q & 3) * 32);
    };
    constexpr int NR = ONE ? 1 : 4;  // accumulator rows in use
#pragma unroll
    for (int q = 0; q < XD; ++q) xa[q] = load_x(q);
    f32x4 ch;
    constexpr int NG = WGSZ ? 4 * KPW / CPG : 1;
    float chg[NG];  // WGSZ: each group's sum x . (128 + q), scaled after the run
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = q >> 2, t = q & 3;
      // keep each step's work after the wait for its own weights: left
      // free, the scheduler hoists later steps' unpacking to the top, and
      // the first MFMA then waits for every load of the run
      if (t == 0) __builtin_amdgcn_sched_barrier(0);
      if (q + XD < NQ) xa[(q + XD) % (XD + 1)] = load_x(q + XD);
      const u32x4 a = xa[q % (XD + 1)];
      const int gl = i * (4 / CPG) + t / CPG;  // group within this wave's run
      const bool fresh = (t % CPG) == 0;
      const uint32_t z = (ASYM && !WGSZ) ? (zrow_l[gl] >> zshift) & 0xFu : 8u;
      if constexpr (DT == DT_F16) {
        const u32x4 bq = qz_word_f16(wv[i][t], mask_v, neg_magic_pair<DT>(z));  // q - z, exact
        ch = mfma16x16x32<DT>(a, bq, fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : ch);
      } else {
        const u32x4 bq = magic_word<DT>(wv[i][t], mask_v);  // 128 + q, exact
        ch = mfma16x16x32<DT>(a, bq, fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : ch);
      }
      if (t % CPG == CPG - 1) {
        if constexpr (WGSZ) {
          chg[gl] = ch[0];
        } else {
          const float sc = act_to_f32<DT>(srow_l[gl]);
          if constexpr (DT == DT_BF16) {
            // s * (x . (128 + q) - (128 + z) * xsum); -(128 + z) * s is exact
            const float szc = -(128.0f + (float)z) * sc;
            const float* xs = xsum + gl * 16 + 4 * row4;
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r] = __builtin_fmaf(sc, ch[r], __builtin_fmaf(szc, xs[r], acc[r]));
          } else {
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r] = __builtin_fmaf(sc, ch[r], acc[r]);
          }
        }
      }
    }
    if constexpr (WGSZ) {
      // the workgroup's scales and zero points have landed (every wave waits
      // for its own global->LDS loads, then the barrier); then the groups in
      // run order, the same operations in the same order as applying each
      // group at its end
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* ssh = reinterpret_cast<const uint16_t*>(wgsz) + (wave * 16 + col) * 8;
      const uint32_t* zsh = reinterpret_cast<const uint32_t*>(wgsz + 32 * gwg);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float sc = act_to_f32<DT>(ssh[g]);
        const int gw = wave * NG + g;  // group within the workgroup's range
        const uint32_t z = ASYM ? (zsh[((gw >> 2) * 2 + (col >> 3)) * 4 + (gw & 3)] >> zshift) & 0xFu : 8u;
        const float szc = -(128.0f + (float)z) * sc;
        acc[0] = __builtin_fmaf(sc, chg[g], __builtin_fmaf(szc, xsum[g * 16 + 4 * row4], acc[0]));
      }
    }
  } else {
    // unrolled at compile time, so that wv[] is never indexed dynamically
    // (which would put it in scratch memory)
    static_for<0, KPW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (i >= my_steps) return;
      __builtin_amdgcn_sched_barrier(0);  // this step's work after its own wait
      if ((my_first + i) * 4 + 4 <= p.nchunks)
        kstep(wv[i], i, std::true_type{});
      else
        kstep(wv[i], i, std::false_type{});
    });
  }

  // ---- 4. reduce the waves in order, then the K ranges ----
  if constexpr (ONE) {
    if (p.splits == 1) {
      // one token, one K range: the sums are register 0 of lanes 0..15
      red[wave * 256 + lane] = acc[0];
      __syncthreads();
      const int nn = n0 + tid;
      if (tid < kGemvRowsPerTile && nn < p.N) {
        float v = 0.f;
        for (int w = 0; w < nwaves; ++w) v += red[w * 256 + tid];
        if (p.bias) v += act_to_f32<DT>(p.bias[nn]);
        p.y[nn] = f32_to_act<DT>(v * p.yscale);
      }
      return;
    }
  }
  if (p.splits == 1 && p.M <= 4) {
    // up to four tokens, one K range: token m's sums are register m of lanes
    // 0..15 (the general path's order: waves in order, then bias, rounding)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * 256 + r * 64 + lane] = acc[r];
    __syncthreads();
    const int m = tid >> 4, nn = n0 + (tid & 15);
    if (tid < 16 * p.M && nn < p.N) {
      float v = 0.f;
      for (int w = 0; w < nwaves; ++w) v += red[w * 256 + m * 64 + (tid & 15)];
      if (p.bias) v += act_to_f32<DT>(p.bias[nn]);
      p.y[(size_t)m * p.N + nn] = f32_to_act<DT>(v * p.yscale);
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave * 256 + r * 64 + lane] = acc[r];
  __syncthreads();
  finish_tile<DT>(p, red, nwaves, 256, tile, split, &last_flag);
}

// ---------------------------------------------------------------------------
// M <= 8: a few tokens, one K range, every wave a run of KPW complete k-steps
// (the last wave's run may be shorter by whole parts of a run)
// ---------------------------------------------------------------------------
// The kernel above stages each wave's scales, zero points and bf16 x group
// sums through LDS and meets twice at workgroup barriers; for a few tokens
// that bookkeeping costs about as much time as the dequantisation.  This
// instance keeps only x in LDS:
// * A row i of the MFMA is token i mod MT (MT = 1, 2 or 4 token rows; three
//   tokens run with MT = 4), so every 16-lane row of a result holds the same
//   dot products: register r is token r.  Each 16-lane row R therefore
//   finishes only the groups it owns -- the R-th quarter of the wave's run.
//   With eight token rows (five to eight tokens, only M staged) rows R and
//   R + 2 hold tokens 4 (R mod 2) + r and finish half the groups each.  A
//   16-lane row fetches only its groups' scales and zero points: one small
//   load per tensor and wave, straight into registers (the scale / zero-point
//   carrier of "[ROCm] Converge the two W4A16 linear kernels onto the
//   upstream shell", "What this does": no per-group metadata loads), issued
//   after the weights, since only the end of the run needs them: the waits
//   for the weights, which complete in issue order, never wait for them.
// * Both dtypes multiply x by the exact magic value (128 or 1024) + q and
//   remove (magic + z) per group with the group's sum of x (the general
//   kernel's bf16 scheme; for fp16 it saves the packed subtraction, 4 of 11
//   VALU instructions per weight word).  The group sums of x come from the
//   matrix cores: an MFMA whose A rows are 16 chunks of one token's x and
//   whose B is all ones gives the 16 chunk sums, its rows ordered so that
//   16-lane row R receives the chunks of its own groups.
// * The 16-lane rows are added with permlane swaps; the waves through LDS
//   after one barrier, in wave order.

// waves per SIMD the register budget is sized for (more tokens and longer
// runs hold more group sums)
constexpr int one_waves_per_simd(int kpw, int gs, int mt) {
  return mt == 8 ? 4
                 : ((128 * kpw / gs) * mt > 16 || (kpw == 8 && gs == 64) ? 5 : (kpw == 8 || gs == 32 || mt > 1 ? 6 : 8));
}

// 16-lane row R of the result takes vR (each v uniform across the wave): two
// 16-lane swaps pair rows (0, 1) and (2, 3), one 32-lane swap joins the
// halves.  (A select on the row index would be turned by the compiler into a
// dynamic index of the source array, kept in scratch memory; a hand-written
// v_cndmask would read MFMA results without the wait states the compiler
// inserts for its own instructions.)
__device__ __forceinline__ float row_select(float v0, float v1, float v2, float v3) {
  const auto b = [](float f) { return __builtin_bit_cast(uint32_t, f); };
  const auto lo = __builtin_amdgcn_permlane16_swap(b(v0), b(v1), false, false);  // rows 0, 2: v0; 1, 3: v1
  const auto hi = __builtin_amdgcn_permlane16_swap(b(v2), b(v3), false, false);  // rows 0, 2: v2; 1, 3: v3
  const auto r = __builtin_amdgcn_permlane32_swap(lo[0], hi[0], false, false);   // rows 2, 3 from hi
  return __builtin_bit_cast(float, (uint32_t)r[0]);
}

// the sum of v over the four 16-lane rows, in lanes 0..15: rows (0 + 2) and
// (1 + 3), then their sum
__device__ __forceinline__ float rows_sum(float v) {
  const uint32_t a = __builtin_bit_cast(uint32_t, v);
  const auto hi = __builtin_amdgcn_permlane32_swap(a, a, false, false);  // [1]: lanes 32..63 in 0..31
  v += __builtin_bit_cast(float, (uint32_t)hi[1]);
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto odd = __builtin_amdgcn_permlane16_swap(b, b, false, false);  // [1]: lanes 16..31 in 0..15
  return v + __builtin_bit_cast(float, (uint32_t)odd[1]);
}

// 16-lane rows 0 and 1 keep a, rows 2 and 3 take b from rows 0 and 1 (one
// 32-lane swap)
__device__ __forceinline__ float half_select(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                  false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]);
}

// v of 16-lane rows 0 + 2 and 1 + 3, in lanes 0..31
__device__ __forceinline__ float halves_sum(float v) {
  const uint32_t a = __builtin_bit_cast(uint32_t, v);
  const auto hi = __builtin_amdgcn_permlane32_swap(a, a, false, false);  // [1]: lanes 32..63 in 0..31
  return v + __builtin_bit_cast(float, (uint32_t)hi[1]);
}

// a lane's NW consecutive 32-bit words, read as one load where possible
template <int NW>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    w[0] = *p;
  } else if constexpr (NW == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else {
    static_assert(NW % 4 == 0, "words");
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4 v = reinterpret_cast<const u32x4*>(p)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

// The few-token instance's arguments past the ten preloaded ones.
// Expert-indexed mode (single token): workgroup z is slot z, whose expert
// ids[z] selects slice e of the weight / scale / zp / bias stacks.  K split
// (splits > 1): workgroup y is K range y, of runs_per_split runs; partial
// sums go to partial[split][M][N] and the last workgroup of a tile to arrive
// (counters[tile], zero between calls) adds them in range order.
struct OneArgs {
  const int32_t* ids;
  const float* weights;  // router weight per slot, or NULL: 1
  int topk, experts, x_per_slot;
  size_t w_estride, s_estride, z_estride;  // words / halves / words per expert
  float* partial;
  uint32_t* counters;
  int splits, runs_per_split;
};

// PART: the last wave's run may be shorter (otherwise every run is whole and
// the masks and clamps below compile away).  MODE: ONE_PLAIN, ONE_MOE
// (expert-indexed, MT == 1) or ONE_SPLIT (K ranges; a plain launch computes
// its runs from the wave index alone, with no wait for an argument load
// before the weight addresses).
enum { ONE_PLAIN = 0, ONE_MOE = 1, ONE_SPLIT = 2 };
template <int DT, int GS, bool ASYM, int KPW, int MT, bool PART, int MODE>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(one_waves_per_simd(KPW, GS, MT)))) void gemv_one_kernel(
    const uint16_t* a_x, const uint32_t* a_wq, const uint16_t* a_scales, const uint32_t* a_zp, int N, int K,
    int sG, int M, const uint16_t* bias, uint16_t* y, const OneArgs moe) {
  constexpr bool MOE = MODE == ONE_MOE, SPLIT = MODE == ONE_SPLIT;
  constexpr int CPG = GS / 32;            // 32-k chunks per group
  constexpr int NC = 4 * KPW;             // chunks of a run
  constexpr int NGW = NC / CPG;           // groups of a run
  constexpr int QR = MT == 8 ? 2 : 4;     // parts of the run's groups: quarters, or halves
  constexpr int OWN = NGW / QR;           // groups each 16-lane row finishes
  constexpr int SLOTS = MT == 8 ? 4 : MT; // result registers in use: token slots per 16-lane row
  constexpr int KR = KPW * kGemvKStep;    // k of a run
  constexpr int XPL = KR / 8 / 64;        // 16-byte x segments per lane and token
  // staged token rows are KR halves apart plus 64 bytes, so that the token
  // rows one MFMA operand read touches start in different LDS banks (KR
  // halves alone is a multiple of the bank span: four token rows read the
  // same banks, a 4-way conflict on every operand read)
  constexpr int XR = KR + (MT > 1 ? 32 : 0);
  constexpr int SW = (OWN + 1) / 2;       // words holding the owned scales
  static_assert(OWN >= 1 && OWN <= 4 && XPL >= 1 && (MT == 1 || MT == 2 || MT == 4 || MT == 8), "instance");
  static_assert(!MOE || MT == 1, "one token per slot");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  float yscale = 1.f;
  if constexpr (MOE) {
    const int slot = blockIdx.z;
    const int e = moe.ids[slot];
    y += (size_t)slot * N;
    if (e < 0 || e >= moe.experts) {
      // not an expert: a zero row (the whole workgroup leaves here)
      const int nz = blockIdx.x * kGemvRowsPerTile + tid;
      if (tid < kGemvRowsPerTile && nz < N) y[nz] = 0;
      return;
    }
    a_wq += (size_t)e * moe.w_estride;
    a_scales += (size_t)e * moe.s_estride;
    if constexpr (ASYM) a_zp += (size_t)e * moe.z_estride;
    if (bias) bias += (size_t)e * N;
    a_x += (size_t)(moe.x_per_slot ? slot : slot / moe.topk) * K;
    if (moe.weights) yscale = moe.weights[slot];
  }
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  const int col = lane & 15;   // MFMA column: output row within the tile
  const int row4 = lane >> 4;  // 16-lane row
  // the part of the run's groups this 16-lane row finishes, and the token of
  // its result register r: with up to four token rows every 16-lane row holds
  // every token (register r is token r) and finishes a quarter; with eight,
  // rows R and R + 2 hold tokens 4 (R mod 2) + r and finish a half each
  const int part = MT == 8 ? row4 >> 1 : row4;
  const int n0 = blockIdx.x * kGemvRowsPerTile;
  const int n = min(n0 + col, N - 1);  // rows past N read row N - 1
  // The last run may stop short of KPW k-steps, after a whole number of parts
  // (the host checks), and with a K split the last range may hold fewer runs
  // than waves: a 16-lane row's groups then lie entirely inside K or entirely
  // past it.  Past K, every load is clamped to valid memory (a wave with no
  // run reads the last one) and the row's groups are dropped at the end.
  const int ksteps = K >> 7;
  const int run = SPLIT ? (int)blockIdx.y * moe.runs_per_split + wave : wave;  // this wave's run of KPW k-steps
  const int runc = PART ? min(run, (ksteps - 1) / KPW) : run;
  const int kw0 = runc * KR;           // first k of this wave's run
  const int g0 = kw0 / GS;             // first group of the run
  const bool own_valid = !PART || (run * KPW + part * (KPW / QR)) < ksteps;
  const int gown = g0 + (own_valid ? part * OWN : 0);  // first group this 16-lane row finishes
  // token rows staged in LDS: MT, or the M tokens of an eight-row instance
  const int rows = MT == 8 ? M : MT;
  // one LDS region per wave: its x ([rows][XR]), then its sums ([MT][16]);
  // only the final sum over the waves needs the number of waves, which is
  // read from the dispatch (no wait for it before the run's loads)
  const int region = rows * 2 * XR + 64 * MT;  // bytes
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem + (size_t)wave * region);
  auto red_of = [&](int w) { return reinterpret_cast<float*>(smem + (size_t)w * region + rows * 2 * XR); };

  // ---- 1. loads: x, then the weights, then scales and zero points ----
  // (the metadata is needed only after the run, so the waits for the weights
  // never wait for it; token rows past M read token M - 1)
  u32x4 xr[MT][XPL];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (MT == 8 && m >= M) break;  // wave-uniform
    const char* xb = reinterpret_cast<const char*>(a_x + (size_t)min(m, M - 1) * K + kw0);
#pragma unroll
    for (int j = 0; j < XPL; ++j)
      xr[m][j] = *reinterpret_cast<const u32x4*>(
          xb + 2u * (uint32_t)(PART ? min(8 * (lane + 64 * j), K - 8 - kw0) : 8 * (lane + 64 * j)));
  }
  __builtin_amdgcn_sched_barrier(0);
  const WeightWalk ww = weight_walk(a_wq, N, K, K >> 5, n0, col, row4);
  u32x4 wv[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i)
    wv[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(ww.at(PART ? min(runc * KPW + i, ksteps - 1) : run * KPW + i)));
  __builtin_amdgcn_sched_barrier(0);
  uint32_t sw[SW];
  if constexpr (OWN == 1) {
    sw[0] = a_scales[(size_t)n * sG + gown];
  } else {
    load_words<SW>(reinterpret_cast<const uint32_t*>(a_scales + (size_t)n * sG + gown), sw);
  }
  // the owned groups' zero-point words
  constexpr int ZW = ASYM ? OWN : 1;
  uint32_t zw[ZW];
  if constexpr (ASYM) {
    load_words<ZW>(a_zp + (size_t)(n >> 3) * sG + gown, zw);
  } else {
    zw[0] = 0u;
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. x to this wave's LDS region; group sums of x ----
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (MT == 8 && m >= M) break;  // wave-uniform
#pragma unroll
    for (int j = 0; j < XPL; ++j) *reinterpret_cast<u32x4*>(xs + m * XR + 8 * (lane + 64 * j)) = xr[m][j];
  }
  float xsum[SLOTS][OWN];
  {
    constexpr uint32_t ONE2 = DT == DT_BF16 ? 0x3F803F80u : 0x3C003C00u;  // 1.0 in both halves
    const u32x4 ones = {ONE2, ONE2, ONE2, ONE2};
    if constexpr (MT <= 4) {
      // MFMA b of token m: A row i is chunk (NC/4) (i / 4) + 4 b + i % 4 of
      // the token's run and B is all ones, so the result rows 4R .. 4R+3 of
      // 16-lane row R are the sums of the chunks of R's own groups
      const uint16_t* xa0 = xs + ((NC / 4) * (col >> 2) + (col & 3)) * 32 + 8 * row4;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int b = 0; b < NC / 16; ++b) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(xa0 + m * XR + 4 * 32 * b);
          const f32x4 d = mfma16x16x32<DT>(a, ones, f32x4{0.f, 0.f, 0.f, 0.f});
          if constexpr (CPG == 4) {
            xsum[m][b] = (d[0] + d[1]) + (d[2] + d[3]);
          } else if constexpr (CPG == 2) {
            xsum[m][2 * b] = d[0] + d[1];
            xsum[m][2 * b + 1] = d[2] + d[3];
          } else {
            xsum[m][4 * b] = d[0];
            xsum[m][4 * b + 1] = d[1];
            xsum[m][4 * b + 2] = d[2];
            xsum[m][4 * b + 3] = d[3];
          }
        }
      }
    } else {
      // owned group t: A row i is token 4 ((i / 4) mod 2) + i % 4 over chunk c
      // of the group in half i / 8, B all ones, chained over the group's
      // chunks: register r of 16-lane row R is the group's sum of x for the
      // row's token slot r
      const int tk = min(4 * ((col >> 2) & 1) + (col & 3), M - 1);
      const uint16_t* xa0 = xs + tk * XR + (col >> 3) * (NC / 2) * 32 + 8 * row4;
#pragma unroll
      for (int t = 0; t < OWN; ++t) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CPG; ++c)
          d = mfma16x16x32<DT>(*reinterpret_cast<const u32x4*>(xa0 + (t * CPG + c) * 32), ones, d);
#pragma unroll
        for (int r = 0; r < SLOTS; ++r) xsum[r][t] = d[r];
      }
    }
  }

  // ---- 3. dot products, one k-step at a time as its weights arrive ----
  // (the loop of the kernel above: x fragments from LDS two chunks ahead, one
  // MFMA chain per group, x multiplied by magic + q; A row i reads token
  // i mod MT)
  const uint32_t mask_v = vgpr_const(0x000F000Fu);
  const int arow = MT == 8 ? min(col & 7, M - 1) : (col & (MT - 1));
  const uint16_t* xrow = xs + arow * XR + 8 * row4;
  const int zshift = 4 * (n & 7);
  constexpr int XD = 2;
  u32x4 xa[XD + 1];
  auto load_x = [&](int q) { return *reinterpret_cast<const u32x4*>(xrow + q * 32); };
#pragma unroll
  for (int q = 0; q < XD; ++q) xa[q] = load_x(q);
  float chg[NGW][SLOTS];
  f32x4 ch;
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    const int i = q >> 2, t = q & 3;
    if (t == 0) __builtin_amdgcn_sched_barrier(0);  // each step's work after its own wait
    if (q + XD < NC) xa[(q + XD) % (XD + 1)] = load_x(q + XD);
    const u32x4 a = xa[q % (XD + 1)];
    const int gl = q / CPG;
    const bool fresh = (q % CPG) == 0;
    const u32x4 bq = magic_word<DT>(wv[i][t], mask_v);
    ch = mfma16x16x32<DT>(a, bq, fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : ch);
    if (q % CPG == CPG - 1) {
#pragma unroll
      for (int r = 0; r < SLOTS; ++r) chg[gl][r] = ch[r];
    }
  }

  // ---- 4. each 16-lane row scales its own groups; rows, then waves, added ----
  float acc[SLOTS];
#pragma unroll
  for (int r = 0; r < SLOTS; ++r) acc[r] = 0.f;
#pragma unroll
  for (int t = 0; t < OWN; ++t) {
    // the group of 16-lane row R is part * OWN + t of the run
    const uint32_t sbits = (sw[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
    const float s = act_to_f32<DT>((uint16_t)sbits);
    const uint32_t z = ASYM ? (zw[t] >> zshift) & 0xFu : 8u;
    const float szc = own_valid ? -(Magic<DT>::value + (float)z) * s : 0.f;  // exact
    const float sv = own_valid ? s : 0.f;
#pragma unroll
    for (int r = 0; r < SLOTS; ++r) {
      float v;
      if constexpr (MT == 8)
        v = half_select(chg[t][r], chg[OWN + t][r]);
      else
        v = row_select(chg[t][r], chg[OWN + t][r], chg[2 * OWN + t][r], chg[3 * OWN + t][r]);
      acc[r] = __builtin_fmaf(sv, v, __builtin_fmaf(szc, xsum[r][t], acc[r]));
    }
  }
#pragma unroll
  for (int r = 0; r < SLOTS; ++r) {
    if constexpr (MT == 8) {
      // rows 0 + 2 (tokens 0..3) and 1 + 3 (tokens 4..7), in lanes 0..31
      const float v = halves_sum(acc[r]);
      if (lane < 32) red_of(wave)[(4 * row4 + r) * 16 + col] = v;
    } else {
      const float v = rows_sum(acc[r]);
      if (lane < 16) red_of(wave)[r * 16 + lane] = v;
    }
  }
  __syncthreads();
  // 16 M outputs (a workgroup of one wave covers eight tokens in two passes)
  for (int e = tid; e < 16 * M; e += blockDim.x) {
    const int m = e >> 4;
    const int nn = n0 + (e & 15);
    if (nn < N) {
      float v = 0.f;
      for (int w = 0; w < nwaves; ++w) v += red_of(w)[m * 16 + (e & 15)];
      if constexpr (!SPLIT) {
        if (bias) v += act_to_f32<DT>(bias[nn]);
        y[(size_t)m * N + nn] = f32_to_act<DT>(MOE ? v * yscale : v);
      } else {
        store_coherent(moe.partial + ((size_t)blockIdx.y * M + m) * N + nn, v);
      }
    }
  }
  if constexpr (!SPLIT) return;
  const int splits = moe.splits;
  // K split: every thread's partial sums have completed (stores count in
  // vmcnt; the barrier does not wait for them), then one arrival; the last
  // workgroup of the tile adds the K ranges in order
  __shared__ uint32_t last_range;
  wait_vm_all();
  __syncthreads();
  if (tid == 0) last_range = arrive(moe.counters + blockIdx.x) == (uint32_t)(splits - 1);
  __syncthreads();
  if (!last_range) return;
  for (int e = tid; e < 16 * M; e += blockDim.x) {
    const int m = e >> 4;
    const int nn = n0 + (e & 15);
    if (nn < N) {
      float v = 0.f;
      for (int sp = 0; sp < splits; ++sp) v += load_coherent(moe.partial + ((size_t)sp * M + m) * N + nn);
      if (bias) v += act_to_f32<DT>(bias[nn]);
      y[(size_t)m * N + nn] = f32_to_act<DT>(v);
    }
  }
  if (tid == 0) reset_counter(moe.counters + blockIdx.x);  // ready for the next call
}

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------

// one wave's staging region of the M <= 16 kernel: x rows of its run (padded
// by 16 bytes), the scales of its 16 rows and groups, the zero-point words
size_t gemv_lds_bytes(int waves, int64_t M, int kpw, int group) {
  const size_t red = (size_t)waves * 256 * sizeof(float);
  return red + (size_t)waves * (size_t)gemv_wave_lds_bytes((int)M, kpw, group);
}

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int group, int dtype, int cu_count) {
  GemvPlan p;
  p.tiles = (int)((N + kGemvRowsPerTile - 1) / kGemvRowsPerTile);
  p.ksteps = (int)((K + kGemvKStep - 1) / kGemvKStep);
  // k-steps per wave: a power of two, at most kGemvStepsPerWave; with x
  // staged, also small enough that a lane stages at most kGemvXSegsPerThread
  // x segments (M * 16 * kpw segments per wave, 64 lanes): kpw <= 4 * XPT / M.
  // The scale and zero-point staging then needs at most 32 * kpw / group and
  // 4 * kpw / group loads per lane, which the kernel's fixed counts cover.
  // measured on the decode layers: 8 k-steps per wave for one bf16 token, 4
  // for up to 8 tokens, 1 above (deeper waves are slower there); one fp16
  // token and two to four tokens keep 8 only where 4 would need more than
  // kGemvMaxWaves waves and so a K split (M = 2 with 4: 6-13 % faster on K =
  // 2560-4096 layers, 28 % slower on K = 9728, where it splits; one fp16
  // token with 4: 8-9 % faster on K = 2560 and 4096, whose dequantisation
  // costs more VALU work per weight than bf16's and gains from more waves)
  int kpw = kGemvStepsPerWave;
  const bool deep = (M == 1 && dtype == DT_BF16) || (M <= 4 && p.ksteps > 4 * kGemvMaxWaves);
  while (kpw > 1 && (M * kpw > 4 * kGemvXSegsPerThread || (kpw > 4 && !deep) || M > 8)) kpw >>= 1;
  // tuning overrides: k-steps per wave (a smaller power of two) and a
  // minimum number of K splits
  const Tuning& tu = tuning();
  if (tu.gemv_kpw >= 1 && tu.gemv_kpw <= kpw && (tu.gemv_kpw & (tu.gemv_kpw - 1)) == 0) kpw = tu.gemv_kpw;
  p.kpw = kpw;
  // A K split costs a partial-sum hand-off (2-4 us of coherent memory round
  // trips), more than it saves by filling idle CUs: measured at M = 1 on
  // 16-160-tile layers (K = 2560-14336), no split is 10-70 % faster.  So K is
  // split only (below) when a workgroup's waves or LDS demand it (at most
  // kGemvMaxWaves waves, LDS within the budget).
  int splits = 1;
  if (tu.gemv_splits >= 1) splits = tu.gemv_splits;  // raised below if it must be
  const size_t budget = p.tiles <= cu_count ? kGemvLdsBudget : kGemvLdsBudgetShared;
  for (;;) {
    if (splits > p.ksteps) splits = p.ksteps;
    const int kps = (p.ksteps + splits - 1) / splits;
    const int waves = (kps + kpw - 1) / kpw;
    if (splits == p.ksteps ||
        (waves <= kGemvMaxWaves && gemv_lds_bytes(waves, M, kpw, group) <= budget))
      break;
    ++splits;
  }
  p.ksteps_per_split = (p.ksteps + splits - 1) / splits;
  p.splits = (p.ksteps + p.ksteps_per_split - 1) / p.ksteps_per_split;
  p.waves = (p.ksteps_per_split + kpw - 1) / kpw;
  p.lds_bytes = gemv_lds_bytes(p.waves, M, kpw, group);
  // up to eight tokens: the few-token instance, when K is a whole number of
  // 128-k steps in runs of 8 (else 4) for at most kGemvMaxWaves waves, the
  // last run a whole number of parts (quarter runs, half runs for eight
  // token rows), a 16-lane row finishes at most 4 groups, the group sums per
  // result register and run are at most 32, and the staged x fits the LDS
  // budget (one K range, no tail chunks)
  // (runs of 8 first; four and eight token rows measured faster with runs of
  // 4 where those fit: -1 to -9 % on the decode layers; whole runs before a
  // shorter last run)
  // Eight token rows (five to eight tokens): where the general kernel would
  // split K they remove the hand-off (14336 x 4096 at M = 5: 13.5 -> 9.0 us;
  // K = 9728 at M = 5 / 6: -16 / -23 %); elsewhere, with the staged token
  // rows in different LDS banks, they are as fast or faster too (Llama decode
  // step at M = 5: -12 %, 4096 x 28672 17.6 -> 14.2 us; Qwen3-4B at
  // M = 5 / 6 / 8: -7 / -5 / -7 %).
  const int mt = gemv_one_rows(M);
  if (mt && K % kGemvKStep == 0 && !tu.gemv_no_one && tu.gemv_splits <= 1) {
    const int a = mt >= 4 ? 4 : 8, b = mt >= 4 ? 8 : 4;
    const int slots = mt == 8 ? 4 : mt, parts = mt == 8 ? 2 : 4;  // result registers, group parts
    const int order[4][2] = {{a, 0}, {b, 0}, {a, 1}, {b, 1}};  // (k-steps per wave, shorter last run)
    // one K range first; then, where the general kernel splits K too (so no
    // workspace is needed that it would not need), K ranges of at most
    // kGemvMaxWaves runs each, the partial sums handed over through the
    // workspace (tiles within the counter region). Split, one and two token
    // rows pay where they need no more K ranges than the general kernel
    // (28672 x 4096: M = 1 / 2 at g128 -21 / -10 %; at g32, 4 ranges against
    // its 2, +9 / +2 %); four and eight token rows where the grid is at most
    // two rounds of one workgroup per CU, with the whole LDS of the CU (four
    // rows try runs of 8 first: 28672 x 4096 at M = 3 / 4: -8 / -10 %;
    // 14336 x 4096 g64 at M = 4: -15 %; 20480 x 1280 g64: -14 / -16 %;
    // 65536 x 1024 at M = 4: -39 %; eight rows on 14336 x 4096 at M = 6-8:
    // -12 %; in more rounds the general kernel's smaller workgroups win:
    // 28672 x 8192 and 20480 x 5120 at M = 3, +6 / +15 %).  Where workgroups
    // share CUs, each may use half the LDS (two per CU; eight tokens on
    // 4096 x 6144 / 28672: -31 / -36 %).
    const int order_split4[4][2] = {{8, 0}, {4, 0}, {8, 1}, {4, 1}};
    for (int pass = 0; pass < (p.splits > 1 ? 2 : 1) && !p.one_kpw; ++pass) {
      for (const auto& o : (pass == 1 && mt == 4 ? order_split4 : order)) {
        const int k = o[0];
        if (tu.gemv_kpw >= 1 && k != tu.gemv_kpw) continue;
        const int ngw = kGemvKStep * k / group;
        const int runs = (p.ksteps + k - 1) / k;
        const int rest = p.ksteps % k;
        const int splits = pass == 0 ? 1 : (runs + kGemvMaxWaves - 1) / kGemvMaxWaves;
        const int waves = (runs + splits - 1) / splits;
        if (ngw > 16 || ngw / parts > 4 || ngw * slots > 32 || (rest != 0) != (o[1] != 0) || rest % (k / parts) ||
            waves > kGemvMaxWaves || (pass == 1 && (splits < 2 || p.tiles > kMaxCounters ||
                           (mt <= 2 ? splits > p.splits : (int64_t)p.tiles * splits > 2 * cu_count))))
          continue;
        const size_t lds = gemv_one_lds_bytes(waves, k, mt, M);
        const bool whole_cu = (int64_t)p.tiles * splits <= cu_count || (pass == 1 && (mt == 8 || (mt == 4 && k == 8)));
        const size_t one_budget = whole_cu ? kGemvLdsBudget : kGemvLdsBudget / 2;
        if (lds > one_budget) continue;
        p.one_kpw = k;
        p.one_mt = mt;
        p.one_waves = waves;
        p.one_splits = splits;
        p.one_lds_bytes = lds;
        break;
      }
    }
  }
  return p;
}

// enough for whichever kernel runs (the few-token instance falls back to the
// general kernel for unaligned scales or zero points)
size_t gemv_workspace_bytes(const GemvPlan& p, int64_t M, int64_t N) {
  const int splits = p.splits > p.one_splits ? p.splits : p.one_splits;
  if (splits <= 1) return 0;
  return kCounterBytes + (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
}

// x loads per lane an instance stages: the plan gives M <= 2 at 8 k-steps per
// wave (1 for the single-token instance) and M <= 16 at one k-step, so these
// cover the M * 16 * kpw segments of a wave's run with no spare registers
constexpr int small_xpt(int kpw, bool one) {
  return one ? 2 : (kpw == 8 || kpw == 1 ? 4 : kGemvXSegsPerThread);
}

// the small kernel is instantiated per k-steps per wave, so that its
// branch-free path covers every wave whose run is complete
template <int DT, int GS, bool ASYM, bool MOE>
static hipError_t launch_small(const GemvParams& prm, const GemvPlan& plan, dim3 grid, dim3 block,
                               hipStream_t s) {
  const bool one = plan.kpw == 8 && prm.M == 1;
  // three or four tokens at 8 k-steps (K too long for 4 without a split)
  // stage up to 8 x segments per lane
  const bool x8 = !MOE && plan.kpw == 8 && prm.M > 2;
  const int xpt = one ? small_xpt(8, true) : (x8 ? 8 : small_xpt(plan.kpw, false));
  if ((int64_t)prm.M * 16 * plan.kpw > 64 * xpt) return hipErrorInvalidConfiguration;
  // the workgroup-shared scale / zero-point instance: every wave a full run
  // of 8 k-steps in one K range, and 16-byte pieces of scales and zero points
  const auto aligned16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool wgsz = DT == DT_BF16 && GS == 128 && one && plan.splits == 1 && prm.gmul == 1 &&
                    plan.ksteps == 8 * plan.waves && plan.waves <= kGemvMaxWaves &&
                    (prm.sG & 7) == 0 && aligned16(prm.scales) && (!prm.zp || aligned16(prm.zp)) &&
                    (!MOE || ((prm.s_estride & 7) == 0 && (prm.z_estride & 3) == 0)) &&
                    !tuning().gemv_no_wgsz;
  switch (plan.kpw) {
    case 8:
      if (one) {
        if constexpr (DT == DT_BF16 && GS == 128) {
          if (wgsz) {
            hipLaunchKernelGGL((gemv_small_kernel<DT, GS, ASYM, 8, small_xpt(8, true), true, MOE, true>), grid, block, plan.lds_bytes, s, prm.x, prm.wq, prm.scales, prm.zp, prm.M, prm.N, prm.K, prm.sG, prm.gmul, prm.ksteps_per_split, prm);
            break;
          }
        }
        hipLaunchKernelGGL((gemv_small_kernel<DT, GS, ASYM, 8, small_xpt(8, true), true, MOE, false>), grid, block, plan.lds_bytes, s, prm.x, prm.wq, prm.scales, prm.zp, prm.M, prm.N, prm.K, prm.sG, prm.gmul, prm.ksteps_per_split, prm);
      } else if (x8) {
        if constexpr (!MOE)
          hipLaunchKernelGGL((gemv_small_kernel<DT, GS, ASYM, 8, 8, false, MOE, false>), grid, block, plan.lds_bytes, s, prm.x, prm.wq, prm.scales, prm.zp, prm.M, prm.N, prm.K, prm.sG, prm.gmul, prm.ksteps_per_split, prm);
      } else {
        hipLaunchKernelGGL((gemv_small_kernel<DT, GS, ASYM, 8, small_xpt(8, false), false, MOE, false>), grid, block, plan.lds_bytes, s, prm.x, prm.wq, prm.scales, prm.zp, prm.M, prm.N, prm.K, prm.sG, prm.gmul, prm.ksteps_per_split, prm);
      }
      break;
    case 4: hipLaunchKernelGGL((gemv_small_kernel<DT, GS, ASYM, 4, small_xpt(4, false), false, MOE, false>), grid, block, plan.lds_bytes, s, prm.x, prm.wq, prm.scales, prm.zp, prm.M, prm.N, prm.K, prm.sG, prm.gmul, prm.ksteps_per_split, prm); break;
    case 2: hipLaunchKernelGGL((gemv_small_kernel<DT, GS, ASYM, 2, small_xpt(2, false), false, MOE, false>), grid, block, plan.lds_bytes, s, prm.x, prm.wq, prm.scales, prm.zp, prm.M, prm.N, prm.K, prm.sG, prm.gmul, prm.ksteps_per_split, prm); break;
    case 1: hipLaunchKernelGGL((gemv_small_kernel<DT, GS, ASYM, 1, small_xpt(1, false), false, MOE, false>), grid, block, plan.lds_bytes, s, prm.x, prm.wq, prm.scales, prm.zp, prm.M, prm.N, prm.K, prm.sG, prm.gmul, prm.ksteps_per_split, prm); break;
    default: return hipErrorInvalidConfiguration;
  }
  return hipGetLastError();
}

template <int DT, int GS, bool ASYM>
static hipError_t launch_t(const GemvParams& prm, const GemvPlan& plan, int launch_tiles, hipStream_t s) {
  dim3 grid(launch_tiles, plan.splits, prm.slots);
  dim3 block(plan.waves * 64);
  return prm.moe_ids ? launch_small<DT, GS, ASYM, true>(prm, plan, grid, block, s)
                     : launch_small<DT, GS, ASYM, false>(prm, plan, grid, block, s);
}

template <int DT, int GS>
static hipError_t launch_z(const GemvParams& prm, const GemvPlan& plan, int lt, hipStream_t s) {
  return prm.zp ? launch_t<DT, GS, true>(prm, plan, lt, s) : launch_t<DT, GS, false>(prm, plan, lt, s);
}

template <int DT>
static hipError_t launch_g(const GemvParams& prm, int group, const GemvPlan& plan, int lt, hipStream_t s) {
  switch (group) {
    case 32: return launch_z<DT, 32>(prm, plan, lt, s);
    case 64: return launch_z<DT, 64>(prm, plan, lt, s);
    case 128: return launch_z<DT, 128>(prm, plan, lt, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int GS, bool ASYM, int KPW, int MT>
static hipError_t launch_one_k(const LinearArgs& a, const GemvPlan& plan, hipStream_t s, const MoeArgs* moe,
                               void* workspace) {
  // instances: at most 16 groups a run, at most 4 finished by a 16-lane row,
  // at most 32 group sums per result register
  constexpr int NGW = kGemvKStep * KPW / GS;
  constexpr int SLOTS = MT == 8 ? 4 : MT, PARTS = MT == 8 ? 2 : 4;
  if constexpr (NGW > 16 || NGW / PARTS > 4 || NGW * SLOTS > 32) {
    return hipErrorInvalidConfiguration;
  } else {
    // a run shorter than KPW k-steps, or a K range with fewer runs than waves
    const int runs = (int)((a.K / kGemvKStep + KPW - 1) / KPW);
    const bool part = (int64_t)runs * KPW * kGemvKStep != a.K || plan.one_splits * plan.one_waves != runs;
    OneArgs om{};
    om.splits = plan.one_splits;
    om.runs_per_split = plan.one_waves;
    if (plan.one_splits > 1) {
      om.counters = static_cast<uint32_t*>(workspace);
      om.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    }
    auto kern = plan.one_splits > 1
                    ? (part ? gemv_one_kernel<DT, GS, ASYM, KPW, MT, true, ONE_SPLIT>
                            : gemv_one_kernel<DT, GS, ASYM, KPW, MT, false, ONE_SPLIT>)
                    : (part ? gemv_one_kernel<DT, GS, ASYM, KPW, MT, true, ONE_PLAIN>
                            : gemv_one_kernel<DT, GS, ASYM, KPW, MT, false, ONE_PLAIN>);
    if (moe) {
      if constexpr (MT == 1) {
        om.ids = moe->ids;
        om.weights = moe->weights;
        om.topk = (int)moe->topk;
        om.experts = (int)moe->experts;
        om.x_per_slot = moe->x_per_slot ? 1 : 0;
        om.w_estride = (size_t)a.N * (size_t)(a.K / 8);
        om.s_estride = (size_t)a.N * (size_t)a.sG;
        om.z_estride = (size_t)(a.N / 8) * (size_t)a.sG;
        kern = part ? gemv_one_kernel<DT, GS, ASYM, KPW, MT, true, ONE_MOE>
                    : gemv_one_kernel<DT, GS, ASYM, KPW, MT, false, ONE_MOE>;
      } else {
        return hipErrorInvalidConfiguration;
      }
    }
    const dim3 grid(plan.tiles, plan.one_splits, moe ? (unsigned)moe->slots : 1u), block(64 * plan.one_waves);
    hipLaunchKernelGGL(kern, grid, block, plan.one_lds_bytes, s,
                       static_cast<const uint16_t*>(a.x), reinterpret_cast<const uint32_t*>(a.wq),
                       static_cast<const uint16_t*>(a.scales), reinterpret_cast<const uint32_t*>(a.zp), (int)a.N,
                       (int)a.K, a.sG, (int)a.M, static_cast<const uint16_t*>(a.bias), static_cast<uint16_t*>(a.y),
                       om);
    return hipGetLastError();
  }
}

template <int DT, int GS, bool ASYM>
static hipError_t launch_one(const LinearArgs& a, const GemvPlan& plan, hipStream_t s, const MoeArgs* moe,
                             void* ws) {
  const int key = plan.one_kpw * 10 + plan.one_mt;
  switch (key) {
    case 81: return launch_one_k<DT, GS, ASYM, 8, 1>(a, plan, s, moe, ws);
    case 82: return launch_one_k<DT, GS, ASYM, 8, 2>(a, plan, s, moe, ws);
    case 84: return launch_one_k<DT, GS, ASYM, 8, 4>(a, plan, s, moe, ws);
    case 41: return launch_one_k<DT, GS, ASYM, 4, 1>(a, plan, s, moe, ws);
    case 42: return launch_one_k<DT, GS, ASYM, 4, 2>(a, plan, s, moe, ws);
    case 44: return launch_one_k<DT, GS, ASYM, 4, 4>(a, plan, s, moe, ws);
    case 88: return launch_one_k<DT, GS, ASYM, 8, 8>(a, plan, s, moe, ws);
    case 48: return launch_one_k<DT, GS, ASYM, 4, 8>(a, plan, s, moe, ws);
    default: return hipErrorInvalidConfiguration;
  }
}

template <int DT>
static hipError_t launch_one_g(const LinearArgs& a, const GemvPlan& plan, hipStream_t s, const MoeArgs* moe,
                               void* ws) {
  const bool asym = a.zp != nullptr;
  switch (a.group) {
    case 32: return asym ? launch_one<DT, 32, true>(a, plan, s, moe, ws) : launch_one<DT, 32, false>(a, plan, s, moe, ws);
    case 64: return asym ? launch_one<DT, 64, true>(a, plan, s, moe, ws) : launch_one<DT, 64, false>(a, plan, s, moe, ws);
    case 128:
      return asym ? launch_one<DT, 128, true>(a, plan, s, moe, ws) : launch_one<DT, 128, false>(a, plan, s, moe, ws);
    default: return hipErrorInvalidValue;
  }
}

bool gemv_one_runs(const LinearArgs& a, const GemvPlan& plan, const MoeArgs* moe) {
  const auto aligned16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  // expert-indexed: one token per slot, and every expert's scale and zero-point
  // slices 16-byte aligned like the first
  if (moe && (a.M != 1 || ((size_t)a.N * (size_t)a.sG) % 8 || ((size_t)(a.N / 8) * (size_t)a.sG) % 4 ||
              moe->slots < 1 || moe->slots > kMaxGridZ || plan.one_splits != 1))
    return false;
  // the K ranges cover K, the last one not empty; split tiles within the
  // counter region
  const int64_t range = (int64_t)plan.one_waves * plan.one_kpw * kGemvKStep;
  return plan.one_kpw != 0 && gemv_one_rows(a.M) == plan.one_mt && a.gmul == 1 && aligned16(a.scales) &&
         (!a.zp || aligned16(a.zp)) && plan.one_waves >= 1 && plan.one_waves <= kGemvMaxWaves &&
         plan.one_splits >= 1 && (plan.one_splits == 1 || plan.tiles <= kMaxCounters) &&
         (int64_t)(plan.one_splits - 1) * range < a.K && (int64_t)plan.one_splits * range >= a.K &&
         a.K % kGemvKStep == 0;
}

hipError_t launch_gemv(const LinearArgs& a, const GemvPlan& plan, void* workspace,
                       hipStream_t stream, const MoeArgs* moe) {
  if (gemv_one_runs(a, plan, moe)) {
    if (plan.one_splits > 1 && !workspace) return hipErrorInvalidValue;
    return a.dtype == DT_F16 ? launch_one_g<DT_F16>(a, plan, stream, moe, workspace)
                             : launch_one_g<DT_BF16>(a, plan, stream, moe, workspace);
  }
  if (plan.waves < 1 || plan.waves > kGemvMaxWaves || plan.lds_bytes > kGemvLdsBudget ||
      plan.kpw < 1 || plan.kpw > kGemvStepsPerWave)
    return hipErrorInvalidConfiguration;
  // expert-indexed: one M = 1 product per slot, one K range
  if (a.M < 1 || a.M > kGemvMaxM) return hipErrorInvalidConfiguration;
  if (moe && (a.M != 1 || plan.splits != 1 || moe->slots < 1 ||
              moe->slots > kMaxGridZ))
    return hipErrorInvalidConfiguration;
  GemvParams prm;
  prm.yscale = 1.0f;
  prm.moe_ids = nullptr;
  prm.moe_weights = nullptr;
  prm.topk = prm.experts = prm.x_per_slot = 0;
  prm.w_estride = prm.s_estride = prm.z_estride = 0;
  prm.slots = 1;
  if (moe) {
    prm.moe_ids = moe->ids;
    prm.moe_weights = moe->weights;
    prm.topk = (int)moe->topk;
    prm.experts = (int)moe->experts;
    prm.x_per_slot = moe->x_per_slot ? 1 : 0;
    prm.w_estride = (size_t)a.N * (size_t)(a.K / 8);
    prm.s_estride = (size_t)a.N * (size_t)a.sG;
    prm.z_estride = (size_t)(a.N / 8) * (size_t)a.sG;
    prm.slots = (int)moe->slots;
  }
  prm.x = static_cast<const uint16_t*>(a.x);
  prm.wq = reinterpret_cast<const uint32_t*>(a.wq);
  prm.scales = static_cast<const uint16_t*>(a.scales);
  prm.zp = reinterpret_cast<const uint32_t*>(a.zp);
  prm.bias = static_cast<const uint16_t*>(a.bias);
  prm.y = static_cast<uint16_t*>(a.y);
  prm.counters = nullptr;
  prm.partial = nullptr;
  prm.tile_base = 0;
  if (plan.splits > 1) {
    prm.counters = static_cast<uint32_t*>(workspace);
    prm.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
  }
  prm.M = (int)a.M;
  prm.N = (int)a.N;
  prm.K = (int)a.K;
  prm.G = (int)(a.K / a.group);
  prm.sG = a.sG;
  prm.gmul = a.gmul;
  prm.nchunks = (int)(a.K / 32);
  prm.ksteps = plan.ksteps;
  prm.ksteps_per_split = plan.ksteps_per_split;
  prm.splits = plan.splits;
  prm.kpw = plan.kpw;
  prm.waves = plan.waves;
  {
    int lg = 0;
    while ((1 << lg) < plan.kpw * (kGemvKStep / 8)) ++lg;
    prm.lg_xsegs_per_wave = lg;
    lg = 0;
    while ((1 << lg) < plan.kpw * kGemvKStep / a.group) ++lg;
    prm.lg_groups_per_wave = lg;
    prm.wave_lds_bytes = gemv_wave_lds_bytes((int)a.M, plan.kpw, a.group);
  }
  // With a K split every row tile of a launch needs its own completion
  // counter, and the counter region holds kMaxCounters: a layer with more row
  // tiles is launched in chunks of row tiles, one after another on the stream
  // (each chunk's last workgroups leave its counters zero for the next).
  const int chunk = plan.splits > 1 ? (int)kMaxCounters : plan.tiles;
  for (int t0 = 0; t0 < plan.tiles; t0 += chunk) {
    prm.tile_base = t0;
    const int lt = min(chunk, plan.tiles - t0);
    const hipError_t e = a.dtype == DT_F16 ? launch_g<DT_F16>(prm, a.group, plan, lt, stream)
                                           : launch_g<DT_BF16>(prm, a.group, plan, lt, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace w4a16
