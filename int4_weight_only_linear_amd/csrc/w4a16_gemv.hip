// Skinny split-K W4A16 decode kernel for gfx950 (M <= 64).
//
// The pages' decode path ("[ROCm][Kernel] Add HybridW4A16LinearKernel: Triton
// prefill + HIP skinny decode", description) is a split-K skinny GEMM for
// small M that dequantises with the exponent-OR trick.  This kernel keeps the
// split-K idea and the trick, and re-plans the rest for CDNA4:
//
// * Work unit: 16 output rows (the MFMA column tile) x one 128-wide k-step.
//   Each lane of a wave issues one 16-byte non-temporal load per k-step: lane
//   (j = lane % 16, r = lane / 16) reads chunk r (32 k) of row n0 + j.  A
//   4x4 dword transpose across the four 16-lane rows (permlane swaps) then
//   leaves, in register t, word r of chunk t -- exactly the B operand layout
//   of v_mfma_f32_16x16x32 for chunk t.
// * The scale is factored out of the dot product: per group the wave forms
//   sum_k x[m,k] * (q[n,k] - z[n,g]) in fp32 and then adds s[n,g] times that
//   sum into the accumulator.  For fp16, B = (1024 + q) - (1024 + z) is exact
//   with one packed add per weight pair; bf16 has no packed add on gfx950, so
//   it multiplies B = 128 + q (the AND-OR alone, exact) and removes the
//   offset with a second MFMA against the constant B = -(128 + z).  Nothing
//   is rounded to the activation dtype before the output, and no per-weight
//   multiply by the scale is needed.
// * x rows (M <= 16 per MFMA row tile, zero-padded) are read straight from
//   global memory (L2-resident), so there is no LDS staging and no limit on
//   K * M (the pages' converged kernel streams the overflow from global for
//   the same reason, "[ROCm] Converge the two W4A16 linear kernels onto the
//   upstream shell", "What this does").
// * The waves of a workgroup take the k-steps of its K range in turn and are
//   reduced through LDS in wave order; with several K ranges per row tile the
//   partial sums go through the workspace and the last workgroup to arrive
//   adds them in range order.  Results do not depend on scheduling.
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
  uint32_t* counters;  // [tiles] when splits > 1; zero between calls
  int M, N, K, G;
  int nchunks;  // K / 32
  int ksteps;   // ceil(nchunks / 4)
  int ksteps_per_split;
  int splits;
};

template <int DT, int MT, int GS, bool ASYM>
__global__ __launch_bounds__(1024) void gemv_kernel(const GemvParams p) {
  constexpr int CPG = GS / 32;  // 32-k chunks per quantisation group (1, 2 or 4)
  constexpr int NEL = MT * 256;  // accumulator elements per wave
  __shared__ float red[kGemvMaxWaves * NEL];
  __shared__ int last_flag;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int col = lane & 15;  // MFMA column = output row within the tile
  const int row4 = lane >> 4;  // 16-lane row of the wave
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int n = tile * kGemvRowsPerTile + col;
  const bool nvalid = n < p.N;
  const uint32_t* wrow = p.wq + (size_t)(nvalid ? n : 0) * (p.K >> 3);
  const uint16_t* srow = p.scales + (size_t)(nvalid ? n : 0) * p.G;

  const int ks_begin = split * p.ksteps_per_split;
  const int ks_end = min(p.ksteps, ks_begin + p.ksteps_per_split);

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ks = ks_begin + wave; ks < ks_end; ks += nwaves) {
    const int c0 = ks * 4;
    u32x4 wv = {0u, 0u, 0u, 0u};
    if (nvalid && c0 + row4 < p.nchunks)
      wv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow + (size_t)(c0 + row4) * 4));
    transpose_rows4(wv);

    f32x4 tmp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) tmp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint32_t bc = neg_magic_pair<DT>(8u);

#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = c0 + t;
      if (c >= p.nchunks) break;
      const int grp = c / CPG;
      if (ASYM && (t % CPG == 0)) {
        const uint32_t z = nvalid ? zero_point(p.zp, n, p.G, grp) : 8u;
        bc = neg_magic_pair<DT>(z);
      }
      u32x4 bq;
      if constexpr (DT == DT_F16) {
        // fp16: (1024 + q) - (1024 + z) is exact, so B = q - z directly
        const half2_t nmz = __builtin_bit_cast(half2_t, bc);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bq[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, magic_pair<DT>(wv[t], i)) + nmz);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) bq[i] = magic_pair<DT>(wv[t], i);
      }
      const u32x4 bcv = {bc, bc, bc, bc};
      const int k = c * 32 + row4 * 8;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + col;
        u32x4 a = {0u, 0u, 0u, 0u};
        if (m < p.M) a = *reinterpret_cast<const u32x4*>(p.x + (size_t)m * p.K + k);
        tmp[mt] = mfma16x16x32<DT>(a, bq, tmp[mt]);
        // bf16 has no packed add on gfx950: B = 128 + q, and a second MFMA
        // against the constant -(128 + z) removes the offset in fp32
        if constexpr (DT == DT_BF16) tmp[mt] = mfma16x16x32<DT>(a, bcv, tmp[mt]);
      }
      if ((t % CPG == CPG - 1) || c + 1 == p.nchunks) {
        const float s = nvalid ? act_to_f32<DT>(srow[grp]) : 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt] += s * tmp[mt];
          tmp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }

  // ---- cross-wave reduction in wave order ----
  float* mine = red + wave * NEL;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mine[(mt * 4 + r) * 64 + lane] = acc[mt][r];
  __syncthreads();

  for (int e = threadIdx.x; e < NEL; e += blockDim.x) {
    float v = 0.f;
    for (int w = 0; w < nwaves; ++w) v += red[w * NEL + e];
    const int mt = e >> 8;
    const int r = (e >> 6) & 3;
    const int l = e & 63;
    const int m = mt * 16 + 4 * (l >> 4) + r;
    const int nn = tile * kGemvRowsPerTile + (l & 15);
    if (m < p.M && nn < p.N) {
      if (p.splits == 1) {
        if (p.bias) v += act_to_f32<DT>(p.bias[nn]);
        p.y[(size_t)m * p.N + nn] = f32_to_act<DT>(v);
      } else {
        p.partial[((size_t)split * p.M + m) * p.N + nn] = v;
      }
    }
  }

  if (p.splits == 1) return;

  // ---- split fix-up: the last workgroup of this row tile adds the ranges ----
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == (uint32_t)(p.splits - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int e = threadIdx.x; e < 16 * p.M; e += blockDim.x) {
    const int m = e >> 4;
    const int nn = tile * kGemvRowsPerTile + (e & 15);
    if (nn < p.N) {
      float v = 0.f;
      for (int s = 0; s < p.splits; ++s) {
        float* src = p.partial + ((size_t)s * p.M + m) * p.N + nn;
        v += *src;
        // leave the whole workspace zero: a later call of another shape may
        // place its counters where these partial sums were
        *src = 0.f;
      }
      if (p.bias) v += act_to_f32<DT>(p.bias[nn]);
      p.y[(size_t)m * p.N + nn] = f32_to_act<DT>(v);
    }
  }
  if (threadIdx.x == 0) p.counters[tile] = 0u;  // ready for the next call
}

// ---------------------------------------------------------------------------

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int cu_count) {
  GemvPlan p;
  p.tiles = (int)((N + kGemvRowsPerTile - 1) / kGemvRowsPerTile);
  p.ksteps = (int)((K + kGemvKStep - 1) / kGemvKStep);
  p.mtiles = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  int splits = 1;
  if (p.tiles < cu_count) {
    splits = (cu_count + p.tiles - 1) / p.tiles;
    if (splits > p.ksteps) splits = p.ksteps;
  }
  p.ksteps_per_split = (p.ksteps + splits - 1) / splits;
  p.splits = (p.ksteps + p.ksteps_per_split - 1) / p.ksteps_per_split;
  int waves = (p.ksteps_per_split + 1) / 2;
  if (waves < 1) waves = 1;
  if (waves > kGemvMaxWaves) waves = kGemvMaxWaves;
  p.waves = waves;
  return p;
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t gemv_workspace_bytes(const GemvPlan& p, int64_t M, int64_t N) {
  if (p.splits <= 1) return 0;
  return align_up((size_t)p.tiles * sizeof(uint32_t), 256) +
         (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

template <int DT, int MT, int GS, bool ASYM>
static hipError_t launch_t(const GemvParams& prm, const GemvPlan& plan, hipStream_t s) {
  dim3 grid(plan.tiles, plan.splits);
  dim3 block(plan.waves * 64);
  hipLaunchKernelGGL((gemv_kernel<DT, MT, GS, ASYM>), grid, block, 0, s, prm);
  return hipGetLastError();
}

template <int DT, int MT, int GS>
static hipError_t launch_z(const GemvParams& prm, const GemvPlan& plan, hipStream_t s) {
  return prm.zp ? launch_t<DT, MT, GS, true>(prm, plan, s) : launch_t<DT, MT, GS, false>(prm, plan, s);
}

template <int DT, int MT>
static hipError_t launch_g(const GemvParams& prm, int group, const GemvPlan& plan, hipStream_t s) {
  switch (group) {
    case 32: return launch_z<DT, MT, 32>(prm, plan, s);
    case 64: return launch_z<DT, MT, 64>(prm, plan, s);
    case 128: return launch_z<DT, MT, 128>(prm, plan, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
static hipError_t launch_m(const GemvParams& prm, int group, const GemvPlan& plan, hipStream_t s) {
  switch (plan.mtiles) {
    case 1: return launch_g<DT, 1>(prm, group, plan, s);
    case 2: return launch_g<DT, 2>(prm, group, plan, s);
    case 4: return launch_g<DT, 4>(prm, group, plan, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const LinearArgs& a, const GemvPlan& plan, void* workspace,
                       hipStream_t stream) {
  GemvParams prm;
  prm.x = static_cast<const uint16_t*>(a.x);
  prm.wq = reinterpret_cast<const uint32_t*>(a.wq);
  prm.scales = static_cast<const uint16_t*>(a.scales);
  prm.zp = reinterpret_cast<const uint32_t*>(a.zp);
  prm.bias = static_cast<const uint16_t*>(a.bias);
  prm.y = static_cast<uint16_t*>(a.y);
  prm.counters = nullptr;
  prm.partial = nullptr;
  if (plan.splits > 1) {
    prm.counters = static_cast<uint32_t*>(workspace);
    prm.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           align_up((size_t)plan.tiles * sizeof(uint32_t), 256));
  }
  prm.M = (int)a.M;
  prm.N = (int)a.N;
  prm.K = (int)a.K;
  prm.G = (int)(a.K / a.group);
  prm.nchunks = (int)(a.K / 32);
  prm.ksteps = plan.ksteps;
  prm.ksteps_per_split = plan.ksteps_per_split;
  prm.splits = plan.splits;
  return a.dtype == DT_F16 ? launch_m<DT_F16>(prm, a.group, plan, stream)
                           : launch_m<DT_BF16>(prm, a.group, plan, stream);
}

}  // namespace w4a16
