// Prefill W4A16 GEMM for gfx950: dequantise weight tiles into LDS, multiply
// with bf16/fp16 MFMA, accumulate in fp32.
//
// The pages route M above the decode threshold to a fused dequantise-then-
// GEMM kernel ("[ROCm][Kernel] Add HybridW4A16LinearKernel: Triton prefill +
// HIP skinny decode", description).  Here that kernel is hand-written HIP:
//
// * Workgroup tile BM x BN = 128 x 128, k-tile BK = 64, 256 threads (4
//   waves, each a 64 x 64 sub-tile of 4 x 4 v_mfma_f32_16x16x32 tiles).
// * Per k-tile each thread loads 64 B of x and one 16-byte weight chunk
//   (32 k of one row), dequantises the chunk exactly -- (q - z) * s rounded
//   once to the activation dtype, the same value w4a16_dequant returns -- and
//   stores both to LDS.  The next k-tile's global loads are in flight while
//   the current one is multiplied (two LDS buffers).
// * LDS rows are padded by 16 bytes so the 16 lanes that read one MFMA
//   operand column hit different banks.
#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row, in 16-bit elements
constexpr int kThreads = 256;
constexpr size_t kLdsBytes = 2 * (size_t)(BM + BN) * LDK * sizeof(uint16_t);
static_assert(kLdsBytes <= 160 * 1024, "GEMM tiles exceed the 160 KiB of LDS per CU");

struct GemmParams {
  const uint16_t* x;
  const uint32_t* wq;
  const uint16_t* scales;
  const uint32_t* zp;
  const uint16_t* bias;
  uint16_t* y;
  int M, N, K, G;
  int nchunks;
};

template <int DT, int GS, bool ASYM>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int nkt = (p.K + BK - 1) / BK;

  // loader roles
  const int b_row = tid >> 1;    // weight row within the tile
  const int b_chunk = tid & 1;   // which 32-k chunk of the k-tile
  const int b_n = n0 + b_row;
  const bool b_nvalid = b_n < p.N;
  const uint32_t* b_src = p.wq + (size_t)(b_nvalid ? b_n : 0) * (p.K >> 3);

  u32x4 areg[4];
  u32x4 breg;
  uint16_t b_sbits = 0;
  uint32_t b_z = 8u;
  bool b_valid = false;

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3;
      const int seg = id & 7;
      const int m = m0 + row;
      const int k = kt * BK + seg * 8;
      areg[i] = u32x4{0u, 0u, 0u, 0u};
      if (m < p.M && k < p.K) areg[i] = *reinterpret_cast<const u32x4*>(p.x + (size_t)m * p.K + k);
    }
    const int c = kt * 2 + b_chunk;
    b_valid = b_nvalid && c < p.nchunks;
    breg = u32x4{0u, 0u, 0u, 0u};
    if (b_valid) {
      breg = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b_src + (size_t)c * 4));
      const int grp = (c * 32) / GS;
      b_sbits = p.scales[(size_t)b_n * p.G + grp];
      b_z = ASYM ? zero_point(p.zp, b_n, p.G, grp) : 8u;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3;
      const int seg = id & 7;
      *reinterpret_cast<u32x4*>(&As[buf][row * LDK + seg * 8]) = areg[i];
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(&Bs[buf][b_row * LDK + b_chunk * 32]);
    if (b_valid) {
      const GroupConst<DT> gc = group_const<DT>(b_sbits, b_z);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t o[4];
        dequant_word_exact<DT>(breg[w], gc.s_pair, gc.nmz_pair, gc.s_f32, gc.c_f32, o);
        *reinterpret_cast<u32x4*>(dst + w * 4) = u32x4{o[0], o[1], o[2], o[3]};
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) *reinterpret_cast<u32x4*>(dst + w * 4) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int frag_row = lane & 15;
  const int frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&As[buf][(wm * 64 + i * 16 + frag_row) * LDK + kk + frag_k]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(&Bs[buf][(wn * 64 + j * 16 + frag_row) * LDK + kk + frag_k]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32<DT>(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: + bias in fp32, one rounding to the activation dtype
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nn = n0 + wn * 64 + j * 16 + (lane & 15);
    if (nn >= p.N) continue;
    const float b = p.bias ? act_to_f32<DT>(p.bias[nn]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (m < p.M) {
          float v = acc[i][j][r];
          if (p.bias) v += b;
          p.y[(size_t)m * p.N + nn] = f32_to_act<DT>(v);
        }
      }
    }
  }
}

template <int DT, int GS, bool ASYM>
hipError_t launch_t(const GemmParams& prm, hipStream_t s) {
  dim3 grid((prm.N + BN - 1) / BN, (prm.M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_kernel<DT, GS, ASYM>), grid, dim3(kThreads), 0, s, prm);
  return hipGetLastError();
}

template <int DT, int GS>
hipError_t launch_z(const GemmParams& prm, hipStream_t s) {
  return prm.zp ? launch_t<DT, GS, true>(prm, s) : launch_t<DT, GS, false>(prm, s);
}

template <int DT>
hipError_t launch_g(const GemmParams& prm, int group, hipStream_t s) {
  switch (group) {
    case 32: return launch_z<DT, 32>(prm, s);
    case 64: return launch_z<DT, 64>(prm, s);
    case 128: return launch_z<DT, 128>(prm, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_gemm(const LinearArgs& a, void*, int, hipStream_t stream) {
  GemmParams prm;
  prm.x = static_cast<const uint16_t*>(a.x);
  prm.wq = reinterpret_cast<const uint32_t*>(a.wq);
  prm.scales = static_cast<const uint16_t*>(a.scales);
  prm.zp = reinterpret_cast<const uint32_t*>(a.zp);
  prm.bias = static_cast<const uint16_t*>(a.bias);
  prm.y = static_cast<uint16_t*>(a.y);
  prm.M = (int)a.M;
  prm.N = (int)a.N;
  prm.K = (int)a.K;
  prm.G = (int)(a.K / a.group);
  prm.nchunks = (int)(a.K / 32);
  return a.dtype == DT_F16 ? launch_g<DT_F16>(prm, a.group, stream)
                           : launch_g<DT_BF16>(prm, a.group, stream);
}

}  // namespace w4a16
