// Prefill W4A16 GEMM for gfx950: dequantise weight tiles into LDS, multiply
// with bf16/fp16 MFMA, accumulate in fp32.
//
// The pages route M above the decode threshold to a fused dequantise-then-
// GEMM kernel ("[ROCm][Kernel] Add HybridW4A16LinearKernel: Triton prefill +
// HIP skinny decode", description).  Here that kernel is hand-written HIP:
//
// * Workgroup tile BM x BN = 128 x 128, k-tile BK = 128 (one stored 128-k run
//   of each weight row), 256 threads (4 waves, each a 64 x 64 sub-tile of
//   4 x 4 v_mfma_f32_16x16x32 tiles).
// * Per k-tile each thread loads 128 B of x and two 16-byte pieces of one
//   weight row's run, dequantises them exactly -- (q - z) * s rounded once to
//   the activation dtype, the same value w4a16_dequant returns -- and stores
//   both to LDS in k order.  The next k-tile's global loads are issued before
//   the current one is multiplied.
// * LDS rows are padded by 16 bytes so the 16 lanes that read one MFMA
//   operand column hit different banks.
#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 128;
constexpr int LDK = BK + 8;  // padded LDS row, in 16-bit elements
constexpr int kThreads = 256;
constexpr int A_LOADS = BM * BK / 8 / kThreads;  // 16-byte x loads per thread (8)
constexpr size_t kLdsBytes = (size_t)(BM + BN) * LDK * sizeof(uint16_t);
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
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int nkt = (p.K + BK - 1) / BK;
  const int words_per_row = p.K >> 3;

  // weight loader: row b_row, 16-byte pieces b_q and b_q + 1 (stored words
  // 4*b_q .. 4*b_q + 7 of the row's run)
  const int b_row = tid >> 1;
  const int b_q0 = (tid & 1) * 2;
  const int b_n = n0 + b_row;
  const bool b_nvalid = b_n < p.N;
  const uint32_t* b_src = p.wq + (size_t)(b_nvalid ? b_n : 0) * words_per_row;

  u32x4 areg[A_LOADS];
  u32x4 breg[2];
  uint16_t b_s[2][4];
  uint32_t b_z[2][4];

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 4;  // 16 segments per 128-k row
      const int seg = id & 15;
      const int m = m0 + row;
      const int k = kt * BK + seg * 8;
      areg[i] = u32x4{0u, 0u, 0u, 0u};
      if (m < p.M && k < p.K) areg[i] = *reinterpret_cast<const u32x4*>(p.x + (size_t)m * p.K + k);
    }
    const bool complete = (kt + 1) * BK <= p.K;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = b_q0 + h;  // piece within the run
      breg[h] = u32x4{0u, 0u, 0u, 0u};
      const int w0 = kt * 16 + q * 4;  // first stored word of the piece
      if (b_nvalid && w0 < words_per_row) {
        breg[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b_src + w0));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // word t of the piece holds slice 4t + q of a complete run, or
          // slice 4q + t of an incomplete one (stored in order)
          const int slice = kt * 16 + (complete ? 4 * t + q : 4 * q + t);
          const int grp = min((slice * 8) / GS, p.G - 1);
          b_s[h][t] = p.scales[(size_t)b_n * p.G + grp];
          b_z[h][t] = ASYM ? zero_point(p.zp, b_n, p.G, grp) : 8u;
        }
      }
    }
  };

  auto store_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int id = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(&As[(id >> 4) * LDK + (id & 15) * 8]) = areg[i];
    }
    const bool complete = (kt + 1) * BK <= p.K;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = b_q0 + h;
      const int w0 = kt * 16 + q * 4;
      const bool valid = b_nvalid && w0 < words_per_row;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ks = complete ? 4 * t + q : 4 * q + t;  // slice within the tile
        u32x4 o4 = {0u, 0u, 0u, 0u};
        if (valid && (complete || kt * 16 + ks < words_per_row)) {
          const GroupConst<DT> gc = group_const<DT>(b_s[h][t], b_z[h][t]);
          uint32_t o[4];
          dequant_word_exact<DT>(breg[h][t], gc.s_pair, gc.nmz_pair, gc.s_f32, gc.c_f32, o);
          o4 = u32x4{o[0], o[1], o[2], o[3]};
        }
        *reinterpret_cast<u32x4*>(&Bs[b_row * LDK + ks * 8]) = o4;
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(0);
  const int frag_row = lane & 15;
  const int frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();  // the previous tile's MFMAs are done with the LDS
    store_tile(kt);
    __syncthreads();
    if (kt + 1 < nkt) load_tile(kt + 1);  // in flight while this tile is multiplied
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&As[(wm * 64 + i * 16 + frag_row) * LDK + kk + frag_k]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(&Bs[(wn * 64 + j * 16 + frag_row) * LDK + kk + frag_k]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32<DT>(af[i], bf[j], acc[i][j]);
    }
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
