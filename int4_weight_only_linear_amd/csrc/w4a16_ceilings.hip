// Measurement kernels for the ceilings the W4A16 path is judged against on
// one MI355X (gfx950).  They are not part of the linear layer: bench.py times
// them beside it, on the same buffers and launch shapes, so that its roofline
// fractions can be read against what this device actually sustains as well
// as against the published peaks.
//
//   w4a16c_stream_read    plain streaming read of a buffer (16-byte
//                         non-temporal loads, grid-stride): the HBM read rate
//                         a kernel that only reads reaches on these bytes.
//   w4a16c_decode_loads   the decode kernel's weight loads alone, in its
//                         grid: one workgroup per 16-row tile, each wave a run
//                         of kpw contiguous 1 KiB loads, nothing computed.
//                         With a tile stride above the packed tile's bytes it
//                         reads a row-padded copy instead (row-stride padding
//                         against HBM channel camping, the MI355X analogue of
//                         the cache-cliff padding the page "Converge the two
//                         W4A16 linear kernels onto the upstream shell"
//                         describes in "What this does").
//   w4a16c_mfma_loop      independent chains of 32x32x16 bf16 MFMAs on
//                         register operands drawn from a hash (random bits, as
//                         real operands are: the clock under load depends on
//                         them), one or more waves per SIMD: the matrix-core
//                         rate this device sustains, clock included.
//
// Every kernel folds what it reads into a value that is stored only when it
// equals a constant no input produces in practice, so the loads cannot be
// removed, and nothing is written otherwise.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16_ceilings.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr uint32_t kNever = 0x9E3779B9u;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                          uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    acc ^= __builtin_nontemporal_load(p + i);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == kNever) sink[0] = acc.x;
}

// One workgroup per 16-row tile (blockIdx.x), `waves` waves; wave w loads
// k-steps w*KPW .. w*KPW + KPW - 1 of the tile (those below ksteps), each a
// contiguous 1 KiB block at tile start + 1024 * step, lane l its 16 bytes.
// As in the decode kernel, every load of the wave is issued before the first
// is used (KPW is a compile-time count, the loop unrolled; a wave past the
// last k-step re-reads the last block, as the decode kernel does).
template <int KPW>
__global__ __launch_bounds__(1024) void decode_loads_kernel(const char* __restrict__ base,
                                                            int64_t tile_stride, int ksteps,
                                                            uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* tile = base + (int64_t)blockIdx.x * tile_stride + 16 * lane;
  const int first = wave * KPW;
  u32x4 v[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int ks = min(first + i, ksteps - 1);
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tile + 1024 * (int64_t)ks));
  }
  u32x4 acc = v[0];
#pragma unroll
  for (int i = 1; i < KPW; ++i) acc ^= v[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == kNever) sink[0] = acc.x;
}

__device__ __forceinline__ uint32_t hash32(uint32_t v) {
  v ^= v >> 16;
  v *= 0x7FEB352Du;
  v ^= v >> 15;
  v *= 0x846CA68Bu;
  v ^= v >> 16;
  return v;
}

// Four independent accumulator chains per wave, `iters` rounds of four
// MFMAs.  The operands are bf16 bit patterns from a hash with the exponent
// field kept in a normal range (finite, non-trivial products).
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, uint32_t seed, uint32_t* sink) {
  const uint32_t id = (blockIdx.x * blockDim.x + threadIdx.x) * 16u + seed;
  u32x4 a[2], b[2];
  for (int i = 0; i < 2; ++i)
    for (int e = 0; e < 4; ++e) {
      // sign and mantissa random, exponent 120..135 in both halves
      a[i][e] = (hash32(id + 8 * i + e) & 0x807F807Fu) | 0x3C003C00u | ((hash32(id ^ 0x55u) & 0x00F000F0u) << 3);
      b[i][e] = (hash32(id + 8 * i + e + 4) & 0x807F807Fu) | 0x3C003C00u | ((hash32(id ^ 0xAAu) & 0x00F000F0u) << 3);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, a[0]), a1 = __builtin_bit_cast(bf16x8_t, a[1]);
  const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, b[0]), b1 = __builtin_bit_cast(bf16x8_t, b[1]);
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (__builtin_bit_cast(uint32_t, s) == kNever) sink[0] = 1u;
}

int grid_for(int64_t n16) {
  int64_t b = (n16 + 255) / 256;
  if (b > 256 * 32) b = 256 * 32;
  return (int)(b < 1 ? 1 : b);
}

}  // namespace

extern "C" {

int w4a16c_stream_read(const void* buf, uint64_t bytes, void* sink, void* stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || bytes % 16) return (int)hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid_for(n16)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), n16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

int w4a16c_decode_loads(const void* wq, uint64_t buf_bytes, int64_t tiles, int64_t K, int64_t tile_stride,
                        int32_t kpw, int32_t waves, void* sink, void* stream) {
  if (!wq || !sink || (reinterpret_cast<uintptr_t>(wq) & 15) || tiles < 1 || K < 128 || K % 128 ||
      kpw < 1 || kpw > 16 || (kpw & (kpw - 1)) || waves < 1 || waves > 16 || tile_stride < 8 * K ||
      tile_stride % 16 ||
      (uint64_t)(tiles - 1) * (uint64_t)tile_stride + (uint64_t)(8 * K) > buf_bytes ||
      (int64_t)waves * kpw < K / 128 || tiles > 0x7FFFFFFF)
    return (int)hipErrorInvalidValue;
  const dim3 grid((uint32_t)tiles), block(64 * waves);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* b = static_cast<const char*>(wq);
  uint32_t* k = static_cast<uint32_t*>(sink);
  const int ks = (int)(K / 128);
  switch (kpw) {
    case 1: hipLaunchKernelGGL(decode_loads_kernel<1>, grid, block, 0, s, b, tile_stride, ks, k); break;
    case 2: hipLaunchKernelGGL(decode_loads_kernel<2>, grid, block, 0, s, b, tile_stride, ks, k); break;
    case 4: hipLaunchKernelGGL(decode_loads_kernel<4>, grid, block, 0, s, b, tile_stride, ks, k); break;
    case 8: hipLaunchKernelGGL(decode_loads_kernel<8>, grid, block, 0, s, b, tile_stride, ks, k); break;
    case 16: hipLaunchKernelGGL(decode_loads_kernel<16>, grid, block, 0, s, b, tile_stride, ks, k); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int w4a16c_mfma_loop(int32_t blocks, int32_t iters, uint32_t seed, void* sink, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     seed, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

}  // extern "C"
