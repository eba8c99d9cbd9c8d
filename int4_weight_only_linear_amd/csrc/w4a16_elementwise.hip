// Elementwise device kernels: exact dequantisation of the packed weights to
// the activation dtype (the per-weight value the linear kernels are defined
// against, and the building block of a dequantised prefill copy), and the
// device-side unpacking of the 4-bit codes.  Both are memory bound: one
// thread per weight word, 16-byte stores.
#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

template <int DT, bool ASYM>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ zp,
                                                      uint16_t* __restrict__ w, int64_t N,
                                                      int64_t K, int group, int sG, int gmul) {
  const int64_t words_per_row = K >> 3;
  const int64_t total = N * words_per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t n;
    int j;
    locate_word(idx, N, (int)words_per_row, n, j);
    const int64_t grp = ((int64_t)j * 8) / group;
    const uint16_t sbits = scales[n * sG + grp * gmul];
    const uint32_t z = ASYM ? zero_point(zp, (int)n, sG, (int)grp * gmul) : 8u;
    const GroupConst<DT> gc = group_const<DT>(sbits, z);
    *reinterpret_cast<u32x4*>(w + n * K + (int64_t)j * 8) = dequant_word<DT>(
        __builtin_nontemporal_load(wq + idx), gc.s_pair, gc.nmz_pair, gc.s_f32, gc.c_f32);
  }
}

// nibble t holds k-offset (0,2,4,6,1,3,5,7)[t] of the word's slice; output
// bytes in k order
__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* __restrict__ wq,
                                                     uint8_t* __restrict__ q, int64_t words,
                                                     int64_t N, int words_per_row) {
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < words;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t w = wq[idx];
    int64_t n;
    int j;
    locate_word(idx, N, words_per_row, n, j);
    const int64_t slice = n * words_per_row + j;
    const uint32_t even = w & 0x0000FFFFu;  // k = 0, 2, 4, 6 in nibbles 0..3
    const uint32_t odd = w >> 16;           // k = 1, 3, 5, 7 in nibbles 4..7
    uint32_t lo = 0, hi = 0;                // bytes k = 0..3 and 4..7
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo |= ((even >> (4 * i)) & 0xFu) << (16 * i);
      lo |= ((odd >> (4 * i)) & 0xFu) << (16 * i + 8);
      hi |= ((even >> (4 * i + 8)) & 0xFu) << (16 * i);
      hi |= ((odd >> (4 * i + 8)) & 0xFu) << (16 * i + 8);
    }
    *reinterpret_cast<u32x2*>(q + slice * 8) = u32x2{lo, hi};
  }
}

// p[0 .. n) = 0 with vector stores (a kernel rather than a memset, so that a
// caller may capture it in a graph)
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

int grid_for(int64_t items, int threads) {
  int64_t blocks = (items + threads - 1) / threads;
  const int64_t cap = 256 * 64;  // enough to fill the chip; the loops stride
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

hipError_t launch_dequant(const int32_t* wq, const void* scales, const int32_t* zp, int sG, int gmul, void* w,
                          int64_t N, int64_t K, int group, int dtype, hipStream_t stream) {
  const int64_t words = N * (K >> 3);
  const int blocks = grid_for(words, 256);
  const uint32_t* wqu = reinterpret_cast<const uint32_t*>(wq);
  const uint32_t* zpu = reinterpret_cast<const uint32_t*>(zp);
  const uint16_t* s = static_cast<const uint16_t*>(scales);
  uint16_t* out = static_cast<uint16_t*>(w);
  if (dtype == DT_F16) {
    if (zp)
      hipLaunchKernelGGL((dequant_kernel<DT_F16, true>), blocks, 256, 0, stream, wqu, s, zpu, out, N, K, group, sG, gmul);
    else
      hipLaunchKernelGGL((dequant_kernel<DT_F16, false>), blocks, 256, 0, stream, wqu, s, zpu, out, N, K, group, sG, gmul);
  } else {
    if (zp)
      hipLaunchKernelGGL((dequant_kernel<DT_BF16, true>), blocks, 256, 0, stream, wqu, s, zpu, out, N, K, group, sG, gmul);
    else
      hipLaunchKernelGGL((dequant_kernel<DT_BF16, false>), blocks, 256, 0, stream, wqu, s, zpu, out, N, K, group, sG, gmul);
  }
  return hipGetLastError();
}

hipError_t launch_zero_words(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / sizeof(uint32_t));
  hipLaunchKernelGGL(zero_words_kernel, grid_for(n, 256), 256, 0, stream, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_unpack(const int32_t* wq, uint8_t* q, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t words = N * (K >> 3);
  hipLaunchKernelGGL(unpack_kernel, grid_for(words, 256), 256, 0, stream,
                     reinterpret_cast<const uint32_t*>(wq), q, words, N, (int)(K >> 3));
  return hipGetLastError();
}

}  // namespace w4a16
