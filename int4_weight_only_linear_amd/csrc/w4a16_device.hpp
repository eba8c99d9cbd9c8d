// Device-side building blocks shared by the W4A16 kernels (gfx950 only).
//
// Weight words follow the layout of include/w4a16.h: nibble t of a word holds
// k-offset (0,2,4,6,1,3,5,7)[t] of its 8-k slice, so (w >> 4i) & 0x000F000F
// places the consecutive pair (k = 2i, 2i+1) in the low and high 16-bit
// halves; complete 128-k runs of a row store their 16 words as a 4x4
// transpose (word 4r+t holds slice 4t+r), so a 16-byte load of words
// 4r..4r+3 yields slice r of each of the run's four 32-k chunks.
//
// Dequantisation uses the exponent-OR ("magic number") trick named in the
// description of "[ROCm][Kernel] Add HybridW4A16LinearKernel: Triton prefill
// + HIP skinny decode": OR-ing a nibble into the mantissa of a power of two
// whose unit in the last place is 1 yields magic + q exactly, with no integer
// to float conversion.  fp16 uses 1024 (0x6400), bf16 uses 128 (0x4300).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };

template <int DT>
struct Magic;
template <>
struct Magic<DT_F16> {
  static constexpr uint32_t pair = 0x64006400u;  // two fp16 1024.0
  static constexpr uint32_t neg = 0xE400u;       // fp16 -1024.0; OR a nibble z for -(1024+z)
  static constexpr float value = 1024.0f;
};
template <>
struct Magic<DT_BF16> {
  static constexpr uint32_t pair = 0x43004300u;  // two bf16 128.0
  static constexpr uint32_t neg = 0xC300u;       // bf16 -128.0; OR a nibble z for -(128+z)
  static constexpr float value = 128.0f;
};

// magic + q for the weight pair (k = 2i, 2i+1) of a word, as two act values
template <int DT>
__device__ __forceinline__ uint32_t magic_pair(uint32_t w, int i) {
  return ((w >> (4 * i)) & 0x000F000Fu) | Magic<DT>::pair;
}

// A 32-bit constant the compiler must keep in a VGPR.  gfx9 VOP3 encodings
// take no literal constants and read at most one SGPR, so (w & mask) | magic
// becomes a single v_and_or_b32 only when one of the two constants already
// sits in a VGPR; otherwise the compiler splits it into v_and_b32 + v_or_b32.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// The four magic pairs of one word: out[i] = magic + (k = 2i, 2i+1), three
// shifts and four AND-ORs.  mask_v = vgpr_const(0x000F000F).
template <int DT>
__device__ __forceinline__ u32x4 magic_word(uint32_t w, uint32_t mask_v) {
  return u32x4{(w & mask_v) | Magic<DT>::pair, ((w >> 4) & mask_v) | Magic<DT>::pair,
               ((w >> 8) & mask_v) | Magic<DT>::pair, ((w >> 12) & mask_v) | Magic<DT>::pair};
}

// fp16 pair add on scalar words.  (Applying __builtin_bit_cast to an element
// of an ext_vector in an unrolled loop was miscompiled by this compiler: the
// later elements read the already-updated first one.  Keep such arithmetic
// on scalars and build vectors from the results.)
__device__ __forceinline__ uint32_t add_f16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) + __builtin_bit_cast(half2_t, b));
}

// fp16: the four pairs q - z of one word, exact: (1024 + q) + (-(1024 + z))
__device__ __forceinline__ u32x4 qz_word_f16(uint32_t w, uint32_t mask_v, uint32_t nmz) {
  constexpr uint32_t P = Magic<DT_F16>::pair;
  const uint32_t p0 = (w & mask_v) | P, p1 = ((w >> 4) & mask_v) | P;
  const uint32_t p2 = ((w >> 8) & mask_v) | P, p3 = ((w >> 12) & mask_v) | P;
  return u32x4{add_f16x2(p0, nmz), add_f16x2(p1, nmz), add_f16x2(p2, nmz), add_f16x2(p3, nmz)};
}

// acc + (low half + high half) of a bf16 pair, in fp32
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}

// The 8-k slice held by stored word j of a row of J words (see above).
__device__ __forceinline__ int slice_of_stored_word(int j, int J) {
  const int run = j >> 4, p = j & 15;
  if ((run + 1) * 16 > J) return j;
  return (run << 4) + 4 * (p & 3) + (p >> 2);
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time, so
// register arrays indexed by I are never indexed dynamically
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Row n and 8-k slice of the word at flat index idx of the packed weights
// (N rows of J words).  Complete 16-row tiles are stored tile-major: per
// complete run a 256-word block whose 16-byte piece 16 r + row holds run
// words 4r..4r+3 of that row, then the rows' incomplete runs row after row;
// a final incomplete tile keeps its rows one after another.
__device__ __forceinline__ void locate_word(int64_t idx, int64_t N, int J, int64_t& n, int& slice) {
  const int64_t tile_words = 16 * (int64_t)J;
  const int64_t tile = idx / tile_words;
  if (tile >= (N >> 4)) {
    n = idx / J;
    slice = slice_of_stored_word((int)(idx - n * J), J);
    return;
  }
  const int off = (int)(idx - tile * tile_words);
  const int runs = J >> 4;
  if (off < 256 * runs) {
    const int piece = (off & 255) >> 2, e = off & 3;
    n = tile * 16 + (piece & 15);
    slice = ((off >> 8) << 4) + 4 * e + (piece >> 4);  // run word 4r+e holds slice 4e+r
  } else {
    const int tail = J - (runs << 4);
    const int t = off - 256 * runs;
    const int row = t / tail;
    n = tile * 16 + row;
    slice = (runs << 4) + (t - row * tail);
  }
}

// -(magic + z) in both halves of a word
template <int DT>
__device__ __forceinline__ uint32_t neg_magic_pair(uint32_t z) {
  const uint32_t h = Magic<DT>::neg | z;
  return h | (h << 16);
}

template <int DT>
__device__ __forceinline__ float act_to_f32(uint16_t b) {
  if constexpr (DT == DT_F16) {
    return (float)__builtin_bit_cast(_Float16, b);
  } else {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
  }
}

// float32 -> activation dtype, round to nearest even (v_cvt_f16_f32 /
// v_cvt_pk_bf16_f32 under the default rounding mode)
template <int DT>
__device__ __forceinline__ uint16_t f32_to_act(float f) {
  if constexpr (DT == DT_F16) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  } else {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  }
}

template <int DT>
__device__ __forceinline__ uint32_t f32x2_to_act_pair(float lo, float hi) {
  if constexpr (DT == DT_F16) {
    half2_t h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    bf16x2_t h = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, h);
  }
}

// 16x16x32 MFMA, fp32 accumulate.  Operand layout (per lane l of the wave):
//   A[i][k]: i = l % 16, k = 8 * (l / 16) + e, e = 0..7 (the 8 packed values)
//   B[k][j]: j = l % 16, same k
//   D[i][j]: j = l % 16, i = 4 * (l / 16) + r, r = 0..3
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32x16 MFMA, fp32 accumulate.  Operand layout (per lane l of the wave):
//   A[i][k]: i = l % 32, k = 8 * (l / 32) + e, e = 0..7 (the 8 packed values)
//   B[k][j]: j = l % 32, same k
//   D[i][j]: j = l % 32, i = 8 * (r / 4) + 4 * (l / 32) + r % 4, r = 0..15
template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
}

// 4x4 transpose of dwords across the four 16-lane rows of a wave:
// on entry lane row j holds v[t] = element (j, t); on exit it holds (t, j).
// Two rounds of row swaps: rows {0,1} <-> {2,3}, then odd <-> even rows.
__device__ __forceinline__ void transpose_rows4(u32x4& v) {
  auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v[0] = c[0];
  v[1] = c[1];
  v[2] = d[0];
  v[3] = d[1];
}

// v & 0x0F0F0F0F as one v_and_b32 the optimiser cannot see through
__device__ __forceinline__ uint32_t mask_nibbles(uint32_t v) {
  uint32_t r;
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(r) : "v"(v));
  return r;
}

// Exact dequantisation of one word (8 weights) to activation-dtype pairs:
// element i holds k = 2i (low half) and 2i+1 (high half), each (q - z) * s
// rounded once to nearest even.
//   fp16: (magic + q) - (magic + z) is exact in fp16 (|q - z| <= 15), the
//         product with s is one correctly rounded fp16 multiply.
//   bf16: the codes become fp32 through byte conversions (the even and odd
//         nibbles masked into bytes), then fma(q, s, -z * s): q * s and z * s
//         need at most 4 + 8 significant bits, so both and their difference
//         (q - z) * s are exact in fp32, and one nearest-even conversion per
//         pair rounds them to bf16.
//   bf16, FP8Q: the masked bytes are read as OCP e4m3 numbers instead: a
//         byte b in [0, 15] is exactly b * 2^-9 (b < 8 are the subnormals,
//         b >= 8 the lowest normal binade, both spaced 2^-9), and one
//         v_cvt_pk_f32_fp8 converts two of them, where the byte form takes
//         one instruction per code (19 VALU per word instead of 23).  With
//         s_f32 = s * 2^9 the fma's exact product is again q * s, so the
//         result is bit-identical as long as s * 2^9 is finite (|s| < 2^119).
// s_pair: the scale in both halves and nmz_pair = -(magic + z) in both halves
// (fp16); s_f32 = s (s * 2^9 with FP8Q) and c_f32 = -z * s (bf16); the
// constants come from group_const<DT, FP8Q>.
template <int DT, bool FP8Q = false>
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, uint32_t s_pair, uint32_t nmz_pair,
                                              float s_f32, float c_f32) {
  if constexpr (DT == DT_F16) {
    const half2_t s2 = __builtin_bit_cast(half2_t, s_pair);
    const half2_t nmz = __builtin_bit_cast(half2_t, nmz_pair);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t v = __builtin_bit_cast(half2_t, magic_pair<DT_F16>(w, i));
      v = v + nmz;
      v = v * s2;
      o[i] = __builtin_bit_cast(uint32_t, v);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
  } else {
    // nibbles 0,2,4,6 (k = 0, 4, 1, 5) and 1,3,5,7 (k = 2, 6, 3, 7) in bytes;
    // the masks are opaque to the compiler, which would otherwise fold each
    // byte conversion back into a per-nibble bitfield extract
    const uint32_t ev = mask_nibbles(w);
    const uint32_t od = mask_nibbles(w >> 4);
    if constexpr (!FP8Q) {
      auto f = [&](uint32_t v, int b) {
        return __builtin_fmaf((float)((v >> (8 * b)) & 0xFFu), s_f32, c_f32);
      };
      return u32x4{f32x2_to_act_pair<DT_BF16>(f(ev, 0), f(ev, 2)),
                   f32x2_to_act_pair<DT_BF16>(f(od, 0), f(od, 2)),
                   f32x2_to_act_pair<DT_BF16>(f(ev, 1), f(ev, 3)),
                   f32x2_to_act_pair<DT_BF16>(f(od, 1), f(od, 3))};
    } else {
      // bytes (0, 1) and (2, 3) of each masked word
      const f32x2 e0 = __builtin_amdgcn_cvt_pk_f32_fp8(ev, false);
      const f32x2 e1 = __builtin_amdgcn_cvt_pk_f32_fp8(ev, true);
      const f32x2 o0 = __builtin_amdgcn_cvt_pk_f32_fp8(od, false);
      const f32x2 o1 = __builtin_amdgcn_cvt_pk_f32_fp8(od, true);
      auto f = [&](float q) { return __builtin_fmaf(q, s_f32, c_f32); };
      return u32x4{f32x2_to_act_pair<DT_BF16>(f(e0[0]), f(e1[0])),
                   f32x2_to_act_pair<DT_BF16>(f(o0[0]), f(o1[0])),
                   f32x2_to_act_pair<DT_BF16>(f(e0[1]), f(e1[1])),
                   f32x2_to_act_pair<DT_BF16>(f(o0[1]), f(o1[1]))};
    }
  }
}

// per (row, group) constants for dequant_word
template <int DT>
struct GroupConst {
  uint32_t s_pair;
  uint32_t nmz_pair;
  float s_f32;
  float c_f32;
};

template <int DT, bool FP8Q = false>
__device__ __forceinline__ GroupConst<DT> group_const(uint16_t s_bits, uint32_t z) {
  GroupConst<DT> g;
  g.s_pair = (uint32_t)s_bits | ((uint32_t)s_bits << 16);
  g.nmz_pair = neg_magic_pair<DT>(z);
  g.s_f32 = act_to_f32<DT>(s_bits);
  g.c_f32 = -(float)z * g.s_f32;  // exact: 4 + 8 significant bits (bf16 only)
  if constexpr (FP8Q && DT == DT_BF16) g.s_f32 *= 512.0f;  // undoes the codes' 2^-9
  return g;
}

// s_waitcnt vmcnt(0): every vector memory access of this wave has completed
// (gfx9 counts stores in vmcnt too).  expcnt and lgkmcnt fields left at their
// maxima, so only vmcnt is waited for.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Cross-workgroup hand-off of fp32 partial sums (split K) without
// cache-wide maintenance.  Every XCD has its own L2, so agent-scope
// release/acquire fences write back and invalidate the whole L2 of the XCD
// (buffer_wbl2 / buffer_inv); done by every split workgroup, that costs far
// more than the hand-off and evicts the weights the other workgroups are
// streaming.  Instead the partial sums themselves are written and read with
// agent-scope relaxed atomic accesses (write-through to, and reads from, the
// device-coherent level), and the order comes from explicit waits: each wave
// waits for its own partial-sum stores to complete (wait_vm_all: a workgroup
// barrier alone does not wait for outstanding stores), then a workgroup
// barrier, then one thread increments the completion counter; the counter's
// result, shared through LDS and a barrier, orders the last workgroup's
// loads after every other workgroup's completed stores.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_pair(uint64_t* p, float lo, float hi) {
  const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, lo) |
                     ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void load_coherent_pair(const uint64_t* p, float& lo, float& hi) {
  const uint64_t v = __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lo = __builtin_bit_cast(float, (uint32_t)v);
  hi = __builtin_bit_cast(float, (uint32_t)(v >> 32));
}
__device__ __forceinline__ uint32_t arrive(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t zero_point(const uint32_t* zp, int n, int G, int grp) {
  return (zp[(size_t)(n >> 3) * G + grp] >> (4 * (n & 7))) & 0xFu;
}

}  // namespace w4a16
