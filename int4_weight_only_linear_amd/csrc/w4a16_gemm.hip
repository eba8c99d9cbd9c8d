// Prefill W4A16 GEMM for gfx950: y = x . dequant(Wq)^T (+ bias) with fp16 /
// bf16 MFMA and fp32 accumulation.
//
// The pages route M above the decode threshold to a fused dequantise-then-
// GEMM kernel ("[ROCm][Kernel] Add HybridW4A16LinearKernel: Triton prefill +
// HIP skinny decode", description).  Here it is hand-written for CDNA4:
//
// * A workgroup (4 waves) owns BM = 32*MB tokens by 256 output features; each
//   wave owns 64 features (two 32-wide blocks) across all BM tokens, so every
//   weight is dequantised exactly once per workgroup, by the wave that
//   multiplies it.
// * A k-step is one stored 128-k run of each weight row.  The weights are the
//   MFMA A operand (v_mfma_f32_32x32x16): lane (j, h) needs 8 consecutive k of
//   row j, i.e. one packed word, and the run's 4x4 word transpose puts the
//   eight words a lane needs for the whole k-step into two 16-byte loads.
//   They are dequantised in registers (the exact per-weight value that
//   w4a16_dequant returns) and fed straight to the MFMA: no LDS round trip.
// * The activations x are the B operand.  They are staged in LDS by direct
//   global->LDS loads (global_load_lds_dwordx4), double buffered, with the
//   16-byte pieces of each 256-byte row XOR-swizzled by (row mod 16) so the
//   fragment reads of 16 consecutive lanes hit 16 different bank groups.
// * The output tile of a wave is 64 features x BM tokens; in the MFMA result
//   layout a lane holds 4 consecutive features of one token, and one
//   permlane32 swap turns two such quads into 16 contiguous output bytes.
// * Work units (tile, K split) are remapped so that consecutive units -- the
//   same token rows, neighbouring features -- run on the same XCD and share
//   its L2.  With more than one split, units store fp32 partial tiles and the
//   last one to finish a tile adds them up in split order (deterministic).
// * DENSE instances multiply already dequantised act-dtype weights w[N, K]
//   (the dequantised prefill copy): the same tiles, staging, pipeline and
//   epilogue, with each lane's A fragments loaded straight from w's rows
//   (eight 16-byte loads per column block and k-step) instead of unpacked
//   from codes.
#include <algorithm>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"


namespace w4a16 {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;         // k per step: one stored run of every row
constexpr int kXRowBytes = 256;  // one staged x row: 128 k of 16-bit values
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

struct GemmParams {
  const uint16_t* x;
  const uint32_t* wq;
  const uint16_t* scales;
  const uint32_t* zp;
  const uint16_t* bias;
  uint16_t* y;
  float* partial;
  uint32_t* counters;
  int M, N, K, G;
  int sG, gmul;        // scale / zero-point index of (row n, group g): n * sG + g * gmul
  int wpr;             // words per weight row, K / 8
  int nsteps;          // ceil(K / 128)
  int full_steps;      // K / 128: steps over complete (transposed) runs
  int tiles_n;         // tiles per row of the plan's tile grid
  int units;           // grid size: this launch's tiles * splits
  // a tail launch covers tiles tile0.. of the plan's grid, each with two
  // tiles half as tall (this launch's instance; sub_m = 1); otherwise
  // tile0 = 0 and sub_m = 0 (sub_m is a shift and a mask: 0 or 1 only)
  int tile0, sub_m;
  int splits;
  int steps_per_split;
  int vec_store;       // y rows are 16-byte aligned and N % 8 == 0
  int two_pass;        // K split: store plain partials [split][M][np], summed by a second kernel
  int np;              // partial row stride: N rounded up to 8
};

// Workgroups are dispatched round-robin over the XCDs; give each XCD a
// contiguous range of work units instead.
__device__ __forceinline__ int xcd_unit(int b, int units) {
  const int q = units / kXcds, r = units % kXcds;
  const int xcd = b % kXcds, local = b / kXcds;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

template <int DT, int GS, bool ASYM, int MB, int CB, bool DENSE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmParams p) {
  static_assert(!DENSE || (GS == 128 && !ASYM), "dense instances carry no quantisation");
  constexpr int BM = 32 * MB;
  constexpr int BN = 128 * CB;           // output features: 32 CB per wave
  constexpr int XBUF = BM * kXRowBytes;  // bytes of one x buffer
  constexpr int NDMA = BM / 16;          // 1 KiB global->LDS loads per wave and step
  constexpr int GPS = kBK / GS;          // groups per k-step
  // two separate arrays, so the compiler can tell that loads into one buffer
  // never alias fragment reads of the other (no wait on the former before
  // the latter)
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[XBUF];
  __shared__ __attribute__((aligned(1024))) unsigned char xs1[XBUF];
  // 32-token tiles prefetch two k-steps ahead: a third x buffer
  __shared__ __attribute__((aligned(1024))) unsigned char xs2[MB == 1 ? XBUF : 16];
  __shared__ uint32_t last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31;
  const int h = lane >> 5;

  const int unit = xcd_unit(blockIdx.x, p.units);
  const int tile = unit / p.splits;
  const int split = unit - tile * p.splits;
  // this launch's tile `tile` is half r of the plan's tile w (the same tile
  // when tile0 = 0 and sub_m = 0); a half wholly past M has nothing to do
  const int w = p.tile0 + (tile >> p.sub_m);
  const int wm = w / p.tiles_n;
  const int mt = (wm << p.sub_m) + (tile & p.sub_m);
  const int nt = w - wm * p.tiles_n;
  const int m0 = mt * BM;
  if (m0 >= p.M) return;
  const int nw0 = nt * BN + wave * 32 * CB;  // first output feature of this wave
  const int s_begin = split * p.steps_per_split;
  const int s_end = min(p.nsteps, s_begin + p.steps_per_split);
  const int s_full_end = min(s_end, p.full_steps);

  // ---- x staging: load d of this wave writes LDS rows row0 + 4d + lane/16;
  // lane position (lane & 15) of a row holds the row's piece pos ^ (row & 15).
  const int row0 = wave * (BM / 4);
  uint32_t xoff[NDMA];
#pragma unroll
  for (int d = 0; d < NDMA; ++d) {
    const int row = row0 + 4 * d + (lane >> 4);
    const int piece = (lane & 15) ^ (row & 15);
    const int m = min(m0 + row, p.M - 1);
    xoff[d] = ((uint32_t)m * (uint32_t)p.K + 8u * (uint32_t)piece) * 2u;
  }
  auto stage_x = [&](int s, lds_u8* buf, bool tail, int d0, int d1) {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(p.x) + (size_t)s * kXRowBytes;
    const int kvalid = p.K - s * kBK;  // < 128 only on the last, incomplete run
#pragma unroll
    for (int d = d0; d < d1; ++d) {
      uint32_t off = xoff[d];
      if (tail) {
        // pieces past K would read beyond the row (and the buffer, on the
        // last row): point them at piece 0; their k-steps are never used
        const int row = row0 + 4 * d + (lane >> 4);
        const int piece = (lane & 15) ^ (row & 15);
        if (8 * piece >= kvalid) off -= 16u * (uint32_t)piece;
      }
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + off),
                                       buf + (row0 + 4 * d) * kXRowBytes,
                                       16, 0, 0);
    }
  };

  // ---- weights: lane j of column block cb reads row n = nw0 + 32 cb + j,
  // pieces h and h + 2 (16 bytes each) of every run.  In a complete 16-row
  // tile, run s is a 1 KiB block at tile start + 1024 s and piece pc of row
  // n is its piece 16 pc + (n mod 16); a final incomplete tile keeps its
  // rows one after another (64-byte runs).  The incomplete last run of a
  // row (slice order) is tail_w[cb] words in, T = wpr - 16 full_steps words.
  int nrow[CB];
  uint32_t woff[CB][2];   // [cb][pc]: byte offset of piece h + 2 pc in run 0
  uint32_t rshift[CB];    // run s starts s << rshift bytes further
  uint32_t tail_w[CB];
  // DENSE: byte offset of k = 8 h in row n of w; k-step s adds 256 s bytes
  // and k-sub ks 32 ks
  uint32_t doff[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = min(nw0 + 32 * cb + j, p.N - 1);
    nrow[cb] = n;
    doff[cb] = (uint32_t)n * (uint32_t)p.K * 2u + 16u * (uint32_t)h;
    const int jj = n & 15;
    const uint32_t t0 = (uint32_t)(n - jj) * (uint32_t)p.wpr;  // tile start, words
    const int tail_words = p.wpr - 16 * p.full_steps;
    if (n - jj + 16 <= p.N) {
      woff[cb][0] = t0 * 4u + (uint32_t)(16 * h + jj) * 16u;
      woff[cb][1] = woff[cb][0] + 512u;
      rshift[cb] = 10u;
      tail_w[cb] = t0 + 256u * (uint32_t)p.full_steps + (uint32_t)(jj * tail_words);
    } else {
      woff[cb][0] = (uint32_t)n * (uint32_t)p.wpr * 4u + 16u * (uint32_t)h;
      woff[cb][1] = woff[cb][0] + 32u;
      rshift[cb] = 6u;
      tail_w[cb] = (uint32_t)n * (uint32_t)p.wpr + 16u * (uint32_t)p.full_steps;
    }
  }

  constexpr int WP = DENSE ? 8 : 2;  // 16-byte weight pieces per column block and k-step
  struct StepRegs {
    u32x4 w[CB][WP];      // [cb][piece]: word t of piece pc is k-sub 2t + pc
                          // (DENSE: piece ks holds k-sub ks as 8 act values)
    uint16_t s[CB][GPS];  // scales of the step's groups
    uint32_t z[CB][GPS];  // packed zero-point words
  };
  // complete run: pieces h and h + 2 of the run's four 16-byte pieces
  auto load_full = [&](int s, StepRegs& r) {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(p.wq);
    if constexpr (DENSE) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          r.w[cb][ks] = *reinterpret_cast<const u32x4*>(base + (uint32_t)(s * 256 + 32 * ks) + doff[cb]);
      return;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const uint32_t run = (uint32_t)s << rshift[cb];
#pragma unroll
      for (int pc = 0; pc < 2; ++pc)
        r.w[cb][pc] = *reinterpret_cast<const u32x4*>(base + run + woff[cb][pc]);
    }
  };
  // incomplete run, stored in slice order: k-sub ks of half h is word 2 ks + h
  auto load_tail = [&](int s, StepRegs& r) {
    const int nks = (p.K - s * kBK) / 16;
    if constexpr (DENSE) {
      const unsigned char* base = reinterpret_cast<const unsigned char*>(p.wq);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          r.w[cb][ks] = ks < nks ? *reinterpret_cast<const u32x4*>(base + (uint32_t)(s * 256 + 32 * ks) + doff[cb])
                                 : u32x4{0u, 0u, 0u, 0u};
      return;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint32_t v = 0u;
        if (ks < nks) v = p.wq[(size_t)tail_w[cb] + 2 * ks + h];
        r.w[cb][ks & 1][ks >> 1] = v;
      }
  };
  auto load_meta = [&](int s, StepRegs& r) {
    if constexpr (DENSE) return;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) {
        const int g = min(s * GPS + gi, p.G - 1);
        r.s[cb][gi] = p.scales[(size_t)nrow[cb] * p.sG + g * p.gmul];
        if constexpr (ASYM) r.z[cb][gi] = p.zp[(size_t)(nrow[cb] >> 3) * p.sG + g * p.gmul];
      }
  };

  // ---- x fragment reads: row 32 rb + j, piece 2 ks + h, at position
  // (2 ks + h) ^ (j & 15) = 2 (ks ^ c2) + (h ^ c1)
  const int c2 = (j & 15) >> 1;
  const uint32_t xlane = (uint32_t)j * kXRowBytes + (uint32_t)((h ^ (j & 1)) << 4);

  f32x16 acc[MB][CB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][cb][e] = 0.f;

  auto group_consts = [&](const StepRegs& r, GroupConst<DT> (&gc)[CB][GPS]) {
    if constexpr (DENSE) return;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) {
        const uint32_t z = ASYM ? (r.z[cb][gi] >> (4 * (nrow[cb] & 7))) & 0xFu : 8u;
        gc[cb][gi] = group_const<DT, true>(r.s[cb][gi], z);
      }
  };
  auto weights = [&](const StepRegs& r, const GroupConst<DT> (&gc)[CB][GPS], int ks, u32x4 (&a)[CB]) {
    if constexpr (DENSE) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) a[cb] = r.w[cb][ks];
      return;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const GroupConst<DT>& g = gc[cb][(16 * ks) / GS];
      a[cb] = dequant_word<DT, true>(r.w[cb][ks & 1][ks >> 1], g.s_pair, g.nmz_pair, g.s_f32, g.c_f32);
    }
  };
  auto xfrags = [&](const lds_u8* buf, int ks, u32x4 (&b)[MB]) {
    const lds_u8* src = buf + xlane + (uint32_t)((ks ^ c2) << 5);
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) b[rb] = *(lds_u32x4*)(src + rb * 32 * kXRowBytes);
  };
  auto mfmas = [&](const u32x4 (&a)[CB], const u32x4 (&b)[MB]) {
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mfma32x32x16<DT>(a[cb], b[rb], acc[rb][cb]);
  };

  // Pipeline state carried across k-steps: the operands of the k-sub about
  // to be multiplied (by parity) and the current step's group constants.
  u32x4 a[2][CB], b[2][MB];
  GroupConst<DT> gc[CB][GPS];

  // Own x pieces landed in LDS, own loads and LDS reads retired, then the
  // workgroup barrier (no memory fence beyond that is needed: the x pieces
  // reach LDS before their load counter drops).
  auto step_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // 32-token tiles: the step after next has issued its metadata, then its
  // WP * CB weight loads and NDMA x loads, each one instruction and the last
  // vector memory instructions before this barrier; waiting until at most
  // those are outstanding leaves them in flight and covers everything older
  // (the next step's loads and x pieces)
  constexpr int kKeep = WP * CB + NDMA;
  static_assert(kKeep < 64, "vmcnt");
  auto step_barrier_keep = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    // vmcnt(kKeep) (bits 3:0 and 15:14), expcnt any, lgkmcnt(0)
    __builtin_amdgcn_s_waitcnt((kKeep & 15) | ((kKeep >> 4) << 14) | (7 << 4));
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // One complete k-step, software pipelined: the x fragments and dequantised
  // weights of k-sub ks + 1 are produced while the MFMAs of ks run, and the
  // scheduler is told to interleave them (per MFMA: a few VALU ops and at
  // most one LDS read) so the matrix core never waits on either.  The global
  // loads of the next k-step are spread over k-subs 0..5 (issue(ks)).  The
  // step's single barrier sits before its last k-sub: by then every wave's
  // loads of the next step have landed and every wave has read its last
  // fragments of this step, so the next step's first fragments (nbuf, nr)
  // are produced while the last MFMAs of this one run.  On the last step
  // nbuf / nr hold valid but unused data and the prefetch is simply wasted.
  auto compute = [&](const lds_u8* buf, const StepRegs& r, const lds_u8* nbuf,
                     const StepRegs& nr, auto&& issue, auto&& barrier) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int c = ks & 1, nx = c ^ 1;
      if (ks < 7) {
        xfrags(buf, ks + 1, b[nx]);
        weights(r, gc, ks + 1, a[nx]);
      } else {
        barrier();
        group_consts(nr, gc);
        xfrags(nbuf, 0, b[nx]);
        weights(nr, gc, 0, a[nx]);
      }
      const int nvm = issue(ks);
      mfmas(a[c], b[c]);
#pragma unroll
      for (int i = 0; i < CB * MB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (i < MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, (24 * CB + CB * MB - 1) / (CB * MB), 0);  // VALU
        if (i < nvm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the incomplete last run: nks < 8 k-subs, not pipelined
  auto compute_tail = [&](const lds_u8* buf, const StepRegs& r, int nks) {
    GroupConst<DT> gc[CB][GPS];
    group_consts(r, gc);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < nks) {
        u32x4 a[CB], b[MB];
        xfrags(buf, ks, b);
        weights(r, gc, ks, a);
        mfmas(a, b);
      }
    }
  };

  lds_u8* const buf0 = (lds_u8*)xs0;
  lds_u8* const buf1 = (lds_u8*)xs1;

  // the next k-step's global loads, spread over k-subs 0..5 of the current
  // one: weights first (k-sub 0), then metadata, then the x pieces
  constexpr int kMetaLoads = DENSE ? 0 : CB * GPS * (ASYM ? 2 : 1);
  auto issue_next = [&](int ks, int sn, lds_u8* buf, StepRegs& r) -> int {
    constexpr int DPK = (NDMA + 5) / 6;  // x loads per k-sub
    int n = 0;
    if (ks == 0) {
      load_full(sn, r);
      n += WP * CB;
    }
    if (ks == 1) {
      load_meta(sn, r);
      n += kMetaLoads;
    }
    if (ks < 6) {
      const int d0 = ks * DPK, d1 = min(NDMA, d0 + DPK);
      if (d0 < d1) stage_x(sn, buf, false, d0, d1);
      n += max(0, d1 - d0);
    }
    return n;
  };
  auto no_issue = [](int) -> int { return 0; };
  // 32-token tiles: the step after next, all at the first k-sub, in the
  // order step_barrier_keep's count relies on (metadata, weights, x pieces)
  auto issue_deep = [&](int ks, int sn, lds_u8* buf, StepRegs& r) -> int {
    if (ks == 0) {
      __builtin_amdgcn_sched_barrier(0);
      load_meta(sn, r);
      __builtin_amdgcn_sched_barrier(0);
      load_full(sn, r);
      __builtin_amdgcn_sched_barrier(0);
      stage_x(sn, buf, false, 0, NDMA);
      __builtin_amdgcn_sched_barrier(0);
    }
    return 0;
  };

  // ---- main loop over complete runs, two steps per iteration so that each
  // LDS buffer and register set is a compile-time choice; the loop has no
  // exit in its middle (an odd last step is peeled), which lets the
  // accumulators stay in the same registers throughout
  StepRegs ra = {}, rb_ = {};
  int s = s_begin;
  const int nfull = s_full_end - s_begin;
  if constexpr (MB == 1) {
    // 32-token tiles: three x buffers and register sets, the loads of step
    // s + 2 issued during step s (a thin tile's k-step is shorter than a
    // memory round trip); steps past the range reload the last one into the
    // free set (never used)
    StepRegs rc_ = {};
    lds_u8* const buf2 = (lds_u8*)xs2;
    if (nfull > 0) {
      stage_x(s, buf0, false, 0, NDMA);
      load_full(s, ra);
      load_meta(s, ra);
      issue_deep(0, min(s + 1, s_full_end - 1), buf1, rb_);
      step_barrier_keep();  // step s landed everywhere; s + 1 may be in flight
      group_consts(ra, gc);
      xfrags(buf0, 0, b[0]);
      weights(ra, gc, 0, a[0]);
      int left = nfull;
      for (; left >= 3; left -= 3) {
        compute(buf0, ra, buf1, rb_, [&](int ks) { return issue_deep(ks, min(s + 2, s_full_end - 1), buf2, rc_); },
                step_barrier_keep);
        ++s;
        compute(buf1, rb_, buf2, rc_, [&](int ks) { return issue_deep(ks, min(s + 2, s_full_end - 1), buf0, ra); },
                step_barrier_keep);
        ++s;
        compute(buf2, rc_, buf0, ra, [&](int ks) { return issue_deep(ks, min(s + 2, s_full_end - 1), buf1, rb_); },
                step_barrier_keep);
        ++s;
      }
      // the last one or two steps issue nothing and wait for everything at
      // their barrier (loads whose registers are never read again may be
      // dropped by the compiler, which would upset a partial count)
      if (left >= 1) {
        compute(buf0, ra, buf1, rb_, no_issue, step_barrier);
        ++s;
      }
      if (left >= 2) {
        compute(buf1, rb_, buf2, rc_, no_issue, step_barrier);
        ++s;
      }
      wait_vm_all();  // no prefetch in flight (into LDS or registers) past the loop
    }
  } else if (nfull > 0) {
    stage_x(s, buf0, false, 0, NDMA);
    load_full(s, ra);
    load_meta(s, ra);
    __syncthreads();  // step s landed everywhere
    group_consts(ra, gc);
    xfrags(buf0, 0, b[0]);
    weights(ra, gc, 0, a[0]);
    for (int it = 0; it < (nfull >> 1); ++it) {
      compute(buf0, ra, buf1, rb_, [&](int ks) { return issue_next(ks, s + 1, buf1, rb_); }, step_barrier);
      ++s;
      // after the last pair there is no next step: load a valid one into the
      // free buffer instead of branching (never used)
      const int sn = min(s + 1, s_full_end - 1);
      compute(buf1, rb_, buf0, ra, [&](int ks) { return issue_next(ks, sn, buf0, ra); }, step_barrier);
      ++s;
    }
    if (nfull & 1) {
      compute(buf0, ra, buf1, rb_, no_issue, step_barrier);
      ++s;
    }
  }
  // ---- the incomplete last run (K % 128 != 0), unpipelined
  if (s < s_end) {
    __syncthreads();  // every wave is done with both buffers
    stage_x(s, buf0, true, 0, NDMA);
    load_tail(s, ra);
    load_meta(s, ra);
    wait_vm_all();
    __syncthreads();
    compute_tail(buf0, ra, (p.K - s * kBK) / 16);
  }

  // ---- split-K: store the partial tile; the last unit of the tile sums them
  // in split order (cross-workgroup hand-off as described at store_coherent).
  // Values travel in 8-byte pairs; thread tid's pair i of a partial tile sits
  // at pair index i * kThreads + tid.  The sum runs over chunks of kChunk
  // values: for each split in turn all of a chunk's loads are issued before
  // any is used, so a chunk costs one memory round trip per split.
  // (compiled for the 128-token tile only: in the taller tiles' kernels this
  // block costs the accumulators their registers, and the planner uses the
  // two-pass form at small M only)
  if constexpr (MB == 1 || MB == 4) if (p.splits > 1 && p.two_pass) {
    // plain fp32 partial sums, row-major [split][M][np]; splitk_reduce_kernel
    // adds the splits in order.  acc[rb][cb][4a + e] is token m0 + 32 rb + j,
    // feature nw0 + 32 cb + 8a + 4h + e: four consecutive features, 16 bytes.
    float* part = p.partial + (size_t)split * p.M * p.np;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      const int m = m0 + 32 * rb + j;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int n = nw0 + 32 * cb + 8 * a + 4 * h;
          if (m < p.M && n < p.np)
            *reinterpret_cast<f32x4*>(part + (size_t)m * p.np + n) =
                f32x4{acc[rb][cb][4 * a], acc[rb][cb][4 * a + 1], acc[rb][cb][4 * a + 2],
                      acc[rb][cb][4 * a + 3]};
        }
    }
    return;
  }
  if (p.splits > 1) {
    constexpr int NV = MB * CB * 16;  // accumulator values per thread
    constexpr int kChunk = NV < 64 ? NV : 64;
    static_assert(NV % kChunk == 0, "chunking");
    const size_t slot = (size_t)BM * BN / 2;  // pairs per partial tile
    auto val = [&](int q) -> float { return acc[q / (16 * CB)][(q / 16) % CB][q % 16]; };
    uint64_t* mine = reinterpret_cast<uint64_t*>(p.partial) + (size_t)(tile * p.splits + split) * slot;
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) store_coherent_pair(mine + (size_t)i * kThreads + tid, val(2 * i), val(2 * i + 1));
    // every thread's partial sums have completed (stores count in vmcnt on
    // gfx950; the barrier itself does not wait for them), then one arrival
    wait_vm_all();
    __syncthreads();
    if (tid == 0) last_flag = (arrive(p.counters + tile) == (uint32_t)(p.splits - 1));
    __syncthreads();
    if (!last_flag) return;
    const uint64_t* first = reinterpret_cast<const uint64_t*>(p.partial) + (size_t)tile * p.splits * slot;
#pragma unroll
    for (int c0 = 0; c0 < NV; c0 += kChunk) {
      float t[kChunk];
      for (int sp = 0; sp < p.splits; ++sp) {
        float u[kChunk];
        if (sp == split) {
#pragma unroll
          for (int e = 0; e < kChunk; ++e) u[e] = val(c0 + e);
        } else {
#pragma unroll
          for (int e = 0; e < kChunk; e += 2)
            load_coherent_pair(first + sp * slot + (size_t)((c0 + e) / 2) * kThreads + tid, u[e], u[e + 1]);
        }
#pragma unroll
        for (int e = 0; e < kChunk; ++e) t[e] = sp == 0 ? u[e] : t[e] + u[e];
      }
#pragma unroll
      for (int e = 0; e < kChunk; ++e) acc[(c0 + e) / (16 * CB)][((c0 + e) / 16) % CB][(c0 + e) % 16] = t[e];
    }
    if (tid == 0) reset_counter(p.counters + tile);  // ready for the next call
  }

  // ---- epilogue: + bias in fp32, one rounding, 16-byte stores
  // acc[rb][cb][4a + e] is token m0 + 32 rb + j, feature nw0 + 32 cb + 8a + 4h + e
  float bias_f[CB][4][4];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = nw0 + 32 * cb + 8 * a + 4 * h + e;
        bias_f[cb][a][e] = (p.bias && n < p.N) ? act_to_f32<DT>(p.bias[n]) : 0.f;
      }
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    const int m = m0 + 32 * rb + j;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      uint32_t q[4][2];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x16& v = acc[rb][cb];
        q[a][0] = f32x2_to_act_pair<DT>(v[4 * a] + bias_f[cb][a][0], v[4 * a + 1] + bias_f[cb][a][1]);
        q[a][1] = f32x2_to_act_pair<DT>(v[4 * a + 2] + bias_f[cb][a][2], v[4 * a + 3] + bias_f[cb][a][3]);
      }
      // lanes h = 0 / 1 of quads (a, a + 1) hold features 8a + 0..3 / 8a + 4..7;
      // after the swap lane h holds the 8 features 8(a + h) + 0..7
#pragma unroll
      for (int a = 0; a < 4; a += 2) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(q[a][0], q[a + 1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(q[a][1], q[a + 1][1], false, false);
        const u32x4 out = u32x4{s0[0], s1[0], s0[1], s1[1]};
        const int n = nw0 + 32 * cb + 8 * (a + h);
        if (m < p.M) {
          uint16_t* dst = p.y + (size_t)m * p.N + n;
          if (p.vec_store) {
            if (n < p.N) *reinterpret_cast<u32x4*>(dst) = out;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < p.N) dst[e] = (uint16_t)(out[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
}

// The K split's second pass: y = sum of the splits' fp32 partials, in split
// order, + bias in fp32, one rounding.  One thread per row and 4 consecutive
// features.
template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y, int M, int N,
                                                            int np, int splits) {
  const int qpr = np >> 2;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= (int64_t)M * qpr) return;
  const int m = (int)(q / qpr), n = (int)(q % qpr) * 4;
  const size_t plane = (size_t)M * np;
  const float* src = partial + (size_t)m * np + n;
  f32x4 s = *reinterpret_cast<const f32x4*>(src);
  for (int sp = 1; sp < splits; ++sp) s += *reinterpret_cast<const f32x4*>(src + sp * plane);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (n + e < N) {
      float v = s[e];
      if (bias) v += act_to_f32<DT>(bias[n + e]);
      y[(size_t)m * N + n + e] = f32_to_act<DT>(v);
    }
}

template <int DT, int GS, bool ASYM, int MB, int CB, bool DENSE>
hipError_t launch_t(const GemmParams& prm, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<DT, GS, ASYM, MB, CB, DENSE>), dim3(prm.units), dim3(kThreads), 0, s, prm);
  return hipGetLastError();
}

// tile shapes: 32 mb tokens x 128 cb features; cb = 1 only for mb 1, 4 and 8
template <int DT, int GS, bool ASYM, bool DENSE = false>
hipError_t launch_mb(const GemmParams& prm, int mb, int cb, hipStream_t s) {
  if (cb == 1) {
    switch (mb) {
      case 1: return launch_t<DT, GS, ASYM, 1, 1, DENSE>(prm, s);
      case 4: return launch_t<DT, GS, ASYM, 4, 1, DENSE>(prm, s);
      case 8: return launch_t<DT, GS, ASYM, 8, 1, DENSE>(prm, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (mb) {
    case 1: return launch_t<DT, GS, ASYM, 1, 2, DENSE>(prm, s);
    case 4: return launch_t<DT, GS, ASYM, 4, 2, DENSE>(prm, s);
    case 6: return launch_t<DT, GS, ASYM, 6, 2, DENSE>(prm, s);
    case 8: return launch_t<DT, GS, ASYM, 8, 2, DENSE>(prm, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int GS>
hipError_t launch_z(const GemmParams& prm, int mb, int cb, hipStream_t s) {
  return prm.zp ? launch_mb<DT, GS, true>(prm, mb, cb, s) : launch_mb<DT, GS, false>(prm, mb, cb, s);
}

template <int DT>
hipError_t launch_g(const GemmParams& prm, int group, int mb, int cb, hipStream_t s) {
  switch (group) {
    case 32: return launch_z<DT, 32>(prm, mb, cb, s);
    case 64: return launch_z<DT, 64>(prm, mb, cb, s);
    case 128: return launch_z<DT, 128>(prm, mb, cb, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Tile shape and K split.  Cost model in cycles of one CU, fitted to
// measured k-step times (about 380 cycles per 32 tokens and 128 features of
// the tile plus a fixed 1000: MFMA issue, dequantisation and staging share
// one instruction stream per SIMD); units run in rounds of cu_count; splitting
// K adds the partial-tile hand-off.  Narrow tiles (128 features, one column
// block per wave) double the tile count at small M, where 256-feature tiles
// leave CUs idle or need K splits whose partial sums outweigh the weights.
// Tile heights 192 and 256 with 256-feature tiles, for the dtype / group /
// zero-point combinations whose kernel instances spill registers to scratch
// memory with this compiler (fp16 with groups of 32, or of 64 with zero
// points; bf16 with groups of 32 without): a k-step of four or two groups
// keeps its group constants and the next step's metadata beside 192-256
// accumulators.  Measured at M = 1920 on 6144x4096 they run 1.2-3.6x slower
// than the 128-token tile, so the planner leaves them out.
// Dense instances (no group constants) at tile heights 192 and 256 with
// 256-feature tiles: their eight 16-byte weight pieces per column block and
// k-step stand where the codes and metadata stood.
bool dense_tall_tile_spills(int dtype) {
  (void)dtype;
  return false;
}

bool wide_tall_tile_spills(int group, int dtype, bool asym) {
  if (dtype == DT_F16) return group == 32 || (group == 64 && asym);
  return group == 32 && !asym;
}

// Up to 64 tokens: 32-token tiles of 128 features (the weights of a tile
// are dequantised once for at most 32 tokens, so at small M the matrix cores
// no longer multiply up to 96 padding rows of a 128-token tile).  A thin
// tile's k-step is shorter than a memory round trip, so it prefetches two
// k-steps (the kernel's MB == 1 loop) and K is split until enough units are
// resident; time model in microseconds, fitted to every K split (1-16, both
// hand-off forms) at M = 16 and 48 on ten Llama- and Qwen-shaped layers
// (K 2560-28672; mean error 6 %, its picks 3.6 % from the best on average,
// 18 % at worst): 0.528 * k-steps per unit * max(1, units / 224) +
// 0.528 per extra K range + partial-sum traffic (0.108 us per MB two-pass,
// 0.314 one-pass) + 4.91 (- 0.06 two-pass).
// Against the 128-token tiles' plans: M = 9-32 -15 to -33 % on eight layers
// (Llama and Qwen shapes, fp16 and bf16, groups 32 and 128); M = 48 / 64
// lower where K <= 16384; 28672 x 4096 keeps the 128-token tiles above
// M = 32 (a tie at M = 48).
// the second kernel of a tail launch: its start after the first one drains
constexpr double kTailLaunchCycles = 4000.0;

static GemmPlan plan_gemm_thin(int64_t M, int64_t N, int64_t K) {
  GemmPlan best{};
  double best_t = 0.0;
  const int nsteps = (int)((K + kBK - 1) / kBK);
  const int64_t tiles_n = (N + 127) / 128;
  const int64_t tiles = ((M + 31) / 32) * tiles_n;
  for (int splits = 1; splits <= 16 && splits <= nsteps; ++splits) {
    const int sps = (nsteps + splits - 1) / splits;
    if ((nsteps + sps - 1) / sps != splits) continue;
    const int64_t units = tiles * splits;
    const double resident = units > 224 ? (double)units / 224.0 : 1.0;
    const double part_mb = splits > 1 ? (double)splits * (double)M * (double)N * 4.0 / 1e6 : 0.0;
    for (int tp = 0; tp < (splits > 1 ? 2 : 1); ++tp) {
      if (tp == 0 && splits > 1 && tiles > kMaxCounters) continue;
      const double t = 0.528 * sps * resident + 0.528 * (splits - 1) + (tp ? 0.108 : 0.314) * part_mb + 4.91 -
                       0.06 * tp;
      if (best.units == 0 || t < best_t) {
        best_t = t;
        best.mb = 1;
        best.cb = 1;
        best.splits = splits;
        best.steps_per_split = sps;
        best.tiles_n = (int)tiles_n;
        best.tiles = (int)tiles;
        best.units = (int)units;
        best.two_pass = tp == 1;
      }
    }
  }
  return best;
}

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int group, int dtype, bool asym, int cu_count,
                   bool dense) {
  GemmPlan best{};
  const bool tall_wide_ok = dense ? !dense_tall_tile_spills(dtype) : !wide_tall_tile_spills(group, dtype, asym);
  // where the tall wide tiles are left out, narrow tiles are tried first, so
  // that near-ties go to them: at M = 1920 on 6144x4096 they beat the
  // 128-token wide tile by 1-20 % for those combinations
  const int cb_order[2] = {tall_wide_ok ? 2 : 1, tall_wide_ok ? 1 : 2};
  double best_cost = 0.0;
  // (the dense instances too: the same tiles and splits)
  const bool thin = M <= 32 || (M <= 64 && K <= 16384);
  if (thin) best = plan_gemm_thin(M, N, K);
  const int nsteps = (int)((K + kBK - 1) / kBK);
  const int cus = cu_count > 0 ? cu_count : 256;
  for (int cb : cb_order) {
    if (thin) break;
    const int64_t bn = 128 * cb;
    const int64_t tiles_n = (N + bn - 1) / bn;
    for (int mb : {8, 6, 4}) {
      if (cb == 1 && mb == 6) continue;
      if (cb == 2 && mb > 4 && !tall_wide_ok) continue;
      const int64_t bm = 32 * mb;
      const int64_t tiles = ((M + bm - 1) / bm) * tiles_n;
      for (int splits = 1; splits <= 16 && splits <= nsteps; ++splits) {
        const int sps = (nsteps + splits - 1) / splits;
        const int real_splits = (nsteps + sps - 1) / sps;
        if (real_splits != splits) continue;

        const int64_t units = tiles * splits;
        const int64_t rounds = (units + cus - 1) / cus;
        // a split unit writes its fp32 partial tile; the tile's last unit then
        // reads the others back, one memory round trip (~2500 cycles) per
        // split and 64-value chunk, plus the bytes (mostly from L2 / MALL)
        const double fixup = splits > 1 ? 2.0 * bm * bn * 4 / 40.0 +
                                             2500.0 * splits * (16.0 * cb * mb / 64.0) : 0.0;
        const double loop = sps * (380.0 * cb * mb + 1000.0);
        const double cost = (double)rounds * (loop + fixup);
        // two passes: each unit stores its partial tile (~64 bytes a cycle),
        // then a second kernel reads all partials plus its launch; the
        // partials' round trip is taken as 3 TB/s at 2.1 GHz (fitted to every
        // plan timed at M = 128-512 on 4096x6144, 4096x28672 and 14336x4096)
        const double np = (double)((N + 7) / 8 * 8);
        const double cost2 = (double)rounds * (loop + bm * bn * 4 / 64.0) +
                             (splits * (double)M * np * 4.0 + (double)M * N * 2.0) * (2.1e9 / 3e12) + 3000.0;
        for (int tp = 0; tp < (splits > 1 && mb == 4 ? 2 : 1); ++tp) {
          const double c = tp ? cost2 : cost;
          if (tp == 0 && splits > 1 && tiles > kMaxCounters) continue;
          if (best.units == 0 || c < best_cost * 0.98) {
            best_cost = c;
            best = GemmPlan{};
            best.mb = mb;
            best.cb = cb;
            best.splits = splits;
            best.steps_per_split = sps;
            best.tiles_n = (int)tiles_n;
            best.tiles = (int)tiles;
            best.units = (int)units;
            best.two_pass = tp == 1;
          }
        }
        // Tail launch: where the unsplit 256-token tiles end in a partial
        // round, the tiles past the last full round run as a second launch of
        // 128-token tiles, in one round; halves wholly past M cost nothing
        // (4096 x 28672 at M = 1920: 896 tiles of 256 x 256 are 3.5 rounds, the
        // last half of the CUs idle; as 3 rounds plus 144 tiles of 128 x 256
        // it measured -5.6 %).  A tail k-step takes at least 0.8 of the plan
        // tile's (its loads' round trip, not its MFMAs, sets the pace: measured
        // 0.77-0.82 for 128 x 256 tails, 0.89 for 128 x 128 tails of 256 x 256
        // tiles, which the planner therefore never picks).
        if (mb == 8 && splits == 1 && units > cus && units % cus != 0) {
          const int64_t full = units / cus * cus;
          int64_t busy = 0;  // halves with output to compute
          for (int64_t w = full; w < tiles; ++w) busy += (w / tiles_n) * bm + bm / 2 < M ? 2 : 1;
          const double tstep = std::max(380.0 * cb * 4 + 1000.0, 0.8 * (380.0 * cb * mb + 1000.0));
          const double tc = (double)(full / cus) * loop + (double)((busy + cus - 1) / cus) * nsteps * tstep +
                            kTailLaunchCycles;
          if (tc < best_cost * 0.98) {
            best_cost = tc;
            best = GemmPlan{};
            best.mb = mb;
            best.cb = cb;
            best.splits = 1;
            best.steps_per_split = sps;
            best.tiles_n = (int)tiles_n;
            best.tiles = (int)tiles;
            best.units = (int)full;
            best.tail_mb = 4;
            best.tail_tile0 = (int)full;
            best.tail_units = (int)(2 * (tiles - full));
          }
        }
      }
    }
  }
  // tuning override "mb,splits[,two_pass[,cb]]" (tile 32*mb x 128*cb, K ranges), e.g. for sweeps
  const Tuning& tu = tuning();
  if (tu.gemm_tile_n >= 2) {
    const int mb = tu.gemm_tile[0], splits = tu.gemm_tile[1];
    const int tp = tu.gemm_tile_n >= 3 ? tu.gemm_tile[2] : 0;
    const int cb = tu.gemm_tile_n >= 4 ? tu.gemm_tile[3] : 2;
    if ((mb == 1 || mb == 4 || mb == 6 || mb == 8) &&
        (cb == 2 || (cb == 1 && mb != 6)) && splits >= 1 && splits <= nsteps && (tp == 0 || mb == 1 || mb == 4)) {
      const int sps = (nsteps + splits - 1) / splits;
      const int64_t tiles_n = (N + 128 * cb - 1) / (128 * cb);
      const int64_t tiles = ((M + 32 * mb - 1) / (32 * mb)) * tiles_n;
      if (splits == 1 || tp == 1 || tiles <= kMaxCounters) {
        best = GemmPlan{};
        best.two_pass = splits > 1 && tp == 1;
        best.mb = mb;
        best.cb = cb;
        best.steps_per_split = sps;
        best.splits = (nsteps + sps - 1) / sps;
        best.tiles_n = (int)tiles_n;
        best.tiles = (int)tiles;
        best.units = (int)(tiles * best.splits);
      }
    }
  }
  return best;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int group, int dtype, bool asym,
                            int cu_count, bool dense) {
  const GemmPlan p = plan_gemm(M, N, K, group, dtype, asym, cu_count, dense);
  if (p.splits <= 1) return 0;
  if (p.two_pass)
    return kCounterBytes + (size_t)p.splits * (size_t)M * (size_t)((N + 7) / 8 * 8) * sizeof(float);
  return kCounterBytes + (size_t)p.units * (size_t)(32 * p.mb) * (size_t)(128 * p.cb) * sizeof(float);
}

hipError_t launch_gemm(const LinearArgs& a, void* workspace, int cu_count, hipStream_t stream) {
  const GemmPlan plan = plan_gemm(a.M, a.N, a.K, a.group, a.dtype, a.zp != nullptr, cu_count, a.dense);
  GemmParams prm;
  prm.x = static_cast<const uint16_t*>(a.x);
  prm.wq = reinterpret_cast<const uint32_t*>(a.wq);
  prm.scales = static_cast<const uint16_t*>(a.scales);
  prm.zp = reinterpret_cast<const uint32_t*>(a.zp);
  prm.bias = static_cast<const uint16_t*>(a.bias);
  prm.y = static_cast<uint16_t*>(a.y);
  prm.counters = nullptr;
  prm.partial = nullptr;
  if (plan.splits > 1) {
    if (workspace == nullptr) return hipErrorInvalidValue;
    prm.counters = static_cast<uint32_t*>(workspace);
    prm.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
  }
  prm.M = (int)a.M;
  prm.N = (int)a.N;
  prm.K = (int)a.K;
  prm.G = (int)(a.K / a.group);
  prm.sG = a.sG;
  prm.gmul = a.gmul;
  prm.wpr = (int)(a.K / 8);
  prm.nsteps = (int)((a.K + kBK - 1) / kBK);
  prm.full_steps = (int)(a.K / kBK);
  prm.tiles_n = plan.tiles_n;
  prm.units = plan.units;
  prm.tile0 = 0;
  prm.sub_m = 0;
  prm.splits = plan.splits;
  prm.steps_per_split = plan.steps_per_split;
  prm.vec_store = (a.N % 8 == 0) && (reinterpret_cast<uintptr_t>(a.y) % 16 == 0);
  prm.two_pass = plan.splits > 1 && plan.two_pass;
  if (prm.two_pass && plan.mb != 1 && plan.mb != 4) return hipErrorInvalidConfiguration;
  if (plan.tail_units > 0 && (2 * plan.tail_mb != plan.mb || plan.splits != 1)) return hipErrorInvalidConfiguration;
  prm.np = (int)((a.N + 7) / 8 * 8);
  hipError_t e;
  if (a.dense)
    e = a.dtype == DT_F16 ? launch_mb<DT_F16, 128, false, true>(prm, plan.mb, plan.cb, stream)
                          : launch_mb<DT_BF16, 128, false, true>(prm, plan.mb, plan.cb, stream);
  else
    e = a.dtype == DT_F16 ? launch_g<DT_F16>(prm, a.group, plan.mb, plan.cb, stream)
                          : launch_g<DT_BF16>(prm, a.group, plan.mb, plan.cb, stream);
  if (e == hipSuccess && plan.tail_units > 0) {
    GemmParams t = prm;
    t.units = plan.tail_units;
    t.tile0 = plan.tail_tile0;
    t.sub_m = 1;
    if (a.dense)
      e = a.dtype == DT_F16 ? launch_mb<DT_F16, 128, false, true>(t, plan.tail_mb, plan.cb, stream)
                            : launch_mb<DT_BF16, 128, false, true>(t, plan.tail_mb, plan.cb, stream);
    else
      e = a.dtype == DT_F16 ? launch_g<DT_F16>(t, a.group, plan.tail_mb, plan.cb, stream)
                            : launch_g<DT_BF16>(t, a.group, plan.tail_mb, plan.cb, stream);
  }
  if (e != hipSuccess || !prm.two_pass) return e;
  const int64_t quads = (int64_t)prm.M * (prm.np / 4);
  const int blocks = (int)((quads + 255) / 256);
  if (a.dtype == DT_F16)
    hipLaunchKernelGGL(splitk_reduce_kernel<DT_F16>, dim3(blocks), dim3(256), 0, stream, prm.partial,
                       prm.bias, prm.y, prm.M, prm.N, prm.np, prm.splits);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<DT_BF16>, dim3(blocks), dim3(256), 0, stream, prm.partial,
                       prm.bias, prm.y, prm.M, prm.N, prm.np, prm.splits);
  return hipGetLastError();
}

}  // namespace w4a16
