/*
 * libw4a16_ceilings -- measurement kernels for the ceilings of the W4A16
 * linear path on one MI355X (gfx950).  Not part of the linear layer: the
 * benchmark times them beside it to state what this device sustains (HBM
 * read rate of the same bytes, the decode kernel's load pattern alone, the
 * matrix-core rate under sustained load) next to the published peaks.
 *
 * All pointers are device pointers owned by the caller; launches are
 * asynchronous on `stream` (a hipStream_t, NULL = default).  Each kernel
 * writes `sink` (4 bytes) only if what it read folds to one fixed constant,
 * which keeps its loads from being optimised away.  Each function returns a
 * hipError_t value (0 = success; hipErrorInvalidValue for arguments outside
 * the rules below, checked on the host before any launch).
 */
#ifndef W4A16_CEILINGS_H
#define W4A16_CEILINGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16) of `buf` (16-byte aligned) once, with
 * 16-byte non-temporal loads, grid-stride over at most 8192 workgroups. */
int w4a16c_stream_read(const void* buf, uint64_t bytes, void* sink, void* stream);

/* The decode kernel's weight loads alone: `tiles` workgroups of `waves`
 * waves (1..16); tile t starts at wq + t * tile_stride and holds K/128 blocks
 * of 1 KiB (K a multiple of 128); wave w loads blocks w*kpw .. w*kpw + kpw - 1
 * (kpw 1, 2, 4, 8 or 16; all issued before any is used; blocks past K/128
 * read the last block), lane l bytes 16 l .. 16 l + 15 of each.  Requires
 * waves * kpw >= K/128, tile_stride >= 8*K (the packed tile, 16 rows of K/2
 * bytes) and a multiple of 16, and the last tile inside buf_bytes.  A stride
 * above 8*K reads a row-tile-padded copy of the weights. */
int w4a16c_decode_loads(const void* wq, uint64_t buf_bytes, int64_t tiles, int64_t K,
                        int64_t tile_stride, int32_t kpw, int32_t waves, void* sink, void* stream);

/* `blocks` workgroups of 4 waves; each wave runs `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 on operands hashed from its thread
 * index and `seed` (4 * 32768 flops per wave and round). */
int w4a16c_mfma_loop(int32_t blocks, int32_t iters, uint32_t seed, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_CEILINGS_H */
