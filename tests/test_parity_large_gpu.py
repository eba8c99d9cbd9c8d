"""GPU parity at the largest packed weight the entry points take.

The decode and prefill kernels address the weights with 32-bit byte offsets
(the entry points reject N*K/2 >= 4 GiB).  Here N*K/2 = 4 GiB - 32 KiB
(K = 4096, N = 2^21 - 16, group 128, asymmetric, bf16): every tile past byte
2^31 and the last tile are reached, and sampled 16-row tiles are compared
with the oracle within the usual tolerance.  The codes and zero points are
drawn as uniform words in the stored layout (synth.stored_words); the oracle
unpacks each sampled tile on its own (a complete tile is self-contained, a
CPU pin in test_oracle_pins).
"""
import numpy as np
import pytest

import oracle as O
from synth import stored_words, to_act_bits, stream_seed
from gpu_util import assert_close, bits_to_device, device_to_bits, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import int4_weight_only_linear_amd as L  # noqa: E402  (fails loudly if the library is missing)

K, GS = 4096, 128
N = (1 << 21) - 16
WPR, G = K // 8, K // GS
TILE_BYTES = 16 * K // 2
BLOCK_ROWS = 1 << 16


def sampled_tiles():
    last = N // 16 - 1
    half = (1 << 31) // TILE_BYTES  # the first tile that starts at byte 2^31
    rng = np.random.default_rng(stream_seed("large-tiles"))
    extra = rng.choice(last + 1, size=6, replace=False)
    return sorted({0, 1, half - 1, half, half + 1, last - 1, last, *map(int, extra)})


@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
def test_weights_just_under_4gib():
    dev = torch.device("cuda:0")
    tiles = sampled_tiles()
    assert N * K // 2 == (1 << 32) - (1 << 15)
    note(f"[gpu] large: drawing and uploading {N * K // 2 / 2**30:.3f} GiB of packed weights")
    wq = torch.empty((N, WPR), dtype=torch.int32, device=dev)
    tile_words = {}
    for r0 in range(0, N, BLOCK_ROWS):
        rows = min(BLOCK_ROWS, N - r0)
        words = stored_words("large-w", r0, rows, WPR)
        wq[r0:r0 + rows].copy_(torch.from_numpy(words.view(np.int32)))
        for t in tiles:
            if r0 <= 16 * t < r0 + rows:
                tile_words[t] = words[16 * t - r0:16 * t - r0 + 16].copy()
        del words
    zpk = stored_words("large-z", 0, N // 8, G)
    rng = np.random.default_rng(stream_seed("large-s"))
    s_bits = to_act_bits(np.abs(rng.normal(0.0, 0.02, size=(N, G))).astype(np.float32) + 1e-3, O.BF16)
    s = bits_to_device(s_bits, O.BF16, dev)
    zp = torch.from_numpy(zpk.view(np.int32)).to(dev)
    torch.cuda.synchronize()
    for path, M in ((L.PATH_GEMV, 1), (L.PATH_GEMV, 5), (L.PATH_GEMM, 64)):
        note(f"[gpu] large: path={path} M={M}")
        x_bits = to_act_bits(np.random.default_rng(stream_seed("large-x", M)).normal(
            0.0, 1.0, size=(M, K)).astype(np.float32), O.BF16)
        x = bits_to_device(x_bits, O.BF16, dev)
        y = L.w4a16_linear_path(x, wq, s, zp, None, group_size=GS, path=path)
        torch.cuda.synchronize()
        yb = device_to_bits(y)
        for t in tiles:
            r = slice(16 * t, 16 * t + 16)
            ref = O.linear_ref(x_bits, tile_words[t].view(np.int32), s_bits[r], zpk[2 * t:2 * t + 2].view(np.int32),
                               None, M, 16, K, GS, O.BF16)
            assert_close(yb[:, r], ref, O.BF16, f"path={path} M={M} tile={t}")
        del x, y


@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
def test_expert_stack_past_4gib():
    # 68 experts of N 16384 x K 8192 (64 MiB packed each, 4.25 GiB in all):
    # expert 64 starts at byte 2^32 of the stack.  Slots routed to experts on
    # both sides of it; three 16-row tiles of each slot's output are compared
    # with the oracle.
    dev = torch.device("cuda:0")
    E, Ne, Ke, topk, M = 68, 16384, 8192, 4, 4
    wpr, Ge = Ke // 8, Ke // GS
    ids = np.array([[0, 63, 64, 67], [65, 1, 66, 62], [64, 67, 2, 33], [63, 65, 10, 50]], dtype=np.int32)
    tiles = (0, 257, Ne // 16 - 1)
    note(f"[gpu] large: drawing and uploading {E * Ne * Ke / 2 / 2**30:.2f} GiB of expert weights")
    wq = torch.empty((E, Ne, wpr), dtype=torch.int32, device=dev)
    tile_words = {}
    for e in range(E):
        words = stored_words("large-moe-w", e * Ne, Ne, wpr)
        wq[e].copy_(torch.from_numpy(words.view(np.int32)))
        if e in ids:
            for t in tiles:
                tile_words[e, t] = words[16 * t:16 * t + 16].copy()
        del words
    zpk = stored_words("large-moe-z", 0, E * Ne // 8, Ge).reshape(E, Ne // 8, Ge)
    rng = np.random.default_rng(stream_seed("large-moe-s"))
    s_bits = to_act_bits(np.abs(rng.normal(0.0, 0.02, size=(E, Ne, Ge))).astype(np.float32) + 1e-3, O.BF16)
    x_bits = to_act_bits(rng.normal(0.0, 1.0, size=(M, Ke)).astype(np.float32), O.BF16)
    tw = rng.random((M, topk)).astype(np.float32)
    y = L.w4a16_moe_linear(bits_to_device(x_bits, O.BF16, dev), wq, bits_to_device(s_bits, O.BF16, dev),
                           torch.from_numpy(ids).to(dev), torch.from_numpy(zpk.view(np.int32)).to(dev),
                           None, torch.from_numpy(tw).to(dev), group_size=GS)
    torch.cuda.synchronize()
    yb = device_to_bits(y)
    for m in range(M):
        for j in range(topk):
            e, slot = int(ids[m, j]), m * topk + j
            for t in tiles:
                r = slice(16 * t, 16 * t + 16)
                ref = O.linear_ref(x_bits[m:m + 1], tile_words[e, t].view(np.int32), s_bits[e, r],
                                   zpk[e, 2 * t:2 * t + 2].view(np.int32), None, 1, 16, Ke, GS, O.BF16)
                assert_close(yb[slot:slot + 1, r], ref * float(tw[m, j]), O.BF16,
                             f"slot {slot} expert {e} tile {t}")
