"""The C-ABI boundary on the host: the library loads, exports what the header
declares, packs exactly as the oracle does, and validates arguments without a
device.  No compute call reaches a GPU here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import int4_weight_only_linear_amd as L
from int4_weight_only_linear_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z_]+)\s*\(", text)))


def test_header_declares_the_bound_functions():
    assert _declared_functions() == sorted(B.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_abi_version():
    assert L.w4a16_abi_version() == L.ABI_VERSION == 4  # 4: w4a16_plan_info gained the tail fields
    m = re.search(r"#define W4A16_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == L.w4a16_abi_version()
    m = re.search(r"#define W4A16_GEMV_MAX_M (\d+)", open(HEADER).read())
    assert int(m.group(1)) == L.GEMV_MAX_M
    m = re.search(r"#define W4A16_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == L.NOALLOC_SCRATCH_BYTES


# ---- packing: the library's C++ against the oracle --------------------------

@pytest.mark.parametrize("N,K", [(1, 8), (8, 32), (37, 96), (256, 256), (64, 4096), (40, 160), (17, 416), (48, 352)])
def test_pack_weights_matches_oracle(N, K):
    q = np.random.default_rng(N * 7 + K).integers(0, 16, (N, K), dtype=np.uint8)
    wq = L.w4a16_pack_weights(q)
    assert np.array_equal(wq, O.pack_weights(q))
    assert np.array_equal(L.w4a16_unpack_weights(wq), q)
    assert np.array_equal(O.unpack_weights(wq), q)


def test_unpack_weights_all_words_matches_oracle():
    for shape in ((16, 64), (40, 52), (33, 12)):
        words = np.random.default_rng(3).integers(0, 2**32, shape, dtype=np.uint64)
        words = words.astype(np.uint32).view(np.int32)
        assert np.array_equal(L.w4a16_unpack_weights(words), O.unpack_weights(words))
        assert np.array_equal(L.w4a16_pack_weights(L.w4a16_unpack_weights(words)), words)


@pytest.mark.parametrize("N,G", [(8, 1), (16, 3), (4096, 32)])
def test_pack_zeros_matches_oracle(N, G):
    z = np.random.default_rng(N + G).integers(0, 16, (N, G), dtype=np.uint8)
    zpk = L.w4a16_pack_zeros(z)
    assert np.array_equal(zpk, O.pack_zeros(z))
    assert np.array_equal(L.w4a16_unpack_zeros(zpk), z)


def test_pack_worked_words():
    assert L.w4a16_pack_weights(np.arange(8, dtype=np.uint8)[None]).view(np.uint32)[0, 0] == 0x75316420
    assert L.w4a16_pack_zeros(np.arange(8, dtype=np.uint8)[:, None]).view(np.uint32)[0, 0] == 0x76543210


def test_pack_errors():
    with pytest.raises(L.W4A16Error, match="exceeds 15"):
        L.w4a16_pack_weights(np.full((1, 8), 16, dtype=np.uint8))
    with pytest.raises(L.W4A16Error, match="K % 8"):
        B._check(B.lib.w4a16_pack_weights(np.zeros(12, np.uint8).ctypes.data, 1, 12,
                                          np.zeros(2, np.int32).ctypes.data))
    with pytest.raises(L.W4A16Error, match="N % 8"):
        B._check(B.lib.w4a16_pack_zeros(np.zeros(12, np.uint8).ctypes.data, 12, 1,
                                        np.zeros(2, np.int32).ctypes.data))
    with pytest.raises(L.W4A16Error, match="NULL"):
        B._check(B.lib.w4a16_pack_weights(None, 1, 8, None))


# ---- argument validation (host only: fake, never dereferenced pointers) -----

P = 1 << 20  # a 256-byte aligned fake address; check_args never dereferences


def _args(**kw):
    a = dict(x=P, wq=2 * P, s=3 * P, zp=None, bias=None, y=4 * P, M=1, N=64, K=256, g=128, dt=1)
    a.update(kw)
    return a


def _check(**kw):
    a = _args(**kw)
    return B.lib.w4a16_check_args(a["x"], a["wq"], a["s"], a["zp"], a["bias"], a["y"], a["M"],
                                  a["N"], a["K"], a["g"], a["dt"])


def test_check_args_accepts_valid():
    assert _check() == 0
    assert _check(zp=5 * P, bias=6 * P, dt=0, g=32, K=96, M=5) == 0
    assert L.w4a16_last_error() == ""


@pytest.mark.parametrize("kw,status,msg", [
    (dict(g=16), 2, "group size"),
    (dict(g=256, K=512), 2, "group size"),     # neither the accept set nor K
    (dict(K=200), 1, "multiple of the group"),
    (dict(K=(1 << 24) + 128), 2, "K above"),
    (dict(K=1 << 25, g=1 << 25), 2, "K above"),  # per-channel
    (dict(K=64, g=128), 1, "multiple of the group"),
    (dict(N=0), 1, "N must be"),
    (dict(M=-1), 1, "M must be"),
    (dict(dt=2), 1, "dtype"),
    (dict(zp=5 * P, N=60), 1, "N % 8"),
    (dict(x=None), 1, "NULL"),
    (dict(y=None), 1, "NULL"),
    (dict(x=P + 8), 3, "x must be 16-byte"),
    (dict(wq=2 * P + 4), 3, "wq must be 16-byte"),
    (dict(s=3 * P + 1), 3, "2-byte"),
    (dict(zp=5 * P + 2), 3, "zp must be 4-byte"),
    (dict(y=P + 64), 1, "overlap"),            # y inside x
    (dict(y=2 * P, x=P), 1, "overlap"),        # y on top of wq
])
def test_check_args_rejects(kw, status, msg):
    assert _check(**kw) == status
    assert msg in L.w4a16_last_error()


def test_m_zero_is_accepted_without_pointers():
    assert _check(M=0, x=None, wq=None, s=None, y=None) == 0


def test_linear_rejects_before_touching_a_device():
    # invalid arguments are reported by validation, before any HIP call
    st = B.lib.w4a16_linear(P, 2 * P, 3 * P, None, None, 4 * P, 1, 64, 256, 48, 1, None, 0, None)
    assert st == 2 and "group size" in L.w4a16_last_error()
    st = B.lib.w4a16_linear_path(P, 2 * P, 3 * P, None, None, 4 * P, 1, 64, 256, 128, 1, None, 0,
                                 None, 7)
    assert st == 1 and "unknown path" in L.w4a16_last_error()


def test_zero_point_dtype_message_is_the_pages():
    torch = pytest.importorskip("torch")
    golden = [l for l in open(os.path.join(GOLDEN, "zp_dtype_error.txt")) if not l.startswith("#")]
    want = golden[0].strip()
    x = torch.zeros(1, 256, dtype=torch.float16)
    wq = torch.zeros(64, 32, dtype=torch.int32)
    s = torch.zeros(64, 2, dtype=torch.float16)
    zp = torch.zeros(64, 2, dtype=torch.float16)     # the unpacked contract the pages reject
    with pytest.raises(RuntimeError) as e:
        L.w4a16_linear(x, wq, s, zp, group_size=128)
    assert str(e.value).startswith(want)
    assert "torch.float16" in str(e.value)


# ---- path selection and workspace sizing (host logic) -----------------------

def test_select_path_by_m():
    sel = lambda M, N, K, g=128: L.w4a16_select_path(M, N, K, g, 1, 1)
    # the decode kernel up to M = 8 everywhere
    for (N, K) in ((4096, 4096), (6144, 4096), (14336, 4096), (4096, 14336), (2560, 9728), (4096, 28672)):
        for M in (1, 5, 8):
            assert sel(M, N, K) == L.PATH_GEMV, (M, N, K)
    # K <= 4096: up to M = 16 below 20 M weights, 9 above, 8 on N >= 14336 (any group)
    for (N, K) in ((4096, 4096), (2560, 4096), (6144, 2560)):
        for M in (9, 16):
            assert sel(M, N, K) == L.PATH_GEMV, (M, N, K)
        assert sel(17, N, K) == L.PATH_GEMM
    assert sel(9, 6144, 4096) == L.PATH_GEMV and sel(10, 6144, 4096) == L.PATH_GEMM
    for g in (32, 64, 128):
        assert sel(8, 14336, 4096, g) == L.PATH_GEMV
        for M in (9, 16):
            assert sel(M, 14336, 4096, g) == L.PATH_GEMM
    # 4096 < K <= 16384: up to M = 12 below 32 M weights, 8 above; longer K: 8
    for M in (9, 12):
        assert sel(M, 2560, 9728) == L.PATH_GEMV
    for M in (13, 16):
        assert sel(M, 2560, 9728) == L.PATH_GEMM
    for M in (9, 12, 16, 1920):
        assert sel(M, 4096, 14336) == L.PATH_GEMM
        assert sel(M, 4096, 28672) == L.PATH_GEMM
    # K > 16384 from 160 Mi weights with groups of 64 or more: up to M = 6
    for g in (64, 128):
        assert sel(6, 8192, 28672, g) == L.PATH_GEMV and sel(7, 8192, 28672, g) == L.PATH_GEMM
    assert sel(8, 8192, 28672, 32) == L.PATH_GEMV and sel(9, 8192, 28672, 32) == L.PATH_GEMM
    assert sel(8, 5120, 20480) == L.PATH_GEMV  # 100 Mi weights
    for M in (17, 32, 65, 128, 1920):
        assert sel(M, 4096, 4096) == L.PATH_GEMM


def test_select_path_env_override(tuning_env):
    tuning_env("W4A16_FORCE_PATH", "gemm")
    assert L.w4a16_select_path(1, 4096, 4096, 128, 1, 1) == L.PATH_GEMM
    tuning_env("W4A16_FORCE_PATH", "gemv")
    assert L.w4a16_select_path(128, 4096, 4096, 128, 1, 1) == L.PATH_GEMV


def test_workspace_size():
    # enough row tiles for every CU: no split, no workspace
    assert L.w4a16_workspace_size(1, 28672, 4096, 128, 1, 1) == 0
    # 160 row tiles: not split (a split costs more than the idle CUs)
    assert L.w4a16_workspace_size(1, 2560, 4096, 128, 0, 0) == 0
    # 3 row tiles: not split either (the hand-off costs more than idle CUs)
    assert L.w4a16_workspace_size(1, 40, 4096, 128, 1, 1) == 0
    # more k-steps than 16 waves of 8 take (K = 20480: 160 steps): K is split
    assert L.w4a16_workspace_size(1, 40, 20480, 128, 1, 1) > 0
    # two to four tokens take 8 steps a wave where 4 would need more than 16
    # waves (76 steps), so K stays whole
    assert L.w4a16_workspace_size(4, 2560, 9728, 128, 0, 0) == 0
    # more k-steps than one workgroup's waves take (M = 5: 4 steps a wave, 76
    # steps): K is split and the workspace holds counters + partials
    ws = L.w4a16_workspace_size(5, 2560, 9728, 128, 0, 0)
    assert ws > 0
    tiles = 2560 // 16
    assert ws >= 256 * ((tiles * 4 + 255) // 256) + 2 * 5 * 2560 * 4
    assert L.w4a16_workspace_size(0, 2560, 9728, 128, 0, 0) == 0
    # the prefill GEMM: enough tiles to fill the CUs, no split
    assert L.w4a16_workspace_size(1920, 28672, 4096, 128, 1, 1, L.PATH_GEMM) == 0
    # a single 128-token tile row: K is split; counters region + fp32 partial tiles
    ws = L.w4a16_workspace_size(128, 4096, 4096, 128, 1, 1, L.PATH_GEMM)
    assert ws >= 64 * 1024 + 2 * 128 * 4096 * 4


def test_dense_workspace_size_and_argument_checks():
    # the dense instances of the prefill GEMM plan like the symmetric group-128
    # GEMM: the same tile and split choices, so the same split workspace
    for (M, N, K) in ((1920, 4096, 4096), (128, 4096, 4096), (130, 200, 640), (1, 64, 256)):
        for dt in (L.W4A16_F16, L.W4A16_BF16):
            want = L.w4a16_workspace_size(M, N, K, 128, dt, False, L.PATH_GEMM)
            assert L.w4a16_dense_workspace_size(M, N, K, dt, 1) == want
            assert L.w4a16_dense_workspace_size(M, N, K, dt, 0) == want
    assert L.w4a16_dense_workspace_size(1920, 4096, 4096, L.W4A16_BF16, 0) == 0   # no split
    assert L.w4a16_dense_workspace_size(128, 4096, 4096, L.W4A16_BF16, 0) > 64 * 1024
    assert L.w4a16_dense_workspace_size(0, 4096, 4096, L.W4A16_BF16, 1) == 0
    # rejected before any device is touched
    st = B.lib.w4a16_linear_dense(None, None, None, None, 4, 8, 64, 7, None, 0, None)
    assert st == 1 and "dtype" in L.w4a16_last_error()
    st = B.lib.w4a16_linear_dense(None, None, None, None, 4, 8, 48, L.W4A16_BF16, None, 0, None)
    assert st == 1 and "multiple of 32" in L.w4a16_last_error()
    st = B.lib.w4a16_linear_dense(None, None, None, None, 4, 8, 64, L.W4A16_BF16, None, 0, None)
    assert st == 1 and "NULL" in L.w4a16_last_error()
    st = B.lib.w4a16_linear_dense(P + 8, 2 * P, None, 4 * P, 4, 8, 64, L.W4A16_BF16, None, 0, None)
    assert st == 3 and "16-byte" in L.w4a16_last_error()
    st = B.lib.w4a16_linear_dense(P, 2 * P, None, 4 * P, 4, 1 << 20, 4096, L.W4A16_BF16, None, 0, None)
    assert st == 2 and "4 GiB" in L.w4a16_last_error()
    assert B.lib.w4a16_linear_dense(None, None, None, None, 0, 8, 64, L.W4A16_BF16, None, 0, None) == 0


def test_per_channel_group_accept_set():
    ok = lambda M, N, K, g, zp=0: B.lib.w4a16_check_args(
        1024, 1024, 1024, 1024 if zp else None, None, 1 << 30, M, N, K, g, L.W4A16_BF16)
    assert ok(1, 64, 4096, 4096, 1) == 0      # per-channel, K a multiple of 128
    assert ok(1, 64, 320, 320) == 0            # per-channel, K a multiple of 64
    assert ok(1, 64, 96, 96) == 0              # per-channel, K a multiple of 32
    assert ok(1, 64, 40, 40) == 2              # K not a multiple of 32
    assert ok(1, 64, 512, 256) == 2            # neither the accept set nor K
    assert "per-channel" in L.w4a16_last_error()
    assert L.w4a16_workspace_size(1, 64, 4096, 4096, L.W4A16_BF16, True) >= 0


def test_gemm_planner_skips_exactly_the_spilling_tiles():
    # The planner leaves out the 192- and 256-token x 256-feature tiles for
    # fp16 with groups of 32 (either quantisation) or asymmetric groups of 64,
    # and bf16 with symmetric groups of 32 (wide_tall_tile_spills in
    # w4a16_gemm.hip): those must be exactly the GEMM instances the compiler
    # spills registers for, read from the build's resource-usage record.
    import json
    path = os.path.join(ROOT, "_build", "w4a16_gemm.hip.o.resources.json")
    if not os.path.exists(path):
        pytest.skip("no build record here")
    with open(path) as f:
        res = json.load(f)
    spilling = set()
    for name, r in res.items():
        m = re.search(r"gemm_kernelILi(\d)ELi(\d+)ELb(\d)ELi(\d)ELi(\d)E", name)
        if m and r.get("VGPRs Spill", 0) > 16:
            spilling.add(tuple(int(v) for v in m.groups()))
    excluded = {(0, 32, 0), (0, 32, 1), (0, 64, 1), (1, 32, 0)}  # (dtype, group, asym)
    assert spilling == {(dt, g, a, mb, 2) for (dt, g, a) in excluded for mb in (6, 8)}


def test_gemm_tail_launch_plans():
    # Where K is not split and the 256-token tiles end in a partial round of
    # workgroups, the planner may run the tiles past the last full round as a
    # second launch of 128-token tiles (two per tile): the ones with output to
    # compute fit in one round, and no workspace is needed.
    cus = 256  # the planning CU count without a device, and MI355X's
    seen = set()
    for (K, N) in ((4096, 6144), (4096, 28672), (14336, 4096), (2560, 19456), (1024, 16512), (2048, 8264),
                   (1024, 28672), (1024, 8264)):
        for M in (128, 200, 520, 777, 1000, 1300, 1920, 2100, 4096):
            for dt, g, asym in ((O.BF16, 128, True), (O.F16, 32, True), (O.BF16, 64, False)):
                p = L.w4a16_plan(M, N, K, g, dt, asym, L.PATH_GEMM)
                if not p["tail_tiles"]:
                    assert p["tail_tile_tokens"] == 0 and p["tail_tile_features"] == 0, p
                    continue
                tt, tf = p["tail_tile_tokens"], p["tail_tile_features"]
                sm, sn = 2, 1
                assert (p["tile_tokens"], tt, tf) == (256, 128, p["tile_features"]), p
                assert p["splits"] == 1 and not p["two_pass"] and p["launches"] == 2 and p["workspace_bytes"] == 0, p
                full = p["tiles"] // cus * cus
                assert p["tiles"] % cus and full >= cus, p
                assert p["tail_tiles"] == (p["tiles"] - full) * sm * sn, p
                tn = -(-N // p["tile_features"])
                busy = sum(1 for w in range(full, p["tiles"]) for a in range(sm) for b in range(sn)
                           if ((w // tn) * sm + a) * tt < M and ((w % tn) * sn + b) * tf < N)
                assert 0 < busy <= cus, (M, N, K, p)
                seen.add(tf)
    assert seen == {128, 256}, seen
    # the Llama-3.1-8B up-projection shape at M = 1920: 896 tiles of 256 x 256,
    # the last 128 as 128 x 256 tiles (the half past M exits at once)
    p = L.w4a16_plan(1920, 28672, 4096, 128, O.BF16, True, L.PATH_GEMM)
    assert (p["tile_tokens"], p["tile_features"], p["tiles"]) == (256, 256, 896), p
    assert (p["tail_tile_tokens"], p["tail_tile_features"], p["tail_tiles"]) == (128, 256, 256), p


# ---- launch plans: the completion counters of one launch fit their region -----

KMAXC = 64 * 1024 // 4  # completion counters in the workspace's counter region


@pytest.mark.parametrize("path", [L.PATH_GEMV, L.PATH_GEMM])
def test_every_plan_keeps_its_counters_in_the_counter_region(path):
    # every launch's tiles that keep a completion counter must fit the 64 KiB
    # region; decode layers with more row tiles than that and a K split run
    # as several launches, each covering at most KMAXC row tiles
    Ms = (1, 2, 3, 4, 5, 8, 16) if path == L.PATH_GEMV else (17, 64, 128, 1920)
    Ns = (16, 4096, 262144, 262160, 280000, (1 << 21) - 16)
    Ks = (128, 4096, 8320, 9728, 28672, 1 << 20, 1 << 24)
    seen_chunked = False
    for M in Ms:
        for N in Ns:
            for K in Ks:
                for g in (32, 128):
                    p = L.w4a16_plan(M, N, K, g, L.W4A16_BF16, True, path)
                    assert p["path"] == path
                    assert p["counter_tiles"] <= KMAXC, (M, N, K, g, p)
                    if p["splits"] > 1 and not p["two_pass"]:
                        per_launch = -(-p["tiles"] // p["launches"]) if path == L.PATH_GEMV else p["tiles"]
                        assert per_launch <= KMAXC, (M, N, K, g, p)
                        assert p["workspace_bytes"] >= 64 * 1024
                    if path == L.PATH_GEMV and p["splits"] > 1:
                        assert p["launches"] == -(-p["tiles"] // KMAXC)
                        seen_chunked |= p["launches"] > 1
                    assert p["workspace_bytes"] == L.w4a16_workspace_size(M, N, K, g, L.W4A16_BF16, True, path)
    assert seen_chunked or path == L.PATH_GEMM


@pytest.mark.parametrize("M,N,K", [(1, 280000, 28672), (5, 270000, 9728), (5, 262160, 8320)])
def test_split_decode_beyond_the_counter_region_is_chunked(M, N, K):
    # shapes whose forced K split has more row tiles than there are counters
    p = L.w4a16_plan(M, N, K, 128, L.W4A16_BF16, True, L.PATH_GEMV)
    tiles = -(-N // 16)
    assert p["tiles"] == tiles > KMAXC and p["splits"] >= 2
    assert p["launches"] == -(-tiles // KMAXC) >= 2 and p["counter_tiles"] == KMAXC
    assert p["workspace_bytes"] == 64 * 1024 + p["splits"] * M * N * 4


def test_plan_reports_the_few_token_instance():
    # up to eight tokens with K a whole number of 128-k steps in runs of 8 or 4
    # (at most 16 waves, the last run shorter by whole parts), at most 4
    # groups finished by a 16-lane row, at most 32 group sums per result
    # register and the staged x within the LDS budget take the few-token
    # instance; it never splits K
    for dt in (L.W4A16_F16, L.W4A16_BF16):
        for (M, K, g, waves) in ((1, 4096, 128, 4), (1, 4096, 32, 8), (1, 14336, 128, 14), (1, 2560, 64, 5),
                                 (1, 512, 32, 1), (2, 4096, 128, 4), (2, 4096, 64, 4), (2, 4096, 32, 8),
                                 (3, 4096, 128, 8), (4, 4096, 128, 8), (4, 4096, 64, 8), (4, 14336, 128, 14),
                                 # a last run shorter by whole parts
                                 (1, 9728, 128, 10), (1, 1280, 128, 2), (2, 2176, 128, 5), (4, 3456, 128, 7),
                                 # eight token rows (five to eight tokens)
                                 (5, 14336, 128, 14), (5, 9728, 128, 10), (6, 9728, 128, 10), (7, 9728, 128, 10),
                                 (5, 4096, 128, 8), (8, 4096, 128, 8), (8, 512, 128, 1), (7, 2560, 128, 5)):
            p = L.w4a16_plan(M, 4096, K, g, dt, True, L.PATH_GEMV)
            assert (p["kernel"], p["waves"], p["splits"], p["launches"]) == (1, waves, 1, 1), (M, K, g, p)
        # more than 16 runs: K ranges of at most 16 runs, partial sums through
        # the workspace (counters for every row tile), only where the general
        # kernel splits K too (no new workspace need); one and two token rows
        # in no more K ranges than it, four and eight token rows with at most
        # two rounds of one workgroup per CU (four rows try runs of 8 first)
        for (M, N, K, g, waves, splits) in ((1, 4096, 28672, 128, 14, 2), (2, 4096, 28672, 128, 14, 2),
                                            (1, 4096, 1 << 16, 128, 16, 4), (4, 1024, 1 << 16, 128, 16, 4),
                                            (3, 1280, 20480, 64, 14, 3), (4, 1280, 20480, 64, 14, 3),
                                            (3, 4096, 28672, 128, 14, 2), (4, 4096, 28672, 128, 14, 2),
                                            (4, 4096, 14336, 64, 14, 2), (6, 4096, 14336, 128, 14, 2),
                                            (8, 4096, 14336, 128, 14, 2), (5, 4096, 14336, 64, 14, 2)):
            p = L.w4a16_plan(M, N, K, g, dt, True, L.PATH_GEMV)
            assert (p["kernel"], p["waves"], p["splits"], p["launches"], p["counter_tiles"]) == \
                (1, waves, splits, 1, N // 16), (M, N, K, g, p)
            assert p["workspace_bytes"] >= 64 * 1024 + splits * M * N * 4
        for (M, K, g) in ((9, 4096, 128), (16, 4096, 128), (1, 4160, 64), (1, 14336, 32), (3, 14336, 64),
                          (4, 4096, 32), (8, 4096, 32),
                          # more K ranges than the general kernel's
                          (1, 28672, 32), (2, 28672, 32)):
            assert L.w4a16_plan(M, 4096, K, g, dt, True, L.PATH_GEMV)["kernel"] == 0, (M, K, g)
        # four token rows in more than two rounds of workgroups
        for (M, N, K) in ((3, 8192, 28672), (4, 8192, 28672), (3, 5120, 20480), (4, 5120, 20480)):
            assert L.w4a16_plan(M, N, K, 128, dt, True, L.PATH_GEMV)["kernel"] == 0, (M, N, K)
        # per-channel scales stay on the general kernel
        assert L.w4a16_plan(1, 4096, 4096, 4096, dt, False, L.PATH_GEMV)["kernel"] == 0
        # the prefill GEMM reports 0
        assert L.w4a16_plan(64, 4096, 4096, 128, dt, True, L.PATH_GEMM)["kernel"] == 0


def test_few_token_split_needs_no_workspace_the_general_kernel_would_not(tuning_env):
    # the few-token instance splits K only where the general kernel splits it
    # too, so a caller's workspace need (zero or not) is the same with the
    # instance on or off; its launches stay within 16 waves and the counter
    # region
    shapes = [(M, N, K, g) for M in (1, 2, 3, 4, 5, 8) for N in (16, 136, 1024, 4096, 28672)
              for K in (128, 1152, 4096, 9728, 14336, 20480, 28672, 1 << 16) for g in (32, 64, 128)]
    for dt in (L.W4A16_F16, L.W4A16_BF16):
        on = [L.w4a16_plan(M, N, K, g, dt, True, L.PATH_GEMV) for (M, N, K, g) in shapes]
        tuning_env("W4A16_GEMV_NO_ONE", "1")
        off = [L.w4a16_plan(M, N, K, g, dt, True, L.PATH_GEMV) for (M, N, K, g) in shapes]
        tuning_env("W4A16_GEMV_NO_ONE", None)
        split_seen = False
        for shape, a, b in zip(shapes, on, off):
            assert (a["workspace_bytes"] > 0) == (b["workspace_bytes"] > 0), (shape, a, b)
            if a["kernel"] == 1:
                assert 1 <= a["waves"] <= 16 and a["launches"] == 1, (shape, a)
                if a["splits"] > 1:
                    split_seen = True
                    assert b["splits"] > 1 and a["counter_tiles"] == a["tiles"] <= KMAXC, (shape, a, b)
                    M, N = shape[0], shape[1]
                    assert a["workspace_bytes"] >= 64 * 1024 + a["splits"] * M * N * 4, (shape, a)
            else:
                assert a == b, (shape, a, b)
        assert split_seen


def test_plan_errors():
    with pytest.raises(L.W4A16Error, match="M <= 16"):
        L.w4a16_plan(17, 64, 256, 128, 1, False, L.PATH_GEMV)
    with pytest.raises(L.W4A16Error, match="group size"):
        L.w4a16_plan(1, 64, 256, 48, 1, False)
    with pytest.raises(L.W4A16Error, match="unknown path"):
        L.w4a16_plan(1, 64, 256, 128, 1, False, 9)


# ---- the pages' accept set, as stored in tests/golden/accept_set.json --------

def test_accept_set_golden_drives_validation():
    import json
    g = json.load(open(os.path.join(GOLDEN, "accept_set.json")))
    dts = {"float16": L.W4A16_F16, "bfloat16": L.W4A16_BF16}
    for dt_name in g["act_dtypes"]:
        for gs in g["group_sizes"]:
            for wt in g["weight_types"]:
                zp = 5 * P if wt == "uint4" else None   # uint4b8: no zero points
                assert _check(dt=dts[dt_name], g=gs, K=4 * gs, zp=zp) == 0, (dt_name, gs, wt)
                # K must be a multiple of the group (the K divisibility rule)
                assert _check(dt=dts[dt_name], g=gs, K=4 * gs + 8, zp=zp) != 0
    # group sizes outside the set (and not per-channel) are refused
    for gs in (16, 48, 96, 256):
        if gs not in g["group_sizes"]:
            assert _check(g=gs, K=4 * 256) == 2
    # a dtype code outside the two act dtypes is refused
    assert _check(dt=len(g["act_dtypes"])) == 1
    # uint4b8 means the stored code carries a bias of 8: symmetric == zero point 8
    assert O.SYMMETRIC_ZERO == g["symmetric_zero_point"]
    # the pages route M <= 5 to their skinny decode kernel; the measured MI355X
    # bound keeps every such M on the decode kernel
    for M in range(1, g["decode_m_threshold_on_pages"] + 1):
        for K in (2560, 4096, 14336, 28672):
            assert L.w4a16_select_path(M, 4096, K, 128, L.W4A16_BF16, True) == L.PATH_GEMV


# ---- the benchmark's ceiling kernels: library, header and host checks ---------

def test_ceilings_library_exports_its_header_and_checks_arguments():
    from int4_weight_only_linear_amd import ceilings as C
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "w4a16_ceilings.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(w4a16c_[a-z_]+)\s*\(", text)))
    assert declared == sorted(C.SIGNATURES)
    lib = ctypes.CDLL(C.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    # refused on the host, before any launch (hipErrorInvalidValue = 1)
    assert C.lib.w4a16c_stream_read(None, 64, P, None) == 1
    assert C.lib.w4a16c_stream_read(P + 8, 64, P, None) == 1
    K = 4096
    assert C.lib.w4a16c_decode_loads(P, 16 * 8 * K, 17, K, 8 * K, 8, 4, P, None) == 1      # tiles past the buffer
    assert C.lib.w4a16c_decode_loads(P, 16 * 8 * K, 16, K, 8 * K - 16, 8, 4, P, None) == 1  # stride below a tile
    assert C.lib.w4a16c_decode_loads(P, 16 * 8 * K, 16, K, 8 * K, 4, 4, P, None) == 1      # waves * kpw < K/128
    assert C.lib.w4a16c_decode_loads(P, 16 * 8 * K, 16, K, 8 * K, 8, 17, P, None) == 1     # more than 16 waves
    assert C.lib.w4a16c_mfma_loop(0, 10, 1, P, None) == 1


def test_gemm_plans_hold_their_invariants_on_random_shapes():
    # Any GEMM plan: its tiles cover M x N exactly once; K ranges of whole
    # 128-k steps with none empty; a tail launch only for unsplit 256-token
    # tiles past whole rounds, in one round of 128-token tiles; the workspace
    # is the counter region plus the plan's fp32 partials, nothing without a
    # split; and the counters of a one-pass split fit their region.
    hyp = pytest.importorskip("hypothesis")
    st = pytest.importorskip("hypothesis.strategies")
    kinds = set()

    @hyp.settings(max_examples=400, deadline=None, derandomize=True)
    @hyp.given(M=st.integers(9, 8192), N=st.integers(1, 40000).map(lambda n: 8 * n),
               ksteps=st.integers(1, 160), g=st.sampled_from([32, 64, 128]), dt=st.sampled_from([O.F16, O.BF16]),
               zp=st.booleans())
    def check(M, N, ksteps, g, dt, zp):
        K = 128 * ksteps
        p = L.w4a16_plan(M, N, K, g, dt, zp, L.PATH_GEMM)
        bm, bn = p["tile_tokens"], p["tile_features"]
        assert bm in (32, 128, 192, 256) and bn in (128, 256), p
        assert p["tiles"] == -(-M // bm) * -(-N // bn), p
        s = p["splits"]
        assert 1 <= s <= ksteps, p
        sps = -(-ksteps // s)
        assert -(-ksteps // sps) == s, p  # every K range holds steps
        if p["tail_tiles"]:
            full = p["tiles"] // 256 * 256
            assert bm == 256 and s == 1 and not p["two_pass"] and p["launches"] == 2, p
            assert (p["tail_tile_tokens"], p["tail_tile_features"]) == (128, bn), p
            assert full >= 256 and p["tiles"] > full and p["tail_tiles"] == 2 * (p["tiles"] - full), p
        ws = p["workspace_bytes"]
        if s == 1:
            assert ws == 0 and p["launches"] == (2 if p["tail_tiles"] else 1), p
        elif p["two_pass"]:
            assert ws == KMAXC * 4 + s * M * (-(-N // 8) * 8) * 4 and p["launches"] == 2, p
        else:
            assert p["tiles"] <= KMAXC and p["counter_tiles"] == p["tiles"], p
            assert ws == KMAXC * 4 + p["tiles"] * s * bm * bn * 4, p
        assert ws == L.w4a16_workspace_size(M, N, K, g, dt, zp, L.PATH_GEMM)
        kinds.add("tail" if p["tail_tiles"] else "unsplit" if s == 1 else "two-pass" if p["two_pass"] else "one-pass")

    check()
    assert kinds == {"tail", "unsplit", "two-pass", "one-pass"}, kinds


def test_decode_plans_hold_their_invariants_on_random_shapes():
    # Any decode plan (M <= 16): one workgroup per 16-row tile per K range; at
    # most 16 waves; the few-token instance only for M <= 8 with K a whole
    # number of 128-k steps, its K ranges covering K with none empty; split
    # tiles keep their counters in the region (several launches beyond it);
    # a workspace exactly when some K is split, sized for the larger split.
    hyp = pytest.importorskip("hypothesis")
    st = pytest.importorskip("hypothesis.strategies")
    kinds = set()

    @hyp.settings(max_examples=400, deadline=None, derandomize=True)
    @hyp.given(M=st.integers(1, 16), N=st.integers(1, 20000).map(lambda n: 8 * n),
               kg=st.integers(1, 400), g=st.sampled_from([32, 64, 128]), dt=st.sampled_from([O.F16, O.BF16]),
               zp=st.booleans())
    def check(M, N, kg, g, dt, zp):
        K = g * kg
        p = L.w4a16_plan(M, N, K, g, dt, zp, L.PATH_GEMV)
        assert p["path"] == L.PATH_GEMV and p["tiles"] == -(-N // 16), p
        assert 1 <= p["waves"] <= 16 and p["splits"] >= 1, p
        ksteps = -(-K // 128)
        s, w = p["splits"], p["waves"]
        if p["kernel"] == 1:
            assert M <= 8 and K % 128 == 0 and p["launches"] == 1, p
            # K ranges of w runs of 4 or 8 k-steps cover K, the last range not empty
            assert any((s - 1) * w * kpw < ksteps <= s * w * kpw for kpw in (4, 8)), p
            assert s == 1 or p["tiles"] <= KMAXC, p
        else:
            # K ranges of ceil(ksteps / s) steps, each in w runs of 1-8 steps
            kps = -(-ksteps // s)
            assert s <= ksteps and -(-ksteps // kps) == s, p
            assert any(-(-kps // kpw) == w for kpw in (1, 2, 4, 8)), p
            if s > 1:
                assert p["launches"] == -(-p["tiles"] // KMAXC), p
        assert p["counter_tiles"] <= KMAXC, p
        ws = p["workspace_bytes"]
        if ws == 0:
            assert s == 1 and p["counter_tiles"] == 0, p
        if s > 1:
            assert ws >= KMAXC * 4 + s * M * N * 4, p
        assert ws == L.w4a16_workspace_size(M, N, K, g, dt, zp, L.PATH_GEMV)
        kinds.add((p["kernel"], p["splits"] > 1))

    check()
    assert kinds == {(0, False), (0, True), (1, False), (1, True)}, kinds
