"""GPU parity: libw4a16 (through its C ABI) against the CPU oracle.

Integer work (device unpacking) and the dequantised weights are compared bit
for bit; linear outputs within the stated tolerance (max|y - y_ref| <=
5e-3 * max|y_ref| for bf16, 2e-3 for fp16), plus bit-exact properties
(one-hot activations, all-eight weights, symmetric == asymmetric with zero
point 8, power-of-two scaling, run-to-run determinism).
"""
import numpy as np
import pytest

import oracle as O
from synth import make_case, stream_seed, stored_words, to_act_bits, CONFIGS
from gpu_util import DeviceCase, assert_close, bits_to_device, device_to_bits, note, oracle_rows, sample_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import int4_weight_only_linear_amd as L  # noqa: E402  (fails loudly if the library is missing)

GEMV, GEMM, AUTO = L.PATH_GEMV, L.PATH_GEMM, L.PATH_AUTO


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    note(f"[gpu] {request.node.nodeid}")


def paths_for(M):
    return (GEMV, GEMM) if M <= L.GEMV_MAX_M else (GEMM,)


# ---- integer and dequantisation work: bit exact -----------------------------

@pytest.mark.parametrize("N,K", [(8, 32), (37, 96), (256, 256), (4096, 14336)])
def test_unpack_device_bit_exact(N, K):
    q = np.random.default_rng(N + K).integers(0, 16, (N, K), dtype=np.uint8)
    wq = torch.from_numpy(L.w4a16_pack_weights(q)).cuda()
    got = L.w4a16_unpack_device(wq).cpu().numpy()
    assert np.array_equal(got, O.unpack_weights(O.pack_weights(q)))
    assert np.array_equal(got, q)


@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("N,K", [(8, 128), (40, 384), (264, 1152)])
def test_dequant_bit_exact(dt, sym, g, N, K):
    c = make_case(1, N, K, g, dt, sym, False, seed=("dq", N, K, g, dt, sym))
    d = DeviceCase(c)
    w = device_to_bits(L.w4a16_dequant(d.wq, d.s, d.zp, group_size=g))
    zpk = None if sym else O.pack_zeros(c.zp)
    ref = O.dequant_act(O.pack_weights(c.q), c.s_bits, zpk, N, K, g, dt)
    assert np.array_equal(w, ref)


@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("N,K,g", [(24, 224, 32), (56, 320, 64), (48, 96, 32), (16, 1184, 32)])
def test_dequant_bit_exact_incomplete_runs(dt, N, K, g):
    c = make_case(1, N, K, g, dt, False, False, seed=("dqtail", N, K, g, dt))
    d = DeviceCase(c)
    w = device_to_bits(L.w4a16_dequant(d.wq, d.s, d.zp, group_size=g))
    ref = O.dequant_act(O.pack_weights(c.q), c.s_bits, O.pack_zeros(c.zp), N, K, g, dt)
    assert np.array_equal(w, ref)


@pytest.mark.parametrize("name,dt,sym", [("llama", O.BF16, False), ("qwen", O.F16, True)])
def test_dequant_bit_exact_full_layer(name, dt, sym):
    K, N = (4096, 4096) if name == "llama" else (2560, 6144)
    c = make_case(1, N, K, 128, dt, sym, False, seed=("dqfull", name))
    d = DeviceCase(c)
    w = device_to_bits(L.w4a16_dequant(d.wq, d.s, d.zp, group_size=128))
    zpk = None if sym else O.pack_zeros(c.zp)
    assert np.array_equal(w, O.dequant_act(O.pack_weights(c.q), c.s_bits, zpk, N, K, 128, dt))


def test_dequant_scale_extremes_bit_exact():
    # scales spanning the formats' range, including fp16 subnormal products
    for dt in (O.F16, O.BF16):
        c = make_case(1, 16, 128, 32, dt, False, False, seed=("dqx", dt))
        rng = np.random.default_rng(11)
        s = (2.0 ** rng.uniform(-14 if dt == O.F16 else -60, 10, c.s_bits.shape)).astype(np.float32)
        c.s_bits = O.f32_to_act_bits(s, dt)
        d = DeviceCase(c)
        w = device_to_bits(L.w4a16_dequant(d.wq, d.s, d.zp, group_size=32))
        assert np.array_equal(w, O.dequant_act(O.pack_weights(c.q), c.s_bits, O.pack_zeros(c.zp),
                                               16, 128, 32, dt))


# ---- linear: tolerance parity on grids that span tiles and ragged tails ------

@pytest.mark.parametrize("path", [GEMV, GEMM, AUTO])
def test_tiny_config(path):
    # M=1, K=N=256, group 32, symmetric, fp16, no bias
    c = make_case(1, 256, 256, 32, O.F16, True, False, seed=("tiny",))
    assert_close(DeviceCase(c).run(path), oracle_rows(c), O.F16, "tiny")


GRID = [
    # (M, N, K, g)
    (1, 8, 128, 32), (1, 40, 384, 128), (3, 264, 1152, 64), (5, 128, 4096, 128),
    (16, 520, 640, 32), (17, 96, 512, 128), (40, 264, 1152, 64), (64, 136, 256, 32),
    (70, 264, 1152, 128), (130, 200, 640, 64), (257, 136, 384, 32),
    # K not a multiple of 128 (an incomplete last run of 1, 2 or 3 chunks),
    # with complete 16-row tiles and an incomplete last tile
    (1, 48, 416, 32), (5, 40, 224, 32), (9, 24, 320, 64), (33, 56, 160, 32),
    (130, 72, 608, 32), (200, 264, 1216, 64),
]


@pytest.mark.parametrize("M,N,K,g", GRID)
@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("sym,bias", [(True, False), (False, True)])
def test_linear_grid(M, N, K, g, dt, sym, bias):
    c = make_case(M, N, K, g, dt, sym, bias, seed=("grid", M, N, K, g, dt, sym, bias))
    d = DeviceCase(c)
    ref = oracle_rows(c)
    for path in paths_for(M):
        assert_close(d.run(path), ref, dt, f"path {path}")


@pytest.mark.parametrize("N,K,sym,bias", [
    (1032, 1024, False, True),    # one wave per workgroup, incomplete last row tile
    (1024, 4096, False, False),   # four waves
    (1048, 14336, True, True),    # fourteen waves, incomplete last row tile
    (1024, 16384, False, False),  # sixteen waves, the most a workgroup has
])
def test_decode_workgroup_scales(tuning_env, N, K, sym, bias):
    # one token, bf16, groups of 128, K a whole number of 8-step runs and one
    # K range: the instance whose workgroup fetches all its waves' scales and
    # zero points at once.  Same arithmetic in the same order as the per-wave
    # instance (bit-identical), and within tolerance of the oracle.
    tuning_env("W4A16_GEMV_NO_ONE", "1")  # the general kernel's two instances
    c = make_case(1, N, K, 128, O.BF16, sym, bias, seed=("wgsz", N, K, sym, bias))
    d = DeviceCase(c)
    y_shared = d.run(GEMV)
    tuning_env("W4A16_GEMV_NO_WGSZ", "1")
    y_wave = d.run(GEMV)
    assert np.array_equal(y_shared, y_wave)
    assert_close(y_shared, oracle_rows(c), O.BF16, "workgroup scales")


def _general_splits(tuning_env, M, N, K, g, dt):
    # K ranges of the general decode kernel for the shape (the few-token
    # instance off)
    tuning_env("W4A16_GEMV_NO_ONE", "1")
    splits = L.w4a16_plan(M, N, K, g, dt, True, GEMV)["splits"]
    tuning_env("W4A16_GEMV_NO_ONE", None)
    return splits


def _few_token_instance_expected(M, N, K, g, general_splits):
    # the planner's rule: K a whole number of 128-k steps in runs of 8 or 4
    # (four and eight token rows try 4 first; whole runs before a last run
    # shorter by whole parts), at most 4 groups finished by a 16-lane row, at
    # most 32 group sums per result register, the staged x within the LDS
    # budget (token rows 1, 2, 4, or 8 for five to eight); one K range of at
    # most 16 runs first, then, where the general kernel splits K too, K
    # ranges of at most 16 runs (row tiles within the 16384 counters; one and
    # two token rows in no more K ranges than the general kernel, four and
    # eight token rows with the grid within twice the 256 CUs and the whole
    # LDS, four rows trying runs of 8 first); half the LDS budget where
    # workgroups share CUs
    ks, tiles = K // 128, -(-N // 16)
    mt = {1: 1, 2: 2, 3: 4, 4: 4}.get(M, 8 if 5 <= M <= 8 else 0)
    if not mt or K % 128:
        return False
    slots, parts = (4, 2) if mt == 8 else (mt, 4)
    a, b = (4, 8) if mt >= 4 else (8, 4)
    for split_pass in ((False, True) if general_splits > 1 else (False,)):
        x, y = (8, 4) if split_pass and mt == 4 else (a, b)
        for kpw, short in ((x, False), (y, False), (x, True), (y, True)):
            ngw, rest, runs = 128 * kpw // g, ks % kpw, -(-ks // kpw)
            splits = -(-runs // 16) if split_pass else 1
            waves = -(-runs // splits)
            full = tiles * splits <= 256 or (split_pass and (mt == 8 or (mt == 4 and kpw == 8)))
            budget = (160 * 1024 - 16 * 320 - 256) // (1 if full else 2)
            lds = waves * (64 * mt + (M if mt == 8 else mt) * (2 * kpw * 128 + (64 if mt > 1 else 0)))
            if (ngw <= 16 and ngw // parts <= 4 and ngw * slots <= 32 and (rest != 0) == short
                    and rest % (kpw // parts) == 0 and waves <= 16 and lds <= budget
                    and (not split_pass or (splits >= 2 and tiles <= 16384 and (
                        splits <= general_splits if mt <= 2 else tiles * splits <= 512)))):
                return True
    return False


@pytest.mark.parametrize("N,K", [(264, 512), (1048, 2048), (520, 2560), (776, 14336),
                                 # a last run shorter by whole quarter runs
                                 (136, 1280), (264, 2176), (136, 3456), (520, 9728)])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("sym,bias", [(True, False), (False, True)])
def test_decode_single_token_instance(tuning_env, N, K, g, dt, sym, bias):
    # one token: the few-token instance (each 16-lane row finishes a quarter
    # of the groups, metadata in registers, x group sums on the matrix cores)
    # against the oracle, and the general kernel on the same case
    gs = _general_splits(tuning_env, 1, N, K, g, dt)
    plan = L.w4a16_plan(1, N, K, g, dt, not sym, GEMV)
    assert plan["kernel"] == int(_few_token_instance_expected(1, N, K, g, gs)), (N, K, g, plan)
    c = make_case(1, N, K, g, dt, sym, bias, seed=("one", N, K, g, dt, sym, bias))
    d = DeviceCase(c)
    ref = oracle_rows(c)
    assert_close(d.run(GEMV), ref, dt, f"kernel {plan['kernel']}")
    tuning_env("W4A16_GEMV_NO_ONE", "1")
    assert L.w4a16_plan(1, N, K, g, dt, not sym, GEMV)["kernel"] == 0
    assert_close(d.run(GEMV), ref, dt, "general kernel")


@pytest.mark.parametrize("M", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("N,K", [(264, 512), (1048, 4096), (520, 2560), (776, 14336), (264, 2176), (136, 9728)])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("dt", [O.F16, O.BF16])
def test_decode_few_token_instance(tuning_env, M, N, K, g, dt):
    # two to eight tokens (three run as four token rows, the fourth never
    # stored; five to eight as eight rows, only M staged; K = 512 is one wave,
    # whose 64 threads store eight tokens in two passes): asymmetric with
    # bias, and symmetric, against the oracle; the general kernel on the same
    # cases
    gs = _general_splits(tuning_env, M, N, K, g, dt)
    plan = L.w4a16_plan(M, N, K, g, dt, True, GEMV)
    assert plan["kernel"] == int(_few_token_instance_expected(M, N, K, g, gs)), (M, N, K, g, plan)
    for sym, bias in ((False, True), (True, False)):
        c = make_case(M, N, K, g, dt, sym, bias, seed=("few", M, N, K, g, dt, sym, bias))
        d = DeviceCase(c)
        ref = oracle_rows(c)
        assert_close(d.run(GEMV), ref, dt, f"M={M} kernel {plan['kernel']} sym={sym}")
    tuning_env("W4A16_GEMV_NO_ONE", "1")
    assert_close(d.run(GEMV), ref, dt, "general kernel")


@pytest.mark.parametrize("dt", [O.F16, O.BF16])
def test_decode_single_token_instance_four_step_runs(tuning_env, dt):
    # runs of 4 k-steps where 8 would also fit (8 waves instead of 4)
    N, K, g = 1048, 4096, 128
    tuning_env("W4A16_GEMV_KPW", "4")
    plan = L.w4a16_plan(1, N, K, g, dt, True, GEMV)
    assert plan["kernel"] == 1 and plan["waves"] == 8, plan
    c = make_case(1, N, K, g, dt, False, True, seed=("one4", dt))
    assert_close(DeviceCase(c).run(GEMV), oracle_rows(c), dt, "4-step runs")


def test_decode_single_token_unaligned_scales_fall_back():
    # scales only 2-byte aligned: the general kernel runs instead
    import torch
    N, K, g = 520, 2048, 128
    c = make_case(1, N, K, g, O.BF16, False, True, seed=("one-unaligned",))
    d = DeviceCase(c)
    store = torch.empty(N * (K // g) + 1, dtype=d.s.dtype, device=d.s.device)
    s_off = store[1:].view(N, K // g)
    s_off.copy_(d.s)
    assert s_off.data_ptr() % 16 != 0
    y = L.w4a16_linear_path(d.x, d.wq, s_off, d.zp, d.bias, group_size=g, path=GEMV)
    torch.cuda.synchronize()
    assert_close(device_to_bits(y), oracle_rows(c), O.BF16, "unaligned scales")


@pytest.mark.parametrize("M,N,K,g,splits", [(1, 264, 28672, 128, 2), (2, 520, 28672, 128, 2),
                                              (3, 136, 28672, 64, 4), (2, 136, 1 << 16, 64, 4),
                                              (1, 1048, 1 << 16, 128, 4), (4, 40, 20480, 128, 2),
                                              (3, 520, 28672, 128, 2), (4, 264, 14336, 64, 2),
                                              # eight token rows
                                              (6, 520, 14336, 128, 2), (8, 136, 20480, 64, 3),
                                              (7, 264, 28672, 128, 4)])
@pytest.mark.parametrize("dt", [O.F16, O.BF16])
def test_decode_few_token_instance_k_split(tuning_env, M, N, K, g, splits, dt):
    # more than 16 runs, where the general kernel splits K too: K ranges of at
    # most 16 runs, fp32 partial sums through the workspace, the last
    # workgroup of a row tile adding them in range order; twice (the counters
    # must be zero again), bit-identical, and against the oracle and the
    # general kernel
    plan = L.w4a16_plan(M, N, K, g, dt, True, GEMV)
    assert (plan["kernel"], plan["splits"]) == (1, splits), plan
    c = make_case(M, N, K, g, dt, False, True, seed=("fewsplit", M, N, K, g, dt))
    d = DeviceCase(c)
    ref = oracle_rows(c)
    y = d.run(GEMV)
    assert_close(y, ref, dt, f"{splits} K ranges")
    assert np.array_equal(d.run(GEMV), y)
    tuning_env("W4A16_GEMV_NO_ONE", "1")
    assert_close(d.run(GEMV), ref, dt, "general kernel")


def test_ragged_n_not_multiple_of_eight_symmetric():
    # symmetric weights allow any N; N = 13 leaves a partial row tile
    for dt in (O.F16, O.BF16):
        c = make_case(3, 13, 256, 64, dt, True, True, seed=("rag13", dt))
        d = DeviceCase(c)
        for path in (GEMV, GEMM):
            assert_close(d.run(path), oracle_rows(c), dt, f"path {path}")


def test_k_single_group_and_odd_chunks():
    # K = 96 (three 32-k chunks: a partial 128-k step) and K = g
    for K, g in ((96, 32), (32, 32), (64, 64), (128, 128), (160, 32)):
        c = make_case(2, 24, K, g, O.BF16, False, False, seed=("kodd", K, g))
        d = DeviceCase(c)
        for path in (GEMV, GEMM):
            assert_close(d.run(path), oracle_rows(c), O.BF16, f"K={K} path {path}")


def test_m_zero_is_a_no_op():
    c = make_case(1, 64, 256, 128, O.F16, True, False, seed=("m0",))
    d = DeviceCase(c)
    x0 = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    y = L.w4a16_linear(x0, d.wq, d.s, None, group_size=128)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 64)


# ---- bit-exact properties ------------------------------------------------------

@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("g", [32, 128])
def test_one_hot_x_reproduces_dequantised_weight(dt, g):
    N, K = 48, 512
    c = make_case(1, N, K, g, dt, False, False, seed=("onehot", dt, g))
    d = DeviceCase(c)
    W = O.dequant_act(O.pack_weights(c.q), c.s_bits, O.pack_zeros(c.zp), N, K, g, dt)
    one = 0x3C00 if dt == O.F16 else 0x3F80
    for k in (0, 1, 6, 7, 8, 31, 32, 100, 255, 256, 511):
        x = np.zeros((1, K), dtype=np.uint16)
        x[0, k] = one
        d.set_x(x)
        for path in (GEMV, GEMM):
            y = d.run(path)
            assert np.array_equal(y[0], W[:, k]), f"k={k} path={path}"


@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("sym,g", [(True, 128), (False, 32)])
def test_gemm_operands_are_the_dequantised_weights(dt, sym, g):
    # x = identity (M = K tokens): y[k, n] = w[n, k] exactly, so every MFMA
    # operand the GEMM builds is compared bit for bit with the oracle's
    # dequantised weight, over scales spanning the format (bf16 up to 2^118:
    # the GEMM reads the codes as e4m3 numbers b * 2^-9 and multiplies by
    # s * 2^9, exact while that stays finite)
    N, K = 40, 256
    c = make_case(1, N, K, g, dt, sym, False, seed=("gemmop", dt, sym, g))
    rng = np.random.default_rng(13)
    lo, hi = (-14, 10) if dt == O.F16 else (-60, 118)
    sgn = np.where(rng.random(c.s_bits.shape) < 0.5, -1.0, 1.0)
    c.s_bits = O.f32_to_act_bits((sgn * 2.0 ** rng.uniform(lo, hi, c.s_bits.shape)).astype(np.float32), dt)
    c.s_bits[0, 0] = O.f32_to_act_bits(np.array([2.0 ** hi], np.float32), dt)[0]
    d = DeviceCase(c)
    zpk = None if sym else O.pack_zeros(c.zp)
    W = O.dequant_act(O.pack_weights(c.q), c.s_bits, zpk, N, K, g, dt)
    one = 0x3C00 if dt == O.F16 else 0x3F80
    d.set_x((np.eye(K) * one).astype(np.uint16))
    y = d.run(GEMM)
    # a zero weight (q = z) with a negative scale is -0; the fp32 sum that
    # starts from +0 returns +0, so the sign of zero is not compared
    nz = lambda a: np.where(a == 0x8000, 0, a)
    assert np.array_equal(nz(y), nz(W.T))


@pytest.mark.parametrize("path,few", [(GEMV, True), (GEMV, False), (GEMM, True)])  # few: decode kernels only
@pytest.mark.parametrize("dt", [O.F16, O.BF16])
def test_all_eights_symmetric_gives_bias(tuning_env, path, dt, few):
    # every weight is (8 - 8) * s = +0.  The GEMM multiplies those zeros, and
    # the general decode kernel's fp16 path multiplies q - z = 0: both give the
    # bias (or +0) bit for bit.  The general kernel's bf16 path and the
    # few-token instance (both dtypes) form sum x*(magic+q) - (magic+z)*sum x
    # in fp32, so they leave a residue of the order of fp32 round-off of those
    # sums, proportional to the magic offset (128 for bf16, 1024 for fp16):
    # 1e-4 absolute at 128.
    if not few:
        tuning_env("W4A16_GEMV_NO_ONE", "1")
    kernel = L.w4a16_plan(4, 64, 512, 64, dt, False, path)["kernel"]
    assert kernel == int(path == GEMV and few)
    for bias in (False, True):
        c = make_case(4, 64, 512, 64, dt, True, bias, seed=("eights", bias, dt))
        c.q[:] = 8
        y = DeviceCase(c).run(path)
        want = np.broadcast_to(c.bias_bits, y.shape) if bias else np.zeros_like(y)
        if path == GEMV and (dt == O.BF16 or kernel == 1):
            f = O.bf16_bits_to_f64 if dt == O.BF16 else O.f16_bits_to_f64
            err = np.abs(f(y) - f(want)).max()
            assert err <= 1e-4 * (128 if dt == O.BF16 else 1024) / 128
        else:
            assert np.array_equal(y, want)     # +0.0 exactly, no negative zeros


@pytest.mark.parametrize("path", [GEMV, GEMM])
@pytest.mark.parametrize("dt", [O.F16, O.BF16])
def test_symmetric_equals_asymmetric_with_eight(path, dt):
    c = make_case(5, 128, 1024, 128, dt, True, True, seed=("se", dt))
    y_sym = DeviceCase(c).run(path)
    c.zp = np.full((128, 8), 8, dtype=np.uint8)
    y_asym = DeviceCase(c).run(path)
    assert np.array_equal(y_sym, y_asym)


@pytest.mark.parametrize("path", [GEMV, GEMM])
def test_power_of_two_scaling_is_exact(path):
    c = make_case(3, 64, 1024, 128, O.F16, False, False, seed=("p2",))
    y1 = O.f16_bits_to_f64(DeviceCase(c).run(path))
    c.s_bits = O.f32_to_f16_bits(O.f16_bits_to_f64(c.s_bits).astype(np.float32) * 4)
    y4 = O.f16_bits_to_f64(DeviceCase(c).run(path))
    assert np.array_equal(y4, 4 * y1)


def test_determinism_with_split_k(tuning_env):
    # the general decode kernel at M = 5 takes 4 k-steps a wave: K = 9728 (76
    # steps) needs more than 16 waves, so K is split across two workgroups
    # (the few-token instance would run it unsplit)
    tuning_env("W4A16_GEMV_NO_ONE", "1")
    assert L.w4a16_plan(5, 2560, 9728, 128, O.BF16, True, GEMV)["splits"] == 2
    c = make_case(5, 2560, 9728, 128, O.BF16, False, False, seed=("det",))
    d = DeviceCase(c)
    a = d.run(GEMV)
    for _ in range(3):
        assert np.array_equal(d.run(GEMV), a)
    assert_close(a, oracle_rows(c), O.BF16, "split-K")


@pytest.mark.parametrize("M,N,K,g,sym", [(3, 2560, 9728, 128, True), (4, 2560, 9728, 128, False),
                                         (4, 264, 9728, 128, False), (3, 40, 9728, 64, False)])
def test_decode_three_four_tokens_long_k_unsplit(M, N, K, g, sym):
    # three or four tokens where 4 k-steps a wave would need more than 16
    # waves: 8 k-steps a wave, 8 x segments per lane, one K range
    assert L.w4a16_workspace_size(M, N, K, g, O.BF16, not sym, GEMV) == 0
    c = make_case(M, N, K, g, O.BF16, sym, True, seed=("x8", M, N, K, g, sym))
    assert_close(DeviceCase(c).run(GEMV), oracle_rows(c), O.BF16, "3-4 tokens, long K")


def test_workspace_reuse_across_shapes():
    # one workspace shared by split-K calls of different shapes, in an order
    # where a later call's counters sit where an earlier call's partial sums were
    # (every shape needs more than 16 waves for one K range, so each is split)
    # (or, at M <= 4 and 8 k-steps a wave, more LDS than one workgroup holds)
    shapes = [(5, 264, 20480, 128), (4, 2560, 20480, 128), (2, 40, 20480, 64), (3, 1024, 16384, 32)]
    cases = [make_case(M, N, K, g, O.BF16, False, False, seed=("reuse", M, N, K, g))
             for (M, N, K, g) in shapes]
    for (M, N, K, g) in shapes:
        assert L.w4a16_plan(M, N, K, g, O.BF16, True, GEMV)["splits"] > 1, (M, N, K, g)
    devs = [DeviceCase(c) for c in cases]
    refs = [oracle_rows(c) for c in cases]
    for _ in range(2):
        for d, ref in zip(devs, refs):
            assert_close(d.run(GEMV), ref, O.BF16, "reuse")


@pytest.mark.parametrize("M", [3, 4])
def test_decode_long_k_one_tile_per_cu_unsplit(M):
    # three or four tokens on a 14336 x 4096 layer (256 row tiles, one per CU):
    # with nearly all of the CU's LDS for one workgroup, K stays whole
    N, K = 4096, 14336
    assert L.w4a16_plan(M, N, K, 128, O.BF16, True, GEMV)["splits"] == 1
    c = make_case(M, N, K, 128, O.BF16, False, False, seed=("lds160", M))
    assert_close(DeviceCase(c).run(GEMV), oracle_rows(c), O.BF16, f"M={M}")


def test_workspace_errors():
    # K = 20480 needs more than 16 waves of 8 k-steps: the decode kernel splits
    # K and needs a workspace
    c = make_case(1, 40, 20480, 128, O.BF16, False, False, seed=("ws",))
    d = DeviceCase(c)
    need = L.w4a16_workspace_size(1, 40, 20480, 128, O.BF16, True, GEMV)
    assert need > 0
    y = torch.empty((1, 40), dtype=torch.bfloat16, device="cuda")
    from int4_weight_only_linear_amd import _binding as B
    st = B.lib.w4a16_linear_path(d.x.data_ptr(), d.wq.data_ptr(), d.s.data_ptr(), d.zp.data_ptr(),
                                 None, y.data_ptr(), 1, 40, 20480, 128, O.BF16, None, 0,
                                 torch.cuda.current_stream().cuda_stream, GEMV)
    assert st == 6 and "workspace" in L.w4a16_last_error()


# ---- the workloads at full size ------------------------------------------------

def _config_points(name):
    c = CONFIGS[name]
    for li, layer in enumerate(c.layers):
        for g in c.groups:
            for sym in c.symmetric:
                for dt in c.dtypes:
                    for bias in c.bias:
                        yield pytest.param(name, li, layer.K, layer.N, g, sym, dt, bias,
                                           id=f"{name}-K{layer.K}-N{layer.N}-g{g}-{'sym' if sym else 'asym'}-{'f16' if dt == 0 else 'bf16'}{'-bias' if bias else ''}")


ALL_POINTS = [p for n in ("llama8b_decode", "qwen3_4b_decode", "llama8b_prefill", "sweep")
              for p in _config_points(n)]


def _every_row(name, K, g):
    # every output row is compared, except on the sweep's 28672 x 4096 layer
    # with groups of 32 or 64 (sampled rows: the oracle's whole-layer cost
    # there would dominate the suite); its groups of 128 run in full
    return not (name == "sweep" and K == 28672 and g != 128)


@pytest.mark.parametrize("name,li,K,N,g,sym,dt,bias", ALL_POINTS)
def test_config_full_size(name, li, K, N, g, sym, dt, bias):
    # rows of y are independent, so one oracle product over the largest M
    # serves every M of the point (its first M rows)
    Ms = CONFIGS[name].Ms
    c = make_case(max(Ms), N, K, g, dt, sym, bias, seed=(name, li, g, sym, dt, bias))
    d = DeviceCase(c)
    rows = np.arange(N) if _every_row(name, K, g) else sample_rows(N, seed=li)
    ref_all = oracle_rows(c, None if len(rows) == N else rows)
    full_x = c.x_bits
    for M in Ms:
        d.set_x(full_x[:M].copy())
        for path in (AUTO,) + paths_for(M):
            y = d.run(path)
            assert_close(y[:, rows], ref_all[:M], dt, f"M={M} path={path}")


# ---- one GPU's share under 8-way tensor parallelism ---------------------------

@pytest.mark.parametrize("layer,K,N,Ms", [
    ("qkv", 4096, 768, (1, 5, 1920)),      # column-parallel: N / 8
    ("o", 512, 4096, (1, 5)),              # row-parallel: K / 8 (four 128-k steps)
    ("gate_up", 4096, 3584, (1, 5, 1920)),
    ("down", 1792, 4096, (1, 5, 1920)),    # fourteen 128-k steps
])
def test_tensor_parallel_shard_shapes(layer, K, N, Ms):
    # the Llama-3.1-8B layers' 8-way shards at their real shapes, on the
    # path the dispatcher picks and on each kernel that serves the M; every
    # output row against the oracle
    c = make_case(max(Ms), N, K, 128, O.BF16, False, True, seed=("tp8", layer))
    d = DeviceCase(c)
    ref_all = oracle_rows(c)
    full_x = c.x_bits
    for M in Ms:
        d.set_x(full_x[:M].copy())
        for path in (AUTO,) + paths_for(M):
            assert_close(d.run(path), ref_all[:M], O.BF16, f"{layer} M={M} path={path}")


# ---- dequantised prefill copy: dense product over w4a16_dequant's weights -----

@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("M,N,K,g,sym,bias", [
    (1, 64, 256, 32, True, False), (130, 200, 640, 64, False, True),
    (257, 136, 416, 32, False, False), (1920, 512, 1024, 128, False, True),
])
def test_dense_prefill_copy(dt, M, N, K, g, sym, bias):
    c = make_case(M, N, K, g, dt, sym, bias, seed=("dense", M, N, K, g, dt, sym, bias))
    d = DeviceCase(c)
    w = L.w4a16_dequant(d.wq, d.s, d.zp, group_size=g)
    y = L.w4a16_linear_dense(d.x, w, d.bias)
    torch.cuda.synchronize()
    # the reference multiplies the same rounded weights, exactly (float64)
    zpk = None if sym else O.pack_zeros(c.zp)
    W = O.act_bits_to_f64(O.dequant_act(O.pack_weights(c.q), c.s_bits, zpk, N, K, g, dt), dt)
    ref = O.act_bits_to_f64(c.x_bits, dt) @ W.T
    if bias:
        ref = ref + O.act_bits_to_f64(c.bias_bits, dt)[None, :]
    got = device_to_bits(y)
    assert_close(got, ref, dt, "dense copy")
    # and the W4A16 prefill GEMM, which multiplies the same rounded weights
    assert_close(d.run(GEMM), ref, dt, "prefill GEMM vs the same weights")


@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("tile", ["8,1,0,2", "6,1,0,2", "4,1,0,1", "4,3,0,2", "4,4,1,1"])
@pytest.mark.parametrize("M,N,K,g,sym", [(300, 520, 1024, 128, False), (130, 200, 416, 32, True)])
def test_dense_copy_equals_prefill_gemm_bit_for_bit(tuning_env, dt, tile, M, N, K, g, sym):
    # with the tile and K split forced to be the same, the dense instance and
    # the W4A16 GEMM multiply the same rounded weights in the same order
    tuning_env("W4A16_GEMM_TILE", tile)
    c = make_case(M, N, K, g, dt, sym, True, seed=("densebits", M, N, K, g, dt, sym))
    d = DeviceCase(c)
    w = L.w4a16_dequant(d.wq, d.s, d.zp, group_size=g)
    y_dense = device_to_bits(L.w4a16_linear_dense(d.x, w, d.bias))
    assert np.array_equal(y_dense, d.run(GEMM)), f"tile {tile}"


# ---- per-channel scales: group_size == K (one scale and zero point per row) ----

@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("M,N,K,sym,bias", [
    (1, 64, 4096, False, False), (5, 40, 320, True, True), (33, 24, 96, False, True),
    (130, 72, 1152, False, False), (2, 200, 416, False, True),
])
def test_per_channel_scales(dt, M, N, K, sym, bias):
    c = make_case(M, N, K, K, dt, sym, bias, seed=("perchan", M, N, K, dt, sym, bias))
    d = DeviceCase(c)
    ref = oracle_rows(c)
    for path in paths_for(M):
        assert_close(d.run(path), ref, dt, f"per-channel path {path}")
    w = device_to_bits(L.w4a16_dequant(d.wq, d.s, d.zp, group_size=K))
    zpk = None if sym else O.pack_zeros(c.zp)
    assert np.array_equal(w, O.dequant_act(O.pack_weights(c.q), c.s_bits, zpk, N, K, K, dt))


# ---- expert-indexed decode (fused-MoE skinny GEMM) ------------------------------

def _moe_case(E, topk, M, N, K, g, dt, sym, bias, weights, x_per_slot, seed, invalid=True):
    cases = [make_case(1, N, K, g, dt, sym, bias, seed=(seed, "expert", e)) for e in range(E)]
    rng = np.random.default_rng(stream_seed("moe-ids", seed, E, topk, M))
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32)
    if invalid and M * topk >= 3:
        ids.flat[1] = -1
        ids.flat[M * topk - 1] = E
    w = rng.random((M, topk)).astype(np.float32) if weights else None
    xc = make_case(M * topk if x_per_slot else M, N, K, g, dt, sym, False, seed=(seed, "x"))
    host = dict(
        wq=np.stack([L.w4a16_pack_weights(c.q) for c in cases]),
        s=np.stack([c.s_bits for c in cases]),
        zp=None if sym else np.stack([L.w4a16_pack_zeros(c.zp) for c in cases]),
        bias=np.stack([c.bias_bits for c in cases]) if bias else None,
        x=xc.x_bits, ids=ids, w=w)
    return host


def _moe_device(h, dt):
    from gpu_util import bits_to_device
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dict(wq=t(h["wq"]), s=bits_to_device(h["s"], dt, "cuda:0"),
                zp=t(h["zp"]), bias=None if h["bias"] is None else bits_to_device(h["bias"], dt, "cuda:0"),
                x=bits_to_device(h["x"], dt, "cuda:0"), ids=t(h["ids"]), w=t(h["w"]))


@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("E,topk,M,N,K,g,sym,bias,weights,xps", [
    (8, 2, 3, 48, 256, 64, False, True, True, False),
    (16, 4, 2, 40, 416, 32, True, False, False, True),
    (4, 1, 5, 24, 4096, 128, False, False, True, False),
    (6, 3, 1, 200, 320, 320, False, True, False, False),   # per-channel scales
])
def test_moe_linear(dt, E, topk, M, N, K, g, sym, bias, weights, xps):
    h = _moe_case(E, topk, M, N, K, g, dt, sym, bias, weights, xps, seed=("moe", E, topk, M, N, K, g))
    d = _moe_device(h, dt)
    y = L.w4a16_moe_linear(d["x"], d["wq"], d["s"], d["ids"], d["zp"], d["bias"], d["w"],
                           group_size=g, x_per_slot=xps)
    torch.cuda.synchronize()
    ref = O.moe_linear_ref(h["x"], h["wq"].view(np.int32).reshape(E * N, K // 8).reshape(E, N, K // 8),
                           h["s"], h["zp"], h["bias"], h["ids"], h["w"], M, topk, E, N, K, g, dt,
                           x_per_slot=xps)
    got = device_to_bits(y)
    assert_close(got, ref, dt, "moe")
    bad = [i for i, e in enumerate(h["ids"].ravel()) if not 0 <= e < E]
    assert np.all(got[bad] == 0)


def test_moe_linear_full_size_sampled():
    # Qwen3-30B-A3B-shaped experts (hidden 2048, expert intermediate 768, gate and
    # up fused: N = 1536), 128 experts, top-8, 4 tokens; 8 slots checked
    E, topk, M, N, K, g, dt = 128, 8, 4, 1536, 2048, 128, O.BF16
    h = _moe_case(E, topk, M, N, K, g, dt, False, False, True, False, seed="moefull", invalid=False)
    d = _moe_device(h, dt)
    y = device_to_bits(L.w4a16_moe_linear(d["x"], d["wq"], d["s"], d["ids"], d["zp"], None, d["w"],
                                          group_size=g))
    for slot in (0, 5, 9, 14, 19, 22, 27, 31):
        m, j = divmod(slot, topk)
        e = int(h["ids"][m, j])
        ref = O.linear_ref(h["x"][m:m + 1], h["wq"][e], h["s"][e], h["zp"][e], None, 1, N, K, g, dt)[0]
        ref = ref * float(h["w"][m, j])
        assert_close(y[slot:slot + 1], ref[None, :], dt, f"moe slot {slot}")


@pytest.mark.parametrize("g,kmax", [(128, 15360), (64, 13312), (32, 9216)])
def test_moe_linear_k_bound(g, kmax):
    # one workgroup per slot: the largest K the header states runs (against
    # the oracle), the next multiple of 128 is refused before any launch; for
    # groups of 64 and 128, K = 16384 (16 runs of 8 k-steps on the
    # single-token instance) runs too
    E, topk, M, N, dt = 2, 1, 1, 32, O.BF16
    h = _moe_case(E, topk, M, N, kmax, g, dt, False, False, False, False, seed=("moek", g), invalid=False)
    d = _moe_device(h, dt)
    y = device_to_bits(L.w4a16_moe_linear(d["x"], d["wq"], d["s"], d["ids"], d["zp"], None, None, group_size=g))
    e = int(h["ids"][0, 0])
    ref = O.linear_ref(h["x"][0:1], h["wq"][e], h["s"][e], h["zp"][e], None, 1, N, kmax, g, dt)
    assert_close(y, ref, dt, f"moe K={kmax}")
    K2 = kmax + 128
    wq2 = torch.zeros((E, N, K2 // 8), dtype=torch.int32, device="cuda:0")
    s2 = torch.zeros((E, N, K2 // g), dtype=torch.bfloat16, device="cuda:0")
    zp2 = torch.zeros((E, N // 8, K2 // g), dtype=torch.int32, device="cuda:0")
    x2 = torch.zeros((M, K2), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(L.W4A16Error, match="too large for one decode workgroup"):
        L.w4a16_moe_linear(x2, wq2, s2, d["ids"], zp2, None, None, group_size=g)
    if g >= 64:
        K3 = 16384
        h = _moe_case(E, topk, M, N, K3, g, dt, False, False, False, False, seed=("moek3", g), invalid=False)
        d = _moe_device(h, dt)
        y = device_to_bits(L.w4a16_moe_linear(d["x"], d["wq"], d["s"], d["ids"], d["zp"], None, None,
                                              group_size=g))
        e = int(h["ids"][0, 0])
        ref = O.linear_ref(h["x"][0:1], h["wq"][e], h["s"][e], h["zp"][e], None, 1, N, K3, g, dt)
        assert_close(y, ref, dt, f"moe K={K3}")


# ---- GEMM K split: last-workgroup hand-off and the two-pass form ----------------

@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("tile", ["4,3,0", "4,3,1", "6,5,0", "8,2,0", "4,7,1",
                                  "4,1,0,1", "4,3,0,1", "4,3,1,1", "8,1,0,1", "8,2,0,1"])
@pytest.mark.parametrize("M,N,K,g,bias", [(130, 200, 640, 64, True), (128, 264, 1216, 32, False),
                                          (300, 56, 2048, 128, True)])
def test_gemm_k_split_forms(tuning_env, dt, tile, M, N, K, g, bias):
    tuning_env("W4A16_GEMM_TILE", tile)
    c = make_case(M, N, K, g, dt, False, bias, seed=("ksplit", M, N, K, g, dt, bias))
    d = DeviceCase(c)
    y1 = d.run(GEMM)
    assert_close(y1, oracle_rows(c), dt, f"GEMM tile {tile}")
    assert np.array_equal(d.run(GEMM), y1), "split-K result changed between runs"


@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("tile", ["1,1,0,1", "1,3,0,1", "1,5,1,1", "1,2,0", "1,4,1", "1,9,1,1"])
@pytest.mark.parametrize("M,N,K,g,sym,bias", [(1, 200, 1216, 32, False, True), (17, 264, 2048, 64, True, False),
                                              (33, 13, 1152, 128, True, True), (64, 520, 4096, 128, False, False)])
def test_gemm_thin_tiles(tuning_env, dt, tile, M, N, K, g, sym, bias):
    # 32-token tiles (128 or 256 features): one K range, the last-workgroup
    # hand-off and the two-pass form; ragged N, K tails, one token and M past
    # a tile; against the oracle, twice bit-identical
    tuning_env("W4A16_GEMM_TILE", tile)
    plan = L.w4a16_plan(M, N, K, g, dt, not sym, GEMM)
    assert plan["tile_tokens"] == 32, plan
    c = make_case(M, N, K, g, dt, sym, bias, seed=("thin", M, N, K, g, dt, sym, bias))
    d = DeviceCase(c)
    y1 = d.run(GEMM)
    assert_close(y1, oracle_rows(c), dt, f"GEMM tile {tile}")
    assert np.array_equal(d.run(GEMM), y1), "split-K result changed between runs"


def test_gemm_planner_takes_thin_tiles_up_to_64_tokens():
    # 32-token tiles up to M = 32, and to M = 64 where K <= 16384
    for (K, N) in ((4096, 14336), (28672, 4096), (4096, 6144), (14336, 4096)):
        for M in (1, 9, 16, 32, 48, 64):
            thin = M <= 32 or K <= 16384
            assert (L.w4a16_plan(M, N, K, 128, O.BF16, True, GEMM)["tile_tokens"] == 32) == thin, (M, N, K)
        assert L.w4a16_plan(65, N, K, 128, O.BF16, True, GEMM)["tile_tokens"] >= 128


# ---- random shapes through the automatic path ----------------------------------

def _random_shape(i):
    # seeded per index: decode and GEMM sizes, ragged N (multiples of 8 with
    # zero points, any N without), K a multiple of the group (often of 128),
    # every group, dtype, quantisation and bias
    r = np.random.default_rng(stream_seed(("random-shape", i)))
    g = int(r.choice([32, 64, 128]))
    sym = bool(r.integers(2))
    M = int(r.integers(1, 17)) if r.random() < 0.5 else int(r.integers(17, 400))
    N = int(r.integers(1, 260)) * 8 - (int(r.integers(0, 8)) if sym else 0)
    K = g * int(r.integers(1, 4096 // g + 1))
    if r.random() < 0.5:
        K = max(128, K // 128 * 128)
    return M, max(N, 1), K, g, int(r.choice([O.F16, O.BF16])), sym, bool(r.integers(2))


@pytest.mark.parametrize("i", range(40))
def test_random_shapes_match_the_oracle(i):
    M, N, K, g, dt, sym, bias = _random_shape(i)
    c = make_case(M, N, K, g, dt, sym, bias, seed=("random", i))
    y = DeviceCase(c).run(L.PATH_AUTO)
    assert_close(y, oracle_rows(c), dt, f"shape {(M, N, K, g, dt, sym, bias)}")


def _random_large_shape(i):
    # seeded per index: prefill sizes whose plans take the tall and wide tiles,
    # K splits and tail launches
    r = np.random.default_rng(stream_seed(("random-large-shape", i)))
    g = int(r.choice([32, 64, 128]))
    M = int(r.integers(400, 2049))
    N = int(r.integers(256, 2049)) * 8
    K = g * int(r.integers(128 // g, 8192 // g + 1))
    return M, N, K, g, int(r.choice([O.F16, O.BF16])), bool(r.integers(2)), bool(r.integers(2))


@pytest.mark.parametrize("i", range(24))
def test_random_large_shapes_match_the_oracle_on_sampled_rows(i):
    M, N, K, g, dt, sym, bias = _random_large_shape(i)
    c = make_case(M, N, K, g, dt, sym, bias, seed=("random-large", i))
    y = DeviceCase(c).run(L.PATH_AUTO)
    rows = sample_rows(N, seed=i, blocks=6)
    assert_close(y[:, rows], oracle_rows(c, rows), dt, f"shape {(M, N, K, g, dt, sym, bias)}")


# ---- GEMM tail launch: the tiles past the last full round as smaller tiles ------

_TAIL_CASES = [
    # M, N, K, g, dt, sym, bias: 256-token tiles, the tail in 128-token tiles
    (1300, 28672, 1024, 128, O.BF16, False, True),   # 256 features, the last tiles' upper halves past M
    (1300, 28672, 1024, 128, O.F16, True, False),    # the same in fp16, symmetric
    (1000, 16512, 1024, 32, O.F16, False, True),     # 128 features, both halves of every tail tile
    (1000, 8264, 2048, 32, O.F16, False, False),     # 128 features, N not a multiple of the tile
    (2100, 8264, 1024, 32, O.F16, True, True),       # ragged M and N
]


@pytest.mark.parametrize("M,N,K,g,dt,sym,bias", _TAIL_CASES)
def test_gemm_tail_launch(tuning_env, M, N, K, g, dt, sym, bias):
    # every output against the oracle, and bit-identical to the same tiles
    # run without the tail launch (each output's sums in the same order)
    plan = L.w4a16_plan(M, N, K, g, dt, not sym, GEMM)
    assert plan["tail_tiles"] > 0 and plan["launches"] == 2 and plan["workspace_bytes"] == 0, plan
    c = make_case(M, N, K, g, dt, sym, bias, seed=("tail", M, N, K, g, dt, sym, bias))
    d = DeviceCase(c)
    y = d.run(GEMM)
    assert_close(y, oracle_rows(c), dt, "GEMM with a tail launch")
    tuning_env("W4A16_GEMM_TILE", f"{plan['tile_tokens'] // 32},1,0,{plan['tile_features'] // 128}")
    assert L.w4a16_plan(M, N, K, g, dt, not sym, GEMM)["tail_tiles"] == 0
    assert np.array_equal(d.run(GEMM), y), "tail launch differs from the same tiles without it"


def test_dense_copy_with_tail_launch():
    M, N, K, g = 1300, 28672, 1024, 128
    assert L.w4a16_plan(M, N, K, g, O.BF16, True, GEMM)["tail_tiles"] > 0
    c = make_case(M, N, K, g, O.BF16, False, True, seed=("densetail", M, N, K))
    d = DeviceCase(c)
    w = L.w4a16_dequant(d.wq, d.s, d.zp, group_size=g)
    assert np.array_equal(device_to_bits(L.w4a16_linear_dense(d.x, w, d.bias)), d.run(GEMM))


# ---- graph capture: every entry point replays to its eager result --------------

def _graph_replays_match(run_eager, run_captured, reps=3):
    eager = run_eager()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            out = run_captured()
    torch.cuda.synchronize()
    for _ in range(reps):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        run_eager()                         # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K,g,path,tile", [
    (1, 4096, 4096, 128, GEMV, None),        # decode, no split
    (5, 40, 9728, 64, GEMV, None),           # decode, K split (workspace counters)
    (130, 200, 640, 64, GEMM, "4,3,0"),      # GEMM, last-workgroup hand-off
    (128, 264, 1216, 32, GEMM, "4,4,1"),     # GEMM, two-pass split
    (300, 520, 1024, 128, GEMM, None),       # GEMM, no split
    (2, 1048, 28672, 128, GEMV, None),       # decode, few-token instance with a K split
    (17, 264, 2048, 64, GEMM, "1,3,0,1"),    # GEMM 32-token tiles, last-workgroup hand-off
    (33, 520, 4096, 128, GEMM, "1,5,1,1"),   # GEMM 32-token tiles, two-pass split
    (1300, 28672, 1024, 128, GEMM, None),    # GEMM with a tail launch (two kernels)
])
def test_graph_capture_linear(tuning_env, M, N, K, g, path, tile):
    if tile:
        tuning_env("W4A16_GEMM_TILE", tile)
    c = make_case(M, N, K, g, O.BF16, False, True, seed=("graph", M, N, K, g, path))
    d = DeviceCase(c)
    need = L.w4a16_workspace_size(M, N, K, g, O.BF16, True, path)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda") if need else None
    y_cap = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def run(out=None):
        return L.w4a16_linear_path(d.x, d.wq, d.s, d.zp, d.bias, group_size=g, path=path, out=out,
                                   workspace=ws)
    _graph_replays_match(lambda: run(), lambda: run(y_cap))


def test_graph_capture_dense_and_moe():
    c = make_case(128, 136, 512, 64, O.F16, False, True, seed=("graphdense",))
    d = DeviceCase(c)
    w = L.w4a16_dequant(d.wq, d.s, d.zp, group_size=64)
    ws = torch.zeros(L.w4a16_dense_workspace_size(128, 136, 512, O.F16, True), dtype=torch.uint8,
                     device="cuda")
    y_cap = torch.empty((128, 136), dtype=torch.float16, device="cuda")
    _graph_replays_match(lambda: L.w4a16_linear_dense(d.x, w, d.bias, workspace=ws),
                         lambda: L.w4a16_linear_dense(d.x, w, d.bias, out=y_cap, workspace=ws))
    h = _moe_case(8, 2, 3, 48, 256, 64, O.BF16, False, True, True, False, seed="graphmoe")
    m = _moe_device(h, O.BF16)
    y_moe = torch.empty((6, 48), dtype=torch.bfloat16, device="cuda")
    run = lambda out=None: L.w4a16_moe_linear(m["x"], m["wq"], m["s"], m["ids"], m["zp"], m["bias"],
                                              m["w"], group_size=64, out=out)
    _graph_replays_match(lambda: run(), lambda: run(y_moe))


# ---- guard bands: nothing is written outside y and the workspace ---------------

CANARY16 = 0x7E5A          # an unlikely output pattern (a bf16 / fp16 NaN-free value)
CANARY8 = 0xA5


@pytest.mark.parametrize("M,N,K,g,path,tile,ypad", [
    (1, 4096, 4096, 128, GEMV, None, 64),      # decode, one K range, aligned y
    (4, 264, 1152, 64, GEMV, None, 3),         # decode, ragged tile, y at a 6-byte offset
    (5, 264, 20480, 128, GEMV, None, 64),      # decode, K split (counters + partials)
    (5, 264, 9728, 128, GEMV, None, 3),        # decode, eight token rows, shorter last run
    (3, 40, 20480, 32, GEMV, None, 5),         # decode, K split, incomplete tile
    (300, 520, 1024, 128, GEMM, None, 64),     # GEMM, no split, 16-byte stores
    (130, 200, 640, 64, GEMM, "4,3,0", 3),     # GEMM, last-workgroup hand-off, element stores
    (17, 264, 2048, 64, GEMM, "1,3,0,1", 3),   # GEMM 32-token tiles, hand-off, element stores
    (40, 13, 1152, 128, GEMM, "1,5,1,1", 7),   # GEMM 32-token tiles, two-pass, N not a multiple of 8
    (128, 264, 1216, 32, GEMM, "4,4,1", 64),   # GEMM, two-pass split
    (129, 13, 256, 64, GEMM, "4,2,1", 7),      # GEMM, two-pass, N not a multiple of 8
    (1300, 28672, 1024, 128, GEMM, None, 3),   # GEMM with a tail launch, element stores
])
def test_guard_bands_around_y_and_workspace(tuning_env, M, N, K, g, path, tile, ypad):
    if tile:
        tuning_env("W4A16_GEMM_TILE", tile)
    sym = N % 8 != 0
    c = make_case(M, N, K, g, O.BF16, sym, True, seed=("guard", M, N, K, g, path))
    d = DeviceCase(c)
    inputs = [t for t in (d.x, d.wq, d.s, d.zp, d.bias) if t is not None]
    before = [t.clone() for t in inputs]
    # y inside a larger buffer whose margins hold a canary
    ybuf = torch.full((ypad + M * N + 64,), CANARY16, dtype=torch.int16, device="cuda")
    y = ybuf.view(torch.bfloat16)[ypad:ypad + M * N].view(M, N)
    need = L.w4a16_workspace_size(M, N, K, g, O.BF16, not sym, path)
    guard = 4096
    wbuf = torch.full((need + 2 * guard,), CANARY8, dtype=torch.uint8, device="cuda")
    wbuf[guard:guard + need].zero_()
    ws = wbuf[guard:guard + need] if need else None
    for _ in range(2):
        L.w4a16_linear_path(d.x, d.wq, d.s, d.zp, d.bias, group_size=g, path=path, out=y, workspace=ws)
        torch.cuda.synchronize()
        assert_close(device_to_bits(y), oracle_rows(c), O.BF16, "guarded y")
        yb = ybuf.cpu().numpy().view(np.uint16)
        assert np.all(yb[:ypad] == CANARY16) and np.all(yb[ypad + M * N:] == CANARY16), "write outside y"
        wb = wbuf.cpu().numpy()
        assert np.all(wb[:guard] == CANARY8) and np.all(wb[guard + need:] == CANARY8), "write outside workspace"
        if need:
            # every completed call leaves the counter region zero
            assert not wb[guard:guard + 64 * 1024].any(), "counters not reset"
        for t, t0 in zip(inputs, before):
            assert torch.equal(t, t0), "an input was modified"


# ---- negative and extreme scales on both kernels -------------------------------

@pytest.mark.parametrize("dt", [O.F16, O.BF16])
@pytest.mark.parametrize("sym,g", [(True, 128), (False, 32), (False, 128)])
@pytest.mark.parametrize("M", [1, 4])
def test_negative_and_extreme_scales(dt, sym, g, M):
    # each 16-row tile draws a base exponent over most of the format's range,
    # every (row, group) scale a random sign and a further factor of 2^[-3, 3];
    # outputs are compared tile by tile, relative to the tile's largest output
    N, K = 320, 1024
    c = make_case(M, N, K, g, dt, sym, False, seed=("xscale", dt, sym, g, M))
    rng = np.random.default_rng(stream_seed("xscale", dt, sym, g, M))
    lo, hi = (-20, 3) if dt == O.F16 else (-90, 90)
    base = np.repeat(rng.uniform(lo, hi, N // 16), 16)[:, None]
    e = base + rng.uniform(-3, 3, c.s_bits.shape)
    sgn = np.where(rng.random(c.s_bits.shape) < 0.5, -1.0, 1.0)
    c.s_bits = O.f32_to_act_bits((sgn * 2.0 ** e).astype(np.float32), dt)
    d = DeviceCase(c)
    # the decode kernel never rounds a weight, so it is held to the exact
    # oracle; the prefill GEMM multiplies the weights rounded once to the act
    # dtype (the values w4a16_dequant returns), and with scales that vary by
    # 2^6 inside a tile that rounding alone can reach the bf16 bound relative
    # to the tile's largest output, so the GEMM is held to the product over
    # the same rounded weights
    zpk = None if sym else O.pack_zeros(c.zp)
    W = O.act_bits_to_f64(O.dequant_act(O.pack_weights(c.q), c.s_bits, zpk, N, K, g, dt), dt)
    refs = {GEMV: oracle_rows(c), GEMM: O.act_bits_to_f64(c.x_bits, dt) @ W.T}
    for path in (GEMV, GEMM):
        y = d.run(path)
        for t in range(N // 16):
            r = slice(16 * t, 16 * t + 16)
            assert_close(y[:, r], refs[path][:, r], dt, f"path {path} tile {t} (2^{base[16 * t, 0]:.0f})")


# ---- a split decode layer with more row tiles than completion counters ---------

@pytest.mark.parametrize("M", [3, 5])
def test_split_decode_past_the_counter_region(M):
    # N = 262160 rows = 16385 row tiles, one more than the 16384 counters; K =
    # 8320 makes three and five tokens split K, so the call runs as two
    # launches (tiles 0..16383, then 16384).  Tiles on both sides of the chunk
    # boundary are compared with the oracle, twice (the first call's counters
    # must be zero again for the second).
    N, K, g = 262160, 8320, 128
    wpr, G = K // 8, K // g
    plan = L.w4a16_plan(M, N, K, g, O.BF16, True, GEMV)
    assert plan["splits"] >= 2 and plan["launches"] == 2 and plan["tiles"] == 16385, plan
    dev = torch.device("cuda:0")
    tiles = sorted({0, 1, 9000, 16382, 16383, 16384})
    note(f"[gpu] chunked split: drawing {N * K // 2 / 2**30:.2f} GiB of packed weights")
    wq = torch.empty((N, wpr), dtype=torch.int32, device=dev)
    tile_words = {}
    block = 1 << 15
    for r0 in range(0, N, block):
        rows = min(block, N - r0)
        words = stored_words("chunked-w", r0, rows, wpr)
        wq[r0:r0 + rows].copy_(torch.from_numpy(words.view(np.int32)))
        for t in tiles:
            if r0 <= 16 * t < r0 + rows:
                tile_words[t] = words[16 * t - r0:16 * t - r0 + 16].copy()
        del words
    zpk = stored_words("chunked-z", 0, N // 8, G)
    rng = np.random.default_rng(stream_seed("chunked-s"))
    s_bits = to_act_bits((np.abs(rng.normal(0.0, 0.02, size=(N, G))) + 1e-3).astype(np.float32), O.BF16)
    x_bits = to_act_bits(rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32), O.BF16)
    s, zp = bits_to_device(s_bits, O.BF16, dev), torch.from_numpy(zpk.view(np.int32)).to(dev)
    x = bits_to_device(x_bits, O.BF16, dev)
    ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
    first = None
    for rep in range(2):
        y = L.w4a16_linear_path(x, wq, s, zp, None, group_size=g, path=GEMV, workspace=ws)
        torch.cuda.synchronize()
        yb = device_to_bits(y)
        assert not ws[:64 * 1024].any().item(), "counters not reset"
        for t in tiles:
            r = slice(16 * t, 16 * t + 16)
            ref = O.linear_ref(x_bits, tile_words[t].view(np.int32), s_bits[r],
                               zpk[2 * t:2 * t + 2].view(np.int32), None, M, 16, K, g, O.BF16)
            assert_close(yb[:, r], ref, O.BF16, f"M={M} tile={t} call {rep}")
        if first is None:
            first = yb
        else:
            assert np.array_equal(first, yb)
