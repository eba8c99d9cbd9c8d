"""The allocation-free entry point (w4a16_linear_noalloc) through the C ABI:
same results as w4a16_linear with a caller's workspace, on split and unsplit
plans of both kernels, two calls in a row with the second one smaller, and a
clear refusal above the scratch it holds."""
import ctypes

import numpy as np
import pytest

import oracle as O
from synth import make_case
from gpu_util import DeviceCase, assert_close, device_to_bits, note, oracle_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import int4_weight_only_linear_amd as L  # noqa: E402
from int4_weight_only_linear_amd import _binding as B  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    note(f"[gpu] {request.node.nodeid}")


def _noalloc(d, y):
    c = d.case
    st = B.lib.w4a16_linear_noalloc(d.x.data_ptr(), d.wq.data_ptr(), d.s.data_ptr(),
                                    None if d.zp is None else d.zp.data_ptr(),
                                    None if d.bias is None else d.bias.data_ptr(), y.data_ptr(),
                                    c.M, c.N, c.K, c.group, c.dtype,
                                    torch.cuda.current_stream().cuda_stream)
    B._check(st)
    torch.cuda.synchronize()
    return device_to_bits(y)


def _with_workspace(d):
    c = d.case
    need = L.w4a16_workspace_size(c.M, c.N, c.K, c.group, c.dtype, c.zp is not None)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    y = L.w4a16_linear(d.x, d.wq, d.s, d.zp, d.bias, group_size=c.group, workspace=ws)
    torch.cuda.synchronize()
    return device_to_bits(y), need


# pairs of calls: the second smaller than the first (M, N, K, g, dtype, sym, bias)
PAIRS = [
    # decode with a K split (counters + partials in the scratch), then a
    # smaller split decode
    ((5, 1024, 20480, 128, O.BF16, False, True), (3, 264, 20480, 32, O.F16, True, False)),
    # prefill GEMM with a K split (128 tokens: few tiles), then a smaller one
    ((128, 4096, 4096, 128, O.BF16, False, False), (130, 200, 640, 64, O.F16, False, True)),
    # a plan with no split (no scratch), then a split decode
    ((1, 4096, 4096, 128, O.BF16, False, False), (5, 40, 9728, 64, O.BF16, False, True)),
    # the GEMM's 32-token tiles with a K split, then a smaller one
    ((40, 4096, 14336, 128, O.BF16, False, True), (17, 264, 2048, 64, O.F16, True, False)),
    # a GEMM plan with a tail launch (two kernels, no scratch), then a split decode
    ((1300, 28672, 1024, 128, O.BF16, False, True), (5, 40, 9728, 64, O.BF16, False, True)),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_linear_with_workspace(first, second):
    for i, (M, N, K, g, dt, sym, bias) in enumerate((first, second)):
        c = make_case(M, N, K, g, dt, sym, bias, seed=("noalloc", M, N, K, g, dt, sym, bias))
        d = DeviceCase(c)
        want, need = _with_workspace(d)
        assert need <= L.NOALLOC_SCRATCH_BYTES
        y = torch.empty((M, N), dtype=d.x.dtype, device="cuda")
        got = _noalloc(d, y)
        assert np.array_equal(got, want), f"call {i}: differs from w4a16_linear"
        assert_close(got, oracle_rows(c), dt, f"call {i} vs oracle")
        # and again: the scratch keeps the previous call's contents
        assert np.array_equal(_noalloc(d, y), want), f"call {i}, repeated"


def test_noalloc_refuses_beyond_its_scratch():
    # M = 256 on 131072 x 16384 splits K four ways into fp32 partial tiles
    # just above the scratch; refused before any launch (no data is read)
    M, N, K, g = 256, 16384, 131072, 128
    need = L.w4a16_workspace_size(M, N, K, g, O.BF16, True)
    assert need > L.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((N, K // 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((N, K // g), dtype=torch.bfloat16, device="cuda")
    zp = torch.zeros((N // 8, K // g), dtype=torch.int32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = B.lib.w4a16_linear_noalloc(x.data_ptr(), wq.data_ptr(), s.data_ptr(), zp.data_ptr(), None,
                                    y.data_ptr(), M, N, K, g, O.BF16,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 2 and "scratch" in L.w4a16_last_error()
