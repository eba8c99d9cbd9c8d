"""bench.py host logic (no GPU): the single-GPU refusal and the algorithmic
byte count the decode roofline divides by."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_decode_bytes_counts_each_operand_once():
    # Llama-3.1-8B gate/up projection, one token, asymmetric g128: packed codes
    # N*K/2, bf16 scales 2*N*G, packed zero points 4*(N/8)*G, x 2*K, y 2*N
    N, K, g = 28672, 4096, 128
    G = K // g
    assert bench.decode_bytes(1, N, K, g) == N * K // 2 + 2 * N * G + 4 * (N // 8) * G + 2 * K + 2 * N
    # symmetric: no zero points; bias adds one act-dtype value per row; M scales x and y only
    assert bench.decode_bytes(1, N, K, g, asym=False) == N * K // 2 + 2 * N * G + 2 * K + 2 * N
    assert bench.decode_bytes(4, N, K, g, asym=False, bias=True) == \
        N * K // 2 + 2 * N * G + 4 * 2 * K + 4 * 2 * N + 2 * N
    # the four decode layers' mean: the per-launch figure the roofline uses
    total = sum(bench.decode_bytes(1, n, k, g) for (k, n) in bench.DECODE_LAYERS)
    assert total // len(bench.DECODE_LAYERS) == 28362752


def test_perf_compare_normalises_by_the_control():
    base = dict(control=dict(stream_read_GBs=5000.0, mfma_TFLOPs=1800.0),
                points_us={"llama8b_decode 4096x4096 M=1": 4.0, "llama8b_prefill 4096x6144 M=1920": 90.0})
    # 30 % slower on a box whose control is as fast: a regression
    now = dict(control=dict(stream_read_GBs=5000.0, mfma_TFLOPs=1800.0),
               points_us={"llama8b_decode 4096x4096 M=1": 5.2, "llama8b_prefill 4096x6144 M=1920": 90.0})
    res = {r["point"]: r for r in bench.perf_compare(base, now)}
    assert res["llama8b_decode 4096x4096 M=1"]["regressed"]
    assert not res["llama8b_prefill 4096x6144 M=1920"]["regressed"]
    # the same times on a box whose streaming read is 30 % slower: none
    now["control"]["stream_read_GBs"] = 5000.0 / 1.3
    res = {r["point"]: r for r in bench.perf_compare(base, now)}
    assert not res["llama8b_decode 4096x4096 M=1"]["regressed"]
    assert abs(res["llama8b_decode 4096x4096 M=1"]["normalized_ratio"] - 1.0) < 1e-3
    # prefill points are normalised by the MFMA control, not the stream read
    now["points_us"]["llama8b_prefill 4096x6144 M=1920"] = 120.0
    res = {r["point"]: r for r in bench.perf_compare(base, now)}
    assert res["llama8b_prefill 4096x6144 M=1920"]["regressed"]
    assert res["llama8b_prefill 4096x6144 M=1920"]["control"] == "mfma"


def test_prefill_profiles_pair_each_first_launch_with_its_tail():
    # The 4096 x 28672 prefill layer at M = 1920 runs as a first launch plus
    # a tail launch whose grid equals the 14336 x 4096 layer's: the summaries
    # must tell them apart by their tiles and add the two kernels of a call.
    layers = bench.profile_layers("prefill")
    big = next(l for l in layers if (l["K"], l["N"]) == (4096, 28672))
    other = next(l for l in layers if (l["K"], l["N"]) == (14336, 4096))
    assert big["tail_grid"] and big["tail_tile"] == (4, 2) and big["tile"] == (8, 2)
    assert big["tail_grid"] == other["grid"] and other["tile"] == (8, 2) and not other["tail_grid"]
    d = lambda grid, tile, t0, t1: dict(grid=grid, tile=tile, start=t0, end=t1)
    disp = [d(big["grid"], (8, 2), 0, 300), d(big["tail_grid"], (4, 2), 300, 370),
            d(other["grid"], (8, 2), 400, 600),
            d(big["grid"], (8, 2), 700, 1010), d(big["tail_grid"], (4, 2), 1010, 1085)]
    calls = bench._layer_calls(big, disp)
    assert [sum(x["end"] - x["start"] for x in c) for c in calls] == [370, 385]
    assert [len(c) for c in bench._layer_calls(other, disp)] == [1]
    assert bench._gemm_tile("gemm_kernel<1, 128, true, 4, 2, false>") == (4, 2)
    assert bench._gemm_tile("gemv_one_kernel<1, 128, true, 8, 1, false, 0>") is None
