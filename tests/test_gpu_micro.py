"""The microbenchmarks behind the measured ceilings in bench.py's output:
each runs, returns finite values, and reads a known property of gfx950
(a 32x32x16 bf16 MFMA occupies a SIMD's matrix pipe for 32 clocks; the
shader clock is at most 2.4 GHz; streaming HBM stays under 8 TB/s; an LDS
read serves at most 256 bytes per clock per CU)."""

import math

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def micro():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from differential_attention_forward_amd import micro

    micro.lib()
    return micro


def test_mfma_issue_interval_and_clock(micro):
    r = micro.mfma(iters=8000, reps=2)
    assert 0.8 < r["clock_ghz"] <= 2.5, r
    assert 30.0 <= r["cycles_per_mfma_per_simd"] <= 40.0, r
    assert r["tflops"] <= 2.5e3 * 1.02, r


def test_streaming_bandwidths(micro):
    for name, fn in (("read", micro.hbm_read), ("copy", micro.hbm_copy), ("dma", micro.lds_dma)):
        r = fn(nbytes=1 << 30, reps=2)
        print(name, r, flush=True)
        assert math.isfinite(r["gbs"]) and 1000.0 < r["gbs"] < 8000.0, (name, r)


@pytest.mark.parametrize("transposing", [False, True])
def test_lds_read_rate(micro, transposing):
    r = micro.lds_read(transposing, iters=4000, reps=2)
    assert 32.0 < r["bytes_per_clk_cu"] <= 256.0, r


def test_valu_beside_mfma(micro):
    add = (micro.valu(0, False, iters=1000), micro.valu(0, True, iters=1000))
    dot = (micro.valu(1, False, iters=1000), micro.valu(1, True, iters=1000))
    print("add", add, "dot2c", dot, flush=True)
    assert all(3.0 < x < 200.0 for x in add + dot)
