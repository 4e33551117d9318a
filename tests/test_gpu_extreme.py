"""Parity on rows whose scores are all far below zero, or all far above it.

Queries and keys are drawn as c u + 0.2 z and -/+ c u + 0.2 z' (u a fixed
unit vector, z, z' standard normal), so every score q.k / sqrt(D) sits near
-/+ c^2 / sqrt(D) with a spread of a few units: around -300 or +300 in the
base-2 units the kernels work in (on the positive side the second half of
the keys scores another +300).  Softmax is invariant to a shift shared by a row
(paperleet "Differential Transformer Attention": each map is a row softmax),
so the maps, and the output, are those of ordinary scores; the float64 oracle
computes them exactly.  A kernel that scaled its running state by 2^(-m) with
the row's first block maximum m would overflow on the negative side (2^300
is beyond fp32) and turn the empty accumulators into NaN; on the positive
side a first exponential pass against a stale reference can overflow, which
the rescale path must repair."""

import math

import numpy as np
import pytest
import torch

import differential_attention_forward_amd as da
import oracle
from workloads import decode_inputs, prefill_inputs, v2_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCORE = 300.0  # target |score| in base-2 units
# fp32: a score s summed from D fp32 products carries an absolute rounding
# error of about 2^-24 sqrt(D) |s| in the exponent, ~3e-4 at |s| = 600 and
# D = 64 (the positive side's second half), i.e. a relative error of that
# size in every weight and a few 1e-4 on outputs of magnitude ~3: the usual
# 1e-4 assumes moderate scores.  bf16 keeps its usual bound.
TOL = {"fp32": 1e-4 + 3 * 2.0 ** -24 * 8 * (2 * SCORE), "bf16": 2e-2}


@pytest.fixture(params=[-1.0, 1.0], ids=["negative", "positive"])
def sign(request):
    """Sign of the scores: every test runs on both sides."""
    return request.param


def say(*a):
    print(*a, flush=True)


def _shift(q, k, D, dtype, sign):
    """q, k (any leading shape, last dim D) moved to scores near sign * SCORE."""
    c = math.sqrt(SCORE * math.sqrt(D) / math.log2(math.e))
    u = torch.ones(D, dtype=torch.float32) / math.sqrt(D)
    qs = (c * u + 0.2 * q.float())
    ks = (sign * c * u + 0.2 * k.float())
    if sign > 0:
        # keys of the second half score another +SCORE: the first block past
        # the step meets a reference ~2^300 too low, its first exponentials
        # overflow, and the rescale must recompute them
        ks[..., ks.shape[-2] // 2:, :] += c * u
    td = {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]
    return qs.to(td), ks.to(td)


def _extreme_prefill(B, H, T, D, dtype, seed, sign):
    x = prefill_inputs(B, H, T, D, dtype, seed=seed)
    x["q1"], x["k1"] = _shift(x["q1"], x["k1"], D, dtype, sign=sign)
    x["q2"], x["k2"] = _shift(x["q2"], x["k2"], D, dtype, sign=sign)
    return x


def _err(gpu, ref):
    g = gpu.double().cpu().numpy()
    assert np.isfinite(g).all(), "non-finite output"
    return float(np.max(np.abs(g - ref)))


def _dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


@pytest.mark.parametrize("dtype,D,causal,headnorm", [
    ("bf16", 64, True, True),     # one-map waves, early fragment reads
    ("bf16", 64, True, False),
    ("bf16", 64, False, True),    # full attention, two maps per wave
    ("bf16", 32, True, True),     # two maps per wave
    ("bf16", 128, False, True),   # D = 128, reads one MFMA ahead
    ("fp32", 64, True, True),
])
def test_prefill_extreme_scores(dtype, D, causal, headnorm, sign):
    x = _extreme_prefill(1, 2, 300, D, dtype, seed=7300 + D, sign=sign)
    lam = torch.tensor([0.3, 1.2], dtype=torch.float32)
    say(f"extreme prefill sign={sign:+.0f} {dtype} D={D} causal={causal} headnorm={headnorm}")
    xd = _dev(x)
    out = da.diffattn_fwd(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV), causal=causal,
                          headnorm=headnorm, lambda_init=0.8, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.diff_attention(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam.numpy(), causal)
    if headnorm:
        ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
    err = _err(out, ref)
    say(f"  max err {err:.3e}")
    assert err <= TOL[dtype], err


def test_long_causal_rows_extreme_scores(sign):
    # T > 4096: the ping-pong kernel; sampled rows against the oracle
    T = 4097
    x = _extreme_prefill(1, 2, T, 64, "bf16", seed=7310, sign=sign)
    lam = torch.tensor([0.5, -0.2], dtype=torch.float32)
    say("extreme prefill, ping-pong kernel, T=4097")
    xd = _dev(x)
    out = da.diffattn_fwd(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV), causal=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(40), np.arange(T - 40, T),
                                     np.random.default_rng(7310).choice(T, 100, replace=False)]))
    for h in range(2):
        ref = oracle.diff_attention_rows(x["q1"][0, h], x["k1"][0, h], x["q2"][0, h], x["k2"][0, h],
                                         x["v"][0, h], float(lam[h]), True, rows)
        err = _err(out[0, h, rows], ref)
        say(f"  h={h} max err {err:.3e}")
        assert err <= TOL["bf16"], (h, err)


def test_window_and_attention_extreme_scores(sign):
    x = _extreme_prefill(1, 2, 1000, 64, "bf16", seed=7320, sign=sign)
    lam = torch.tensor([0.6, 0.9], dtype=torch.float32)
    xd = _dev(x)
    say("extreme window prefill, W=256")
    out = da.diffattn_fwd_window(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV), 256,
                                 headnorm=True, lambda_init=0.8, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.head_rmsnorm(
        oracle.diff_attention(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam.numpy(), True, window=256),
        0.8, 1e-5)
    err = _err(out, ref)
    say(f"  max err {err:.3e}")
    assert err <= TOL["bf16"], err
    for D in (64, 128):
        say(f"extreme standard attention D={D}")
        y = _extreme_prefill(1, 2, 300, D, "bf16", seed=7330 + D, sign=sign)
        # values of the usual scale (the shifted queries are ~5 in size)
        v = y["v"][..., :D].contiguous()
        yd = _dev(y)
        out = da.diffattn_attention_fwd(yd["q1"], yd["k1"], v.to(DEV), causal=True)
        torch.cuda.synchronize()
        err = _err(out, oracle.attention(y["q1"], y["k1"], v, True))
        say(f"  max err {err:.3e}")
        assert err <= TOL["bf16"], (D, err)


def test_training_forward_extreme_scores(sign):
    x = _extreme_prefill(1, 2, 300, 64, "bf16", seed=7340, sign=sign)
    lam = torch.tensor([0.4, 1.1], dtype=torch.float32)
    xd = _dev(x)
    say("extreme training forward")
    out, saved = da.diffattn_fwd_train(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV),
                                       causal=True, headnorm=True, lambda_init=0.8, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.head_rmsnorm(
        oracle.diff_attention(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam.numpy(), True), 0.8, 1e-5)
    err = _err(out, ref)
    say(f"  max err {err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_extreme_scores(dtype, sign):
    B, H, L, D = 2, 3, 3000, 64
    x = decode_inputs(B, H, L, D, dtype, seed=7350)
    x["q1"], x["k1"] = _shift(x["q1"], x["k1"], D, dtype, sign=sign)
    x["q2"], x["k2"] = _shift(x["q2"], x["k2"], D, dtype, sign=sign)
    lam = torch.tensor([0.2, 0.7, 1.3], dtype=torch.float32)
    xd = _dev(x)
    say(f"extreme decode {dtype}")
    out = da.diffattn_decode(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV), num_splits=7)
    torch.cuda.synchronize()
    err = _err(out, oracle.diff_attention_decode(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam.numpy()))
    say(f"  max err {err:.3e}")
    assert err <= TOL[dtype], err


def test_v2_extreme_scores(sign):
    D = 128
    x = v2_inputs(1, 8, 2, 300, D, "bf16", seed=7360, lam_uniform=(0.2, 0.8))
    x["q1"], k = _shift(x["q1"], x["k"], D, "bf16", sign=sign)
    x["q2"], _ = _shift(x["q2"], x["k"], D, "bf16", sign=sign)
    x["k"] = k
    xd = _dev(x)
    say("extreme V2 prefill")
    out = da.diffattn_v2_fwd(xd["q1"], xd["q2"], xd["k"], xd["v"], xd["lam"], causal=True)
    torch.cuda.synchronize()
    err = _err(out, oracle.diff_attention_v2(x["q1"], x["q2"], x["k"], x["v"], x["lam"].numpy(), True))
    say(f"  max err {err:.3e}")
    assert err <= TOL["bf16"], err
    y = v2_inputs(2, 8, 2, 3000, D, "bf16", seed=7361, decode=True, lam_uniform=(0.2, 0.8))
    y["q1"], k = _shift(y["q1"], y["k"], D, "bf16", sign=sign)
    y["q2"], _ = _shift(y["q2"], y["k"], D, "bf16", sign=sign)
    y["k"] = k
    yd = _dev(y)
    say("extreme V2 decode")
    out = da.diffattn_v2_decode(yd["q1"], yd["q2"], yd["k"], yd["v"], yd["lam"])
    torch.cuda.synchronize()
    err = _err(out, oracle.diff_attention_v2_decode(y["q1"], y["q2"], y["k"], y["v"], y["lam"].numpy()))
    say(f"  max err {err:.3e}")
    assert err <= TOL["bf16"], err


def test_backward_extreme_scores(sign):
    # The backward forms probabilities from the saved log-sum-exp.  K's large
    # shared component (|c u| ~ 41) multiplies the bf16 rounding of dS, whose
    # rows cancel only in exact arithmetic, so dQ is held to the backward
    # tests' derived first-order rounding bound (tests/bwd_rounding.py),
    # which needs short sequences: T = 4 (the second half, rows 2 and 3,
    # carrying the positive side's step).
    from tests import bwd_rounding
    from tests.test_gpu_backward import check_grads, dlambda_term_rss
    from workloads import grad_output
    T = 4
    x = _extreme_prefill(1, 2, T, 64, "bf16", seed=7370, sign=sign)
    lam = torch.tensor([0.4, 1.1], dtype=torch.float32)
    dout = grad_output((1, 2, T, 128), seed=7371)
    xd = _dev(x)
    say(f"extreme backward sign={sign:+.0f}")
    out, saved = da.diffattn_fwd_train(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV),
                                       causal=True, headnorm=True, lambda_init=0.8, eps=1e-5)
    g = da.diffattn_bwd(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV), dout.to(DEV), saved,
                        causal=True, headnorm=True, lambda_init=0.8, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.diff_attention_backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam.numpy(), dout,
                                         True, True, 0.8, 1e-5)
    rss = dlambda_term_rss(x, lam.numpy(), dout, True, True, 0.8, 1e-5)
    bound = bwd_rounding.first_order_bound(x, lam.numpy(), dout, True, True, 0.8, 1e-5)
    check_grads(g, ref, f"  extreme T={T} sign={sign:+.0f}", rss, bound)
