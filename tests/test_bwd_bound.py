"""The first-order rounding bound used by the backward parity tests
(tests/bwd_rounding.py), checked on the CPU: its unperturbed chain rule is
the oracle's backward, it is finite, and one full realization of the
kernels' bf16 roundings stays inside it on the short-row draws where the
gradients are worst conditioned."""

import numpy as np
import pytest

import oracle
from tests import bwd_rounding
from workloads import grad_output, prefill_inputs

LAM = np.array([0.35, 1.3])


def _case(T, D, seed):
    x = prefill_inputs(1, 2, T, D, "bf16", seed=seed)
    dout = grad_output((1, 2, T, 2 * D), seed=seed + 100)
    return x, dout


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("headnorm", [True, False])
def test_unperturbed_chain_is_the_oracle(causal, headnorm):
    x, dout = _case(5, 32, 3500)
    got = bwd_rounding.exact(x, LAM, dout, causal, headnorm, 0.6, 1e-5)
    ref = oracle.diff_attention_backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], LAM, dout,
                                         causal, headnorm, 0.6, 1e-5)
    for g, r in zip(got, ref[:5]):
        assert np.max(np.abs(g - r)) <= 1e-12 * max(1.0, float(np.max(np.abs(r))))


@pytest.mark.parametrize("T", [2, 3])
def test_simulated_rounding_within_bound(T):
    worst = 0.0
    for seed in range(3000, 3040):
        x, dout = _case(T, 64, seed)
        ref = bwd_rounding.exact(x, LAM, dout, True, True, 0.6, 1e-5)
        sim = bwd_rounding.simulated(x, LAM, dout, True, True, 0.6, 1e-5)
        bound = bwd_rounding.first_order_bound(x, LAM, dout, True, True, 0.6, 1e-5)
        for s, r, b in zip(sim, ref, bound):
            assert np.isfinite(b).all()
            err = np.abs(s - r)
            assert np.all(err <= b + 1e-12), seed
            worst = max(worst, float(np.max(err / np.maximum(b, 1e-300))))
    # the bound is not far above what rounding does: some element of some
    # draw reaches a sizeable part of it
    assert worst >= 0.1
