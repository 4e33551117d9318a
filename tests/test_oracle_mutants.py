"""Planted mistakes in the oracle (on the CPU) must each trip a pin.

Each mutant replaces one internal step of the float64 oracle with a plausible
wrong version -- a wrong scale, an off-by-one or one-sided mask, transposed
operands, the wrong softmax axis, a flipped lambda sign, a dropped term -- and
the test asserts that at least one of the pin checks then fails.
"""

import math

import numpy as np
import pytest

import oracle.diffattn_oracle as od
from tests import oracle_pins

_REAL_ATTENTION = od.attention  # the real function, wrapped by two mutants below



def _make_scores(scale_fn=None, mask_fn=None, transpose=False):
    def _scores(q, k, rows, causal):
        d = q.shape[-1]
        if rows is None:
            rows = np.arange(q.shape[0])
        s = (k[rows] @ q.T) if transpose else (q[rows] @ k.T)
        s = s * scale_fn(d)
        if causal:
            keys = np.arange(k.shape[0])
            s = np.where(mask_fn(keys[None, :], rows[:, None]), -np.inf, s)
        return s
    return _scores


def _softmax_axis0(s):
    m = np.max(s, axis=0, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=0, keepdims=True)


def _softmax_no_norm(s):
    m = np.max(s, axis=-1, keepdims=True)
    return np.exp(s - m)


def _rows_branch1_mask_only(q1, k1, q2, k2, v, lam, causal, rows, row_block=512):
    q1, k1, q2, k2, v = (od._f64(t) for t in (q1, k1, q2, k2, v))
    rows = np.asarray(rows)
    a1 = od._softmax_rows(od._scores(q1, k1, rows, causal))
    a2 = od._softmax_rows(od._scores(q2, k2, rows, False))
    return (a1 - float(lam) * a2) @ v


def _rows_lam_on_a1(q1, k1, q2, k2, v, lam, causal, rows, row_block=512):
    q1, k1, q2, k2, v = (od._f64(t) for t in (q1, k1, q2, k2, v))
    rows = np.asarray(rows)
    a1 = od._softmax_rows(od._scores(q1, k1, rows, causal))
    a2 = od._softmax_rows(od._scores(q2, k2, rows, causal))
    return (float(lam) * a1 - a2) @ v


def _rows_swapped_branches(q1, k1, q2, k2, v, lam, causal, rows, row_block=512):
    q1, k1, q2, k2, v = (od._f64(t) for t in (q1, k1, q2, k2, v))
    rows = np.asarray(rows)
    a1 = od._softmax_rows(od._scores(q1, k2, rows, causal))
    a2 = od._softmax_rows(od._scores(q2, k1, rows, causal))
    return (a1 - float(lam) * a2) @ v


def _signed_plus(a1, a2, lam):
    lam = od._f64(lam)
    if lam.ndim == 1:
        lam = lam[:, None, None]
    return a1 + lam * a2


def _lambda_plus(lq1, lk1, lq2, lk2, lambda_init):
    a, b, c, d = (od._f64(t) for t in (lq1, lk1, lq2, lk2))
    return np.exp(np.sum(a * b, -1)) + np.exp(np.sum(c * d, -1)) + lambda_init


def _lambda_no_init(lq1, lk1, lq2, lk2, lambda_init):
    a, b, c, d = (od._f64(t) for t in (lq1, lk1, lq2, lk2))
    return np.exp(np.sum(a * b, -1)) - np.exp(np.sum(c * d, -1))


def _lambda_init_zero_based(layer):
    return 0.8 - 0.6 * math.exp(-0.3 * layer)


def _norm_no_scale(o, lambda_init, eps):
    o = od._f64(o)
    return o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps)


def _norm_layernorm(o, lambda_init, eps):
    o = od._f64(o)
    o = o - o.mean(-1, keepdims=True)
    return o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps) * (1 - lambda_init)


def _norm_eps_outside(o, lambda_init, eps):
    o = od._f64(o)
    return o / (np.sqrt(np.mean(o * o, -1, keepdims=True)) + eps) * (1 - lambda_init)


def _attention_mask_ignored(q, k, v, causal=True, row_block=512):
    return _REAL_ATTENTION(q, k, v, False, row_block)


def _attention_keys_as_values(q, k, v, causal=True, row_block=512):
    k64 = od._f64(k)
    return _REAL_ATTENTION(q, k, np.concatenate([k64] * (od._f64(v).shape[-1] // k64.shape[-1]), -1),
                                    causal, row_block)


MUTANTS = {
    "scale_1_over_sqrt_2d": ("_scores", _make_scores(lambda d: 1 / math.sqrt(2 * d), lambda j, i: j > i)),
    "scale_missing": ("_scores", _make_scores(lambda d: 1.0, lambda j, i: j > i)),
    "scale_1_over_d": ("_scores", _make_scores(lambda d: 1.0 / d, lambda j, i: j > i)),
    "mask_excludes_diagonal": ("_scores", _make_scores(lambda d: 1 / math.sqrt(d), lambda j, i: j >= i)),
    "mask_anticausal": ("_scores", _make_scores(lambda d: 1 / math.sqrt(d), lambda j, i: j < i)),
    "mask_missing": ("_scores", _make_scores(lambda d: 1 / math.sqrt(d), lambda j, i: j < 0)),
    "operands_transposed": ("_scores", _make_scores(lambda d: 1 / math.sqrt(d), lambda j, i: j > i, True)),
    "softmax_wrong_axis": ("_softmax_rows", _softmax_axis0),
    "softmax_not_normalised": ("_softmax_rows", _softmax_no_norm),
    "mask_one_branch_only": ("diff_attention_rows", _rows_branch1_mask_only),
    "lambda_on_first_map": ("diff_attention_rows", _rows_lam_on_a1),
    "branches_crossed": ("diff_attention_rows", _rows_swapped_branches),
    "signed_map_plus": ("signed_map", _signed_plus),
    "lambda_plus": ("reparam_lambda", _lambda_plus),
    "lambda_drops_init": ("reparam_lambda", _lambda_no_init),
    "lambda_init_zero_based": ("lambda_init_schedule", _lambda_init_zero_based),
    "norm_without_scale": ("head_rmsnorm", _norm_no_scale),
    "norm_with_mean": ("head_rmsnorm", _norm_layernorm),
    "norm_eps_outside_sqrt": ("head_rmsnorm", _norm_eps_outside),
    "attention_mask_ignored": ("attention", _attention_mask_ignored),
    "attention_keys_as_values": ("attention", _attention_keys_as_values),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(od, attr, fn)
    import oracle
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
