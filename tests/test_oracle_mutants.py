"""Planted mistakes in the oracle (on the CPU) must each trip a pin.

Each mutant replaces one internal step of the float64 oracle with a plausible
wrong version -- a wrong scale, an off-by-one or one-sided mask, transposed
operands, the wrong softmax axis, a flipped lambda sign, a dropped term -- and
the test asserts that at least one of the pin checks then fails.
"""

import math

import numpy as np
import pytest
import torch

import oracle.diffattn_oracle as od
from tests import oracle_pins

_REAL_ATTENTION = od.attention  # the real functions, wrapped by mutants below
_REAL_BACKWARD = od.diff_attention_backward
_REAL_LAMBDA_BACKWARD = od.reparam_lambda_backward
_REAL_V2 = od.diff_attention_v2
_REAL_SCORES = od._scores
_REAL_RAGGED = od.diff_attention_decode_ragged
_REAL_V2_DECODE = od.diff_attention_v2_decode



def _make_scores(scale_fn=None, mask_fn=None, transpose=False):
    def _scores(q, k, rows, causal, window=None):
        d = q.shape[-1]
        if rows is None:
            rows = np.arange(q.shape[0])
        s = (k[rows] @ q.T) if transpose else (q[rows] @ k.T)
        s = s * scale_fn(d)
        if causal:
            keys = np.arange(k.shape[0])
            s = np.where(mask_fn(keys[None, :], rows[:, None]), -np.inf, s)
            if window is not None:
                s = np.where(rows[:, None] - keys[None, :] >= window, -np.inf, s)
        return s
    return _scores


def _scores_window_off_by_one(q, k, rows, causal, window=None):
    # window read as i - W <= j <= i (one key too many)
    return _REAL_SCORES(q, k, rows, causal, None if window is None else window + 1)


def _ragged_off_by_one(q1, k1, q2, k2, v, lam, lengths):
    # one cached row too many per sequence (the row at position n_b)
    lengths = [min(int(n) + 1, od._f64(k1).shape[2]) for n in lengths]
    return _REAL_RAGGED(q1, k1, q2, k2, v, lam, lengths)


def _softmax_axis0(s):
    m = np.max(s, axis=0, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=0, keepdims=True)


def _softmax_no_norm(s):
    m = np.max(s, axis=-1, keepdims=True)
    return np.exp(s - m)


def _rows_branch1_mask_only(q1, k1, q2, k2, v, lam, causal, rows, row_block=512, window=None):
    q1, k1, q2, k2, v = (od._f64(t) for t in (q1, k1, q2, k2, v))
    rows = np.asarray(rows)
    a1 = od._softmax_rows(od._scores(q1, k1, rows, causal, window))
    a2 = od._softmax_rows(od._scores(q2, k2, rows, False))
    return (a1 - float(lam) * a2) @ v


def _rows_lam_on_a1(q1, k1, q2, k2, v, lam, causal, rows, row_block=512, window=None):
    q1, k1, q2, k2, v = (od._f64(t) for t in (q1, k1, q2, k2, v))
    rows = np.asarray(rows)
    a1 = od._softmax_rows(od._scores(q1, k1, rows, causal, window))
    a2 = od._softmax_rows(od._scores(q2, k2, rows, causal, window))
    return (float(lam) * a1 - a2) @ v


def _rows_swapped_branches(q1, k1, q2, k2, v, lam, causal, rows, row_block=512, window=None):
    q1, k1, q2, k2, v = (od._f64(t) for t in (q1, k1, q2, k2, v))
    rows = np.asarray(rows)
    a1 = od._softmax_rows(od._scores(q1, k2, rows, causal, window))
    a2 = od._softmax_rows(od._scores(q2, k1, rows, causal, window))
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


def _lambda_init_decay_02(layer):
    # decay rate 0.2 instead of 0.3
    return 0.8 - 0.6 * math.exp(-0.2 * (layer - 1))


def _lambda_init_amplitude_05(layer):
    # amplitude 0.5 instead of 0.6 (l = 1 would give 0.3)
    return 0.8 - 0.5 * math.exp(-0.3 * (layer - 1))


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


def _softmax_bwd_no_rowsum(a, da):
    return a * da


def _softmax_bwd_wrong_axis(a, da):
    return a * (da - np.sum(da * a, axis=-2, keepdims=True))


def _norm_bwd_no_projection(opre, dy, lambda_init, eps):
    g = 1.0 / np.sqrt(np.mean(opre * opre, axis=-1, keepdims=True) + eps)
    return (1.0 - lambda_init) * g * dy


def _norm_bwd_no_scale(opre, dy, lambda_init, eps):
    return od._head_rmsnorm_backward(opre, dy, 0.0, eps) if lambda_init else dy


def _bwd_dlam_sign(*args, **kw):
    g = _REAL_BACKWARD(*args, **kw)
    return (*g[:5], -g[5])


def _bwd_dk_reversed_keys(*args, **kw):
    # an index slip that writes key j's gradient to key T-1-j
    dq1, dk1, dq2, dk2, dv, dl = _REAL_BACKWARD(*args, **kw)
    return dq1, dk1[..., ::-1, :], dq2, dk2, dv, dl


def _bwd_dv_first_map_only(q1, k1, q2, k2, v, lam, dout, causal=True, headnorm=False, lambda_init=0.8,
                           eps=1e-5):
    g = _REAL_BACKWARD(q1, k1, q2, k2, v, 0.0, dout, causal, headnorm, lambda_init, eps)
    r = _REAL_BACKWARD(q1, k1, q2, k2, v, lam, dout, causal, headnorm, lambda_init, eps)
    return (*r[:4], g[4], r[5])


def _lambda_bwd_self(lq1, lk1, lq2, lk2, dlam):
    a, b, c, d = _REAL_LAMBDA_BACKWARD(lq1, lk1, lq2, lk2, dlam)
    return b, a, d, c


def _lambda_bwd_plus(lq1, lk1, lq2, lk2, dlam):
    a, b, c, d = _REAL_LAMBDA_BACKWARD(lq1, lk1, lq2, lk2, dlam)
    return a, b, -c, -d


def _v2_group_modulo(q1, q2, k, v, lam, causal=True, row_block=512):
    # differential head p reads KV head p % Hkv instead of p // (Hq / Hkv)
    hq, hkv = q1.shape[1], k.shape[1]
    idx = [p % hkv for p in range(hq)]
    kk = torch.as_tensor(np.asarray(od._f64(k))[:, idx])
    vv = torch.as_tensor(np.asarray(od._f64(v))[:, idx])
    return od.diff_attention(q1, kk, q2, kk, vv, lam, causal, row_block)


def _v2_first_query_twice(q1, q2, k, v, lam, causal=True, row_block=512):
    return _REAL_V2(q1, q1, k, v, lam, causal, row_block)


def _v2_decode_wrong_group(q1, q2, k, v, lam):
    return _REAL_V2_DECODE(q1, q2, torch.flip(torch.as_tensor(od._f64(k)), [1]),
                           torch.flip(torch.as_tensor(od._f64(v)), [1]), lam)


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
    "lambda_init_decay_02": ("lambda_init_schedule", _lambda_init_decay_02),
    "lambda_init_amplitude_05": ("lambda_init_schedule", _lambda_init_amplitude_05),
    "norm_without_scale": ("head_rmsnorm", _norm_no_scale),
    "norm_with_mean": ("head_rmsnorm", _norm_layernorm),
    "norm_eps_outside_sqrt": ("head_rmsnorm", _norm_eps_outside),
    "attention_mask_ignored": ("attention", _attention_mask_ignored),
    "attention_keys_as_values": ("attention", _attention_keys_as_values),
    "softmax_bwd_drops_rowsum": ("_softmax_backward_rows", _softmax_bwd_no_rowsum),
    "softmax_bwd_wrong_axis": ("_softmax_backward_rows", _softmax_bwd_wrong_axis),
    "norm_bwd_drops_projection": ("_head_rmsnorm_backward", _norm_bwd_no_projection),
    "norm_bwd_drops_scale": ("_head_rmsnorm_backward", _norm_bwd_no_scale),
    "bwd_dlambda_sign": ("diff_attention_backward", _bwd_dlam_sign),
    "bwd_dk_reversed_keys": ("diff_attention_backward", _bwd_dk_reversed_keys),
    "bwd_dv_first_map_only": ("diff_attention_backward", _bwd_dv_first_map_only),
    "lambda_bwd_own_vector": ("reparam_lambda_backward", _lambda_bwd_self),
    "lambda_bwd_second_sign": ("reparam_lambda_backward", _lambda_bwd_plus),
    "v2_group_modulo": ("diff_attention_v2", _v2_group_modulo),
    "window_off_by_one": ("_scores", _scores_window_off_by_one),
    "ragged_off_by_one": ("diff_attention_decode_ragged", _ragged_off_by_one),
    "v2_first_query_twice": ("diff_attention_v2", _v2_first_query_twice),
    "v2_decode_wrong_group": ("diff_attention_v2_decode", _v2_decode_wrong_group),
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
