"""Float64 CPU oracle for multi-head differential attention (forward only).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The GPU path never routes through
it, and it shares no code, tables or helpers with the HIP library.

What it computes is the plain definition, written out step by step in float64,
with every attention map materialised row by row (no streaming softmax, no
tiling of the key axis, no fusion):

    S1 = Q1 K1^T / sqrt(D) + M,   S2 = Q2 K2^T / sqrt(D) + M
    A1 = softmax_rows(S1),        A2 = softmax_rows(S2)
    O  = (A1 - lam * A2) V

  - paperleet "Differential Transformer Attention", the displayed equation for
    A1, A2 and O, and the sentence defining the causal mask M (0 on allowed
    keys, -inf on future keys, applied to both branches, softmax over keys).
  - aifetchly "Differential Transformer: Canceling LLM Attention Noise",
    section 1 (DiffAttn formulation) and the numerically stable softmax of its
    "Step 1" code (subtract the row maximum, exponentiate, divide by the sum).

lam = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init
  - aifetchly page, section 3 (re-parameterisation of lambda); paperleet page,
    the scalar parameterisation equation and "Formula and conventions".

lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l - 1)), layers counted from 1
  - aifetchly page, section 3; paperleet page, "Formula and conventions".

Optional per-head norm: RMS over the 2D output channels of each token, then a
constant x (1 - lambda_init).
  - aifetchly page, section 4 (per-head normalisation, then the (1 - lambda_init)
    multiplier); the French lesson page, "Le problème" and "V1 contre V2", names
    the per-head norm of V1 as RMSNorm.  Reading taken: RMSNorm without mean
    subtraction and without an affine weight (identity at initialisation), with
    an explicit eps, and the (1 - lambda_init) factor applied only together
    with the norm (the paperleet page returns the aggregate *before* the norm
    and its fixed multiplier).

Decode: one query row per (batch, head) against all L cached keys, no mask;
the same steps as above with T_q = 1.

DIFF V2 (the French lesson page, "V1 contre V2"): twice the query heads, the
baseline's KV heads and head width, one K and one V per group of differential
heads shared by both maps, no per-head norm.  Same steps per differential head
with K1 = K2 = K_g and V = V_g, g = p // (Hq / Hkv).

Readings where the pages are loose (all recorded in the design notes):
  - softmax scale is 1/sqrt(D) with D the width of Q1/K1 (not 2D);
  - lambda is not clamped and may be negative or exceed 1;
  - lambda may differ per head (the French page: "par tête"); a per-layer
    scalar is the case of all heads equal.

Query rows may be processed in blocks purely to bound memory; every row's
two score rows and softmax rows are materialised whole, so blocking changes no
arithmetic.

Pins: every function here is pinned by tests that do not re-type its formula
(see ``tests/test_oracle_pins.py``): the page's printed worked example, the
lambda = 0 reduction to a library attention routine, cancellation of identical
maps at lambda = 1, row sums of 1 - lambda, the exact (1 - lambda) response to a
value offset, the causal first row, the lambda_init values, a library RMS norm,
and an independent pure-Python scalar implementation on tiny inputs.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lambda_init_schedule",
    "reparam_lambda",
    "score_maps",
    "signed_map",
    "diff_attention",
    "diff_attention_rows",
    "head_rmsnorm",
    "diff_attention_decode",
    "diff_attention_decode_ragged",
    "attention",
    "diff_attention_v2",
    "diff_attention_v2_decode",
    "diff_attention_backward",
    "diff_attention_backward_dq_rows",
    "reparam_lambda_backward",
]


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or torch tensor (fp32/bf16) to float64."""
    if hasattr(x, "detach"):  # torch tensor: go through float32 (exact for bf16)
        x = x.detach().to("cpu")
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def lambda_init_schedule(layer: int) -> float:
    """lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l - 1)), l = 1, 2, ...

    aifetchly page, section 3 (depth-dependent initialisation); paperleet page,
    "Formula and conventions" (layers start at 1).
    """
    if layer < 1:
        raise ValueError("layers are counted from 1")
    return 0.8 - 0.6 * math.exp(-0.3 * (layer - 1))


def reparam_lambda(lq1, lk1, lq2, lk2, lambda_init: float) -> np.ndarray:
    """lam = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init, in float64.

    aifetchly page, section 3; paperleet page, scalar parameterisation.
    Vectors of shape [Dl] give a 0-d result; shape [H, Dl] gives one lambda per
    head (the French page: lambda is a learnable scalar per head).
    """
    a, b, c, d = (_f64(t) for t in (lq1, lk1, lq2, lk2))
    dot1 = np.sum(a * b, axis=-1)
    dot2 = np.sum(c * d, axis=-1)
    return np.exp(dot1) - np.exp(dot2) + float(lambda_init)


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis: subtract the row max, exp, normalise.

    aifetchly page, "Step 1" (stable softmax); the French page, "Étape 1".
    Entries equal to -inf (masked keys) become exactly 0.
    """
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _scores(q: np.ndarray, k: np.ndarray, rows: np.ndarray | None, causal: bool,
            window: int | None = None) -> np.ndarray:
    """S = Q K^T / sqrt(D) for the given query rows, with the causal mask.

    paperleet page: scaled scores, M = -inf on keys j > i (future positions).
    q: [Tq_all, D], k: [Tk, D]; rows: indices into q (None = all rows, which are
    then positions 0..Tq-1).

    ``window`` (with causal): sliding-window mask, the French lesson page's
    hybrid stacks ("attention des fenêtres coulissantes").  Reading taken: row
    i sees the W most recent positions including itself, keys j with
    i - W < j <= i; M = -inf on every other key.
    """
    d = q.shape[-1]
    if rows is None:
        rows = np.arange(q.shape[0])
    s = (q[rows] @ k.T) / math.sqrt(d)
    if causal:
        keys = np.arange(k.shape[0])
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
        if window is not None:
            s = np.where(rows[:, None] - keys[None, :] >= window, -np.inf, s)
    return s


def score_maps(q1, k1, q2, k2, causal: bool):
    """Return the two materialised softmax maps A1, A2 (float64).

    Shapes: q*, k* are [..., T, D]; returns [..., T, T] each.  Only meant for
    small T (the maps are T x T).
    """
    q1, k1, q2, k2 = (_f64(t) for t in (q1, k1, q2, k2))
    lead = q1.shape[:-2]
    t = q1.shape[-2]
    a1 = np.empty(lead + (t, k1.shape[-2]))
    a2 = np.empty_like(a1)
    for idx in np.ndindex(*lead):
        a1[idx] = _softmax_rows(_scores(q1[idx], k1[idx], None, causal))
        a2[idx] = _softmax_rows(_scores(q2[idx], k2[idx], None, causal))
    return a1, a2


def signed_map(a1: np.ndarray, a2: np.ndarray, lam) -> np.ndarray:
    """A = A1 - lam * A2 (paperleet page equation for O; aifetchly section 2).

    ``lam`` broadcasts over the leading axes: a scalar, or one value per head
    for maps shaped [B, H, T, T].
    """
    lam = _f64(lam)
    if lam.ndim == 1:
        lam = lam[:, None, None]
    return a1 - lam * a2


def _lam_per_head(lam, h: int) -> np.ndarray:
    lam = _f64(lam)
    if lam.ndim == 0:
        return np.full(h, float(lam))
    if lam.shape != (h,):
        raise ValueError(f"lambda must be a scalar or have shape [{h}]")
    return lam


def diff_attention_rows(q1, k1, q2, k2, v, lam, causal: bool, rows, row_block: int = 512,
                        window: int | None = None):
    """O rows (A1 - lam A2) V for the selected query rows of one (b, h) slice.

    q*, k*: [T, D]; v: [T, 2D]; lam: python/0-d scalar; rows: 1-D int array of
    query positions.  Returns [len(rows), 2D] float64.  Each selected row's two
    score rows over all keys are materialised whole; ``row_block`` only bounds
    how many rows are held at once.  ``window``: sliding-window mask (causal).
    """
    q1, k1, q2, k2, v = (_f64(t) for t in (q1, k1, q2, k2, v))
    lam = float(_f64(lam))
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], v.shape[-1]))
    for s in range(0, rows.shape[0], row_block):
        r = rows[s:s + row_block]
        a1 = _softmax_rows(_scores(q1, k1, r, causal, window))
        a2 = _softmax_rows(_scores(q2, k2, r, causal, window))
        out[s:s + row_block] = (a1 - lam * a2) @ v
    return out


def diff_attention(q1, k1, q2, k2, v, lam, causal: bool = True, row_block: int = 512,
                   window: int | None = None):
    """O = (softmax(Q1K1^T/sqrt(D)+M) - lam softmax(Q2K2^T/sqrt(D)+M)) V.

    paperleet page: q*, k* are [B, H, T, D], v is [B, H, T, 2D], result
    [B, H, T, 2D] (the value aggregate before any head normalisation).
    ``lam`` is a scalar or one value per head [H].  float64 result.
    ``window``: sliding-window mask (with causal), see ``_scores``.
    """
    q1, k1, q2, k2, v = (_f64(t) for t in (q1, k1, q2, k2, v))
    b, h, t, _ = q1.shape
    lam_h = _lam_per_head(lam, h)
    out = np.empty((b, h, t, v.shape[-1]))
    rows = np.arange(t)
    for bi in range(b):
        for hi in range(h):
            out[bi, hi] = diff_attention_rows(
                q1[bi, hi], k1[bi, hi], q2[bi, hi], k2[bi, hi], v[bi, hi],
                lam_h[hi], causal, rows, row_block, window)
    return out


def head_rmsnorm(o, lambda_init: float, eps: float) -> np.ndarray:
    """Y_t = O_t / sqrt(mean_c O_t,c^2 + eps) * (1 - lambda_init).

    Per token, over the 2D channels of one head (aifetchly page, section 4:
    normalise each head separately, then the constant (1 - lambda_init)
    multiplier; the French page names V1's per-head norm as RMSNorm).
    """
    o = _f64(o)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + float(eps)) * (1.0 - float(lambda_init))


def diff_attention_decode(q1, k1, q2, k2, v, lam):
    """Decode: one query per (b, h) against all L cached keys, no mask.

    q*: [B, H, D]; k*: [B, H, L, D]; v: [B, H, L, 2D]; lam scalar or [H].
    Returns [B, H, 2D] float64.  Same definition as ``diff_attention`` with a
    single query row that sees every cached key (the French page, "V1 contre
    V2": decoding reads the value cache; one read of V serves both maps).
    """
    q1, q2 = _f64(q1), _f64(q2)
    b, h, _ = q1.shape
    lam_h = _lam_per_head(lam, h)
    out = np.empty((b, h, v.shape[-1]))
    for bi in range(b):
        for hi in range(h):
            k1s, k2s, vs = _f64(k1[bi, hi]), _f64(k2[bi, hi]), _f64(v[bi, hi])
            out[bi, hi] = diff_attention_rows(
                q1[bi, hi][None, :], k1s, q2[bi, hi][None, :], k2s, vs,
                lam_h[hi], False, np.array([0]))[0]
    return out


def diff_attention_decode_ragged(q1, k1, q2, k2, v, lam, lengths):
    """Decode against caches of different filled lengths per sequence.

    Same as ``diff_attention_decode`` with sequence b seeing only its first
    lengths[b] cached rows (the French page's serving setting: each sequence
    in a decode batch has its own context length).  Reading taken: a length of
    0 leaves no key to attend to and gives a zero output row.
    q*: [B, H, D]; k*: [B, H, L, D]; v: [B, H, L, 2D]; lengths: [B] ints in
    [0, L].  Returns [B, H, 2D] float64.
    """
    q1, q2 = _f64(q1), _f64(q2)
    b, h, _ = q1.shape
    lengths = [int(x) for x in np.asarray(lengths).reshape(-1)]
    out = np.zeros((b, h, v.shape[-1]))
    for bi in range(b):
        n = lengths[bi]
        if n <= 0:
            continue
        out[bi] = diff_attention_decode(q1[bi:bi + 1], _f64(k1[bi:bi + 1, :, :n]), q2[bi:bi + 1],
                                        _f64(k2[bi:bi + 1, :, :n]), _f64(v[bi:bi + 1, :, :n]), lam)[0]
    return out


def _group_of(hq: int, hkv: int) -> int:
    if hkv < 1 or hq % hkv:
        raise ValueError("query heads must be a whole multiple of KV heads")
    return hq // hkv


def diff_attention_v2(q1, q2, k, v, lam, causal: bool = True, row_block: int = 512):
    """DIFF V2 forward with grouped KV heads, float64.

    The French lesson page, "V1 contre V2": V2 doubles the query heads and
    keeps the KV heads of the baseline, at the baseline head width; the two
    queries of a differential head read the same K and V, so each map is
    ordinary attention over that shared cache and the difference is taken
    after attention; the per-head norm of V1 is gone.  The page's exercise
    pairs this with grouped KV heads (8 KV heads for 32 query heads).
    Reading taken: differential head p (of Hq) reads KV head p // (Hq / Hkv),
    the grouping of grouped-query attention.

    q1, q2: [B, Hq, T, D]; k, v: [B, Hkv, T, D]; lam scalar or [Hq].
    O_p = (softmax(Q1_p K_g^T/sqrt(D) + M) - lam_p softmax(Q2_p K_g^T/sqrt(D) + M)) V_g,
    returned as [B, Hq, T, D].
    """
    q1, q2, k, v = (_f64(t) for t in (q1, q2, k, v))
    b, hq, t, _ = q1.shape
    grp = _group_of(hq, k.shape[1])
    lam_h = _lam_per_head(lam, hq)
    out = np.empty((b, hq, t, v.shape[-1]))
    rows = np.arange(t)
    for bi in range(b):
        for p in range(hq):
            g = p // grp
            out[bi, p] = diff_attention_rows(q1[bi, p], k[bi, g], q2[bi, p], k[bi, g], v[bi, g],
                                             lam_h[p], causal, rows, row_block)
    return out


def diff_attention_v2_decode(q1, q2, k, v, lam):
    """DIFF V2 decode: one query pair per (b, differential head) against all L
    cached rows of its KV head, no mask.

    q1, q2: [B, Hq, D]; k, v: [B, Hkv, L, D]; lam scalar or [Hq].  Returns
    [B, Hq, D].  The same steps as ``diff_attention_v2`` for one query row that
    sees every key.
    """
    q1, q2 = _f64(q1), _f64(q2)
    b, hq, _ = q1.shape
    grp = _group_of(hq, k.shape[1])
    lam_h = _lam_per_head(lam, hq)
    out = np.empty((b, hq, v.shape[-1]))
    for bi in range(b):
        for p in range(hq):
            g = p // grp
            ks, vs = _f64(k[bi, g]), _f64(v[bi, g])
            out[bi, p] = diff_attention_rows(q1[bi, p][None, :], ks, q2[bi, p][None, :], ks, vs,
                                             lam_h[p], False, np.array([0]))[0]
    return out


def attention(q, k, v, causal: bool = True, row_block: int = 512):
    """Standard softmax attention softmax(Q K^T / sqrt(D) + M) V, float64.

    The comparison model of the glossary page (a Transformer of the same size;
    the paperleet page: lambda = 0 leaves ordinary attention).  q, k: [B, H, T,
    D]; v: [B, H, T, Dv]; the same scores, mask and row softmax as above, one
    map.  Rows are processed in blocks only to bound memory.
    """
    q, k, v = (_f64(t) for t in (q, k, v))
    b, h, t, _ = q.shape
    out = np.empty((b, h, t, v.shape[-1]))
    for bi in range(b):
        for hi in range(h):
            for s0 in range(0, t, row_block):
                r = np.arange(s0, min(t, s0 + row_block))
                out[bi, hi, r] = _softmax_rows(_scores(q[bi, hi], k[bi, hi], r, causal)) @ v[bi, hi]
    return out


def _softmax_backward_rows(a: np.ndarray, da: np.ndarray) -> np.ndarray:
    """Vector-Jacobian product of the row softmax: given A = softmax(S) by rows
    and dL/dA, dL/dS = A * (dA - rowsum(dA * A)).  Masked entries have A = 0 and
    so get zero gradient."""
    return a * (da - np.sum(da * a, axis=-1, keepdims=True))


def _head_rmsnorm_backward(opre: np.ndarray, dy: np.ndarray, lambda_init: float, eps: float) -> np.ndarray:
    """Vector-Jacobian product of Y = X g (1 - lambda_init), g = (mean_c X^2 + eps)^-1/2,
    per row over the last axis:  dX = (1 - lambda_init) g (dY - X g^2 mean_c(dY X))."""
    g = 1.0 / np.sqrt(np.mean(opre * opre, axis=-1, keepdims=True) + float(eps))
    return (1.0 - float(lambda_init)) * g * (dy - opre * g * g * np.mean(dy * opre, axis=-1, keepdims=True))


def diff_attention_backward(q1, k1, q2, k2, v, lam, dout, causal: bool = True, headnorm: bool = False,
                            lambda_init: float = 0.8, eps: float = 1e-5):
    """Gradients of the forward above (with the optional head norm) given dL/dOut.

    The paperleet page asks for gradients through both Q/K branches, the value
    and the coefficient.  Written out from the chain rule, one (b, h) at a time,
    maps materialised:
        O1 = A1 V, O2 = A2 V, Opre = O1 - lam O2, Out = Opre or norm(Opre)
        dOpre = dOut, or the head-norm vector-Jacobian product of dOut
        dV = A1^T dOpre - lam A2^T dOpre
        dA1 = dOpre V^T,  dA2 = -lam dOpre V^T
        dS1, dS2 = row-softmax vector-Jacobian products of dA1, dA2
        dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D)     (per map)
        dlam = -sum over (b, t, c) of dOpre O2           (one lambda per head)
    Returns dq1, dk1, dq2, dk2, dv ([B, H, ...] float64) and dlam ([H]).
    """
    q1, k1, q2, k2, v, dout = (_f64(t) for t in (q1, k1, q2, k2, v, dout))
    b, h, t, d = q1.shape
    lam_h = _lam_per_head(lam, h)
    c = 1.0 / math.sqrt(d)
    dq1, dk1, dq2, dk2, dv = (np.empty_like(x) for x in (q1, k1, q2, k2, v))
    dlam = np.zeros(h)
    for bi in range(b):
        for hi in range(h):
            lm = lam_h[hi]
            a1 = _softmax_rows(_scores(q1[bi, hi], k1[bi, hi], None, causal))
            a2 = _softmax_rows(_scores(q2[bi, hi], k2[bi, hi], None, causal))
            vv = v[bi, hi]
            o2 = a2 @ vv
            opre = a1 @ vv - lm * o2
            dy = dout[bi, hi]
            dopre = _head_rmsnorm_backward(opre, dy, lambda_init, eps) if headnorm else dy
            dv[bi, hi] = a1.T @ dopre - lm * (a2.T @ dopre)
            dp = dopre @ vv.T
            ds1 = _softmax_backward_rows(a1, dp)
            ds2 = _softmax_backward_rows(a2, -lm * dp)
            dq1[bi, hi] = c * (ds1 @ k1[bi, hi])
            dk1[bi, hi] = c * (ds1.T @ q1[bi, hi])
            dq2[bi, hi] = c * (ds2 @ k2[bi, hi])
            dk2[bi, hi] = c * (ds2.T @ q2[bi, hi])
            dlam[hi] -= np.sum(dopre * o2)
    return dq1, dk1, dq2, dk2, dv, dlam


def diff_attention_backward_dq_rows(q1, k1, q2, k2, v, lam, dout, rows, causal: bool = True,
                                    headnorm: bool = False, lambda_init: float = 0.8,
                                    eps: float = 1e-5):
    """dQ1, dQ2 rows of one (b, h) slice for the selected query rows.

    The same chain rule as diff_attention_backward, restricted to what a query
    row needs (its two score rows, its output row, its dOut row), so that
    long sequences can be checked row by row.  q*, k* [T, D], v [T, 2D],
    dout [T, 2D], lam a float; returns two [len(rows), D] arrays.
    """
    q1, k1, q2, k2, v, dout = (_f64(t) for t in (q1, k1, q2, k2, v, dout))
    rows = np.asarray(rows)
    c = 1.0 / math.sqrt(q1.shape[-1])
    lm = float(lam)
    a1 = _softmax_rows(_scores(q1, k1, rows, causal))
    a2 = _softmax_rows(_scores(q2, k2, rows, causal))
    o2 = a2 @ v
    opre = a1 @ v - lm * o2
    dy = dout[rows]
    dopre = _head_rmsnorm_backward(opre, dy, lambda_init, eps) if headnorm else dy
    dp = dopre @ v.T
    ds1 = _softmax_backward_rows(a1, dp)
    ds2 = _softmax_backward_rows(a2, -lm * dp)
    return c * (ds1 @ k1), c * (ds2 @ k2)


def reparam_lambda_backward(lq1, lk1, lq2, lk2, dlam):
    """Gradients of lam = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init (aifetchly
    page, section 3) with respect to its four vectors, given dL/dlam per head:
    d lq1 = dlam e1 lk1, d lk1 = dlam e1 lq1, d lq2 = -dlam e2 lk2,
    d lk2 = -dlam e2 lq2, with e1 = exp(lq1 . lk1), e2 = exp(lq2 . lk2)."""
    a, b, c, d = (_f64(t) for t in (lq1, lk1, lq2, lk2))
    dl = _f64(dlam)[..., None]
    e1 = np.exp(np.sum(a * b, axis=-1, keepdims=True))
    e2 = np.exp(np.sum(c * d, axis=-1, keepdims=True))
    return dl * e1 * b, dl * e1 * a, -dl * e2 * d, -dl * e2 * c
