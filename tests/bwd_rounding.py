"""Where the backward kernels round, and a first-order bound on what those
roundings do to the gradients.

The gradients of differential attention (the chain rule of the paperleet
page "Differential Transformer Attention", head norm as in aifetchly
"Differential Transformer: Canceling LLM Attention Noise", section 3) are
evaluated here in float64 with a hook at every point where the forward and
backward kernels hold a value in bf16 or rely on a rounded row sum:

  q1, q2    the score operand q log2(e)/sqrt(D) of the forward and of the
            query-side backward kernel (the same rounded values)
  k1, k2    the score operand k log2(e)/sqrt(D) of the key-side kernel
  w1, w2    the forward's probabilities in its P.V products (the saved
            per-map outputs O1, O2 are formed from them)
  l1, l2    the forward's row sum, which normalises O1, O2 and enters the
            saved log-sum-exp that both backward kernels subtract
  d         dOpre, the gradient reaching the pre-norm output
  s1q, s2q  dS of the query-side kernel (A operand of dQ)
  s1k, s2k  dS of the key-side kernel (B operand of dK)
  pv        A1 - lam A2 in the dV product

With rnd(name, x) = x (1 + e_name), every e_name zero, the function is the
exact chain rule; its Jacobian J with respect to all e at e = 0 gives, per
gradient element j, the first-order bound u sum_i |J_ji| on the effect of
relative perturbations |e_i| <= u, i.e. of rounding each of those values
to nearest with unit roundoff u.  bf16 keeps 8 significant bits, so
u = 2^-8; the products that feed a rounding are fp32 (2^-24 each), which the
margin in U covers.  What is not listed (fp32 accumulation, the final bf16
rounding of each gradient) moves an element by a small multiple of 2^-8 of
the tensor's scale and is left to the caller's relative term.

This is test infrastructure: it models the kernels' rounding points to bound
their error; it is not an implementation of the method.
"""

import math

import numpy as np
import torch

U = 2.0 ** -8 + 2.0 ** -20
LOG2E = 1.4426950408889634


def _lse2(s):
    return torch.logsumexp(s * math.log(2.0), dim=-1, keepdim=True) / math.log(2.0)


def backward_chain(x, lam, dout, causal, headnorm, lambda_init, eps, rnd):
    """(dq1, dk1, dq2, dk2, dv) as float64 tensors, with rnd(name, value)
    applied at each rounding point listed in the module docstring."""
    q1, k1, q2, k2, v = (torch.as_tensor(x[n]).double() for n in ("q1", "k1", "q2", "k2", "v"))
    dy = torch.as_tensor(dout).double()
    D = q1.shape[-1]
    T = q1.shape[-2]
    c = LOG2E / math.sqrt(D)
    lam = torch.as_tensor(np.broadcast_to(np.asarray(lam, dtype=np.float64), (q1.shape[1],)).copy())
    lb = lam[None, :, None, None]
    allowed = torch.tril(torch.ones(T, T, dtype=torch.bool)) if causal else torch.ones(T, T, dtype=torch.bool)
    neg = torch.tensor(-math.inf, dtype=torch.float64)

    def scores(a, b):
        return torch.where(allowed, a @ b.transpose(-1, -2), neg)

    # forward: maps from the rounded score operand, row sums, per-map outputs
    s1 = scores(rnd("q1", q1 * c), k1)
    s2 = scores(rnd("q2", q2 * c), k2)
    lse1, lse2 = _lse2(s1), _lse2(s2)
    a1, a2 = torch.exp2(s1 - lse1), torch.exp2(s2 - lse2)
    f1 = rnd("l1", torch.ones_like(lse1))
    f2 = rnd("l2", torch.ones_like(lse2))
    o1 = (rnd("w1", a1) * f1) @ v
    o2 = (rnd("w2", a2) * f2) @ v
    opre = o1 - lb * o2
    if headnorm:
        g = 1.0 / torch.sqrt(torch.mean(opre * opre, dim=-1, keepdim=True) + eps)
        grad = (1.0 - lambda_init) * g * (dy - opre * g * g * torch.mean(dy * opre, dim=-1, keepdim=True))
    else:
        grad = dy
    d = rnd("d", grad)
    dp = d @ v.transpose(-1, -2)
    d1 = torch.sum(d * o1, dim=-1, keepdim=True)
    d2 = -lb * torch.sum(d * o2, dim=-1, keepdim=True)

    # query-side kernel: same score operand as the forward, saved log-sum-exp
    p1, p2 = a1 * f1, a2 * f2
    ds1 = rnd("s1q", p1 * (dp - d1))
    ds2 = rnd("s2q", p2 * (-lb * dp - d2))
    dq1 = ds1 @ k1 / math.sqrt(D)
    dq2 = ds2 @ k2 / math.sqrt(D)

    # key-side kernel: the key is the rounded score operand
    p1k = torch.exp2(scores(q1, rnd("k1", k1 * c)) - lse1) * f1
    p2k = torch.exp2(scores(q2, rnd("k2", k2 * c)) - lse2) * f2
    dk1 = rnd("s1k", p1k * (dp - d1)).transpose(-1, -2) @ q1 / math.sqrt(D)
    dk2 = rnd("s2k", p2k * (-lb * dp - d2)).transpose(-1, -2) @ q2 / math.sqrt(D)
    dv = rnd("pv", p1k - lb * p2k).transpose(-1, -2) @ d
    return dq1, dk1, dq2, dk2, dv


def exact(x, lam, dout, causal, headnorm, lambda_init, eps):
    return tuple(g.numpy() for g in backward_chain(x, lam, dout, causal, headnorm, lambda_init, eps,
                                                    lambda name, val: val))


def _bf16(t):
    return t.float().bfloat16().double()


def simulated(x, lam, dout, causal, headnorm, lambda_init, eps):
    """One realization of the kernels' roundings: every listed value rounded
    to bf16 (the score operands after an fp32 product, as the kernels form
    them), row sums unrounded."""
    def rnd(name, val):
        if name in ("l1", "l2"):
            return val
        if name in ("q1", "q2", "k1", "k2"):
            return _bf16(val.float())
        return _bf16(val)
    return tuple(g.numpy() for g in backward_chain(x, lam, dout, causal, headnorm, lambda_init, eps, rnd))


def first_order_bound(x, lam, dout, causal, headnorm, lambda_init, eps):
    """Per element of (dq1, dk1, dq2, dk2, dv): U sum_i |dG_j / de_i| at e = 0.
    Sized for short sequences (the Jacobian is materialised)."""
    shapes = {}

    def record(name, val):
        shapes[name] = val.shape
        return val

    backward_chain(x, lam, dout, causal, headnorm, lambda_init, eps, record)
    names = list(shapes)

    def f(*es):
        table = dict(zip(names, es))
        return backward_chain(x, lam, dout, causal, headnorm, lambda_init, eps,
                              lambda name, val: val * (1.0 + table[name]))

    zeros = tuple(torch.zeros(shapes[n], dtype=torch.float64) for n in names)
    jac = torch.autograd.functional.jacobian(f, zeros, vectorize=True)
    bounds = []
    for j_out in jac:
        tot = None
        for j_in, z in zip(j_out, zeros):
            part = j_in.abs().sum(dim=tuple(range(j_in.dim() - z.dim(), j_in.dim())))
            tot = part if tot is None else tot + part
        bounds.append((U * tot).numpy())
    return tuple(bounds)
