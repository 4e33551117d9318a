"""Seeded synthetic inputs for differential-attention workloads.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic (no scores, no softmax, no lambda formula).  Both the
float64 oracle and the HIP library are fed the *same* tensors produced here.

Conventions (one recipe for every workload):
  * torch ``Generator`` on the requested device, ``manual_seed(seed)``;
    floating inputs are drawn as float32 ``randn`` and cast to the compute
    dtype with torch's round-to-nearest-even ``.to(torch.bfloat16)``.
  * draw order: Q1, Q2, K1, K2, V, then the four lambda vectors
    (lq1, lk1, lq2, lk2, each [H, Dl] * 0.1), then the workload's extras.
  * small integer choices (needle positions) come from a CPU generator seeded
    with ``seed + 1`` so they do not depend on the device.

Named workloads (the shapes of the pages' problem statement: Q/K [B,H,T,D],
V and O [B,H,T,2D]; decode: one query per (b, h) against an L-row cache):

  tiny_fp32_causal          B1 H2 T128 D32, causal, fp32, seed 0, lambda from
                            vectors [2,32] ~ N(0, 0.1^2), layer 1, no head norm
  prefill_t4k_causal        B2 H16 T4096 D64, causal, bf16, seed 2, lambda from
                            vectors [16,64], layer 12, head norm (eps 1e-5)
  prefill_t32k_needles      B1 H16 T32768 D64, causal, bf16, seed 3; 8 needle
                            keys per head (K1[j] = 4 * Q1[i], i uniform in
                            [j, T)); V gets one shared offset c in R^128;
                            lambda = 0.8 for every head; no head norm
  full_t8k_d128             B4 H8 T8192 D128, full (non-causal), bf16, seed 4,
                            all inputs N(0,1)/sqrt(2), lambda_h ~ U[0.2, 0.8],
                            head norm with lambda_init 0.8 (eps 1e-5)
  decode_l64k               B32 H16, cache L=65536, D64, bf16, seed 5, lambda
                            vectors all zero (so lambda = lambda_init(24)),
                            64 key splits, no head norm

DIFF V2 workloads (the French lesson page, "V1 contre V2" and its exercise of
8 KV heads for 32 query heads; Q1, Q2 [B,H,T,D], K, V [B,Hkv,T,D]):

  v2_prefill_t4k            B2 H16 Hkv4 T4096 D128, causal, bf16, seed 6,
                            lambda_h ~ U[0.2, 0.8]
  v2_decode_l64k            B32 H32 Hkv8, cache L=65536, D128, bf16, seed 7,
                            lambda_h ~ U[0.2, 0.8], default key splits
                            (the same cache bytes per KV head and key as
                            decode_l64k has per head)

V2 draw order: Q1, Q2, K, V (caches one batch row at a time), then lambda.

Workloads of the other rows next to the forward (measured, not part of the
problem statement's configurations):

  bwd_t4k_causal            backward of prefill_t4k_causal's shape (B2 H16
                            T4096 D64 causal bf16, head norm, lambda_init 0.8),
                            seed 8, lambda_h ~ U[0.2, 0.8], dL/dOut ~ N(0,1)
  bwd_t4k_d128              the same flop count at head width 128 (B2 H8
                            T4096 D128), seed 12
  prefill_t32k_window4k     B1 H16 T32768 D64 causal bf16 with a 4096-key
                            sliding window, seed 9, lambda = 0.8
  decode_ragged_l64k        decode_l64k's shape with per-sequence lengths
                            uniform in [1, 65536] (CPU generator, seed 11),
                            seed 10, lambda = lambda_init(24) = zero vectors
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "prefill_inputs", "decode_inputs", "v2_inputs", "make_workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    B: int
    H: int
    T: int                    # query length (prefill) or cache length L (decode)
    D: int
    dtype: str                # "fp32" or "bf16"
    seed: int
    causal: bool = True
    headnorm: bool = False
    eps: float = 1e-5
    layer: int | None = None  # lambda_init taken from the schedule at this layer
    lambda_init: float | None = None  # given directly when no layer is named
    lambda_dl: int = 0        # length of the lambda vectors (0 = none drawn)
    lambda_zero: bool = False  # lambda vectors are all zero (their initial value)
    lam_fixed: float | None = None
    lam_uniform: tuple | None = None
    input_scale: float = 1.0
    needles: int = 0
    value_offset: bool = False
    num_splits: int = 0
    Hkv: int = 0              # DIFF V2: KV heads (0 = the first version)
    window: int = 0           # causal sliding window (0 = none)
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_causal", "prefill", 1, 2, 128, 32, "fp32", 0, causal=True,
                 layer=1, lambda_dl=32),
        Workload("prefill_t4k_causal", "prefill", 2, 16, 4096, 64, "bf16", 2, causal=True,
                 headnorm=True, layer=12, lambda_dl=64),
        Workload("prefill_t32k_needles", "prefill", 1, 16, 32768, 64, "bf16", 3, causal=True,
                 lam_fixed=0.8, lambda_init=0.8, needles=8, value_offset=True),
        Workload("full_t8k_d128", "prefill", 4, 8, 8192, 128, "bf16", 4, causal=False,
                 headnorm=True, lambda_init=0.8, lam_uniform=(0.2, 0.8),
                 input_scale=1.0 / math.sqrt(2.0)),
        Workload("decode_l64k", "decode", 32, 16, 65536, 64, "bf16", 5,
                 layer=24, lambda_dl=64, lambda_zero=True, num_splits=64),
        Workload("v2_prefill_t4k", "v2_prefill", 2, 16, 4096, 128, "bf16", 6, causal=True,
                 lam_uniform=(0.2, 0.8), Hkv=4),
        Workload("v2_decode_l64k", "v2_decode", 32, 32, 65536, 128, "bf16", 7,
                 lam_uniform=(0.2, 0.8), Hkv=8),
        Workload("bwd_t4k_causal", "bwd", 2, 16, 4096, 64, "bf16", 8, causal=True,
                 headnorm=True, lambda_init=0.8, lam_uniform=(0.2, 0.8)),
        Workload("bwd_t4k_d128", "bwd", 2, 8, 4096, 128, "bf16", 12, causal=True,
                 headnorm=True, lambda_init=0.8, lam_uniform=(0.2, 0.8)),
        Workload("prefill_t32k_window4k", "window_prefill", 1, 16, 32768, 64, "bf16", 9,
                 causal=True, lam_fixed=0.8, lambda_init=0.8, window=4096),
        Workload("decode_ragged_l64k", "ragged_decode", 32, 16, 65536, 64, "bf16", 10,
                 layer=24, lambda_dl=64, lambda_zero=True, num_splits=64),
    ]
}


def _tdtype(dtype: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _randn(g, shape, device, scale=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x


def attention_inputs(B, H, T, D, seed=0, device="cpu"):
    """Q, K, V [B,H,T,D] bf16, iid N(0,1) cast with round-to-nearest-even: the
    inputs of the standard-attention comparison kernel (a same-size model has
    head width D = 2 x the differential head width)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return {n: _randn(g, (B, H, T, D), device, 1.0).to(torch.bfloat16) for n in ("q", "k", "v")}


def prefill_inputs(B, H, T, D, dtype="bf16", seed=0, device="cpu", *, input_scale=1.0,
                   lambda_dl=0, lambda_zero=False, lam_fixed=None, lam_uniform=None,
                   needles=0, value_offset=False):
    """Q1, Q2, K1, K2 [B,H,T,D] and V [B,H,T,2D] plus the lambda inputs.

    Returns a dict with q1, q2, k1, k2, v (compute dtype, on ``device``), and,
    when requested, lq1, lk1, lq2, lk2 ([H, Dl] float32) and/or lam ([H]
    float32, lambda given directly), needle_pos ([B, H, needles] key positions,
    CPU int64), needle_query ([B, H, needles] the query row each needle key
    copies, CPU int64) and offset ([2D] float32).
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    gi = torch.Generator(device="cpu")
    gi.manual_seed(seed + 1)
    td = _tdtype(dtype)
    q1 = _randn(g, (B, H, T, D), device, input_scale)
    q2 = _randn(g, (B, H, T, D), device, input_scale)
    k1 = _randn(g, (B, H, T, D), device, input_scale)
    k2 = _randn(g, (B, H, T, D), device, input_scale)
    v = _randn(g, (B, H, T, 2 * D), device, input_scale)
    out = {}
    if lambda_dl:
        for name in ("lq1", "lk1", "lq2", "lk2"):
            if lambda_zero:
                out[name] = torch.zeros((H, lambda_dl), device=device, dtype=torch.float32)
            else:
                out[name] = _randn(g, (H, lambda_dl), device, 0.1)
    if lam_fixed is not None:
        out["lam"] = torch.full((H,), float(lam_fixed), device=device, dtype=torch.float32)
    if lam_uniform is not None:
        lo, hi = lam_uniform
        u = torch.rand((H,), generator=g, device=device, dtype=torch.float32)
        out["lam"] = lo + (hi - lo) * u
    if needles:
        # per (b, h): distinct key positions j, each paired with a query row
        # i >= j so the key is visible under the causal mask; K1[j] <- 4 Q1[i]
        # (a power-of-two multiple: exact in fp32 and after the bf16 cast).
        pos = torch.empty((B, H, needles), dtype=torch.int64)
        qpos = torch.empty((B, H, needles), dtype=torch.int64)
        for b in range(B):
            for h in range(H):
                js = torch.randperm(T, generator=gi)[:needles]
                for n, j in enumerate(js.tolist()):
                    i = int(torch.randint(j, T, (1,), generator=gi))
                    k1[b, h, j] = 4.0 * q1[b, h, i]
                    pos[b, h, n] = j
                    qpos[b, h, n] = i
        out["needle_pos"] = pos
        out["needle_query"] = qpos
    if value_offset:
        c = _randn(g, (2 * D,), device)
        v += c
        out["offset"] = c
    out.update(q1=q1.to(td), q2=q2.to(td), k1=k1.to(td), k2=k2.to(td), v=v.to(td))
    return out


def decode_inputs(B, H, L, D, dtype="bf16", seed=0, device="cpu", *, lambda_dl=0,
                  lambda_zero=False, lam_fixed=None, input_scale=1.0):
    """q1, q2 [B,H,D]; K1, K2 caches [B,H,L,D]; V cache [B,H,L,2D].

    Large caches are drawn one batch row at a time so that the float32
    temporaries stay small; the draw order is q1, q2, then K1, K2, V for
    b = 0, 1, ... in turn.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = _tdtype(dtype)
    q1 = _randn(g, (B, H, D), device, input_scale).to(td)
    q2 = _randn(g, (B, H, D), device, input_scale).to(td)
    k1 = torch.empty((B, H, L, D), device=device, dtype=td)
    k2 = torch.empty((B, H, L, D), device=device, dtype=td)
    v = torch.empty((B, H, L, 2 * D), device=device, dtype=td)
    for b in range(B):
        k1[b] = _randn(g, (H, L, D), device, input_scale).to(td)
        k2[b] = _randn(g, (H, L, D), device, input_scale).to(td)
        v[b] = _randn(g, (H, L, 2 * D), device, input_scale).to(td)
    out = dict(q1=q1, q2=q2, k1=k1, k2=k2, v=v)
    if lambda_dl:
        for name in ("lq1", "lk1", "lq2", "lk2"):
            if lambda_zero:
                out[name] = torch.zeros((H, lambda_dl), device=device, dtype=torch.float32)
            else:
                out[name] = _randn(g, (H, lambda_dl), device, 0.1)
    if lam_fixed is not None:
        out["lam"] = torch.full((H,), float(lam_fixed), device=device, dtype=torch.float32)
    return out


def v2_inputs(B, H, Hkv, T, D, dtype="bf16", seed=0, device="cpu", *, decode=False,
              lam_uniform=None):
    """DIFF V2 inputs: q1, q2 [B,H,T,D] (decode: [B,H,D]), K, V [B,Hkv,T,D],
    iid N(0,1) cast to the compute dtype; lam [H] ~ U[lo, hi] when asked.
    Caches are drawn one batch row at a time (small float32 temporaries)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = _tdtype(dtype)
    qshape = (B, H, D) if decode else (B, H, T, D)
    q1 = _randn(g, qshape, device).to(td)
    q2 = _randn(g, qshape, device).to(td)
    k = torch.empty((B, Hkv, T, D), device=device, dtype=td)
    v = torch.empty((B, Hkv, T, D), device=device, dtype=td)
    for b in range(B):
        k[b] = _randn(g, (Hkv, T, D), device).to(td)
        v[b] = _randn(g, (Hkv, T, D), device).to(td)
    out = dict(q1=q1, q2=q2, k=k, v=v)
    if lam_uniform is not None:
        lo, hi = lam_uniform
        u = torch.rand((H,), generator=g, device=device, dtype=torch.float32)
        out["lam"] = lo + (hi - lo) * u
    return out


def ragged_lengths(B, L, seed):
    """Per-sequence cache lengths uniform in [1, L] (CPU generator), int32."""
    g = torch.Generator()
    g.manual_seed(seed)
    return torch.randint(1, L + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def make_workload(name: str, device="cpu"):
    """Inputs of a named workload, drawn on ``device`` with its recipe."""
    w = WORKLOADS[name]
    if w.kind == "bwd":
        x = prefill_inputs(w.B, w.H, w.T, w.D, w.dtype, w.seed, device, lam_uniform=w.lam_uniform)
        x["dout"] = grad_output(x["v"].shape, seed=w.seed + 100, device=device, dtype=w.dtype)
        return x
    if w.kind == "window_prefill":
        return prefill_inputs(w.B, w.H, w.T, w.D, w.dtype, w.seed, device, lam_fixed=w.lam_fixed)
    if w.kind == "ragged_decode":
        x = decode_inputs(w.B, w.H, w.T, w.D, w.dtype, w.seed, device, lambda_dl=w.lambda_dl,
                          lambda_zero=w.lambda_zero)
        x["lengths"] = ragged_lengths(w.B, w.T, w.seed + 1).to(device)
        return x
    if w.kind in ("v2_prefill", "v2_decode"):
        return v2_inputs(w.B, w.H, w.Hkv, w.T, w.D, w.dtype, w.seed, device,
                         decode=w.kind == "v2_decode", lam_uniform=w.lam_uniform)
    if w.kind == "prefill":
        return prefill_inputs(w.B, w.H, w.T, w.D, w.dtype, w.seed, device,
                              input_scale=w.input_scale, lambda_dl=w.lambda_dl,
                              lambda_zero=w.lambda_zero, lam_fixed=w.lam_fixed,
                              lam_uniform=w.lam_uniform, needles=w.needles,
                              value_offset=w.value_offset)
    return decode_inputs(w.B, w.H, w.T, w.D, w.dtype, w.seed, device,
                         lambda_dl=w.lambda_dl, lambda_zero=w.lambda_zero,
                         lam_fixed=w.lam_fixed, input_scale=w.input_scale)


def grad_output(shape, seed=0, device="cpu", dtype="bf16"):
    """dL/dOut for the backward pass: iid N(0,1) in the compute dtype (a
    synthetic upstream gradient of the attention output's shape)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return _randn(g, tuple(shape), device).to(_tdtype(dtype))
