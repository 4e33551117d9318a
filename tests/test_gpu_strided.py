"""GPU: prefill on strided views, read and written in place, through the C ABI
(diffattn_fwd_strided).

Q1, Q2 and K1, K2 are the two halves of fused [B, T, H, 2D] projections (the
aifetchly page's numpy forward cuts them out of one projection along the
feature axis; the paperleet page allows strided inputs), V is a [B, T, H, 2D]
buffer seen as [B, H, T, 2D], and the output is written into such a buffer.
The strided entry runs the same kernels as diffattn_fwd with per-tensor
strides, so on the same values it must reproduce diffattn_fwd on dense copies
bit for bit; one case is also checked against the float64 oracle
(max |GPU - oracle| <= 2e-2, the bf16 bar of the workload statement).
"""

import numpy as np
import pytest
import torch

import differential_attention_forward_amd as da
import oracle
from workloads import prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    da.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def fused(a, b):
    """[B, T, H, 2D] buffer holding a | b ([B, H, T, D] each) and the two views."""
    B, H, T, D = a.shape
    buf = torch.empty((B, T, H, 2 * D), device=DEV, dtype=a.dtype)
    buf[..., :D] = a.to(DEV).permute(0, 2, 1, 3)
    buf[..., D:] = b.to(DEV).permute(0, 2, 1, 3)
    return buf, buf[..., :D].permute(0, 2, 1, 3), buf[..., D:].permute(0, 2, 1, 3)


def token_major(x):
    """A [B, T, H, W] buffer holding x ([B, H, T, W]) and its [B, H, T, W] view."""
    buf = x.to(DEV).permute(0, 2, 1, 3).contiguous()
    return buf, buf.permute(0, 2, 1, 3)


CASES = [
    # B, H, T, D, causal, headnorm
    (2, 3, 200, 64, True, True),
    (1, 2, 333, 128, False, True),
    (2, 2, 130, 32, True, False),
    (1, 8, 1000, 64, True, False),
    (1, 2, 5000, 64, True, True),
    (2, 4, 257, 128, True, False),
    (1, 1, 1, 64, True, True),
    (3, 1, 65, 32, False, True),
]


@pytest.mark.parametrize("B,H,T,D,causal,headnorm", CASES)
def test_fused_views_match_dense(B, H, T, D, causal, headnorm):
    say(f"strided B={B} H={H} T={T} D={D} causal={causal} headnorm={headnorm}")
    x = prefill_inputs(B, H, T, D, "bf16", seed=900 + T + D)
    lam = torch.linspace(-0.2, 1.1, H, device=DEV)
    _, q1v, q2v = fused(x["q1"], x["q2"])
    _, k1v, k2v = fused(x["k1"], x["k2"])
    _, vv = token_major(x["v"])
    obuf = torch.full((B, T, H, 2 * D), float("nan"), device=DEV, dtype=torch.bfloat16)
    outv = obuf.permute(0, 2, 1, 3)
    if T > 1:
        assert not q1v.is_contiguous() and (H == 1 or not outv.is_contiguous())
    da.diffattn_fwd_strided(q1v, k1v, q2v, k2v, vv, lam, causal=causal, headnorm=headnorm,
                            lambda_init=0.8, eps=1e-5, out=outv)
    dense = da.diffattn_fwd(*(t.to(DEV) for t in (x["q1"], x["k1"], x["q2"], x["k2"], x["v"])), lam,
                            causal=causal, headnorm=headnorm, lambda_init=0.8, eps=1e-5)
    torch.cuda.synchronize()
    assert torch.equal(outv, dense), float((outv.float() - dense.float()).abs().max())


def test_fused_views_against_oracle():
    B, H, T, D = 2, 3, 200, 64
    x = prefill_inputs(B, H, T, D, "bf16", seed=4242)
    lam = torch.tensor([0.1, 0.5, 0.9])
    _, q1v, q2v = fused(x["q1"], x["q2"])
    _, k1v, k2v = fused(x["k1"], x["k2"])
    _, vv = token_major(x["v"])
    out = da.diffattn_fwd_strided(q1v, k1v, q2v, k2v, vv, lam.to(DEV), causal=True, headnorm=True,
                                  lambda_init=0.8, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.head_rmsnorm(oracle.diff_attention(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, True),
                              0.8, 1e-5)
    err = float(np.max(np.abs(out.float().cpu().double().numpy() - ref)))
    assert err <= TOL, err


def test_shared_keys_and_values():
    # head and batch strides of 0: every head of every batch reads the same
    # K1, K2, V slice, as the dense call does on expanded copies
    B, H, T, D = 2, 4, 150, 64
    x = prefill_inputs(1, 1, T, D, "bf16", seed=77)
    q = prefill_inputs(B, H, T, D, "bf16", seed=78)
    k1, k2, v = (x[n].to(DEV) for n in ("k1", "k2", "v"))
    k1b, k2b, vb = (t.expand(B, H, T, t.shape[-1]) for t in (k1, k2, v))
    assert k1b.stride()[:2] == (0, 0)
    lam = 0.6
    q1, q2 = q["q1"].to(DEV), q["q2"].to(DEV)
    out = da.diffattn_fwd_strided(q1, k1b, q2, k2b, vb, lam, causal=True)
    dense = da.diffattn_fwd(q1, k1b.contiguous(), q2, k2b.contiguous(), vb.contiguous(), lam, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)


def test_dense_tensors_take_the_same_path():
    B, H, T, D = 1, 2, 300, 64
    x = prefill_inputs(B, H, T, D, "bf16", seed=5)
    xd = [x[n].to(DEV) for n in ("q1", "k1", "q2", "k2", "v")]
    a = da.diffattn_fwd_strided(*xd, 0.7, causal=False)
    b = da.diffattn_fwd(*xd, 0.7, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
