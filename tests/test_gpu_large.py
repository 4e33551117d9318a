"""Parity beyond 4 GiB per tensor: B = 257, H = 256, T = 512, D = 64 (bf16).

Each of Q1, K1, Q2, K2 then holds 2^31 + 2^24 elements (4.3 GB) and V, the
output and the backward's dOpre twice that; each of the two fp32 maps the
training forward saves holds 17.2 GB.  The heads past the 2^31-element and
2^32-byte marks of these tensors are exactly the ones a 32-bit offset
anywhere in the address arithmetic would misplace, so the sampled heads
always include the last one and heads on both sides of each mark.

Inputs are drawn on the device from a seeded generator (the same recipe as
workloads.prefill_inputs, with device="cuda"); every comparison value comes
from the float64 oracle on slices copied to the host, or from a closed form:
under the causal mask row 0 sees only key 0, so its pre-norm output is
(1 - lambda_h) V_0 (paperleet "Differential Transformer Attention": both maps
are softmax rows, and a one-key softmax is 1), which checks every one of the
65792 heads at once.
"""

import numpy as np
import pytest
import torch

import differential_attention_forward_amd as da
import oracle
from tests.test_gpu_backward import dlambda_term_rss
from workloads import grad_output, prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
B, H, T, D = 257, 256, 512, 64
TOL = 2e-2
LAMBDA_INIT, EPS = 0.8, 1e-5


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def big():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    da.lib()
    say(f"large inputs: B={B} H={H} T={T} D={D} bf16 on the device")
    x = prefill_inputs(B, H, T, D, "bf16", seed=7100, device=DEV)
    assert x["q1"].numel() > 2 ** 31 and x["q1"].numel() * 2 > 2 ** 32
    # lambda varies across heads, so that a head reading another head's lambda
    # or data shows in its output
    lam = torch.linspace(-0.4, 1.3, H, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    yield x, lam
    del x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _slices():
    """(b, h) pairs: the first and last heads, the heads on both sides of the
    2^31-element (and 2^32-byte) mark of Q/K (flat head index 65536) and of
    V, the output and dOpre (32768), of the 2^32-byte mark of the saved fp32
    maps (16384), and a few seeded random ones."""
    flat = [0, B * H - 1, 16383, 16384, 32767, 32768, 65535, 65536]
    rng = np.random.default_rng(7101)
    flat += rng.integers(0, B * H, 4).tolist()
    return sorted({(f // H, f % H) for f in flat})


def _host(x, b, h):
    return {k: x[k][b:b + 1, h:h + 1].cpu() for k in ("q1", "k1", "q2", "k2", "v")}


def _err(gpu, ref):
    return float(np.max(np.abs(gpu.double().cpu().numpy() - ref)))


@pytest.mark.parametrize("causal,headnorm", [(True, True), (False, False)])
def test_prefill_beyond_4gib(big, causal, headnorm):
    x, lam = big
    say(f"large prefill causal={causal} headnorm={headnorm}")
    out = da.diffattn_fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, causal=causal,
                          headnorm=headnorm, lambda_init=LAMBDA_INIT, eps=EPS)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    lam_h = lam.cpu().numpy()
    for b, h in _slices():
        s = _host(x, b, h)
        ref = oracle.diff_attention(s["q1"], s["k1"], s["q2"], s["k2"], s["v"], lam_h[h:h + 1], causal)
        if headnorm:
            ref = oracle.head_rmsnorm(ref, LAMBDA_INIT, EPS)
        err = _err(out[b:b + 1, h:h + 1], ref)
        say(f"  (b={b}, h={h}) max err {err:.3e}")
        assert err <= TOL, (b, h, err)
    if causal:
        # every head's row 0: (1 - lambda_h) V_0, then the head norm
        v0 = x["v"][:, :, 0].double()
        o0 = (1.0 - lam.double())[None, :, None] * v0
        if headnorm:
            o0 = o0 / torch.sqrt(torch.mean(o0 * o0, dim=-1, keepdim=True) + EPS) * (1.0 - LAMBDA_INIT)
        err = (out[:, :, 0].double() - o0).abs()
        worst = int(torch.argmax(err.amax(dim=-1)))
        say(f"  row 0 of all {B * H} heads: max err {float(err.max()):.3e} (head {worst})")
        assert float(err.max()) <= TOL, (divmod(worst, H), float(err.max()))
    del out


def test_train_and_backward_beyond_4gib(big):
    x, lam = big
    say("large training forward and backward")
    dout = grad_output((B, H, T, 2 * D), seed=7102, device=DEV)
    out, saved = da.diffattn_fwd_train(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, causal=True,
                                       headnorm=True, lambda_init=LAMBDA_INIT, eps=EPS)
    assert saved.numel() > 2 ** 35  # two fp32 maps of 16 GiB each, plus the log-sum-exp
    g = da.diffattn_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, dout, saved, causal=True,
                        headnorm=True, lambda_init=LAMBDA_INIT, eps=EPS)
    torch.cuda.synchronize()
    del saved
    names = ("dq1", "dk1", "dq2", "dk2", "dv")
    lam_h = lam.cpu().numpy()
    for b, h in _slices():
        s = _host(x, b, h)
        ref_out = oracle.head_rmsnorm(
            oracle.diff_attention(s["q1"], s["k1"], s["q2"], s["k2"], s["v"], lam_h[h:h + 1], True),
            LAMBDA_INIT, EPS)
        err = _err(out[b:b + 1, h:h + 1], ref_out)
        assert err <= TOL, ("out", b, h, err)
        ref = oracle.diff_attention_backward(s["q1"], s["k1"], s["q2"], s["k2"], s["v"], lam_h[h:h + 1],
                                             dout[b:b + 1, h:h + 1].cpu(), True, True, LAMBDA_INIT, EPS)
        msg = []
        for name, gt, r in zip(names, g[:5], ref[:5]):
            e = _err(gt[b:b + 1, h:h + 1], r)
            scale = float(np.max(np.abs(r)))
            msg.append(f"{name}={e / max(scale, 1e-30):.2e}")
            assert e <= TOL * scale + 1e-4, (name, b, h, e, scale)
        say(f"  (b={b}, h={h}) out {err:.2e} " + " ".join(msg))
    # dlambda of the last head sums over every batch: compare it whole, with
    # the bound of the other backward tests (2% of the larger of |dlambda|,
    # the root-sum-square of its terms and 1)
    hl = H - 1
    s = {k: x[k][:, hl:hl + 1].cpu() for k in ("q1", "k1", "q2", "k2", "v")}
    dh = dout[:, hl:hl + 1].cpu()
    ref = oracle.diff_attention_backward(s["q1"], s["k1"], s["q2"], s["k2"], s["v"], lam_h[hl:hl + 1],
                                         dh, True, True, LAMBDA_INIT, EPS)
    rss = float(dlambda_term_rss(s, lam_h[hl:hl + 1], dh, True, True, LAMBDA_INIT, EPS)[0])
    got = float(g[5][hl])
    want = float(ref[5][0])
    say(f"  dlambda[{hl}] {got:.6e} vs {want:.6e} (terms' rss {rss:.3e})")
    assert abs(got - want) <= TOL * max(abs(want), rss, 1.0) + 1e-4, (got, want, rss)
    del g, out, dout
