"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Tolerances (max |GPU - oracle| over the compared elements): 1e-4 for fp32
inputs, 2e-2 for bf16 inputs, both with fp32 accumulation.  Inputs are the
same seeded tensors on both sides (bf16 values upcast exactly for the oracle).
Full-size workloads are compared on sampled output rows, which the oracle
computes one by one from the complete key range.
"""

import numpy as np
import pytest
import torch

import differential_attention_forward_amd as da
import oracle
from workloads import WORKLOADS, attention_inputs, decode_inputs, make_workload, prefill_inputs

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    da.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def to_dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) and k not in ("needle_pos", "needle_query") else v)
            for k, v in d.items()}


def maxerr(gpu_out, ref):
    return float(np.max(np.abs(gpu_out.detach().float().cpu().numpy().astype(np.float64) - ref)))


def run_fwd(x, lam, causal, headnorm, lambda_init=0.8, eps=1e-5):
    out = da.diffattn_fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, causal=causal,
                          headnorm=headnorm, lambda_init=lambda_init, eps=eps)
    torch.cuda.synchronize()
    return out


def ref_fwd(x, lam, causal, headnorm, lambda_init=0.8, eps=1e-5):
    o = oracle.diff_attention(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, causal)
    return oracle.head_rmsnorm(o, lambda_init, eps) if headnorm else o


# ---- sweep: dtype x head width x mask x head norm, ragged lengths -------------

SWEEP_T = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 257, 1000]


@pytest.mark.parametrize("headnorm", [False, True])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_sweep(dtype, D, causal, headnorm):
    lam = torch.tensor([0.35, 1.3], dtype=torch.float32)
    worst = 0.0
    for i, T in enumerate(SWEEP_T):
        x = prefill_inputs(1, 2, T, D, dtype, seed=1000 + 17 * D + i)
        say(f"fwd {dtype} D={D} T={T} causal={causal} headnorm={headnorm}")
        out = run_fwd(to_dev(x), lam.to(DEV), causal, headnorm)
        err = maxerr(out, ref_fwd(x, lam, causal, headnorm))
        worst = max(worst, err)
        assert err <= TOL[dtype], (T, err)
    say(f"  worst {worst:.3e}")


@pytest.mark.parametrize("headnorm", [False, True])
def test_fwd_long_causal_rows(headnorm):
    # causal rows longer than 4096 take the two-maps-per-wave configuration at
    # D=64 (shorter ones the one-map-per-wave one); sampled rows, full key range
    lam = torch.tensor([0.55, -0.25], dtype=torch.float32)
    for T, seed in ((4097, 31), (5000, 32)):
        x = prefill_inputs(1, 2, T, 64, "bf16", seed=seed)
        say(f"fwd bf16 D=64 T={T} causal headnorm={headnorm}")
        out = run_fwd(to_dev(x), lam.to(DEV), True, headnorm)
        rows = np.unique(np.concatenate([np.arange(40), np.arange(T - 40, T),
                                         np.random.default_rng(seed).choice(T, 200, replace=False)]))
        for h in range(2):
            ref = oracle.diff_attention_rows(x["q1"][0, h], x["k1"][0, h], x["q2"][0, h], x["k2"][0, h],
                                             x["v"][0, h], float(lam[h]), True, rows)
            if headnorm:
                ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
            assert maxerr(out[0, h, rows], ref) <= TOL["bf16"], (T, h)


@pytest.mark.parametrize("headnorm", [False, True])
def test_fwd_causal_many_heads(headnorm):
    # short causal rows over many heads take the 192-row, three-waves-per-SIMD
    # configuration at D=64 (few heads the 128-row one, as in the sweep above);
    # sampled heads and rows, full key range
    B, H, T = 8, 16, 2048
    x = prefill_inputs(B, H, T, 64, "bf16", seed=41, device=DEV)
    lam = torch.linspace(-0.2, 1.2, H, dtype=torch.float32, device=DEV)
    say(f"fwd bf16 D=64 B={B} H={H} T={T} causal headnorm={headnorm}")
    out = run_fwd(x, lam, True, headnorm)
    rng = np.random.default_rng(41)
    for b, h in ((0, 0), (3, 9), (7, 15)):
        rows = np.unique(np.concatenate([np.arange(32), np.arange(T - 32, T), rng.choice(T, 96, replace=False)]))
        sl = {k: x[k][b, h].cpu() for k in ("q1", "k1", "q2", "k2", "v")}
        ref = oracle.diff_attention_rows(sl["q1"], sl["k1"], sl["q2"], sl["k2"], sl["v"], float(lam[h]), True, rows)
        if headnorm:
            ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
        assert maxerr(out[b, h, rows], ref) <= TOL["bf16"], (b, h)
    del x, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("headnorm", [False, True])
def test_fwd_d32_long_causal_rows(headnorm):
    # D=32 causal rows beyond 2048 keys run one map per wave: 128-row
    # workgroups for few heads, 192-row ones once 128-row workgroups would
    # exceed four per compute unit (B2 H32 T2100: 1088); shorter rows keep
    # both maps per wave (the sweep above).  Sampled heads and rows, full
    # key range, ragged against both row counts.
    rng = np.random.default_rng(47)
    for B, H, T, seed, pairs in ((1, 2, 2049, 45, ((0, 0), (0, 1))), (1, 2, 3001, 46, ((0, 0), (0, 1))),
                                 (2, 32, 2100, 47, ((0, 0), (1, 17), (1, 31)))):
        x = prefill_inputs(B, H, T, 32, "bf16", seed=seed, device=DEV)
        lam = torch.linspace(-0.3, 1.1, H, dtype=torch.float32, device=DEV)
        say(f"fwd bf16 D=32 B={B} H={H} T={T} causal headnorm={headnorm}")
        out = run_fwd(x, lam, True, headnorm)
        for b, h in pairs:
            rows = np.unique(np.concatenate([np.arange(32), np.arange(T - 32, T), rng.choice(T, 96, replace=False)]))
            sl = {k: x[k][b, h].cpu() for k in ("q1", "k1", "q2", "k2", "v")}
            ref = oracle.diff_attention_rows(sl["q1"], sl["k1"], sl["q2"], sl["k2"], sl["v"], float(lam[h]), True,
                                             rows)
            if headnorm:
                ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
            assert maxerr(out[b, h, rows], ref) <= TOL["bf16"], (T, b, h)
        del x, out
        torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [64, 128])
def test_standard_attention(D, causal):
    # the one-map comparison kernel against the oracle's standard attention
    worst = 0.0
    for i, T in enumerate((1, 17, 64, 65, 129, 1000)):
        x = attention_inputs(1, 3, T, D, seed=900 + D + i)
        say(f"attention bf16 D={D} T={T} causal={causal}")
        out = da.diffattn_attention_fwd(*(x[k].to(DEV) for k in ("q", "k", "v")), causal=causal)
        torch.cuda.synchronize()
        err = maxerr(out, oracle.attention(x["q"], x["k"], x["v"], causal))
        worst = max(worst, err)
        assert err <= TOL["bf16"], (T, err)
    say(f"  worst {worst:.3e}")


def test_fwd_fp32_many_heads():
    # fp32 launch shapes over many workgroups (XCD remap, heaviest-first
    # order, ragged last tiles): D=64 one map per wave on 64-key tiles, D=32
    # causal one map per wave on 128-key tiles, D=32 full both maps per wave,
    # D=128 four waves.  Sampled heads and rows, full key range
    rng = np.random.default_rng(61)
    for B, H, T, D, causal, headnorm, seed in ((2, 16, 2500, 64, True, True, 62), (1, 12, 3001, 32, True, False, 63),
                                               (1, 8, 3000, 32, False, True, 64),
                                               (1, 8, 1100, 128, False, False, 65)):
        x = prefill_inputs(B, H, T, D, "fp32", seed=seed, device=DEV)
        lam = torch.linspace(-0.4, 1.3, H, dtype=torch.float32, device=DEV)
        say(f"fwd fp32 D={D} B={B} H={H} T={T} causal={causal} headnorm={headnorm}")
        out = run_fwd(x, lam, causal, headnorm)
        for b, h in ((0, 0), (B - 1, H // 2), (B - 1, H - 1)):
            rows = np.unique(np.concatenate([np.arange(16), np.arange(T - 16, T), rng.choice(T, 48, replace=False)]))
            sl = {k: x[k][b, h].cpu() for k in ("q1", "k1", "q2", "k2", "v")}
            ref = oracle.diff_attention_rows(sl["q1"], sl["k1"], sl["q2"], sl["k2"], sl["v"], float(lam[h]), causal,
                                             rows)
            if headnorm:
                ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
            assert maxerr(out[b, h, rows], ref) <= TOL["fp32"], (D, T, b, h)
        del x, out
        torch.cuda.empty_cache()


def test_standard_attention_long_causal_rows():
    # head width 128, causal rows beyond 4096 keys: 384-row workgroups at
    # three waves per SIMD (shorter rows take 128-row ones, as in the test
    # above)
    T = 4500
    x = attention_inputs(1, 2, T, 128, seed=931)
    say(f"attention bf16 D=128 T={T} causal")
    out = da.diffattn_attention_fwd(*(x[k].to(DEV) for k in ("q", "k", "v")), causal=True)
    torch.cuda.synchronize()
    assert maxerr(out, oracle.attention(x["q"], x["k"], x["v"], True)) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_lambda_range(dtype):
    # lambda is not clamped: negative and > 1 values included
    for lamv in (-0.3, 0.0, 0.2, 0.8, 1.0, 1.5):
        x = prefill_inputs(2, 3, 300, 64, dtype, seed=77)
        out = run_fwd(to_dev(x), lamv, True, False)
        assert maxerr(out, ref_fwd(x, lamv, True, False)) <= TOL[dtype], lamv


@pytest.mark.parametrize("headnorm", [False, True])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_identical_maps_cancel_exactly(dtype, causal, headnorm):
    # paperleet page: identical maps cancel at lambda = 1
    for D in (32, 64, 128):
        x = to_dev(prefill_inputs(1, 2, 200, D, dtype, seed=5))
        out = da.diffattn_fwd(x["q1"], x["k1"], x["q1"], x["k1"], x["v"], 1.0, causal=causal,
                              headnorm=headnorm)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0, D


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_causal_first_row(dtype):
    # row 0 sees only key 0 in both maps: O_0 = (1 - lambda) V_0
    x = prefill_inputs(1, 2, 100, 64, dtype, seed=9)
    out = run_fwd(to_dev(x), 0.6, True, False)
    ref = 0.4 * x["v"][:, :, 0].double().numpy()
    tol = 1e-6 if dtype == "fp32" else 2 ** -8 * np.abs(ref).max() + 1e-6
    assert maxerr(out[:, :, 0], ref) <= tol


def test_value_offset_property_fp32():
    # a value offset shared by every token comes out as (1 - lambda) * offset
    x = to_dev(prefill_inputs(1, 2, 2048, 64, "fp32", seed=13))
    c = torch.randn(128, device=DEV)
    lam = 0.3
    base = run_fwd(x, lam, True, False)
    x2 = dict(x, v=x["v"] + c)
    shifted = run_fwd(x2, lam, True, False)
    diff = (shifted - base - (1 - lam) * c).abs().max().item()
    assert diff <= 1e-4, diff


@pytest.mark.parametrize("D", [32, 64, 128])
def test_output_rounding_is_nearest_even(D):
    """The bf16 output is rounded to nearest, ties to even.  With one key (T = 1,
    or a decode cache of one row) and V = 1 the fp32 result is exactly
    1 - lambda; lambda = -2^-8 puts it halfway between bf16 1.0 (even) and
    1.0078125, lambda = -3 2^-8 halfway between 1.0078125 and 1.015625
    (even).  Nearest-even gives 1.0 and 1.015625; truncation gives 1.0 and
    1.0078125, round-half-up 1.0078125 and 1.015625."""
    lam = torch.tensor([-2.0 ** -8, -3.0 * 2.0 ** -8], dtype=torch.float32, device=DEV)
    want = torch.tensor([1.0, 1.015625], dtype=torch.float32, device=DEV)
    g = torch.Generator().manual_seed(77)
    q = torch.randn((1, 2, 1, D), generator=g).bfloat16().to(DEV)
    k = torch.randn((1, 2, 1, D), generator=g).bfloat16().to(DEV)
    v = torch.ones((1, 2, 1, 2 * D), dtype=torch.bfloat16, device=DEV)
    for causal in (True, False):
        say(f"rounding D={D} causal={causal}")
        out = da.diffattn_fwd(q, k, q, k, v, lam, causal=causal, headnorm=False)
        torch.cuda.synchronize()
        assert torch.equal(out[0, :, 0].float(), want[:, None].expand(2, 2 * D)), out[0, :, 0, :4]
    say(f"rounding decode D={D}")
    out = da.diffattn_decode(q[:, :, 0], k, q[:, :, 0], k, v, lam, headnorm=False)
    torch.cuda.synchronize()
    assert torch.equal(out[0].float(), want[:, None].expand(2, 2 * D)), out[0, :, :4]


def test_repeatable_bitwise():
    x = to_dev(prefill_inputs(2, 4, 1500, 64, "bf16", seed=21))
    a = run_fwd(x, 0.7, True, True)
    b = run_fwd(x, 0.7, True, True)
    assert torch.equal(a, b)


def test_side_stream_launch():
    """A launch given stream= waits for the inputs the current stream is still
    producing, keeps its own temporaries (a scalar lambda's vector, contiguous
    copies, a default workspace) on that stream, and gives the same bits as a
    launch on the current stream."""
    x = to_dev(prefill_inputs(2, 3, 700, 64, "bf16", seed=23))
    ref = run_fwd(x, 0.6, True, True)
    side = torch.cuda.Stream()
    for _ in range(3):
        # inputs produced by kernels queued on the current stream just before
        # the side-stream launch; q1 non-contiguous so the binding copies it
        q1 = (x["q1"].transpose(2, 3) * 1).transpose(2, 3)
        k1, q2, k2, v = (x[n] * 1 for n in ("k1", "q2", "k2", "v"))
        out = da.diffattn_fwd(q1, k1, q2, k2, v, 0.6, causal=True, headnorm=True, stream=side)
        side.synchronize()
        assert torch.equal(out, ref)
    xd = to_dev(decode_inputs(2, 3, 900, 64, "bf16", seed=24))
    dref = da.diffattn_decode(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], 0.7, num_splits=5)
    torch.cuda.synchronize()
    k1 = xd["k1"] * 1
    dout = da.diffattn_decode(xd["q1"], k1, xd["q2"], xd["k2"], xd["v"], 0.7, num_splits=5,
                              stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(dout, dref)


def test_fwd_rejects_empty():
    x = to_dev(prefill_inputs(1, 1, 4, 32, "bf16", seed=1))
    e = {k: v[:, :, :0] for k, v in x.items() if k in ("q1", "k1", "q2", "k2", "v")}
    with pytest.raises(RuntimeError):
        da.diffattn_fwd(e["q1"], e["k1"], e["q2"], e["k2"], e["v"], 0.5)


# ---- lambda --------------------------------------------------------------------

def test_lambda_kernel():
    g = torch.Generator().manual_seed(3)
    vecs = [torch.randn(16, 64, generator=g) * 0.1 for _ in range(4)]
    li = oracle.lambda_init_schedule(12)
    got = da.diffattn_lambda(*[v.to(DEV) for v in vecs], li)
    ref = oracle.reparam_lambda(*vecs, li)
    assert got.shape == (16,)
    assert np.max(np.abs(got.cpu().double().numpy() - ref)) <= 1e-6
    one = da.diffattn_lambda(*[v[0].to(DEV) for v in vecs], li)
    assert one.shape == () and abs(one.item() - ref[0]) <= 1e-6
    z = torch.zeros(16, 64, device=DEV)
    lz = da.diffattn_lambda(z, z, z, z, 0.7993953)
    assert torch.all(lz == torch.tensor(0.7993953, dtype=torch.float32))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_reparam_matches_two_calls(dtype):
    # lambda formed inside the prefill launch: same bits as diffattn_lambda
    # followed by diffattn_fwd, lambda_out equal to diffattn_lambda's output
    g = torch.Generator().manual_seed(17)
    for D, T, causal, headnorm, B, H, Dl in ((32, 129, True, False, 2, 3, 16), (64, 1000, True, True, 3, 4, 64),
                                             (64, 300, False, False, 1, 2, 64), (128, 257, False, True, 2, 2, 40),
                                             (64, 4500, True, False, 1, 2, 64)):
        x = to_dev(prefill_inputs(B, H, T, D, dtype, seed=600 + D + T))
        vecs = [(torch.randn(H, Dl, generator=g) * 0.1).to(DEV) for _ in range(4)]
        li = 0.6
        say(f"fwd_reparam {dtype} D={D} T={T} causal={causal} headnorm={headnorm} B={B} H={H}")
        lam = da.diffattn_lambda(*vecs, li)
        ref = da.diffattn_fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, causal=causal,
                              headnorm=headnorm, lambda_init=li)
        lam_out = torch.full((H,), float("nan"), device=DEV)
        got = da.diffattn_fwd_reparam(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], *vecs, li,
                                      causal=causal, headnorm=headnorm, lambda_out=lam_out)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (D, T)
        assert torch.equal(lam_out, lam), (D, T)
    # and against the oracle once, with lambda from the oracle's own formula
    xc = prefill_inputs(1, 2, 200, 64, dtype, seed=5)
    vc = [torch.randn(2, 32, generator=g) * 0.2 for _ in range(4)]
    out = da.diffattn_fwd_reparam(*(to_dev(xc)[k] for k in ("q1", "k1", "q2", "k2", "v")),
                                  *[v.to(DEV) for v in vc], 0.3, causal=True)
    torch.cuda.synchronize()
    lam_ref = oracle.reparam_lambda(*vc, 0.3)
    assert maxerr(out, ref_fwd(xc, torch.tensor(lam_ref), True, False)) <= TOL[dtype]


def test_lambda_chain_into_fwd():
    w = WORKLOADS["tiny_fp32_causal"]
    x = make_workload(w.name, "cpu")
    xd = to_dev(x)
    li_gpu = da.diffattn_lambda_init(w.layer)
    lam_gpu = da.diffattn_lambda(xd["lq1"], xd["lk1"], xd["lq2"], xd["lk2"], li_gpu)
    out = da.diffattn_fwd(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam_gpu,
                          causal=w.causal, headnorm=w.headnorm)
    torch.cuda.synchronize()
    lam_ref = oracle.reparam_lambda(x["lq1"], x["lk1"], x["lq2"], x["lk2"],
                                    oracle.lambda_init_schedule(w.layer))
    ref = oracle.diff_attention(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam_ref, w.causal)
    err = maxerr(out, ref)
    say(f"tiny fp32 workload: max err {err:.3e}")
    assert err <= TOL["fp32"]


# ---- decode --------------------------------------------------------------------

@pytest.mark.parametrize("headnorm", [False, True])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_sweep(dtype, D, headnorm):
    lam = torch.tensor([0.8, -0.2, 1.1], dtype=torch.float32)
    for L, splits in ((1, 0), (1, 1), (7, 3), (300, 0), (1000, 8), (4097, 0), (4097, 64), (10, 8)):
        x = decode_inputs(2, 3, L, D, dtype, seed=300 + L + D)
        say(f"decode {dtype} D={D} L={L} splits={splits} headnorm={headnorm}")
        xd = to_dev(x)
        out = da.diffattn_decode(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV),
                                 headnorm=headnorm, lambda_init=0.8, eps=1e-5, num_splits=splits)
        torch.cuda.synchronize()
        ref = oracle.diff_attention_decode(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam)
        if headnorm:
            ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
        err = maxerr(out, ref)
        assert err <= TOL[dtype], (L, splits, err)


def test_decode_split_invariance_and_last_row():
    x = to_dev(prefill_inputs(2, 2, 777, 64, "fp32", seed=44))
    fwd = run_fwd(x, 0.45, True, False)[:, :, -1]
    outs = []
    for s in (1, 2, 5, 16, 64, 777):
        o = da.diffattn_decode(x["q1"][:, :, -1], x["k1"], x["q2"][:, :, -1], x["k2"], x["v"],
                               0.45, num_splits=s)
        torch.cuda.synchronize()
        outs.append(o)
        assert (o - fwd).abs().max().item() <= 1e-5, s
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 1e-5


# ---- the named workloads at full size ------------------------------------------
#
# Every output row of the T=4096 workload; at T=32768 and at T=8192 (D=128)
# one row of every 32-row wave slice of every (b, h) (so every workgroup,
# every wave and the tile order the launch uses are covered), plus the first
# and last rows, random rows and the needle rows; every (b, h) row of the
# decode workload.  Each workload runs in the launch configuration
# bench.py times.

def _wave_rows(T, h, extra=(), rng=None, group=32):
    """One row of every ``group``-row slice (its position varying with the
    slice and the head), the first 24 and last 16 rows, 64 random rows and
    ``extra``."""
    rows = {group * g + (g * 37 + h * 11) % group for g in range((T + group - 1) // group)}
    rows |= set(range(min(T, 24))) | set(range(max(0, T - 16), T))
    if rng is not None:
        rows |= set(rng.choice(T, size=min(T, 64), replace=False).tolist())
    rows |= {r for r in extra if 0 <= r < T}
    return np.array(sorted(r for r in rows if r < T))


def _sample_rows(T, rng, extra=()):
    rows = set(range(min(T, 24))) | set(range(max(0, T - 16), T))
    rows |= set(rng.choice(T, size=min(T, 64), replace=False).tolist())
    rows |= {r for r in extra if 0 <= r < T}
    return np.array(sorted(rows))


def _launch_workload(name):
    """Inputs and output of the named prefill workload, launched as bench.py
    launches it (lambda from its vectors inside the prefill launch when the
    workload has vectors)."""
    w = WORKLOADS[name]
    x = make_workload(name, DEV)
    li = w.lambda_init if w.lambda_init is not None else oracle.lambda_init_schedule(w.layer)
    say(f"workload {name}: launching")
    if "lam" in x:
        lam_ref = x["lam"].cpu().double().numpy()
        out = da.diffattn_fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lam"], causal=w.causal,
                              headnorm=w.headnorm, lambda_init=li, eps=w.eps)
    else:
        lam_ref = oracle.reparam_lambda(x["lq1"].cpu(), x["lk1"].cpu(), x["lq2"].cpu(), x["lk2"].cpu(),
                                        oracle.lambda_init_schedule(w.layer))
        out = da.diffattn_fwd_reparam(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"],
                                      x["lq2"], x["lk2"], da.diffattn_lambda_init(w.layer), causal=w.causal,
                                      headnorm=w.headnorm, eps=w.eps)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    return w, x, out, lam_ref, li


def _check_rows(w, x, out, lam_ref, li, b, h, rows):
    sl = {k: x[k][b, h].double().cpu() for k in ("q1", "k1", "q2", "k2", "v")}  # exact upcast
    ref = oracle.diff_attention_rows(sl["q1"], sl["k1"], sl["q2"], sl["k2"], sl["v"], lam_ref[h],
                                     w.causal, rows)
    if w.headnorm:
        ref = oracle.head_rmsnorm(ref, li, w.eps)
    return maxerr(out[b, h, rows], ref)


def test_workload_prefill_t4k_every_row():
    w, x, out, lam_ref, li = _launch_workload("prefill_t4k_causal")
    worst = 0.0
    rows = np.arange(w.T)
    for b in range(w.B):
        for h in range(w.H):
            worst = max(worst, _check_rows(w, x, out, lam_ref, li, b, h, rows))
    say(f"workload prefill_t4k_causal: max err {worst:.3e} over all {w.B * w.H} heads x {w.T} rows")
    del x, out
    torch.cuda.empty_cache()
    assert worst <= TOL[w.dtype]


def test_workload_prefill_t32k_needles():
    w, x, out, lam_ref, li = _launch_workload("prefill_t32k_needles")
    rng = np.random.default_rng(w.seed)
    worst, n = 0.0, 0
    for b in range(w.B):
        for h in range(w.H):
            extra = []
            for j in x["needle_pos"][b, h].tolist():
                extra += [j, j + 1, j + 100]
            # the query rows the needles copy: their maps peak on the needle
            for i in x["needle_query"][b, h].tolist():
                extra += [i - 1, i, i + 1]
            rows = _wave_rows(w.T, h, extra, rng)
            n += len(rows)
            worst = max(worst, _check_rows(w, x, out, lam_ref, li, b, h, rows))
    say(f"workload prefill_t32k_needles: max err {worst:.3e} over {n} rows of {w.B * w.H} heads")
    del x, out
    torch.cuda.empty_cache()
    assert worst <= TOL[w.dtype]


def test_workload_full_t8k_d128():
    w, x, out, lam_ref, li = _launch_workload("full_t8k_d128")
    rng = np.random.default_rng(w.seed)
    worst, n = 0.0, 0
    for b in range(w.B):
        for h in range(w.H):
            rows = _wave_rows(w.T, h, (), rng)
            n += len(rows)
            worst = max(worst, _check_rows(w, x, out, lam_ref, li, b, h, rows))
    say(f"workload full_t8k_d128: max err {worst:.3e} over {n} rows of {w.B * w.H} heads")
    del x, out
    torch.cuda.empty_cache()
    assert worst <= TOL[w.dtype]


def test_workload_tiny_fp32():
    w = WORKLOADS["tiny_fp32_causal"]
    x = make_workload(w.name, "cpu")
    xd = to_dev(x)
    lam = da.diffattn_lambda(xd["lq1"], xd["lk1"], xd["lq2"], xd["lk2"], da.diffattn_lambda_init(1))
    out = da.diffattn_fwd(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam, causal=True)
    torch.cuda.synchronize()
    lam_ref = oracle.reparam_lambda(x["lq1"], x["lk1"], x["lq2"], x["lk2"], oracle.lambda_init_schedule(1))
    assert maxerr(out, oracle.diff_attention(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam_ref, True)) <= 1e-4


def test_workload_decode_l64k_every_row():
    w = WORKLOADS["decode_l64k"]
    say("workload decode_l64k: generating 16 GiB cache")
    x = make_workload(w.name, DEV)
    li = da.diffattn_lambda_init(w.layer)
    lam = da.diffattn_lambda(x["lq1"], x["lk1"], x["lq2"], x["lk2"], li)
    out = da.diffattn_decode(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam,
                             num_splits=w.num_splits)
    torch.cuda.synchronize()
    lam_ref = oracle.lambda_init_schedule(w.layer)  # zero vectors: lambda = lambda_init
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            # one (b, h) slice at a time, upcast exactly on the device
            sl = [x[k][b:b + 1, h:h + 1].double().cpu() for k in ("q1", "k1", "q2", "k2", "v")]
            ref = oracle.diff_attention_decode(*sl, lam_ref)
            worst = max(worst, maxerr(out[b:b + 1, h:h + 1], ref))
        say(f"workload decode_l64k: sequences 0..{b} done, max err {worst:.3e}")
    del x
    torch.cuda.empty_cache()
    assert worst <= TOL["bf16"]


# ---- sliding window (causal): row i sees keys i - W < j <= i ------------------

@pytest.mark.parametrize("headnorm", [False, True])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_fwd_window_sweep(D, headnorm):
    lam = torch.tensor([0.6, -0.2], dtype=torch.float32)
    for i, (T, W) in enumerate(((1, 1), (33, 1), (130, 5), (130, 32), (300, 64), (300, 100),
                                (300, 299), (300, 300), (1000, 257))):
        x = prefill_inputs(1, 2, T, D, "bf16", seed=7000 + D + 13 * i)
        say(f"fwd window bf16 D={D} T={T} W={W} headnorm={headnorm}")
        out = da.diffattn_fwd_window(*(to_dev(x)[k] for k in ("q1", "k1", "q2", "k2", "v")), lam.to(DEV), W,
                                     headnorm=headnorm, lambda_init=0.8, eps=1e-5)
        torch.cuda.synchronize()
        ref = oracle.diff_attention(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, True, window=W)
        if headnorm:
            ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
        err = maxerr(out, ref)
        assert err <= TOL["bf16"], (T, W, err)


def test_fwd_window_long_rows():
    # long rows and few heads (the 128-row one-map configuration with early
    # reads), windows wider than a tile: sampled rows, every key in range
    lam = torch.tensor([0.8, 0.3, -0.1, 1.1], dtype=torch.float32)
    for (B, H, T, W, seed) in ((1, 2, 5000, 700, 41), (2, 4, 3000, 1024, 42)):
        x = prefill_inputs(B, H, T, 64, "bf16", seed=seed)
        say(f"fwd window bf16 D=64 B={B} H={H} T={T} W={W}")
        lh = lam[:H]
        out = da.diffattn_fwd_window(*(to_dev(x)[k] for k in ("q1", "k1", "q2", "k2", "v")), lh.to(DEV), W)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(40), np.arange(T - 40, T), np.arange(W - 5, W + 5),
                                         np.random.default_rng(seed).choice(T, 150, replace=False)]))
        for b in range(B):
            for h in range(H):
                ref = oracle.diff_attention_rows(x["q1"][b, h], x["k1"][b, h], x["q2"][b, h], x["k2"][b, h],
                                                 x["v"][b, h], float(lh[h]), True, rows, window=W)
                assert maxerr(out[b, h, rows], ref) <= TOL["bf16"], (T, W, b, h)


@pytest.mark.parametrize("D,H", [(64, 32), (32, 64)])
def test_fwd_window_many_heads(D, H):
    # enough 192-row workgroups for one map per wave at three waves per
    # SIMD (D=64: 4 x 32 x 6 = 768, at least two per compute unit; D=32:
    # 4 x 64 x 6 = 1536, at least four).  Whole heads against the oracle, a
    # ragged T
    B, T, W = 4, 1000, 300
    x = prefill_inputs(B, H, T, D, "bf16", seed=43 + D)
    lam = torch.linspace(-0.2, 1.2, H)
    say(f"fwd window bf16 D={D} B={B} H={H} T={T} W={W}")
    for headnorm in (False, True):
        out = da.diffattn_fwd_window(*(to_dev(x)[k] for k in ("q1", "k1", "q2", "k2", "v")), lam.to(DEV), W,
                                     headnorm=headnorm, lambda_init=0.8, eps=1e-5)
        torch.cuda.synchronize()
        for (b, h) in ((0, 0), (1, 17), (3, H - 1)):
            ref = oracle.diff_attention_rows(x["q1"][b, h], x["k1"][b, h], x["q2"][b, h], x["k2"][b, h],
                                             x["v"][b, h], float(lam[h]), True, np.arange(T), window=W)
            if headnorm:
                ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
            assert maxerr(out[b, h], ref) <= TOL["bf16"], (b, h, headnorm)


# ---- ragged decode: sequence b sees its first lengths[b] cache rows -----------

@pytest.mark.parametrize("headnorm", [False, True])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_ragged(dtype, headnorm):
    lam = torch.tensor([0.8, -0.3], dtype=torch.float32)
    Lcap = 1500
    x = decode_inputs(5, 2, Lcap, 64, dtype, seed=9100)
    lengths = torch.tensor([0, 1, 777, 1500, 33], dtype=torch.int32)
    xd = to_dev(x)
    for splits in (0, 1, 7, 64):
        say(f"decode ragged {dtype} headnorm={headnorm} splits={splits}")
        out = da.diffattn_decode_ragged(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV),
                                        lengths.to(DEV), headnorm=headnorm, lambda_init=0.8, eps=1e-5,
                                        num_splits=splits)
        torch.cuda.synchronize()
        ref = oracle.diff_attention_decode_ragged(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam,
                                                  lengths.numpy())
        if headnorm:
            ref = oracle.head_rmsnorm(ref, 0.8, 1e-5)
        assert torch.count_nonzero(out[0]).item() == 0          # length 0: zero row
        assert maxerr(out, ref) <= TOL[dtype], splits
    # every length equal to the capacity is the plain decode, bit for bit
    full = torch.full((5,), Lcap, dtype=torch.int32, device=DEV)
    a = da.diffattn_decode_ragged(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV), full,
                                  headnorm=headnorm, num_splits=16)
    b = da.diffattn_decode(xd["q1"], xd["k1"], xd["q2"], xd["k2"], xd["v"], lam.to(DEV),
                           headnorm=headnorm, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- the measured workloads of the other rows, at their bench sizes -----------

def test_workload_prefill_t32k_window4k():
    """B1 H16 T32768 D64, 4096-key window: every head, one row of every
    32-row wave slice plus the rows around the window edge.  The oracle runs
    on the keys a group of rows can see, [first row - W + 1, last row]: the
    causal and window masks depend only on query - key, so the shift leaves
    its rows unchanged."""
    name = "prefill_t32k_window4k"
    w = WORKLOADS[name]
    x = make_workload(name, DEV)
    say(f"workload {name}: launching")
    out = da.diffattn_fwd_window(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lam"], w.window,
                                 headnorm=w.headnorm, lambda_init=w.lambda_init, eps=w.eps)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    lam_ref = x["lam"].cpu().double().numpy()
    worst = 0.0
    for h in range(w.H):
        rows = _wave_rows(w.T, h, [w.window - 2, w.window - 1, w.window, w.window + 1])
        sl = {k: x[k][0, h].double().cpu().numpy() for k in ("q1", "k1", "q2", "k2", "v")}
        for c0 in range(0, w.T, 256):
            r = rows[(rows >= c0) & (rows < c0 + 256)]
            if r.size == 0:
                continue
            k0, k1 = max(0, int(r[0]) - w.window + 1), int(r[-1]) + 1
            ref = oracle.diff_attention_rows(*(sl[k][k0:k1] for k in ("q1", "k1", "q2", "k2", "v")),
                                             lam_ref[h], True, r - k0, window=w.window)
            if w.headnorm:
                ref = oracle.head_rmsnorm(ref, w.lambda_init, w.eps)
            worst = max(worst, maxerr(out[0, h, r], ref))
        say(f"workload {name}: heads 0..{h} done, max err {worst:.3e}")
    del x, out
    torch.cuda.empty_cache()
    assert worst <= TOL[w.dtype]


def test_workload_decode_ragged_l64k():
    """B32 H16 L65536 D64 with the bench's seeded lengths: every (b, h) row,
    each cache slice upcast exactly on the device up to its sequence's
    length."""
    name = "decode_ragged_l64k"
    w = WORKLOADS[name]
    x = make_workload(name, DEV)
    li = da.diffattn_lambda_init(w.layer)
    lam = da.diffattn_lambda(x["lq1"], x["lk1"], x["lq2"], x["lk2"], li)
    say(f"workload {name}: launching")
    out = da.diffattn_decode_ragged(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, x["lengths"],
                                    num_splits=w.num_splits)
    torch.cuda.synchronize()
    lam_ref = oracle.reparam_lambda(x["lq1"].cpu(), x["lk1"].cpu(), x["lq2"].cpu(), x["lk2"].cpu(),
                                    oracle.lambda_init_schedule(w.layer))
    lengths = x["lengths"].cpu().numpy()
    worst = 0.0
    for b in range(w.B):
        n = int(lengths[b])
        for h in range(w.H):
            q = {k: x[k][b:b + 1, h:h + 1].double().cpu() for k in ("q1", "q2")}
            kv = {k: x[k][b:b + 1, h:h + 1, :n].double().cpu() for k in ("k1", "k2", "v")}
            ref = oracle.diff_attention_decode_ragged(q["q1"], kv["k1"], q["q2"], kv["k2"], kv["v"],
                                                      lam_ref[h:h + 1], np.array([n]))
            worst = max(worst, maxerr(out[b:b + 1, h:h + 1], ref))
        if b % 8 == 7:
            say(f"workload {name}: sequences 0..{b} done, max err {worst:.3e}")
    del x, out
    torch.cuda.empty_cache()
    assert worst <= TOL[w.dtype]
