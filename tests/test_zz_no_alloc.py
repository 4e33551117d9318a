"""diffattn_decode_noalloc, the decode entry point that allocates nothing,
against diffattn_decode with a workspace of its own: the same kernels on the
same inputs, so the outputs must agree bit for bit.  Two calls in a row, the
second smaller, so the second runs on what the first left in the library's
array; then a call whose partial states would not fit is refused."""

import ctypes

import pytest
import torch

import differential_attention_forward_amd as da
from workloads import decode_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _both(B, H, L, D, dtype, seed, splits, headnorm):
    x = {k: t.to(DEV) for k, t in decode_inputs(B, H, L, D, dtype, seed=seed).items()}
    lam = torch.linspace(0.2, 0.9, H, dtype=torch.float32, device=DEV)
    ref = da.diffattn_decode(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, headnorm=headnorm,
                             lambda_init=0.5, num_splits=splits)
    out = torch.full_like(ref, float("nan"))
    da.diffattn_decode_noalloc(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam,
                               headnorm=headnorm, lambda_init=0.5, num_splits=splits, out=out)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_workspace_decode_twice(dtype):
    cases = ((4, 8, 5000, 128, 0, True), (1, 2, 700, 64, 3, False))
    for i, (B, H, L, D, splits, hn) in enumerate(cases):
        need = da.diffattn_decode_workspace_bytes(B, H, L, D, splits)
        assert 0 < need <= da.DIFFATTN_NOALLOC_SCRATCH_BYTES
        say(f"noalloc {dtype} B={B} H={H} L={L} D={D} splits={splits} headnorm={hn}")
        out, ref = _both(B, H, L, D, dtype, 4100 + i, splits, hn)
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref)


def test_noalloc_refuses_oversized_split_state():
    say("noalloc oversized")
    x = {k: t.to(DEV) for k, t in decode_inputs(1, 2, 8192, 128, "bf16", seed=4200).items()}
    lam = torch.full((2,), 0.5, dtype=torch.float32, device=DEV)
    assert da.diffattn_decode_workspace_bytes(1, 2, 8192, 128, 8192) > da.DIFFATTN_NOALLOC_SCRATCH_BYTES
    out = torch.empty((1, 2, 256), dtype=torch.bfloat16, device=DEV)
    st = da.lib().diffattn_decode_noalloc(
        da.DIFFATTN_BF16, 1, 2, 8192, 128, x["q1"].data_ptr(), x["k1"].data_ptr(), x["q2"].data_ptr(),
        x["k2"].data_ptr(), x["v"].data_ptr(), lam.data_ptr(), 0, ctypes.c_float(0.8),
        ctypes.c_float(1e-5), 8192, out.data_ptr(), None)
    assert st == 3  # DIFFATTN_ERR_WORKSPACE, before any launch
