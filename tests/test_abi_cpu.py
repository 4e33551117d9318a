"""The C ABI on the host: the library loads, exports what the header declares,
and rejects invalid arguments before any HIP call (no GPU needed).

Pointers passed here are fake addresses; validation only compares them and
returns before anything dereferences or launches.  The few checks that a
valid call gets past validation make it only where no HIP device is visible
(it then fails at the launch); with a device it would launch kernels on
unmapped addresses, so there they are skipped.
"""

import ctypes
import math
import os
import re

import pytest

import differential_attention_forward_amd as da
import oracle

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = da.DIFFATTN_F32, da.DIFFATTN_BF16


@pytest.fixture(scope="module")
def L():
    return da.lib()


def _no_device():
    import torch
    return torch.cuda.device_count() == 0  # counts devices without initialising one


def test_header_symbols_exported(L):
    names = da.header_functions()
    assert len(names) == 20, names
    assert "diffattn_fwd_reparam" in names and "diffattn_attention_fwd" in names
    assert "diffattn_v2_fwd" in names and "diffattn_v2_decode" in names
    assert "diffattn_fwd_train" in names and "diffattn_bwd" in names
    for n in names:
        assert hasattr(L, n), n


def test_micro_library_exports_its_header():
    from differential_attention_forward_amd import micro

    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                       "diffattn_micro.h")
    names = re.findall(r"^int (diffattn_micro_\w+)\(", open(hdr).read(), re.M)
    assert len(names) == 6 and set(names) == set(micro._SIGS)
    handle = micro.lib()
    for n in names:
        getattr(handle, n)


def test_status_strings(L):
    for s in range(5):
        assert da.diffattn_status_string(s)
    assert da.diffattn_status_string(99) == "unknown status"


def test_lambda_init_matches_oracle(L):
    for layer in (1, 2, 3, 12, 13, 24, 100):
        got = da.diffattn_lambda_init(layer)
        assert abs(got - oracle.lambda_init_schedule(layer)) <= 6e-8
    assert math.isnan(da.diffattn_lambda_init(0))
    # the same hand-computed values that pin the oracle (fp32 result)
    from tests.oracle_pins import LAMBDA_INIT_ROUNDED, LAMBDA_INIT_VALUES
    for layer, val in LAMBDA_INIT_VALUES.items():
        assert abs(da.diffattn_lambda_init(layer) - val) <= 1.5e-7, (layer, val)
    for layer, val in LAMBDA_INIT_ROUNDED.items():
        assert round(da.diffattn_lambda_init(layer), 3) == val


def test_decode_split_helpers(L):
    assert da.diffattn_decode_default_splits(32, 16, 65536) >= 1
    assert da.diffattn_decode_default_splits(1, 1, 100) == 1
    assert da.diffattn_decode_default_splits(0, 1, 1) == 0
    assert da.diffattn_decode_workspace_bytes(32, 16, 65536, 64, 64) == 32 * 16 * 64 * 2 * 130 * 4
    s = da.diffattn_decode_default_splits(2, 3, 5000)
    assert da.diffattn_decode_workspace_bytes(2, 3, 5000, 32, 0) == 2 * 3 * s * 2 * 66 * 4
    assert da.diffattn_decode_workspace_bytes(1, 1, 10, 64, 11) == 0
    assert da.diffattn_decode_workspace_bytes(1, 1, 10, 64, -1) == 0


# fake, well-separated, 256-byte aligned device addresses
BASE = 1 << 40
def P(i, off=0):
    return ctypes.c_void_p(BASE + i * (1 << 32) + off)


def fwd(L, dtype=BF16, B=1, H=2, T=8, D=64, ptrs=None, causal=1, headnorm=0, eps=1e-5):
    p = ptrs or [P(i) for i in range(7)]
    return L.diffattn_fwd(dtype, B, H, T, D, p[0], p[1], p[2], p[3], p[4], p[5], causal,
                          headnorm, ctypes.c_float(0.8), ctypes.c_float(eps), p[6], None)


def test_fwd_validation(L):
    assert fwd(L, ptrs=[P(0), None, P(2), P(3), P(4), P(5), P(6)]) == INVALID
    assert fwd(L, ptrs=[P(i) for i in range(6)] + [None]) == INVALID
    assert fwd(L, B=0) == INVALID
    assert fwd(L, H=0) == INVALID
    assert fwd(L, T=0) == INVALID
    assert fwd(L, headnorm=1, eps=0.0) == INVALID
    assert fwd(L, headnorm=1, eps=-1.0) == INVALID
    assert fwd(L, headnorm=1, eps=float("nan")) == INVALID
    assert fwd(L, dtype=7) == UNSUPPORTED
    for d in (16, 48, 96, 256):
        assert fwd(L, D=d) == UNSUPPORTED
    bad = [P(i) for i in range(7)]
    bad[2] = P(2, 8)
    assert fwd(L, ptrs=bad) == UNSUPPORTED
    bad = [P(i) for i in range(7)]
    bad[6] = P(6, 4)
    assert fwd(L, ptrs=bad) == UNSUPPORTED
    # out overlapping an input
    alias = [P(i) for i in range(7)]
    alias[6] = P(4, 256)
    assert fwd(L, ptrs=alias) == INVALID
    alias[6] = P(0)
    assert fwd(L, ptrs=alias) == INVALID


def fwdr(L, dtype=BF16, B=1, H=2, T=8, D=64, ptrs=None, vecs=None, Dl=16, lam_out=None,
         headnorm=0, eps=1e-5):
    p = ptrs or [P(i) for i in range(6)]
    vv = vecs or [P(10 + i) for i in range(4)]
    return L.diffattn_fwd_reparam(dtype, B, H, T, D, p[0], p[1], p[2], p[3], p[4], vv[0], vv[1],
                                  vv[2], vv[3], Dl, 1, headnorm, ctypes.c_float(0.8),
                                  ctypes.c_float(eps), lam_out, p[5], None)


def test_fwd_reparam_validation(L):
    # the tensor checks are those of diffattn_fwd
    assert fwdr(L, ptrs=[P(0), None, P(2), P(3), P(4), P(6)]) == INVALID
    assert fwdr(L, T=0) == INVALID
    assert fwdr(L, headnorm=1, eps=0.0) == INVALID
    assert fwdr(L, dtype=7) == UNSUPPORTED
    assert fwdr(L, D=48) == UNSUPPORTED
    # the lambda vectors and the optional lambda copy
    assert fwdr(L, vecs=[P(10), None, P(12), P(13)]) == INVALID
    assert fwdr(L, Dl=0) == INVALID
    assert fwdr(L, vecs=[P(10), P(11, 2), P(12), P(13)]) == UNSUPPORTED
    assert fwdr(L, lam_out=P(20, 2)) == UNSUPPORTED
    assert fwdr(L, lam_out=P(11, 4)) == INVALID          # lambda_out inside a vector
    assert fwdr(L, lam_out=P(5, 64)) == INVALID          # lambda_out inside out
    assert fwdr(L, lam_out=P(3, 16)) == INVALID          # lambda_out inside an input
    assert fwdr(L, vecs=[P(10), P(11), P(12), P(5, 8)]) == INVALID  # out over a vector
    # a valid call only fails at the launch: no GPU here, so it must not report
    # a validation error (OK or ERR_HIP)
    if _no_device():
        assert fwdr(L, lam_out=P(20)) in (OK, 4)


def att(L, dtype=BF16, B=1, H=2, T=8, D=128, ptrs=None):
    p = ptrs or [P(i) for i in range(4)]
    return L.diffattn_attention_fwd(dtype, B, H, T, D, p[0], p[1], p[2], 1, p[3], None)


def test_attention_validation(L):
    assert att(L, ptrs=[P(0), None, P(2), P(3)]) == INVALID
    assert att(L, ptrs=[P(0), P(1), P(2), None]) == INVALID
    assert att(L, B=0) == INVALID
    assert att(L, T=0) == INVALID
    assert att(L, dtype=F32) == UNSUPPORTED
    for d in (32, 96, 256):
        assert att(L, D=d) == UNSUPPORTED
    assert att(L, ptrs=[P(0), P(1, 8), P(2), P(3)]) == UNSUPPORTED
    assert att(L, ptrs=[P(0), P(1), P(2), P(2, 512)]) == INVALID   # out over v


def dec(L, dtype=BF16, B=1, H=2, Lk=64, D=64, splits=0, ws=None, wsb=1 << 20, ptrs=None):
    p = ptrs or [P(i) for i in range(7)]
    return L.diffattn_decode(dtype, B, H, Lk, D, p[0], p[1], p[2], p[3], p[4], p[5], 0,
                             ctypes.c_float(0.8), ctypes.c_float(1e-5), splits,
                             ws if ws is not None else P(8), wsb, p[6], None)


def test_decode_validation(L):
    assert dec(L, Lk=0) == INVALID
    assert dec(L, splits=-1) == INVALID
    assert dec(L, Lk=10, splits=11) == INVALID
    assert dec(L, D=80) == UNSUPPORTED
    assert dec(L, ws=ctypes.c_void_p(0)) == WORKSPACE
    need = da.diffattn_decode_workspace_bytes(1, 2, 64, 64, 4)
    assert dec(L, splits=4, wsb=need - 1) == WORKSPACE
    bad = [P(i) for i in range(7)]
    bad[1] = P(1, 2)
    assert dec(L, ptrs=bad) == UNSUPPORTED
    assert dec(L, ws=P(8, 8)) == UNSUPPORTED
    # workspace overlapping the value cache
    assert dec(L, ws=P(4, 64)) == INVALID


def dec_na(L, dtype=BF16, B=1, H=2, Lk=64, D=64, splits=0, ptrs=None):
    p = ptrs or [P(i) for i in range(7)]
    return L.diffattn_decode_noalloc(dtype, B, H, Lk, D, p[0], p[1], p[2], p[3], p[4], p[5], 0,
                                     ctypes.c_float(0.8), ctypes.c_float(1e-5), splits, p[6], None)


def test_decode_noalloc_validation(L):
    """Argument errors, and a split count whose partial states would not fit
    the library's array, are reported before the array is looked up."""
    assert dec_na(L, Lk=0) == INVALID
    assert dec_na(L, splits=-1) == INVALID
    assert dec_na(L, Lk=10, splits=11) == INVALID
    assert dec_na(L, D=80) == UNSUPPORTED
    bad = [P(i) for i in range(7)]
    bad[6] = P(4, 64)  # output inside the value cache
    assert dec_na(L, ptrs=bad) != OK
    nul = [P(i) for i in range(7)]
    nul[0] = None
    assert dec_na(L, ptrs=nul) == INVALID
    cap = da.DIFFATTN_NOALLOC_SCRATCH_BYTES
    assert da.diffattn_decode_workspace_bytes(1, 2, 8192, 128, 8192) > cap
    assert dec_na(L, Lk=8192, D=128, splits=8192) == WORKSPACE
    assert dec_na(L, B=4096, H=8, Lk=64, D=128, splits=1) == WORKSPACE


def test_noalloc_scratch_size_matches_header():
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "diffattn.h")
    m = re.search(r"#define DIFFATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(hdr).read())
    assert m and int(m.group(1)) << int(m.group(2)) == da.DIFFATTN_NOALLOC_SCRATCH_BYTES


def fwin(L, dtype=BF16, window=4, ptrs=None, T=8, D=64):
    p = ptrs or [P(i) for i in range(7)]
    return L.diffattn_fwd_window(dtype, 1, 2, T, D, p[0], p[1], p[2], p[3], p[4], p[5], window, 0,
                                 ctypes.c_float(0.8), ctypes.c_float(1e-5), p[6], None)


def test_fwd_window_validation(L):
    assert fwin(L, window=0) == INVALID
    assert fwin(L, window=-3) == INVALID
    assert fwin(L, dtype=F32) == UNSUPPORTED
    assert fwin(L, D=96) == UNSUPPORTED
    assert fwin(L, T=0) == INVALID
    assert fwin(L, ptrs=[P(0), P(1), P(2), P(3), P(4), None, P(6)]) == INVALID     # lambda
    assert fwin(L, ptrs=[P(0), P(1), P(2), P(3), P(4), P(5), P(4, 64)]) == INVALID  # out over v


def dense_strides(B, H, T, D):
    """(batch, head, row) element strides of dense q1, k1, q2, k2, v, out."""
    out = []
    for w in (D, D, D, D, 2 * D, 2 * D):
        out += [H * T * w, T * w, w]
    return out


def fstr(L, dtype=BF16, B=1, H=2, T=8, D=64, strides=None, ptrs=None, headnorm=0, eps=1e-5):
    p = ptrs or [P(i) for i in range(7)]
    st = strides if strides is not None else dense_strides(B, H, T, D)
    arr = (ctypes.c_longlong * 18)(*st) if st is not None else None
    return L.diffattn_fwd_strided(dtype, B, H, T, D, p[0], p[1], p[2], p[3], p[4], arr, p[5], 1,
                                  headnorm, ctypes.c_float(0.8), ctypes.c_float(eps), p[6], None)


def test_fwd_strided_validation(L):
    B, H, T, D = 1, 2, 8, 64
    st = dense_strides(B, H, T, D)
    assert L.diffattn_fwd_strided(BF16, B, H, T, D, P(0), P(1), P(2), P(3), P(4), None, P(5), 1, 0,
                                  ctypes.c_float(0.8), ctypes.c_float(1e-5), P(6), None) == INVALID
    assert fstr(L, ptrs=[P(0), None, P(2), P(3), P(4), P(5), P(6)]) == INVALID
    assert fstr(L, ptrs=[P(0), P(1), P(2), P(3), P(4), None, P(6)]) == INVALID   # lambda
    assert fstr(L, T=0) == INVALID
    assert fstr(L, headnorm=1, eps=0.0) == INVALID
    assert fstr(L, dtype=F32) == UNSUPPORTED
    assert fstr(L, D=96, strides=dense_strides(B, H, T, 96)) == UNSUPPORTED
    bad = list(st)
    bad[2] = -64                                                  # negative row stride
    assert fstr(L, strides=bad) == INVALID
    bad = list(st)
    bad[5] = 68                                                   # k1 row stride not 16-byte
    assert fstr(L, strides=bad) == UNSUPPORTED
    bad = list(st)
    bad[17] = 64                                                  # out rows of 128 overlap
    assert fstr(L, strides=bad) == INVALID
    bad = list(st)
    bad[16] = 0                                                   # both heads write one slice
    assert fstr(L, strides=bad) == INVALID
    bad = list(st)
    bad[14] = 1 << 27                                             # v row stride past 2 GiB
    assert fstr(L, T=64, strides=bad) == UNSUPPORTED
    # out's span reaches into v's
    assert fstr(L, ptrs=[P(0), P(1), P(2), P(3), P(4), P(5), P(4, 64)]) == INVALID
    # interleaved halves of one fused projection: q1 and q2 overlap as inputs (allowed);
    # the output may not land inside the fused buffer
    fused = [H * T * 2 * D, 2 * D, 2 * H * D]                     # a [B, T, H, 2D] view's strides
    st2 = fused + fused + fused + fused + [H * T * 2 * D, T * 2 * D, 2 * D] * 2
    ptrs = [P(0), P(1), P(0, 2 * D), P(1, 2 * D), P(4), P(5), P(0, 32)]
    assert fstr(L, strides=st2, ptrs=ptrs) == INVALID


def v2f(L, dtype=BF16, B=1, H=4, Hkv=2, T=8, D=64, ptrs=None):
    p = ptrs or [P(i) for i in range(6)]
    return L.diffattn_v2_fwd(dtype, B, H, Hkv, T, D, p[0], p[1], p[2], p[3], p[4], 1, p[5], None)


def test_v2_fwd_validation(L):
    assert v2f(L, ptrs=[P(0), None, P(2), P(3), P(4), P(5)]) == INVALID
    assert v2f(L, ptrs=[P(0), P(1), P(2), P(3), None, P(5)]) == INVALID   # lambda
    assert v2f(L, B=0) == INVALID
    assert v2f(L, Hkv=0) == INVALID
    assert v2f(L, H=6, Hkv=4) == INVALID                                  # H not a multiple
    assert v2f(L, dtype=F32) == UNSUPPORTED
    for d in (32, 96):
        assert v2f(L, D=d) == UNSUPPORTED
    assert v2f(L, ptrs=[P(0), P(1), P(2, 8), P(3), P(4), P(5)]) == UNSUPPORTED
    assert v2f(L, ptrs=[P(0), P(1), P(2), P(3), P(4), P(3, 64)]) == INVALID   # out over v


def v2d(L, dtype=BF16, B=1, H=4, Hkv=2, Lk=64, D=64, splits=0, ws=None, wsb=1 << 20, ptrs=None):
    p = ptrs or [P(i) for i in range(6)]
    return L.diffattn_v2_decode(dtype, B, H, Hkv, Lk, D, p[0], p[1], p[2], p[3], p[4], splits,
                                ws if ws is not None else P(8), wsb, p[5], None)


def test_v2_decode_validation(L):
    assert v2d(L, Lk=0) == INVALID
    assert v2d(L, H=6, Hkv=4) == INVALID
    assert v2d(L, splits=-1) == INVALID
    assert v2d(L, Lk=10, splits=11) == INVALID
    assert v2d(L, H=16, Hkv=2) == UNSUPPORTED                            # group of 8
    assert v2d(L, dtype=F32) == UNSUPPORTED
    assert v2d(L, D=32) == UNSUPPORTED
    assert v2d(L, ws=ctypes.c_void_p(0)) == WORKSPACE
    need = da.diffattn_v2_decode_workspace_bytes(1, 4, 2, 64, 64, 4)
    assert need == 1 * 4 * 4 * 2 * (64 + 2) * 4
    assert v2d(L, splits=4, wsb=need - 1) == WORKSPACE
    assert v2d(L, ws=P(3, 64)) == INVALID                                # workspace over v
    assert da.diffattn_v2_decode_workspace_bytes(1, 4, 2, 0, 64) == 0


def test_decode_ragged_validation(L):
    p = [P(i) for i in range(7)]

    def rag(lens, ws=None, wsb=1 << 20):
        return L.diffattn_decode_ragged(BF16, 2, 2, 64, 64, p[0], p[1], p[2], p[3], p[4], p[5], lens, 0,
                                        ctypes.c_float(0.8), ctypes.c_float(1e-5), 0,
                                        ws if ws is not None else P(8), wsb, p[6], None)
    assert rag(None) == INVALID
    assert rag(P(9, 2)) == UNSUPPORTED           # misaligned lengths
    assert rag(P(6, 4)) == INVALID               # lengths inside the output
    assert rag(P(8, 16)) == INVALID              # lengths inside the workspace
    assert rag(P(9), ws=ctypes.c_void_p(0)) == WORKSPACE


def test_lambda_validation(L):
    p = [P(i) for i in range(5)]
    f = ctypes.c_float(0.2)
    assert L.diffattn_lambda(p[0], p[1], p[2], p[3], 0, 8, f, p[4], None) == INVALID
    assert L.diffattn_lambda(p[0], p[1], p[2], p[3], 2, 0, f, p[4], None) == INVALID
    assert L.diffattn_lambda(None, p[1], p[2], p[3], 2, 8, f, p[4], None) == INVALID
    assert L.diffattn_lambda(p[0], p[1], p[2], p[3], 2, 8, f, P(0, 4), None) == INVALID
    assert L.diffattn_lambda(p[0], p[1], p[2], p[3], 2, 8, f, P(4, 2), None) == UNSUPPORTED


def test_binding_requires_device_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 32)
    with pytest.raises(TypeError):
        da.diffattn_fwd(x, x, x, x, torch.zeros(1, 1, 4, 64), 0.5)


def test_training_sizes(L):
    b, h, t, d = 2, 3, 100, 64
    assert da.diffattn_train_saved_bytes(b, h, t, d) == 2 * b * h * t * 2 * d * 4 + b * h * 2 * t * 4
    tp = 128
    ws = (b * h * t * 2 * d * 2 + 255) // 256 * 256 + (b * h * 4 * tp * 4 + 255) // 256 * 256 + b * h * 2 * 4
    assert da.diffattn_bwd_workspace_bytes(b, h, t, d) == ws
    assert da.diffattn_train_saved_bytes(1, 1, 8, 32) == 2 * 8 * 64 * 4 + 2 * 8 * 4
    for args in ((0, 1, 8, 64), (1, 1, 0, 64), (1, 1, 8, 16), (1, 1, 8, 96)):
        assert da.diffattn_train_saved_bytes(*args) == 0
        assert da.diffattn_bwd_workspace_bytes(*args) == 0


def fwdt(L, dtype=BF16, B=1, H=2, T=8, D=64, ptrs=None, saved_bytes=1 << 20):
    p = ptrs or [P(i) for i in range(8)]
    return L.diffattn_fwd_train(dtype, B, H, T, D, p[0], p[1], p[2], p[3], p[4], p[5], 1, 0,
                                ctypes.c_float(0.8), ctypes.c_float(1e-5), p[6], p[7],
                                saved_bytes, None)


def test_fwd_train_validation(L):
    assert fwdt(L, ptrs=[P(i) for i in range(7)] + [None]) == INVALID
    assert fwdt(L, ptrs=[P(0), None] + [P(i) for i in range(2, 8)]) == INVALID
    assert fwdt(L, T=0) == INVALID
    assert fwdt(L, dtype=F32) == UNSUPPORTED
    for d in (16, 96):
        assert fwdt(L, D=d) == UNSUPPORTED
    assert fwdt(L, saved_bytes=da.diffattn_train_saved_bytes(1, 2, 8, 64) - 1) == WORKSPACE
    bad = [P(i) for i in range(8)]
    bad[7] = P(7, 8)
    assert fwdt(L, ptrs=bad) == UNSUPPORTED
    alias = [P(i) for i in range(8)]
    alias[7] = P(6, 256)       # saved inside out
    assert fwdt(L, ptrs=alias) == INVALID
    alias[7] = P(4)            # saved over v
    assert fwdt(L, ptrs=alias) == INVALID
    if _no_device():
        assert fwdt(L) in (OK, 4)


def bwd(L, dtype=BF16, B=1, H=2, T=8, D=64, ins=None, outs=None, vecs=None, dvecs=None, Dl=16,
        saved_bytes=1 << 20, ws=None, wsb=1 << 20, headnorm=0, eps=1e-5):
    i = ins or [P(k) for k in range(8)]          # q1 k1 q2 k2 v lambda dout saved
    o = outs or [P(10 + k) for k in range(6)]    # dq1 dk1 dq2 dk2 dv dlambda
    vv = vecs if vecs is not None else [None] * 4
    dv = dvecs if dvecs is not None else [None] * 4
    return L.diffattn_bwd(dtype, B, H, T, D, i[0], i[1], i[2], i[3], i[4], i[5], i[6], i[7],
                          saved_bytes, 1, headnorm, ctypes.c_float(0.8), ctypes.c_float(eps),
                          o[0], o[1], o[2], o[3], o[4], o[5], vv[0], vv[1], vv[2], vv[3], Dl,
                          dv[0], dv[1], dv[2], dv[3], ws if ws is not None else P(30), wsb, None)


def test_bwd_validation(L):
    vecs = [P(20 + k) for k in range(4)]
    dvecs = [P(24 + k) for k in range(4)]
    assert bwd(L, ins=[P(0), None] + [P(k) for k in range(2, 8)]) == INVALID
    assert bwd(L, ins=[P(k) for k in range(7)] + [None]) == INVALID
    assert bwd(L, outs=[P(10 + k) for k in range(5)] + [None]) == INVALID
    assert bwd(L, T=0) == INVALID
    assert bwd(L, headnorm=1, eps=0.0) == INVALID
    assert bwd(L, vecs=vecs, dvecs=[P(24), P(25), None, P(27)]) == INVALID   # some, not all
    assert bwd(L, vecs=vecs, dvecs=dvecs, Dl=0) == INVALID
    assert bwd(L, dtype=F32) == UNSUPPORTED
    assert bwd(L, D=96) == UNSUPPORTED
    assert bwd(L, ins=[P(0), P(1, 8)] + [P(k) for k in range(2, 8)]) == UNSUPPORTED
    assert bwd(L, vecs=[P(20), P(21, 2), P(22), P(23)], dvecs=dvecs) == UNSUPPORTED
    assert bwd(L, saved_bytes=da.diffattn_train_saved_bytes(1, 2, 8, 64) - 1) == WORKSPACE
    assert bwd(L, wsb=da.diffattn_bwd_workspace_bytes(1, 2, 8, 64) - 1) == WORKSPACE
    assert bwd(L, ws=ctypes.c_void_p(0)) == WORKSPACE
    # outputs overlapping inputs, each other, or the workspace
    assert bwd(L, outs=[P(10), P(11), P(12), P(13), P(4, 256), P(15)]) == INVALID   # dv over v
    assert bwd(L, outs=[P(10), P(10, 512), P(12), P(13), P(14), P(15)]) == INVALID  # dk1 over dq1
    assert bwd(L, outs=[P(10), P(11), P(12), P(13), P(14), P(7, 16)]) == INVALID    # dlambda in saved
    assert bwd(L, ws=P(6)) == INVALID                                                # workspace over dout
    assert bwd(L, vecs=vecs, dvecs=[P(24), P(25), P(26), P(20)]) == INVALID          # dlk2 over lq1
    if _no_device():
        assert bwd(L, vecs=vecs, dvecs=dvecs) in (OK, 4)
        assert bwd(L) in (OK, 4)


# fake device addresses 2^40 bytes apart, for shapes whose tensors exceed 4 GiB
def F(i):
    return ctypes.c_void_p((1 << 40) * (i + 1))


def test_grid_limits(L):
    """Shapes whose launch grid one dispatch cannot express (more than 2^32 - 1
    work-items) are refused with ERR_UNSUPPORTED before anything runs; the
    largest accepted shapes get past validation."""
    far = [F(i) for i in range(8)]
    # prefill / training / backward: 4 B H (T + 255) <= 2^32 - 1
    H = 1 << 20
    assert 4 * H * (768 + 255) <= 2 ** 32 - 1 < 4 * H * (769 + 255)
    assert fwd(L, B=1, H=H, T=769, D=32, ptrs=far[:7]) == UNSUPPORTED
    assert att(L, B=1, H=H, T=769, D=64, ptrs=far[:4]) == UNSUPPORTED
    assert fwdt(L, B=1, H=H, T=769, D=32, ptrs=far) == UNSUPPORTED
    assert bwd(L, B=1, H=H, T=769, D=32, ins=far, outs=[F(10 + k) for k in range(6)],
               ws=F(20)) == UNSUPPORTED
    assert da.diffattn_train_saved_bytes(1, H, 769, 32) == 0
    assert da.diffattn_bwd_workspace_bytes(1, H, 769, 32) == 0
    assert da.diffattn_train_saved_bytes(1, H, 768, 32) > 0
    # decode: B H S split-K workgroups of 256 threads
    big_ws = 1 << 39
    assert dec(L, B=1024, H=256, Lk=64, D=32, splits=64, ws=F(8), wsb=big_ws, ptrs=far[:7]) == UNSUPPORTED
    assert v2d(L, B=1024, H=256, Hkv=256, Lk=64, D=64, splits=64, ws=F(8), wsb=big_ws,
               ptrs=far[:6]) == UNSUPPORTED
    # lambda: one 64-thread workgroup per head
    p = [F(i) for i in range(5)]
    assert L.diffattn_lambda(p[0], p[1], p[2], p[3], 1 << 26, 8, ctypes.c_float(0.2), p[4],
                             None) == UNSUPPORTED
    if _no_device():
        assert fwd(L, B=1, H=H, T=768, D=32, ptrs=far[:7]) in (OK, 4)
        assert dec(L, B=1024, H=255, Lk=64, D=32, splits=64, ws=F(8), wsb=big_ws,
                   ptrs=far[:7]) in (OK, 4)
        assert L.diffattn_lambda(p[0], p[1], p[2], p[3], (1 << 26) - 1, 8, ctypes.c_float(0.2),
                                 p[4], None) in (OK, 4)
