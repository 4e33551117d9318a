"""Measured ceilings of one MI355X (gfx950), from libdiffattn_micro.so
(``csrc/micro.hip``, declared in ``include/diffattn_micro.h``).

Each function launches one microbenchmark kernel on the current stream,
times it with HIP events on that stream and returns what it measured:

* mfma: bf16 v_mfma_f32_32x32x16_bf16 throughput (TFLOP/s), its issue
  interval per SIMD in shader clocks, and the shader clock the waves ran at
  (s_memtime cycles over s_memrealtime ticks of 10 ns);
* hbm_read, hbm_copy: streaming HBM bandwidth (GB/s, 1e9 bytes);
* lds_dma: global -> LDS DMA stream bandwidth (the prefill's tile staging);
* lds_read: LDS bytes per clock per CU for ds_read_b128 and for
  ds_read_b64_tr_b16;
* valu: shader clocks per VALU instruction on a wave (fp32 add, v_dot2c,
  v_exp) alone on its SIMD and next to an MFMA-streaming wave.

Measurement only: nothing on the attention path calls this module.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None
_VP, _I, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "diffattn_micro_mfma": [_I, _I, _VP, _SZ, _VP, _SZ, _VP],
    "diffattn_micro_hbm_read": [_VP, _SZ, _I, _VP, _SZ, _VP],
    "diffattn_micro_hbm_copy": [_VP, _VP, _SZ, _I, _VP],
    "diffattn_micro_lds_dma": [_VP, _SZ, _I, _VP, _SZ, _VP],
    "diffattn_micro_lds_read": [_I, _I, _I, _VP, _SZ, _VP, _SZ, _VP],
    "diffattn_micro_valu": [_I, _I, _I, _I, _VP, _SZ, _VP, _SZ, _VP],
}
MFMA_FLOPS = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16
REALTIME_HZ = 100e6  # s_memrealtime


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libdiffattn_micro.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m differential_attention_forward_amd.build`")
        h = ctypes.CDLL(path)
        for name, args in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = _I
            fn.argtypes = args
        _lib = h
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(err: int, what: str) -> None:
    if err != 0:
        raise RuntimeError(f"{what}: HIP error {err}")


def _time_ms(launch, reps: int) -> float:
    launch()  # warm-up (clocks, code object load)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        launch()
    t1.record()
    t1.synchronize()
    return t0.elapsed_time(t1) / reps


def _waves(clk: torch.Tensor):
    """(cycles, realtime ticks) per timed wave from the clock records."""
    c = clk.view(-1, 4).cpu().double()
    timed = c[:, 3] > c[:, 2]
    return (c[timed, 1] - c[timed, 0]), (c[timed, 3] - c[timed, 2])


def _cus() -> int:
    return torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count


def _bufs(blocks: int, threads: int = 512):
    sink = torch.empty(blocks * threads, device="cuda", dtype=torch.float32)
    clk = torch.zeros(blocks * (threads // 64) * 4, device="cuda", dtype=torch.int64)
    return sink, clk


def mfma(iters: int = 60000, reps: int = 3) -> dict:
    blocks = 2 * _cus()  # 16 waves per CU, 4 per SIMD
    sink, clk = _bufs(blocks)
    L = lib()

    def launch():
        clk.zero_()
        _check(L.diffattn_micro_mfma(blocks, iters, sink.data_ptr(), sink.numel(), clk.data_ptr(),
                                     clk.numel(), _stream()), "micro mfma")

    ms = _time_ms(launch, reps)
    cyc, ticks = _waves(clk)
    ghz = float(cyc.sum() / ticks.sum()) * REALTIME_HZ / 1e9
    flops = blocks * 8 * iters * 8 * MFMA_FLOPS
    per_simd = blocks * 8 * iters * 8 / (4 * _cus())  # MFMAs each SIMD's pipe ran
    return {
        "tflops": flops / (ms * 1e-3) / 1e12,
        "clock_ghz": ghz,
        # the waves of a SIMD share its matrix pipe and need not run side by
        # side, so the issue interval comes from the kernel's duration
        "cycles_per_mfma_per_simd": ms * 1e-3 * ghz * 1e9 / per_simd,
        "tflops_at_2p4ghz": flops / (ms * 1e-3) / 1e12 * 2.4 / ghz,
        "ms": ms,
    }


GRIDS_PER_CU = (2, 4, 8, 16, 32)  # grid sizes the streaming benchmarks try; the best counts


def hbm_read(nbytes: int = 4 << 30, reps: int = 5) -> dict:
    src = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    L = lib()
    best = None
    for g in GRIDS_PER_CU:
        blocks = g * _cus()
        sink, _ = _bufs(blocks, 256)
        ms = _time_ms(lambda: _check(L.diffattn_micro_hbm_read(src.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                                               sink.numel(), _stream()), "micro hbm_read"), reps)
        if best is None or ms < best[0]:
            best = (ms, blocks)
    return {"gbs": nbytes / (best[0] * 1e-3) / 1e9, "bytes": nbytes, "ms": best[0], "blocks": best[1]}


def hbm_copy(nbytes: int = 2 << 30, reps: int = 5) -> dict:
    src = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    dst = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    L = lib()
    best = None
    for g in GRIDS_PER_CU:
        blocks = g * _cus()
        ms = _time_ms(lambda: _check(L.diffattn_micro_hbm_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks,
                                                               _stream()), "micro hbm_copy"), reps)
        if best is None or ms < best[0]:
            best = (ms, blocks)
    return {"gbs": 2 * nbytes / (best[0] * 1e-3) / 1e9, "bytes_each_way": nbytes, "ms": best[0],
            "blocks": best[1]}


def lds_dma(nbytes: int = 4 << 30, reps: int = 5) -> dict:
    unit = 8192 * max(GRIDS_PER_CU) * _cus()
    nbytes -= nbytes % unit
    src = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    L = lib()
    best = None
    for g in GRIDS_PER_CU:
        blocks = g * _cus()
        sink, _ = _bufs(blocks)
        ms = _time_ms(lambda: _check(L.diffattn_micro_lds_dma(src.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                                              sink.numel(), _stream()), "micro lds_dma"), reps)
        if best is None or ms < best[0]:
            best = (ms, blocks)
    return {"gbs": nbytes / (best[0] * 1e-3) / 1e9, "bytes": nbytes, "ms": best[0], "blocks": best[1]}


def lds_read(transposing: bool, iters: int = 20000, reps: int = 3) -> dict:
    blocks = _cus()
    sink, clk = _bufs(blocks)
    L = lib()

    def launch():
        clk.zero_()
        _check(L.diffattn_micro_lds_read(int(transposing), blocks, iters, sink.data_ptr(), sink.numel(),
                                         clk.data_ptr(), clk.numel(), _stream()), "micro lds_read")

    _time_ms(launch, reps)
    cyc, _ = _waves(clk)
    per_instr = 512 if transposing else 1024
    return {"bytes_per_clk_cu": 8 * iters * 8 * per_instr / float(cyc.max()),
            "instr": "ds_read_b64_tr_b16" if transposing else "ds_read_b128"}


def valu(kind: int, with_mfma: bool, iters: int = 4000) -> float:
    """Shader clocks per instruction of a VALU wave (kind 0 add, 1 v_dot2c,
    2 v_exp, 3 v_exp alternating with adds, 4 v_exp alternating with bf16
    pair conversions), alone on its SIMD or next to an MFMA-streaming wave."""
    blocks = _cus()
    sink, clk = _bufs(blocks)
    L = lib()
    mfma_iters = 13 * iters if with_mfma else 0  # outlasts the VALU waves at up to 100 clocks per op

    def launch():
        clk.zero_()
        _check(L.diffattn_micro_valu(kind, mfma_iters, blocks, iters, sink.data_ptr(), sink.numel(),
                                     clk.data_ptr(), clk.numel(), _stream()), "micro valu")

    _time_ms(launch, 2)
    cyc, _ = _waves(clk)
    return float(cyc.mean()) / (iters * 32)


def run_all() -> dict:
    """Every microbenchmark once (about two seconds on one MI355X)."""
    out = {"mfma_bf16": mfma(), "hbm_read": hbm_read(), "hbm_copy": hbm_copy(), "lds_dma": lds_dma(),
           "lds_read_b128": lds_read(False), "lds_read_tr16": lds_read(True)}
    names = ("add_f32", "dot2c_f32_bf16", "exp_f32", "exp_f32_with_add_f32", "exp_f32_with_cvt_pk_bf16")
    out["valu_clocks_per_op"] = {n: {"alone": valu(k, False), "beside_mfma": valu(k, True)}
                                 for k, n in enumerate(names)}
    torch.cuda.empty_cache()
    return out
