#!/usr/bin/env python3
"""Throughput of the differential-attention forward on one MI355X.

One "step" is one pass of the path over one batch of synthetic input that is
already resident in HBM:
  prefill workloads   one prefill kernel; when the workload derives lambda
                      from its four vectors, that kernel forms it too
                      (diffattn_fwd_reparam)
  decode workload     lambda kernel + split-K partial kernel + reduce kernel

Before the W warm-up steps each workload runs untimed steps for about
SETTLE_S seconds, so that the GPU clock has ramped up before timing starts
(a handful of sub-millisecond steps is not enough for that).

The printed JSON line reports the primary workload (default: the causal T=4096
bf16 prefill, B2 H16 D64, head norm on) as TFLOP/s counted as
8 * T_eff * T * D * B * H per forward (T_eff = (T+1)/2 causal, T full), and
the other workloads (causal T=32768, full T=8192 D=128, decode L=65536, and
the DIFF V2 prefill and decode with grouped KV heads) under "also", together
with standard softmax attention of the same size as the two causal workloads
(head width 2D) and the time ratio of the two.  "roofline" gives the dominant kernel's algorithmic rate (from HIP
events around each launch on the launch stream) against the MI355X peak
(bf16 dense MFMA 2.5 PFLOP/s, fp32 MFMA 157.3 TFLOP/s, HBM 8 TB/s).
"cpu_baseline" times the float64 oracle on the host cores on a bounded sample
of the primary workload.  "micro" holds the measured ceilings of this GPU
(differential_attention_forward_amd/micro.py: bf16 MFMA throughput and the
shader clock it runs at, HBM read and copy, the global -> LDS DMA stream, LDS
read rates, VALU issue beside an MFMA stream), and each roofline adds its
bound's measured ceiling ("measured_peak", "frac_of_measured").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DiffAttn fwd TFLOP/s (bf16 causal T=4k/32k) & % MFMA peak; decode HBM GB/s"
PEAK = {"bf16_mfma_tflops": 2500.0, "fp32_mfma_tflops": 157.3, "hbm_gbs": 8000.0}
PRIMARY = "prefill_t4k_causal"
OTHERS = ["prefill_t32k_needles", "full_t8k_d128", "decode_l64k", "v2_prefill_t4k", "v2_decode_l64k",
          "bwd_t4k_causal", "bwd_t4k_d128", "prefill_t32k_window4k", "decode_ragged_l64k"]
CSRC = os.path.join(ROOT, "differential_attention_forward_amd", "csrc")
KERNEL_FILE = {"prefill": "prefill.hip", "decode": "decode.hip", "v2_decode": "decode.hip",
               "backward": "backward.hip"}
KERNEL_NAME = {"prefill": "fwd_bf16_kernel", "decode": "decode_partial_kernel",
               "v2_decode": "decode_v2_mma_kernel"}
# which kernel dominates each workload kind (the backward has four of comparable weight)
KIND_KERNEL = {"prefill": "prefill", "v2_prefill": "prefill", "window_prefill": "prefill",
               "decode": "decode", "ragged_decode": "decode", "v2_decode": "v2_decode"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kind):
    h = hashlib.sha256()
    for f in (KERNEL_FILE[kind], "common.h", "kernels.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def dominant_kernel(w):
    """The kernel that does a workload's work: the launch choice of the
    library's prefill dispatch (bf16, D = 64, causal, T > 4096 rows: the
    ping-pong kernel; other prefill shapes: fwd_bf16_kernel)."""
    kind = KIND_KERNEL[w.kind]
    if kind == "prefill" and w.kind == "prefill" and w.dtype == "bf16" and w.D == 64 and w.causal and w.T > 4096:
        return "fwd_pp_kernel"
    return KERNEL_NAME[kind]


def measured_traffic(kind, kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}:{workload}")
    if not rec or rec.get("source_hash") != source_hash(kind):
        return None
    return rec.get("bytes_per_launch")


def visible_pairs(w):
    """(query, key) pairs a head's mask allows: T^2 full, T(T+1)/2 causal,
    sum_i min(i + 1, W) with a sliding window W."""
    if w.window and w.window < w.T:
        wn = w.window
        return wn * (wn + 1) / 2.0 + (w.T - wn) * float(wn)
    return w.T * (w.T + 1) / 2.0 if w.causal else float(w.T) * w.T


def prefill_flops(w):
    """Per visible (query, key) pair and head: two D-wide score dot products
    and one signed weighted sum over the value row (2D wide in the first
    version, D wide in V2), 2 flops per multiply-add.  Backward: the two
    score recomputations (4D), dP = dOpre V^T (4D), dV from the signed map
    (4D), dQ1 and dQ2 (4D), dK1 and dK2 (4D): 20 D per pair."""
    per_pair = {"v2_prefill": 6.0, "bwd": 20.0}.get(w.kind, 8.0) * w.D
    return per_pair * visible_pairs(w) * w.B * w.H


def decode_bytes(w, lengths=None):
    """Cache bytes one step must read: K1, K2 (D) and V (2D) per key and head;
    V2: one K and one V (D each) per key and KV head; ragged: the filled rows
    of each sequence only."""
    es = 2 if w.dtype == "bf16" else 4
    if w.kind == "v2_decode":
        return float(w.B * w.Hkv * w.T * 2 * w.D * es)
    keys = float(sum(int(n) for n in lengths)) if lengths is not None else float(w.B * w.T)
    return keys * w.H * 4 * w.D * es


SETTLE_S = 0.4


def settle(torch, step, seconds=SETTLE_S):
    """Untimed steps for about `seconds` of wall time (clock ramp-up)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n


def time_steps(torch, step, steps, warmup):
    settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_kernel(torch, launch, steps):
    """Mean, median and minimum duration of one launch, from events recorded
    around each launch on the current (launch) stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return sum(t) / steps, t[len(t) // 2], t[0]


def bench_workload(torch, da, name, steps, warmup, keep=False):
    """Times the named workload.  With ``keep``, also returns its inputs and
    the output of the timed launches (for the oracle comparison)."""
    from workloads import WORKLOADS, make_workload

    w = WORKLOADS[name]
    log(f"[bench] {name}: generating inputs")
    x = make_workload(name, "cuda")
    torch.cuda.synchronize()
    li = w.lambda_init if w.lambda_init is not None else (
        da.diffattn_lambda_init(w.layer) if w.layer else 0.0)  # V2 has no lambda_init-scaled norm
    lam = x.get("lam")
    lam_buf = torch.empty(w.H, device="cuda", dtype=torch.float32)
    if w.kind == "bwd":
        lamv, out = x["lam"], None
        _, saved = da.diffattn_fwd_train(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lamv, causal=w.causal,
                                         headnorm=w.headnorm, lambda_init=li, eps=w.eps)
        ws = torch.empty(max(da.diffattn_bwd_workspace_bytes(w.B, w.H, w.T, w.D), 16), device="cuda",
                         dtype=torch.uint8)

        def kernel():
            da.diffattn_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lamv, x["dout"], saved,
                            causal=w.causal, headnorm=w.headnorm, lambda_init=li, eps=w.eps, workspace=ws)
    elif w.kind == "window_prefill":
        out = torch.empty_like(x["v"])

        def kernel():
            da.diffattn_fwd_window(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, w.window,
                                   headnorm=w.headnorm, lambda_init=li, eps=w.eps, out=out)
    elif w.kind == "ragged_decode":
        out = torch.empty((w.B, w.H, 2 * w.D), device="cuda", dtype=x["v"].dtype)
        ws = torch.empty(da.diffattn_decode_workspace_bytes(w.B, w.H, w.T, w.D, w.num_splits) // 4,
                         device="cuda", dtype=torch.float32)

        def kernel():
            da.diffattn_decode_ragged(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam_buf, x["lengths"],
                                      num_splits=w.num_splits, workspace=ws, out=out)
    elif w.kind == "v2_prefill":
        out = torch.empty_like(x["q1"])

        def kernel():
            da.diffattn_v2_fwd(x["q1"], x["q2"], x["k"], x["v"], lam, causal=w.causal, out=out)
    elif w.kind == "v2_decode":
        out = torch.empty((w.B, w.H, w.D), device="cuda", dtype=x["q1"].dtype)
        ws = torch.empty(da.diffattn_v2_decode_workspace_bytes(w.B, w.H, w.Hkv, w.T, w.D, w.num_splits) // 4,
                         device="cuda", dtype=torch.float32)

        def kernel():
            da.diffattn_v2_decode(x["q1"], x["q2"], x["k"], x["v"], lam, num_splits=w.num_splits,
                                  workspace=ws, out=out)
    elif w.kind == "prefill":
        out = torch.empty_like(x["v"])

        if lam is not None:
            def kernel():
                da.diffattn_fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, causal=w.causal,
                                headnorm=w.headnorm, lambda_init=li, eps=w.eps, out=out)
        else:
            # lambda from its four vectors inside the prefill launch (the
            # whole path, lambda included, is this one kernel)
            def kernel():
                da.diffattn_fwd_reparam(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"],
                                        x["lq2"], x["lk2"], li, causal=w.causal, headnorm=w.headnorm,
                                        eps=w.eps, out=out)
    else:
        out = torch.empty((w.B, w.H, 2 * w.D), device="cuda", dtype=x["v"].dtype)
        ws = torch.empty(da.diffattn_decode_workspace_bytes(w.B, w.H, w.T, w.D, w.num_splits) // 4,
                         device="cuda", dtype=torch.float32)

        def kernel():
            da.diffattn_decode(x["q1"], x["k1"], x["q2"], x["k2"], x["v"],
                               lam if lam is not None else lam_buf, headnorm=w.headnorm,
                               lambda_init=li, eps=w.eps, num_splits=w.num_splits,
                               workspace=ws, out=out)

    def step():
        if lam is None and w.kind in ("decode", "ragged_decode"):
            da.diffattn_lambda(x["lq1"], x["lk1"], x["lq2"], x["lk2"], li, out=lam_buf)
        kernel()

    log(f"[bench] {name}: {warmup} warmup + {steps} timed steps")
    ms, wall = time_steps(torch, step, steps, warmup)
    kern_ms, kern_med, kern_min = time_kernel(torch, kernel, steps)
    log(f"[bench] {name}: {ms:.4f} ms/step, kernel {kern_ms:.4f} ms")
    if w.kind in ("prefill", "v2_prefill", "bwd", "window_prefill"):
        work = prefill_flops(w)
        value = work / (ms * 1e-3) / 1e12
        achieved = work / (kern_ms * 1e-3) / 1e12
        peak = PEAK["bf16_mfma_tflops"] if w.dtype == "bf16" else PEAK["fp32_mfma_tflops"]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": (measured_traffic("prefill", dominant_kernel(w), name) if w.kind in KIND_KERNEL
                            else measured_traffic("backward", "bwd_kernels", name)),
                "kernel": "bwd_prep + bwd_kv + bwd_q + bwd_lambda kernels" if w.kind == "bwd" else dominant_kernel(w),
                "algorithmic_per_launch": work}
        unit = "TFLOP/s"
    else:
        work = decode_bytes(w, x["lengths"].tolist() if "lengths" in x else None)
        value = work / (ms * 1e-3) / 1e9
        achieved = work / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_gbs"],
                "unit": "GB/s", "frac": round(achieved / PEAK["hbm_gbs"], 4),
                "traffic": measured_traffic(KIND_KERNEL[w.kind], dominant_kernel(w), name),
                "kernel": dominant_kernel(w),
                "algorithmic_per_launch": work}
        unit = "GB/s"
    res = {"workload": name, "value": round(value, 3), "unit": unit, "ms_per_step": round(ms, 5),
           "kernel_ms": round(kern_ms, 5), "kernel_ms_median": round(kern_med, 5),
           "kernel_ms_min": round(kern_min, 5), "wall_s": round(wall, 4), "roofline": roof,
           "shape": {"B": w.B, "H": w.H, ("L" if w.kind.endswith("decode") else "T"): w.T, "D": w.D,
                     "causal": False if w.kind.endswith("decode") else w.causal,
                     "headnorm": w.headnorm, "dtype": w.dtype, **({"Hkv": w.Hkv} if w.Hkv else {}),
                     **({"window": w.window} if w.window else {})}}
    if keep:
        return res, x, out
    del x, out
    torch.cuda.empty_cache()
    return res


def attach_measured_peak(res, measured):
    """Adds the microbenchmarked ceiling of the workload's bound (bf16 MFMA
    throughput at the clock it sustains, or streaming HBM read) to its
    roofline, with the achieved rate as a fraction of it."""
    roof = res.get("roofline") if isinstance(res, dict) else None
    if not roof or "achieved" not in roof:
        return
    if roof["bound"] == "mfma" and roof["peak"] == PEAK["bf16_mfma_tflops"]:
        m = measured["mfma_bf16"]["tflops"]
    elif roof["bound"] == "hbm":
        m = measured["hbm_read"]["gbs"]
    else:
        return
    roof["measured_peak"] = round(m, 1)
    roof["frac_of_measured"] = round(roof["achieved"] / m, 4)


def bench_same_size_attention(torch, da, name, steps, warmup, diff_ms):
    """Standard softmax attention of the same size as the named causal
    differential workload (head width 2D, same B, H, T, same 8 T_eff T D B H
    flops): the comparison the glossary page makes between the two kinds of
    model, here on the forward kernels alone."""
    from workloads import WORKLOADS, attention_inputs

    w = WORKLOADS[name]
    x = attention_inputs(w.B, w.H, w.T, 2 * w.D, seed=w.seed + 100, device="cuda")
    out = torch.empty_like(x["v"])

    def step():
        da.diffattn_attention_fwd(x["q"], x["k"], x["v"], causal=w.causal, out=out)

    ms, _ = time_steps(torch, step, steps, warmup)
    work = prefill_flops(w)
    log(f"[bench] same-size standard attention for {name}: {ms:.4f} ms/step")
    del x, out
    torch.cuda.empty_cache()
    return {"workload": f"standard attention, B{w.B} H{w.H} T{w.T} head width {2 * w.D}, "
                        f"{'causal' if w.causal else 'full'}, bf16",
            "value": round(work / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
            "differential_over_standard_time": round(diff_ms / ms, 4)}


def bench_fused_views(torch, da, name, steps, warmup):
    """The named causal workload with Q1|Q2 and K1|K2 as the halves of fused
    token-major [B, T, H, 2D] projections, V read from and the output written
    to token-major [B, T, H, 2D] buffers, through the strided entry point (no
    copies), against what the dense entry point costs once the four views are
    copied out to dense tensors first."""
    from workloads import WORKLOADS, make_workload

    w = WORKLOADS[name]
    x = make_workload(name, "cuda")
    li = w.lambda_init if w.lambda_init is not None else da.diffattn_lambda_init(w.layer)
    lam = da.diffattn_lambda(x["lq1"], x["lk1"], x["lq2"], x["lk2"], li) if "lam" not in x else x["lam"]

    def fused(a, b):
        buf = torch.cat([a.permute(0, 2, 1, 3), b.permute(0, 2, 1, 3)], dim=-1).contiguous()
        return buf[..., :w.D].permute(0, 2, 1, 3), buf[..., w.D:].permute(0, 2, 1, 3)

    q1, q2 = fused(x["q1"], x["q2"])
    k1, k2 = fused(x["k1"], x["k2"])
    v = x["v"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    out = torch.empty((w.B, w.T, w.H, 2 * w.D), device="cuda", dtype=x["v"].dtype).permute(0, 2, 1, 3)
    dense_out = torch.empty_like(x["v"])
    del x

    def strided():
        da.diffattn_fwd_strided(q1, k1, q2, k2, v, lam, causal=w.causal, headnorm=w.headnorm,
                                lambda_init=li, eps=w.eps, out=out)

    def copy_then_dense():
        da.diffattn_fwd(q1, k1, q2, k2, v, lam, causal=w.causal, headnorm=w.headnorm, lambda_init=li,
                        eps=w.eps, out=dense_out)  # the binding makes the inputs contiguous first

    ms, _ = time_steps(torch, strided, steps, warmup)
    ms_copy, _ = time_steps(torch, copy_then_dense, steps, warmup)
    work = prefill_flops(w)
    log(f"[bench] fused-projection views for {name}: {ms:.4f} ms/step strided, {ms_copy:.4f} with copies")
    del q1, q2, k1, k2, v, out, dense_out
    torch.cuda.empty_cache()
    return {"workload": f"{name} on token-major fused-projection views (strided entry point)",
            "value": round(work / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
            "ms_per_step_copy_then_dense": round(ms_copy, 5)}


def cpu_baseline(torch, name, x, out, budget_s=12.0):
    """The float64 oracle, as it stands, on the host cores: whole heads of the
    workload (every query row of each (b, h), on the inputs the timed kernel
    read, with the workload's own lambda and lambda_init) until ~budget_s
    seconds, and the largest |GPU - oracle| over the output rows of those
    heads that the timed kernel wrote."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from workloads import WORKLOADS

    w = WORKLOADS[name]
    li = w.lambda_init if w.lambda_init is not None else oracle.lambda_init_schedule(w.layer)
    if "lam" in x:
        lam = x["lam"].cpu().double().numpy()
    else:
        lam = oracle.reparam_lambda(x["lq1"].cpu(), x["lk1"].cpu(), x["lq2"].cpu(), x["lk2"].cpu(), li)
    heads, worst, t0 = 0, 0.0, time.perf_counter()
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    for (b, h) in pairs:
        sl = {k: x[k][b, h].cpu() for k in ("q1", "k1", "q2", "k2", "v")}
        o = oracle.diff_attention_rows(sl["q1"], sl["k1"], sl["q2"], sl["k2"], sl["v"], lam[h],
                                       w.causal, np.arange(w.T))
        if w.headnorm:
            o = oracle.head_rmsnorm(o, li, w.eps)
        heads += 1
        worst = max(worst, float(np.max(np.abs(out[b, h].float().cpu().numpy().astype(np.float64) - o))))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = prefill_flops(w) / (w.B * w.H) * heads
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": model,
            "max_abs_err": worst, "tolerance": 2e-2 if w.dtype == "bf16" else 1e-4,
            "sample": f"{heads} of {w.B * w.H} (b,h) heads of {name}, all {w.T} query rows, "
                      f"float64 numpy (includes the per-head comparison with the timed kernel's "
                      f"output), {dt:.1f} s wall, host os.cpu_count()={os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=PRIMARY)
    ap.add_argument("--primary-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--micro", action="store_true",
                    help="only run the microbenchmarks (measured MFMA, HBM, LDS-DMA, LDS and VALU "
                         "ceilings and the shader clock under MFMA load) and print them")
    ap.add_argument("--no-micro", action="store_true", help="skip the microbenchmarks")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times): the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over (batch, head) with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import differential_attention_forward_amd as da
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20)
        src = torch.ones(n // 4, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)
        return
    if args.micro:
        from differential_attention_forward_amd import micro

        print(json.dumps({"micro": micro.run_all(), "gpu": torch.cuda.get_device_name(0)}), flush=True)
        return
    da.lib()
    w = WORKLOADS[args.workload]
    want_cpu = not args.no_cpu_baseline and w.kind == "prefill"
    if want_cpu:
        primary, px, pout = bench_workload(torch, da, args.workload, args.steps, args.warmup, keep=True)
        # the oracle runs after the other workloads; its inputs and the timed
        # output move to host memory meanwhile
        px = {k: v.cpu() for k, v in px.items() if isinstance(v, torch.Tensor)}
        pout = pout.cpu()
        torch.cuda.empty_cache()
    else:
        primary = bench_workload(torch, da, args.workload, args.steps, args.warmup)
    also = {}
    if not args.primary_only:
        for name in OTHERS + [PRIMARY]:
            if name != args.workload and name not in also:
                also[name] = bench_workload(torch, da, name, args.steps, args.warmup)
        for name in ("prefill_t4k_causal", "prefill_t32k_needles"):
            diff_ms = (primary if name == args.workload else also[name])["ms_per_step"]
            also[f"same_size_attention_{name}"] = bench_same_size_attention(
                torch, da, name, args.steps, args.warmup, diff_ms)
        also["fused_views_prefill_t4k_causal"] = bench_fused_views(
            torch, da, "prefill_t4k_causal", args.steps, args.warmup)
    measured = None
    if not args.no_micro:
        from differential_attention_forward_amd import micro

        log("[bench] microbenchmarks (measured ceilings)")
        measured = micro.run_all()
        for res in [primary, *also.values()]:
            attach_measured_peak(res, measured)
    cpu = None
    if want_cpu:
        log("[bench] cpu baseline (float64 oracle) and its comparison with the timed output")
        cpu = cpu_baseline(torch, args.workload, px, pout)
    line = {
        "metric": METRIC, "value": primary["value"], "unit": primary["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": primary["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": args.workload, **primary["shape"]},
        "roofline": primary["roofline"], "cpu_baseline": cpu,
        "micro": measured,
        "also": also,
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
