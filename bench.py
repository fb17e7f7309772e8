#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's layer forward (bf16) on one MI355X.

A step is one pass of the per-rank hot path over one batch of synthetic input
already resident in HBM: QKV column-parallel GEMM + bias, attention
out-projection row-parallel GEMM, fc1 column-parallel GEMM with fused bias +
GeLU (or SwiGLU), fc2 row-parallel GEMM (and for the MoE workload the router
and the grouped expert GEMMs).  The default workload is one rank's share of a
GPT-3 175B-shaped layer at TP=8 (2048 tokens); --workload picks another.

Timing is cold by default: before every timed step an untimed 1 GiB write
evicts the 256 MB memory-side cache (the rank's weights would otherwise stay
resident across steps), and each step is bracketed by HIP events.  The same
steps back to back (warm) are timed as well and reported beside it.

Prints one JSON line: TFLOP/s (algorithmic 2*M*N*K over the step's GEMMs),
the dominant kernel's roofline position (HIP events around that kernel in
every timed step, on the stream the kernels are launched on; events without
the system-scope cache fence, so timing does not flush the caches) against
the nominal dense bf16 peak and against a peak calibrated on this GPU with an
MFMA-only loop, and the CPU oracle timed on a bounded sample of the same
workload on this host's cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk
MFMA_FP8_PEAK_TFLOPS = 5033.2    # dense fp8 MFMA: twice the bf16 rate
HBM_PEAK_GBS = 8000.0
METRIC = "TFLOP/s per TP-rank QKV+MLP forward (bf16) and % of MI355X MFMA peak"
WORKLOADS = {"gpt345m": 1, "gpt3_175b_rank0": 2, "llama70b_rank0": 3, "moe": 4, "tiny": 0}


KERNEL_SOURCES = ("gemm_kernel.h", "gemm.h", "gemm.hip", "gemm_fwd_col.hip", "gemm_fwd_swiglu.hip", "gemm_fwd_row.hip",
                  "gemm_grouped.hip", "moe.hip", "rope.hip")


def kernel_source_hash():
    """Hash of the sources of the forward GEMM, grouped-GEMM, MoE and RoPE kernels: a counter record taken on
    other sources is not used."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "megatron_tensor_transformer_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel_label, cold=True):
    """HBM bytes per launch of the dominant kernel (in cold or warm steps) from the committed rocprofv3 counter
    runs, if they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(workload, {}).get(kernel_label)
    if not e or e.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e["hbm_bytes_per_launch" if cold else "hbm_bytes_per_launch_warm"]


class _FenceFreeEvents:
    """HIP events (created with hipEventDisableSystemFence) recorded on one stream, for timing only."""
    _FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, stream_handle):
        import ctypes
        self._c = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._stream = ctypes.c_void_p(stream_handle)

    def record(self):
        e = self._c.c_void_p()
        if self._hip.hipEventCreateWithFlags(self._c.byref(e), self._FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        if self._hip.hipEventRecord(e, self._stream) != 0:
            raise RuntimeError("hipEventRecord failed")
        return e

    def elapsed_ms(self, e0, e1):
        ms = self._c.c_float()
        if self._hip.hipEventElapsedTime(self._c.byref(ms), e0, e1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def release(self, events):
        for e in events:
            self._hip.hipEventDestroy(e)


def backward_gemms(w, timer, reps=5):
    """The backward GEMMs of the workload's linears (dgrad dX = dY . Wt, wgrad dWt = dY^T . X into fp32),
    on synthetic operands of the same shapes: event time per launch (median of reps) and TFLOP/s."""
    import torch
    import megatron_tensor_transformer_03_amd as mtp
    import synth
    per, flop_total, us_total = {}, 0, 0.0
    for i, (label, M, N, K) in enumerate(w.gemms):
        if label in per:  # shards of one linear: the same shapes
            continue
        X = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        Wt = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
        dY = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        synth.gpu_normal_bf16_(X, 9001 + 3 * i, 1.0)
        synth.gpu_normal_bf16_(Wt, 9002 + 3 * i, 0.02)
        synth.gpu_normal_bf16_(dY, 9003 + 3 * i, 1.0)
        dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        dW = torch.zeros(N, K, dtype=torch.float32, device="cuda")
        ws = mtp.workspace_for([(M, K, N, "dgrad"), (N, K, M, "wgrad")])
        res = {}
        for name, fn in (("dgrad", lambda: mtp.mtp_linear_dgrad(dY, Wt, None, False, dX, workspace=ws)),
                         ("wgrad", lambda: mtp.mtp_linear_wgrad(dY, X, dW, True, workspace=ws))):
            fn()
            torch.cuda.synchronize()
            ev = []
            for _ in range(reps):
                e0 = timer.record()
                fn()
                ev.append((e0, timer.record()))
            torch.cuda.synchronize()
            t = sorted(timer.elapsed_ms(a, b) for a, b in ev)[reps // 2]
            timer.release([e for pair in ev for e in pair])
            res[name + "_us"] = round(1000 * t, 2)
            res[name + "_tflops"] = round(2 * M * N * K / (t * 1e-3) / 1e12, 1)
            flop_total += 2 * M * N * K
            us_total += 1000 * t
        per[label] = res
        del X, Wt, dY, dX, dW
    tf = flop_total / (us_total * 1e-6) / 1e12
    return {"per_linear": per, "flop": flop_total, "us": round(us_total, 2), "achieved": round(tf, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}


def _median_us(timer, fn, reps=5):
    import torch
    fn()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        e0 = timer.record()
        fn()
        ev.append((e0, timer.record()))
    torch.cuda.synchronize()
    t = sorted(timer.elapsed_ms(a, b) for a, b in ev)[reps // 2]
    timer.release([e for pair in ev for e in pair])
    return 1000 * t


def norm_and_bda(w, timer):
    """The norm prologue and the bias-dropout-add epilogue at the workload's shapes (synthetic operands):
    the row-statistics kernel against the HBM roofline, and the fused GEMMs beside the plain ones."""
    import torch
    import megatron_tensor_transformer_03_amd as mtp
    import synth
    shapes = {label: (M, N, K) for label, M, N, K in w.gemms}
    if "qkv" not in shapes or "fc2" not in shapes:
        return None
    kind = mtp.NORM_RMS if w.dims.get("act") == mtp.ACT_SWIGLU else mtp.NORM_LAYER
    M, N, H = shapes["qkv"]
    X = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    Wt = torch.empty(N, H, dtype=torch.bfloat16, device="cuda")
    g = torch.empty(1, H, dtype=torch.bfloat16, device="cuda")
    synth.gpu_normal_bf16_(X, 9101, 1.0)
    synth.gpu_normal_bf16_(Wt, 9102, 0.02)
    synth.gpu_normal_bf16_(g, 9103, 0.1)
    g.add_(1.0)
    stats = torch.empty(M, 2, dtype=torch.float32, device="cuda")
    Wf = torch.empty_like(Wt)
    colsum = torch.empty(N, dtype=torch.float32, device="cuda")
    bias_f = torch.empty(N, dtype=torch.float32, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    beta = None if kind == mtp.NORM_RMS else g
    cs = None if kind == mtp.NORM_RMS else colsum
    t_stats = _median_us(timer, lambda: mtp.mtp_norm_stats(X, stats, kind, 1e-5))
    t_fold = _median_us(timer, lambda: mtp.mtp_norm_fold_weights(Wt, g[0], None if beta is None else beta[0], None,
                                                                 Wf, cs, bias_f))
    ws = mtp.workspace_for([(M, N, H, mtp.ACT_NONE)])
    t_fused = _median_us(timer, lambda: mtp.mtp_norm_column_linear(X, stats, Wf, cs, bias_f, Y, workspace=ws))
    t_plain = _median_us(timer, lambda: mtp.mtp_column_linear(X, Wt, None, Y, workspace=ws))
    stat_bytes = M * H * 2 + 8 * M
    gbs = stat_bytes / (t_stats * 1e-6) / 1e9
    del Wt, Wf, Y
    # fc2 with the bias-dropout-add epilogue (p = 0.1, a synthetic keep mask) beside the plain bf16 epilogue
    M2, N2, K2 = shapes["fc2"]
    Z = torch.empty(M2, K2, dtype=torch.bfloat16, device="cuda")
    W2 = torch.empty(N2, K2, dtype=torch.bfloat16, device="cuda")
    R = torch.empty(M2, N2, dtype=torch.bfloat16, device="cuda")
    synth.gpu_normal_bf16_(Z, 9104, 1.0)
    synth.gpu_normal_bf16_(W2, 9105, 0.02)
    synth.gpu_normal_bf16_(R, 9106, 1.0)
    keep = torch.from_numpy(synth.keep_bits(9107, M2, N2, 0.1)).cuda()
    Y2 = torch.empty(M2, N2, dtype=torch.bfloat16, device="cuda")
    ws2 = mtp.workspace_for([(M2, N2, K2, mtp.ACT_NONE)])
    t_bda = _median_us(timer, lambda: mtp.mtp_row_linear_bda(Z, W2, R, Y2, keep=keep, p_drop=0.1, workspace=ws2))
    t_row = _median_us(timer, lambda: mtp.mtp_row_linear_partial(Z, W2, None, False, None, Y2, workspace=ws2))
    return {"norm": "rmsnorm" if kind == mtp.NORM_RMS else "layernorm",
            "stats_kernel": {"bound": "hbm", "us": round(t_stats, 2), "bytes": stat_bytes, "achieved": round(gbs, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "fold_us_once_per_weight_update": round(t_fold, 2),
            "qkv_norm_epilogue_us": round(t_fused, 2), "qkv_plain_us": round(t_plain, 2),
            "fc2_bias_dropout_add_us": round(t_bda, 2), "fc2_plain_us": round(t_row, 2)}


def fp8_gemms(w, timer):
    """The workload's linears as E4M3 GEMMs (per-tensor scaled codes of synthetic operands): the GEMM against
    the dense fp8 MFMA peak beside the bf16 one, and the activation quantization against the HBM roofline."""
    import torch
    import megatron_tensor_transformer_03_amd as mtp
    import synth
    per, flop_total, us_total, q_total = {}, 0, 0.0, 0.0
    for i, (label, M, N, K) in enumerate(w.gemms):
        if label in per:
            continue
        act = mtp.ACT_SWIGLU if (label == "fc1" and w.dims.get("act") == mtp.ACT_SWIGLU) else mtp.ACT_NONE
        X = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        Wt = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
        synth.gpu_normal_bf16_(X, 9201 + 2 * i, 1.0)
        synth.gpu_normal_bf16_(Wt, 9202 + 2 * i, 0.02)
        Xq = torch.empty(M, K, dtype=torch.uint8, device="cuda")
        Wq = torch.empty(N, K, dtype=torch.uint8, device="cuda")
        amax = torch.zeros(mtp.FP8_WS_FLOATS, dtype=torch.float32, device="cuda")
        sx = torch.zeros(1, dtype=torch.float32, device="cuda")
        sw = torch.zeros(1, dtype=torch.float32, device="cuda")
        mtp.mtp_fp8_quantize(Wt, Wq, amax, sw)
        nout = N // 2 if act == mtp.ACT_SWIGLU else N
        Y = torch.empty(M, nout, dtype=torch.bfloat16, device="cuda")
        t_q = _median_us(timer, lambda: mtp.mtp_fp8_quantize(X, Xq, amax, sx))
        hist = torch.full((16,), 4.5, dtype=torch.float32, device="cuda")
        t_qd = _median_us(timer, lambda: mtp.mtp_fp8_quantize_delayed(X, Xq, hist, 3, amax, sx))
        ws = mtp.workspace_for([(M, N, K, ("fp8", act))])
        t_g = _median_us(timer, lambda: mtp.mtp_fp8_column_linear(Xq, sx, Wq, sw, None, Y, act, workspace=ws))
        fl = 2 * M * N * K
        # HBM bytes: current scaling reads X twice (amax, then codes) and writes the codes; delayed scaling
        # reads it once
        qb, qdb = 5 * M * K, 3 * M * K
        per[label] = {"gemm_us": round(t_g, 2), "tflops": round(fl / (t_g * 1e-6) / 1e12, 1),
                      "quantize_us": round(t_q, 2), "quantize_gbs": round(qb / (t_q * 1e-6) / 1e9, 1),
                      "quantize_delayed_us": round(t_qd, 2),
                      "quantize_delayed_gbs": round(qdb / (t_qd * 1e-6) / 1e9, 1)}
        flop_total += fl
        us_total += t_g
        q_total += t_q
        del X, Wt, Xq, Wq, Y
    tf = flop_total / (us_total * 1e-6) / 1e12
    return {"per_linear": per, "achieved": round(tf, 1), "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_FP8_PEAK_TFLOPS, 4), "gemm_us": round(us_total, 2),
            "quantize_us": round(q_total, 2)}


def prenorm_layer(w, timer, steps=10):
    """The composed TP = 1 pre-norm layer (norm-folded QKV, attention bias-dropout-add, norm-folded fc1, MLP
    bias-dropout-add; core attention aside): microseconds per step and per launch."""
    import torch
    import megatron_tensor_transformer_03_amd as mtp
    from megatron_tensor_transformer_03_amd.layer import PreNormLayer
    import synth
    if w.dims.get("p", 1) != 1 or "nq" not in w.dims or "E" in w.dims:
        return None
    hx = synth.prenorm_inputs(w)
    dev = lambda a: torch.from_numpy(a.view("int16")).cuda().view(torch.bfloat16)
    ex = {k: dev(hx[k]) for k in ("g1", "beta1", "g2", "beta2")}
    ex.update(keep1=torch.from_numpy(hx["keep1"]).cuda(), keep2=torch.from_numpy(hx["keep2"]).cuda(),
              p_drop=hx["p_drop"])
    kind = mtp.NORM_RMS if w.dims.get("act") == mtp.ACT_SWIGLU else mtp.NORM_LAYER
    layer = PreNormLayer(w.dims, synth.device_inputs(w), ex, kind)
    for _ in range(3):
        layer.step()
    torch.cuda.synchronize()
    per = {}
    for _ in range(3):
        marks = []
        layer.step(lambda label: marks.append((label, timer.record())))
        torch.cuda.synchronize()
        for (label, e0), (_, e1) in zip(marks[:-1], marks[1:]):
            per.setdefault(label, []).append(1000 * timer.elapsed_ms(e0, e1))
        timer.release(e for _, e in marks)
    e0 = timer.record()
    for _ in range(steps):
        layer.step()
    e1 = timer.record()
    torch.cuda.synchronize()
    us = 1000 * timer.elapsed_ms(e0, e1) / steps
    timer.release([e0, e1])
    gemm_flop = sum(2 * m * n * k for _, m, n, k in w.gemms)
    return {"us_per_step": round(us, 2), "gemm_tflops": round(gemm_flop / (us * 1e-6) / 1e12, 1),
            "per_launch_us": {k: round(sum(v) / len(v), 2) for k, v in per.items()}}


def cpu_baseline(w, budget_s):
    """The oracle on a bounded row sample of the same workload; TFLOP/s of algorithmic work done."""
    import numpy as np
    import oracle
    import synth
    d = w.dims
    t0 = time.perf_counter()
    if "E" in d:
        # route everything, then expert MLPs for token chunks until the budget is spent
        logits = synth.host_rows(w.tensors["logits"])
        E, F, H, k = d["E"], d["F"], d["H"], d["k"]
        W1 = [synth.host_rows(w.tensors["W1t"], range(e * 2 * F, (e + 1) * 2 * F)) for e in range(E)]
        W2 = [synth.host_rows(w.tensors["W2t"], range(e * H, (e + 1) * H)) for e in range(E)]
        X = synth.host_rows(w.tensors["X"])
        t0 = time.perf_counter()
        done, tok = 0, 0
        per_token = k * 2 * (2 * F * H + H * F)
        while tok < d["T"] and time.perf_counter() - t0 < budget_s:
            toks = list(range(tok, min(tok + 4, d["T"])))
            oracle.moe_mlp(X, logits, W1, W2, k, tokens=toks)
            tok += len(toks)
            done += len(toks) * per_token
        el = time.perf_counter() - t0
        return dict(value=done / el / 1e12, unit="TFLOP/s", cores=oracle.num_threads(), kind="oracle",
                    sample=f"{tok} of {d['T']} tokens (routing + both expert MLPs per token), fp64, {el:.1f} s")
    p = d["p"]
    h = {k: synth.host_rows(v) for k, v in w.tensors.items() if k not in ("X", "ctx")}
    t0 = time.perf_counter()
    rows_done, flop = 0, 0
    per_row = w.flop // d["M"]  # every GEMM of the step has M = tokens rows
    chunk = 16
    while rows_done < d["M"] and time.perf_counter() - t0 < budget_s:
        rows = list(range(rows_done, min(rows_done + chunk, d["M"])))
        X = synth.host_rows(w.tensors["X"], rows)
        if "nq" in d:
            oracle.qkv(X, h["Wqkv_t"], h.get("bqkv"), d["nq"] // p, d["ng"] // p, d["d"])
        if "ctx" in w.tensors:
            oracle.linear(synth.host_rows(w.tensors["ctx"], rows), h["Wo_t"], h.get("bo") if p == 1 else None)
        if d["ranks"] == "all":
            oracle.mlp(X, h["W1t"], h.get("b1"), h["W2t"], h.get("b2"), d["act"], p)
        else:
            Z = oracle.round_bf16(oracle.linear(X, h["W1t"], h.get("b1"), d["act"]))
            oracle.linear(Z, h["W2t"])
        rows_done += len(rows)
        flop += len(rows) * per_row
    el = time.perf_counter() - t0
    return dict(value=flop / el / 1e12, unit="TFLOP/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{rows_done} of {d['M']} token rows through every GEMM of the step, fp64, {el:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt3_175b_rank0", choices=sorted(WORKLOADS))
    ap.add_argument("--warm", action="store_true",
                    help="time back-to-back steps as the headline (default: a 1 GiB cache-evicting write before each "
                         "timed step; warm figures are reported in either case)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-GEMM, norm/bias-dropout-add and FP8 measurements")
    ap.add_argument("--graphs", action="store_true",
                    help="replay the step as HIP graphs (captured from the same calls) instead of launching each "
                         "call from Python; on ROCm 7 graph launches cost more than they save at this step size")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--vs-hipblaslt", action="store_true",
                    help="only time three plain column GEMMs (8192^3, 4096x7168x8192 and 2048x12288x6144, no "
                         "bias or activation) through this library and through torch's linear (hipBLASLt): 3 "
                         "warm-up launches each, then 5 alternating batches of 4, the median batch; also the "
                         "side-by-side counter run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Each rank's share is the single-GPU kernel; see the sharding notes in the design document.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import megatron_tensor_transformer_03_amd as mtp
    from megatron_tensor_transformer_03_amd.layer import RankForward
    import synth
    from synth import configs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mtp.lib()  # fail loudly if the HIP library is missing

    if args.copy_calibration:
        n = 1 << 28  # 1 GiB of fp32
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n, "launches": 5}), flush=True)
        return

    if args.vs_hipblaslt:
        res = {}
        for (M, N, K) in [(8192, 8192, 8192), (4096, 7168, 8192), (2048, 12288, 6144)]:
            X = torch.randn(M, K, device="cuda").to(torch.bfloat16)
            W = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
            Y = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
            ws = mtp.workspace_for([(M, N, K, mtp.ACT_NONE)])
            fns = [("mtp", lambda: mtp.mtp_column_linear(X, W, None, Y, workspace=ws)),
                   ("hipblaslt", lambda: torch.nn.functional.linear(X, W))]
            for _, fn in fns:  # warm-up (code loading, clocks)
                for _ in range(3):
                    fn()
            times = {name: [] for name, _ in fns}
            for _ in range(5):  # the two libraries alternate; the median of 5 batches of 4 launches
                for name, fn in fns:
                    torch.cuda.synchronize()
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    for _ in range(4):
                        fn()
                    b.record()
                    b.synchronize()
                    times[name].append(a.elapsed_time(b) / 4 * 1000)
            for name, t in times.items():
                res[f"{name} {M}x{N}x{K}"] = round(sorted(t)[2], 1)
        print(json.dumps({"us_per_launch": res}), flush=True)
        return

    w = configs.by_index(WORKLOADS[args.workload])
    inputs = synth.device_inputs(w)
    run = RankForward(w.dims, inputs)
    torch.cuda.synchronize()
    # one side stream for everything (graph capture needs a non-default stream)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)

    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()

    # HIP events without the system-scope fence: a default event record writes back and invalidates the
    # caches, which costs several microseconds per record and slows the following kernel.
    timer = _FenceFreeEvents(stream.cuda_stream)

    # per-GEMM times from a short pass with an event around every launch (outside the timed region); an
    # unmarked step is enqueued first so the GPU is busy while the marked launches are issued (otherwise the
    # first interval would include the host's launch time on an idle GPU)
    per_kernel = {}
    for _ in range(min(5, max(args.steps, 1))):
        marks = []
        run.step()
        run.step(lambda label: marks.append((label, timer.record())))
        torch.cuda.synchronize()
        for (label, e0), (_, e1) in zip(marks[:-1], marks[1:]):
            per_kernel.setdefault(label, []).append(timer.elapsed_ms(e0, e1))
        timer.release(e for _, e in marks)

    flop_by_label = {}
    for label, m, n, k in w.gemms:
        flop_by_label[label] = flop_by_label.get(label, 0) + 2 * m * n * k
    if "E" in w.dims:
        flop_by_label = {"moe_mlp": w.flop}
    if w.dims.get("ranks") == "all" and w.dims.get("p", 1) > 1:
        flop_by_label = {"mlp": w.flop}
    avg = {lb: sum(v) / len(v) for lb, v in per_kernel.items()}
    dom = max((lb for lb in avg if lb in flop_by_label), key=lambda lb: avg[lb])

    # Timed region: K whole steps; the dominant kernel is bracketed by events in every step (on the stream
    # the library launches on), the only events inside the region.  With --graphs the launches before the
    # dominant kernel, the dominant kernel, and the launches after it are replayed as three HIP graphs
    # (captured from the same C-ABI calls).
    calls = run.calls()
    idx = [lb for lb, _ in calls].index(dom)
    segments = [calls[:idx], calls[idx:idx + 1], calls[idx + 1:]]
    if not args.graphs:
        launchers = [(lambda seg=seg: [fn() for _, fn in seg]) for seg in segments]
    else:
        launchers = []
        for seg in segments:
            if not seg:
                launchers.append(lambda: None)
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for _, fn in seg:
                    fn()
            launchers.append(g.replay)
        torch.cuda.synchronize()
        for _ in range(2):  # replay once untimed
            for launch in launchers:
                launch()
        torch.cuda.synchronize()
    pre, dom_launch, post = launchers

    # Cold: an untimed write of 1 GiB before every timed step evicts the 256 MB memory-side cache; each step is
    # bracketed by events (the flush lies outside every bracket).  Warm: the same steps back to back.
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def timed(cold):
        step_ms, dom_ms = [], []
        torch.cuda.synchronize()
        ev_all = []
        if not cold:
            start = timer.record()
        for _ in range(args.steps):
            if cold:
                flush_buf.fill_(1.0)
                s0 = timer.record()
            pre()
            e0 = timer.record()
            dom_launch()
            e1 = timer.record()
            post()
            if cold:
                s1 = timer.record()
                ev_all.append((s0, e0, e1, s1))
            else:
                ev_all.append((None, e0, e1, None))
        if not cold:
            stop = timer.record()
        torch.cuda.synchronize()
        for s0, e0, e1, s1 in ev_all:
            dom_ms.append(timer.elapsed_ms(e0, e1))
            if cold:
                step_ms.append(timer.elapsed_ms(s0, s1))
        events = [e for quad in ev_all for e in quad if e is not None]
        if cold:
            ms = sum(step_ms) / len(step_ms)
        else:
            ms = timer.elapsed_ms(start, stop) / args.steps
            events += [start, stop]
        timer.release(events)
        return ms, sum(dom_ms) / len(dom_ms)

    ms_warm, dom_warm = timed(False)
    ms_cold, dom_cold = timed(True)
    del flush_buf
    ms, dom_avg = (ms_warm, dom_warm) if args.warm else (ms_cold, dom_cold)
    achieved = flop_by_label[dom] / (dom_avg * 1e-3) / 1e12
    flop = w.flop
    value = flop / (ms * 1e-3) / 1e12

    # calibrated peak: an MFMA-only loop over every CU (8 waves each), about 20 ms
    cal_out = torch.empty(4096, dtype=torch.float32, device="cuda")
    cal_blocks, cal_iters = 4 * torch.cuda.get_device_properties(0).multi_processor_count, 20000
    mtp.mtp_mfma_calibrate(cal_out, cal_blocks, 200)
    torch.cuda.synchronize()
    c0 = timer.record()
    mtp.mtp_mfma_calibrate(cal_out, cal_blocks, cal_iters)
    c1 = timer.record()
    torch.cuda.synchronize()
    cal_ms = timer.elapsed_ms(c0, c1)
    timer.release([c0, c1])
    cal_peak = cal_blocks * 8 * cal_iters * 8 * 32768 / (cal_ms * 1e-3) / 1e12
    traffic = measured_traffic(w.name, dom, cold=not args.warm)

    # non-GEMM kernels of the step, against the HBM roofline: algorithmic bytes per launch / event time
    aux = {}
    if "rope" in avg and "rope" in w.dims:
        dd = w.dims
        heads = (dd["nq"] + dd["ng"]) // dd["p"]
        rope_bytes = dd["M"] * heads * dd["rope"]["rotary_dim"] * 2 * 2 + 4 * dd["M"]
        gbs = rope_bytes / (avg["rope"] * 1e-3) / 1e9
        aux["rope"] = {"bound": "hbm", "us": round(1000 * avg["rope"], 2), "bytes": rope_bytes,
                       "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4)}

    # the backward GEMMs of the same linears (outside the timed region; dense layers only)
    bwd = None if ("E" in w.dims or args.no_backward) else backward_gemms(w, timer)
    nb = None if ("E" in w.dims or args.no_backward) else norm_and_bda(w, timer)
    f8 = None if ("E" in w.dims or args.no_backward) else fp8_gemms(w, timer)
    pre = None if args.no_backward else prenorm_layer(w, timer)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "desc": w.desc, "flop_per_step": flop,
                   "launch": "hip_graph" if args.graphs else "eager",
                   "timing": "warm (steps back to back)" if args.warm else
                             "cold (1 GiB write before each timed step evicts the 256 MB memory-side cache)",
                   "pct_of_mfma_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
                   "calibrated_mfma_peak_tflops": round(cal_peak, 1),
                   "pct_of_calibrated_peak": round(100 * value / cal_peak, 2),
                   "cold": {"ms_per_step": round(ms_cold, 5), "value": round(flop / (ms_cold * 1e-3) / 1e12, 2),
                            "dominant_kernel_us": round(1000 * dom_cold, 2)},
                   "warm": {"ms_per_step": round(ms_warm, 5), "value": round(flop / (ms_warm * 1e-3) / 1e12, 2),
                            "dominant_kernel_us": round(1000 * dom_warm, 2)},
                   "gemms": [[lb, m, n, k] for lb, m, n, k in w.gemms],
                   "per_gemm_us": {lb: round(1000 * v, 2) for lb, v in avg.items()},
                   "per_gemm_tflops": {lb: round(flop_by_label[lb] / (avg[lb] * 1e-3) / 1e12, 1)
                                       for lb in avg if lb in flop_by_label},
                   "aux_kernels": aux, "backward_gemms": bwd, "norm_and_bda": nb, "fp8_gemms": f8,
                   "prenorm_layer": pre},
        "roofline": {"bound": "mfma", "kernel": dom, "kernel_us": round(1000 * dom_avg, 2),
                     "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "calibrated_peak": round(cal_peak, 1), "frac_of_calibrated": round(achieved / cal_peak, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
