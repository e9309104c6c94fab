"""Throughput of one tensor-parallel rank's MLP shard, forward + backward.

One step = the whole shard path on one batch, inputs resident in HBM:
  forward   FC1 (+ activation epilogue) -> FC2             tp_mlp_shard_fwd
  sum       Y = Y_0 + 7 stand-in partials of the other ranks  tp_partial_sum
  backward  dH (+ activation-derivative epilogue), dB, dA, dX tp_mlp_shard_bwd
  sum       dX = dX_0 + 7 stand-in partials                   tp_partial_sum
The metric counts the GEMM FLOPs only (2 M N K per product: 9 products for
SwiGLU, 6 for GeLU); the step time includes the two partial sums.  The sums
stand in for the rank's all-reduces and, like communication, run by default
on a second stream beside the GEMMs that do not depend on them (sum(Y) beside
the backward, sum(dX) beside the next forward); --overlap 0 runs the step in
order on one stream, and the default run also times that form
("serial_step").

Prints one JSON line.  Only one GPU is used: --gpus above 1 exits.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# copy of known size run outside the timed region: under a counter profile
# its FETCH_SIZE / WRITE_SIZE calibrate the GEMM kernels' byte counts
CALIB_COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_c4_swiglu.txt")
CLOCK_FILE = os.path.join(ROOT, "profiles", "gemm_clock_c4_swiglu.txt")
KERNEL_SOURCES = ["gemm_bf16.hip", "common.h", "api.hip"]


def kernel_source_hash() -> str:
    """Hash of the GEMM sources, to tell whether recorded counters still
    describe the kernels being timed."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tensor_transformer_mlp_02_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_field(path, key):
    """A figure from a committed counter summary, or None when the file is
    missing or was taken on other kernel sources."""
    try:
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_source_hash") != kernel_source_hash():
            return None
        return float(fields[key])
    except (OSError, KeyError, ValueError):
        return None


def recorded_traffic():
    """HBM bytes per GEMM launch (FETCH_SIZE + WRITE_SIZE, calibrated)."""
    return recorded_field(TRAFFIC_FILE, "hbm_bytes_per_gemm_launch")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c4_bf16_swiglu_fwdbwd")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--fp8", type=int, default=1,
                   help="1: also time the FP8 forward and backward at the same shape")
    p.add_argument("--moe", type=int, default=1,
                   help="1: also time the MoE dispatch/combine row moves")
    p.add_argument("--overlap", type=int, default=1,
                   help="1: partial sums on a second stream, overlapping the GEMMs; "
                        "0: everything in order on one stream")
    p.add_argument("--sum-workgroups", type=int, default=256,
                   help="workgroup cap of the overlapped partial sums")
    p.add_argument("--side", type=int, default=1,
                   help="0: time the step only (no reduce-scatter, accumulation, MoE or FP8 "
                        "side measurements), as for the profiler's per-kernel summaries")
    p.add_argument("--cpu-tokens", type=int, default=0,
                   help="tokens of the oracle sample (0: sized to ~15 s)")
    return p.parse_args()


def gemm_flops(w, N=None):
    N = w.N if N is None else N
    per = 2.0 * N * w.H * w.Ft
    n_fwd = 3 if w.act == 1 else 2
    return per * n_fwd * (3 if w.backward else 1)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, tokens):
    """The fp64 oracle, as it stands, on a token sample of the workload."""
    import numpy as np
    import oracle
    import workloads as wl
    d = wl.gen_mlp_inputs(w, n_rows=max(tokens, 1))
    t0 = time.perf_counter()
    f = oracle.mlp_fwd(d["X"], d["A"], d["B"], w.act, d["A_up"])
    if w.backward:
        oracle.mlp_bwd(d["X"], d["A"], d["B"], w.act, d["dY"], f, d["A_up"])
    dt = time.perf_counter() - t0
    return dt, gemm_flops(w, tokens)


def grouped_expert_timing(torch, tp, wl, stream, reps=20):
    """The grouped local experts on the grouped-expert workload (16384 tokens
    routed top-2 over 64 experts, local experts 0..7, H = 4096, F = 1408,
    SwiGLU): forward and backward launches over the ragged rows, in
    algorithmic TFLOP/s (18 H F per row for forward + backward)."""
    from tensor_transformer_mlp_02_amd.tensors import to_device, ExpertBuffers
    w5 = wl.WORKLOADS["c5_bf16_grouped_swiglu"]
    g = wl.gen_grouped_inputs(w5)
    off = g["offsets"]
    R, E, H, F = int(off[-1]), len(off) - 1, w5.H, w5.F
    d = {k: to_device(g[k]) for k in ("X_perm", "Wg", "Wu", "Wd", "dY_perm")}
    desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
    buf = ExpertBuffers(desc, off)

    def fwd():
        tp.tp_grouped_expert_fwd(desc, off, d["X_perm"], d["Wg"], d["Wu"], d["Wd"], buf.Z,
                                 buf.H, buf.Y, stream=stream)

    def bwd():
        tp.tp_grouped_expert_bwd(desc, off, d["X_perm"], d["Wg"], d["Wu"], d["Wd"], buf.Z,
                                 buf.H, d["dY_perm"], buf.dX, buf.dWg, buf.dWu, buf.dWd,
                                 buf.ws, buf.ws_bytes, stream=stream)
    fwd(); bwd()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(reps):
        fwd()
    ev[1].record(stream)
    for _ in range(reps):
        bwd()
    ev[2].record(stream)
    torch.cuda.synchronize()
    f_ms = ev[0].elapsed_time(ev[1]) / reps
    b_ms = ev[1].elapsed_time(ev[2]) / reps
    f_fl, b_fl = 6.0 * H * F * R, 12.0 * H * F * R
    tf = (f_fl + b_fl) / ((f_ms + b_ms) * 1e-3) / 1e12
    return {"rows": R, "experts": E, "rows_per_expert": [int(x) for x in off[1:] - off[:-1]],
            "H": H, "F": F, "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "fwd_tflops": round(f_fl / (f_ms * 1e-3) / 1e12, 1),
            "bwd_tflops": round(b_fl / (b_ms * 1e-3) / 1e12, 1),
            "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def moe_dispatch_timing(torch, tp, wl, dev, stream, reps=20):
    """Token dispatch and combine around the grouped experts on the
    grouped-expert workload's routing (16384 tokens, top-2 of 64 experts,
    local experts 0..7, H = 4096): permute, weighted combine and the
    combine's backward, each in GB/s of algorithmic row traffic."""
    import numpy as np
    w5 = wl.WORKLOADS["c5_bf16_grouped_swiglu"]
    logits = wl.normal(1000 * w5.cid + wl.K_LOGITS, (w5.tokens, w5.n_route), 1.0)
    ids, off = wl.route_top2_local(logits, w5.experts, w5.topk)
    rw = wl.route_weights(logits, ids, off)
    ptr, rows = wl.token_rows(ids, w5.tokens)
    N, H, R = w5.tokens, w5.H, len(ids)
    tab = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ids_d, ptr_d, rows_d, rw_d = tab(ids.astype(np.int32)), tab(ptr), tab(rows), tab(rw)
    g = torch.Generator(device=dev).manual_seed(1000 * w5.cid + 91)
    X = torch.randn((N, H), generator=g, device=dev).to(torch.bfloat16)
    dY = torch.randn((N, H), generator=g, device=dev).to(torch.bfloat16)
    Yp = torch.randn((R, H), generator=g, device=dev).to(torch.bfloat16)
    Xp = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    Y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    dYp = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dw = torch.empty(R, dtype=torch.float32, device=dev)
    calls = {
        "permute": (lambda: tp.tp_moe_permute(wl.DT_BF16, N, H, R, ids_d, X, Xp, stream=stream),
                    2 * R * H * 2),
        "combine": (lambda: tp.tp_moe_combine(wl.DT_BF16, N, H, R, ptr_d, rows_d, rw_d, Yp, Y,
                                              stream=stream), (R + N) * H * 2),
        "combine_bwd": (lambda: tp.tp_moe_combine_bwd(wl.DT_BF16, N, H, R, ids_d, rw_d, dY, Yp,
                                                      dYp, dw, stream=stream), 3 * R * H * 2),
    }
    out = {"tokens": N, "H": H, "rows": R}
    for name, (fn, nbytes) in calls.items():
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        out[name] = {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    return out


PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA (twice the bf16 rate)


def fp8_timing(torch, tp, wl, w, X, A, Au, B, dY, stream, reps=10):
    """The shard forward and backward on FP8 codes at the same shape
    (E4M3 weights and activations, E5M2 gradients): the GEMM calls alone,
    and the quantization each needs (forward: X and the weights' transposes;
    backward: dY and its transpose, the transposes of X's and H's codes, the
    weights in their own layout)."""
    dev = X.device
    N, Hd, Ft = w.N, w.H, w.Ft
    sw = Au is not None
    zw = 2 * Ft if sw else Ft
    s = lambda v: torch.tensor([v], dtype=torch.float32, device=dev)
    sx, sa, sdy = s(32.0), s(4096.0), s(1024.0)
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=dev)
    Xq, Aq_t, Bq_t = u8(N, Hd), u8(Ft, Hd), u8(Hd, Ft)
    Auq_t = u8(Ft, Hd) if sw else None
    amax = torch.zeros(8, dtype=torch.float32, device=dev)
    qs = torch.tensor([1 / 32.0, 1 / 4096.0, 1 / 4096.0, 1 / 4096.0, 32.0],
                      dtype=torch.float32, device=dev)
    Z = torch.empty((N, zw), dtype=torch.bfloat16, device=dev)
    Hh = torch.empty((N, Ft), dtype=torch.bfloat16, device=dev)
    Hq = u8(N, Ft)
    Y = torch.empty((N, Hd), dtype=torch.bfloat16, device=dev)
    desc = dict(S=w.S, B=w.B, H=Hd, F_shard=Ft, T=w.T, act=w.act, dtype=w.dtype)
    E4, E5 = tp.TP_FP8_E4M3, tp.TP_FP8_E5M2
    # backward operands and outputs
    dYq, dYq_t, Xq_t, Hq_t = u8(N, Hd), u8(Hd, N), u8(Hd, N), u8(Ft, N)
    Aq, Bq = u8(Hd, Ft), u8(Ft, Hd)
    Auq = u8(Hd, Ft) if sw else None
    qb = torch.tensor([1 / 1024.0, 1 / 4096.0, 1 / 32.0, 1 / 32.0, 1 / 4096.0, 4096.0,
                       1 / 4096.0], dtype=torch.float32, device=dev)
    dX = torch.empty((N, Hd), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((Hd, Ft), dtype=torch.float32, device=dev)
    dAu = torch.empty((Hd, Ft), dtype=torch.float32, device=dev) if sw else None
    dB = torch.empty((Ft, Hd), dtype=torch.float32, device=dev)
    dZq, dZq_t = u8(N, zw), u8(zw, N)

    def quant_fwd():
        tp.tp_fp8_quantize(E4, False, N, Hd, X, sx, Xq, amax[0:1], stream=stream)
        tp.tp_fp8_quantize(E4, True, Hd, Ft, A, sa, Aq_t, amax[1:2], stream=stream)
        if sw:
            tp.tp_fp8_quantize(E4, True, Hd, Ft, Au, sa, Auq_t, amax[2:3], stream=stream)
        tp.tp_fp8_quantize(E4, True, Ft, Hd, B, sa, Bq_t, amax[3:4], stream=stream)

    def fwd():
        tp.tp_mlp_shard_fwd_fp8(desc, Xq, Aq_t, Auq_t, Bq_t, qs, Z, Hh, Hq, amax[0:1], Y,
                                stream=stream)

    def quant_bwd():
        tp.tp_fp8_quantize(E5, False, N, Hd, dY, sdy, dYq, amax[4:5], stream=stream)
        tp.tp_fp8_transpose(N, Hd, dYq, dYq_t, stream=stream)
        tp.tp_fp8_transpose(N, Hd, Xq, Xq_t, stream=stream)
        tp.tp_fp8_transpose(N, Ft, Hq, Hq_t, stream=stream)
        tp.tp_fp8_transpose(Ft, Hd, Aq_t, Aq, stream=stream)
        if sw:
            tp.tp_fp8_transpose(Ft, Hd, Auq_t, Auq, stream=stream)
        tp.tp_fp8_transpose(Hd, Ft, Bq_t, Bq, stream=stream)

    def bwd():
        tp.tp_mlp_shard_bwd_fp8(desc, dYq, dYq_t, Xq_t, Hq_t, Aq, Auq, Bq, Z, qb, dX, dA, dAu,
                                dB, dZq, dZq_t, amax[5:6], stream=stream)

    quant_fwd(); fwd(); quant_bwd(); bwd()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    ev[0].record(stream)
    for _ in range(reps):
        quant_fwd()
    ev[1].record(stream)
    for _ in range(reps):
        fwd()
    ev[2].record(stream)
    for _ in range(reps):
        quant_bwd()
    ev[3].record(stream)
    for _ in range(reps):
        bwd()
    ev[4].record(stream)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) / reps for i in range(4)]
    f_fl = 2.0 * N * Hd * Ft * (3 if sw else 2)
    b_fl = 2 * f_fl
    tf = lambda fl, t: round(fl / (t * 1e-3) / 1e12, 1)
    fwd_d = {"gemm_ms": round(ms[1], 4), "gemm_tflops": tf(f_fl, ms[1]),
             "gemm_frac_of_fp8_peak": round(f_fl / (ms[1] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
             "quantize_ms": round(ms[0], 4),
             "forward_tflops_with_quantize": tf(f_fl, ms[0] + ms[1]),
             "bf16_forward_ms_for_comparison": None}
    bwd_d = {"ms": round(ms[3], 4), "tflops": tf(b_fl, ms[3]),
             "frac_of_fp8_peak": round(b_fl / (ms[3] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
             "quantize_transpose_ms": round(ms[2], 4),
             "backward_tflops_with_quantize": tf(b_fl, ms[2] + ms[3]),
             "step_tflops_with_quantize": tf(f_fl + b_fl, sum(ms)),
             "bf16_backward_ms_for_comparison": None}
    return fwd_d, bwd_d


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs one tensor-parallel rank's shard on ONE GPU; multi-GPU runs "
              "(collectives across GPUs) are not part of this library", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import tensor_transformer_mlp_02_amd as tp
    from tensor_transformer_mlp_02_amd.tensors import to_device, ShardBuffers
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    assert w.dtype == wl.DT_BF16
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    d = wl.gen_mlp_inputs(w)
    X, A, B = to_device(d["X"]), to_device(d["A"]), to_device(d["B"])
    Au = to_device(d["A_up"]) if d["A_up"] is not None else None
    dY = to_device(d["dY"]) if w.backward else None
    desc = dict(S=w.S, B=w.B, H=w.H, F_shard=w.Ft, T=w.T, act=w.act, dtype=w.dtype)
    buf = ShardBuffers(desc, backward=w.backward)
    # the other T-1 ranks' partial outputs: seeded stand-ins of the same shape
    stand = [to_device(p) for p in wl.gen_partials(w, w.T - 1, (w.N, w.H), 0.05)]
    Ysum = torch.empty_like(buf.Y)
    dXsum = torch.empty_like(buf.Y)
    count = w.N * w.H
    stream = torch.cuda.current_stream()

    # The partial sums stand in for the all-reduces of a real rank, so by
    # default they run on a second stream (default priority) like
    # communication would: sum(Y) overlaps the backward GEMMs and sum(dX) the
    # next forward, each on a capped number of workgroups.  Events keep every
    # dependency: a sum starts after the GEMM that wrote its input, and the
    # next write of Y (forward) or dX (backward) waits for the sum that reads
    # it.  overlap=False runs everything in order on the compute stream.
    def run_steps(overlap, steps, warmup):
        side = torch.cuda.Stream(device=dev) if overlap else stream

        def psum(*a, stream):
            if overlap:
                return tp.tp_partial_sum_capped(*a, args.sum_workgroups, stream=stream)
            return tp.tp_partial_sum(*a, stream=stream)
        y_ready, dx_ready = torch.cuda.Event(), torch.cuda.Event()
        y_read, dx_read = torch.cuda.Event(), torch.cuda.Event()
        y_read.record(side)
        dx_read.record(side)

        def step(ev=None):
            if ev: ev[0].record(stream)
            stream.wait_event(y_read)
            tp.tp_mlp_shard_fwd(desc, X, A, Au, B, buf.Z, buf.H, buf.Y, stream=stream)
            if ev: ev[1].record(stream)
            y_ready.record(stream)
            side.wait_event(y_ready)
            if ev: ev[5].record(side)
            psum(w.dtype, w.T, [buf.Y] + stand, count, Ysum, stream=side)
            if ev: ev[6].record(side)
            y_read.record(side)
            if w.backward:
                if ev: ev[2].record(stream)
                stream.wait_event(dx_read)
                tp.tp_mlp_shard_bwd(desc, X, A, Au, B, buf.Z, buf.H, dY, buf.dX, buf.dA,
                                    buf.dA_up, buf.dB, buf.ws, buf.ws_bytes, stream=stream)
                if ev: ev[3].record(stream)
                dx_ready.record(stream)
                side.wait_event(dx_ready)
                if ev: ev[7].record(side)
                psum(w.dtype, w.T, [buf.dX] + stand, count, dXsum, stream=side)
                if ev: ev[8].record(side)
                dx_read.record(side)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        # timed region: K whole steps between two events on the compute
        # stream (the last one after it has waited for the side stream);
        # per-call events on each stream split the time between the GEMM
        # calls and the sums
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(9)] for _ in range(steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(stream)
        side.wait_event(t_start)
        for k in range(steps):
            step(evs[k])
        done = torch.cuda.Event()
        done.record(side)
        stream.wait_event(done)
        t_end.record(stream)
        torch.cuda.synchronize()
        ms = t_start.elapsed_time(t_end) / steps
        fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        ps = [e[5].elapsed_time(e[6]) for e in evs]
        bwd_ms = 0.0
        if w.backward:
            bwd_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
            ps += [e[7].elapsed_time(e[8]) for e in evs]
        return ms, fwd_ms, bwd_ms, float(np.mean(ps))

    # calibration copy (one partial sum of a single buffer = a copy)
    n_calib = CALIB_COPY_BYTES // 2
    calib_src = torch.zeros(n_calib, dtype=torch.bfloat16, device=dev)
    calib_dst = torch.empty_like(calib_src)
    tp.tp_partial_sum(w.dtype, 1, [calib_src], n_calib, calib_dst)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    ms, fwd_ms, bwd_ms, ps_ms = run_steps(bool(args.overlap), args.steps, args.warmup)
    # the same steps in order on one stream: the GEMMs and the sums undisturbed
    serial = None
    if args.overlap and args.side:
        serial = run_steps(False, args.steps, args.warmup)

    # sequence-parallel form of the same exchange (outside the timed step):
    # rank 0's [S/T,B,H] slice of the sum, the reduce-scatter arithmetic
    rs = None
    if args.side and w.S % w.T == 0:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        slice_out = torch.empty((w.S // w.T) * w.B * w.H, dtype=Ysum.dtype, device=dev)
        for _ in range(3):
            tp.tp_partial_sum_scatter(w.dtype, w.T, [buf.Y] + stand, w.S, w.B, w.H, 0, slice_out)
        reps = 20
        e0.record(stream)
        for _ in range(reps):
            tp.tp_partial_sum_scatter(w.dtype, w.T, [buf.Y] + stand, w.S, w.B, w.H, 0, slice_out)
        e1.record(stream)
        torch.cuda.synchronize()
        rs_ms = e0.elapsed_time(e1) / reps
        rs_bytes = (w.T + 1) * slice_out.numel() * 2
        rs = {"us": round(rs_ms * 1e3, 2), "GBps": round(rs_bytes / (rs_ms * 1e-3) / 1e9, 1),
              "hbm_frac": round(rs_bytes / (rs_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
              "bytes": rs_bytes}

    # gradient-accumulation form of the backward (weight gradients added
    # into the fp32 buffers), timed beside the plain backward
    acc_cmp = None
    if args.side and w.backward:
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            tp.tp_mlp_shard_bwd(desc, X, A, Au, B, buf.Z, buf.H, dY, buf.dX, buf.dA,
                                buf.dA_up, buf.dB, buf.ws, buf.ws_bytes, stream=stream)
        e1.record(stream)
        for _ in range(reps):
            tp.tp_mlp_shard_bwd_accum(desc, X, A, Au, B, buf.Z, buf.H, dY, buf.dX, buf.dA,
                                      buf.dA_up, buf.dB, buf.ws, buf.ws_bytes, stream=stream)
        e2.record(stream)
        torch.cuda.synchronize()
        acc_cmp = {"bwd_ms": round(e0.elapsed_time(e1) / reps, 4),
                   "bwd_accum_ms": round(e1.elapsed_time(e2) / reps, 4)}

    moe = moe_dispatch_timing(torch, tp, wl, dev, stream) if (args.side and args.moe) else None
    grouped = grouped_expert_timing(torch, tp, wl, stream) if (args.side and args.moe) else None
    f8 = f8b = None
    if (args.side and args.fp8 and w.dtype == wl.DT_BF16 and w.H % 128 == 0 and w.Ft % 128 == 0
            and w.N % 128 == 0 and w.backward):
        f8, f8b = fp8_timing(torch, tp, wl, w, X, A, Au, B, dY, stream)
        f8["bf16_forward_ms_for_comparison"] = round(fwd_ms, 4)
        f8b["bf16_backward_ms_for_comparison"] = round(bwd_ms, 4)

    flops = gemm_flops(w)
    value = flops / (ms * 1e-3) / 1e12
    gemm_ms = fwd_ms + bwd_ms
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    n_gemm = (2 + (4 if w.backward else 0))
    ps_bytes = (w.T + 1) * count * 2
    # algorithmic HBM bytes of the GEMM launches of one step: every operand
    # read once, every output written once (bf16 activations, fp32 weight
    # gradients)
    N, Hd, Ft = w.N, w.H, w.Ft
    e2, e4 = 2, 4
    nz = 2 if w.act == 1 else 1          # Z_save columns per Ft (G|U)
    fwd_bytes = (N * Hd + nz * Hd * Ft) * e2 + (nz + 1) * N * Ft * e2 \
        + (N * Ft + Ft * Hd) * e2 + N * Hd * e2
    bwd_bytes = 0
    if w.backward:
        bwd_bytes = (N * Hd + Ft * Hd + nz * N * Ft) * e2 + nz * N * Ft * e2 \
            + (N * Ft + N * Hd) * e2 + Ft * Hd * e4 \
            + (N * Hd + nz * N * Ft) * e2 + nz * Hd * Ft * e4 \
            + (nz * N * Ft + nz * Hd * Ft) * e2 + N * Hd * e2
    algo_bytes = fwd_bytes + bwd_bytes
    ps_gbs = ps_bytes / (ps_ms * 1e-3) / 1e9
    # the shader clock the GEMMs ran at under load (counter summary of the
    # same kernels): the MFMA peak at that clock is what the silicon offered
    sclk = recorded_field(CLOCK_FILE, "sclk_ghz_gemm_mean")

    line = {
        "metric": "TP-shard MLP fwd+bwd TFLOP/s on 1 GPU + % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal draws, rounded to bf16)",
        "config": {"workload": w.name, "S": w.S, "B": w.B, "H": w.H, "F": w.F, "T": w.T,
                   "F_shard": w.Ft, "act": "swiglu" if w.act == 1 else "gelu_tanh",
                   "rank": "one tensor-parallel rank; the other 7 ranks' partials are "
                           "seeded stand-ins",
                   "partial_sums": ("second stream, overlapping the GEMMs, at most %d "
                                    "workgroups" % args.sum_workgroups) if args.overlap
                                   else "in order on the compute stream",
                   "act_derivative": "epilogue of the dY B^T GEMM (dZ written once)",
                   "caches": "nothing is warmed on purpose: each step's two partial sums "
                             "stream 1.1 GB through HBM (non-temporal), and each GEMM finds "
                             "in the 256 MB Infinity Cache only what the launches before it "
                             "left there"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "kernel": "bf16 MFMA GEMM with fused epilogues (%d launches per step)" % n_gemm,
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_traffic(),
            "algorithmic_bytes_per_launch": round(algo_bytes / n_gemm),
        },
        "clock_under_load": None if sclk is None else {
            "sclk_ghz": sclk,
            "peak_at_sclk": round(PEAK_BF16_TFLOPS * sclk / 2.4, 1),
            "frac_at_sclk": round(gemm_tflops / (PEAK_BF16_TFLOPS * sclk / 2.4), 4),
            "source": "profiles/gemm_clock_c4_swiglu.txt (rocprofv3 SQ_BUSY_CYCLES)"},
        "breakdown_ms": {"fwd_gemms": round(fwd_ms, 4), "bwd_gemms": round(bwd_ms, 4),
                         "partial_sum_each": round(ps_ms, 4),
                         "partial_sum_GBps": round(ps_gbs, 1),
                         "partial_sum_hbm_frac": round(ps_gbs / PEAK_HBM_GBS, 4)},
        "serial_step": None if serial is None else {
            "note": "the same steps in order on one stream (sums not overlapped)",
            "ms_per_step": round(serial[0], 4),
            "tflops": round(flops / (serial[0] * 1e-3) / 1e12, 2),
            "gemm_tflops": round(flops / ((serial[1] + serial[2]) * 1e-3) / 1e12, 2),
            "gemm_frac_of_bf16_peak": round(
                flops / ((serial[1] + serial[2]) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "breakdown_ms": {"fwd_gemms": round(serial[1], 4), "bwd_gemms": round(serial[2], 4),
                             "partial_sum_each": round(serial[3], 4)},
            "partial_sum_GBps": round(ps_bytes / (serial[3] * 1e-3) / 1e9, 1),
            "partial_sum_hbm_frac": round(ps_bytes / (serial[3] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "reduce_scatter_rank0": rs,
        "grad_accumulation": acc_cmp,
        "moe_dispatch_combine": moe,
        "grouped_experts": grouped,
        "fp8_forward": f8,
        "fp8_backward": f8b,
    }

    if not args.no_cpu_baseline:
        import oracle
        tokens = args.cpu_tokens
        if tokens <= 0:
            dt, fl = cpu_baseline(w, 128)           # calibrate on 128 tokens
            rate = fl / max(dt, 1e-6)
            tokens = int(max(16, min(w.N, 20.0 * rate / gemm_flops(w, 1))))
        dt, fl = cpu_baseline(w, tokens)
        line["cpu_baseline"] = {
            "value": round(fl / dt / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"fp64 oracle, forward+backward of the same shard on {tokens} of "
                      f"{w.N} tokens ({fl / 1e9:.1f} GFLOP in {dt:.1f} s)",
            "cpu": cpu_model(),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
