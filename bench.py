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
the backward, sum(dX) beside the next forward).

Caches: the headline steps rotate several input sets (X, the weights, dY;
together well over the 256 MB Infinity Cache), so every step reads its
inputs cold, as a layer of a real model would.  The same steps on one input
set ("warm") are timed beside them.  `value` is the GEMM FLOPs of a step over
the median of the timed steps' durations (each step's interval between the
starts of consecutive steps on the compute stream).

Every GEMM launch inside the timed steps is bracketed by HIP events on its
own stream (the library's tp_launch_events hook), so each kernel's duration
comes from the same run; `roofline` is the longest (dominant) one.

Prints one JSON line.  Only one GPU is used: --gpus above 1 exits.
"""
import argparse
import ctypes
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA (twice the bf16 rate)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# copy of known size run outside the timed region: under a counter profile
# its FETCH_SIZE / WRITE_SIZE calibrate the GEMM kernels' byte counts
CALIB_COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_c4_swiglu.txt")
KERNEL_SOURCES = ["gemm_bf16.hip", "common.h", "api.hip"]
# 60 % of the bf16 peak, as GEMM time per step (the shard targets)
TARGET_FRAC = 0.60


def kernel_source_hash() -> str:
    """Hash of the GEMM sources, to tell whether recorded counters still
    describe the kernels being timed."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tensor_transformer_mlp_02_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_fields(path):
    """The key: value lines of a committed counter summary, or None when the
    file is missing or was taken on other kernel sources."""
    try:
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_source_hash") != kernel_source_hash():
            return None
        return fields
    except OSError:
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c4_bf16_swiglu_fwdbwd")
    p.add_argument("--sets", type=int, default=3,
                   help="input sets rotated over the headline steps (cold caches)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--fp8", type=int, default=1,
                   help="1: also time the FP8 forward and backward at the same shape")
    p.add_argument("--moe", type=int, default=1,
                   help="1: also time the grouped experts and the MoE dispatch/combine")
    p.add_argument("--overlap", type=int, default=1,
                   help="1: partial sums on a second stream, overlapping the GEMMs; "
                        "0: everything in order on one stream")
    p.add_argument("--sum-workgroups", type=int, default=192,
                   help="workgroup cap of the overlapped partial sums")
    p.add_argument("--sum-y-after", default="FC2",
                   help="launch after which the overlapped sum(Y) starts: FC2 (as soon as Y "
                        "is written) or a backward GEMM (dH, dB, dA, dX)")
    p.add_argument("--side", type=int, default=1,
                   help="0: time the headline steps only (no warm, in-order, other-shape, "
                        "reduce-scatter, accumulation, MoE or FP8 measurements), as for "
                        "the profiler's per-kernel summaries")
    p.add_argument("--only", default="", choices=["", "grouped", "fp8", "dact"],
                   help="time only the grouped experts, the FP8 shard, or the two "
                        "placements of the activation derivative in the backward (for the "
                        "profiler's per-kernel summaries); prints their JSON")
    p.add_argument("--grouped-offsets", default="both", choices=["both", "host", "device"],
                   help="with the grouped experts: time the calls with host offsets, with "
                        "device offsets, or both")
    p.add_argument("--clock", type=int, default=1,
                   help="1: sample the shader clock while the steps run again")
    p.add_argument("--cpu-tokens", type=int, default=0,
                   help="tokens of the oracle sample (0: sized to ~20 s)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# HIP events through the runtime torch has loaded (the library and torch
# share it): raw handles for the library's launch-timing hook
# ---------------------------------------------------------------------------
class HipEvents:
    def __init__(self, torch):
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.lib = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        self.made = []

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        self.made += out
        return out

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def wait(self, stream, ev):
        if self.lib.hipStreamWaitEvent(stream.cuda_stream, ev, 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def ms(self, a, b):
        t = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)

    def free(self):
        for h in self.made:
            self.lib.hipEventDestroy(h)
        self.made = []


def median(xs):
    import numpy as np
    return float(np.median(np.asarray(xs, dtype=np.float64)))


def tflops(fl, ms):
    return fl / (ms * 1e-3) / 1e12


# ---------------------------------------------------------------------------
# shader clock sampled while the GEMMs run (amdsmi gpu metrics)
# ---------------------------------------------------------------------------
def sysfs_sclk_path(bus):
    """The kernel driver's shader-clock level file (pp_dpm_sclk) of the card
    on PCI bus `bus`, or None."""
    import glob
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            bdf = os.path.basename(os.path.realpath(dev))  # e.g. 0000:75:00.0
            if int(bdf.split(":")[1], 16) == bus and os.path.exists(dev + "/pp_dpm_sclk"):
                return dev + "/pp_dpm_sclk"
        except (ValueError, IndexError, OSError):
            continue
    return None


class ClockSampler:
    """Samples the GPU's current shader clock every few ms in a thread: the
    level the kernel driver marks current in the card's pp_dpm_sclk (it
    follows the load), else amdsmi's gpu metrics (whose current clocks stay
    at an idle value on some machines).  Reports None when neither gives a
    plausible reading."""

    def __init__(self, torch):
        self.samples, self.avg_samples, self.error, self.h, self.raw = [], [], None, None, None
        bus = torch.cuda.get_device_properties(0).pci_bus_id
        self.sysfs = sysfs_sclk_path(bus)
        try:
            import amdsmi
            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if int(bdf.split(":")[1], 16) == bus:
                    self.h = h
            if self.h is None and self.sysfs is None:
                self.error = "no clock source for the device's PCI bus"
        except Exception as e:  # metrics are context: never fail the bench
            if self.sysfs is None:
                self.error = f"{type(e).__name__}: {e}"

    def _read_sysfs(self):
        """The current level of pp_dpm_sclk in MHz (the line marked '*')."""
        with open(self.sysfs) as fh:
            for line in fh:
                if line.rstrip().endswith("*"):
                    return float(line.split(":", 1)[1].strip().lower().split("mhz")[0])
        return None

    def _read(self):
        """(current clock, the firmware's average clock) in MHz."""
        if self.sysfs is not None:
            v = self._read_sysfs()
            if self.raw is None:
                self.raw = {"pp_dpm_sclk": v}
            return v, None
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        if self.raw is None:
            self.raw = {k: m.get(k) for k in ("current_gfxclks", "current_gfxclk",
                                              "average_gfxclk_frequency")}
        cl = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and 0 < c < 10000]
        if not cl and isinstance(m.get("current_gfxclk"), int):
            cl = [m["current_gfxclk"]]
        avg = m.get("average_gfxclk_frequency")
        avg = avg if isinstance(avg, int) and 0 < avg < 10000 else None
        return (sum(cl) / len(cl) if cl else None), avg

    def run(self, fn):
        """fn() runs GPU work; sample until it returns."""
        if self.h is None and self.sysfs is None:
            fn()
            return
        stop = threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    v, a = self._read()
                    if v:
                        self.samples.append(v)
                    if a:
                        self.avg_samples.append(a)
                except Exception as e:
                    self.error = f"{type(e).__name__}: {e}"
                    return
                time.sleep(0.002)
        t = threading.Thread(target=loop, daemon=True)
        t.start()
        try:
            fn()
        finally:
            stop.set()
            t.join()

    @staticmethod
    def _median_ghz(xs):
        """Median of the samples in GHz, or None when too few or implausible
        for a loaded MI355X (outside 0.5..3 GHz: an idle or stale reading)."""
        if len(xs) < 5:
            return None
        v = median(xs) / 1000.0
        return v if 0.5 <= v <= 3.0 else None

    def ghz(self):
        return self._median_ghz(self.samples)

    def avg_ghz(self):
        return self._median_ghz(self.avg_samples)


# ---------------------------------------------------------------------------
# workload arithmetic
# ---------------------------------------------------------------------------
GEMM_ROLES_FWD = ["FC1", "FC2"]
GEMM_ROLES_BWD = ["dH", "dB", "dA", "dX"]


def role_flops(w, N=None):
    """Algorithmic FLOPs of each GEMM launch of one step."""
    N = w.N if N is None else N
    per = 2.0 * N * w.H * w.Ft
    sw = w.act == 1
    f = {"FC1": per * (2 if sw else 1), "FC2": per}
    if w.backward:
        f.update({"dH": per, "dB": per, "dA": per * (2 if sw else 1),
                  "dX": per * (2 if sw else 1)})
    return f


def gemm_flops(w, N=None):
    return sum(role_flops(w, N).values())


def role_bytes(w):
    """Algorithmic HBM bytes of each GEMM launch: operands read once, outputs
    written once (bf16 activations, fp32 weight gradients)."""
    N, Hd, Ft = w.N, w.H, w.Ft
    nz = 2 if w.act == 1 else 1
    e2, e4 = 2, 4
    b = {"FC1": (N * Hd + nz * Hd * Ft) * e2 + (nz + 1) * N * Ft * e2,
         "FC2": (N * Ft + Ft * Hd) * e2 + N * Hd * e2}
    if w.backward:
        b.update({"dH": (N * Hd + Ft * Hd + nz * N * Ft) * e2 + nz * N * Ft * e2,
                  "dB": (N * Ft + N * Hd) * e2 + Ft * Hd * e4,
                  "dA": (N * Hd + nz * N * Ft) * e2 + nz * Hd * Ft * e4,
                  "dX": (nz * N * Ft + nz * Hd * Ft) * e2 + N * Hd * e2})
    return b


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, tokens):
    """The fp64 oracle, as it stands, on a token sample of the workload.
    Returns its time, the sample's GEMM FLOPs, and the sample's inputs and
    oracle results (for sample_parity)."""
    import oracle
    import workloads as wl
    d = wl.gen_mlp_inputs(w, n_rows=max(tokens, 1))
    t0 = time.perf_counter()
    f = oracle.mlp_fwd(d["X"], d["A"], d["B"], w.act, d["A_up"])
    b = None
    if w.backward:
        b = oracle.mlp_bwd(d["X"], d["A"], d["B"], w.act, d["dY"], f, d["A_up"])
    dt = time.perf_counter() - t0
    return dt, gemm_flops(w, tokens), (d, f, b)


def sample_parity(torch, tp, w, d, f, b):
    """The HIP shard on the CPU baseline's token sample against the oracle's
    results there: relative Frobenius error ||gpu - oracle|| / ||oracle|| of
    each output tensor (the same inputs; the bar is 2e-2 for bf16 storage,
    1e-5 for fp32)."""
    import numpy as np
    import oracle
    from tensor_transformer_mlp_02_amd.tensors import to_device, to_host, ShardBuffers
    N = d["X"].shape[0]
    desc = dict(S=N, B=1, H=w.H, F_shard=w.Ft, T=w.T, act=w.act, dtype=w.dtype)
    dev = {k: (to_device(d[k]) if d.get(k) is not None else None)
           for k in ("X", "A", "A_up", "B", "dY")}
    buf = ShardBuffers(desc, backward=w.backward)
    tp.tp_mlp_shard_fwd(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], buf.Z, buf.H, buf.Y)
    if w.backward:
        tp.tp_mlp_shard_bwd(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], buf.Z, buf.H,
                            dev["dY"], buf.dX, buf.dA, buf.dA_up, buf.dB, buf.ws, buf.ws_bytes)
    torch.cuda.synchronize()

    def rel(got, ref):
        got = oracle.to_f64(got)
        ref = np.asarray(ref, np.float64)
        nr = np.linalg.norm(ref)
        return float(np.linalg.norm(got - ref) / nr) if nr else float(np.abs(got).max())

    Z = to_host(buf.Z)
    Ft = w.Ft
    errs = {}
    if w.act == 1:
        errs["G"] = rel(Z[:, :Ft], f["Z"])
        errs["U"] = rel(Z[:, Ft:], f["U"])
    else:
        errs["Z"] = rel(Z, f["Z"])
    errs["H"] = rel(to_host(buf.H), f["H"])
    errs["Y"] = rel(to_host(buf.Y), f["Y"])
    if b is not None:
        errs["dX"] = rel(to_host(buf.dX), b["dX"])
        errs["dA"] = rel(to_host(buf.dA), b["dA"])
        if w.act == 1:
            errs["dA_up"] = rel(to_host(buf.dA_up), b["dA_up"])
        errs["dB"] = rel(to_host(buf.dB), b["dB"])
    bar = 2e-2 if w.dtype == 1 else 1e-5
    return {"tokens": int(N), "rel_frob": {k: float(f"{v:.3e}") for k, v in errs.items()},
            "bar": bar, "within_bar": bool(max(errs.values()) <= bar)}


# ---------------------------------------------------------------------------
# the shard step
# ---------------------------------------------------------------------------
class ShardBench:
    """Inputs (several sets), outputs and stand-in partials of one dense
    workload, and its timed steps."""

    def __init__(self, torch, tp, wl, w, n_sets, hev, sum_workgroups, streams):
        from tensor_transformer_mlp_02_amd.tensors import to_device, ShardBuffers
        self.torch, self.tp, self.w, self.hev = torch, tp, w, hev
        self.stream, self.side = streams
        self.sum_workgroups = sum_workgroups
        self.sets = []
        for s in range(max(1, n_sets)):
            d = wl.gen_mlp_inputs(w, set_index=s)
            self.sets.append({k: (to_device(v) if v is not None else None)
                              for k, v in d.items() if k in ("X", "A", "A_up", "B", "dY")})
        self.desc = dict(S=w.S, B=w.B, H=w.H, F_shard=w.Ft, T=w.T, act=w.act, dtype=w.dtype)
        self.buf = ShardBuffers(self.desc, backward=w.backward)
        self.stand = [to_device(p) for p in wl.gen_partials(w, w.T - 1, (w.N, w.H), 0.05)]
        self.Ysum = torch.empty_like(self.buf.Y)
        self.dXsum = torch.empty_like(self.buf.Y)
        self.count = w.N * w.H

    def input_bytes(self, n_sets):
        s = self.sets[0]
        return n_sets * sum(t.numel() * t.element_size() for t in s.values() if t is not None)

    def run(self, n_sets, overlap, steps, warmup, timed=True, y_after="FC2"):
        """Warmup + timed steps rotating the first n_sets input sets.  Returns
        per-step durations (ms) and each launch's durations by role.
        y_after: the launch after which sum(Y) may start (FC2: as soon as Y
        is written; a backward GEMM's name: once that GEMM has finished, so
        the sum overlaps the later ones)."""
        torch, tp, w, hev = self.torch, self.tp, self.w, self.hev
        stream = self.stream
        side = self.side if overlap else stream
        buf, stand, count = self.buf, self.stand, self.count
        desc = self.desc

        def psum(T, parts, out, st):
            if overlap:
                return tp.tp_partial_sum_capped(w.dtype, T, parts, count, out,
                                                self.sum_workgroups, stream=st)
            return tp.tp_partial_sum(w.dtype, T, parts, count, out, stream=st)

        # events keep every dependency: a sum starts after the GEMM that
        # wrote its input, and the next write of Y (forward) or dX (backward)
        # waits for the sum that reads it
        y_ready, dx_ready = torch.cuda.Event(), torch.cuda.Event()
        y_read, dx_read = torch.cuda.Event(), torch.cuda.Event()
        y_read.record(side)
        dx_read.record(side)
        n_ev = 2 * (len(GEMM_ROLES_FWD) + 1 + (len(GEMM_ROLES_BWD) + 1 if w.backward else 0))

        # the launch events double as the dependency that delays sum(Y)
        # until a backward GEMM has finished (its "after" event)
        late_y = y_after != "FC2" and w.backward and overlap
        if late_y and y_after not in GEMM_ROLES_BWD:
            raise ValueError(f"y_after must be FC2 or one of {GEMM_ROLES_BWD}")
        # order of the timed units within a step
        order = GEMM_ROLES_FWD + ([] if late_y else ["sumY"]) + \
            (GEMM_ROLES_BWD + (["sumY"] if late_y else []) + ["sumdX"] if w.backward else [])
        unit = {r: i for i, r in enumerate(order)}

        def step(k, evs=None):
            s = self.sets[k % n_sets]
            if evs is not None:
                tp.tp_launch_events(evs)
            stream.wait_event(y_read)
            tp.tp_mlp_shard_fwd(desc, s["X"], s["A"], s["A_up"], s["B"], buf.Z, buf.H, buf.Y,
                                stream=stream)
            y_ready.record(stream)
            if not late_y:
                side.wait_event(y_ready)
                psum(w.T, [buf.Y] + stand, self.Ysum, side)
                y_read.record(side)
            if w.backward:
                stream.wait_event(dx_read)
                tp.tp_mlp_shard_bwd(desc, s["X"], s["A"], s["A_up"], s["B"], buf.Z, buf.H,
                                    s["dY"], buf.dX, buf.dA, buf.dA_up, buf.dB, buf.ws,
                                    buf.ws_bytes, stream=stream)
                dx_ready.record(stream)
                if late_y:
                    hev.wait(side, evs[2 * unit[y_after] + 1])
                    psum(w.T, [buf.Y] + stand, self.Ysum, side)
                    y_read.record(side)
                side.wait_event(dx_ready)
                psum(w.T, [buf.dX] + stand, self.dXsum, side)
                dx_read.record(side)
            if evs is not None:
                used = tp.tp_launch_events_used()
                tp.tp_launch_events(None)
                if used != n_ev:
                    raise RuntimeError(f"{used} launch events recorded, {n_ev} expected")

        for k in range(warmup):
            step(k, hev.create(n_ev) if late_y else None)
        torch.cuda.synchronize()
        if not timed:
            hev.free()
            return None

        def timed_pass(first, with_launch_events):
            """`steps` steps, each started by a timing event; with launch
            events, every launch of the step is also bracketed by a pair."""
            starts = hev.create(steps + 1)
            launch_evs = [hev.create(n_ev) if with_launch_events else None
                          for _ in range(steps)]
            torch.cuda.synchronize()
            for k in range(steps):
                hev.record(starts[k], stream)
                if k == 0:
                    side.wait_stream(stream)
                step(first + k, launch_evs[k])
            side_done = torch.cuda.Event()
            side_done.record(side)
            stream.wait_event(side_done)
            hev.record(starts[steps], stream)
            torch.cuda.synchronize()
            step_ms = [hev.ms(starts[k], starts[k + 1]) for k in range(steps)]
            total_ms = hev.ms(starts[0], starts[steps])
            per_role = None
            if with_launch_events:
                per_role = {r: [hev.ms(e[2 * i], e[2 * i + 1]) for e in launch_evs]
                            for i, r in enumerate(order)}
            return step_ms, total_ms, per_role

        # A timing event between two kernels makes the second wait for the
        # first to drain completely (~12 us per launch boundary on MI355X),
        # so the step times come from steps that record only their start,
        # and the per-launch durations from a second pass of the same steps
        # with every launch bracketed (the launches' own durations are what
        # that pass measures; the gaps it adds between them are not counted).
        if late_y:
            # the launch events are also the dependency that delays sum(Y)
            step_ms, total_ms, per_role = timed_pass(warmup, True)
            launch_step_ms = step_ms
        else:
            step_ms, total_ms, _ = timed_pass(warmup, False)
            launch_step_ms, _, per_role = timed_pass(warmup + steps, True)
        hev.free()
        return {"step_ms": step_ms, "total_ms": total_ms, "roles": per_role,
                "launch_pass_step_ms": launch_step_ms}


def summarize(w, res, label):
    """Median step, GEMM time per step and each GEMM launch's figures."""
    fl = role_flops(w)
    flops = sum(fl.values())
    med = median(res["step_ms"])
    roles = {}
    for r, f in fl.items():
        us = median(res["roles"][r]) * 1e3
        roles[r] = {"us": round(us, 1), "tflops": round(tflops(f, us * 1e-3), 1),
                    "frac": round(tflops(f, us * 1e-3) / PEAK_BF16_TFLOPS, 4)}
    gemm_ms = sum(median(res["roles"][r]) for r in fl)
    out = {"inputs": label,
           "ms_per_step_median": round(med, 4),
           "ms_per_step_mean": round(res["total_ms"] / len(res["step_ms"]), 4),
           "launch_timing_pass_ms_per_step": round(median(res["launch_pass_step_ms"]), 4),
           "tflops": round(tflops(flops, med), 2),
           "gemm_ms": round(gemm_ms, 4),
           "gemm_tflops": round(tflops(flops, gemm_ms), 2),
           "gemm_frac_of_bf16_peak": round(tflops(flops, gemm_ms) / PEAK_BF16_TFLOPS, 4),
           "gemm_target_ms_at_60pct": round(flops / (TARGET_FRAC * PEAK_BF16_TFLOPS * 1e12) * 1e3,
                                            4),
           "launches": roles}
    sums = [x for r in ("sumY", "sumdX") if r in res["roles"] for x in res["roles"][r]]
    if sums:
        ps_ms = median(sums)
        ps_bytes = (w.T + 1) * w.N * w.H * 2
        out["partial_sum_us"] = round(ps_ms * 1e3, 1)
        out["partial_sum_GBps"] = round(ps_bytes / (ps_ms * 1e-3) / 1e9, 1)
        out["partial_sum_hbm_frac"] = round(ps_bytes / (ps_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    return out


# ---------------------------------------------------------------------------
# side measurements
# ---------------------------------------------------------------------------
def grouped_expert_timing(torch, tp, wl, hev, n_sets, steps=20, warmup=3, capacity=None):
    """The grouped local experts on the grouped-expert workload (16384 tokens
    routed top-2 over 64 experts, local experts 0..7, H = 4096, F = 1408,
    SwiGLU): forward and backward over the ragged rows, rotating input sets,
    each launch timed with events; algorithmic TFLOP/s (6 H F per row
    forward, 12 H F backward).  The step median comes from steps that record
    only their start; the launch durations from as many steps with every
    launch bracketed.  With `capacity` the row offsets stay in GPU memory
    (the device-offset calls) and the row buffers hold `capacity` rows, of
    which the routed ones are the first."""
    from tensor_transformer_mlp_02_amd.tensors import to_device, ExpertBuffers
    w5 = wl.WORKLOADS["c5_bf16_grouped_swiglu"]
    sets = []
    for s in range(n_sets):
        g = wl.gen_grouped_inputs(w5, set_index=s)
        d = {k: to_device(g[k]) for k in ("X_perm", "Wg", "Wu", "Wd", "dY_perm")}
        if capacity is not None:
            for k in ("X_perm", "dY_perm"):
                full = torch.zeros((capacity, w5.H), dtype=d[k].dtype, device=d[k].device)
                full[:d[k].shape[0]].copy_(d[k])
                d[k] = full
        sets.append(d)
    off = g["offsets"]
    R, E, H, F = int(off[-1]), len(off) - 1, w5.H, w5.F
    desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
    # (buffers sized by the last offset: `capacity` rows in the device case)
    buf = ExpertBuffers(desc, off if capacity is None else [0] * E + [capacity])
    off_dev = (torch.tensor(off, dtype=torch.int32, device="cuda")
               if capacity is not None else None)
    stream = torch.cuda.current_stream()
    roles = ["FC1", "FC2", "dH", "dWd", "dWg|dWu", "dX"]

    def step(k, evs=None):
        d = sets[k % n_sets]
        if evs is not None:
            tp.tp_launch_events(evs)
        if capacity is None:
            tp.tp_grouped_expert_fwd(desc, off, d["X_perm"], d["Wg"], d["Wu"], d["Wd"], buf.Z,
                                     buf.H, buf.Y, stream=stream)
            tp.tp_grouped_expert_bwd(desc, off, d["X_perm"], d["Wg"], d["Wu"], d["Wd"], buf.Z,
                                     buf.H, d["dY_perm"], buf.dX, buf.dWg, buf.dWu, buf.dWd,
                                     buf.ws, buf.ws_bytes, stream=stream)
        else:
            tp.tp_grouped_expert_fwd_devoff(desc, capacity, off_dev, d["X_perm"], d["Wg"],
                                            d["Wu"], d["Wd"], buf.Z, buf.H, buf.Y, stream=stream)
            tp.tp_grouped_expert_bwd_devoff(desc, capacity, off_dev, d["X_perm"], d["Wg"],
                                            d["Wu"], d["Wd"], buf.Z, buf.H, d["dY_perm"], buf.dX,
                                            buf.dWg, buf.dWu, buf.dWd, buf.ws, buf.ws_bytes,
                                            stream=stream)
        if evs is not None:
            tp.tp_launch_events(None)
    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()

    def timed_pass(first, with_launch_events):
        # (launch events stall each launch boundary: the step times come from
        # a pass without them, the launch durations from a pass with them)
        starts = hev.create(steps + 1)
        evs = [hev.create(2 * len(roles)) if with_launch_events else None
               for _ in range(steps)]
        for k in range(steps):
            hev.record(starts[k], stream)
            step(first + k, evs[k])
        hev.record(starts[steps], stream)
        torch.cuda.synchronize()
        s_ms = median([hev.ms(starts[k], starts[k + 1]) for k in range(steps)])
        p = None
        if with_launch_events:
            p = {r: median([hev.ms(e[2 * i], e[2 * i + 1]) for e in evs])
                 for i, r in enumerate(roles)}
        return s_ms, p

    step_ms, _ = timed_pass(warmup, False)
    launch_pass_ms, per = timed_pass(warmup + steps, True)
    hev.free()
    fl = {"FC1": 4.0 * H * F * R, "FC2": 2.0 * H * F * R, "dH": 2.0 * H * F * R,
          "dWd": 2.0 * H * F * R, "dWg|dWu": 4.0 * H * F * R, "dX": 4.0 * H * F * R}
    tot = sum(fl.values())
    f_ms = per["FC1"] + per["FC2"]
    b_ms = sum(per[r] for r in roles[2:])
    return {"rows": R, "experts": E, "rows_per_expert": [int(x) for x in off[1:] - off[:-1]],
            "H": H, "F": F, "inputs": f"{n_sets} input sets rotated",
            "offsets": "host" if capacity is None else "device",
            "buffer_rows": R if capacity is None else capacity,
            "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "step_ms_median": round(step_ms, 4),
            "launch_timing_pass_step_ms": round(launch_pass_ms, 4),
            "tflops": round(tflops(tot, step_ms), 1),
            "frac_of_bf16_peak": round(tflops(tot, step_ms) / PEAK_BF16_TFLOPS, 4),
            "launches": {r: {"us": round(per[r] * 1e3, 1),
                             "tflops": round(tflops(fl[r], per[r]), 1),
                             "frac": round(tflops(fl[r], per[r]) / PEAK_BF16_TFLOPS, 4)}
                         for r in roles}}


def grouped_timing_all(torch, tp, wl, hev, n_sets, offsets="both"):
    """The grouped experts with host offsets, then with device offsets on
    buffers of exactly the routed rows and on buffers of every row that
    could be routed here (tokens x top-k: the size a caller that never
    reads the counts back must provide).  offsets: "both", "host" or
    "device" (one kind per profiled run keeps its per-kernel figures
    apart)."""
    w5 = wl.WORKLOADS["c5_bf16_grouped_swiglu"]
    res = grouped_expert_timing(torch, tp, wl, hev, n_sets) if offsets != "device" else {}
    if offsets == "host":
        return res
    rows = int(wl.gen_grouped_inputs(w5)["offsets"][-1])
    keep = ("buffer_rows", "fwd_ms", "bwd_ms", "step_ms_median", "tflops", "frac_of_bf16_peak")
    dev = {}
    for name, cap in (("exact", rows), ("tokens_x_topk", w5.tokens * w5.topk)):
        r = grouped_expert_timing(torch, tp, wl, hev, n_sets, capacity=cap)
        dev[name] = {k: r[k] for k in keep}
        dev[name]["launch_us"] = {k: v["us"] for k, v in r["launches"].items()}
    res["device_offsets"] = dev
    return res


def moe_dispatch_timing(torch, tp, wl, dev, stream, hev, reps=20):
    """Token dispatch and combine around the grouped experts on the
    grouped-expert workload's routing (16384 tokens, top-2 of 64 experts,
    local experts 0..7, H = 4096): permute, weighted combine and the
    combine's backward, each in GB/s of algorithmic row traffic (median of
    event-timed launches)."""
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
        evs = hev.create(2 * reps)
        for k in range(reps):
            tp.tp_launch_events(evs[2 * k:2 * k + 2])
            fn()
        tp.tp_launch_events(None)
        torch.cuda.synchronize()
        us = median([hev.ms(evs[2 * k], evs[2 * k + 1]) for k in range(reps)]) * 1e3
        out[name] = {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    hev.free()
    return out


def fp8_timing(torch, tp, wl, w, X, A, Au, B, dY, stream, hev, reps=10):
    """The shard forward and backward on FP8 codes at the same shape
    (E4M3 weights and activations, E5M2 gradients): the GEMM calls alone,
    and the quantization each needs (forward: X and the weights' transposes;
    backward: dY and its transpose, the transposes of X's and H's codes, the
    weights in their own layout).  Medians of event-timed repetitions."""
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
    torch.cuda.synchronize()
    parts = [quant_fwd, fwd, quant_bwd, bwd]
    evs = hev.create(reps * 5)
    for k in range(reps):
        for i, fn in enumerate(parts):
            hev.record(evs[5 * k + i], stream)
            fn()
        hev.record(evs[5 * k + 4], stream)
    torch.cuda.synchronize()
    ms = [median([hev.ms(evs[5 * k + i], evs[5 * k + i + 1]) for k in range(reps)])
          for i in range(4)]
    hev.free()
    # each launch of the two calls, timed on its own (launch-timing hook)
    f_units = ["zero h_amax", "FC1", "FC2"]
    b_units = ["zero dz_amax", "dH", "dZ code transpose", "dB", "dA", "dX"]
    per = {u: [] for u in f_units + b_units}
    for k in range(reps):
        for fn, units in ((fwd, f_units), (bwd, b_units)):
            ev = hev.create(2 * len(units))
            tp.tp_launch_events(ev)
            fn()
            tp.tp_launch_events(None)
            torch.cuda.synchronize()
            for i, u in enumerate(units):
                per[u].append(hev.ms(ev[2 * i], ev[2 * i + 1]))
    hev.free()
    per = {u: median(v) for u, v in per.items()}
    # the next step's scales from the amax history (window 16): one call for
    # the E4M3 tensors (X, A, A_up, B, H), one for the E5M2 ones (dY, dZ),
    # on buffers of their own (the scales timed above stay as they are)
    hist = torch.zeros((7, 16), dtype=torch.float32, device=dev)
    am = amax[:7].clone()
    sc = torch.ones(7, dtype=torch.float32, device=dev)
    inv = torch.ones(7, dtype=torch.float32, device=dev)
    su_ev = hev.create(2 * reps)
    for k in range(reps):
        hev.record(su_ev[2 * k], stream)
        tp.tp_fp8_scale_update(E4, 5, 16, hist[:5], am[:5], sc[:5], inv[:5], stream=stream)
        tp.tp_fp8_scale_update(E5, 2, 16, hist[5:], am[5:], sc[5:], inv[5:], stream=stream)
        hev.record(su_ev[2 * k + 1], stream)
    torch.cuda.synchronize()
    su_us = median([hev.ms(su_ev[2 * k], su_ev[2 * k + 1]) for k in range(reps)]) * 1e3
    hev.free()
    f_fl = 2.0 * N * Hd * Ft * (3 if sw else 2)
    b_fl = 2 * f_fl
    tf = lambda fl, t: round(tflops(fl, t), 1)
    per_fl = {"FC1": 2.0 * N * Hd * Ft * (2 if sw else 1), "FC2": 2.0 * N * Hd * Ft,
              "dH": 2.0 * N * Hd * Ft, "dB": 2.0 * N * Hd * Ft,
              "dA": 2.0 * N * Hd * Ft * (2 if sw else 1), "dX": 2.0 * N * Hd * Ft * (2 if sw else 1)}
    launches = {u: {"us": round(per[u] * 1e3, 1)} for u in per}
    for u, fl in per_fl.items():
        launches[u]["frac_of_fp8_peak"] = round(tflops(fl, per[u]) / PEAK_FP8_TFLOPS, 4)
    fwd_d = {"gemm_ms": round(ms[1], 4), "gemm_tflops": tf(f_fl, ms[1]),
             "gemm_frac_of_fp8_peak": round(tflops(f_fl, ms[1]) / PEAK_FP8_TFLOPS, 4),
             "quantize_ms": round(ms[0], 4),
             "forward_tflops_with_quantize": tf(f_fl, ms[0] + ms[1])}
    bwd_d = {"ms": round(ms[3], 4), "tflops": tf(b_fl, ms[3]),
             "frac_of_fp8_peak": round(tflops(b_fl, ms[3]) / PEAK_FP8_TFLOPS, 4),
             "quantize_transpose_ms": round(ms[2], 4),
             "backward_tflops_with_quantize": tf(b_fl, ms[2] + ms[3]),
             "step_tflops_with_quantize": tf(f_fl + b_fl, sum(ms)),
             "launches": launches,
             "scale_update": {"tensors": 7, "window": 16, "calls": 2, "us": round(su_us, 1)}}
    return fwd_d, bwd_d


def reduce_scatter_timing(torch, tp, w, sb, hev, reps=20):
    """Sequence-parallel form of the same exchange: rank 0's [S/T,B,H] slice
    of the sum (the reduce-scatter arithmetic)."""
    stream = torch.cuda.current_stream()
    out = torch.empty((w.S // w.T) * w.B * w.H, dtype=sb.Ysum.dtype, device=sb.Ysum.device)
    parts = [sb.buf.Y] + sb.stand
    for _ in range(3):
        tp.tp_partial_sum_scatter(w.dtype, w.T, parts, w.S, w.B, w.H, 0, out)
    evs = hev.create(2 * reps)
    for k in range(reps):
        tp.tp_launch_events(evs[2 * k:2 * k + 2])
        tp.tp_partial_sum_scatter(w.dtype, w.T, parts, w.S, w.B, w.H, 0, out, stream=stream)
    tp.tp_launch_events(None)
    torch.cuda.synchronize()
    ms = median([hev.ms(evs[2 * k], evs[2 * k + 1]) for k in range(reps)])
    hev.free()
    nbytes = (w.T + 1) * out.numel() * 2
    return {"us": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bytes": nbytes}


def accumulation_timing(torch, tp, sb, hev, reps=5):
    """The backward with the weight gradients added into the fp32 buffers,
    beside the plain backward (median of event-timed calls)."""
    stream = torch.cuda.current_stream()
    s, b, d = sb.sets[0], sb.buf, sb.desc
    out = {}
    for name, fn in (("bwd_ms", tp.tp_mlp_shard_bwd), ("bwd_accum_ms", tp.tp_mlp_shard_bwd_accum)):
        evs = hev.create(2 * reps)
        for k in range(reps):
            hev.record(evs[2 * k], stream)
            fn(d, s["X"], s["A"], s["A_up"], s["B"], b.Z, b.H, s["dY"], b.dX, b.dA, b.dA_up,
               b.dB, b.ws, b.ws_bytes, stream=stream)
            hev.record(evs[2 * k + 1], stream)
        torch.cuda.synchronize()
        out[name] = round(median([hev.ms(evs[2 * k], evs[2 * k + 1]) for k in range(reps)]), 4)
    hev.free()
    return out


def dact_placement_timing(torch, tp, w, sb, hev, reps=5):
    """The backward with the activation derivative in the epilogue of dY B^T
    (tp_mlp_shard_bwd, the default) beside the backward whose dA and dX
    GEMMs form dZ from dH and Z as they load it
    (tp_mlp_shard_bwd_dact_prologue): each call's median duration, and each
    launch's from the same calls with every launch bracketed by events."""
    stream = torch.cuda.current_stream()
    s, b, d = sb.sets[0], sb.buf, sb.desc
    # the saved Z and H of this input set
    tp.tp_mlp_shard_fwd(d, s["X"], s["A"], s["A_up"], s["B"], b.Z, b.H, b.Y, stream=stream)
    fl = role_flops(w)
    out = {}
    for name, fn in (("epilogue", tp.tp_mlp_shard_bwd),
                     ("operand_loads", tp.tp_mlp_shard_bwd_dact_prologue)):
        calls = hev.create(2 * reps)
        per = [hev.create(2 * len(GEMM_ROLES_BWD)) for _ in range(reps)]
        for k in range(2 * reps):
            timed_launches = k >= reps
            if timed_launches:
                tp.tp_launch_events(per[k - reps])
            else:
                hev.record(calls[2 * k], stream)
            fn(d, s["X"], s["A"], s["A_up"], s["B"], b.Z, b.H, s["dY"], b.dX, b.dA, b.dA_up,
               b.dB, b.ws, b.ws_bytes, stream=stream)
            if timed_launches:
                tp.tp_launch_events(None)
            else:
                hev.record(calls[2 * k + 1], stream)
        torch.cuda.synchronize()
        ms = median([hev.ms(calls[2 * k], calls[2 * k + 1]) for k in range(reps)])
        launches = {}
        for i, r in enumerate(GEMM_ROLES_BWD):
            us = median([hev.ms(e[2 * i], e[2 * i + 1]) for e in per]) * 1e3
            launches[r] = {"us": round(us, 1), "tflops": round(tflops(fl[r], us * 1e-3), 1)}
        out[name] = {"bwd_ms": round(ms, 4),
                     "tflops": round(tflops(sum(fl[r] for r in GEMM_ROLES_BWD), ms), 1),
                     "launches": launches}
        hev.free()
    out["default"] = "epilogue"
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs one tensor-parallel rank's shard on ONE GPU; multi-GPU runs "
              "(collectives across GPUs) are not part of this library", file=sys.stderr)
        sys.exit(2)

    import torch
    import tensor_transformer_mlp_02_amd as tp
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    assert w.dtype == wl.DT_BF16
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    hev = HipEvents(torch)
    overlap = bool(args.overlap)
    # the compute and side streams are made once, one after the other: HIP
    # hands new streams hardware queues in turn, so two consecutive ones
    # never share a queue (a shared queue would run the sums in order)
    streams = (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev))
    torch.cuda.set_stream(streams[0])
    progress = lambda msg: print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # calibration copy (one partial sum of a single buffer = a copy)
    n_calib = CALIB_COPY_BYTES // 2
    calib_src = torch.zeros(n_calib, dtype=torch.bfloat16, device=dev)
    calib_dst = torch.empty_like(calib_src)
    tp.tp_partial_sum(w.dtype, 1, [calib_src], n_calib, calib_dst)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    if args.only == "grouped":
        print(json.dumps({"grouped_experts": grouped_timing_all(torch, tp, wl, hev, args.sets,
                                                                args.grouped_offsets)}),
              flush=True)
        return
    if args.only == "fp8":
        d0 = wl.gen_mlp_inputs(w)
        from tensor_transformer_mlp_02_amd.tensors import to_device
        t = {k: (to_device(v) if v is not None else None) for k, v in d0.items()
             if k in ("X", "A", "A_up", "B", "dY")}
        f8, f8b = fp8_timing(torch, tp, wl, w, t["X"], t["A"], t["A_up"], t["B"], t["dY"],
                             torch.cuda.current_stream(), hev)
        print(json.dumps({"fp8_forward": f8, "fp8_backward": f8b}), flush=True)
        return
    progress(f"{w.name}: drawing {args.sets} input sets")
    sb = ShardBench(torch, tp, wl, w, args.sets, hev, args.sum_workgroups, streams)
    if args.only == "dact":
        print(json.dumps({"act_derivative_placement": dact_placement_timing(torch, tp, w, sb,
                                                                            hev)}), flush=True)
        return
    progress("headline steps")
    cold = sb.run(args.sets, overlap, args.steps, args.warmup, y_after=args.sum_y_after)
    head = summarize(w, cold, f"{args.sets} input sets rotated "
                              f"({sb.input_bytes(args.sets) / 2**20:.0f} MiB): cold caches")
    warm = serial = None
    if args.side:
        progress("warm and in-order steps")
        warm = summarize(w, sb.run(1, overlap, args.steps, args.warmup,
                                   y_after=args.sum_y_after),
                         "one input set: warm caches")
        if overlap:
            serial = summarize(w, sb.run(args.sets, False, args.steps, args.warmup),
                               f"{args.sets} input sets rotated, in order on one stream")

    clock = None
    if args.clock:
        progress("clock sampling")
        cs = ClockSampler(torch)
        n_clock = max(50, int(400.0 / max(head["ms_per_step_median"], 0.1)))
        cs.run(lambda: sb.run(args.sets, overlap, 0, n_clock, timed=False,
                              y_after=args.sum_y_after))
        ghz = cs.ghz()
        avg = cs.avg_ghz()
        gemm_tf = head["gemm_tflops"]
        clock = {"sclk_ghz": None if ghz is None else round(ghz, 3),
                 "avg_gfxclk_ghz": None if avg is None else round(avg, 3),
                 "samples": len(cs.samples),
                 "source": ("the driver's current shader-clock level (pp_dpm_sclk)"
                            if cs.sysfs else
                            "amdsmi gpu metrics (mean of the per-XCD current graphics clocks; "
                            "the firmware's average clock beside it)")
                           + f", median of samples every ~2 ms while {n_clock} more headline "
                             "steps ran in this process",
                 "first_sample": cs.raw,
                 "error": cs.error}
        if ghz:
            clock["bf16_peak_at_sclk"] = round(PEAK_BF16_TFLOPS * ghz / 2.4, 1)
            clock["gemm_frac_at_sclk"] = round(gemm_tf / (PEAK_BF16_TFLOPS * ghz / 2.4), 4)

    rs = acc_cmp = dact_cmp = None
    if args.side and w.S % w.T == 0:
        rs = reduce_scatter_timing(torch, tp, w, sb, hev)
    if args.side and w.backward:
        acc_cmp = accumulation_timing(torch, tp, sb, hev)
        progress("activation-derivative placement")
        dact_cmp = dact_placement_timing(torch, tp, w, sb, hev)
    f8 = f8b = None
    if (args.side and args.fp8 and w.H % 128 == 0 and w.Ft % 128 == 0 and w.N % 128 == 0
            and w.backward):
        progress("fp8")
        s0 = sb.sets[0]
        f8, f8b = fp8_timing(torch, tp, wl, w, s0["X"], s0["A"], s0["A_up"], s0["B"], s0["dY"],
                             torch.cuda.current_stream(), hev)
    del sb
    torch.cuda.empty_cache()

    # the other dense shard shapes: GeLU forward only, and with the backward
    others = {}
    if args.side:
        for name in ("c2_bf16_gelu_fwd", "c3_bf16_gelu_fwdbwd"):
            if name == w.name:
                continue
            progress(name)
            wo = wl.WORKLOADS[name]
            so = ShardBench(torch, tp, wl, wo, args.sets, hev, args.sum_workgroups, streams)
            r = summarize(wo, so.run(args.sets, overlap, args.steps, args.warmup,
                                     y_after=args.sum_y_after),
                          f"{args.sets} input sets rotated: cold caches")
            r["gflop_per_step"] = round(gemm_flops(wo) / 1e9, 1)
            others[name] = r
            del so
            torch.cuda.empty_cache()

    moe = grouped = None
    if args.side and args.moe:
        progress("grouped experts and MoE row moves")
        moe = moe_dispatch_timing(torch, tp, wl, dev, torch.cuda.current_stream(), hev)
        grouped = grouped_timing_all(torch, tp, wl, hev, args.sets, args.grouped_offsets)

    flops = gemm_flops(w)
    value = tflops(flops, head["ms_per_step_median"])
    # dominant kernel: the GEMM launch with the longest median duration
    dom = max(head["launches"], key=lambda r: head["launches"][r]["us"])
    dl = head["launches"][dom]
    rb = role_bytes(w)
    traffic = recorded_fields(TRAFFIC_FILE)
    dom_traffic = None
    if traffic is not None:
        try:
            dom_traffic = float(traffic[f"hbm_bytes_{dom}"])
        except (KeyError, ValueError):
            dom_traffic = None

    line = {
        "metric": "TP-shard MLP fwd+bwd TFLOP/s on 1 GPU + % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step_median"],
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
                                    "workgroups" % args.sum_workgroups) if overlap
                                   else "in order on the compute stream",
                   "act_derivative": "epilogue of the dY B^T GEMM (dZ written once)",
                   "caches": head["inputs"],
                   "timing": "median of the timed steps' intervals (a HIP event at each "
                             "step's start on the compute stream); per-launch durations "
                             "from a second pass of as many steps with every launch "
                             "bracketed by HIP events (such events stall each launch "
                             "boundary, so they stay out of the headline steps)"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "kernel": f"{dom} GEMM (the longest launch of the step)",
            "bound": "mfma",
            "achieved": dl["tflops"],
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": dl["frac"],
            "traffic": dom_traffic,
            "algorithmic_bytes": rb[dom],
            "flops_per_launch": role_flops(w)[dom],
            "launch_us_median": dl["us"],
        },
        "step": head,
        "warm_step": warm,
        "serial_step": serial,
        "clock_under_load": clock,
        "other_shapes": others or None,
        "reduce_scatter_rank0": rs,
        "grad_accumulation": acc_cmp,
        "act_derivative_placement": dact_cmp,
        "moe_dispatch_combine": moe,
        "grouped_experts": grouped,
        "fp8_forward": f8,
        "fp8_backward": f8b,
    }
    if f8b is not None:
        f8b["bf16_backward_ms_for_comparison"] = round(
            sum(head["launches"][r]["us"] for r in GEMM_ROLES_BWD) / 1e3, 4)
        f8["bf16_forward_ms_for_comparison"] = round(
            sum(head["launches"][r]["us"] for r in GEMM_ROLES_FWD) / 1e3, 4)

    if not args.no_cpu_baseline:
        import oracle
        progress("cpu baseline")
        tokens = args.cpu_tokens
        if tokens <= 0:
            dt, fl, _ = cpu_baseline(w, 128)        # calibrate on 128 tokens
            rate = fl / max(dt, 1e-6)
            tokens = int(max(16, min(w.N, 20.0 * rate / gemm_flops(w, 1))))
        dt, fl, (d_s, f_s, b_s) = cpu_baseline(w, tokens)
        line["cpu_baseline"] = {
            "value": round(fl / dt / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"fp64 oracle, forward+backward of the same shard on {tokens} of "
                      f"{w.N} tokens ({fl / 1e9:.1f} GFLOP in {dt:.1f} s)",
            "cpu": cpu_model(),
        }
        progress("parity on the baseline's sample")
        line["parity"] = sample_parity(torch, tp, w, d_s, f_s, b_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
