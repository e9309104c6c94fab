"""GPU parity of the grouped experts with device-resident row offsets
(tp_grouped_expert_fwd_devoff / tp_grouped_expert_bwd_devoff).

The offsets live in an int32 GPU tensor (here written by a torch kernel on
the same stream, as a routing step would), the buffers hold R rows.  Checked:
whole tensors against the fp64 oracle's grouped forward and backward on
ragged splits with empty experts (the 256-row kernels' spare workgroups and
every kernel the launcher can pick), rows past the last offset left
unwritten, offsets out of order or out of range taken clamped, weight
gradients accumulated, the full grouped workload against the host-offset
call, and a captured graph replayed after the offsets changed in place.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_02_amd as tp
import workloads as wl
from tensor_transformer_mlp_02_amd.tensors import to_device, to_host, ExpertBuffers
from parity import TOL, assert_close, f64, sample_idx

pytestmark = pytest.mark.gpu

SENTINEL = 0x7fc1  # a bf16 NaN no kernel writes


def _inputs(counts, H, F, R=None, seed=85):
    E = len(counts)
    off = np.zeros(E + 1, np.int64)
    off[1:] = np.cumsum(counts)
    R = int(off[-1]) if R is None else R
    return {
        "offsets": off, "R": R,
        "X_perm": wl.normal_bf16(1000 * seed + 1, (R, H), 1.0),
        "Wg": wl.normal_bf16(1000 * seed + 2, (E, H, F), 0.05),
        "Wu": wl.normal_bf16(1000 * seed + 3, (E, H, F), 0.05),
        "Wd": wl.normal_bf16(1000 * seed + 4, (E, F, H), 0.05),
        "dY_perm": wl.normal_bf16(1000 * seed + 5, (R, H), 1e-2),
    }


class _Out:
    """[R]-row outputs filled with a sentinel, fp32 weight gradients."""

    def __init__(self, E, H, F, R):
        def bf(shape):
            return torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        self.Z, self.H, self.Y, self.dX = bf((R, 2 * F)), bf((R, F)), bf((R, H)), bf((R, H))
        self.dWg = torch.full((E, H, F), float("nan"), device="cuda")
        self.dWu = torch.full((E, H, F), float("nan"), device="cuda")
        self.dWd = torch.full((E, F, H), float("nan"), device="cuda")
        desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
        self.ws_bytes = tp.tp_grouped_expert_devoff_workspace(desc, R)
        self.ws = torch.empty(max(16, self.ws_bytes), dtype=torch.uint8, device="cuda")


def _device_offsets(counts):
    """E+1 int32 offsets computed on the GPU from per-expert counts."""
    c = torch.tensor(list(counts), dtype=torch.int32, device="cuda")
    return torch.cat([torch.zeros(1, dtype=torch.int32, device="cuda"),
                      torch.cumsum(c, 0, dtype=torch.int32)])


def _run(d, H, F, off_dev, accumulate=False, out=None):
    E = d["Wg"].shape[0]
    R = d["R"]
    desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
    dev = {k: to_device(d[k]) for k in ("X_perm", "Wg", "Wu", "Wd", "dY_perm")}
    o = out if out is not None else _Out(E, H, F, R)
    print(f"[gpu] devoff fwd H={H} F={F} R={R} offsets={off_dev.tolist()}", flush=True)
    tp.tp_grouped_expert_fwd_devoff(desc, R, off_dev, dev["X_perm"], dev["Wg"], dev["Wu"],
                                    dev["Wd"], o.Z, o.H, o.Y)
    print(f"[gpu] devoff bwd accumulate={accumulate}", flush=True)
    tp.tp_grouped_expert_bwd_devoff(desc, R, off_dev, dev["X_perm"], dev["Wg"], dev["Wu"],
                                    dev["Wd"], o.Z, o.H, dev["dY_perm"], o.dX, o.dWg, o.dWu,
                                    o.dWd, o.ws, o.ws_bytes, accumulate=accumulate)
    torch.cuda.synchronize()
    return dev, o


def _clamped(vals, R):
    """The offsets as the kernels take them."""
    out, prev = [], 0
    for i, v in enumerate(vals):
        prev = min(max(int(v), 0 if i == 0 else prev), R)
        out.append(prev)
    return np.array(out, np.int64)


def _check_oracle(d, off, o, H, F):
    """Rows [off[0], off[E]) and every weight gradient against the oracle;
    the other rows still hold the sentinel."""
    lo, hi = int(off[0]), int(off[-1])
    E = len(off) - 1
    tol = TOL[wl.DT_BF16]
    rel = off - lo
    X, dY = d["X_perm"][lo:hi], d["dY_perm"][lo:hi]
    f = oracle.grouped_fwd(X, rel, d["Wg"], d["Wu"], d["Wd"])
    b = oracle.grouped_bwd(X, rel, d["Wg"], d["Wu"], d["Wd"], dY, f)
    Z = f64(to_host(o.Z[lo:hi]))
    assert_close("G", Z[:, :F], f["G"], tol)
    assert_close("U", Z[:, F:], f["U"], tol)
    assert_close("H", f64(to_host(o.H[lo:hi])), f["H"], tol)
    assert_close("Y", f64(to_host(o.Y[lo:hi])), f["Y"], tol)
    assert_close("dX", f64(to_host(o.dX[lo:hi])), b["dX"], tol)
    for k in ("dWg", "dWu", "dWd"):
        g = to_host(getattr(o, k))
        for e in range(E):
            assert_close(f"{k}[{e}]", g[e], b[k][e], tol)   # empty experts: exact zeros
    for t in (o.Z, o.H, o.Y, o.dX):
        bits = t.view(torch.int16)
        assert bool((bits[:lo] == SENTINEL).all()) and bool((bits[hi:] == SENTINEL).all())


SPLITS = [
    # (counts, H, F): k extents off the 64- and 32-wide tiles (the general
    # kernel), whole 64-wide tiles (the hand-ordered kernel), empty experts
    # first, inside and last, remainders 1 .. 255 rows past a tile row
    ([37, 0, 300, 5], 264, 136),
    ([0, 257, 576, 3, 0, 289, 200, 321, 0], 512, 192),
    ([1, 1, 1, 1, 1, 1, 1, 1], 64, 64),
    ([0, 0, 700], 128, 96),
]


@pytest.mark.parametrize("counts,H,F", SPLITS)
def test_ragged_splits_whole_tensors(counts, H, F):
    d = _inputs(counts, H, F)
    _, o = _run(d, H, F, _device_offsets(counts))
    _check_oracle(d, d["offsets"], o, H, F)


def test_rows_past_the_last_offset_are_left_alone():
    """R = 900 rows of buffer, 611 routed: rows 611.. keep their contents."""
    counts, H, F = [300, 0, 311], 256, 128
    d = _inputs(counts, H, F, R=900)
    _, o = _run(d, H, F, _device_offsets(counts))
    _check_oracle(d, d["offsets"], o, H, F)


def test_capacity_far_above_the_routed_rows():
    """A buffer of 20000 rows with 851 routed (the grid has ~25 times the
    tiles needed): the routed rows against the oracle, the rest untouched."""
    counts, H, F = [300, 0, 511, 40], 256, 128
    d = _inputs(counts, H, F, R=20000)
    _, o = _run(d, H, F, _device_offsets(counts))
    _check_oracle(d, d["offsets"], o, H, F)


def test_half_height_tiles_decided_on_the_device():
    """Few rows per expert: the 128-row tiles take fewer tile-area waves,
    which the kernels decide from the device offsets as the host does from
    host ones, so the same kernels run the same sums: every output equals
    the host-offset call's bit for bit, and the oracle's to the bar."""
    counts, H, F = [100, 60, 0, 200, 30], 512, 256
    d = _inputs(counts, H, F, seed=87)
    dev, o = _run(d, H, F, _device_offsets(counts))
    off = d["offsets"]
    desc = dict(H=H, F=F, E=len(counts), dtype=wl.DT_BF16)
    ref = ExpertBuffers(desc, off)
    print("[gpu] host-offset grouped fwd+bwd", flush=True)
    tp.tp_grouped_expert_fwd(desc, off, dev["X_perm"], dev["Wg"], dev["Wu"], dev["Wd"],
                             ref.Z, ref.H, ref.Y)
    tp.tp_grouped_expert_bwd(desc, off, dev["X_perm"], dev["Wg"], dev["Wu"], dev["Wd"],
                             ref.Z, ref.H, dev["dY_perm"], ref.dX, ref.dWg, ref.dWu, ref.dWd,
                             ref.ws, ref.ws_bytes)
    torch.cuda.synchronize()
    for k in ("Z", "H", "Y", "dX", "dWg", "dWu", "dWd"):
        assert torch.equal(getattr(o, k), getattr(ref, k)), k
    _check_oracle(d, off, o, H, F)


def test_thin_remainder_tiles_decided_on_the_device():
    """Rows ending 33, 64, 3 and 1 rows past a multiple of 256 at H = F =
    4096: the 256-row tiles fill whole waves only if those remainders go to
    the 32-row tiles, which the kernels decide from the device offsets as
    the host does from host ones.  The same kernels then run the same sums:
    every output equals the host-offset call's bit for bit; the remainder
    rows and 16 more per expert against the oracle."""
    counts = [1024 + 33, 0, 2048 + 64, 3, 1024 + 1, 0]
    H = F = 4096
    d = _inputs(counts, H, F, seed=86)
    dev, o = _run(d, H, F, _device_offsets(counts), out=None)
    off = d["offsets"]
    E = len(counts)
    desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
    ref = ExpertBuffers(desc, off)
    print("[gpu] host-offset grouped fwd+bwd", flush=True)
    tp.tp_grouped_expert_fwd(desc, off, dev["X_perm"], dev["Wg"], dev["Wu"], dev["Wd"],
                             ref.Z, ref.H, ref.Y)
    tp.tp_grouped_expert_bwd(desc, off, dev["X_perm"], dev["Wg"], dev["Wu"], dev["Wd"],
                             ref.Z, ref.H, dev["dY_perm"], ref.dX, ref.dWg, ref.dWu, ref.dWd,
                             ref.ws, ref.ws_bytes)
    torch.cuda.synchronize()
    for k in ("Z", "H", "Y", "dX", "dWg", "dWu", "dWd"):
        assert torch.equal(getattr(o, k), getattr(ref, k)), k
    rows, sub = [], [0]
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        tail = lo + ((hi - lo) // 256) * 256
        r = np.union1d(np.arange(tail, hi), lo + sample_idx(hi - lo, 16)) if hi > lo else []
        rows.extend(list(r))
        sub.append(sub[-1] + len(r))
    rows = np.array(rows, dtype=np.int64)
    f = oracle.grouped_fwd(d["X_perm"][rows], sub, d["Wg"], d["Wu"], d["Wd"])
    b = oracle.grouped_bwd(d["X_perm"][rows], sub, d["Wg"], d["Wu"], d["Wd"],
                           d["dY_perm"][rows], f)
    tol = TOL[wl.DT_BF16]
    assert_close("Y rows", f64(to_host(o.Y[rows])), f["Y"], tol)
    assert_close("H rows", f64(to_host(o.H[rows])), f["H"], tol)
    assert_close("dX rows", f64(to_host(o.dX[rows])), b["dX"], tol)


@pytest.mark.parametrize("vals", [
    [5, 80, 30, 250, 7],          # first offset past 0, out of order, past R
    [-40, 100, 100, 90, -3],      # negative, equal, decreasing
    [0, 2 ** 31 - 1, 0, 0, 0],    # the largest int32
])
def test_out_of_range_offsets_are_taken_clamped(vals):
    H, F, R = 128, 64, 200
    d = _inputs([R], H, F, R=R)
    d["Wg"] = wl.normal_bf16(91, (4, H, F), 0.05)
    d["Wu"] = wl.normal_bf16(92, (4, H, F), 0.05)
    d["Wd"] = wl.normal_bf16(93, (4, F, H), 0.05)
    off_dev = torch.tensor(vals, dtype=torch.int32, device="cuda")
    _, o = _run(d, H, F, off_dev)
    _check_oracle(d, _clamped(vals, R), o, H, F)


def test_looped_launches_on_a_large_buffer():
    """H = 4096 on a buffer of 20000 rows with 851 routed: the worst-case
    grids of FC2 and dX (82 tile rows x 16) exceed three waves, so they run
    as loops over their tiles on one workgroup per compute unit; whole
    tensors against the oracle, the unrouted rows untouched."""
    counts, H, F = [300, 0, 511, 40], 4096, 512
    d = _inputs(counts, H, F, R=20000, seed=89)
    _, o = _run(d, H, F, _device_offsets(counts))
    _check_oracle(d, d["offsets"], o, H, F)


def test_full_grouped_workload_on_capacity_buffers_bitwise():
    """The full grouped workload on buffers of tokens x top-k = 32768 rows
    (every row-ragged launch loops over its tiles): the offsets call for
    the tilings the host-offset call picks (256-row tiles for FC1, 32-row
    remainders for FC2 and dX, 128-row tiles for dH), and the looped
    kernels compute each tile as the others do, so every output equals the
    host-offset call's bit for bit."""
    w = wl.WORKLOADS["c5_bf16_grouped_swiglu"]
    g = wl.gen_grouped_inputs(w)
    H, F, E = w.H, w.F, w.experts
    off = g["offsets"]
    R = int(off[-1])
    cap = w.tokens * w.topk
    d = {k: g[k] for k in ("Wg", "Wu", "Wd")}
    d["R"] = cap
    for k in ("X_perm", "dY_perm"):
        full = np.zeros((cap, H), np.uint16)
        full[:R] = g[k]
        d[k] = full
    dev, o = _run(d, H, F, _device_offsets(np.diff(off)))
    desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
    ref = ExpertBuffers(desc, off)
    print("[gpu] host-offset grouped fwd+bwd", flush=True)
    Xp, dYp = dev["X_perm"][:R].contiguous(), dev["dY_perm"][:R].contiguous()
    tp.tp_grouped_expert_fwd(desc, off, Xp, dev["Wg"], dev["Wu"], dev["Wd"], ref.Z, ref.H, ref.Y)
    tp.tp_grouped_expert_bwd(desc, off, Xp, dev["Wg"], dev["Wu"], dev["Wd"], ref.Z, ref.H, dYp,
                             ref.dX, ref.dWg, ref.dWu, ref.dWd, ref.ws, ref.ws_bytes)
    torch.cuda.synchronize()
    for k in ("Z", "H", "Y", "dX"):
        assert torch.equal(getattr(o, k)[:R], getattr(ref, k)), k
        assert bool((getattr(o, k)[R:].view(torch.int16) == SENTINEL).all()), k
    for k in ("dWg", "dWu", "dWd"):
        assert torch.equal(getattr(o, k), getattr(ref, k)), k


def test_sixty_four_experts():
    """E = 64 (the most a call takes: every lane of the offset scan holds an
    expert, the last reading the table's 65th entry), a third of them
    empty: whole tensors against the oracle."""
    rng = np.random.default_rng(88)
    counts = [int(c) if rng.random() > 0.33 else 0 for c in rng.integers(1, 90, 64)]
    H, F = 64, 64
    d = _inputs(counts, H, F, seed=88)
    _, o = _run(d, H, F, _device_offsets(counts))
    _check_oracle(d, d["offsets"], o, H, F)


def test_no_rows():
    """R = 0: the forward writes nothing, the backward's weight gradients
    are sums over no rows (zeros; unchanged when accumulating).  The empty
    row buffers get distinct dummy addresses."""
    H, F, E = 64, 32, 3
    desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
    W = [torch.randn(s, device="cuda").to(torch.bfloat16) for s in ((E, H, F), (E, H, F), (E, F, H))]
    off_dev = torch.tensor([0, 7, 9, 400], dtype=torch.int32, device="cuda")   # clamped to 0
    e = torch.empty(16 * 16, dtype=torch.uint8, device="cuda")
    ptr = [e.data_ptr() + 16 * k for k in range(8)]
    print("[gpu] devoff R=0", flush=True)
    tp.tp_grouped_expert_fwd_devoff(desc, 0, off_dev, ptr[0], *W, ptr[1], ptr[2], ptr[3])
    for accumulate in (False, True):
        dW = [torch.full(s, 3.0, device="cuda") for s in ((E, H, F), (E, H, F), (E, F, H))]
        tp.tp_grouped_expert_bwd_devoff(desc, 0, off_dev, ptr[0], *W, ptr[1], ptr[2], ptr[4],
                                        ptr[5], *dW, None, 0, accumulate=accumulate)
        torch.cuda.synchronize()
        for t in dW:
            assert bool((t == (3.0 if accumulate else 0.0)).all())


def test_weight_gradients_accumulate():
    counts, H, F = [90, 0, 400, 13], 192, 128
    d = _inputs(counts, H, F)
    off_dev = _device_offsets(counts)
    E = len(counts)
    o = _Out(E, H, F, d["R"])
    base = [torch.randn(t.shape, device="cuda") for t in (o.dWg, o.dWu, o.dWd)]
    for t, b0 in zip((o.dWg, o.dWu, o.dWd), base):
        t.copy_(b0)
    _run(d, H, F, off_dev, accumulate=True, out=o)
    plain = _Out(E, H, F, d["R"])
    _run(d, H, F, off_dev, out=plain)
    for k, b0 in zip(("dWg", "dWu", "dWd"), base):
        # the same fp32 sums, then one fp32 addition on either side
        torch.testing.assert_close(getattr(o, k), b0 + getattr(plain, k), rtol=1e-6, atol=1e-6)


def test_full_grouped_workload_against_host_offsets():
    """The full grouped workload (4079 rows over 8 experts): every element
    against the host-offset call (summation order may differ: the host
    call can pick other tile shapes), sampled rows and columns against the
    oracle, bit-identical run to run."""
    w = wl.WORKLOADS["c5_bf16_grouped_swiglu"]
    d = wl.gen_grouped_inputs(w)
    H, F, E = w.H, w.F, w.experts
    off = d["offsets"]
    counts = np.diff(off)
    d["R"] = int(off[-1])
    off_dev = _device_offsets(counts)
    dev, o = _run(d, H, F, off_dev)
    _, o2 = _run(d, H, F, off_dev)
    for k in ("Z", "H", "Y", "dX", "dWg", "dWu", "dWd"):
        assert torch.equal(getattr(o, k), getattr(o2, k)), k
    desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
    ref = ExpertBuffers(desc, off)
    print("[gpu] host-offset grouped fwd+bwd", flush=True)
    tp.tp_grouped_expert_fwd(desc, off, dev["X_perm"], dev["Wg"], dev["Wu"], dev["Wd"],
                             ref.Z, ref.H, ref.Y)
    tp.tp_grouped_expert_bwd(desc, off, dev["X_perm"], dev["Wg"], dev["Wu"], dev["Wd"],
                             ref.Z, ref.H, dev["dY_perm"], ref.dX, ref.dWg, ref.dWu, ref.dWd,
                             ref.ws, ref.ws_bytes)
    torch.cuda.synchronize()
    tol = TOL[wl.DT_BF16]
    for k in ("Z", "H", "Y", "dX"):
        assert_close(f"{k} vs host offsets", f64(to_host(getattr(o, k))),
                     f64(to_host(getattr(ref, k))), tol)
    for k in ("dWg", "dWu", "dWd"):
        a, b = to_host(getattr(o, k)), to_host(getattr(ref, k))
        for e in range(E):
            assert_close(f"{k}[{e}] vs host offsets", a[e], b[e], tol)
    rows, sub = [], [0]
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        r = lo + sample_idx(hi - lo, 8)
        rows.extend(r.tolist())
        sub.append(sub[-1] + len(r))
    rows = np.array(rows)
    f = oracle.grouped_fwd(d["X_perm"][rows], sub, d["Wg"], d["Wu"], d["Wd"])
    b = oracle.grouped_bwd(d["X_perm"][rows], sub, d["Wg"], d["Wu"], d["Wd"],
                           d["dY_perm"][rows], f)
    assert_close("Y rows", f64(to_host(o.Y[rows])), f["Y"], tol)
    assert_close("dX rows", f64(to_host(o.dX[rows])), b["dX"], tol)
    cols = sample_idx(F, 16)
    Wg = np.ascontiguousarray(d["Wg"][:, :, cols])
    Wu = np.ascontiguousarray(d["Wu"][:, :, cols])
    Wd = np.ascontiguousarray(d["Wd"][:, cols, :])
    fn = oracle.grouped_fwd(d["X_perm"], off, Wg, Wu, Wd)
    bn = oracle.grouped_bwd(d["X_perm"], off, Wg, Wu, Wd, d["dY_perm"], fn)
    assert_close("dWg cols", to_host(o.dWg[:, :, cols]), bn["dWg"], tol)
    assert_close("dWu cols", to_host(o.dWu[:, :, cols]), bn["dWu"], tol)
    assert_close("dWd rows", to_host(o.dWd[:, cols, :]), bn["dWd"], tol)


def test_captured_graph_follows_offsets_changed_in_place():
    """Forward and backward captured once, replayed after the offsets tensor
    was rewritten in place (eager work and synchronization between replays):
    each replay equals the eager calls on those offsets, bit for bit."""
    H, F, R = 256, 128, 700
    splits = [[300, 0, 311, 89], [0, 700, 0, 0], [1, 2, 3, 600]]
    d = _inputs([R], H, F, R=R)
    E = len(splits[0])
    d["Wg"] = wl.normal_bf16(94, (E, H, F), 0.05)
    d["Wu"] = wl.normal_bf16(95, (E, H, F), 0.05)
    d["Wd"] = wl.normal_bf16(96, (E, F, H), 0.05)
    desc = dict(H=H, F=F, E=E, dtype=wl.DT_BF16)
    dev = {k: to_device(d[k]) for k in ("X_perm", "Wg", "Wu", "Wd", "dY_perm")}
    off_dev = _device_offsets(splits[0])
    g_out = _Out(E, H, F, R)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # one eager call on the capture stream first
        _run(d, H, F, off_dev, out=g_out)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    print("[gpu] devoff capture", flush=True)
    with torch.cuda.graph(graph):
        tp.tp_grouped_expert_fwd_devoff(desc, R, off_dev, dev["X_perm"], dev["Wg"], dev["Wu"],
                                        dev["Wd"], g_out.Z, g_out.H, g_out.Y)
        tp.tp_grouped_expert_bwd_devoff(desc, R, off_dev, dev["X_perm"], dev["Wg"], dev["Wu"],
                                        dev["Wd"], g_out.Z, g_out.H, dev["dY_perm"], g_out.dX,
                                        g_out.dWg, g_out.dWu, g_out.dWd, g_out.ws,
                                        g_out.ws_bytes)
    for counts in splits + splits[:1]:
        off_dev.copy_(_device_offsets(counts))
        for t in (g_out.Z, g_out.H, g_out.Y, g_out.dX):
            t.view(torch.int16).fill_(SENTINEL)
        print(f"[gpu] devoff replay counts={counts}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        eager_off = _device_offsets(counts)
        _, e_out = _run(d, H, F, eager_off)
        for k in ("Z", "H", "Y", "dX", "dWg", "dWu", "dWd"):
            a, b = getattr(g_out, k), getattr(e_out, k)
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (counts, k)
