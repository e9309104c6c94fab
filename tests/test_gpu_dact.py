"""GPU parity of tp_mlp_shard_bwd_dact_prologue: the backward whose dA and
dX GEMMs form dZ from dH and the saved activations as they load it.

Its weight and input gradients are checked against the fp64 oracle's
backward of the same shard (whole tensors on small shapes with ragged
tails and at the full SwiGLU workload, sampled rows and columns at the full
SwiGLU and GeLU workloads),
dH (left in the workspace) against the oracle's dY B^T, and every result
against the default backward's (the derivative in the epilogue), to the
same bar: the two differ only in rounding (dZ is formed from the stored
bf16 dH here, from dH's fp32 sums there).
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_02_amd as tp
import workloads as wl
from tensor_transformer_mlp_02_amd.tensors import to_device, to_host, ShardBuffers
from parity import TOL, assert_close, f64, sample_idx

pytestmark = pytest.mark.gpu


def _desc(w, N):
    return dict(S=N, B=1, H=w.H, F_shard=w.Ft, T=w.T, act=w.act, dtype=w.dtype)


def _run(w, d):
    """Forward, then both backwards into separate buffers."""
    N = d["X"].shape[0]
    desc = _desc(w, N)
    dev = {k: (to_device(d[k]) if d.get(k) is not None else None)
           for k in ("X", "A", "A_up", "B", "dY")}
    ref = ShardBuffers(desc)
    pro = ShardBuffers(desc)
    print(f"[gpu] dact fwd {desc}", flush=True)
    tp.tp_mlp_shard_fwd(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], ref.Z, ref.H, ref.Y)
    print(f"[gpu] dact bwd (epilogue) {desc}", flush=True)
    tp.tp_mlp_shard_bwd(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], ref.Z, ref.H, dev["dY"],
                        ref.dX, ref.dA, ref.dA_up, ref.dB, ref.ws, ref.ws_bytes)
    for t in (pro.dX, pro.dA, pro.dB) + ((pro.dA_up,) if pro.dA_up is not None else ()):
        t.view(torch.uint8).fill_(0xff)  # NaN / -NaN bit patterns: every element must be written
    print(f"[gpu] dact bwd (loads) {desc}", flush=True)
    tp.tp_mlp_shard_bwd_dact_prologue(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], ref.Z,
                                      ref.H, dev["dY"], pro.dX, pro.dA, pro.dA_up, pro.dB,
                                      pro.ws, pro.ws_bytes)
    torch.cuda.synchronize()
    return desc, dev, ref, pro


def _dh(buf, w, N, rows=None):
    dt = torch.bfloat16 if w.dtype == wl.DT_BF16 else torch.float32
    n = N * w.Ft * (2 if dt == torch.bfloat16 else 4)
    h = buf.ws[:n].view(dt).reshape(N, w.Ft)
    return f64(to_host(h if rows is None else h[rows]))


def _against_default(w, ref, pro, tol):
    assert_close("dX vs default", f64(to_host(pro.dX)), f64(to_host(ref.dX)), tol)
    assert_close("dA vs default", to_host(pro.dA), to_host(ref.dA), tol)
    assert_close("dB vs default", to_host(pro.dB), to_host(ref.dB), tol)
    if w.act == wl.ACT_SWIGLU:
        assert_close("dA_up vs default", to_host(pro.dA_up), to_host(ref.dA_up), tol)


SMALL = [
    # (dtype, act, N, H, Ft): several 256-wide tiles with ragged tails
    (wl.DT_BF16, wl.ACT_GELU_TANH, 300, 520, 392),
    (wl.DT_BF16, wl.ACT_SWIGLU, 300, 520, 392),
    (wl.DT_BF16, wl.ACT_SWIGLU, 513, 264, 136),
    # a [dG | dU] split that is not a multiple of 64 (k tiles of dX straddle
    # it; the weights go through registers too) nor of 256 (dA's tiles too)
    (wl.DT_BF16, wl.ACT_SWIGLU, 300, 544, 416),
    (wl.DT_BF16, wl.ACT_SWIGLU, 1, 8, 8),
    (wl.DT_BF16, wl.ACT_GELU_TANH, 77, 8, 600),
    (wl.DT_F32, wl.ACT_GELU_TANH, 300, 132, 100),
    (wl.DT_F32, wl.ACT_SWIGLU, 70, 68, 36),
]


@pytest.mark.parametrize("dtype,act,N,H,Ft", SMALL)
def test_small_shapes_whole_tensors(dtype, act, N, H, Ft):
    w = wl.Workload(90 + SMALL.index((dtype, act, N, H, Ft)), "dact", dtype, act,
                    S=N, B=1, H=H, F=Ft, T=1, w_std=0.05)
    d = wl.gen_mlp_inputs(w)
    desc, dev, ref, pro = _run(w, d)
    tol = TOL[dtype]
    f = oracle.mlp_fwd(d["X"], d["A"], d["B"], act, d["A_up"])
    b = oracle.mlp_bwd(d["X"], d["A"], d["B"], act, d["dY"], f, d["A_up"])
    assert_close("dH (workspace)", _dh(pro, w, N), oracle.matmul("nt", f64(d["dY"]), f64(d["B"])),
                 tol)
    assert_close("dX", f64(to_host(pro.dX)), b["dX"], tol)
    assert_close("dA", to_host(pro.dA), b["dA"], tol)
    assert_close("dB", to_host(pro.dB), b["dB"], tol)
    if act == wl.ACT_SWIGLU:
        assert_close("dA_up", to_host(pro.dA_up), b["dA_up"], tol)
    _against_default(w, ref, pro, tol)


@pytest.mark.parametrize("name", ["c3_bf16_gelu_fwdbwd", "c4_bf16_swiglu_fwdbwd"])
def test_full_size_sampled(name, n_rows=128, n_cols=64):
    w = wl.WORKLOADS[name]
    d = wl.gen_mlp_inputs(w)
    desc, dev, ref, pro = _run(w, d)
    tol = TOL[w.dtype]
    rows = sample_idx(w.N, n_rows)
    sub = {k: (d[k][rows] if k in ("X", "dY") else d[k]) for k in d}
    f = oracle.mlp_fwd(sub["X"], d["A"], d["B"], w.act, d["A_up"])
    b = oracle.mlp_bwd(sub["X"], d["A"], d["B"], w.act, sub["dY"], f, d["A_up"])
    assert_close("dH rows", _dh(pro, w, w.N, rows),
                 oracle.matmul("nt", f64(sub["dY"]), f64(d["B"])), tol)
    assert_close("dX rows", f64(to_host(pro.dX[rows])), b["dX"], tol)
    # weight gradients: the shard narrowed to sampled columns, all tokens
    cols = sample_idx(w.Ft, n_cols)
    An = np.ascontiguousarray(d["A"][:, cols]); Bn = np.ascontiguousarray(d["B"][cols, :])
    Aun = np.ascontiguousarray(d["A_up"][:, cols]) if d["A_up"] is not None else None
    fn = oracle.mlp_fwd(d["X"], An, Bn, w.act, Aun)
    bn = oracle.mlp_bwd(d["X"], An, Bn, w.act, d["dY"], fn, Aun)
    assert_close("dA cols", to_host(pro.dA[:, cols]), bn["dA"], tol)
    assert_close("dB rows", to_host(pro.dB[cols, :]), bn["dB"], tol)
    if w.act == wl.ACT_SWIGLU:
        assert_close("dA_up cols", to_host(pro.dA_up[:, cols]), bn["dA_up"], tol)
    _against_default(w, ref, pro, tol)


def test_run_to_run_bitwise():
    w = wl.Workload(99, "dact", wl.DT_BF16, wl.ACT_SWIGLU, S=700, B=1, H=520, F=392, T=1,
                    w_std=0.05)
    d = wl.gen_mlp_inputs(w)
    _, _, _, p1 = _run(w, d)
    _, _, _, p2 = _run(w, d)
    for a, b in ((p1.dX, p2.dX), (p1.dA, p2.dA), (p1.dA_up, p2.dA_up), (p1.dB, p2.dB)):
        assert torch.equal(a, b)


def test_empty_batch():
    """N = 0: no dH or dX; the weight gradients are sums over no tokens."""
    for dt, act in ((wl.DT_BF16, wl.ACT_SWIGLU), (wl.DT_F32, wl.ACT_GELU_TANH)):
        H, Ft = 64, 32
        desc = dict(S=0, B=4, H=H, F_shard=Ft, T=1, act=act, dtype=dt)
        tdt = torch.bfloat16 if dt == wl.DT_BF16 else torch.float32
        A = torch.randn((H, Ft), device="cuda").to(tdt)
        Au = torch.randn((H, Ft), device="cuda").to(tdt) if act == wl.ACT_SWIGLU else None
        B = torch.randn((Ft, H), device="cuda").to(tdt)
        buf = ShardBuffers(desc)
        buf.dA.fill_(float("nan")); buf.dB.fill_(float("nan"))
        if buf.dA_up is not None:
            buf.dA_up.fill_(float("nan"))
        e = torch.empty(64 * 16, dtype=torch.uint8, device="cuda")
        ptr = [e.data_ptr() + 16 * k for k in range(8)]
        print(f"[gpu] dact bwd empty {desc}", flush=True)
        tp.tp_mlp_shard_bwd_dact_prologue(desc, ptr[0], A, Au, B, ptr[1], ptr[2], ptr[4],
                                          ptr[5], buf.dA, buf.dA_up, buf.dB, None, 0)
        torch.cuda.synchronize()
        assert torch.count_nonzero(buf.dA).item() == 0 and not torch.isnan(buf.dA).any()
        assert torch.count_nonzero(buf.dB).item() == 0 and not torch.isnan(buf.dB).any()
        if buf.dA_up is not None:
            assert torch.count_nonzero(buf.dA_up).item() == 0


def test_swiglu_full_size_whole_tensors():
    """Every element of dX, dA, dA_up, dB and dH at the full SwiGLU shard."""
    w = wl.WORKLOADS["c4_bf16_swiglu_fwdbwd"]
    d = wl.gen_mlp_inputs(w)
    desc, dev, ref, pro = _run(w, d)
    tol = TOL[w.dtype]
    f = oracle.mlp_fwd(d["X"], d["A"], d["B"], w.act, d["A_up"])
    b = oracle.mlp_bwd(d["X"], d["A"], d["B"], w.act, d["dY"], f, d["A_up"])
    assert_close("dH (workspace)", _dh(pro, w, w.N),
                 oracle.matmul("nt", f64(d["dY"]), f64(d["B"])), tol)
    assert_close("dX", f64(to_host(pro.dX)), b["dX"], tol)
    assert_close("dA", to_host(pro.dA), b["dA"], tol)
    assert_close("dA_up", to_host(pro.dA_up), b["dA_up"], tol)
    assert_close("dB", to_host(pro.dB), b["dB"], tol)
