"""Randomized-shape parity (GPU): a bounded, seeded sweep of small shard
and grouped-expert shapes against the fp64 oracle, whole tensors, at the
same bars as the fixed-shape parity tests.  Shapes include N = 1, H and
F/T that are not multiples of any tile (multiples of the vector width only:
8 for bf16, 4 for fp32), both activations, both storage types, and grouped
calls with empty experts.  hypothesis runs derandomized (the same examples
every run) and stops at the first failing example, which it shrinks.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import workloads as wl
from parity import TOL, assert_close, f64
from tensor_transformer_mlp_02_amd.tensors import to_host
from test_gpu_parity import _check_full, _grouped_inputs, _run_grouped, _run_shard

pytestmark = pytest.mark.gpu

SETTINGS = dict(deadline=None, derandomize=True, database=None, print_blob=True,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@st.composite
def shard_shapes(draw):
    dtype = draw(st.sampled_from([wl.DT_F32, wl.DT_BF16]))
    act = draw(st.sampled_from([wl.ACT_GELU_TANH, wl.ACT_SWIGLU]))
    vec = 8 if dtype == wl.DT_BF16 else 4
    N = draw(st.one_of(st.just(1), st.integers(1, 300)))
    H = vec * draw(st.integers(1, 520 // vec))
    Ft = vec * draw(st.integers(1, 600 // vec))
    return dtype, act, N, H, Ft


@settings(max_examples=24, **SETTINGS)
@given(shard_shapes())
def test_random_shard_shapes(shape):
    dtype, act, N, H, Ft = shape
    cid = 300 + (N * 7 + H * 13 + Ft * 17 + act) % 600
    w = wl.Workload(cid, "sweep", dtype, act, S=N, B=1, H=H, F=Ft, T=1,
                    w_std=0.5 / np.sqrt(H))
    d = wl.gen_mlp_inputs(w)
    print(f"[gpu] sweep shard dtype={dtype} act={act} N={N} H={H} Ft={Ft}", flush=True)
    _, buf = _run_shard(w, d)
    _check_full(w, d, buf)


@st.composite
def grouped_shapes(draw):
    E = draw(st.integers(1, 8))
    counts = draw(st.lists(st.one_of(st.just(0), st.integers(1, 300)), min_size=E, max_size=E))
    H = 8 * draw(st.integers(1, 40))
    F = 8 * draw(st.integers(1, 40))
    return counts, H, F


@settings(max_examples=10, **SETTINGS)
@given(grouped_shapes())
def test_random_grouped_shapes(shape):
    counts, H, F = shape
    if sum(counts) == 0:
        counts = counts[:-1] + [1]
    w, d = _grouped_inputs(counts, H, F, seed=400 + (sum(counts) + H + F) % 300)
    print(f"[gpu] sweep grouped counts={counts} H={H} F={F}", flush=True)
    _, buf = _run_grouped(d, H, F)
    f = oracle.grouped_fwd(d["X_perm"], d["offsets"], d["Wg"], d["Wu"], d["Wd"])
    b = oracle.grouped_bwd(d["X_perm"], d["offsets"], d["Wg"], d["Wu"], d["Wd"],
                           d["dY_perm"], f)
    tol = TOL[wl.DT_BF16]
    Z = f64(to_host(buf.Z))
    assert_close("G", Z[:, :F], f["G"], tol)
    assert_close("U", Z[:, F:], f["U"], tol)
    assert_close("H", f64(to_host(buf.H)), f["H"], tol)
    assert_close("Y", f64(to_host(buf.Y)), f["Y"], tol)
    assert_close("dX", f64(to_host(buf.dX)), b["dX"], tol)
    for k in ("dWg", "dWu", "dWd"):
        g = to_host(getattr(buf, k))
        for e in range(len(counts)):
            assert_close(f"{k}[{e}]", g[e], b[k][e], tol)


@settings(max_examples=12, **SETTINGS)
@given(shard_shapes())
def test_random_shard_shapes_derivative_in_loads(shape):
    """The backward that forms dZ in the dA / dX operand loads, on the same
    kind of shapes (k tiles that straddle the [dG | dU] split included)."""
    from test_gpu_dact import _run
    dtype, act, N, H, Ft = shape
    cid = 900 + (N * 5 + H * 11 + Ft * 3 + act) % 600
    w = wl.Workload(cid, "sweep", dtype, act, S=N, B=1, H=H, F=Ft, T=1,
                    w_std=0.5 / np.sqrt(H))
    d = wl.gen_mlp_inputs(w)
    print(f"[gpu] sweep dact dtype={dtype} act={act} N={N} H={H} Ft={Ft}", flush=True)
    _, _, _, pro = _run(w, d)
    f = oracle.mlp_fwd(d["X"], d["A"], d["B"], act, d["A_up"])
    b = oracle.mlp_bwd(d["X"], d["A"], d["B"], act, d["dY"], f, d["A_up"])
    tol = TOL[dtype]
    assert_close("dX", f64(to_host(pro.dX)), b["dX"], tol)
    assert_close("dA", to_host(pro.dA), b["dA"], tol)
    assert_close("dB", to_host(pro.dB), b["dB"], tol)
    if act == wl.ACT_SWIGLU:
        assert_close("dA_up", to_host(pro.dA_up), b["dA_up"], tol)


@st.composite
def grouped_shapes_with_capacity(draw):
    counts, H, F = draw(grouped_shapes())
    return counts, H, F, draw(st.one_of(st.just(0), st.integers(1, 600)))


@settings(max_examples=10, **SETTINGS)
@given(grouped_shapes_with_capacity())
def test_random_grouped_shapes_device_offsets(shape):
    """The device-offset grouped calls on the same kind of ragged splits,
    with buffers up to 600 rows larger than the routed rows: whole tensors
    against the oracle, the unrouted rows untouched."""
    from test_gpu_devoff import _check_oracle, _device_offsets, _inputs, _run
    counts, H, F, slack = shape
    if sum(counts) == 0:
        counts = counts[:-1] + [1]
    R = sum(counts) + slack
    d = _inputs(counts, H, F, R=R, seed=700 + (sum(counts) + H + F + slack) % 300)
    print(f"[gpu] sweep grouped device offsets counts={counts} H={H} F={F} R={R}", flush=True)
    _, o = _run(d, H, F, _device_offsets(counts))
    _check_oracle(d, d["offsets"], o, H, F)
