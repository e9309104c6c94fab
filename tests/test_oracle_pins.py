"""Pins of the fp64 oracle against facts that do not come from the oracle.

The pages print no worked numeric example, so the oracle is pinned by
closed forms, the sharding algebra the pages state, central finite
differences of the scalar loss <dY, Y>, a library matmul, and exact
power-of-two scaling.  Each test names the mistake it would catch.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import ACT_GELU_TANH, ACT_SWIGLU

RNG = np.random.default_rng(12345)


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ----------------------------------------------------------------------------
# activations: closed forms
# ----------------------------------------------------------------------------
GRID = np.linspace(-8.0, 8.0, 3201)


def test_gelu_closed_forms():
    assert oracle.gelu_tanh(0.0) == 0.0
    # gelu(z) - gelu(-z) = z for the tanh form (tanh is odd): catches a
    # dropped 1/2 or a sign error inside the tanh argument.
    for z in GRID:
        assert abs(oracle.gelu_tanh(z) - oracle.gelu_tanh(-z) - z) <= 1e-14 * max(1.0, abs(z))
    # derivative at 0 is exactly 1/2
    assert oracle.gelu_tanh_grad(0.0) == 0.5
    # second-order coefficient: (gelu(z) + gelu(-z)) / (2 z^2) -> phi(0) =
    # 1/sqrt(2 pi), the Gaussian density at 0 (the tanh form matches the
    # exact GeLU to second order).  Catches a wrong sqrt(2/pi).
    z = 1e-4
    even = (oracle.gelu_tanh(z) + oracle.gelu_tanh(-z)) / (2 * z * z)
    assert abs(even - 1.0 / math.sqrt(2 * math.pi)) < 1e-7
    # distance to the exact x*Phi(x) (Python's math.erf, independent of the
    # oracle) stays within the tanh approximation's known error.
    dev = max(abs(oracle.gelu_tanh(z) - z * 0.5 * (1 + math.erf(z / math.sqrt(2))))
              for z in GRID)
    assert dev < 4.8e-4
    # asymptotes
    assert abs(oracle.gelu_tanh(30.0) - 30.0) < 1e-12
    assert abs(oracle.gelu_tanh(-30.0)) < 1e-12


def test_gelu_grad_matches_central_difference():
    for z in GRID:
        h = 1e-5
        fd = (oracle.gelu_tanh(z + h) - oracle.gelu_tanh(z - h)) / (2 * h)
        assert abs(fd - oracle.gelu_tanh_grad(z)) < 1e-9


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.silu_grad(0.0) == 0.5
    for z in GRID:
        # silu(z) - silu(-z) = z (since sigmoid(z) + sigmoid(-z) = 1)
        assert abs(oracle.silu(z) - oracle.silu(-z) - z) <= 1e-14 * max(1.0, abs(z))
        assert abs(oracle.sigmoid(z) - 1.0 / (1.0 + math.exp(-z))) < 1e-15
        h = 1e-5
        fd = (oracle.silu(z + h) - oracle.silu(z - h)) / (2 * h)
        assert abs(fd - oracle.silu_grad(z)) < 1e-9
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12


# ----------------------------------------------------------------------------
# product loops against a library matmul
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (17, 9, 33), (64, 48, 40)])
def test_matmul_loops_vs_numpy(shape):
    M, N, K = shape
    A = RNG.standard_normal((M, K)); B = RNG.standard_normal((K, N))
    assert rel(oracle.matmul("nn", A, B), A @ B) < 1e-13
    Bs = RNG.standard_normal((N, K))
    assert rel(oracle.matmul("nt", A, Bs), A @ Bs.T) < 1e-13
    As = RNG.standard_normal((K, M))
    assert rel(oracle.matmul("tn", As, B), As.T @ B) < 1e-13


def test_identity_activation_mlp_vs_numpy():
    """With act = identity the MLP is linear: Y = X A B, dX = dY B^T A^T,
    dA = X^T dY B^T, dB = (X A)^T dY.  Catches a transposed operand or a
    swapped gradient anywhere in the shard's loops."""
    N, H, Ft = 13, 24, 40
    X = RNG.standard_normal((N, H)); A = RNG.standard_normal((H, Ft))
    B = RNG.standard_normal((Ft, H)); dY = RNG.standard_normal((N, H))
    f = oracle.mlp_fwd(X, A, B, oracle.ACT_IDENTITY)
    assert rel(f["Y"], X @ A @ B) < 1e-13
    b = oracle.mlp_bwd(X, A, B, oracle.ACT_IDENTITY, dY, f)
    assert rel(b["dX"], dY @ B.T @ A.T) < 1e-13
    assert rel(b["dA"], X.T @ (dY @ B.T)) < 1e-13
    assert rel(b["dB"], (X @ A).T @ dY) < 1e-13


# ----------------------------------------------------------------------------
# finite differences of L = <dY, Y> on tiny shapes, every entry
# ----------------------------------------------------------------------------
def _loss(X, A, B, act, dY, Au=None):
    return float(np.sum(oracle.mlp_fwd(X, A, B, act, Au)["Y"] * dY))


def _fd_grad(fn, theta, idxs=None):
    g = np.zeros_like(theta)
    it = np.ndindex(theta.shape) if idxs is None else idxs
    for ix in it:
        old = theta[ix]
        h = 1e-6 * max(1.0, abs(old))
        theta[ix] = old + h; lp = fn()
        theta[ix] = old - h; lm = fn()
        theta[ix] = old
        g[ix] = (lp - lm) / (2 * h)
    return g


@pytest.mark.parametrize("act", [ACT_GELU_TANH, ACT_SWIGLU])
def test_finite_differences_tiny_every_entry(act):
    N, H, F, T = 4, 8, 16, 2
    X = RNG.standard_normal((N, H))
    A = RNG.standard_normal((H, F)) * 0.5
    Au = RNG.standard_normal((H, F)) * 0.5 if act == ACT_SWIGLU else None
    B = RNG.standard_normal((F, H)) * 0.5
    dY = RNG.standard_normal((N, H))
    res = oracle.sharded_fwd_bwd(X, A, B, T, act, dY, Au)
    Ft = F // T
    for i, rec in enumerate(res["shards"]):
        sl = slice(i * Ft, (i + 1) * Ft)
        Ai = np.ascontiguousarray(A[:, sl]); Bi = np.ascontiguousarray(B[sl, :])
        Aui = None if Au is None else np.ascontiguousarray(Au[:, sl])
        fn = lambda: _loss(X, Ai, Bi, act, dY, Aui)
        b = rec["bwd"]
        for theta, an in ((X, b["dX"]), (Ai, b["dA"]), (Bi, b["dB"])) + \
                (((Aui, b["dA_up"]),) if Aui is not None else ()):
            fd = _fd_grad(fn, theta)
            assert rel(an, fd) < 1e-7
            assert np.max(np.abs(an - fd)) < 1e-6 * max(1.0, np.max(np.abs(fd)))
    # the input gradient of the unsharded MLP equals the sum of shard partials
    fn_full = lambda: _loss(X, A, B, act, dY, Au)
    fd_full = _fd_grad(fn_full, X)
    assert rel(res["dX"], fd_full) < 1e-7


def test_finite_differences_sampled_small_workload():
    """256 sampled entries per tensor at the fp32 workload's full size."""
    import workloads
    w = workloads.WORKLOADS["c1_f32_gelu_t2"]
    d = workloads.gen_mlp_inputs(w, shard=1)
    X, A, B, dY = (oracle.to_f64(d[k]) for k in ("X", "A", "B", "dY"))
    f = oracle.mlp_fwd(X, A, B, ACT_GELU_TANH)
    b = oracle.mlp_bwd(X, A, B, ACT_GELU_TANH, dY, f)
    fn = lambda: _loss(X, A, B, ACT_GELU_TANH, dY)
    rng = np.random.default_rng(7)
    for theta, an in ((X, b["dX"]), (A, b["dA"]), (B, b["dB"])):
        flat = rng.choice(theta.size, size=256, replace=False)
        idxs = [np.unravel_index(int(k), theta.shape) for k in flat]
        fd = _fd_grad(fn, theta, idxs)
        sel = tuple(np.array(idxs).T)
        scale = np.max(np.abs(an))
        assert np.max(np.abs(fd[sel] - an[sel])) < 1e-6 * scale


# ----------------------------------------------------------------------------
# sharding algebra the pages state
# ----------------------------------------------------------------------------
@pytest.fixture(scope="module")
def c1_sharded():
    import workloads
    w = workloads.WORKLOADS["c1_f32_gelu_t2"]
    d = workloads.gen_mlp_inputs(w)
    res = oracle.sharded_fwd_bwd(d["X"], d["A_full"], d["B_full"], w.T, w.act, d["dY"])
    return w, d, res


def test_column_shards_concatenate_bitwise(c1_sharded):
    """§三 3.1: each column shard computes its own block of output columns."""
    w, d, res = c1_sharded
    Zcat = np.concatenate([r["fwd"]["Z"] for r in res["shards"]], axis=1)
    Hcat = np.concatenate([r["fwd"]["H"] for r in res["shards"]], axis=1)
    assert np.array_equal(Zcat, res["full_fwd"]["Z"])
    assert np.array_equal(Hcat, res["full_fwd"]["H"])


def test_row_partials_sum_to_unsharded(c1_sharded):
    """§三 3.2/3.3: the sum over shards of Y_i is the unsharded output."""
    w, d, res = c1_sharded
    assert rel(res["Y"], res["full_fwd"]["Y"]) < 1e-12
    # and a single partial is not the full output (catches a sum that
    # double-counts or a shard that silently used the full weights)
    assert rel(res["shards"][0]["fwd"]["Y"], res["full_fwd"]["Y"]) > 0.1


def test_dx_partials_sum_to_unsharded(c1_sharded):
    """§三 3.1: dL/dX = sum_i dL/dZ_i A_i^T (the backward all-reduce)."""
    w, d, res = c1_sharded
    assert rel(res["dX"], res["full_bwd"]["dX"]) < 1e-12


def test_weight_grads_are_slices_bitwise(c1_sharded):
    w, d, res = c1_sharded
    Ft = w.Ft
    for i, rec in enumerate(res["shards"]):
        sl = slice(i * Ft, (i + 1) * Ft)
        assert np.array_equal(rec["bwd"]["dA"], res["full_bwd"]["dA"][:, sl])
        assert np.array_equal(rec["bwd"]["dB"], res["full_bwd"]["dB"][sl, :])


def test_indivisible_width_rejected():
    A = np.zeros((4, 10)); B = np.zeros((10, 4))
    with pytest.raises(ValueError):
        oracle.shard_weights(A, B, 3)


@pytest.mark.parametrize("act", [ACT_GELU_TANH, ACT_SWIGLU])
def test_weight_grads_add_over_microbatches(act):
    """Gradient accumulation ([P1] §五 5.2): the weight gradients of a batch
    split into microbatches (rows), added up, are the whole batch's weight
    gradients, because each is a sum over rows; dX of each microbatch is the
    matching rows of the whole batch's dX.  Checked against numpy on the
    whole batch (an accumulation that overwrote, or summed the wrong rows,
    fails)."""
    rng = np.random.default_rng(11)
    N, H, F = 23, 12, 16
    X = rng.standard_normal((N, H)); dY = rng.standard_normal((N, H))
    A = rng.standard_normal((H, F)) * 0.3; B = rng.standard_normal((F, H)) * 0.3
    Au = rng.standard_normal((H, F)) * 0.3 if act == ACT_SWIGLU else None
    whole = oracle.mlp_bwd(X, A, B, act, dY, oracle.mlp_fwd(X, A, B, act, Au), Au)
    acc = {k: np.zeros_like(whole[k]) for k in ("dA", "dB")}
    if act == ACT_SWIGLU:
        acc["dA_up"] = np.zeros_like(whole["dA_up"])
    for lo, hi in ((0, 5), (5, 17), (17, 23)):
        f = oracle.mlp_fwd(X[lo:hi], A, B, act, Au)
        g = oracle.mlp_bwd(X[lo:hi], A, B, act, dY[lo:hi], f, Au)
        for k in acc:
            acc[k] += g[k]
        assert rel(g["dX"], whole["dX"][lo:hi]) < 1e-13
    for k in acc:
        assert rel(acc[k], whole[k]) < 1e-13
    # and the whole-batch dB is numpy's H^T dY
    Hh = oracle.mlp_fwd(X, A, B, act, Au)["H"]
    assert rel(whole["dB"], Hh.T @ dY) < 1e-13


def test_t1_shard_is_full_mlp_bitwise():
    N, H, F = 6, 16, 24
    X = RNG.standard_normal((N, H)); A = RNG.standard_normal((H, F)) * 0.3
    B = RNG.standard_normal((F, H)) * 0.3; dY = RNG.standard_normal((N, H))
    res = oracle.sharded_fwd_bwd(X, A, B, 1, ACT_GELU_TANH, dY)
    assert np.array_equal(res["Y"], res["full_fwd"]["Y"])
    assert np.array_equal(res["dX"], res["full_bwd"]["dX"])


@pytest.mark.parametrize("act", [ACT_GELU_TANH, ACT_SWIGLU])
def test_power_of_two_scaling_exact(act):
    """dY -> 2 dY doubles every gradient; B -> 2 B doubles Y: both exact in
    binary floating point, so any data-dependent slip shows bitwise."""
    N, H, Ft = 9, 16, 24
    X = RNG.standard_normal((N, H)); A = RNG.standard_normal((H, Ft)) * 0.3
    Au = RNG.standard_normal((H, Ft)) * 0.3 if act == ACT_SWIGLU else None
    B = RNG.standard_normal((Ft, H)) * 0.3; dY = RNG.standard_normal((N, H))
    f = oracle.mlp_fwd(X, A, B, act, Au)
    b1 = oracle.mlp_bwd(X, A, B, act, dY, f, Au)
    b2 = oracle.mlp_bwd(X, A, B, act, 2 * dY, f, Au)
    for k in ("dX", "dA", "dB") + (("dA_up",) if Au is not None else ()):
        assert np.array_equal(b2[k], 2 * b1[k])
    f2 = oracle.mlp_fwd(X, A, 2 * B, act, Au)
    assert np.array_equal(f2["Y"], 2 * f["Y"])


def test_swiglu_matches_gate_up_definition():
    """SwiGLU with the up projection replaced by a copy of the gate's
    weights is silu(z) * z; and with up weights zero the output is zero."""
    N, H, Ft = 5, 8, 12
    X = RNG.standard_normal((N, H)); A = RNG.standard_normal((H, Ft))
    B = RNG.standard_normal((Ft, H))
    f = oracle.mlp_fwd(X, A, B, ACT_SWIGLU, A.copy())
    Z = X @ A
    assert rel(f["H"], Z * Z / (1 + np.exp(-Z))) < 1e-14
    f0 = oracle.mlp_fwd(X, A, B, ACT_SWIGLU, np.zeros_like(A))
    assert not np.any(f0["Y"])


# ----------------------------------------------------------------------------
# partial sum
# ----------------------------------------------------------------------------
def test_partial_sum_pins():
    P = RNG.standard_normal((7, 5))
    assert np.array_equal(oracle.partial_sum([P]), P)
    # values with 8 significant bits: every running sum up to 8*P is exact
    P = np.ldexp(np.round(np.ldexp(P, 7)), -7)
    for T in (2, 4, 8):
        assert np.array_equal(oracle.partial_sum([P] * T), T * P)
    # integers: exact in fp64
    parts = [RNG.integers(-1000, 1000, size=(11,)).astype(np.float64) for _ in range(5)]
    assert np.array_equal(oracle.partial_sum(parts), np.sum(parts, axis=0))


def test_reduce_scatter_pins():
    """Sequence-parallel slices: the T ranks' slices, stacked in rank order
    along the sequence, are the full sum (numpy's, on integer data where
    fp64 is exact); rank r's slice holds sequence rows r*S/T onwards (a
    shifted index or a slice taken along B instead of S fails); T = 1 keeps
    everything; S must divide by T."""
    S, B, H, T = 12, 3, 8, 4
    parts = [RNG.integers(-500, 500, size=(S, B, H)).astype(np.float64) for _ in range(T)]
    full = np.sum(parts, axis=0)
    slices = [oracle.reduce_scatter(parts, S, B, H, r) for r in range(T)]
    assert all(sl.shape == (S // T, B, H) for sl in slices)
    assert np.array_equal(np.concatenate(slices, axis=0), full)
    # sequence row s of rank 2's slice is global row 2*S/T + s
    marker = [np.zeros((S, B, H)) for _ in range(T)]
    marker[1][7, 2, 5] = 1.0
    assert oracle.reduce_scatter(marker, S, B, H, 2)[1, 2, 5] == 1.0
    assert not np.any(oracle.reduce_scatter(marker, S, B, H, 1))
    assert np.array_equal(oracle.reduce_scatter(parts[:1], S, B, H, 0), parts[0])
    with pytest.raises(ValueError):
        oracle.reduce_scatter(parts[:3] + parts[:2], S, B, H, 0)   # T = 5 does not divide 12


# ----------------------------------------------------------------------------
# grouped experts
# ----------------------------------------------------------------------------
def _small_grouped(counts, H=16, F=24, seed=3):
    rng = np.random.default_rng(seed)
    E = len(counts)
    offsets = np.zeros(E + 1, np.int64); offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    X = rng.standard_normal((R, H)); dY = rng.standard_normal((R, H))
    Wg = rng.standard_normal((E, H, F)) * 0.3
    Wu = rng.standard_normal((E, H, F)) * 0.3
    Wd = rng.standard_normal((E, F, H)) * 0.3
    return X, dY, offsets, Wg, Wu, Wd


def test_grouped_rows_match_dense_on_gathered_tokens():
    """Expert e's rows equal the dense SwiGLU MLP with expert e's weights run
    over all tokens and then gathered, with numpy doing the gather and the
    products (catches an offset or expert-index slip)."""
    import workloads
    w = workloads.WORKLOADS["c5_bf16_grouped_swiglu"]
    d = workloads.gen_grouped_inputs(w, tokens=256, H=16, F=24)
    n_tok = 256
    Xtok = oracle.to_f64(workloads.normal_bf16(1000 * w.cid + workloads.K_X, (n_tok, 16), 1.0))
    g = oracle.grouped_fwd(d["X_perm"], d["offsets"], d["Wg"], d["Wu"], d["Wd"])
    for e in range(w.experts):
        lo, hi = d["offsets"][e], d["offsets"][e + 1]
        Gd = Xtok @ oracle.to_f64(d["Wg"][e]); Ud = Xtok @ oracle.to_f64(d["Wu"][e])
        Hd = Gd / (1 + np.exp(-Gd)) * Ud
        Yd = Hd @ oracle.to_f64(d["Wd"][e])
        toks = d["token_ids"][lo:hi]
        assert rel(g["Y"][lo:hi], Yd[toks]) < 1e-12


def test_grouped_empty_expert_and_permutation():
    counts = [3, 0, 5, 2]
    X, dY, off, Wg, Wu, Wd = _small_grouped(counts)
    f = oracle.grouped_fwd(X, off, Wg, Wu, Wd)
    b = oracle.grouped_bwd(X, off, Wg, Wu, Wd, dY, f)
    assert not np.any(b["dWg"][1]) and not np.any(b["dWu"][1]) and not np.any(b["dWd"][1])
    # permuting rows inside a segment permutes the per-row outputs and
    # leaves the weight gradients unchanged up to summation order
    perm = np.arange(X.shape[0]); perm[3:8] = perm[3:8][::-1]
    f2 = oracle.grouped_fwd(X[perm], off, Wg, Wu, Wd)
    b2 = oracle.grouped_bwd(X[perm], off, Wg, Wu, Wd, dY[perm], f2)
    assert np.array_equal(f2["Y"], f["Y"][perm])
    assert np.array_equal(b2["dX"], b["dX"][perm])
    assert rel(b2["dWg"], b["dWg"]) < 1e-14
    assert rel(b2["dWd"], b["dWd"]) < 1e-14


def test_grouped_weight_grad_finite_difference():
    counts = [2, 3]
    X, dY, off, Wg, Wu, Wd = _small_grouped(counts, H=6, F=8)
    f = oracle.grouped_fwd(X, off, Wg, Wu, Wd)
    b = oracle.grouped_bwd(X, off, Wg, Wu, Wd, dY, f)
    fn = lambda: float(np.sum(oracle.grouped_fwd(X, off, Wg, Wu, Wd)["Y"] * dY))
    for theta, an in ((Wg, b["dWg"]), (Wu, b["dWu"]), (Wd, b["dWd"]), (X, b["dX"])):
        fd = _fd_grad(fn, theta)
        assert rel(an, fd) < 1e-7


# ----------------------------------------------------------------------------
# MoE dispatch and combine
# ----------------------------------------------------------------------------
def _moe_small(n_tok=40, H=16, F=24, seed=31):
    import workloads
    w = workloads.WORKLOADS["c5_bf16_grouped_swiglu"]
    d = workloads.gen_moe_inputs(w, tokens=n_tok, H=H, F=F)
    return w, d


def test_moe_layer_equals_per_token_expert_sum():
    """permute -> grouped experts -> weighted combine equals, token by token,
    the router-weighted sum of the dense SwiGLU MLPs of the experts the token
    picked (computed one token at a time), with zeros for tokens that picked
    no local expert."""
    w, d = _moe_small()
    Xp = oracle.moe_permute(d["X"], d["token_ids"])
    g = oracle.grouped_fwd(Xp, d["offsets"], d["Wg"], d["Wu"], d["Wd"])
    Y = oracle.moe_combine(g["Y"], d["token_ids"], d["X"].shape[0], d["row_weight"])
    X = oracle.to_f64(d["X"])
    off = d["offsets"]
    expect = np.zeros_like(Y)
    for e in range(len(off) - 1):
        for r in range(int(off[e]), int(off[e + 1])):
            t = int(d["token_ids"][r])
            f = oracle.mlp_fwd(X[t:t + 1], oracle.to_f64(d["Wg"][e]), oracle.to_f64(d["Wd"][e]),
                               ACT_SWIGLU, oracle.to_f64(d["Wu"][e]))
            expect[t] += float(d["row_weight"][r]) * f["Y"][0]
    assert rel(Y, expect) < 1e-13
    routed = np.zeros(X.shape[0], bool); routed[d["token_ids"]] = True
    assert not np.any(Y[~routed]) and routed.any() and (~routed).any()


def test_moe_permute_then_unweighted_combine_restores_tokens():
    w, d = _moe_small(seed=5)
    ids = d["token_ids"]
    # keep each token's first row only: the combine then gives the token back
    first = np.unique(ids, return_index=True)[1]
    X = oracle.to_f64(d["X"])
    Y = oracle.moe_combine(oracle.moe_permute(X, ids[first]), ids[first], X.shape[0])
    assert np.array_equal(Y[ids[first]], X[ids[first]])
    # with all rows: each token comes back times the number of its rows
    Y2 = oracle.moe_combine(oracle.moe_permute(X, ids), ids, X.shape[0])
    cnt = np.bincount(ids, minlength=X.shape[0]).astype(float)
    assert np.array_equal(Y2, cnt[:, None] * X)


def test_moe_combine_backward_by_finite_differences():
    """L = <dY, combine(Y_perm, w)> is linear in w and in Y_perm, so central
    differences are exact up to rounding: dL/dw[r] and dL/dY_perm[r, h] match
    the backward's d_weight and dY_perm."""
    rng = np.random.default_rng(2)
    n_tok, H = 9, 5
    ids = np.array([0, 3, 3, 7, 8, 1, 0, 7], np.int64)
    w = rng.random(len(ids))
    Yp = rng.standard_normal((len(ids), H))
    dY = rng.standard_normal((n_tok, H))
    L = lambda Yp_, w_: float(np.sum(dY * oracle.moe_combine(Yp_, ids, n_tok, w_)))
    dYp, dw = oracle.moe_combine_bwd(dY, Yp, ids, w)
    h = 1e-3
    for r in range(len(ids)):
        e = np.zeros_like(w); e[r] = h
        assert abs((L(Yp, w + e) - L(Yp, w - e)) / (2 * h) - dw[r]) < 1e-10
        for c in range(H):
            E = np.zeros_like(Yp); E[r, c] = h
            assert abs((L(Yp + E, w) - L(Yp - E, w)) / (2 * h) - dYp[r, c]) < 1e-10


def test_token_row_lists():
    """The per-token row lists invert the row -> token map: every row once,
    each token's rows ascending, and tok_ptr counts match."""
    import workloads
    w, d = _moe_small(n_tok=200)
    ids, ptr, rows = d["token_ids"], d["tok_ptr"], d["tok_rows"]
    assert ptr[0] == 0 and ptr[-1] == len(ids)
    assert np.array_equal(np.sort(rows), np.arange(len(ids)))
    for t in range(len(ptr) - 1):
        rs = rows[ptr[t]:ptr[t + 1]]
        assert np.all(ids[rs] == t) and np.all(np.diff(rs) > 0)
    assert np.all(d["row_weight"] > 0) and np.all(d["row_weight"] < 1)


# ----------------------------------------------------------------------------
# FP8 encoding
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("fmt,tdt", [("e4m3", "float8_e4m3fn"), ("e5m2", "float8_e5m2")])
def test_fp8_codes_round_trip_and_match_torch(fmt, tdt):
    """Every finite code decodes to a value that encodes back to the same
    code; decoding agrees with torch's float8 type on all of them; encoding
    agrees with torch's (round to nearest even) cast on random in-range
    values and on every midpoint between neighbouring codes."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ebits = 4 if fmt == "e4m3" else 5
    mbits = 7 - ebits
    emask = ((1 << ebits) - 1) << mbits
    finite = codes[((codes & emask) != emask) | ((fmt == "e4m3") & ((codes & 0x7f) != 0x7f))]
    vals = oracle.fp8_decode(finite, fmt)
    assert np.array_equal(oracle.fp8_encode(vals, fmt), finite)
    tv = torch.from_numpy(finite.copy()).view(getattr(torch, tdt)).to(torch.float64).numpy()
    assert np.array_equal(vals, tv)
    vmax = oracle.FP8_FORMATS[fmt][2]
    pos = np.sort(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(4)
    x = np.concatenate([mids, -mids, rng.uniform(-vmax, vmax, 20000),
                        rng.standard_normal(20000) * 1e-3]).astype(np.float32)
    want = torch.from_numpy(x).to(getattr(torch, tdt)).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_encode(x, fmt), want)


def test_fp8_saturation_and_signed_zero():
    assert oracle.fp8_encode(np.array([448.0, 449.0, 500.0, 1e9]), "e4m3").tolist() == [0x7e] * 4
    assert oracle.fp8_encode(np.array([-1e9]), "e4m3")[0] == 0xfe
    assert oracle.fp8_encode(np.array([57344.0, 1e9]), "e5m2").tolist() == [0x7b] * 2
    assert oracle.fp8_encode(np.array([-0.0, 0.0]), "e4m3").tolist() == [0x80, 0x00]
    # ties to even: 1 + 1/16 lies halfway between codes 0x38 (1.0) and 0x39
    assert oracle.fp8_encode(np.array([1.0625, 1.1875]), "e4m3").tolist() == [0x38, 0x3a]
    # smallest subnormal 2^-9 and half of it (tie to even: 0)
    assert oracle.fp8_encode(np.array([2.0 ** -9, 2.0 ** -10]), "e4m3").tolist() == [0x01, 0x00]


def test_fp8_forward_reduces_to_the_bf16_forward_on_exact_codes():
    """With unit scales and operands that are exactly representable in E4M3
    (small integers and halves), the FP8 forward is the plain forward on the
    decoded values, and H's codes are H's own encoding."""
    rng = np.random.default_rng(6)
    N, H, F = 7, 16, 8
    X = rng.integers(-4, 5, (N, H)) / 2.0
    A = rng.integers(-2, 3, (H, F)) / 8.0
    Au = rng.integers(-2, 3, (H, F)) / 8.0
    B = rng.integers(-2, 3, (F, H)) / 8.0
    q = lambda m: oracle.fp8_encode(m, "e4m3")
    for act in (ACT_GELU_TANH, ACT_SWIGLU):
        f8 = oracle.mlp_fwd_fp8(q(X), q(A.T), q(B.T), act, (1, 1, 1, 1, 1),
                                q(Au.T) if act == ACT_SWIGLU else None)
        f = oracle.mlp_fwd(X, A, B, act, Au if act == ACT_SWIGLU else None)
        assert rel(f8["Z"], f["Z"]) < 1e-15 and rel(f8["H"], f["H"]) < 1e-15
        Hd = oracle.fp8_decode(f8["Hq"])
        assert np.array_equal(f8["Hq"], q(f["H"].astype(np.float32)))
        assert rel(f8["Y"], Hd @ B) < 1e-15
        assert f8["h_amax"] == np.max(np.abs(f["H"]))


def _exact_bwd_case(act, rng):
    """Operands exactly representable in E4M3 / E5M2 (small multiples of
    powers of two), Z and U on a grid that keeps every activation
    derivative away from zero (so no dZ falls below E5M2's normal range)."""
    N, H, F = 6, 16, 8
    X = rng.integers(-4, 5, (N, H)) / 2.0
    Hh = rng.integers(-4, 5, (N, F)) / 4.0
    A = rng.integers(-2, 3, (H, F)) / 8.0
    Au = rng.integers(-2, 3, (H, F)) / 8.0
    B = rng.integers(-2, 3, (F, H)) / 8.0
    dY = rng.integers(-3, 4, (N, H)) / 16.0
    grid = np.array([-2.0, -1.5, -1.0, -0.5, 0.5, 1.0, 1.5, 2.0])
    Z = rng.choice(grid, (N, F))
    U = rng.choice(grid, (N, F))
    return X, Hh, A, Au, B, dY, Z, U


@pytest.mark.parametrize("act", [ACT_GELU_TANH, ACT_SWIGLU])
def test_fp8_backward_reduces_to_the_plain_backward_on_exact_codes(act):
    """Unit scales and exact codes: dZ is the plain backward's (definition
    pinned by finite differences above), its codes are its own E5M2
    encoding, and dB, dA, dX are numpy's products of the decoded codes."""
    sw = act == ACT_SWIGLU
    X, Hh, A, Au, B, dY, Z, U = _exact_bwd_case(act, np.random.default_rng(8))
    q4 = lambda m: oracle.fp8_encode(m, "e4m3")
    b8 = oracle.mlp_bwd_fp8(oracle.fp8_encode(dY, "e5m2"), q4(X), q4(Hh), q4(A), q4(B), Z, act,
                            (1, 1, 1, 1, 1, 1, 1), U if sw else None, q4(Au) if sw else None)
    ref = oracle.mlp_bwd(X, A, B, act, dY, {"Z": Z, "U": U if sw else None, "H": Hh},
                         Au if sw else None)
    dZ = np.concatenate([ref["dZ"], ref["dU"]], axis=1) if sw else ref["dZ"]
    assert rel(b8["dZ"], dZ) < 1e-15
    assert np.array_equal(b8["dZq"], oracle.fp8_encode(dZ.astype(np.float32), "e5m2"))
    assert b8["dz_amax"] == np.max(np.abs(dZ))
    dZd = oracle.fp8_decode(b8["dZq"], "e5m2")
    # quantization really moved dZ (so the checks below see the codes)
    assert np.any(dZd != dZ)
    F = A.shape[1]
    assert rel(b8["dB"], Hh.T @ dY) < 1e-15
    assert rel(b8["dA"], X.T @ dZd[:, :F]) < 1e-15
    if sw:
        assert rel(b8["dA_up"], X.T @ dZd[:, F:]) < 1e-15
        assert rel(b8["dX"], dZd @ np.concatenate([A, Au], axis=1).T) < 1e-15
    else:
        assert b8["dA_up"] is None
        assert rel(b8["dX"], dZd @ A.T) < 1e-15


@pytest.mark.parametrize("act", [ACT_GELU_TANH, ACT_SWIGLU])
def test_fp8_backward_power_of_two_scales_cancel(act):
    """Each tensor quantized with its own power-of-two scale and passed its
    inverse: the decoded products, dZ and its codes are unchanged from the
    unit-scale run apart from dZq's exponent (scaled by dz_scale), so a
    scale applied to the wrong product shows up as a power of two."""
    sw = act == ACT_SWIGLU
    X, Hh, A, Au, B, dY, Z, U = _exact_bwd_case(act, np.random.default_rng(9))
    sdy, sb, sh, sx, sa, sdz = 4.0, 16.0, 2.0, 8.0, 32.0, 64.0
    q4 = lambda m, s: oracle.fp8_quantize(m, s)[0]
    unit = oracle.mlp_bwd_fp8(oracle.fp8_encode(dY, "e5m2"), q4(X, 1), q4(Hh, 1), q4(A, 1),
                              q4(B, 1), Z, act, (1,) * 7, U if sw else None,
                              q4(Au, 1) if sw else None)
    sc = oracle.mlp_bwd_fp8(oracle.fp8_quantize(dY, sdy, "e5m2")[0], q4(X, sx), q4(Hh, sh),
                            q4(A, sa), q4(B, sb), Z, act,
                            (1 / sdy, 1 / sb, 1 / sh, 1 / sx, 1 / sa, sdz, 1 / sdz),
                            U if sw else None, q4(Au, sa) if sw else None)
    for k in ("dZ", "dB", "dA", "dX") + (("dA_up",) if sw else ()):
        assert np.array_equal(sc[k], unit[k]), k
    assert np.array_equal(oracle.fp8_decode(sc["dZq"], "e5m2"),
                          oracle.fp8_decode(unit["dZq"], "e5m2") * sdz)
    assert sc["dz_amax"] == unit["dz_amax"]


def _exact_fwd_case(act, rng):
    """Forward operands exact in E4M3 at every power-of-two scale used below,
    chosen so that H lands in E4M3's normal range at both H scales (no
    subnormal or saturated code, so scaling H by a power of two scales its
    codes' values exactly): each column of A (and A_up) picks one entry of X,
    so Z (G, U) lies on the grid +-{0.5, 1, 1.5, 2}."""
    N, H, F = 9, 16, 8
    grid = np.array([-2.0, -1.5, -1.0, -0.5, 0.5, 1.0, 1.5, 2.0])
    X = rng.choice(grid, (N, H))
    A = np.zeros((H, F)); Au = np.zeros((H, F))
    A[rng.integers(0, H, F), np.arange(F)] = 1.0
    Au[rng.integers(0, H, F), np.arange(F)] = 1.0
    B = rng.integers(-2, 3, (F, H)) / 8.0
    return X, A, Au, B


@pytest.mark.parametrize("act", [ACT_GELU_TANH, ACT_SWIGLU])
def test_fp8_forward_power_of_two_scales_cancel(act):
    """Per-tensor scaling of the forward ("Megatron-LM 源码精读——大模型并行训练全景"
    §八 8.2: one scale per tensor; "Megatron Core 带读" §10: quantize by the
    scale, FP8 product, dequantize): every tensor quantized with its own
    power-of-two scale and dequantized by its inverse gives the unit-scale
    run's Z, U, H, Y bit for bit, and H's codes carry exactly h_scale.  A
    scale applied to the wrong product, an inverse swapped between the gate
    and up weights, or FC2 dequantized by h_scale instead of 1/h_scale each
    move a result by a power of two and fail here."""
    sw = act == ACT_SWIGLU
    X, A, Au, B = _exact_fwd_case(act, np.random.default_rng(12))
    q = lambda m, s: oracle.fp8_quantize(m, s)[0]
    unit = oracle.mlp_fwd_fp8(q(X, 1), q(A, 1).T, q(B, 1).T, act, (1, 1, 1, 1, 1),
                              q(Au, 1).T if sw else None)
    sx, sa, sau, sb, sh = 8.0, 32.0, 2.0, 64.0, 16.0
    sc = oracle.mlp_fwd_fp8(q(X, sx), q(A, sa).T, q(B, sb).T, act,
                            (1 / sx, 1 / sa, 1 / sau, 1 / sb, sh), q(Au, sau).T if sw else None)
    # the codes really changed (the scales reached the quantizer)
    assert not np.array_equal(q(X, sx), q(X, 1)) and not np.array_equal(q(B, sb), q(B, 1))
    for k in ("Z", "H", "Y") + (("U",) if sw else ()):
        assert np.array_equal(sc[k], unit[k]), k
    hu = oracle.fp8_decode(unit["Hq"])
    assert np.min(np.abs(hu)) >= 2.0 ** -6 and np.max(np.abs(hu)) * sh <= 448.0
    assert np.array_equal(oracle.fp8_decode(sc["Hq"]), hu * sh)
    assert sc["h_amax"] == unit["h_amax"]
    # and the scaled run is not the unit one by accident: a wrong FC2 scale
    # (h_scale * b_inv) would give Y * h_scale^2
    wrong = oracle.mlp_fwd_fp8(q(X, sx), q(A, sa).T, q(B, sb).T, act,
                               (1 / sx, 1 / sa, 1 / sau, 1 / sb, 1 / sh),
                               q(Au, sau).T if sw else None)
    assert not np.array_equal(wrong["Y"], unit["Y"])


@pytest.mark.parametrize("act", [ACT_GELU_TANH, ACT_SWIGLU])
def test_fp8_forward_rounding_scales_dequantize_the_right_products(act):
    """Scales that are not powers of two (the fused fp32 factors round): each
    product of decoded codes, divided by the exact product of its two
    scales, matches the oracle's dequantized sums to fp32 rounding of the
    factor (three roundings, < 2e-7 relative), so each inverse multiplies
    its own product at any scale."""
    sw = act == ACT_SWIGLU
    rng = np.random.default_rng(13)
    N, H, F = 11, 32, 16
    X = rng.standard_normal((N, H))
    A = rng.standard_normal((H, F)) * 0.05
    Au = rng.standard_normal((H, F)) * 0.05
    B = rng.standard_normal((F, H)) * 0.05
    sx, sa, sau, sb, sh = 37.0, 3000.0, 2500.0, 5000.0, 123.0
    q = lambda m, s: oracle.fp8_quantize(m, s)[0]
    Xq, Aq, Auq, Bq = q(X, sx), q(A, sa), q(Au, sau), q(B, sb)
    f = oracle.mlp_fwd_fp8(Xq, Aq.T, Bq.T, act, (1 / sx, 1 / sa, 1 / sau, 1 / sb, sh),
                           Auq.T if sw else None)
    Xd, Ad, Aud, Bd = (oracle.fp8_decode(c) for c in (Xq, Aq, Auq, Bq))
    G = Xd @ Ad / (sx * sa)
    assert np.max(np.abs(f["Z"] - G)) <= 2e-7 * np.max(np.abs(G))
    if sw:
        Uv = Xd @ Aud / (sx * sau)
        assert np.max(np.abs(f["U"] - Uv)) <= 2e-7 * np.max(np.abs(Uv))
    Hd = oracle.fp8_decode(f["Hq"])
    Y = Hd @ Bd / (sh * sb)
    assert np.max(np.abs(f["Y"] - Y)) <= 2e-7 * np.max(np.abs(Y))
    # H's codes are the encoding of H * h_scale taken in fp32
    assert np.array_equal(f["Hq"], oracle.fp8_encode(
        (f["H"].astype(np.float32) * np.float32(sh)).astype(np.float32)))


# ----------------------------------------------------------------------------
# FP8 delayed scaling: the next scale from the amax history ([P1] §8.2)
# ----------------------------------------------------------------------------
def _step(hist, amax, scale, fmt="e4m3", margin=0):
    return oracle.fp8_scale_update(np.asarray(hist, np.float32), np.asarray(amax, np.float32),
                                   np.asarray(scale, np.float32), fmt, margin)


def test_fp8_scale_closed_forms():
    r = _step(np.zeros((3, 4)), [448.0, 2.0, 0.5], [1.0, 1.0, 1.0])
    assert r["scale"].tolist() == [1.0, 224.0, 896.0]          # fmax / amax, exactly
    # (1/224 and 1/896 are not binary fractions: their fp32 roundings)
    assert r["scale_inv"].tolist() == [1.0, float(np.float32(1 / 224.0)),
                                       float(np.float32(1 / 896.0))]
    assert r["amax"].tolist() == [0.0, 0.0, 0.0]
    assert r["history"][:, 0].tolist() == [448.0, 2.0, 0.5]
    assert _step(np.zeros((1, 2)), [57344.0], [3.0], "e5m2")["scale"].tolist() == [1.0]
    assert _step(np.zeros((1, 2)), [2.0], [3.0], "e4m3", margin=2)["scale"].tolist() == [56.0]


def test_fp8_scale_follows_the_window_maximum():
    """A window of 3: the scale follows the largest of the last 3 amax
    values; 8 drops out after three more steps."""
    hist, amax, scale = np.zeros((1, 3), np.float32), None, np.ones(1, np.float32)
    seen = []
    for a in (8.0, 1.0, 2.0, 1.0, 1.0):
        r = _step(hist, [a], scale)
        hist, scale = r["history"], r["scale"]
        seen.append(float(scale[0]))
    assert seen == [56.0, 56.0, 56.0, 224.0, 224.0]
    assert hist[0].tolist() == [1.0, 1.0, 2.0]


def test_fp8_scale_kept_without_a_finite_positive_amax():
    hist = np.array([[0, 0], [0, -5], [np.nan, 0], [np.inf, 0]], np.float32)
    amax = np.array([0, 0, np.nan, np.inf], np.float32)
    r = _step(hist, amax, [5.0, 6.0, 7.0, 8.0])
    assert r["scale"].tolist() == [5.0, 6.0, 7.0, 8.0]
    assert np.isnan(r["history"][2, 0]) and np.isinf(r["history"][3, 0])
    assert r["history"][2, 1] != r["history"][2, 1]       # the NaN moved back one place
    # a finite value elsewhere in the window still sets the scale
    r = _step([[np.inf, 4.0, 0.0]], [np.nan], [1.0])
    assert r["scale"].tolist() == [112.0]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_scaled_amax_reaches_the_largest_code(fmt):
    """Quantizing the window's maximum with the new scale gives the format's
    largest finite value (never beyond): the scale uses the whole range."""
    rng = np.random.default_rng(7)
    m = np.float32(10.0) ** rng.uniform(-20, 20, 200).astype(np.float32)
    fmax = oracle.FP8_FORMATS[fmt][2]
    r = _step(np.zeros((m.size, 1)), m, np.ones(m.size), fmt)
    y = (m * r["scale"]).astype(np.float32)
    assert np.all(np.abs(y.astype(np.float64) / fmax - 1.0) <= 2.0 ** -23)
    assert np.all(oracle.fp8_decode(oracle.fp8_encode(y, fmt), fmt) == fmax)
    assert np.all(np.abs(r["scale"].astype(np.float64) * r["scale_inv"] - 1.0) <= 2.0 ** -23)
