"""fp64 CPU oracle of the tensor-parallel MLP shard (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the GPU library: the C
loop nests live in ``tp_mlp_oracle.c`` (built by ``oracle/build.py`` with
gcc), and this wrapper only converts storage arrays to float64, allocates
outputs and loops over shards / experts.

What each function computes, and the passage it follows ([P1] is the page
"Megatron-LM 源码精读——大模型并行训练全景", [P3] "Megatron Core 带读"):

* ``mlp_fwd`` / ``mlp_bwd`` -- one shard of the paired column -> act -> row
  MLP and its backward (Megatron-LM 源码精读——大模型并行训练全景, §三
  3.1-3.4; SwiGLU: same page, §七).
* ``sharded_fwd`` / ``sharded_bwd`` -- all T shards of a full weight pair,
  plus the sums over shards (the forward all-reduce of Y_i and the backward
  all-reduce of dX_i, same page §三 3.3 diagram), and the unsharded MLP.
* ``partial_sum`` -- the all-reduce arithmetic over resident partials.
* ``grouped_fwd`` / ``grouped_bwd`` -- each local expert runs the SwiGLU MLP
  on its own routed rows (Megatron Core 带读 §09; Megatron-LM 源码精读
  docs index, "MoE 层与 Expert Parallelism": grouped-GEMM expert compute).
* ``reduce_scatter`` -- the sequence-parallel split of the summed partials.
* ``moe_permute`` / ``moe_combine`` / ``moe_combine_bwd`` -- token dispatch
  to the local experts and the weighted merge back (Megatron Core 带读 §09).
* ``fp8_encode`` / ``fp8_decode`` / ``fp8_quantize`` / ``mlp_fwd_fp8`` /
  ``mlp_bwd_fp8`` -- per-tensor E4M3 / E5M2 quantization and the shard's
  forward and backward on codes (Megatron-LM 源码精读 §8.2; Megatron Core
  带读 §10).
* ``fp8_scale_update`` -- the next per-tensor scales from each tensor's
  amax history (same passages).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from workloads import bf16_bits_to_f32, DT_BF16, ACT_SWIGLU, ACT_GELU_TANH

ACT_IDENTITY = 99

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from oracle.build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_num_threads.restype = ctypes.c_int
    for name in ("orc_gelu_tanh", "orc_gelu_tanh_grad", "orc_sigmoid",
                 "orc_silu", "orc_silu_grad"):
        f = getattr(lib, name)
        f.restype = ctypes.c_double
        f.argtypes = [ctypes.c_double]
    for name in ("orc_matmul_nn", "orc_matmul_nt", "orc_matmul_tn"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [_i64, _i64, _i64, _d, _d, _d]
    lib.orc_mlp_fwd.restype = ctypes.c_int
    lib.orc_mlp_fwd.argtypes = [_i64, _i64, _i64, ctypes.c_int] + [_d] * 8
    lib.orc_mlp_bwd.restype = ctypes.c_int
    lib.orc_mlp_bwd.argtypes = [_i64, _i64, _i64, ctypes.c_int] + [_d] * 14
    lib.orc_partial_sum.restype = ctypes.c_int
    lib.orc_partial_sum.argtypes = [ctypes.c_int, _i64, ctypes.POINTER(_d), _d]
    _lib = lib
    return lib


def num_threads() -> int:
    return _load().orc_num_threads()


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_d)


def to_f64(a, dtype=None) -> np.ndarray:
    """Storage array (float32 or uint16 bf16 bits) -> float64, exactly."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.ascontiguousarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# scalar activations (exposed for the closed-form pins)
# ----------------------------------------------------------------------------
def gelu_tanh(z: float) -> float:
    return _load().orc_gelu_tanh(float(z))


def gelu_tanh_grad(z: float) -> float:
    return _load().orc_gelu_tanh_grad(float(z))


def silu(g: float) -> float:
    return _load().orc_silu(float(g))


def silu_grad(g: float) -> float:
    return _load().orc_silu_grad(float(g))


def sigmoid(g: float) -> float:
    return _load().orc_sigmoid(float(g))


def matmul(kind: str, A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The oracle's own product loops: 'nn' A@B, 'nt' A@B.T, 'tn' A.T@B."""
    lib = _load()
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    if kind == "nn":
        M, K = A.shape; N = B.shape[1]; f = lib.orc_matmul_nn
    elif kind == "nt":
        M, K = A.shape; N = B.shape[0]; f = lib.orc_matmul_nt
    elif kind == "tn":
        K, M = A.shape; N = B.shape[1]; f = lib.orc_matmul_tn
    else:
        raise ValueError(kind)
    C = np.empty((M, N), np.float64)
    f(M, N, K, _p(A), _p(B), _p(C))
    return C


# ----------------------------------------------------------------------------
# one shard
# ----------------------------------------------------------------------------
def mlp_fwd(X, A, B, act, A_up=None) -> dict:
    """One shard's forward.  Returns Z (gate G for SwiGLU), U (SwiGLU),
    H (post-activation) and Y (the shard's partial output), all float64."""
    lib = _load()
    X, A, B, A_up = (to_f64(t) for t in (X, A, B, A_up))
    N, Hd = X.shape
    Ft = A.shape[1]
    assert A.shape == (Hd, Ft) and B.shape == (Ft, Hd)
    Z = np.empty((N, Ft)); Hact = np.empty((N, Ft)); Y = np.empty((N, Hd))
    U = np.empty((N, Ft)) if act == ACT_SWIGLU else None
    rc = lib.orc_mlp_fwd(N, Hd, Ft, act, _p(X), _p(A), _p(A_up), _p(B),
                         _p(Z), _p(U), _p(Hact), _p(Y))
    if rc != 0:
        raise ValueError(f"orc_mlp_fwd failed ({rc})")
    return {"Z": Z, "U": U, "H": Hact, "Y": Y}


def mlp_bwd(X, A, B, act, dY, fwd: dict, A_up=None) -> dict:
    """One shard's backward from the forward's saved tensors.  Returns dX
    (the shard's partial), dA, dA_up (SwiGLU), dB, dZ (dG), dU (SwiGLU)."""
    lib = _load()
    X, A, B, A_up, dY = (to_f64(t) for t in (X, A, B, A_up, dY))
    N, Hd = X.shape
    Ft = A.shape[1]
    sw = act == ACT_SWIGLU
    dX = np.empty((N, Hd)); dA = np.empty((Hd, Ft)); dB = np.empty((Ft, Hd))
    dAup = np.empty((Hd, Ft)) if sw else None
    dZ = np.empty((N, Ft)); dU = np.empty((N, Ft)) if sw else None
    rc = lib.orc_mlp_bwd(N, Hd, Ft, act, _p(X), _p(A), _p(A_up), _p(B),
                         _p(fwd["Z"]), _p(fwd["U"]), _p(fwd["H"]), _p(dY),
                         _p(dX), _p(dA), _p(dAup), _p(dB), _p(dZ), _p(dU))
    if rc != 0:
        raise ValueError(f"orc_mlp_bwd failed ({rc})")
    return {"dX": dX, "dA": dA, "dA_up": dAup, "dB": dB, "dZ": dZ, "dU": dU}


def partial_sum(parts) -> np.ndarray:
    """Sum of T partial outputs, elementwise, fp64."""
    lib = _load()
    parts = [to_f64(p) for p in parts]
    shape = parts[0].shape
    flat = [np.ascontiguousarray(p.reshape(-1)) for p in parts]
    arr = (_d * len(flat))(*[_p(p) for p in flat])
    out = np.empty(flat[0].shape[0])
    rc = lib.orc_partial_sum(len(flat), flat[0].shape[0], arr, _p(out))
    if rc != 0:
        raise ValueError(f"orc_partial_sum failed ({rc})")
    return out.reshape(shape)


def reduce_scatter(parts, S, B, H, rank) -> np.ndarray:
    """Sequence-parallel reduce-scatter ([P1] §三 3.5; [P3] §06): the sum of
    the T partial [S,B,H] outputs, of which rank keeps sequence rows
    rank*S/T .. (rank+1)*S/T - 1.  Written as its definition: the full sum,
    then the rank's slice."""
    T = len(parts)
    if S % T:
        raise ValueError("S must be divisible by T")
    full = partial_sum([np.asarray(p).reshape(S, B, H) for p in parts])
    m = S // T
    return full[rank * m:(rank + 1) * m]


# ----------------------------------------------------------------------------
# MoE dispatch and combine around the grouped experts ([P3] §09: router ->
# top-k experts -> tokens sent to their experts -> expert compute -> results
# merged by weight -> back in token order)
# ----------------------------------------------------------------------------
def moe_permute(X, token_ids) -> np.ndarray:
    """Row r of the expert-sorted matrix is token token_ids[r]."""
    return to_f64(X)[np.asarray(token_ids, np.int64)]


def moe_combine(Y_perm, token_ids, n_tok, row_weight=None) -> np.ndarray:
    """Y[t] = sum over the rows r holding token t of w[r] Y_perm[r] (w = 1
    when None); a token without rows gets zeros."""
    Yp = to_f64(Y_perm)
    w = np.ones(len(token_ids)) if row_weight is None else np.asarray(row_weight, np.float64)
    Y = np.zeros((n_tok, Yp.shape[1]))
    for r, t in enumerate(np.asarray(token_ids, np.int64)):
        Y[t] += w[r] * Yp[r]
    return Y


def moe_combine_bwd(dY, Y_perm, token_ids, row_weight):
    """Backward of moe_combine: dY_perm[r] = w[r] dY[t(r)], and the weight
    gradient dw[r] = <dY[t(r)], Y_perm[r]>."""
    dY = to_f64(dY)
    Yp = to_f64(Y_perm)
    t = np.asarray(token_ids, np.int64)
    w = np.asarray(row_weight, np.float64)
    dYp = w[:, None] * dY[t]
    dw = np.einsum("rh,rh->r", dY[t], Yp)
    return dYp, dw


# ----------------------------------------------------------------------------
# FP8 ([P1] §8.2: E4M3 forward / E5M2 backward, per-tensor scaling from
# amax; [P3] §10: quantize by scale/amax -> FP8 kernel -> dequantize).
# Formats as in the OCP 8-bit floating point definition: E4M3 (bias 7, no
# infinities, largest finite 448) and E5M2 (bias 15, largest finite 57344).
# ----------------------------------------------------------------------------
FP8_FORMATS = {"e4m3": (4, 3, 448.0), "e5m2": (5, 2, 57344.0)}


def fp8_encode(y, fmt="e4m3") -> np.ndarray:
    """Round-to-nearest-even code of each value, saturating at the largest
    finite value (values beyond it take its code).  Input: exact values
    (float32 or float64 arrays); NaN is not expected."""
    ebits, mbits, vmax = FP8_FORMATS[fmt]
    bias = (1 << (ebits - 1)) - 1
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.minimum(np.abs(y), vmax)
    out = np.zeros(a.shape, np.uint8)
    emin = 1 - bias
    nz = a > 0
    e = np.zeros(a.shape, np.int64)
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64)
    # guard the log2 rounding at exact powers of two
    e[nz] -= (np.ldexp(1.0, e[nz]) > a[nz])
    e[nz] += (np.ldexp(1.0, e[nz] + 1) <= a[nz])
    sub = nz & (e < emin)
    nor = nz & ~sub

    def rne(u):
        f = np.floor(u)
        r = u - f
        f = f + ((r > 0.5) | ((r == 0.5) & (np.mod(f, 2) == 1)))
        return f.astype(np.int64)

    # subnormals: units of 2^(emin - mbits); a result of 2^mbits is the
    # smallest normal's code, which the formula already produces
    out[sub] = rne(a[sub] / np.ldexp(1.0, emin - mbits)).astype(np.uint8)
    m = a[nor] / np.ldexp(1.0, e[nor]) - 1.0
    q = rne(m * (1 << mbits))
    en = e[nor] + (q == (1 << mbits))
    q = np.where(q == (1 << mbits), 0, q)
    out[nor] = (((en + bias) << mbits) | q).astype(np.uint8)
    return out | sign


def fp8_decode(code, fmt="e4m3") -> np.ndarray:
    """Value of each finite code (float64)."""
    ebits, mbits, _ = FP8_FORMATS[fmt]
    bias = (1 << (ebits - 1)) - 1
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    val = np.where(e == 0, np.ldexp(m.astype(np.float64), 1 - bias - mbits),
                   np.ldexp(1.0 + m / (1 << mbits), e - bias))
    return s * val


def fp8_quantize(x, scale, fmt="e4m3"):
    """Per-tensor quantization: the code of x * scale, the product taken in
    float32 (as the device does), and amax = max |x|."""
    xs = (to_f64(x).astype(np.float32) * np.float32(scale)).astype(np.float32)
    return fp8_encode(xs, fmt), float(np.max(np.abs(to_f64(x)))) if np.size(x) else 0.0


def fp8_scale_update(history, amax, scale, fmt="e4m3", margin=0) -> dict:
    """Delayed per-tensor scaling ([P1] §8.2: each tensor's scale is derived
    from the history of its amax; [P3] §10: the scale comes from amax, then
    the tensor is quantized with it).  One step for n tensors, float32:

    * the window: each row of history [n, len] (newest first) moves one
      place back, its oldest value dropping out, and this step's amax takes
      the front; amax is then cleared for the next step;
    * its maximum m: the largest finite positive value in the row;
    * the scale: the format's largest finite value over m, times
      2^-margin, so a tensor no larger than m in magnitude quantizes without
      saturating; with no such value the previous scale is kept;
    * its inverse 1 / scale (what dequantization multiplies by).

    Each division and product is one float32 operation (the device's)."""
    h = np.array(history, dtype=np.float32, copy=True)
    a = np.array(amax, dtype=np.float32, copy=True)
    sc = np.array(scale, dtype=np.float32, copy=True)
    n, length = h.shape
    window = np.empty_like(h)
    window[:, 1:] = h[:, :length - 1]
    window[:, 0] = a
    fmax = np.float32(FP8_FORMATS[fmt][2])
    mult = np.float32(2.0 ** -margin)
    for t in range(n):
        ok = [v for v in window[t] if np.isfinite(v) and v > 0]
        if ok:
            m = np.float32(max(ok))
            sc[t] = np.float32(np.float32(fmax / m) * mult)
    with np.errstate(divide="ignore"):
        inv = (np.float32(1.0) / sc).astype(np.float32)
    return {"history": window, "amax": np.zeros_like(a), "scale": sc, "scale_inv": inv}


def mlp_fwd_fp8(Xq, Aq_t, Bq_t, act, scales, Auq_t=None) -> dict:
    """One shard's forward on E4M3 operands (codes).  Xq [N,H]; the weights
    as quantized transposes: Aq_t, Auq_t [Ft,H], Bq_t [H,Ft].  scales =
    (x_inv, a_inv, au_inv, b_inv, h_scale), float32.  FC1's sums are scaled
    by float32(x_inv * a_inv) (the up projection by x_inv * au_inv), the
    activation gives H, H is quantized with h_scale (its codes are the
    FC2 operand), and FC2's sums are scaled by float32(float32(1 / h_scale)
    * b_inv).  The products are the oracle's own loops on the decoded
    values.  Returns Z (G), U, H, Hq (codes), h_amax, Y (float64)."""
    x_inv, a_inv, au_inv, b_inv, h_scale = (np.float32(v) for v in scales)
    X = fp8_decode(Xq)
    dg = float(np.float32(x_inv * a_inv))
    Ad = fp8_decode(Aq_t).T * dg
    Aud = fp8_decode(Auq_t).T * float(np.float32(x_inv * au_inv)) if act == ACT_SWIGLU else None
    # FC1 and the activation (FC2 of this call is not used: its operand is
    # the quantized H)
    f = mlp_fwd(X, Ad, np.zeros((Ad.shape[1], X.shape[1])), act, Aud)
    Hq = fp8_encode((f["H"].astype(np.float32) * h_scale).astype(np.float32))
    dy = float(np.float32(np.float32(np.float32(1.0) / h_scale) * b_inv))
    Y = matmul("nt", fp8_decode(Hq), fp8_decode(Bq_t)) * dy
    return {"Z": f["Z"], "U": f["U"], "H": f["H"], "Hq": Hq,
            "h_amax": float(np.max(np.abs(f["H"]))) if f["H"].size else 0.0, "Y": Y}


def mlp_bwd_fp8(dYq, Xq, Hq, Aq, Bq, Z, act, scales, U=None, Auq=None) -> dict:
    """One shard's backward on FP8 codes ([P1] §8.2: gradients in E5M2,
    weights and activations in E4M3).  Codes in their logical layouts: dYq
    [N,H] (E5M2), Xq [N,H], Hq [N,Ft] (E4M3), Aq, Auq [H,Ft], Bq [Ft,H]
    (E4M3); Z (the gate G for SwiGLU) and U are the forward's saved values.
    scales = (dy_inv, b_inv, h_inv, x_inv, a_inv, dz_scale, dz_inv); the
    gate and up weights share a_inv.  Steps, each product's code sums
    scaled by the float32 product of the two inverse scales:
      dH = dY B^T (dy_inv b_inv), dZ (and dU) from dH and the activation's
        derivative at the saved Z (U), as in the plain backward;
      dZq = E5M2 codes of float32(dZ) * dz_scale (the concatenation [dG|dU]
        for SwiGLU), dz_amax = max |dZ|;
      dB = H^T dY (h_inv dy_inv); dA (| dA_up) = X^T dZq (x_inv dz_inv);
      dX = dZq [A | A_up]^T (dz_inv a_inv).
    Returns float64 dZ (the [dG|dU] values before quantization), dZq,
    dz_amax, dA, dA_up, dB, dX."""
    dy_inv, b_inv, h_inv, x_inv, a_inv, dz_scale, dz_inv = (np.float32(v) for v in scales)
    sw = act == ACT_SWIGLU
    f32 = lambda a, b: float(np.float32(a * b))
    dY = fp8_decode(dYq, "e5m2")
    Xd, Hd, Ad, Bd = fp8_decode(Xq), fp8_decode(Hq), fp8_decode(Aq), fp8_decode(Bq)
    Aud = fp8_decode(Auq) if sw else None
    # dH's scale is folded into B; the plain backward then gives the
    # activation derivative (its own dA, dX, dB are not the FP8 ones)
    b = mlp_bwd(Xd, Ad, Bd * f32(dy_inv, b_inv), act, dY,
                {"Z": to_f64(Z), "U": to_f64(U) if sw else None, "H": Hd}, Aud)
    dZ = np.concatenate([b["dZ"], b["dU"]], axis=1) if sw else b["dZ"]
    dZq = fp8_encode((dZ.astype(np.float32) * dz_scale).astype(np.float32), "e5m2")
    dZd = fp8_decode(dZq, "e5m2")
    Ft = Ad.shape[1]
    dB = matmul("tn", Hd, dY) * f32(h_inv, dy_inv)
    dAc = matmul("tn", Xd, dZd) * f32(x_inv, dz_inv)
    Wc = np.concatenate([Ad, Aud], axis=1) if sw else Ad
    dX = matmul("nt", dZd, Wc) * f32(dz_inv, a_inv)
    return {"dZ": dZ, "dZq": dZq, "dz_amax": float(np.max(np.abs(dZ))) if dZ.size else 0.0,
            "dA": dAc[:, :Ft], "dA_up": dAc[:, Ft:] if sw else None, "dB": dB, "dX": dX}


# ----------------------------------------------------------------------------
# all shards of a full weight pair, and the unsharded MLP
# ----------------------------------------------------------------------------
def shard_weights(A_full, B_full, T, A_up_full=None):
    """Column split of A (and A_up) and row split of B into T shards; the
    shard width is F/T and must divide exactly (§三 3.1: the per-partition
    output size is the full size divided by the world size)."""
    F = A_full.shape[1]
    if F % T:
        raise ValueError("F must be divisible by T")
    Ft = F // T
    shards = []
    for i in range(T):
        sl = slice(i * Ft, (i + 1) * Ft)
        shards.append((np.ascontiguousarray(A_full[:, sl]),
                       np.ascontiguousarray(B_full[sl, :]),
                       None if A_up_full is None else np.ascontiguousarray(A_up_full[:, sl])))
    return shards


def sharded_fwd_bwd(X, A_full, B_full, T, act, dY=None, A_up_full=None) -> dict:
    """Every shard's forward (+backward), the sums over shards, and the
    unsharded MLP run on the full weights (T=1)."""
    X64, A64, B64 = to_f64(X), to_f64(A_full), to_f64(B_full)
    Au64 = to_f64(A_up_full)
    dY64 = to_f64(dY)
    out = {"shards": []}
    for (Ai, Bi, Aui) in shard_weights(A64, B64, T, Au64):
        f = mlp_fwd(X64, Ai, Bi, act, Aui)
        rec = {"fwd": f}
        if dY64 is not None:
            rec["bwd"] = mlp_bwd(X64, Ai, Bi, act, dY64, f, Aui)
        out["shards"].append(rec)
    out["Y"] = partial_sum([r["fwd"]["Y"] for r in out["shards"]])
    full_f = mlp_fwd(X64, A64, B64, act, Au64)
    out["full_fwd"] = full_f
    if dY64 is not None:
        out["dX"] = partial_sum([r["bwd"]["dX"] for r in out["shards"]])
        out["full_bwd"] = mlp_bwd(X64, A64, B64, act, dY64, full_f, Au64)
    return out


# ----------------------------------------------------------------------------
# grouped local experts
# ----------------------------------------------------------------------------
def grouped_fwd(X_perm, offsets, Wg, Wu, Wd) -> dict:
    """Rows [o_e, o_{e+1}) of X_perm run expert e's SwiGLU MLP (expert
    tensor-parallel size 1).  Returns G, U, H [R,F] and Y [R,H]."""
    X = to_f64(X_perm)
    R, Hd = X.shape
    E, _, F = np.asarray(Wg).shape
    G = np.zeros((R, F)); U = np.zeros((R, F)); Hh = np.zeros((R, F)); Y = np.zeros((R, Hd))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        f = mlp_fwd(np.ascontiguousarray(X[lo:hi]), to_f64(Wg[e]), to_f64(Wd[e]),
                    ACT_SWIGLU, to_f64(Wu[e]))
        G[lo:hi], U[lo:hi], Hh[lo:hi], Y[lo:hi] = f["Z"], f["U"], f["H"], f["Y"]
    return {"G": G, "U": U, "H": Hh, "Y": Y}


def grouped_bwd(X_perm, offsets, Wg, Wu, Wd, dY_perm, fwd: dict) -> dict:
    """Backward of ``grouped_fwd``: dX [R,H], dWg/dWu [E,H,F], dWd [E,F,H]
    (an expert with no rows has zero weight gradients)."""
    X = to_f64(X_perm)
    dY = to_f64(dY_perm)
    R, Hd = X.shape
    E, _, F = np.asarray(Wg).shape
    dX = np.zeros((R, Hd))
    dWg = np.zeros((E, Hd, F)); dWu = np.zeros((E, Hd, F)); dWd = np.zeros((E, F, Hd))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        sub = {"Z": np.ascontiguousarray(fwd["G"][lo:hi]),
               "U": np.ascontiguousarray(fwd["U"][lo:hi]),
               "H": np.ascontiguousarray(fwd["H"][lo:hi])}
        b = mlp_bwd(np.ascontiguousarray(X[lo:hi]), to_f64(Wg[e]), to_f64(Wd[e]),
                    ACT_SWIGLU, np.ascontiguousarray(dY[lo:hi]), sub, to_f64(Wu[e]))
        dX[lo:hi] = b["dX"]
        dWg[e], dWu[e], dWd[e] = b["dA"], b["dA_up"], b["dB"]
    return {"dX": dX, "dWg": dWg, "dWu": dWu, "dWd": dWd}
