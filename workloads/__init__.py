"""Seeded synthetic inputs for the tensor-parallel MLP shard.

This module is shared by the GPU path's tests/bench and by the oracle's
tests.  It holds no arithmetic of the MLP itself: only random draws, the
bf16 storage encoding (round-to-nearest-even of a float32, and its exact
decode), the table of workload shapes, and the token -> local-expert routing
that produces the grouped workload's ragged row lists.

Shapes and distributions follow the workloads stated for the method:
hidden states ``[S, B, H]`` flattened to ``[N, H]`` with ``n = s*B + b``
(Megatron Core 带读 §02, the hidden/partial shape walk-through), a column
shard ``A_i [H, F/T]`` and a row shard ``B_i [F/T, H]``
(Megatron-LM 源码精读——大模型并行训练全景, §三 3.1/3.2).

Seeds: tensor ``k`` of workload ``c`` uses ``PCG64(1000*c + k)`` with
k: X=1, A/Ag=2, Au=3, B=4, dY=5, router logits=6, partial stand-ins 7...
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "normal", "normal_bf16", "route_top2_local", "gen_mlp_inputs",
    "gen_grouped_inputs", "gen_partials",
]

ACT_GELU_TANH = 0
ACT_SWIGLU = 1
DT_F32 = 0
DT_BF16 = 1

K_X, K_A, K_AUP, K_B, K_DY, K_LOGITS, K_PARTIAL0 = 1, 2, 3, 4, 5, 6, 7
K_DY_TOKENS = 80   # token-level dY of the MoE layer (past the partial stand-ins' seeds)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload: shard shapes, activation, storage type, distributions."""
    cid: int            # seed namespace (1..5)
    name: str
    dtype: int          # DT_F32 / DT_BF16
    act: int            # ACT_GELU_TANH / ACT_SWIGLU
    S: int
    B: int
    H: int
    F: int              # full intermediate width (all T shards)
    T: int
    w_std: float
    x_std: float = 1.0
    dy_std: float = 1e-2
    backward: bool = True
    full_weights: bool = False   # draw the full A/B and slice (small case only)
    experts: int = 0             # >0: grouped expert workload (expert TP = 1)
    tokens: int = 0
    n_route: int = 0             # experts the router chooses from
    topk: int = 0

    @property
    def N(self) -> int:
        return self.S * self.B

    @property
    def Ft(self) -> int:
        assert self.F % self.T == 0
        return self.F // self.T


WORKLOADS = {
    # fp32 GeLU(tanh), both shards of T=2, checked against the unsharded MLP.
    "c1_f32_gelu_t2": Workload(1, "c1_f32_gelu_t2", DT_F32, ACT_GELU_TANH,
                               S=32, B=4, H=64, F=256, T=2, w_std=0.02,
                               full_weights=True),
    # one rank of T=8, bf16 GeLU, forward only.
    "c2_bf16_gelu_fwd": Workload(2, "c2_bf16_gelu_fwd", DT_BF16, ACT_GELU_TANH,
                                 S=2048, B=4, H=4096, F=16384, T=8, w_std=0.02,
                                 backward=False),
    # same shard with the backward.
    "c3_bf16_gelu_fwdbwd": Workload(3, "c3_bf16_gelu_fwdbwd", DT_BF16,
                                    ACT_GELU_TANH, S=2048, B=4, H=4096,
                                    F=16384, T=8, w_std=0.02),
    # Llama-style SwiGLU shard of T=8.
    "c4_bf16_swiglu_fwdbwd": Workload(4, "c4_bf16_swiglu_fwdbwd", DT_BF16,
                                      ACT_SWIGLU, S=4096, B=1, H=8192,
                                      F=28672, T=8, w_std=0.015),
    # one rank's 8 local experts of a top-2-of-64 router, SwiGLU, expert TP 1.
    "c5_bf16_grouped_swiglu": Workload(5, "c5_bf16_grouped_swiglu", DT_BF16,
                                       ACT_SWIGLU, S=16384, B=1, H=4096,
                                       F=1408, T=1, w_std=0.02, experts=8,
                                       tokens=16384, n_route=64, topk=2),
}


# --------------------------------------------------------------------------
# bf16 storage encoding
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite (normal draws); NaN/Inf are not produced here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------
def normal(seed: int, shape, std: float) -> np.ndarray:
    """float32 N(0, std^2) draw from PCG64(seed)."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def normal_bf16(seed: int, shape, std: float) -> np.ndarray:
    """bf16 bit patterns of ``normal(seed, shape, std)``."""
    return f32_to_bf16_bits(normal(seed, shape, std))


# extra input sets of a workload (cache-cold timing rotates several) draw
# with seeds 1000*c + SET_STRIDE*s + k, s >= 1; set 0 is the workload's own
SET_STRIDE = 200


def _draw(w: Workload, k: int, shape, std: float, set_index: int = 0) -> np.ndarray:
    seed = 1000 * w.cid + SET_STRIDE * set_index + k
    if w.dtype == DT_BF16:
        return normal_bf16(seed, shape, std)
    return normal(seed, shape, std)


def gen_mlp_inputs(w: Workload, shard: int = 0, n_rows: Optional[int] = None,
                   set_index: int = 0) -> dict:
    """Inputs of one tensor-parallel shard of a dense workload.

    Returns a dict of storage arrays (float32, or uint16 bf16 bits):
    X [N,H], A [H,Ft], A_up [H,Ft] (SwiGLU only, else None), B [Ft,H],
    dY [N,H] (None for forward-only workloads).  For ``full_weights``
    workloads the full A [H,F] / B [F,H] are drawn once and the shard's
    column / row slice is returned, plus ``A_full``/``B_full``.  Other
    workloads draw the shard's weights directly at shard shape.
    ``n_rows`` truncates the token dimension (a prefix of the same draw is
    NOT guaranteed; it is a smaller draw of its own, for small tests).
    ``set_index`` > 0 draws another input set of the same shapes and
    distributions (other seeds), for timing with cold caches.
    """
    N = w.N if n_rows is None else n_rows
    H, F, Ft = w.H, w.F, w.Ft
    out = {}
    if set_index:
        assert not w.full_weights
        d = lambda k, shape, std: _draw(w, k, shape, std, set_index)
        out["X"] = d(K_X, (N, H), w.x_std)
        out["A"] = d(K_A, (H, Ft), w.w_std)
        out["A_up"] = d(K_AUP, (H, Ft), w.w_std) if w.act == ACT_SWIGLU else None
        out["B"] = d(K_B, (Ft, H), w.w_std)
        out["dY"] = d(K_DY, (N, H), w.dy_std) if w.backward else None
        return out
    out["X"] = _draw(w, K_X, (N, H), w.x_std)
    if w.full_weights:
        A_full = _draw(w, K_A, (H, F), w.w_std)
        B_full = _draw(w, K_B, (F, H), w.w_std)
        out["A_full"], out["B_full"] = A_full, B_full
        out["A"] = np.ascontiguousarray(A_full[:, shard * Ft:(shard + 1) * Ft])
        out["B"] = np.ascontiguousarray(B_full[shard * Ft:(shard + 1) * Ft, :])
        if w.act == ACT_SWIGLU:
            Au_full = _draw(w, K_AUP, (H, F), w.w_std)
            out["A_up_full"] = Au_full
            out["A_up"] = np.ascontiguousarray(Au_full[:, shard * Ft:(shard + 1) * Ft])
        else:
            out["A_up"] = None
    else:
        out["A"] = _draw(w, K_A, (H, Ft), w.w_std)
        out["A_up"] = _draw(w, K_AUP, (H, Ft), w.w_std) if w.act == ACT_SWIGLU else None
        out["B"] = _draw(w, K_B, (Ft, H), w.w_std)
    out["dY"] = _draw(w, K_DY, (N, H), w.dy_std) if w.backward else None
    return out


def route_top2_local(logits: np.ndarray, n_local: int, topk: int = 2):
    """Token -> local expert rows from router scores.

    Each token picks the ``topk`` experts with the largest score (softmax is
    monotone, so the choice on logits equals the choice on probabilities;
    ties go to the lower expert id).  Picks that land on experts
    ``0..n_local-1`` become rows, ordered by (expert, token); a token that
    picks two local experts yields two rows.  Returns (token_ids [R] int64,
    offsets [n_local+1] int64).  Routing as in Megatron Core 带读 §09
    (router scores -> top-k experts -> local experts compute).
    """
    n_tok, n_exp = logits.shape
    # stable sort of -logits: equal scores keep ascending expert id
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    rows_e, rows_t = [], []
    for e in range(n_local):
        toks = np.nonzero((order == e).any(axis=1))[0]
        rows_t.append(toks.astype(np.int64))
        rows_e.append(np.full(toks.shape, e, dtype=np.int64))
    token_ids = np.concatenate(rows_t) if rows_t else np.zeros(0, np.int64)
    counts = np.array([len(t) for t in rows_t], dtype=np.int64)
    offsets = np.zeros(n_local + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return token_ids, offsets


def gen_grouped_inputs(w: Workload, tokens: Optional[int] = None,
                       H: Optional[int] = None, F: Optional[int] = None,
                       set_index: int = 0) -> dict:
    """Inputs of the grouped local-expert workload.

    X_perm [R,H] (rows of the token matrix gathered in (expert, token)
    order), offsets [E+1], token_ids [R], Wg/Wu [E,H,F], Wd [E,F,H],
    dY_perm [R,H].  ``tokens``/``H``/``F`` shrink the problem for tests.
    ``set_index`` > 0 redraws the tokens, weights and dY (other seeds) over
    the same routing, for timing with cold caches.
    """
    n_tok = w.tokens if tokens is None else tokens
    H = w.H if H is None else H
    F = w.F if F is None else F
    E = w.experts
    seed = 1000 * w.cid
    logits = normal(seed + K_LOGITS, (n_tok, w.n_route), 1.0)
    token_ids, offsets = route_top2_local(logits, E, w.topk)
    X = _draw(w, K_X, (n_tok, H), w.x_std, set_index)
    out = {
        "token_ids": token_ids,
        "offsets": offsets,
        "X_perm": np.ascontiguousarray(X[token_ids]),
        "Wg": _draw(w, K_A, (E, H, F), w.w_std, set_index),
        "Wu": _draw(w, K_AUP, (E, H, F), w.w_std, set_index),
        "Wd": _draw(w, K_B, (E, F, H), w.w_std, set_index),
        "dY_perm": _draw(w, K_DY, (len(token_ids), H), w.dy_std, set_index),
        "logits": logits,
    }
    return out


def route_weights(logits: np.ndarray, token_ids: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Router output for each expert-sorted row: the softmax probability
    (over all experts' logits of its token, no renormalisation over the
    chosen ones) of the row's expert, float32.  The router is not part of
    the path; this is the combine's weight input, drawn from the same
    seeded logits the routing used."""
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    E = len(offsets) - 1
    w = np.empty(len(token_ids), np.float32)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        w[lo:hi] = p[token_ids[lo:hi], e]
    return w


def token_rows(token_ids: np.ndarray, n_tok: int):
    """Inverse of the row -> token map: for each token, the rows that hold
    it, in increasing row order (= expert order).  Returns (tok_ptr [N+1],
    tok_rows [R]) as int32 (CSR)."""
    order = np.argsort(token_ids, kind="stable")
    counts = np.bincount(token_ids, minlength=n_tok) if len(token_ids) else np.zeros(n_tok, int)
    ptr = np.zeros(n_tok + 1, np.int64)
    ptr[1:] = np.cumsum(counts)
    return ptr.astype(np.int32), order.astype(np.int32)


def gen_moe_inputs(w: Workload, tokens: Optional[int] = None, H: Optional[int] = None,
                   F: Optional[int] = None) -> dict:
    """Token-level inputs around the grouped experts: X [N,H] (tokens),
    dY [N,H], the routing rows (token_ids, offsets), their router weights,
    the per-token row lists, and the expert weights.  Same seeds as
    gen_grouped_inputs, so X[token_ids] is its X_perm."""
    g = gen_grouped_inputs(w, tokens, H, F)
    n_tok = w.tokens if tokens is None else tokens
    H = w.H if H is None else H
    X = _draw(w, K_X, (n_tok, H), w.x_std)
    ptr, rows = token_rows(g["token_ids"], n_tok)
    return {
        "X": X,
        "dY": _draw(w, K_DY_TOKENS, (n_tok, H), w.dy_std),
        "token_ids": g["token_ids"].astype(np.int32),
        "offsets": g["offsets"],
        "row_weight": route_weights(g["logits"], g["token_ids"], g["offsets"]),
        "tok_ptr": ptr,
        "tok_rows": rows,
        "Wg": g["Wg"], "Wu": g["Wu"], "Wd": g["Wd"],
    }


def gen_partials(w: Workload, T: int, shape, std: float, dtype: Optional[int] = None) -> list:
    """T seeded stand-in partial outputs, N(0, std^2), in the storage type."""
    dt = w.dtype if dtype is None else dtype
    outs = []
    for i in range(T):
        seed = 1000 * w.cid + K_PARTIAL0 + i
        if dt == DT_BF16:
            outs.append(normal_bf16(seed, shape, std))
        else:
            outs.append(normal(seed, shape, std))
    return outs
