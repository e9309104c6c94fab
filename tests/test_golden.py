"""The pages' shape and sharding statements (tests/golden/page_shapes.txt,
each line cited) against the library's size arithmetic and the oracle's
sharding, on the CPU.  The library is asked only for sizes (workspace
query, the binding's size checks) and argument checks, which touch no GPU.
"""
import ctypes
import os

import numpy as np
import pytest

import oracle
import tensor_transformer_mlp_02_amd as tp

HERE = os.path.dirname(os.path.abspath(__file__))


def load():
    ex = {}
    for line in open(os.path.join(HERE, "golden", "page_shapes.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        key, src, fields = (x.strip() for x in line.split("|"))
        assert src.startswith("[P"), f"{key}: no citation"
        ex[key] = {k: int(v) for k, v in (f.split("=") for f in fields.split())}
    return ex


EX = load()


def test_column_shard_width_and_workspace():
    e = EX["column_output"]
    assert e["O"] // e["p"] == e["local_cols"]
    desc = dict(S=e["S"], B=e["B"], H=e["H"], F_shard=e["local_cols"], T=e["p"],
                act=tp.TP_ACT_GELU_TANH, dtype=tp.TP_BF16)
    # the backward's dZ holds this shard's local output [S,B,O/p] (bf16)
    assert tp.tp_mlp_shard_bwd_workspace(desc) == e["S"] * e["B"] * e["local_cols"] * 2


def test_row_partials_sum_to_the_full_output():
    e = EX["row_partial"]
    rng = np.random.default_rng(5)
    N = e["S"] * e["B"]
    X = rng.standard_normal((N, e["I"]))
    W = rng.standard_normal((e["I"], e["O"]))
    parts = [X[:, i * e["in_cols"]:(i + 1) * e["in_cols"]] @ W[i * e["in_cols"]:(i + 1) * e["in_cols"]]
             for i in range(e["p"])]
    assert all(p.shape == (N, e["partial_cols"]) for p in parts)
    assert np.allclose(oracle.partial_sum(parts), X @ W, rtol=1e-12, atol=1e-12)


def test_divide_rule():
    e = EX["divide"]
    A = np.zeros((8, e["F"])); B = np.zeros((e["F"], 8))
    shards = oracle.shard_weights(A, B, e["T"])
    assert len(shards) == e["T"] and shards[0][0].shape[1] == e["Ft"]
    with pytest.raises(ValueError):
        oracle.shard_weights(np.zeros((8, e["F_bad"])), np.zeros((e["F_bad"], 8)), e["T"])


def test_mlp_widths():
    e = EX["mlp_widths"]
    assert e["F"] == 4 * e["d"]


def test_sequence_parallel_slice_and_volume():
    s, v = EX["sp_slice"], EX["sp_volume"]
    assert s["S"] // s["T"] == s["rows_per_rank"]
    assert v["S"] * v["B"] * v["H"] // v["T"] == v["elems_per_rank"]
    parts = [np.full((s["S"], s["B"], s["H"]), float(i)) for i in range(s["T"])]
    out = oracle.reduce_scatter(parts, s["S"], s["B"], s["H"], rank=1)
    assert out.shape == (s["rows_per_rank"], s["B"], s["H"]) and out.size == v["elems_per_rank"]
    # the library's reduce-scatter needs whole sequence slices: S a multiple
    # of T (checked before any GPU call)
    fake = [(1 << 44) + (k << 40) for k in range(s["T"] + 2)]
    with pytest.raises(tp.TpError) as err:
        tp.tp_partial_sum_scatter(tp.TP_BF16, s["T"] + 1, fake[:s["T"] + 1], s["S"], s["B"],
                                  s["H"], 1, fake[-1])
    assert err.value.status == 2   # TP_ERR_SHAPE


def test_three_d_layout_arithmetic():
    e = EX["dp_example"]
    assert e["TP"] * e["PP"] * e["DP"] == e["W"]
