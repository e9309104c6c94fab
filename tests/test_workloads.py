"""Seeded generator: determinism, bf16 rounding, routing invariants."""
import numpy as np

import workloads as wl


def test_same_seed_same_bytes():
    a = wl.normal_bf16(42, (33, 17), 0.02)
    b = wl.normal_bf16(42, (33, 17), 0.02)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    c = wl.normal_bf16(43, (33, 17), 0.02)
    assert not np.array_equal(a, c)


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20,
                  -1.0 - 2**-8 - 2**-20, 0.0, -0.0, 3.140625, 2.0**-130],
                 dtype=np.float32)
    got = wl.f32_to_bf16_bits(x)
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF81, 0x0000, 0x8000,
                     0x4049, 0x0008], dtype=np.uint16)
    # 2^-130 is a float32 subnormal (bits 0x00080000); bf16 shares float32's
    # exponent range, so it is exact there too (bits 0x0008)
    assert np.array_equal(got, want)
    back = wl.bf16_bits_to_f32(got)
    assert back[0] == 1.0 and back[2] == np.float32(1.0 + 4 * 2**-8)


def test_bf16_rounding_matches_torch():
    import torch
    x = wl.normal(5, (4096,), 3.0)
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_workload_shapes():
    w = wl.WORKLOADS["c4_bf16_swiglu_fwdbwd"]
    assert (w.N, w.H, w.Ft) == (4096, 8192, 3584)
    w = wl.WORKLOADS["c2_bf16_gelu_fwd"]
    assert (w.N, w.H, w.Ft) == (8192, 4096, 2048) and not w.backward
    w = wl.WORKLOADS["c1_f32_gelu_t2"]
    d = wl.gen_mlp_inputs(w, shard=1)
    assert d["A"].shape == (64, 128) and d["B"].shape == (128, 64)
    assert np.array_equal(d["A"], d["A_full"][:, 128:])
    assert np.array_equal(d["B"], d["B_full"][128:, :])


def test_routing_invariants():
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((3000, 64)).astype(np.float32)
    tok, off = wl.route_top2_local(logits, 8, 2)
    # softmax is monotone: top-2 of probabilities equals top-2 of logits
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    top_p = np.argsort(-p, axis=1, kind="stable")[:, :2]
    picks_local = int(np.sum(top_p < 8))
    assert off[-1] == picks_local == len(tok)
    # at most two rows per token
    assert np.bincount(tok, minlength=3000).max() <= 2
    for e in range(8):
        seg = tok[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)           # (expert, token) order
        assert np.all((top_p[seg] == e).any(axis=1))
    # ties go to the lower expert id
    tie = np.zeros((1, 64), np.float32); tie[0, 5] = tie[0, 3] = 1.0
    t2, o2 = wl.route_top2_local(tie, 8, 2)
    assert list(np.diff(o2)) == [0, 0, 0, 1, 0, 1, 0, 0]


def test_grouped_workload_counts():
    w = wl.WORKLOADS["c5_bf16_grouped_swiglu"]
    d = wl.gen_grouped_inputs(w, tokens=2048, H=8, F=16)
    counts = np.diff(d["offsets"])
    assert counts.sum() == len(d["token_ids"]) == d["X_perm"].shape[0]
    assert abs(counts.sum() - 2048 * 2 * 8 / 64) < 0.25 * 2048 * 2 * 8 / 64


def test_extra_input_sets_are_other_draws_of_the_same_shapes():
    """Input sets used for cache-cold timing: set 0 is the workload's own
    draw; other sets have the same shapes and distributions but other
    seeds."""
    w = wl.Workload(77, "tiny", wl.DT_BF16, wl.ACT_SWIGLU, S=16, B=2, H=64, F=256, T=4,
                    w_std=0.02)
    d0 = wl.gen_mlp_inputs(w)
    assert all(np.array_equal(d0[k], wl.gen_mlp_inputs(w, set_index=0)[k])
               for k in ("X", "A", "A_up", "B", "dY"))
    d1 = wl.gen_mlp_inputs(w, set_index=1)
    for k in ("X", "A", "A_up", "B", "dY"):
        assert d1[k].shape == d0[k].shape and d1[k].dtype == d0[k].dtype
        assert not np.array_equal(d1[k], d0[k]), k
