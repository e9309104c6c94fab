"""GPU: the allocation-free backward (tp_mlp_shard_bwd_noalloc, dZ in the
library's per-GPU scratch array) against tp_mlp_shard_bwd with a caller
workspace: two calls in a row, the second on a smaller input (the scratch
then holds the first call's larger dZ), each bit for bit equal to the
workspace call (same kernels, same order) and within the bf16 bar of the
fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_02_amd as tp
import workloads as wl
from parity import TOL, assert_close, f64
from tensor_transformer_mlp_02_amd.tensors import to_device, to_host, ShardBuffers

pytestmark = pytest.mark.gpu

CASES = [
    # (act, N, H, Ft): the second is smaller, with ragged edges
    (wl.ACT_SWIGLU, 2048, 1024, 1536),
    (wl.ACT_GELU_TANH, 300, 520, 392),
]


def test_noalloc_backward_matches_workspace_backward():
    for k, (act, N, H, Ft) in enumerate(CASES):
        w = wl.Workload(97 + k, "noalloc", wl.DT_BF16, act, S=N, B=1, H=H, F=Ft, T=1,
                        w_std=0.05)
        d = wl.gen_mlp_inputs(w)
        desc = dict(S=N, B=1, H=H, F_shard=Ft, T=1, act=act, dtype=wl.DT_BF16)
        dev = {n: (to_device(d[n]) if d[n] is not None else None)
               for n in ("X", "A", "A_up", "B", "dY")}
        ref = ShardBuffers(desc)
        print(f"[gpu] noalloc case {k}: {desc}", flush=True)
        tp.tp_mlp_shard_fwd(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], ref.Z, ref.H, ref.Y)
        tp.tp_mlp_shard_bwd(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], ref.Z, ref.H,
                            dev["dY"], ref.dX, ref.dA, ref.dA_up, ref.dB, ref.ws, ref.ws_bytes)
        out = {"dX": torch.full_like(ref.dX, float("nan")),
               "dA": torch.full_like(ref.dA, float("nan")),
               "dA_up": torch.full_like(ref.dA_up, float("nan")) if ref.dA_up is not None
               else None,
               "dB": torch.full_like(ref.dB, float("nan"))}
        tp.tp_mlp_shard_bwd_noalloc(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], ref.Z,
                                    ref.H, dev["dY"], out["dX"], out["dA"], out["dA_up"],
                                    out["dB"])
        torch.cuda.synchronize()
        for n, t in out.items():
            if t is None:
                continue
            assert np.array_equal(to_host(t), to_host(getattr(ref, n))), n
        f = oracle.mlp_fwd(d["X"], d["A"], d["B"], act, d["A_up"])
        b = oracle.mlp_bwd(d["X"], d["A"], d["B"], act, d["dY"], f, d["A_up"])
        tol = TOL[wl.DT_BF16]
        assert_close("dX", f64(to_host(out["dX"])), b["dX"], tol)
        assert_close("dA", to_host(out["dA"]), b["dA"], tol)
        assert_close("dB", to_host(out["dB"]), b["dB"], tol)
        if out["dA_up"] is not None:
            assert_close("dA_up", to_host(out["dA_up"]), b["dA_up"], tol)
