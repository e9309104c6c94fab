"""GPU check of the launch-timing hook (tp_launch_events): every product of
a forward and backward call records one pair of events on the call's
stream, the times are positive and add up to no more than the whole call,
and the results are the same bits as an untimed call."""
import numpy as np
import pytest
import torch

import tensor_transformer_mlp_02_amd as tp
import workloads as wl
from tensor_transformer_mlp_02_amd.tensors import to_device, to_host, ShardBuffers

pytestmark = pytest.mark.gpu


def test_launch_events_time_each_gemm():
    from bench import HipEvents
    w = wl.Workload(95, "timing", wl.DT_BF16, wl.ACT_SWIGLU, S=512, B=2, H=1024, F=2048, T=1,
                    w_std=0.02)
    d = wl.gen_mlp_inputs(w)
    dev = {k: to_device(d[k]) for k in ("X", "A", "A_up", "B", "dY")}
    desc = dict(S=w.S, B=w.B, H=w.H, F_shard=w.Ft, T=w.T, act=w.act, dtype=w.dtype)
    print(f"[gpu] launch events {desc}", flush=True)
    outs = []
    hev = HipEvents(torch)
    stream = torch.cuda.current_stream()
    for timed in (False, True):
        buf = ShardBuffers(desc)
        evs = hev.create(12 + 2)
        if timed:
            hev.record(evs[12], stream)
            tp.tp_launch_events(evs[:12])
        tp.tp_mlp_shard_fwd(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], buf.Z, buf.H, buf.Y)
        tp.tp_mlp_shard_bwd(desc, dev["X"], dev["A"], dev["A_up"], dev["B"], buf.Z, buf.H,
                            dev["dY"], buf.dX, buf.dA, buf.dA_up, buf.dB, buf.ws, buf.ws_bytes)
        if timed:
            assert tp.tp_launch_events_used() == 12      # FC1, FC2, dH, dB, dA, dX
            tp.tp_launch_events(None)
            hev.record(evs[13], stream)
        torch.cuda.synchronize()
        if timed:
            each = [hev.ms(evs[2 * i], evs[2 * i + 1]) for i in range(6)]
            whole = hev.ms(evs[12], evs[13])
            print("  per GEMM ms:", [round(x, 4) for x in each], "whole", round(whole, 4))
            assert all(x > 0 for x in each) and sum(each) <= whole * 1.001
        outs.append({k: to_host(getattr(buf, k)) for k in ("Y", "dX", "dA", "dA_up", "dB")})
    hev.free()
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k
