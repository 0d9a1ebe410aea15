"""The overlapped schedule (rank_recurrent_state_amd.OverlappedStack) against the same launches
issued one after another on a single stream.

The kernels are deterministic, so if the events order every layer's compression after the
decode launch that filled it, and its next decode launch after the compression, the states and
the read-outs are bit for bit those of the serial schedule. The serial reference below follows
the schedule's specification on its own: layer l compresses first after T - (l mod T) steps,
then every T steps at r + T columns.
"""
import pytest

import synth
from gpu_util import to_device_inputs

pytestmark = pytest.mark.gpu


def test_overlapped_matches_serial():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs
    if rrs.under_profiler():
        pytest.skip("the CU-partitioned schedule is not run under the profiler")
    streams = rrs.partition_streams(4)
    if streams is None:
        pytest.skip("CU-masked streams not available")
    try:
        _run(rrs, torch, streams)
    finally:
        for st in streams:
            st.close()


def _run(rrs, torch, streams):
    L, B, H, r, T = 9, 2, 2, 8, 8
    w = synth.Workload("ovl", synth.GDN, B, H, 128, 128, r, T, 2 * T, 8, synth.BF16, synth.BF16)
    shapes = [rrs.make_shape(w.kind, B, H, 128, 128, r, T, synth.BF16, synth.BF16) for _ in range(L)]
    hc = synth.head_consts(w, 3)
    gen = synth.rng(3)
    vbars = [torch.tensor(hc.vbar, dtype=torch.float32, device="cuda") for _ in range(L)]
    n = w.units
    base = []
    for l in range(L):
        S = torch.zeros((n, 128, 128), dtype=torch.float32, device="cuda")
        o = torch.empty((n, 128), dtype=torch.bfloat16, device="cuda")
        for _ in range(w.prefill):
            d = to_device_inputs(synth.step_inputs(w, hc, gen, n), synth.BF16)
            rrs.seed_dense_decode_step(shapes[l], S, d["q"], d["k"], d["v"], d["beta"], d["g"], o)
        st = rrs.State.empty(shapes[l])
        rrs.seed_state_from_dense(shapes[l], S, vbars[l], st)
        base.append(st)
    steps = 2 * T + 5
    inputs = [[to_device_inputs(synth.step_inputs(w, hc, gen, n), synth.BF16) for _ in range(L)]
              for _ in range(steps)]

    # serial reference on the current stream
    ref = [rrs.State(*[t.clone() for t in st.tensors()]) for st in base]
    o_ref = [torch.empty((n, 128), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    m = [r] * L
    first = [T - (l % T) for l in range(L)]
    for s in range(steps):
        for l in range(L):
            x = inputs[s][l]
            rrs.seed_decode_step(shapes[l], ref[l], m[l], x["q"], x["k"], x["v"], x["beta"], x["g"], vbars[l],
                                 o_ref[l])
            m[l] += 1
            if m[l] == r + (first[l] or T):
                rrs.seed_compress(shapes[l], ref[l], m[l])
                m[l], first[l] = r, 0
    torch.cuda.synchronize()

    # the overlapped schedule
    ovl = [rrs.State(*[t.clone() for t in st.tensors()]) for st in base]
    o_ovl = [torch.empty((n, 128), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    stack = rrs.OverlappedStack(shapes, ovl, *streams)
    stack.start()
    for s in range(steps):
        stack.step(inputs[s], vbars, o_ovl)
    stack.finish()
    torch.cuda.synchronize()
    assert stack.m == m
    for l in range(L):
        assert torch.equal(o_ovl[l], o_ref[l]), l
        for x, y in zip(ovl[l].tensors(), ref[l].tensors()):
            assert torch.equal(x, y), l
