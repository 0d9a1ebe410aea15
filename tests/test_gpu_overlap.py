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


def test_staggered_matches_serial():
    """rank_recurrent_state_amd.StaggeredStack (ragged decode per layer on one stream, the units
    that fill compressed per group of layers on the other) against the same work on one stream:
    every step, the ragged decode of each layer, then one listed compression of all the units
    that filled. The kernels are deterministic, so states and read-outs must agree bit for bit."""
    import numpy as np
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
        _run_staggered(rrs, torch, np, streams)
    finally:
        for st in streams:
            st.close()


def _run_staggered(rrs, torch, np, streams):
    L, B, H, r, T = 7, 8, 2, 8, 8
    U1 = B * H
    w = synth.Workload("stg", synth.GDN, B * L, H, 128, 128, r, T, 2 * T, 8, synth.BF16, synth.BF16)
    sh_all = rrs.make_shape(w.kind, B * L, H, 128, 128, r, T, synth.BF16, synth.BF16)
    shapes = [rrs.make_shape(w.kind, B, H, 128, 128, r, T, synth.BF16, synth.BF16) for _ in range(L)]
    hc = synth.head_consts(w, 5)
    gen = synth.rng(5)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    n = w.units
    S = torch.zeros((n, 128, 128), dtype=torch.float32, device="cuda")
    o = torch.empty((n, 128), dtype=torch.bfloat16, device="cuda")
    for _ in range(w.prefill):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, n), synth.BF16)
        rrs.seed_dense_decode_step(sh_all, S, d["q"], d["k"], d["v"], d["beta"], d["g"], o)
    base = rrs.State.empty(sh_all)
    rrs.seed_state_from_dense(sh_all, S, vbar, base)
    # stagger: request b of every layer sits out the steps from its phase on (ends at r + b mod T)
    phase = torch.tensor([(u % U1) // H % T for u in range(n)], device="cuda")
    for s in range(T - 1):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, n), synth.BF16)
        rrs.seed_decode_step_ragged(sh_all, base, d["q"], d["k"], d["v"], d["beta"], d["g"], vbar, o,
                                    active=(phase > s).to(torch.uint8))
    steps = 2 * T + 3
    inputs = [to_device_inputs(synth.step_inputs(w, hc, gen, n), synth.BF16) for _ in range(steps)]
    per_layer = [[{k: v[l * U1:(l + 1) * U1].contiguous() for k, v in x.items()} for l in range(L)] for x in inputs]

    def views(st):
        return [rrs.State(*[t[l * U1:(l + 1) * U1] for t in st.tensors()]) for l in range(L)]

    # serial reference
    ref = rrs.State(*[t.clone() for t in base.tensors()])
    ref_l = views(ref)
    o_ref = [torch.empty((U1, 128), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    for s in range(steps):
        for l in range(L):
            x = per_layer[s][l]
            rrs.seed_decode_step_ragged(shapes[l], ref_l[l], x["q"], x["k"], x["v"], x["beta"], x["g"], vbar, o_ref[l])
        m = rrs.column_counts(sh_all, ref).numpy()
        full = np.nonzero(m == r + T)[0]
        if len(full):
            rrs.seed_compress_units(sh_all, ref, torch.as_tensor(full, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(rrs.column_counts(sh_all, ref).max()) < r + T

    # the overlapped staggered schedule (groups of about 6 full units: 3 layers per group)
    stg = rrs.State(*[t.clone() for t in base.tensors()])
    stg_l = views(stg)
    o_stg = [torch.empty((U1, 128), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    stack = rrs.StaggeredStack(sh_all, stg, shapes, stg_l, *streams, group_units=6)
    assert len(stack.groups) == 3
    stack.start()
    for s in range(steps):
        stack.step(per_layer[s], [vbar] * L, o_stg)
    stack.finish()
    torch.cuda.synchronize()
    for l in range(L):
        assert torch.equal(o_stg[l], o_ref[l]), l
    for x, y in zip(stg.tensors(), ref.tensors()):
        assert torch.equal(x, y)
