"""The state-energy diagnostic (sink share of the energy) through the C ABI, against the oracle.

After a prefill-end compression and decode steps (uniform, or ragged with staggered counts), the
GPU's (|S~|^2, |a vbar^T|^2, |U V^T|^2) of every unit is compared with the oracle's, computed
from the explicit matrices of the same state read back in fp64. Tolerance: 1e-4 of the unit's
total energy (fp32 sums over up to 64 x 64 Gram products).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
import synth
from gpu_util import host_state, to_device_inputs, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,fdt,ragged", [(synth.GDN, synth.BF16, False), (synth.KDA, synth.F32, False),
                                             (synth.MAMBA2, synth.F16, False), (synth.GDN, synth.BF16, True),
                                             (synth.KDA, synth.F16, True)])
def test_energy_matches_oracle(kind, fdt, ragged):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs

    r, T, batch, heads = 8, 8, 3, 4
    dv = 64 if kind == synth.MAMBA2 else 128
    io = synth.BF16 if fdt == synth.F16 else fdt
    w = synth.Workload("energy", kind, batch, heads, 128, dv, r, T, T, 32, fdt, io)
    sh = rrs.make_shape(kind, batch, heads, 128, dv, r, T, fdt, io)
    hc = synth.head_consts(w, 211)
    gen = synth.rng(211)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    n = w.units
    S = torch.zeros((n, 128, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((n, dv), dtype=torch_dtype(io), device="cuda")
    for _ in range(w.prefill):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, n), io)
        rrs.seed_dense_decode_step(sh, S, d["q"], d["k"], d["v"], d["beta"], d["g"], o)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    phase = np.arange(n) % T
    for s in range(T - 1):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, n), io)
        if ragged:
            act = torch.as_tensor((phase > s).astype(np.uint8), device="cuda")
            rrs.seed_decode_step_ragged(sh, st, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o,
                                        active=act)
        else:
            rrs.seed_decode_step(sh, st, r + s, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o)
        en = rrs.seed_state_energy(sh, st, vbar).double().cpu().numpy()
        counts = rrs.column_counts(sh, st).numpy()
        states = host_state(sh, st, range(n), counts)
        for u in range(n):
            ref = orc.state_energy(states[u][0], hc.vbar[u % heads], states[u][1], states[u][2])
            err = np.abs(en[u] - np.asarray(ref)) / max(ref[0], 1e-30)
            assert np.all(err <= 1e-4), f"step {s} unit {u} (m {counts[u]}): gpu {en[u]} oracle {ref}"
    # the sink's share pooled over heads: in (0, 1] for these states
    share = float(en[:, 1].sum() / en[:, 0].sum())
    assert 0.0 < share <= 1.0 + 1e-6
