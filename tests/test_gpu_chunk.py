"""GPU parity of the chunked update (seed_decode_chunk, through the C ABI) against the oracle.

Protocol (teacher-forced per call): the GPU state before a chunk is read back in fp64, the
oracle takes the chunk's tokens one Lemma 2 step at a time (oracle.factored_chunk) from it, and
the GPU's state after the chunk and every token's read-out are compared with the oracle's:
rel-Frobenius on S~ = a vbar^T + U V^T, rel-L2 on o. Tolerances are the decode step's (1e-5
for fp32, 2e-2 for bf16, 2.5e-3 for fp16 factors): the forward substitution over a chunk sums
up to 32 products per element in fp32, and with unit keys and 0 <= beta <= 1 its entries stay
of the order of the state (measured worst: 1.4e-6 with fp32 factors).
Chunks run back to back, across a compression, with a token that forgets (g = 0) and with the
largest chunk the state has room for. The inputs are the [batch][len][heads] projections of a
batch of sequences.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
import synth
from gpu_util import host_state, out_tolerance, rel_out, relF, to_device_inputs, tolerance, torch_dtype

pytestmark = pytest.mark.gpu


def _rrs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs
    return rrs, torch


def _chunk_inputs(w, hc, gen, L, forget=None):
    """L tokens of inputs for every unit: numpy per-token dicts ([units] leading) and device
    tensors in the [batch][L][heads] layout."""
    import torch
    xs = [synth.step_inputs(w, hc, gen, w.units) for _ in range(L)]
    if forget is not None:
        xs[forget]["g"][:] = 0.0
    B, H = w.batch, w.heads

    def lay(key, dt):
        a = np.stack([x[key] for x in xs])                       # [L][units](...)
        a = a.reshape((L, B, H) + a.shape[2:]).swapaxes(0, 1)    # [B][L][H](...)
        return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device="cuda").to(dt).contiguous()

    io = torch_dtype(w.io_dtype)
    d = {"q": lay("q", io), "k": lay("k", io), "v": lay("v", io),
         "beta": lay("beta", torch.float32), "g": lay("g", torch.float32)}
    return d


def _host_tokens(d, w, L, units):
    """Per-unit lists of per-token float64 inputs, from the device buffers (exact values)."""
    h = {k: v.float().cpu().double().numpy() for k, v in d.items()}
    out = []
    for u in units:
        b, hh = divmod(u, w.heads)
        out.append([{k: h[k][b, t, hh] for k in h} for t in range(L)])
    return out


def _prefilled(w, seed):
    rrs, torch = _rrs()
    sh = rrs.make_shape(w.kind, w.batch, w.heads, w.d_k, w.d_v, w.rank, w.period, w.factor_dtype,
                        w.io_dtype)
    hc = synth.head_consts(w, seed)
    gen = synth.rng(seed)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    S = torch.zeros((w.units, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    o = torch.empty((w.units, w.d_v), dtype=torch_dtype(w.io_dtype), device="cuda")
    for _ in range(w.prefill):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), w.io_dtype)
        rrs.seed_dense_decode_step(sh, S, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], o)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    return rrs, torch, sh, hc, gen, vbar, st


def _tol(w):
    return tolerance(w), out_tolerance(w)


def check_chunk(rrs, torch, w, sh, st, m, L, d, vbar, hc, units):
    """One chunk on the GPU against the oracle's token loop. Returns (err S~, err o)."""
    pre = host_state(sh, st, units, m)
    o = torch.full((w.batch, L, w.heads, w.d_v), float("nan"), dtype=torch_dtype(w.io_dtype), device="cuda")
    rrs.seed_decode_chunk(sh, st, m, L, d["q"], d["k"], d["v"], d["beta"], d["g"], vbar, o)
    torch.cuda.synchronize()
    post = host_state(sh, st, units, m + L)
    og = o.double().cpu().numpy()
    toks = _host_tokens(d, w, L, units)
    eS = eo = 0.0
    for i, u in enumerate(units):
        vb = hc.vbar[u % w.heads]
        a1, U1, V1, outs = orc.factored_chunk(w.kind, *pre[i], vb, toks[i])
        S1 = orc.reconstruct(a1, vb, U1, V1)
        eS = max(eS, relF(orc.reconstruct(*post[i][:1], vb, *post[i][1:]), S1))
        b, hh = divmod(u, w.heads)
        S_t = orc.reconstruct(*pre[i][:1], vb, *pre[i][1:])
        a_t, U_t, V_t = pre[i]
        for t in range(L):
            a_t, U_t, V_t, o_t = orc.factored_step(w.kind, a_t, U_t, V_t, vb, toks[i][t]["q"], toks[i][t]["k"],
                                                   toks[i][t]["v"], toks[i][t]["beta"], toks[i][t]["g"])
            S_t = orc.reconstruct(a_t, vb, U_t, V_t)
            eo = max(eo, rel_out(og[b, t, hh], o_t, S_t, toks[i][t]["q"]))
    return eS, eo


CASES = {
    "gdn:bf16": (synth.GDN, 128, 128, synth.BF16, synth.BF16),
    "gdn:fp16": (synth.GDN, 128, 128, synth.F16, synth.BF16),
    "gdn:fp32": (synth.GDN, 128, 128, synth.F32, synth.F32),
    "gdn64:bf16": (synth.GDN, 64, 64, synth.BF16, synth.BF16),
    "mamba2:bf16": (synth.MAMBA2, 128, 64, synth.BF16, synth.BF16),
    "mamba2:fp32": (synth.MAMBA2, 128, 64, synth.F32, synth.F32),
    "kda:bf16": (synth.KDA, 128, 128, synth.BF16, synth.BF16),
    "kda:fp16": (synth.KDA, 128, 128, synth.F16, synth.BF16),
    "kda:fp32": (synth.KDA, 128, 128, synth.F32, synth.F32),
    "kda64:bf16": (synth.KDA, 64, 128, synth.BF16, synth.BF16),
}


@pytest.mark.parametrize("case", list(CASES))
def test_chunks_against_oracle(case):
    kind, dk, dv, fdt, idt = CASES[case]
    w = synth.Workload("chunk", kind, 2, 3, dk, dv, 16, 16, 32, 24, fdt, idt)
    rrs, torch, sh, hc, gen, vbar, st = _prefilled(w, seed=201 + kind)
    units = list(range(w.units))
    tol, tol_o = _tol(w)
    m = w.rank
    # three chunks fill the window (7 + 1 + 8 tokens), one with a token that forgets
    for L, forget in ((7, None), (1, None), (8, 5)):
        d = _chunk_inputs(w, hc, gen, L, forget)
        eS, eo = check_chunk(rrs, torch, w, sh, st, m, L, d, vbar, hc, units)
        print(f"[chunk] {case} m={m} L={L}: S {eS:.2e} o {eo:.2e}", flush=True)
        assert eS <= tol and eo <= tol_o, (m, L, eS, eo)
        m += L
        np.testing.assert_array_equal(rrs.column_counts(sh, st), m)
    assert m == w.rank + w.period
    rrs.seed_compress(sh, st, m)
    m = w.rank
    d = _chunk_inputs(w, hc, gen, 16)
    eS, eo = check_chunk(rrs, torch, w, sh, st, m, 16, d, vbar, hc, units)
    print(f"[chunk] {case} after compression, L=16: S {eS:.2e} o {eo:.2e}", flush=True)
    assert eS <= tol and eo <= tol_o


def test_largest_chunk():
    """A chunk of 32 tokens (the maximum) into an empty window of 32 slots."""
    w = synth.Workload("chunk32", synth.GDN, 2, 2, 128, 128, 16, 32, 32, 24, synth.BF16, synth.BF16)
    rrs, torch, sh, hc, gen, vbar, st = _prefilled(w, seed=5)
    L = rrs.seed_chunk_max_tokens()
    d = _chunk_inputs(w, hc, gen, L, forget=20)
    eS, eo = check_chunk(rrs, torch, w, sh, st, w.rank, L, d, vbar, hc, list(range(w.units)))
    print(f"[chunk] L={L}: S {eS:.2e} o {eo:.2e}", flush=True)
    assert eS <= tolerance(w) and eo <= out_tolerance(w)


def test_chunk_matches_token_steps():
    """The chunk against len calls of seed_decode_step on a copy of the same state (both HIP):
    the same state up to the storage rounding, and the same read-outs."""
    w = synth.Workload("chunkvs", synth.GDN, 4, 4, 128, 128, 16, 16, 32, 24, synth.BF16, synth.BF16)
    rrs, torch, sh, hc, gen, vbar, st = _prefilled(w, seed=9)
    st2 = rrs.State(*[t.clone() for t in st.tensors()])
    L = 12
    d = _chunk_inputs(w, hc, gen, L)
    o = torch.empty((w.batch, L, w.heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    rrs.seed_decode_chunk(sh, st, w.rank, L, d["q"], d["k"], d["v"], d["beta"], d["g"], vbar, o)
    o1 = torch.empty((w.units, w.d_v), dtype=torch.bfloat16, device="cuda")
    for t in range(L):
        step = {k: v[:, t].reshape(w.units, *v.shape[3:]).contiguous() for k, v in d.items()}
        rrs.seed_decode_step(sh, st2, w.rank + t, step["q"], step["k"], step["v"], step["beta"], step["g"],
                             vbar, o1)
        eo = (o1.float() - o[:, t].reshape(w.units, w.d_v).float()).norm() / o1.float().norm()
        assert eo.item() <= out_tolerance(w), (t, eo.item())
    torch.cuda.synchronize()
    units = list(range(w.units))
    A = host_state(sh, st, units, w.rank + L)
    B = host_state(sh, st2, units, w.rank + L)
    for i, u in enumerate(units):
        vb = hc.vbar[u % w.heads]
        e = relF(orc.reconstruct(*A[i][:1], vb, *A[i][1:]), orc.reconstruct(*B[i][:1], vb, *B[i][1:]))
        assert e <= tolerance(w), (u, e)
    # the keys are stored unchanged by both (bf16 inputs into bf16 factors)
    assert torch.equal(st.U[:, w.rank:w.rank + L], st2.U[:, w.rank:w.rank + L])


def test_full_size_chunk_sampled():
    """gdn-stack36's per-layer shape (4096 units, 128 x 128, r = T = 32) with a 32-token chunk,
    sampled units against the oracle."""
    w = synth.Workload("chunkfull", synth.GDN, 128, 32, 128, 128, 32, 32, 64, 8, synth.BF16, synth.BF16)
    rrs, torch, sh, hc, gen, vbar, st = _prefilled(w, seed=17)
    L = 32
    d = _chunk_inputs(w, hc, gen, L)
    units = [0, 1, 777, 2048, 4095]
    eS, eo = check_chunk(rrs, torch, w, sh, st, w.rank, L, d, vbar, hc, units)
    print(f"[chunk] full size L={L}: S {eS:.2e} o {eo:.2e}", flush=True)
    assert eS <= tolerance(w) and eo <= out_tolerance(w)


@pytest.mark.parametrize("fdt", [synth.BF16, synth.F16])
def test_kda_chunk_folds_channels(fdt):
    """KDA: channels whose scale falls below the floor within a chunk are folded into the
    stored columns (here: half the channels forget at token 3, and a quarter decay by 0.05 per
    token, 0.05^16 being below both floors), and the state stays the oracle's."""
    w = synth.Workload("chunkkda", synth.KDA, 2, 3, 128, 128, 16, 16, 32, 24, fdt, synth.BF16)
    rrs, torch, sh, hc, gen, vbar, st = _prefilled(w, seed=33)
    L = 16
    xs_gen = synth.rng(34)
    d = _chunk_inputs(w, hc, xs_gen, L)
    g = d["g"].clone()
    g[:, 3, :, :64] = 0.0
    g[:, :, :, 96:] = 0.05
    d["g"] = g.contiguous()
    eS, eo = check_chunk(rrs, torch, w, sh, st, w.rank, L, d, vbar, hc, list(range(w.units)))
    scales = st.scale[:, :w.d_k].cpu()
    print(f"[chunk] kda fold {fdt}: S {eS:.2e} o {eo:.2e}; channels at scale 1: "
          f"{int((scales == 1.0).sum())} of {scales.numel()}", flush=True)
    assert eS <= tolerance(w) and eo <= out_tolerance(w)
    assert torch.all(scales[:, :64] == 1.0) and torch.all(scales[:, 96:] == 1.0)
    assert torch.all(torch.isfinite(st.U.float()))


def test_ragged_chunk():
    """Units at different column counts take a chunk each from their own count; a masked unit
    and units without room are left bit for bit as they were, their rows of o unwritten."""
    w = synth.Workload("chunkrag", synth.GDN, 4, 2, 128, 128, 16, 16, 32, 24, synth.BF16, synth.BF16)
    rrs, torch, sh, hc, gen, vbar, st = _prefilled(w, seed=61)
    n, H = w.units, w.heads
    o1 = torch.empty((n, w.d_v), dtype=torch.bfloat16, device="cuda")
    # request b takes 3 b decode steps first: counts 16, 19, 22, 25
    for t in range(9):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, n), synth.BF16)
        act = torch.tensor([1 if (u // H) * 3 > t else 0 for u in range(n)], dtype=torch.uint8, device="cuda")
        rrs.seed_decode_step_ragged(sh, st, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o1, active=act)
    m0 = rrs.column_counts(sh, st).numpy()
    L = 8                                           # 25 + 8 > 32: request 3 has no room
    active = torch.ones(n, dtype=torch.uint8, device="cuda")
    active[0] = 0                                   # and unit 0 is masked out
    d = _chunk_inputs(w, hc, gen, L)
    units = list(range(n))
    pre = host_state(sh, st, units, m0)
    before = [t.clone() for t in st.tensors()]
    o = torch.full((w.batch, L, H, w.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    rrs.seed_decode_chunk_ragged(sh, st, L, d["q"], d["k"], d["v"], d["beta"], d["g"], vbar, o, active=active)
    torch.cuda.synchronize()
    m1 = rrs.column_counts(sh, st).numpy()
    toks = _host_tokens(d, w, L, units)
    og = o.double().cpu().numpy()
    for u in units:
        b, hh = divmod(u, H)
        runs = u != 0 and m0[u] + L <= w.rank + w.period
        if not runs:
            assert m1[u] == m0[u]
            for x, y in zip(before, st.tensors()):
                assert torch.equal(x[u], y[u]), u
            assert np.all(np.isnan(og[b, :, hh])), u
            continue
        assert m1[u] == m0[u] + L
        post = host_state(sh, st, [u], m0[u] + L)[0]
        vb = hc.vbar[hh]
        a1, U1, V1, outs = orc.factored_chunk(w.kind, *pre[u], vb, toks[u])
        S1 = orc.reconstruct(a1, vb, U1, V1)
        eS = relF(orc.reconstruct(post[0], vb, post[1], post[2]), S1)
        assert eS <= tolerance(w), (u, eS)
        a_t, U_t, V_t = pre[u]
        for t in range(L):
            x = toks[u][t]
            a_t, U_t, V_t, o_t = orc.factored_step(w.kind, a_t, U_t, V_t, vb, x["q"], x["k"], x["v"], x["beta"], x["g"])
            assert rel_out(og[b, t, hh], o_t, orc.reconstruct(a_t, vb, U_t, V_t), x["q"]) <= out_tolerance(w)


@pytest.mark.parametrize("kind,fdt", [(synth.GDN, synth.BF16), (synth.KDA, synth.F16), (synth.MAMBA2, synth.BF16)])
def test_chunk_stochastic_rounding(kind, fdt):
    """Stochastically rounded chunk stores stay within the format's tolerance of the oracle
    (KDA with channels that fold), and the draws follow the key."""
    import rank_recurrent_state_amd as rrs_mod
    dv = 64 if kind == synth.MAMBA2 else 128
    w = synth.Workload("chunksr", kind, 2, 3, 128, dv, 16, 16, 32, 24, fdt, synth.BF16)
    rrs, torch, _, hc, gen, vbar, st0 = _prefilled(w, seed=71)
    results = []
    for key in (5, 5, 6):
        sh = rrs_mod.make_shape(kind, w.batch, w.heads, 128, dv, 16, 16, fdt, synth.BF16,
                                rounding=rrs_mod.SEED_ROUND_STOCHASTIC, rng_key=key)
        st = rrs.State(*[t.clone() for t in st0.tensors()])
        d = _chunk_inputs(w, hc, synth.rng(72), 12)
        if kind == synth.KDA:
            g = d["g"].clone()
            g[:, 4, :, :32] = 0.0
            d["g"] = g.contiguous()
        eS, eo = check_chunk(rrs, torch, w, sh, st, w.rank, 12, d, vbar, hc, list(range(w.units)))
        print(f"[chunk] sr {kind} {fdt} key {key}: S {eS:.2e} o {eo:.2e}", flush=True)
        assert eS <= tolerance(w) and eo <= out_tolerance(w)
        results.append([t.clone() for t in st.tensors()])
    assert all(torch.equal(x, y) for x, y in zip(results[0], results[1]))
    assert not torch.equal(results[0][2], results[2][2])          # V differs under another key
