"""HIP-graph replay of the decode and compression launches equals eager execution.

The benchmark replays captured graphs (one per compression window of decode launches, one for
the compressions). Every replay here is checked against the eager result, bit for bit (the
kernels are deterministic), with eager work and synchronisations between replays.
"""
import pytest
import torch

import synth
from gpu_util import shape_of, to_device_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,fdt", [(synth.GDN, synth.BF16), (synth.KDA, synth.F32),
                                      (synth.MAMBA2, synth.BF16)])
def test_graph_replay_matches_eager(kind, fdt):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs

    dv = 64 if kind == synth.MAMBA2 else 128
    w = synth.Workload("graph", kind, 4, 3, 128, dv, 8, 8, 16, 24, fdt, fdt)
    sh = shape_of(w)
    n, T, r = w.units, w.period, w.rank
    hc = synth.head_consts(w, 31)
    gen = synth.rng(31)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    S = torch.zeros((n, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    o = torch.empty((n, w.d_v), dtype=torch.bfloat16 if fdt else torch.float32, device="cuda")
    for _ in range(w.prefill):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, n), w.io_dtype)
        rrs.seed_dense_decode_step(sh, S, d["q"], d["k"], d["v"], d["beta"], d["g"], o)
    pool = [to_device_inputs(synth.step_inputs(w, hc, gen, n), w.io_dtype) for _ in range(2 * T)]
    eager = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, eager)
    graph = rrs.State(*[t.clone() for t in eager.tensors()])
    o_e = torch.empty_like(o)
    o_g = torch.empty_like(o)

    def window(st, out, wi):
        for j in range(T):
            x = pool[wi * T + j]
            rrs.seed_decode_step(sh, st, r + j, x["q"], x["k"], x["v"], x["beta"], x["g"], vbar, out)

    def compress(st):
        rrs.seed_compress(sh, st, r + T)

    # first launches eagerly (raises the LDS limit of the compression kernel before capture)
    window(eager, o_e, 0)
    compress(eager)
    window(graph, o_g, 0)
    compress(graph)
    torch.cuda.synchronize()
    gw = []
    for wi in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            window(graph, o_g, wi)
        gw.append(g)
    gc = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gc):
        compress(graph)
    torch.cuda.synchronize()
    for rep in range(4):
        wi = rep % 2
        window(eager, o_e, wi)
        gw[wi].replay()
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_g), f"replay {rep}: outputs differ"
        for te, tg in zip(eager.tensors(), graph.tensors()):
            assert torch.equal(te, tg), f"replay {rep}: decode state differs"
        compress(eager)
        _ = (S * 2).sum().item()   # unrelated eager work between replays
        gc.replay()
        torch.cuda.synchronize()
        for te, tg in zip(eager.tensors(), graph.tensors()):
            assert torch.equal(te, tg), f"replay {rep}: compressed state differs"


@pytest.mark.parametrize("kind", [synth.GDN, synth.KDA])
def test_graph_replay_chunk_and_spectrum(kind):
    """The chunked update and the spectrum diagnostic captured in a graph: each replay, from a
    fresh copy of the same state, equals the eager call bit for bit (eager work in between)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs

    w = synth.Workload("graphchunk", kind, 2, 3, 128, 128, 16, 16, 32, 24, synth.BF16, synth.BF16)
    sh = shape_of(w)
    n, r, L = w.units, w.rank, 12
    hc = synth.head_consts(w, 41)
    gen = synth.rng(41)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    S = torch.zeros((n, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    o1 = torch.empty((n, w.d_v), dtype=torch.bfloat16, device="cuda")
    for _ in range(w.prefill):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, n), w.io_dtype)
        rrs.seed_dense_decode_step(sh, S, d["q"], d["k"], d["v"], d["beta"], d["g"], o1)
    base = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, base)
    B, H = w.batch, w.heads
    gshape = (B, L, H, w.d_k) if kind == synth.KDA else (B, L, H)
    q = torch.nn.functional.normalize(torch.randn(B, L, H, w.d_k, device="cuda"), dim=-1).bfloat16()
    k = torch.nn.functional.normalize(torch.randn(B, L, H, w.d_k, device="cuda"), dim=-1).bfloat16()
    v = torch.randn(B, L, H, w.d_v, device="cuda").bfloat16()
    beta = torch.rand(B, L, H, device="cuda")
    g = 0.9 + 0.1 * torch.rand(*gshape, device="cuda")

    def run(st, o, spec):
        rrs.seed_decode_chunk(sh, st, r, L, q, k, v, beta, g, vbar, o)
        rrs.seed_state_spectrum(sh, st, out=spec)

    eager = rrs.State(*[t.clone() for t in base.tensors()])
    o_e = torch.empty((B, L, H, w.d_v), dtype=torch.bfloat16, device="cuda")
    sp_e = torch.empty((n, rrs.SEED_SPECTRUM_LEN), dtype=torch.float32, device="cuda")
    run(eager, o_e, sp_e)
    work = rrs.State(*[t.clone() for t in base.tensors()])
    o_g = torch.empty_like(o_e)
    sp_g = torch.empty_like(sp_e)
    run(work, o_g, sp_g)                 # first launches eagerly
    torch.cuda.synchronize()
    g_ = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_):
        run(work, o_g, sp_g)
    for rep in range(3):
        for x, y in zip(work.tensors(), base.tensors()):
            x.copy_(y)
        o_g.zero_()
        sp_g.zero_()
        torch.cuda.synchronize()
        g_.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(sp_g, sp_e), rep
        for x, y in zip(work.tensors(), eager.tensors()):
            assert torch.equal(x, y), rep
