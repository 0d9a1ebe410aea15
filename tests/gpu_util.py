"""Helpers for the GPU parity tests: inputs on the device, state read-back, oracle comparison.

The HIP path is reached only through the C ABI (rank_recurrent_state_amd). The oracle
receives host copies of exactly the values the device buffers hold (bf16 inputs included), so
no cross-device random-number equality is needed. Comparisons are on products, never on
factors: the factored state is reconstructed as S~ = a vbar^T + U V^T.
"""
from __future__ import annotations

import numpy as np

import oracle as orc
import synth


def torch_dtype(code):
    import torch
    return {synth.F32: torch.float32, synth.BF16: torch.bfloat16, synth.F16: torch.float16}[code]


def shape_of(w: synth.Workload, batch=None, heads=None, units_layers=1):
    import rank_recurrent_state_amd as rrs
    return rrs.make_shape(w.kind, batch if batch is not None else w.batch * units_layers,
                          heads if heads is not None else w.heads, w.d_k, w.d_v, w.rank,
                          w.period, w.factor_dtype, w.io_dtype)


def to_device_inputs(x: dict, io_dtype, device="cuda"):
    """numpy step inputs -> device tensors (q, k, v in the io dtype; beta, g fp32)."""
    import torch
    dt = torch_dtype(io_dtype)
    out = {}
    for key in ("q", "k", "v"):
        out[key] = torch.tensor(x[key], dtype=torch.float32, device=device).to(dt).contiguous()
    out["beta"] = torch.tensor(x["beta"], dtype=torch.float32, device=device).contiguous()
    out["g"] = torch.tensor(x["g"], dtype=torch.float32, device=device).contiguous()
    return out


def host_inputs(dx: dict, units) -> list:
    """Per-unit float64 copies of device step inputs (exact values held by the buffers)."""
    h = {k: v.float().cpu().double().numpy() for k, v in dx.items()}
    return [{k: h[k][u] for k in h} for u in units]


def host_state(shape, st, units, m):
    """Read back (a, U, V) in true (decay- and sink-folded) form, float64, for the given units
    (m: the column count, one for all units or one per unit).

    The scale buffer holds the lazy decay (GDN / Mamba-2: slot 0 for the columns j < r, slot
    1 + j - r after; KDA: the per-channel Gamma), then the sink coefficients c of the window's
    columns: the true sink is the decayed stored a plus sum_{j >= r} c[j - r] times true column j.
    """
    import torch
    units = list(units)
    ms = [int(m)] * len(units) if np.ndim(m) == 0 else [int(x) for x in m]
    idx = torch.as_tensor(units, device=st.a.device)
    a = st.a.index_select(0, idx).double().cpu().numpy()
    Ua = st.U.index_select(0, idx).double().cpu().numpy()
    Va = st.V.index_select(0, idx).double().cpu().numpy()
    sc = st.scale.index_select(0, idx).double().cpu().numpy()
    s0 = shape.d_k if shape.kind == synth.KDA else 1 + shape.period
    r = shape.rank
    out = []
    for n in range(len(units)):
        m = ms[n]
        Us, Vs = Ua[n, :m], Va[n, :m]
        if shape.kind == synth.KDA:
            U = (Us * sc[n][None, :s0]).T
            a_true = sc[n][:s0] * a[n]
        else:
            c = np.array([sc[n][0] if j < r else sc[n][1 + j - r] for j in range(m)])
            U = (Us * c[:, None]).T
            a_true = sc[n][0] * a[n]
        for j in range(r, m):
            a_true = a_true + sc[n][s0 + j - r] * U[:, j]
        out.append((a_true, U, Vs.T))
    return out


def relF(A, B):
    nb = np.linalg.norm(B)
    return float(np.linalg.norm(A - B) / nb) if nb > 0 else float(np.linalg.norm(A))


def rel_out(o_gpu, o_ref, S_ref, q) -> float:
    """Relative error of a read-out o = S^T q. The denominator is |o_ref|, floored at
    1e-2 |S|_F |q|: when q is nearly orthogonal to the state, the output is a cancellation far
    below its natural scale and no fp32 evaluation can hold it to a relative bound."""
    den = max(float(np.linalg.norm(o_ref)), 1e-2 * float(np.linalg.norm(S_ref)) * float(np.linalg.norm(q)))
    return float(np.linalg.norm(o_gpu - o_ref) / den) if den > 0 else float(np.linalg.norm(o_gpu))


def tolerance(w_or_dtype) -> float:
    """Relative tolerance by factor storage: about five units of the format's rounding (bf16
    2^-8, fp16 2^-11), and 1e-5 for fp32 factors."""
    code = w_or_dtype.factor_dtype if hasattr(w_or_dtype, "factor_dtype") else w_or_dtype
    return {synth.F32: 1e-5, synth.BF16: 2e-2, synth.F16: 2.5e-3}[code]


def out_tolerance(w) -> float:
    """Tolerance of a read-out o: o is stored in the io dtype, so it is held to the looser of the
    factor and io formats' tolerances (fp16 factors come with bf16 inputs and outputs)."""
    return max(tolerance(w.factor_dtype), tolerance(w.io_dtype))


def near_tie_threshold(code) -> float:
    return {synth.F32: 1e-3, synth.BF16: 5e-2, synth.F16: 1e-2}[code]


def compare_compression(C_before, a, vbar, U_gpu, V_gpu, r, code, a_ref=None):
    """Compare a GPU compression with the oracle's exact truncation of the same content.

    Returns (kind, err, raw, sink). kind "product" holds the reconstructed state S~ to the
    oracle's by rel-Frobenius; kind "optimal" (near ties, where several truncations are correct)
    checks the Eckart-Young optimality criterion instead (0 or inf). In both branches the sink is
    compared as well: a compression never recomputes the split (Lemma 1), so the GPU's sink must
    equal a_ref, the true sink before the call (for the prefill-end compression, the oracle's
    S vbar / |vbar|^2); sink = |a - a_ref| / |a_ref|, and err is the larger of the two.
    raw is the product error against the oracle's truncation whichever branch is taken.
    """
    Ur, Vr, _ = orc.compress(*C_before, r) if isinstance(C_before, tuple) else orc.truncate(C_before, r)
    C = C_before[0] @ C_before[1].T if isinstance(C_before, tuple) else C_before
    if a_ref is None:
        raise ValueError("compare_compression needs the reference sink a_ref")
    S_ref = orc.reconstruct(a_ref, vbar, Ur, Vr)
    S_gpu = orc.reconstruct(a, vbar, U_gpu, V_gpu)
    sink = relF(a, a_ref)
    gap = orc.relative_gap(C, r)
    if gap < near_tie_threshold(code):
        ok = orc.truncation_is_optimal(C, U_gpu @ V_gpu.T, r, tolerance(code), abs_tol=tolerance(code) ** 2)
        return "optimal", max(0.0 if ok else float("inf"), sink), relF(S_gpu, S_ref), sink
    return "product", max(relF(S_gpu, S_ref), sink), relF(S_gpu, S_ref), sink


def check_decode_call(rrs, sh, st, m, dx, vbar_dev, vbar_np, heads, units, o):
    """One teacher-forced decode call on the GPU, compared with the oracle's Lemma 2 step on
    `units`. Returns (max rel error of S~, max rel error of o)."""
    import torch
    pre = host_state(sh, st, units, m)
    rrs.seed_decode_step(sh, st, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar_dev, o)
    post = host_state(sh, st, units, m + 1)
    og = o.index_select(0, torch.as_tensor(list(units), device=o.device)).double().cpu().numpy()
    hx = host_inputs(dx, units)
    eS = eo = 0.0
    for i, u in enumerate(units):
        vb = vbar_np[u % heads]
        X = hx[i]
        a1, U1, V1, o1 = orc.factored_step(sh.kind, *pre[i], vb, X["q"], X["k"], X["v"], X["beta"], X["g"])
        S1 = orc.reconstruct(a1, vb, U1, V1)
        eS = max(eS, relF(orc.reconstruct(post[i][0], vb, post[i][1], post[i][2]), S1))
        eo = max(eo, rel_out(og[i], o1, S1, X["q"]))
    return eS, eo


def check_compress_call(rrs, sh, st, m, vbar_np, heads, units, code):
    """One compression call on the GPU, compared with the oracle's exact truncation of the
    same content on `units`. Returns (worst error per compare_compression, near-tie count);
    check_compress_call.last_raw / .last_sink hold the worst product and sink errors."""
    pre = host_state(sh, st, units, m)
    rrs.seed_compress(sh, st, m)
    post = host_state(sh, st, units, sh.rank)
    worst, ties, raw, sink = 0.0, 0, 0.0, 0.0
    for i, u in enumerate(units):
        vb = vbar_np[u % heads]
        kind, err, rw, sk = compare_compression((pre[i][1], pre[i][2]), post[i][0], vb, post[i][1],
                                                post[i][2], sh.rank, code, a_ref=pre[i][0])
        worst = max(worst, err)
        raw = max(raw, rw)
        sink = max(sink, sk)
        ties += kind == "optimal"
    check_compress_call.last_raw = raw
    check_compress_call.last_sink = sink
    return worst, ties


def check_from_dense_call(rrs, sh, S, vbar_dev, vbar_np, heads, units, code):
    """seed_state_from_dense on the GPU against the oracle's split + truncation of the same
    dense states. Returns (state, worst error, near-tie count); check_from_dense_call.last_sink
    holds the worst sink error |a - S vbar / |vbar|^2| / |S vbar / |vbar|^2|."""
    import torch
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar_dev, st)
    Sg = S.index_select(0, torch.as_tensor(list(units), device=S.device)).double().cpu().numpy()
    post = host_state(sh, st, units, sh.rank)
    worst, ties, sink = 0.0, 0, 0.0
    for i, u in enumerate(units):
        vb = vbar_np[u % heads]
        a_o, _, _, _ = orc.from_dense(Sg[i], vb, sh.rank)
        _, C = orc.sink_split(Sg[i], vb)
        kind, err, _, sk = compare_compression(C, post[i][0], vb, post[i][1], post[i][2], sh.rank, code,
                                               a_ref=a_o)
        worst = max(worst, err)
        sink = max(sink, sk)
        ties += kind == "optimal"
    check_from_dense_call.last_sink = sink
    return st, worst, ties
