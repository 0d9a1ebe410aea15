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
    return torch.bfloat16 if code == synth.BF16 else torch.float32


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


def host_state(shape, st, units, m: int):
    """Read back (a, U, V) in true (decay-folded) form, float64, for the given units.

    U columns: GDN / Mamba-2 fold the per-column scale (slot 0 for j < r, slot 1 + j - r
    after); KDA folds the per-channel Gamma.
    """
    import torch
    idx = torch.as_tensor(list(units), device=st.a.device)
    a = st.a.index_select(0, idx).double().cpu().numpy()
    Us = st.U.index_select(0, idx)[:, :m].double().cpu().numpy()
    Vs = st.V.index_select(0, idx)[:, :m].double().cpu().numpy()
    sc = st.scale.index_select(0, idx).double().cpu().numpy()
    out = []
    for n in range(len(units)):
        if shape.kind == synth.KDA:
            U = (Us[n] * sc[n][None, :]).T
        else:
            c = np.array([sc[n][0] if j < shape.rank else sc[n][1 + j - shape.rank] for j in range(m)])
            U = (Us[n] * c[:, None]).T
        out.append((a[n], U, Vs[n].T))
    return out


def relF(A, B):
    nb = np.linalg.norm(B)
    return float(np.linalg.norm(A - B) / nb) if nb > 0 else float(np.linalg.norm(A))


def tolerance(w_or_dtype) -> float:
    code = w_or_dtype.factor_dtype if hasattr(w_or_dtype, "factor_dtype") else w_or_dtype
    return 2e-2 if code == synth.BF16 else 1e-5


def near_tie_threshold(code) -> float:
    return 5e-2 if code == synth.BF16 else 1e-3


def compare_compression(C_before, a, vbar, U_gpu, V_gpu, r, code, a_ref=None):
    """Compare a GPU compression with the oracle's exact truncation of the same content.

    Returns (kind, err): kind "product" uses rel-Frobenius on S~; kind "optimal" (near ties)
    checks the Eckart-Young optimality criterion and returns the excess ratio.
    """
    Ur, Vr, _ = orc.compress(*C_before, r) if isinstance(C_before, tuple) else orc.truncate(C_before, r)
    C = C_before[0] @ C_before[1].T if isinstance(C_before, tuple) else C_before
    a_ref = a if a_ref is None else a_ref
    S_ref = orc.reconstruct(a_ref, vbar, Ur, Vr)
    S_gpu = orc.reconstruct(a, vbar, U_gpu, V_gpu)
    gap = orc.relative_gap(C, r)
    if gap < near_tie_threshold(code):
        ok = orc.truncation_is_optimal(C, U_gpu @ V_gpu.T, r, tolerance(code), abs_tol=tolerance(code) ** 2)
        return "optimal", (0.0 if ok else float("inf")), relF(S_gpu, S_ref)
    return "product", relF(S_gpu, S_ref), relF(S_gpu, S_ref)
