"""Compression of contents whose spectrum holds clusters of nearly equal singular values.

The compression kernel for 16-bit factors orthogonalises its eigenvectors only within clusters
of eigenvalues (runs of gaps at most 1e-3 of the largest eigenvalue); the vectors of well
separated eigenvalues are kept as the twisted factorisation leaves them. These tests plant
contents U V^T = Q_u diag(s) Q_v^T (random orthonormal Q_u, Q_v) whose kept singular values come
in groups 1e-4 apart, distinct values elsewhere, and a clear gap at the truncation rank, and
hold each compression to the oracle's exact truncation of the content the device holds (the
kept set contains the clusters whole, so the truncated product is unique).
"""
import numpy as np
import pytest

import synth
from gpu_util import check_compress_call, tolerance

pytestmark = pytest.mark.gpu

CASES = [
    # (d_k, d_v, r, T, factor dtype): the 64-wide core (r + T = 64) and the 32-wide one
    (128, 128, 32, 32, synth.BF16),
    (128, 128, 32, 32, synth.F16),
    (128, 64, 16, 16, synth.BF16),
    (128, 128, 16, 16, synth.F16),
]


def _spectrum(r, m, rng):
    """r kept singular values: groups of four 1e-4 apart, then distinct ones; m - r dropped
    ones well below (relative gap at r of about 0.15)."""
    kept = []
    base = 1.0
    while len(kept) < r // 2:
        kept += [base * (1.0 + 1e-4 * i) for i in range(4)]
        base *= 0.8
    kept = kept[: r // 2]
    kept += list(np.linspace(0.4 * base, 0.2, r - len(kept)))
    dropped = list(0.05 * rng.uniform(0.2, 1.0, m - r))
    return np.array(sorted(kept, reverse=True) + sorted(dropped, reverse=True))


@pytest.mark.parametrize("dk,dv,r,T,fdt", CASES)
def test_clustered_spectrum_compression(dk, dv, r, T, fdt):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs

    B, H = 2, 2
    units = B * H
    m = r + T
    sh = rrs.make_shape(synth.GDN, B, H, dk, dv, r, T, fdt, synth.BF16)
    st = rrs.State.empty(sh)
    rng = np.random.default_rng(7000 + dk + r + fdt)
    dt = torch.bfloat16 if fdt == synth.BF16 else torch.float16
    U = np.zeros((units, m, dk))
    V = np.zeros((units, m, dv))
    for u in range(units):
        s = _spectrum(r, m, rng)
        Qu, _ = np.linalg.qr(rng.standard_normal((dk, m)))
        Qv, _ = np.linalg.qr(rng.standard_normal((dv, m)))
        U[u] = (Qu * np.sqrt(s)).T
        V[u] = (Qv * np.sqrt(s)).T
    with torch.no_grad():
        st.U.zero_()
        st.V.zero_()
        st.U[:, :m] = torch.tensor(U).to(dt).to(st.U.device)
        st.V[:, :m] = torch.tensor(V).to(dt).to(st.V.device)
        st.a.copy_(torch.tensor(rng.standard_normal((units, dk)), dtype=torch.float32))
        sl = rrs.seed_scale_len(sh)
        sc = torch.zeros((units, sl), dtype=torch.float32)
        sc[:, : 1 + T] = 1.0                       # slot scales: no decay pending
        cnt = torch.tensor([0, m], dtype=torch.int32).view(torch.float32)
        sc[:, sl - 2] = cnt[0]                     # compression-window count
        sc[:, sl - 1] = cnt[1]                     # column count
        st.scale.copy_(sc)
    vbar = rng.standard_normal((H, dv))
    vbar /= np.linalg.norm(vbar, axis=1, keepdims=True)
    worst, ties = check_compress_call(rrs, sh, st, m, vbar, H, range(units), fdt)
    torch.cuda.synchronize()
    print(f"\n[clusters {dk}x{dv} r{r} T{T} {'bf16' if fdt == synth.BF16 else 'fp16'}] worst {worst:.2e} "
          f"(product {check_compress_call.last_raw:.2e}, sink {check_compress_call.last_sink:.2e}, "
          f"near-ties {ties})", flush=True)
    assert ties == 0
    assert worst <= tolerance(fdt)
