"""fp64 oracle: dense recurrences, sink split, exact truncation, Lemma 2 factored step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import or run it. It is plain NumPy in float64, one unit at a
time, and shares no code with the HIP path.

Sources (all on the pages titled "Shallow Encoding Emits Deep Memories"):

* picx.dev summary, "SEED Architecture": the decode state is S = a vbar^T + U V^T, with vbar a
  fixed per-head direction, a the sink coefficient (d_k) and U (d_k x R), V (d_v x R) the
  content factors.
* picx.dev summary, "Exact Update (Lemma 2)": a+ = g a + beta (omega - g kappa^T a) kappa,
  U+ = [g U, kappa], V+ = [V, beta (eps - g V U^T kappa)], with omega = v^T vbar / |vbar|^2 and
  eps = v - omega vbar.
* picx.dev summary, "Theoretical and Practical Implications", Lemma 1: the sink coefficient and
  the content each follow the head's own recurrence, a_t = Phi_t a_{t-1} + beta omega kappa and
  C_t = Phi_t C_{t-1} + beta kappa eps^T, and the split is never recomputed.
* picx.dev summary, "Open-Loop Error Bound (Corollary 4)": |S~_t - S_t|_F <= eps_bar/(1-g_bar^W).
* thelatestinai.com figures & tables, overview table: both the read-out and the update work on
  the factors, a periodic compression brings them back to rank R, and a state leaving the
  prefill is first brought to the sink plus rank-R form.
* thelatestinai.com figures & tables, state table (State at R / mean / peak, MB) and the
  accounting table ("Shallow state": the sink's coefficient and the factors are counted, the
  mean direction is not).

Readings where the pages are silent (each listed in the design notes):

* Dense recurrences (the pages never print them; these are the forms whose factorisation is
  Lemma 2): GDN S+ = g S + beta kappa (v - g S^T kappa)^T; KDA the same with g replaced by the
  diagonal gate Diag(alpha) acting on the key side; Mamba-2 S+ = g S + beta kappa v^T with
  kappa = B, v = x, beta = dt, g = exp(dt A).
* The read-out is taken after the update: o = S+^T q.
* Compression is the best rank-r approximation of the content U V^T (Eckart-Young), with
  sqrt(sigma) on both factors; the sink coefficient a is not touched by a compression.

Conventions: S is d_k x d_v; U is d_k x m and V is d_v x m (columns are the rank-one terms);
kind 0 = GDN, 1 = KDA, 2 = Mamba-2; g is a scalar (GDN, Mamba-2) or a d_k vector (KDA).
"""
from __future__ import annotations

import numpy as np

GDN, KDA, MAMBA2 = 0, 1, 2

__all__ = [
    "GDN", "KDA", "MAMBA2", "decay", "dense_step", "readout", "sink_split", "truncate",
    "factored_step", "factored_chunk", "compress", "from_dense", "reconstruct", "decay_bound",
    "corollary4_bound", "run_dense", "run_factored", "run_compressed", "singular_values",
    "relative_gap", "truncation_is_optimal", "state_bytes", "dense_state_bytes", "state_energy",
    "content_spectrum", "silu", "head_norm",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def decay(kind: int, g, X):
    """Apply the decay operator G to X (a vector of length d_k or a d_k x n matrix).

    GDN and Mamba-2: G = g I (scalar). KDA: G = Diag(alpha), one gate per key channel, i.e.
    per row of the d_k x d_v state (Lemma 2 with g replaced by the diagonal gate).
    """
    X = _f64(X)
    if kind == KDA:
        gv = _f64(g)
        return gv[:, None] * X if X.ndim == 2 else gv * X
    return float(g) * X


def readout(S, q):
    """o = S^T q: the value-side read-out of a d_k x d_v state for query q."""
    return _f64(S).T @ _f64(q)


def dense_step(kind: int, S, q, kappa, v, beta, g):
    """One dense recurrent step and its read-out (oracle step O1).

    Delta kinds (GDN, KDA): S+ = G S + beta kappa (v - (G S)^T kappa)^T.
    Mamba-2:                S+ = g S + beta kappa v^T.
    Returns (S+, o) with o = S+^T q.
    """
    S = _f64(S)
    kappa = _f64(kappa)
    v = _f64(v)
    Sd = decay(kind, g, S)
    if kind == MAMBA2:
        Sn = Sd + float(beta) * np.outer(kappa, v)
    else:
        err = v - Sd.T @ kappa          # value minus what the decayed state predicts
        Sn = Sd + float(beta) * np.outer(kappa, err)
    return Sn, readout(Sn, q)


def sink_split(S, vbar):
    """Sink split of a dense state (oracle step O2; Lemma 1).

    a = S vbar / |vbar|^2 and C = S - a vbar^T, so that S = a vbar^T + C and C vbar = 0.
    """
    S = _f64(S)
    vbar = _f64(vbar)
    a = S @ vbar / (vbar @ vbar)
    return a, S - np.outer(a, vbar)


def truncate(C, r: int):
    """Best rank-r approximation of C as balanced factors (oracle step O3).

    Full SVD C = sum_i sigma_i y_i z_i^T (sigma descending). U = [sqrt(sigma_i) y_i]_{i<r},
    V = [sqrt(sigma_i) z_i]_{i<r}, zero columns where C has fewer than r singular values.
    Returns (U, V, err) with err = (sum_{i>=r} sigma_i^2)^(1/2) = |C - U V^T|_F.
    """
    C = _f64(C)
    dk, dv = C.shape
    Y, s, Zt = np.linalg.svd(C, full_matrices=False)
    kept = min(r, s.size)
    U = np.zeros((dk, r))
    V = np.zeros((dv, r))
    rs = np.sqrt(s[:kept])
    U[:, :kept] = Y[:, :kept] * rs
    V[:, :kept] = Zt[:kept].T * rs
    err = float(np.sqrt(np.sum(s[kept:] ** 2)))
    return U, V, err


def reconstruct(a, vbar, U, V):
    """Dense form of a factored state: S~ = a vbar^T + U V^T."""
    S = np.outer(_f64(a), _f64(vbar))
    U = _f64(U)
    if U.shape[1]:
        S = S + U @ _f64(V).T
    return S


def factored_step(kind: int, a, U, V, vbar, q, kappa, v, beta, g):
    """Lemma 2 factored step with read-out (oracle step O4).

    1. omega = v^T vbar / |vbar|^2, eps = v - omega vbar (value split along vbar).
    2. a_d = G a, U_d = G U (decay).
    3. Delta kinds: a+ = a_d + beta (omega - kappa^T a_d) kappa, w = beta (eps - V U_d^T kappa).
       Mamba-2 (no delta term): a+ = a_d + beta omega kappa, w = beta eps.
    4. U+ = [U_d, kappa], V+ = [V, w]: one appended column each.
    5. o = vbar (a+^T q) + V+ (U+^T q).
    Returns (a+, U+, V+, o).
    """
    a = _f64(a)
    U = _f64(U)
    V = _f64(V)
    vbar = _f64(vbar)
    q = _f64(q)
    kappa = _f64(kappa)
    v = _f64(v)
    beta = float(beta)
    omega = (v @ vbar) / (vbar @ vbar)
    eps = v - omega * vbar
    a_d = decay(kind, g, a)
    U_d = decay(kind, g, U)
    if kind == MAMBA2:
        a_new = a_d + beta * omega * kappa
        w = beta * eps
    else:
        a_new = a_d + beta * (omega - kappa @ a_d) * kappa
        w = beta * (eps - V @ (U_d.T @ kappa))
    U_new = np.concatenate([U_d, kappa[:, None]], axis=1)
    V_new = np.concatenate([V, w[:, None]], axis=1)
    o = vbar * (a_new @ q) + V_new @ (U_new.T @ q)
    return a_new, U_new, V_new, o


def compress(U, V, r: int):
    """Compression of the content back to rank r (oracle step O5).

    The plain definition: the best rank-r approximation of the content U V^T, by a dense SVD
    (truncate). The sink coefficient is not touched. Returns (U', V', err).
    """
    U = _f64(U)
    V = _f64(V)
    C = U @ V.T if U.shape[1] else np.zeros((U.shape[0], V.shape[0]))
    return truncate(C, r)


def from_dense(S, vbar, r: int):
    """Prefill-end compression of a dense state: sink split then rank-r truncation (O2 + O3)."""
    a, C = sink_split(S, vbar)
    U, V, err = truncate(C, r)
    return a, U, V, err


def decay_bound(kind: int, g) -> float:
    """Spectral-norm bound of one step's transition Phi_t (for Corollary 4's g_bar).

    GDN: |g (I - beta kappa kappa^T)|_2 <= g when 0 <= beta |kappa|^2 <= 2.
    KDA: |(I - beta kappa kappa^T) Diag(alpha)|_2 <= max_i alpha_i under the same condition.
    Mamba-2: Phi = g I.
    """
    return float(np.max(_f64(g)))


def corollary4_bound(eps_bar: float, g_bar: float, W: int) -> float:
    """Open-loop bound eps_bar / (1 - g_bar^W) of Corollary 4 (W = steps between compressions)."""
    return eps_bar / (1.0 - g_bar ** W)


def run_dense(kind: int, S0, inputs: list):
    """Dense trajectory from S0 over a list of step dicts (keys q, k, v, beta, g).

    Returns (states, outputs): S_t and o_t after each step.
    """
    S = _f64(S0).copy()
    states, outs = [], []
    for x in inputs:
        S, o = dense_step(kind, S, x["q"], x["k"], x["v"], x["beta"], x["g"])
        states.append(S)
        outs.append(o)
    return states, outs


def run_factored(kind: int, a0, U0, V0, vbar, inputs: list):
    """Factored trajectory with no compression (m grows by one per step)."""
    a, U, V = _f64(a0).copy(), _f64(U0).copy(), _f64(V0).copy()
    traj = []
    for x in inputs:
        a, U, V, o = factored_step(kind, a, U, V, vbar, x["q"], x["k"], x["v"], x["beta"], x["g"])
        traj.append((a, U, V, o))
    return traj


def factored_chunk(kind: int, a, U, V, vbar, inputs: list):
    """A chunk of tokens on the factored state: the Lemma 2 step of each token in turn.

    A chunked update is defined by the steps it stands for (picx.dev summary, "Exact Update
    (Lemma 2)"; Lemma 1: the sink and the content follow the head's recurrence token by token),
    so the oracle is the plain loop. Returns (a, U, V, outputs) after the last token; U and V
    hold one more column per token, and outputs[t] is token t's read-out.
    """
    a, U, V = _f64(a).copy(), _f64(U).copy(), _f64(V).copy()
    outs = []
    for x in inputs:
        a, U, V, o = factored_step(kind, a, U, V, vbar, x["q"], x["k"], x["v"], x["beta"], x["g"])
        outs.append(o)
    return a, U, V, outs


def run_compressed(kind: int, S0, vbar, inputs: list, r: int, T: int):
    """Oracle driver (step O6): exact and compressed trajectories from one dense state.

    The dense state S0 is compressed at the end of the prefill (sink split + rank-r
    truncation). Then, for each step t = 1..N, the exact path takes a dense step and the
    compressed path takes a Lemma 2 step, followed by a compression to rank r after the read-out
    whenever t is a multiple of T.

    Returns a dict with per-step exact outputs o, compressed outputs o_c, the dense form S~_t of
    the compressed state, the exact S_t, the list of compression errors (the prefill-end one
    first) and the per-step transition bounds.
    """
    S = _f64(S0).copy()
    a, U, V, err0 = from_dense(S, vbar, r)
    errs = [err0]
    out = {"o": [], "o_c": [], "S": [], "S_c": [], "errs": errs, "g_bound": []}
    for t, x in enumerate(inputs, start=1):
        S, o = dense_step(kind, S, x["q"], x["k"], x["v"], x["beta"], x["g"])
        a, U, V, oc = factored_step(kind, a, U, V, vbar, x["q"], x["k"], x["v"], x["beta"], x["g"])
        if t % T == 0:
            U, V, e = compress(U, V, r)
            errs.append(e)
        out["o"].append(o)
        out["o_c"].append(oc)
        out["S"].append(S)
        out["S_c"].append(reconstruct(a, vbar, U, V))
        out["g_bound"].append(decay_bound(kind, x["g"]))
    out["final"] = (a, U, V)
    return out


def singular_values(C):
    return np.linalg.svd(_f64(C), compute_uv=False)


def relative_gap(C, r: int) -> float:
    """(sigma_r - sigma_{r+1}) / sigma_1 of C (1-based sigma), 1.0 when C has rank <= r."""
    s = singular_values(C)
    if s.size <= r or s[0] == 0.0:
        return 1.0
    return float((s[r - 1] - s[r]) / s[0])


def truncation_is_optimal(C, Ct, r: int, delta: float, abs_tol: float = 1e-12,
                          rank_tol: float = 1e-6) -> bool:
    """Optimality test for a candidate rank-r truncation Ct of C.

    When sigma_r and sigma_{r+1} (nearly) tie, several rank-r truncations are correct. Any Ct
    of rank <= r with |C - Ct|_F^2 <= (1 + delta) sum_{i>r} sigma_i^2 is accepted; abs_tol
    (relative to |C|_F^2) absorbs rounding when the tail is zero.
    """
    C = _f64(C)
    Ct = _f64(Ct)
    s = singular_values(C)
    tail = float(np.sum(s[r:] ** 2))
    st = singular_values(Ct)
    if st.size > r and st[r] > rank_tol * max(st[0], 1e-300):
        return False
    resid = float(np.sum((C - Ct) ** 2))
    scale = float(np.sum(s ** 2))
    return resid <= (1.0 + delta) * tail + abs_tol * scale


def state_bytes(n_heads: int, d_k: int, d_v: int, m: float, bytes_per: int = 4) -> float:
    """Bytes of a shallow state: the sink coefficient and m columns of each factor per head.

    The mean direction vbar is shared by all requests and is not counted (thelatestinai.com
    figures & tables, accounting table, "Shallow state").
    """
    return bytes_per * n_heads * (d_k + (d_k + d_v) * m)


def dense_state_bytes(n_heads: int, d_k: int, d_v: int, bytes_per: int = 4) -> float:
    """Bytes of the dense recurrent states: one d_k x d_v matrix per head."""
    return bytes_per * n_heads * d_k * d_v


def state_energy(a, vbar, U, V):
    """(|S~|_F^2, |a vbar^T|_F^2, |U V^T|_F^2) of S~ = a vbar^T + U V^T, from the explicit
    matrices. picx.dev summary, key finding 2 and "Introduction and Theoretical Foundation": the
    state sink's share of the state energy is the sink term's squared Frobenius norm over the
    whole state's."""
    a, vbar, U, V = _f64(a), _f64(vbar), _f64(U), _f64(V)
    sink = np.outer(a, vbar)
    content = U @ V.T
    S = sink + content
    return float(np.sum(S * S)), float(np.sum(sink * sink)), float(np.sum(content * content))


def content_spectrum(U, V, k: int = 32):
    """Rank-energy spectrum of the content C = U V^T: (sigma_1^2 .. sigma_k^2, |C|_F^2).

    picx.dev summary, key finding 2, and thelatestinai.com figures & tables, overview table:
    after the sink, the rest of the state is low-rank, i.e. its energy sits in few singular
    directions. The squared singular values, largest first (zeros past the rank), and the total
    squared Frobenius norm, from the explicit matrix.
    """
    C = _f64(U) @ _f64(V).T
    s = np.linalg.svd(C, compute_uv=False) if C.size else np.zeros(0)
    out = np.zeros(k)
    n = min(k, s.size)
    out[:n] = s[:n] ** 2
    return out, float(np.sum(C * C))


def silu(z):
    """z * sigmoid(z), the gate of a gated head normalisation."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def head_norm(o, weight, eps: float, gate=None, gate_first: bool = False):
    """Per-head RMS normalisation of a read-out, with a weight and an optional gate.

    picx.dev summary, "Theoretical and Practical Implications", practical implications: the
    state sink acts as a bias and gain through the head's normalization. The pages do not print
    the normalisation; this is the plain RMS form of the models named there (Gated DeltaNet,
    Kimi Delta Attention and Mamba-2 heads normalise their d_v read-out by its root mean square
    and a learned per-channel weight, optionally gated):
        x = o, or o * silu(gate) when the gate comes first (Mamba-2's gated norm);
        y = x / sqrt(mean(x^2) + eps) * weight, then * silu(gate) when the gate comes after.
    With o = vbar (a^T q) + V (U^T q), the sink term is a fixed-direction bias inside the norm,
    and its energy sets the gain 1 / rms that the content receives.
    """
    x = _f64(o)
    if gate is not None and gate_first:
        x = x * silu(gate)
    rms = np.sqrt(np.mean(x * x) + float(eps))
    y = x / rms * _f64(weight)
    if gate is not None and not gate_first:
        y = y * silu(gate)
    return y
