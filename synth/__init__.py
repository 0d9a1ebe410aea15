"""Seeded synthetic inputs for the sink + rank-r decode state.

This module only draws random inputs. It holds no step of the method's arithmetic, and both
the fp64 oracle's tests and the HIP path's tests and benchmark take their inputs from here.

Workloads. The method (Shallow Encoding Emits Deep Memories, picx.dev summary, "SEED
Architecture" and "Exact Update (Lemma 2)") acts on the d_k x d_v recurrent state of Gated
DeltaNet (GDN), Kimi Delta Attention (KDA) and Mamba-2 heads. The pages measure on exams and an
agentic-coding serving trace, which are not available here. These seeded synthetic workloads
stand in for that trace's decode phase, at the head shapes the pages' state table implies.

Per-step draws, per unit (one request x one head [x one layer]):

* GDN / KDA: q, k ~ N(0, I) then L2-normalised; v ~ N(0.5 * u_h, I) with u_h ~ N(0, I_dv)
  drawn once per head; beta ~ U(0, 1); gate alpha ~ U(0.9, 1) (a scalar for GDN, one value
  per key channel for KDA).
* Mamba-2: key side = B ~ N(0, I_dstate), query side = C ~ N(0, I_dstate) (not normalised),
  value side = x ~ N(0.5 * u_h, I_headdim); dt = softplus(N(0, 1)); A_h = -U(1, 16) per head;
  the decay handed to the library is exp(dt * A_h) and the input scale beta is dt.
* The head's mean-value direction handed to the library is vbar_h = u_h / |u_h|.

Units are ordered [layer][batch][head]; the head of unit i is i % heads.
"""
from __future__ import annotations

import dataclasses

import numpy as np

GDN, KDA, MAMBA2 = 0, 1, 2
KIND_NAMES = {GDN: "gdn", KDA: "kda", MAMBA2: "mamba2"}
F32, BF16, F16 = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode workload."""

    name: str
    kind: int
    batch: int
    heads: int
    d_k: int          # key side (GDN/KDA key dim, Mamba-2 d_state): the side of the sink a
    d_v: int          # value side (GDN/KDA value dim, Mamba-2 head dim)
    rank: int         # r
    period: int       # T: compress every T decode steps
    steps: int        # decode steps
    prefill: int      # dense tokens that build the initial state
    factor_dtype: int
    io_dtype: int
    layers: int = 1

    @property
    def units(self) -> int:
        return self.layers * self.batch * self.heads

    @property
    def max_cols(self) -> int:
        return self.rank + self.period

    def describe(self) -> str:
        kind = KIND_NAMES[self.kind]
        lay = f"{self.layers} layers x " if self.layers > 1 else ""
        dt = {F32: "fp32", BF16: "bf16", F16: "fp16"}[self.factor_dtype]
        return (f"{kind} {lay}{self.heads} heads x batch {self.batch}, d_k={self.d_k} d_v={self.d_v}, "
                f"r={self.rank} T={self.period}, {self.steps} steps, {dt} factors, "
                f"prefill {self.prefill} tokens")


WORKLOADS = {
    "gdn-tiny": Workload("gdn-tiny", GDN, 1, 1, 64, 64, 8, 8, 64, 32, F32, F32),
    "gdn-layer": Workload("gdn-layer", GDN, 64, 16, 128, 128, 16, 16, 256, 1024, BF16, BF16),
    "kda-layer": Workload("kda-layer", KDA, 256, 32, 128, 128, 32, 32, 512, 1024, BF16, BF16),
    "mamba2-layer": Workload("mamba2-layer", MAMBA2, 512, 64, 128, 64, 16, 16, 512, 1024, BF16, BF16),
    "gdn-stack36": Workload("gdn-stack36", GDN, 128, 32, 128, 128, 32, 32, 1024, 4096, BF16, BF16,
                            layers=36),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


@dataclasses.dataclass
class HeadConsts:
    u: np.ndarray       # [H, d_v] unnormalised value mean per head
    vbar: np.ndarray    # [H, d_v] unit direction handed to the library
    A: np.ndarray       # [H] Mamba-2 A_h (zeros for the other kinds)


def head_consts(w: Workload, seed: int, layers: int = 1) -> HeadConsts:
    """Per-head constants; with layers > 1, layer l's heads are rows l*heads .. (l+1)*heads-1."""
    g = rng(seed * 7919 + 11)
    nh = w.heads * layers
    u = g.standard_normal((nh, w.d_v))
    vbar = u / np.linalg.norm(u, axis=1, keepdims=True)
    A = -g.uniform(1.0, 16.0, size=nh) if w.kind == MAMBA2 else np.zeros(nh)
    return HeadConsts(u, vbar, A)


def unit_heads(w: Workload, units: int) -> np.ndarray:
    """Head-constant row of each unit for units ordered [layer][batch][head]."""
    i = np.arange(units)
    return (i // (w.batch * w.heads)) * w.heads + i % w.heads


def _softplus(x):
    return np.where(x > 20, x, np.log1p(np.exp(np.minimum(x, 20))))


def step_inputs(w: Workload, hc: HeadConsts, gen: np.random.Generator, units: int,
                unit_heads: np.ndarray | None = None) -> dict:
    """One decode step's inputs for `units` units (float64 numpy arrays).

    Returns q [n, d_k], k [n, d_k], v [n, d_v], beta [n], g [n] (KDA: [n, d_k]).
    """
    if unit_heads is None:
        unit_heads = np.arange(units) % w.heads
    q = gen.standard_normal((units, w.d_k))
    k = gen.standard_normal((units, w.d_k))
    if w.kind != MAMBA2:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = gen.standard_normal((units, w.d_v)) + 0.5 * hc.u[unit_heads]
    if w.kind == MAMBA2:
        dt = _softplus(gen.standard_normal(units))
        beta = dt
        g = np.exp(dt * hc.A[unit_heads])
    else:
        beta = gen.uniform(0.0, 1.0, size=units)
        if w.kind == KDA:
            g = gen.uniform(0.9, 1.0, size=(units, w.d_k))
        else:
            g = gen.uniform(0.9, 1.0, size=units)
    return {"q": q, "k": k, "v": v, "beta": beta, "g": g}


def sequence(w: Workload, seed: int, steps: int, units: int | None = None,
             unit_heads: np.ndarray | None = None) -> list:
    """`steps` consecutive step-input dicts from one seeded stream."""
    n = w.units if units is None else units
    gen = rng(seed)
    hc = head_consts(w, seed)
    return [step_inputs(w, hc, gen, n, unit_heads) for _ in range(steps)]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    Input preparation only: values that a bf16 buffer will hold, so that both sides see the
    same numbers.
    """
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    b = (b + 0x7FFF + lsb) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# Device-side generation for large workloads (torch generators on the GPU).
# ----------------------------------------------------------------------------------------------
class DeviceStream:
    """Draws the same distributions as `step_inputs` directly on a torch device.

    Separate generators per tensor family keep the draws reproducible for a given seed.
    """

    def __init__(self, w: Workload, seed: int, device, units: int | None = None):
        import torch

        self.torch = torch
        self.w = w
        self.n = w.units if units is None else units
        self.device = device
        hc = head_consts(w, seed, layers=w.layers)
        self.hc = hc
        self.unit_heads = torch.tensor(unit_heads(w, self.n), device=device)
        self.u = torch.tensor(hc.u, dtype=torch.float32, device=device)
        self.A = torch.tensor(hc.A, dtype=torch.float32, device=device)
        self.gens = {}
        for i, fam in enumerate(("q", "k", "v", "beta", "g")):
            gg = torch.Generator(device=device)
            gg.manual_seed(seed * 1000 + i)
            self.gens[fam] = gg

    def vbar(self, layer: int = 0):
        """[heads, d_v] mean-value directions of one layer."""
        t = self.torch
        h = self.w.heads
        return t.tensor(self.hc.vbar[layer * h:(layer + 1) * h], dtype=t.float32,
                        device=self.device).contiguous()

    def step(self, io_dtype, out: dict | None = None) -> dict:
        t = self.torch
        w, n, dev = self.w, self.n, self.device
        q = t.randn((n, w.d_k), generator=self.gens["q"], device=dev)
        k = t.randn((n, w.d_k), generator=self.gens["k"], device=dev)
        if w.kind != MAMBA2:
            q = q / q.norm(dim=1, keepdim=True)
            k = k / k.norm(dim=1, keepdim=True)
        v = t.randn((n, w.d_v), generator=self.gens["v"], device=dev) + 0.5 * self.u[self.unit_heads]
        if w.kind == MAMBA2:
            dt = t.nn.functional.softplus(t.randn((n,), generator=self.gens["beta"], device=dev))
            beta = dt
            g = t.exp(dt * self.A[self.unit_heads])
        else:
            beta = t.rand((n,), generator=self.gens["beta"], device=dev)
            shape = (n, w.d_k) if w.kind == KDA else (n,)
            g = 0.9 + 0.1 * t.rand(shape, generator=self.gens["g"], device=dev)
        res = {"q": q.to(io_dtype), "k": k.to(io_dtype), "v": v.to(io_dtype),
               "beta": beta.float(), "g": g.float()}
        if out is not None:
            for key, val in res.items():
                out[key].copy_(val)
            return out
        return res


def bytes_of(dtype_code: int) -> int:
    return 4 if dtype_code == F32 else 2


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [
    "GDN", "KDA", "MAMBA2", "F32", "BF16", "F16", "Workload", "WORKLOADS", "HeadConsts", "head_consts",
    "step_inputs", "sequence", "round_bf16", "DeviceStream", "rng", "bytes_of", "ceil_div",
    "unit_heads",
    "KIND_NAMES",
]
