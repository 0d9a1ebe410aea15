#!/usr/bin/env python3
"""Benchmark of the sink + rank-r decode state on one MI355X.

Metric: factored decode head-steps/s and achieved HBM GB/s (as a fraction of the 8 TB/s HBM3E
roofline), against the dense-state kernel. Default workload: a deep hybrid decode stack of 36
Gated DeltaNet layers x 32 heads x 128 requests, d_k = d_v = 128, sink + rank r = 32,
compression every T = 32 steps, bf16 factors with fp32 arithmetic. Dense states are built from
4096 seeded tokens and compressed at the end of the prefill (both untimed), then the decode is
timed.

One step = one decode step of every layer (one launch per layer, as in a served model where the
rest of the layer stack runs between two steps of a layer), plus, every T-th step, the
compression of every layer (one launch per layer). The timed region holds exactly --steps
steps after --warmup untimed ones, bracketed by torch.cuda.synchronize(); inputs are resident
in HBM (a pool of --pool steps of seeded inputs, cycled).

Algorithmic bytes per unit-step of the decode at m columns (what the method must move):
  read the sink a (4 d_k), U and V (f (d_k + d_v) m), q, k, v (e (2 d_k + d_v)), beta and g
  (4 + 4 or 4 d_k); write a (4 d_k), the new column pair (f (d_k + d_v)) and o (e d_v).
  f = factor bytes, e = activation bytes; the lazy decay scales and vbar are not credited.
  The roofline fraction is taken on these bytes. The kernel's own accounting is reported
  beside it: the sink is lazy (a step adds a multiple of its key to a, and the key is the
  column it appends to U, so a step stores that multiple and a is rebuilt only at
  compression), so it reads a_0 and the window's m - r coefficients and writes one float in
  place of a.
Timing: whole compression windows (T decode steps of every layer, then the compression),
at least five of them whatever --steps asks; the median and the spread over the windows are
reported beside the total.
Dense step per unit: 8 d_k d_v (fp32 state read and written) + inputs + o.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Measured HBM traffic of the decode kernel (two rocprofv3 counter runs, scaled by a calibration
# copy); used only while the kernel sources still hash to the digest recorded with it.
def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"k_decode_{workload}_hbm_traffic.txt")
DECODE_SOURCES = ("rank_recurrent_state_amd/csrc/decode.hip", "rank_recurrent_state_amd/csrc/common.hpp",
                  "rank_recurrent_state_amd/csrc/kernels.hpp")
MIN_WINDOWS = 5
METRIC = "factored decode head-steps/s + achieved HBM GB/s (% roofline) vs dense-state kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=32, help="untimed decode steps first")
    ap.add_argument("--workload", default="gdn-stack36")
    ap.add_argument("--factor-dtype", choices=["fp32", "bf16", "fp16"], default=None,
                    help="factor storage other than the workload's own (fp16: with bf16 inputs)")
    ap.add_argument("--no-diagnostics", action="store_true",
                    help="skip everything after the timed steps except the dense baseline (the "
                         "energy, spectrum, chunked-update and overlapped-schedule measurements), "
                         "so that a profile holds only the step's kernels and the baseline")
    ap.add_argument("--overlap-split", type=int, default=4,
                    help="XCDs (of 8) that run the decode in the overlapped schedule; the "
                         "compressions run on the others")
    ap.add_argument("--compress-scan", action="store_true",
                    help="with --staggered: compress with seed_compress_ragged (a wave per unit of "
                         "the stack) instead of listing the units that fill (seed_compress_units)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the overlapped-schedule measurement (decode and compression on "
                         "disjoint XCDs, compressions shifted per layer)")
    ap.add_argument("--rounding", choices=["nearest", "stochastic"], default="nearest",
                    help="rounding of the 16-bit factor stores")
    ap.add_argument("--staggered", action="store_true",
                    help="requests at staggered column counts (request b at r + b mod T): ragged "
                         "decode steps, each followed by a compression of the units that filled")
    ap.add_argument("--stagger-group", type=int, default=1024,
                    help="with --staggered: full units per compression launch in the overlapped schedule")
    ap.add_argument("--pool", type=int, default=64, help="steps of resident inputs, cycled")
    ap.add_argument("--dense-steps", type=int, default=32, help="timed dense-baseline steps")
    ap.add_argument("--prefill", type=int, default=None, help="override the prefill length")
    ap.add_argument("--cpu-units", type=int, default=8192, help="units in the oracle CPU sample (layer-major)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--seed", type=int, default=1005)
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--compress-per-layer", action="store_true",
                    help="one compression launch per layer instead of one over the whole stack")
    ap.add_argument("--source-digest", action="store_true",
                    help="print the digest of the decode kernel sources and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (scales HBM byte counters under a profiler)")
    return ap.parse_args()


def decode_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """Bytes per decode launch from the counter profile, if it matches the current sources."""
    try:
        with open(traffic_file(workload)) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != decode_source_digest() or kv.get("workload") != workload:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def decode_bytes(w, m: int) -> int:
    f = 2 if w.factor_dtype else 4
    e = 2 if w.io_dtype else 4
    gb = 4 * w.d_k if w.kind == 1 else 4
    return (4 * w.d_k + 4 * (m - w.rank) + f * (w.d_k + w.d_v) * m + e * (2 * w.d_k + w.d_v)
            + 4 + gb + 4 + f * (w.d_k + w.d_v) + e * w.d_v)


def decode_bytes_alg(w, m: int) -> int:
    """The algorithmic bytes of one unit-step as the hot-path table defines them: read a (4 d_k),
    U and V (f (d_k + d_v) m), q, k, v and beta, g; write a (4 d_k), the new column pair and o.
    The lazy sink moves fewer bytes than this (it writes one coefficient instead of a, and
    reads the window's coefficients), so the fraction on these bytes is the one reported."""
    f = 2 if w.factor_dtype else 4
    e = 2 if w.io_dtype else 4
    gb = 4 * w.d_k if w.kind == 1 else 4
    return (4 * w.d_k + f * (w.d_k + w.d_v) * m + e * (2 * w.d_k + w.d_v) + 4 + gb
            + 4 * w.d_k + f * (w.d_k + w.d_v) + e * w.d_v)


def compress_bytes(w, m: int) -> int:
    f = 2 if w.factor_dtype else 4
    return f * (w.d_k + w.d_v) * (m + w.rank)


def dense_bytes(w) -> int:
    e = 2 if w.io_dtype else 4
    gb = 4 * w.d_k if w.kind == 1 else 4
    return 8 * w.d_k * w.d_v + e * (2 * w.d_k + w.d_v) + 4 + gb + e * w.d_v


def host_cpu() -> dict:
    """The host's CPU model, its logical CPU count, and the share this process may use: the CPUs
    in its affinity mask, at most 16 (the host cores allotted to one GPU)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cpus = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = cpus
    return {"model": model, "cpus": cpus, "share": max(1, min(16, avail))}


def cpu_worker(job):
    """Oracle (fp64) on a shard of units: one compression window of decode steps plus the
    compression, from host copies of the GPU's states and inputs."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as orc

    kind, r, T, states, inputs, vbars = job
    t0 = time.perf_counter()
    with threadpool_limits(1):
        for (a, U, V), xs, vb in zip(states, inputs, vbars):
            for x in xs:
                a, U, V, _ = orc.factored_step(kind, a, U, V, vb, x["q"], x["k"], x["v"], x["beta"], x["g"])
            U, V, _ = orc.compress(U, V, r)
    _ = np
    return time.perf_counter() - t0


def main():
    args = parse()
    if args.source_digest:
        print(decode_source_digest())
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              "data-parallel over independent units and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rank_recurrent_state_amd as rrs
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    if args.factor_dtype is not None:
        fd = {"fp32": synth.F32, "bf16": synth.BF16, "fp16": synth.F16}[args.factor_dtype]
        w = dataclasses.replace(w, factor_dtype=fd,
                                io_dtype=synth.BF16 if fd == synth.F16 else (w.io_dtype if fd else synth.F32))
    prefill = w.prefill if args.prefill is None else args.prefill
    L = w.layers
    U1 = w.batch * w.heads           # units per launch (one layer)
    N = L * U1
    C = w.rank + w.period
    torch_dt = {synth.F32: torch.float32, synth.BF16: torch.bfloat16, synth.F16: torch.float16}
    io = torch_dt[w.io_dtype]
    fdt = torch_dt[w.factor_dtype]
    rnd = rrs.SEED_ROUND_STOCHASTIC if args.rounding == "stochastic" else rrs.SEED_ROUND_NEAREST
    # stochastic rounding's keys: the per-layer launches index units from 0 in every layer, so
    # each layer takes its own key; the stack-wide compression indexes all units at once
    sh_l = [rrs.make_shape(w.kind, w.batch, w.heads, w.d_k, w.d_v, w.rank, w.period,
                           w.factor_dtype, w.io_dtype, rounding=rnd, rng_key=args.seed * 1000 + l)
            for l in range(L)]
    sh = sh_l[0]
    sh_all = rrs.make_shape(w.kind, w.batch * L, w.heads, w.d_k, w.d_v, w.rank, w.period,
                            w.factor_dtype, w.io_dtype, rounding=rnd, rng_key=args.seed * 1000 + L)
    log(f"[bench] {w.describe()}; {N} units ({L} launches of {U1} per step); {rrs.seed_version()}")

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] calibration copy: 1 GiB read + 1 GiB written")

    # ---- setup (untimed): dense prefill, prefill-end compression, resident input pool -------
    ds = synth.DeviceStream(w, args.seed, dev)
    S = torch.zeros((N, w.d_k, w.d_v), dtype=torch.float32, device=dev)
    o_all = torch.empty((N, w.d_v), dtype=io, device=dev)
    t0 = time.time()
    for t in range(prefill):
        x = ds.step(io)
        rrs.seed_dense_decode_step(sh_all, S, x["q"], x["k"], x["v"], x["beta"], x["g"], o_all)
        if (t + 1) % 512 == 0:
            torch.cuda.synchronize()
            log(f"[bench] dense prefill {t + 1}/{prefill} tokens ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    log(f"[bench] dense prefill done in {time.time() - t0:.1f} s")

    a = torch.zeros((N, w.d_k), dtype=torch.float32, device=dev)
    Uf = torch.zeros((N, C, w.d_k), dtype=fdt, device=dev)
    Vf = torch.zeros((N, C, w.d_v), dtype=fdt, device=dev)
    scale = torch.ones((N, rrs.seed_scale_len(sh)), dtype=torch.float32, device=dev)
    states = [rrs.State(a[l * U1:(l + 1) * U1], Uf[l * U1:(l + 1) * U1], Vf[l * U1:(l + 1) * U1],
                        scale[l * U1:(l + 1) * U1]) for l in range(L)]
    vbars = [ds.vbar(l) for l in range(L)]
    t0 = time.time()
    for l in range(L):
        rrs.seed_state_from_dense(sh_l[l], S[l * U1:(l + 1) * U1], vbars[l], states[l])
        if L > 1 and (l + 1) % 6 == 0:
            torch.cuda.synchronize()
            log(f"[bench] prefill-end compression {l + 1}/{L} layers ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    t_from_dense = time.time() - t0
    log(f"[bench] prefill-end compression done in {t_from_dense:.1f} s")

    T = w.period
    K = max(-(-args.steps // T), MIN_WINDOWS) * T   # whole compression windows, at least five
    Wu = -(-args.warmup // T) * T
    if K != args.steps or Wu != args.warmup:
        log(f"[bench] steps/warmup rounded up to whole windows of T={T} (at least {MIN_WINDOWS} timed): {K}/{Wu}")
    nwin = max(1, min(args.pool // T, (Wu + K) // T))
    P = nwin * T
    pool = []
    for p in range(P):
        x = ds.step(io)
        pool.append([{k: v[l * U1:(l + 1) * U1].contiguous() for k, v in x.items()} for l in range(L)])
    torch.cuda.synchronize()
    o = [torch.empty((U1, w.d_v), dtype=io, device=dev) for _ in range(L)]
    log(f"[bench] input pool: {P} steps resident ({nwin} windows)")

    # host copies for the CPU baseline (taken before the decode touches the states)
    cpu_job = None
    if not args.no_cpu:
        # the first ns units of the stack: whole layers 0, 1, ... (units are layer-major)
        ns = min(args.cpu_units, N)
        nl = -(-ns // U1)
        ah = a[:ns].double().cpu().numpy()
        Uh = Uf[:ns, :w.rank].double().cpu().numpy()
        Vh = Vf[:ns, :w.rank].double().cpu().numpy()
        xs_h = []
        for p in range(T):
            xs_h.append({k: torch.cat([pool[p % P][l][k] for l in range(nl)])[:ns].double().cpu().numpy()
                         for k in pool[p % P][0]})
        vb_h = [vbars[l].double().cpu().numpy() for l in range(nl)]
        cpu_job = (ah, Uh, Vh, xs_h, vb_h, ns)

    def enqueue_window(wi):
        """T decode steps (one launch per layer per step), columns r .. r+T-1 before each."""
        for j in range(T):
            xl = pool[wi * T + j]
            for l in range(L):
                x = xl[l]
                rrs.seed_decode_step(sh_l[l], states[l], w.rank + j, x["q"], x["k"], x["v"], x["beta"],
                                     x["g"], vbars[l], o[l])

    # Every layer reaches r + T columns on the same step, and the layers' states are contiguous,
    # so one compression launch covers the stack (per layer on request).
    state_all = rrs.State(a, Uf, Vf, scale)
    cmp_calls = L if args.compress_per_layer else 1

    def enqueue_compress():
        if args.compress_per_layer:
            for l in range(L):
                rrs.seed_compress(sh_l[l], states[l], w.rank + T)
        else:
            rrs.seed_compress(sh_all, state_all, w.rank + T)

    if args.staggered:
        return run_staggered(args, rrs, torch, w, sh_l, sh_all, states, state_all, pool, vbars, o,
                             prefill, N, U1, L, T, P, nwin, Wu, K)

    for i in range(Wu // T):               # eager warmup (also the first launch of every kernel)
        enqueue_window(i % nwin)
        enqueue_compress()
    torch.cuda.synchronize()
    log(f"[bench] warmup {Wu} steps done")

    graphs = not args.eager
    if graphs:
        g_dec = []
        for wi in range(nwin):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                enqueue_window(wi)
            g_dec.append(g)
        g_cmp = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_cmp):
            enqueue_compress()
        torch.cuda.synchronize()
        log(f"[bench] captured {nwin} decode-window graphs ({T * L} launches each) and a "
            f"compression graph ({cmp_calls} launches)")

    # ---- timed region: K steps = K / T windows of (T decode steps, then the compressions) ---
    nw = K // T
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [(ev(), ev(), ev()) for _ in range(nw)]
    e_begin, e_end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e_begin.record()
    for i in range(nw):
        wi = (Wu // T + i) % nwin
        evs[i][0].record()
        if graphs:
            g_dec[wi].replay()
        else:
            enqueue_window(wi)
        evs[i][1].record()
        if graphs:
            g_cmp.replay()
        else:
            enqueue_compress()
        evs[i][2].record()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t_total = e_begin.elapsed_time(e_end) / 1e3
    t_dec = sum(a_.elapsed_time(b_) for a_, b_, _ in evs) / 1e3
    t_cmp = sum(b_.elapsed_time(c_) for _, b_, c_ in evs) / 1e3
    n_dec_launch = K * L
    n_cmp_launch = nw * cmp_calls
    dec_bytes = nw * L * U1 * sum(decode_bytes_alg(w, w.rank + j) for j in range(T))
    dec_bytes_own = nw * L * U1 * sum(decode_bytes(w, w.rank + j) for j in range(T))
    win_ms = sorted(a_.elapsed_time(c_) / T for a_, _, c_ in evs)        # ms per step, per window
    win_dec_us = sorted(a_.elapsed_time(b_) * 1e3 / (T * L) for a_, b_, _ in evs)
    win_cmp_ms = sorted(b_.elapsed_time(c_) for _, b_, c_ in evs)
    median = lambda xs: (xs[(len(xs) - 1) // 2] + xs[len(xs) // 2]) / 2  # noqa: E731
    windows = {"count": nw, "steps_each": T,
               "ms_per_step": {"median": median(win_ms), "min": win_ms[0], "max": win_ms[-1]},
               "decode_us_per_launch": {"median": median(win_dec_us), "min": win_dec_us[0],
                                        "max": win_dec_us[-1]},
               "compress_ms_per_window": {"median": median(win_cmp_ms), "min": win_cmp_ms[0],
                                          "max": win_cmp_ms[-1]}}
    cmp_bytes = nw * N * compress_bytes(w, w.rank + T)
    head_steps = N * K
    value = head_steps / t_total
    dec_gbs = dec_bytes / t_dec / 1e9
    used_cmp = list(range(nw))
    log(f"[bench] timed {K} steps: {t_total * 1e3:.1f} ms (wall {wall * 1e3:.1f} ms); decode "
        f"{t_dec * 1e3:.1f} ms over {n_dec_launch} launches ({dec_gbs:.0f} GB/s), compress "
        f"{t_cmp * 1e3:.1f} ms over {n_cmp_launch} launches")
    log(f"[bench] {nw} windows: {windows['ms_per_step']['median']:.3f} ms per step median "
        f"({win_ms[0]:.3f} .. {win_ms[-1]:.3f}); decode {windows['decode_us_per_launch']['median']:.2f} us "
        f"per launch median ({win_dec_us[0]:.2f} .. {win_dec_us[-1]:.2f}); compression "
        f"{windows['compress_ms_per_window']['median']:.2f} ms per window median")

    # ---- the state-energy diagnostic (not part of a step): one launch per layer ----------------
    diag = not args.no_diagnostics
    m_now = int(rrs.column_counts(sh_l[0], states[0])[0])
    energy = None
    if diag:
        energy = energy_diagnostic(rrs, torch, w, sh, sh_l, states, vbars, U1, L, N, m_now, dev, ev, log)
    # ---- the content spectrum (not part of a step): one launch per layer ------------------------
    spectrum = None
    if diag and w.factor_dtype != rrs.SEED_F32 and w.rank <= 32:
        sp_out = [torch.empty((U1, rrs.SEED_SPECTRUM_LEN), dtype=torch.float32, device=dev) for _ in range(L)]
        for l in range(L):
            rrs.seed_state_spectrum(sh_l[l], states[l], out=sp_out[l])
        s_a, s_b = ev(), ev()
        torch.cuda.synchronize()
        s_a.record()
        for l in range(L):
            rrs.seed_state_spectrum(sh_l[l], states[l], out=sp_out[l])
        s_b.record()
        torch.cuda.synchronize()
        t_sp = s_a.elapsed_time(s_b) / 1e3
        tot_c = float(sum(x[:, 32].double().sum() for x in sp_out))
        kept = {k: float(sum(x[:, :k].double().sum() for x in sp_out)) / tot_c for k in (1, 4, 16)}
        spectrum = {"ms_per_stack": t_sp * 1e3, "columns": m_now,
                    "content_energy_share_top_k": {str(k): v for k, v in kept.items()}}
        log(f"[bench] content spectrum: {t_sp * 1e3:.2f} ms over the stack at m = {m_now}; share of the "
            f"content energy in the top 1 / 4 / 16 directions: {kept[1]:.3f} / {kept[4]:.3f} / {kept[16]:.3f}")

    # ---- the chunked update (not part of a step): len tokens per unit in one launch, on a copy
    # of layer 0's state, against len decode launches -----------------------------------------
    chunk = None
    if diag and args.rounding == "nearest":
        chunk = {}
        st_c = rrs.State(*[t.clone() for t in states[0].tensors()])
        m0 = int(rrs.column_counts(sh_l[0], st_c)[0])
        io_t = {rrs.SEED_BF16: torch.bfloat16, rrs.SEED_F32: torch.float32}[w.io_dtype]
        Bq, Hq = w.batch, w.heads
        for Lc in ((16,) if w.kind == rrs.SEED_KDA else (16, 32)):   # KDA: 16 tokens per call
            if m0 + Lc > w.rank + T:
                continue
            gq = torch.Generator(device=dev).manual_seed(Lc)
            q_c = torch.randn(Bq, Lc, Hq, w.d_k, device=dev, generator=gq)
            k_c = torch.randn(Bq, Lc, Hq, w.d_k, device=dev, generator=gq)
            if w.kind != rrs.SEED_MAMBA2:
                q_c = q_c / q_c.norm(dim=-1, keepdim=True)
                k_c = k_c / k_c.norm(dim=-1, keepdim=True)
            v_c = torch.randn(Bq, Lc, Hq, w.d_v, device=dev, generator=gq).to(io_t)
            q_c, k_c = q_c.to(io_t), k_c.to(io_t)
            b_c = torch.rand(Bq, Lc, Hq, device=dev, generator=gq)
            g_shape = (Bq, Lc, Hq, w.d_k) if w.kind == rrs.SEED_KDA else (Bq, Lc, Hq)
            g_c = 0.9 + 0.1 * torch.rand(*g_shape, device=dev, generator=gq)
            o_c = torch.empty(Bq, Lc, Hq, w.d_v, dtype=io_t, device=dev)
            rrs.seed_decode_chunk(sh_l[0], st_c, m0, Lc, q_c, k_c, v_c, b_c, g_c, vbars[0], o_c)
            c_ev = [(ev(), ev()) for _ in range(5)]
            torch.cuda.synchronize()
            for a_, b_ in c_ev:
                a_.record()
                rrs.seed_decode_chunk(sh_l[0], st_c, m0, Lc, q_c, k_c, v_c, b_c, g_c, vbars[0], o_c)
                b_.record()
            torch.cuda.synchronize()
            t_c = sorted(a_.elapsed_time(b_) for a_, b_ in c_ev)[2] / 1e3   # median launch
            dec_launch = t_dec / n_dec_launch
            chunk[str(Lc)] = {"us_per_launch": t_c * 1e6, "head_tokens_per_s": U1 * Lc / t_c,
                              "m": m0, "speedup_vs_decode_launches": Lc * dec_launch / t_c}
            log(f"[bench] chunked update, {Lc} tokens x {U1} units at m = {m0}: {t_c * 1e6:.0f} us "
                f"({U1 * Lc / t_c / 1e6:.0f} M head-tokens/s; {Lc * dec_launch / t_c:.2f}x {Lc} decode "
                f"launches)")
        del st_c

    # ---- the head-normalisation epilogue (seed_decode_step_normed): T - 1 steps of layer 0's
    # 4096 units from copies of its state, with and without the epilogue -------------------------
    head_norm = None
    if diag:
        head_norm = head_norm_cost(rrs, torch, w, sh_l[0], states[0], pool, vbars[0], o[0], T, P, ev, log)

    # ---- the overlapped schedule (reported beside the lockstep step) ---------------------------
    overlapped = None if (args.no_overlap or not diag) else run_overlapped(rrs, torch, w, sh_l, states, pool, vbars, o, L, T,
                                                            P, ev, log, split=args.overlap_split)

    # ---- dense-state baseline ----------------------------------------------------------------
    KD = args.dense_steps
    d_ev = [(ev(), ev()) for _ in range(KD)]
    for i in range(2):  # warm
        x = pool[i % P]
        for l in range(L):
            rrs.seed_dense_decode_step(sh, S[l * U1:(l + 1) * U1], x[l]["q"], x[l]["k"], x[l]["v"],
                                       x[l]["beta"], x[l]["g"], o[l])
    torch.cuda.synchronize()
    for i in range(KD):
        x = pool[i % P]
        d_ev[i][0].record()
        for l in range(L):
            rrs.seed_dense_decode_step(sh, S[l * U1:(l + 1) * U1], x[l]["q"], x[l]["k"], x[l]["v"],
                                       x[l]["beta"], x[l]["g"], o[l])
        d_ev[i][1].record()
    torch.cuda.synchronize()
    t_dense = sum(a_.elapsed_time(b_) for a_, b_ in d_ev) / 1e3
    dense_step_ms = t_dense / KD * 1e3
    dense_gbs = KD * N * dense_bytes(w) / t_dense / 1e9
    log(f"[bench] dense baseline: {dense_step_ms:.3f} ms/step ({dense_gbs:.0f} GB/s)")

    # ---- oracle on the host cores (bounded sample) -------------------------------------------
    cpu = None
    if cpu_job is not None:
        import multiprocessing as mp

        ah, Uh, Vh, xs_h, vb_h, ns = cpu_job
        host = host_cpu()
        cores = host["share"]
        states_h = [(ah[u], Uh[u].T.copy(), Vh[u].T.copy()) for u in range(ns)]
        inputs_h = [[{k: x[k][u] for k in x} for x in xs_h] for u in range(ns)]
        heads = [vb_h[u // U1][u % w.heads] for u in range(ns)]
        shards = [(w.kind, w.rank, w.period, states_h[i::cores], inputs_h[i::cores], heads[i::cores])
                  for i in range(cores)]
        c0 = time.perf_counter()
        with mp.get_context("fork").Pool(cores) as pool_:
            cpu_secs = pool_.map(cpu_worker, shards)
        c_wall = time.perf_counter() - c0
        cpu = {"value": ns * w.period / c_wall, "unit": "head-steps/s", "cores": cores,
               "kind": "oracle", "host_cpus": host["cpus"], "cpu_model": host["model"],
               "sample": f"{ns} units (layers 0..{-(-ns // U1) - 1}) x one compression window ({w.period} decode "
                         f"steps + 1 compression), fp64 NumPy oracle, {sum(cpu_secs):.1f} s of "
                         f"CPU work on {cores} processes"}
        log(f"[bench] oracle CPU baseline: {cpu['value']:.0f} head-steps/s on {cores} cores")

    # ---- report ------------------------------------------------------------------------------
    f_b = 2 if w.factor_dtype else 4
    mean_cols = w.rank + w.period / 2
    state_ratio = (4 * w.d_k * w.d_v) / (4 * w.d_k + f_b * (w.d_k + w.d_v) * mean_cols)
    step_ms = t_total / K * 1e3
    dec_step_ms = t_dec / K * 1e3
    avg_launch_us = t_dec / n_dec_launch * 1e6
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.describe()}", "units": N, "launch_units": U1,
                   "layers": L, "factor_storage": {synth.F32: "fp32", synth.BF16: "bf16", synth.F16: "fp16"}[w.factor_dtype],
                   "prefill_tokens": prefill, "rounding": args.rounding},
        "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dec_gbs / HBM_PEAK_GBS, "traffic": (recorded_traffic(w.name)
                                 if args.factor_dtype is None and args.rounding == "nearest" else None),
                     "kernel": "k_decode (factored read-out + update)",
                     "bytes_per_launch": dec_bytes / n_dec_launch,
                     "avg_launch_us": avg_launch_us,
                     "lazy_sink_bytes_per_launch": dec_bytes_own / n_dec_launch,
                     "frac_on_lazy_sink_bytes": dec_bytes_own / t_dec / 1e9 / HBM_PEAK_GBS},
        "windows": windows,
        "cpu_baseline": cpu,
        "decode_only": {"head_steps_per_s": head_steps / t_dec, "ms_per_step": dec_step_ms,
                        "gbs": dec_gbs},
        "compress": {"launches": n_cmp_launch, "ms_per_compression": (t_cmp / max(1, len(used_cmp))) * 1e3,
                     "amortised_ms_per_step": t_cmp / K * 1e3,
                     "gbs": cmp_bytes / t_cmp / 1e9 if t_cmp > 0 else None},
        "dense": {"ms_per_step": dense_step_ms, "gbs": dense_gbs,
                  "head_steps_per_s": N / (dense_step_ms / 1e3)},
        "speedup_vs_dense": {"with_compression": dense_step_ms / step_ms,
                             "decode_only": dense_step_ms / dec_step_ms,
                             "state_byte_ratio_target": state_ratio},
        "setup_s": {"prefill_end_compression": t_from_dense},
        "energy_diagnostic": energy,
        "overlapped_schedule": overlapped,
        "spectrum_diagnostic": spectrum,
        "chunked_update": chunk,
        "head_norm_epilogue": head_norm,
    }
    print(json.dumps(res), flush=True)


def head_norm_cost(rrs, torch, w, sh, state, pool, vbar, o, T, P, ev, log):
    """Per-launch time of T - 1 decode steps of one layer with the head normalisation fused in
    (gated after the norm), against the same steps without it, each on its own copy of the
    layer's state. Returns the two averages, or None when the state is not at r columns."""
    m0 = int(rrs.column_counts(sh, state)[0])
    if m0 != w.rank:
        return None
    weight = torch.rand((w.heads, w.d_v), device=o.device) + 0.5
    gate = torch.randn((sh.units, w.d_v), device=o.device).to(o.dtype)
    res = {}
    for name in ("plain", "normed"):
        st = rrs.State(*[t.clone() for t in state.tensors()])
        for rep in range(2):   # the second pass is timed (the first warms the instruction caches)
            for t_, x_ in zip(st.tensors(), state.tensors()):
                t_.copy_(x_)
            a_, b_ = ev(), ev()
            torch.cuda.synchronize()
            a_.record()
            for j in range(T - 1):
                x = pool[j % P][0]
                if name == "plain":
                    rrs.seed_decode_step(sh, st, w.rank + j, x["q"], x["k"], x["v"], x["beta"], x["g"], vbar, o)
                else:
                    rrs.seed_decode_step_normed(sh, st, w.rank + j, x["q"], x["k"], x["v"], x["beta"], x["g"], vbar,
                                                o, weight, gate=gate, eps=1e-6)
            b_.record()
            torch.cuda.synchronize()
        res[name] = a_.elapsed_time(b_) * 1e3 / (T - 1)
        del st
    out = {"us_per_launch": res["normed"], "plain_us_per_launch": res["plain"],
           "overhead": res["normed"] / res["plain"] - 1.0, "steps": T - 1, "gated": True}
    log(f"[bench] head-norm epilogue: {res['normed']:.2f} us per launch against {res['plain']:.2f} us without "
        f"({100 * out['overhead']:+.1f} %)")
    return out


def energy_diagnostic(rrs, torch, w, sh, sh_l, states, vbars, U1, L, N, m_now, dev, ev, log):
    """seed_state_energy over the stack (one launch per layer), timed; the pooled sink share."""
    en_out = [torch.empty((U1, 3), dtype=torch.float32, device=dev) for _ in range(L)]
    for l in range(L):
        rrs.seed_state_energy(sh_l[l], states[l], vbars[l], out=en_out[l])
    e_a, e_b = ev(), ev()
    torch.cuda.synchronize()
    e_a.record()
    for l in range(L):
        rrs.seed_state_energy(sh_l[l], states[l], vbars[l], out=en_out[l])
    e_b.record()
    torch.cuda.synchronize()
    t_en = e_a.elapsed_time(e_b) / 1e3
    f_b = 2 if w.factor_dtype else 4
    en_bytes = N * (f_b * (w.d_k + w.d_v) * m_now + 4 * w.d_k + 4 * rrs.seed_scale_len(sh) + 12)
    sink_share = float(sum(e[:, 1].sum() for e in en_out) / sum(e[:, 0].sum() for e in en_out))
    log(f"[bench] energy diagnostic: {t_en * 1e3:.2f} ms over the stack at m = {m_now} "
        f"({en_bytes / t_en / 1e9:.0f} GB/s); sink share of the energy {sink_share:.3f}")
    return {"ms_per_stack": t_en * 1e3, "columns": m_now, "gbs": en_bytes / t_en / 1e9,
            "sink_share": sink_share}


def run_overlapped(rrs, torch, w, sh_l, states, pool, vbars, o, L, T, P, ev, log, steps=64, split=4):
    """The same work as the lockstep step, with the compressions overlapped with the decode
    (rank_recurrent_state_amd.OverlappedStack): decode launches on a stream over `split` XCDs,
    each layer's compression on a stream over the others, the layers' windows shifted by l mod T
    steps. Every layer still decodes every step and compresses every T steps at r + T columns.
    Returns ms per step and head-steps/s, or None."""
    if L < 8:
        # one layer (or a few) leaves nothing to overlap with: the layer's own next decode
        # launch waits for its compression, on half the chip
        log("[bench] overlapped schedule: needs a stack of layers, skipped")
        return None
    if rrs.under_profiler():
        log("[bench] overlapped schedule: not run under the profiler (a profiled run of it crashed, "
            "cause not shown), skipped")
        return None
    streams = rrs.partition_streams(split)
    if streams is None:
        log("[bench] overlapped schedule: CU-masked streams not available, skipped")
        return None
    try:
        return _run_overlapped(rrs, torch, sh_l, states, pool, vbars, o, T, P, ev, log, steps, split, streams)
    finally:
        for st in streams:
            st.close()


def _run_overlapped(rrs, torch, sh_l, states, pool, vbars, o, T, P, ev, log, steps, split, streams):
    stack = rrs.OverlappedStack(sh_l, states, *streams)
    cur = torch.cuda.current_stream()
    stack.start()
    for s in range(T):               # warmup: brings every layer onto its shifted window
        stack.step(pool[s % P], vbars, o)
    stack.finish()
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(cur)
    stack.start()
    for s in range(T, T + steps):
        stack.step(pool[s % P], vbars, o)
    stack.finish()
    e1.record(cur)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    units = sum(sh.units for sh in sh_l)
    res = {"ms_per_step": t / steps * 1e3, "head_steps_per_s": units * steps / t, "steps": steps,
           "decode_xcds": split, "compress_xcds": 8 - split}
    log(f"[bench] overlapped schedule (decode on {split} XCDs, per-layer compressions shifted over the "
        f"window on the other {8 - split}): {res['ms_per_step']:.3f} ms per step, "
        f"{res['head_steps_per_s'] / 1e6:.1f} M head-steps/s")
    return res


def run_staggered(args, rrs, torch, w, sh_l, sh_all, states, state_all, pool, vbars, o, prefill, N,
                  U1, L, T, P, nwin, Wu, K):
    """Ragged serving: request b of every layer holds r + (b mod T) columns when the timed steps
    start, so that every step fills, and compresses, the units of one T-th of the requests. A
    step is one ragged decode launch per layer and one compression launch for exactly the units
    that filled (listed; or, with --compress-scan, a launch over the stack that the others leave). Whole-job throughput only: the per-step compressions sit
    in the same graph as the decode launches."""
    dev = torch.device("cuda", 0)
    phase = (torch.arange(U1, device=dev) // w.heads) % T
    # stagger: request b sits out the steps from its phase on
    for s_ in range(T - 1):
        act = (phase > s_).to(torch.uint8)
        xl = pool[s_ % P]
        for l in range(L):
            x = xl[l]
            rrs.seed_decode_step_ragged(sh_l[l], states[l], x["q"], x["k"], x["v"], x["beta"], x["g"],
                                        vbars[l], o[l], active=act)
    torch.cuda.synchronize()
    counts = rrs.column_counts(sh_all, state_all)
    assert int(counts.min()) == w.rank and int(counts.max()) == w.rank + T - 1, "stagger"

    # the units that fill on step j of a window: request b holds r + (b + j) mod T columns
    # before it, so phase T - 1 - j fills (every layer's copy of those requests). The serving
    # loop knows its requests' lengths, so it lists them; --compress-scan starts a wave for
    # every unit of the stack instead and lets the others leave (seed_compress_ragged).
    ustack = torch.arange(N, device=dev, dtype=torch.int64)
    uphase = ((ustack % U1) // w.heads) % T
    full_lists = [ustack[uphase == (T - 1 - j) % T].to(torch.int32).contiguous() for j in range(T)]

    def enqueue_steps(wi):
        for j in range(T):
            xl = pool[wi * T + j]
            for l in range(L):
                x = xl[l]
                rrs.seed_decode_step_ragged(sh_l[l], states[l], x["q"], x["k"], x["v"], x["beta"],
                                            x["g"], vbars[l], o[l])
            if args.compress_scan:
                rrs.seed_compress_ragged(sh_all, state_all, w.rank + T)
            else:
                rrs.seed_compress_units(sh_all, state_all, full_lists[j])

    for i in range(max(1, Wu // T)):
        enqueue_steps(i % nwin)
    torch.cuda.synchronize()
    graphs = not args.eager
    if graphs:
        g_win = []
        for wi in range(nwin):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                enqueue_steps(wi)
            g_win.append(g)
        torch.cuda.synchronize()
        log(f"[bench] captured {nwin} graphs of {T} staggered steps ({T * (L + 1)} launches each)")
    nw = K // T
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(nw):
        wi = i % nwin
        if graphs:
            g_win[wi].replay()
        else:
            enqueue_steps(wi)
    e1.record()
    torch.cuda.synchronize()
    t_total = e0.elapsed_time(e1) / 1e3
    counts = rrs.column_counts(sh_all, state_all)
    assert int(counts.min()) >= w.rank and int(counts.max()) <= w.rank + T - 1, "every full unit compressed"
    step_ms = t_total / K * 1e3
    value = N * K / t_total
    log(f"[bench] staggered: {K} steps in {t_total * 1e3:.1f} ms ({step_ms:.3f} ms/step)")
    overlapped = None
    if L >= 8 and not args.no_overlap:
        overlapped = run_staggered_overlapped(rrs, torch, w, sh_l, sh_all, states, state_all, pool, vbars, o, N, L,
                                              T, P, K, args.overlap_split, args.stagger_group)
    res = {
        "metric": "factored decode head-steps/s (staggered requests, compression when full)",
        "value": value, "unit": "head-steps/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.describe()}, staggered requests", "units": N,
                   "launch_units": U1, "layers": L, "prefill_tokens": prefill,
                   "rounding": args.rounding},
        "roofline": None, "cpu_baseline": None,
        "overlapped_schedule": overlapped,
    }
    print(json.dumps(res), flush=True)


def run_staggered_overlapped(rrs, torch, w, sh_l, sh_all, states, state_all, pool, vbars, o, N, L, T, P, K, split,
                             group_units):
    """The staggered steps with the compressions overlapped (rank_recurrent_state_amd.StaggeredStack):
    ragged decode launches on `split` XCDs, each group of layers' filled units compressed on the
    others as soon as the group has decoded. Eager launches, from the state the serial staggered
    steps left. Returns ms per step, or None."""
    if rrs.under_profiler():
        log("[bench] overlapped staggered schedule: not run under the profiler, skipped")
        return None
    streams = rrs.partition_streams(split)
    if streams is None:
        log("[bench] overlapped staggered schedule: CU-masked streams not available, skipped")
        return None
    try:
        stack = rrs.StaggeredStack(sh_all, state_all, sh_l, states, *streams, group_units=group_units)
        cur = torch.cuda.current_stream()
        stack.start()
        for s_ in range(T):                  # warmup
            stack.step(pool[s_ % P], vbars, o)
        stack.finish()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        stack.start()
        for s_ in range(K):
            stack.step(pool[s_ % P], vbars, o)
        stack.finish()
        e1.record(cur)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3
        counts = rrs.column_counts(sh_all, state_all)
        assert int(counts.min()) >= w.rank and int(counts.max()) <= w.rank + T - 1, "every full unit compressed"
    finally:
        for st in streams:
            st.close()
    res = {"ms_per_step": t / K * 1e3, "head_steps_per_s": N * K / t, "steps": K, "decode_xcds": split,
           "compress_xcds": 8 - split, "layer_groups": len(stack.groups), "eager": True}
    log(f"[bench] overlapped staggered schedule (decode on {split} XCDs, each group of {stack.groups[0][1]} layers' "
        f"filled units compressed on the other {8 - split}): {res['ms_per_step']:.3f} ms per step, "
        f"{res['head_steps_per_s'] / 1e6:.1f} M head-steps/s")
    return res


if __name__ == "__main__":
    main()
