"""Overlapped schedule for a stack of layers: decode and compression on disjoint XCDs.

The decode step is bound by HBM bandwidth and the compression by vector arithmetic, so the two
can share the chip. This host-side scheduler sends every layer's decode launch to a stream
masked to one part of the XCDs and each layer's compression to a stream on the others, and
shifts each layer's compression window so that a step compresses one or two layers instead of
every layer at once. Events keep each layer's order: its compression waits for the decode
launch that filled it, and its next decode launch waits for the compression.

Layer l decodes every step; it compresses when it holds r + T columns, except once at the
start, where it compresses after T - (l mod T) steps instead, which shifts its window by l mod
T steps. Every later window is a full one.

The streams are HIP streams with CU masks of whole 32-CU blocks (masks that split an XCD were
refused by the runtime on MI355X), made and destroyed by libseed itself, so that they belong to
the runtime that launches the kernels. Kernels run unchanged; only the launch order and the
streams differ from a serial schedule of the same launches.

Profiled runs. The first profiled run of this schedule (rocprofv3 kernel trace) ended with a
segmentation fault of the profiled process, and its cause has not been shown: under the
profiler the process maps a second HSA runtime (the profiler's, beside the one bundled with
torch), and the CU-masked queues are the one thing this schedule adds. Until a cause is shown,
partition_streams refuses to run under the profiler.
"""
from __future__ import annotations

import os

from . import _lib


def under_profiler() -> bool:
    """Whether rocprofv3's tool library is loaded into this process (its preload or tool list)."""
    env = os.environ.get("LD_PRELOAD", "") + ":" + os.environ.get("ROCP_TOOL_LIBRARIES", "")
    return "rocprofiler-sdk" in env


def partition_streams(split: int = 4):
    """Two CU-masked streams on disjoint XCDs: the first `split` 32-CU blocks and the rest, as
    _lib.CUMaskedStream objects (the caller closes them). None when the device is not 256 CUs or
    the runtime refuses the masks. Raises RuntimeError under the profiler (see above)."""
    import torch
    if under_profiler():
        raise RuntimeError("the CU-partitioned schedule is not run under rocprofv3 (a profiled run "
                           "of it crashed, cause not shown)")
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    if ncu != 256 or not 0 < split < 8:
        return None
    words = (ncu + 31) // 32
    out = []
    for pick in (lambda i: i // 32 < split, lambda i: i // 32 >= split):
        mask = [0] * words
        for i in range(ncu):
            if pick(i):
                mask[i // 32] |= 1 << (i % 32)
        try:
            out.append(_lib.CUMaskedStream(mask))
        except _lib.SeedError:
            for st in out:
                st.close()
            return None
    return out


class OverlappedStack:
    """Decode launches on `decode_stream`, compressions on `compress_stream` (any two streams;
    partition_streams gives the CU-partitioned pair). shapes and states: one per layer, with
    every layer at rank r columns and the same r, T."""

    def __init__(self, shapes, states, decode_stream, compress_stream):
        import torch
        self.shapes, self.states = list(shapes), list(states)
        # CU-masked streams from partition_streams are used through their torch view
        self.sA = getattr(decode_stream, "torch", decode_stream)
        self.sB = getattr(compress_stream, "torch", compress_stream)
        r, T = self.shapes[0].rank, self.shapes[0].period
        self.r, self.T = r, T
        L = len(self.shapes)
        self.m = [r] * L
        # the first compression of layer l comes after T - (l mod T) steps (never after none)
        self.first = [T - (l % T) for l in range(L)]
        self.pending = [None] * L
        self._torch = torch

    def start(self):
        """Order both streams after the work already queued on the current stream."""
        cur = self._torch.cuda.current_stream()
        self.sA.wait_stream(cur)
        self.sB.wait_stream(cur)

    def step(self, inputs, vbars, outs):
        """One step of every layer: inputs[l] a dict of q, k, v, beta, g for layer l."""
        torch = self._torch
        for l, (sh, st) in enumerate(zip(self.shapes, self.states)):
            if self.pending[l] is not None:
                self.sA.wait_event(self.pending[l])
                self.pending[l] = None
            x = inputs[l]
            _lib.seed_decode_step(sh, st, self.m[l], x["q"], x["k"], x["v"], x["beta"], x["g"], vbars[l],
                                  outs[l], stream=self.sA)
            self.m[l] += 1
            due = self.r + (self.first[l] if self.first[l] else self.T)
            if self.m[l] == due:
                e = torch.cuda.Event()
                e.record(self.sA)
                self.sB.wait_event(e)
                _lib.seed_compress(sh, st, self.m[l], stream=self.sB)
                ec = torch.cuda.Event()
                ec.record(self.sB)
                self.pending[l] = ec
                self.m[l] = self.r
                self.first[l] = 0

    def finish(self):
        """Order the current stream after both streams."""
        cur = self._torch.cuda.current_stream()
        cur.wait_stream(self.sA)
        cur.wait_stream(self.sB)


class StaggeredStack:
    """Ragged serving of a layer stack (requests at staggered column counts, each unit compressed
    on the step it fills), with the compressions overlapped with the decode.

    Every step decodes each layer with seed_decode_step_ragged on `decode_stream`. The units
    that fill on that step (they reach r + T columns) are compressed with seed_compress_units on
    `compress_stream`, one launch per group of consecutive layers, issued as soon as the group's
    last layer has decoded; the group's next decode waits for it. Groups hold about
    `group_units` full units per step, so that a launch fills whole rounds of the compression
    stream's wave slots instead of ending in a partly filled one.

    shape_all / state_all describe the whole stack as one batch (layer-major, the layers'
    states contiguous); shapes / states are the per-layer views the decode launches use. Every
    unit must hold between r and r + T - 1 columns at the start (the column counts are read
    once, here): a unit then fills every T steps, so the lists of units that fill repeat with
    period T and are built once.
    """

    def __init__(self, shape_all, state_all, shapes, states, decode_stream, compress_stream,
                 group_units: int = 1024):
        import numpy as np
        import torch
        self._torch = torch
        self.shapes, self.states = list(shapes), list(states)
        self.sh_all, self.st_all = shape_all, state_all
        self.sA = getattr(decode_stream, "torch", decode_stream)
        self.sB = getattr(compress_stream, "torch", compress_stream)
        L = len(self.shapes)
        U1 = self.shapes[0].units
        r, T = shape_all.rank, shape_all.period
        if shape_all.units != L * U1:
            raise ValueError("shape_all must cover the layers' units")
        m = _lib.column_counts(shape_all, state_all).numpy().astype(np.int64)
        if m.min() < r or m.max() > r + T - 1:
            raise ValueError("every unit must hold r .. r + T - 1 columns")
        fills = []            # fills[j]: stack-wide units that fill on step j of the period
        for _ in range(T):
            m = m + 1
            full = np.nonzero(m == r + T)[0]
            fills.append(full)
            m[full] = r
        per_layer = max(1, max(len(f) for f in fills) // L)
        lpg = max(1, group_units // per_layer)                  # layers per group
        self.groups = [(g, min(g + lpg, L)) for g in range(0, L, lpg)]
        dev = state_all.a.device
        self.lists = []       # lists[j][gi]: int32 device tensor, or None when empty
        for f in fills:
            row = []
            for (l0, l1) in self.groups:
                sel = f[(f >= l0 * U1) & (f < l1 * U1)]
                row.append(torch.as_tensor(sel, dtype=torch.int32, device=dev).contiguous() if len(sel) else None)
            self.lists.append(row)
        self.group_of = [gi for gi, (l0, l1) in enumerate(self.groups) for _ in range(l0, l1)]
        self.pending = [None] * len(self.groups)
        self.j = 0

    def start(self):
        """Order both streams after the work already queued on the current stream."""
        cur = self._torch.cuda.current_stream()
        self.sA.wait_stream(cur)
        self.sB.wait_stream(cur)

    def step(self, inputs, vbars, outs):
        """One step of every layer: inputs[l] a dict of q, k, v, beta, g for layer l."""
        torch = self._torch
        for l, (sh, st) in enumerate(zip(self.shapes, self.states)):
            gi = self.group_of[l]
            l0, l1 = self.groups[gi]
            if l == l0 and self.pending[gi] is not None:
                self.sA.wait_event(self.pending[gi])
                self.pending[gi] = None
            x = inputs[l]
            _lib.seed_decode_step_ragged(sh, st, x["q"], x["k"], x["v"], x["beta"], x["g"], vbars[l], outs[l],
                                         stream=self.sA)
            lst = self.lists[self.j][gi]
            if l == l1 - 1 and lst is not None:
                e = torch.cuda.Event()
                e.record(self.sA)
                self.sB.wait_event(e)
                _lib.seed_compress_units(self.sh_all, self.st_all, lst, stream=self.sB)
                ec = torch.cuda.Event()
                ec.record(self.sB)
                self.pending[gi] = ec
        self.j = (self.j + 1) % len(self.lists)

    def finish(self):
        """Order the current stream after both streams."""
        cur = self._torch.cuda.current_stream()
        cur.wait_stream(self.sA)
        cur.wait_stream(self.sB)
