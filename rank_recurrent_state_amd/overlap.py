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

The streams are HIP streams with CU masks (hipExtStreamCreateWithCUMask) of whole 32-CU blocks:
masks that split an XCD were refused by the runtime on MI355X. Kernels run unchanged; only the
launch order and the streams differ from a serial schedule of the same launches.
"""
from __future__ import annotations

import ctypes

from . import _lib


def partition_streams(split: int = 4):
    """Two torch streams on disjoint XCDs: the first `split` 32-CU blocks and the rest. None
    when the runtime does not provide CU-masked streams or the device is not 256 CUs."""
    import torch
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    if ncu != 256 or not 0 < split < 8:
        return None
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    words = (ncu + 31) // 32
    out = []
    for pick in (lambda i: i // 32 < split, lambda i: i // 32 >= split):
        mask = (ctypes.c_uint32 * words)()
        for i in range(ncu):
            if pick(i):
                mask[i // 32] |= 1 << (i % 32)
        h = ctypes.c_void_p()
        if hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), mask) != 0:
            return None
        out.append(torch.cuda.ExternalStream(h.value))
    return out


class OverlappedStack:
    """Decode launches on `decode_stream`, compressions on `compress_stream` (any two streams;
    partition_streams gives the CU-partitioned pair). shapes and states: one per layer, with
    every layer at rank r columns and the same r, T."""

    def __init__(self, shapes, states, decode_stream, compress_stream):
        import torch
        self.shapes, self.states = list(shapes), list(states)
        self.sA, self.sB = decode_stream, compress_stream
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
