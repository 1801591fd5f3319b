"""One device's share of ZeCO causal linear attention, composed from the four C-ABI calls.

Nothing here computes: each function only sequences library calls (and allocates their
buffers when the caller does not pass them).  The structure follows the linear-decomposition
identity of the review page "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear
Attention" (pith_extraction.key_machinery): local work runs from a zero state, the incoming
state is folded into the state by the All-Scan update and into the outputs by a rank-dk
correction.

``device_step``   -- one device holding one segment: local forward, then the All-Scan update
                     S_out = Lambda_total S_recv + S_loc (a two-entry state scan), then
                     O += (Q * cumulative decay) S_recv.  Without decay there is no decay to
                     prepare (Lambda = 1, cumulative decay = 1): the scan runs as a plain sum.
``segmented_forward`` -- P devices emulated on one GPU: the local forward of all P segments in
                     one launch, the P-entry state scan, and the correction of segments 1..P-1.
"""
from __future__ import annotations

from typing import Optional

import torch

from .binding import la_chunk_fwd, la_cumdecay, la_state_correct, la_state_scan


def _corr_decay(mode: str, decay, cum):
    return None if mode == "none" else (decay if mode == "head" else cum)


class DeviceStep:
    """Buffers and call sequence of one device step; ``run()`` may be timed or graph-captured."""

    def __init__(self, q, k, v, decay, s_recv, *, mode: str, chunk: int = 64, gate_norm: float = 16.0,
                 subseg_chunks: int = 0):
        B, H, L, dk = q.shape
        dv = v.shape[-1]
        dev = q.device
        self.q, self.k, self.v, self.decay = q, k, v, decay
        self.mode, self.chunk, self.gate_norm, self.subseg_chunks = mode, chunk, gate_norm, subseg_chunks
        self.shape = (B, H, L, dk, dv)
        self.o = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
        # scan buffer: slot 0 = incoming state (what the previous device sends), slot 1 = local state
        self.states = torch.zeros((B, H, 2, dk, dv), dtype=torch.float32, device=dev)
        if s_recv is not None:
            self.states[:, :, 0].copy_(s_recv)
        self.totals = torch.ones((B, H, 2, dk), dtype=torch.float32, device=dev)
        self.cum = torch.empty((B, H, L, dk), dtype=torch.float32, device=dev) if mode == "gate" else None

    def run(self, timers: Optional[dict] = None):
        """One step.  ``timers`` optionally maps "fwd", "cum", "scan", "corr" to KernelTimers."""
        B, H, L, dk, dv = self.shape
        t = timers or {}
        la_chunk_fwd(self.q, self.k, self.v, self.decay, None, self.o, self.states[:, :, 1:2], mode=self.mode,
                     chunk=self.chunk, gate_norm=self.gate_norm, subseg_chunks=self.subseg_chunks,
                     timer=t.get("fwd"))
        if self.mode != "none":
            la_cumdecay(self.decay, B, H, L, dk, mode=self.mode, gate_norm=self.gate_norm, cum=self.cum,
                        total=self.totals[:, :, 1:2], want_cum=self.mode == "gate", timer=t.get("cum"))
        la_state_scan(self.states, self.totals if self.mode != "none" else None, self.states, timer=t.get("scan"))
        la_state_correct(self.q, _corr_decay(self.mode, self.decay, self.cum), self.states[:, :, 0:1], self.o,
                         mode=self.mode, timer=t.get("corr"))
        return self.o, self.states[:, :, 1]


def device_step(q, k, v, decay, s_recv, *, mode: str, chunk: int = 64, gate_norm: float = 16.0,
                subseg_chunks: int = 0):
    """Returns (o, s_out) of one device that receives s_recv (None = zero)."""
    return DeviceStep(q, k, v, decay, s_recv, mode=mode, chunk=chunk, gate_norm=gate_norm,
                      subseg_chunks=subseg_chunks).run()


class SegmentedForward:
    """P segments (P emulated devices) of each (b,h) sequence on one GPU; ``run()`` is one pass."""

    def __init__(self, q, k, v, decay, s_in, *, mode: str, nseg: int, chunk: int = 64, gate_norm: float = 16.0,
                 subseg_chunks: int = 0):
        B, H, L, dk = q.shape
        dv = v.shape[-1]
        dev = q.device
        self.q, self.k, self.v, self.decay, self.s_in = q, k, v, decay, s_in
        self.mode, self.nseg, self.chunk, self.gate_norm = mode, nseg, chunk, gate_norm
        self.subseg_chunks = subseg_chunks
        self.shape = (B, H, L, dk, dv)
        self.o = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
        self.states = torch.empty((B, H, nseg, dk, dv), dtype=torch.float32, device=dev)
        self.totals = torch.empty((B, H, nseg, dk), dtype=torch.float32, device=dev)
        self.cum = torch.empty((B, H, L, dk), dtype=torch.float32, device=dev) if mode == "gate" else None

    def run(self, timers: Optional[dict] = None):
        """One pass.  ``timers`` optionally maps "fwd", "cum", "scan", "corr" to KernelTimers."""
        B, H, L, dk, dv = self.shape
        P = self.nseg
        t = timers or {}
        la_chunk_fwd(self.q, self.k, self.v, self.decay, self.s_in, self.o, self.states, mode=self.mode, nseg=P,
                     chunk=self.chunk, gate_norm=self.gate_norm, subseg_chunks=self.subseg_chunks,
                     timer=t.get("fwd"))
        if self.mode != "none":
            la_cumdecay(self.decay, B, H, L, dk, mode=self.mode, nseg=P, gate_norm=self.gate_norm, cum=self.cum,
                        total=self.totals, want_cum=self.mode == "gate", timer=t.get("cum"))
        la_state_scan(self.states, self.totals if self.mode != "none" else None, self.states, timer=t.get("scan"))
        if P > 1:
            la_state_correct(self.q, _corr_decay(self.mode, self.decay, self.cum), self.states[:, :, : P - 1], self.o,
                             mode=self.mode, nseg=P, seg_begin=1, timer=t.get("corr"))
        return self.o, self.states


def segmented_forward(q, k, v, decay, s_in, *, mode: str, nseg: int, chunk: int = 64, gate_norm: float = 16.0,
                      subseg_chunks: int = 0):
    """Returns (o, out_states [B,H,P,dk,dv]); out_states[:, :, -1] is the final state."""
    return SegmentedForward(q, k, v, decay, s_in, mode=mode, nseg=nseg, chunk=chunk, gate_norm=gate_norm,
                            subseg_chunks=subseg_chunks).run()
