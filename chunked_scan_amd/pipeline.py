"""One device's share of ZeCO causal linear attention, composed from the four C-ABI calls.

Nothing here computes: each function only sequences library calls (and allocates their
buffers when the caller does not pass them).  The structure follows the linear-decomposition
identity of the review page "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear
Attention" (pith_extraction.key_machinery): local work runs from a zero state, the incoming
state is folded into the state by the All-Scan update and into the outputs by a rank-dk
correction.

``device_step``   -- one device holding one segment, given the state S_recv it receives.  The
                     segment is cut into G sub-segments, each treated as one more device of the
                     same identity: the local forward of every sub-segment from a zero state (one
                     launch, no second pass over K and V), then one inclusive scan over
                     [S_recv, S_loc,1, ..., S_loc,G] that yields every sub-segment's exact incoming
                     state (its last entry is the All-Scan update S_out = Lambda S_recv + S_loc),
                     then one correction pass O += (Q * cumulative decay) S_in over every
                     sub-segment.  With G = 1 this is the plain form: local forward, two-entry scan,
                     correction by S_recv.  Without decay there is no decay to prepare (Lambda = 1,
                     cumulative decay = 1): the scan runs as a plain sum.  Head decay: Lambda from
                     the closed form, the cumulative decay formed inside the correction.  Gate
                     decay: the forward itself emits Q * cumulative decay and Lambda
                     (la_chunk_fwd_decayed), and the correction adds a plain product.
``ExactStep``     -- the same outputs and S_out from one la_chunk_fwd call that starts from S_recv: the
                     library splits the segment into sub-segments itself, scans their local states
                     with S_recv as the first entry and runs every sub-segment's outputs from its
                     exact incoming state (no correction pass); ``schedule`` picks the library's
                     separate passes or its chained single launch.
``RecvFirstStep`` -- the decomposed step with S_recv taken in at the start of the first sub-segment:
                     the segment is cut into G segments of one segmented forward, the first of
                     which starts from S_recv (it is then exact), the others from zero; the scan
                     over their G local states yields every incoming state, and the correction
                     covers sub-segments 1..G-1 only.  It saves the first sub-segment's correction
                     and one scan entry, at the price of a local forward that needs S_recv.
``segmented_forward`` -- P devices emulated on one GPU: the local forward of all P segments in
                     one launch, the P-entry state scan, and the correction of segments 1..P-1.
"""
from __future__ import annotations

from typing import Optional

import torch

from .binding import la_chunk_fwd, la_chunk_fwd_decayed, la_cumdecay, la_state_correct, la_state_scan


def _tile_flags(B, H, L, nseg, dev):
    """Per-64-token-tile liveness flags of q * cumulative decay, one int32 per tile of each segment."""
    return torch.empty((B, H, nseg, (L // nseg + 63) // 64), dtype=torch.int32, device=dev)


def _forward(step, s_in, s_out, totals, nseg, timers):
    """The local forward and the decay quantities the scan and the correction need."""
    B, H, L, dk, dv = step.shape
    kw = dict(mode=step.mode, nseg=nseg, chunk=step.chunk, gate_norm=step.gate_norm,
              subseg_chunks=step.subseg_chunks)
    if step.mode == "gate":
        la_chunk_fwd_decayed(step.q, step.k, step.v, step.decay, s_in, step.o, s_out, step.qd, totals,
                             step.live, timer=timers.get("fwd"), **kw)
        return
    la_chunk_fwd(step.q, step.k, step.v, step.decay, s_in, step.o, s_out, timer=timers.get("fwd"), **kw)
    if step.mode == "head":
        la_cumdecay(step.decay, B, H, L, dk, mode="head", nseg=nseg, total=totals, want_cum=False,
                    timer=timers.get("cum"))


def _correct(step, s_recv, nseg, seg_begin, timers):
    """O += (Q * cumulative decay) S_recv; in gate mode Q * cum is the forward's q_decayed, and the
    tiles where it is exactly zero (the cumulative decay has underflowed) are skipped."""
    if step.mode == "gate":
        la_state_correct(step.qd, None, s_recv, step.o, mode="none", nseg=nseg, seg_begin=seg_begin,
                         tile_live=step.live, timer=timers.get("corr"))
    else:
        la_state_correct(step.q, step.decay if step.mode == "head" else None, s_recv, step.o, mode=step.mode,
                         nseg=nseg, seg_begin=seg_begin, timer=timers.get("corr"))


def subsegments(B: int, H: int, L: int, target_units: int = 0, min_len: int = 256, dk: int = 128) -> int:
    """Sub-segments per sequence for a device step: about ``target_units`` (b,h,sub-segment) units
    in all, each at least ``min_len`` tokens; G must divide L, and lengths that are whole 64-token
    chunks are preferred.  By default 256 units (one workgroup per compute unit) at dk = 128 and
    512 below: the small-head kernels are latency-bound and several of their workgroups share a
    compute unit (B1 H16 L16k, G = 16 -> 32: dk = 64 step 61.9 -> 54.4 us, dk = 32 41.1 -> 40.4 us;
    G = 64 gains no more at dk = 32, where its 65-entry scan leaves the scan's vector form)."""
    if target_units <= 0:
        target_units = 256 if dk >= 128 else 512
    want = max(1, -(-target_units // max(1, B * H)))
    cands = [g for g in range(1, want + 1) if L % g == 0 and (g == 1 or L // g >= min_len)]
    whole = [g for g in cands if (L // g) % 64 == 0]
    return max(whole or cands)


class DeviceStep:
    """Buffers and call sequence of one device step; ``run()`` may be timed or graph-captured.
    ``subseg`` fixes the number G of sub-segments (0 = ``subsegments()``)."""

    def __init__(self, q, k, v, decay, s_recv, *, mode: str, chunk: int = 64, gate_norm: float = 16.0,
                 subseg_chunks: int = 0, subseg: int = 0):
        B, H, L, dk = q.shape
        dv = v.shape[-1]
        dev = q.device
        G = subseg or subsegments(B, H, L, dk=dk)
        if L % G:
            raise ValueError(f"{G} sub-segments do not divide L = {L}")
        self.q, self.k, self.v, self.decay = q, k, v, decay
        self.mode, self.chunk, self.gate_norm, self.subseg_chunks = mode, chunk, gate_norm, subseg_chunks
        self.G = G
        self.shape = (B, H, L, dk, dv)
        self.o = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
        # scan buffer: slot 0 = incoming state (what the previous device sends), slots 1..G = local
        # states of the sub-segments; after the scan slot p is the incoming state of sub-segment p
        # and slot G the outgoing state
        self.states = torch.zeros((B, H, G + 1, dk, dv), dtype=torch.float32, device=dev)
        if s_recv is not None:
            self.states[:, :, 0].copy_(s_recv)
        self.totals = torch.ones((B, H, G + 1, dk), dtype=torch.float32, device=dev)
        self.qd = torch.empty_like(q) if mode == "gate" else None  # q times its cumulative decay
        self.live = _tile_flags(B, H, L, G, dev) if mode == "gate" else None

    def run(self, timers: Optional[dict] = None):
        """One step.  ``timers`` optionally maps "fwd", "cum", "scan", "corr" to KernelTimers."""
        t = timers or {}
        G = self.G
        _forward(self, None, self.states[:, :, 1:], self.totals[:, :, 1:], G, t)
        la_state_scan(self.states, self.totals if self.mode != "none" else None, self.states, timer=t.get("scan"))
        _correct(self, self.states[:, :, 0:G], G, 0, t)
        return self.o, self.states[:, :, G]


class ExactStep:
    """One device step as a single exact forward from S_recv (la_chunk_fwd with s_in = S_recv);
    ``run()`` may be timed or graph-captured.  Returns (o, s_out [B,H,dk,dv])."""

    def __init__(self, q, k, v, decay, s_recv, *, mode: str, chunk: int = 64, gate_norm: float = 16.0,
                 subseg_chunks: int = 0, schedule: str = "auto"):
        B, H, L, dk = q.shape
        dv = v.shape[-1]
        self.q, self.k, self.v, self.decay, self.s_recv = q, k, v, decay, s_recv
        self.mode, self.chunk, self.gate_norm = mode, chunk, gate_norm
        self.subseg_chunks, self.schedule = subseg_chunks, schedule
        self.shape = (B, H, L, dk, dv)
        self.o = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
        self.s_out = torch.empty((B, H, 1, dk, dv), dtype=torch.float32, device=q.device)

    def run(self, timers: Optional[dict] = None):
        """One step.  ``timers`` optionally maps "fwd" to a KernelTimer."""
        t = timers or {}
        la_chunk_fwd(self.q, self.k, self.v, self.decay, self.s_recv, self.o, self.s_out, mode=self.mode,
                     chunk=self.chunk, gate_norm=self.gate_norm, subseg_chunks=self.subseg_chunks,
                     schedule=self.schedule, timer=t.get("fwd"))
        return self.o, self.s_out[:, :, 0]


class RecvFirstStep:
    """One device step as a segmented forward over G sub-segments whose first starts from S_recv;
    ``run()`` may be timed or graph-captured.  Returns (o, s_out [B,H,dk,dv])."""

    def __init__(self, q, k, v, decay, s_recv, *, mode: str, chunk: int = 64, gate_norm: float = 16.0,
                 subseg_chunks: int = 0, subseg: int = 0):
        B, H, L, dk = q.shape
        G = subseg or subsegments(B, H, L, dk=dk)
        if L % G:
            raise ValueError(f"{G} sub-segments do not divide L = {L}")
        self.G = self.nseg = G
        self.seg = SegmentedForward(q, k, v, decay, s_recv, mode=mode, nseg=G, chunk=chunk, gate_norm=gate_norm,
                                    subseg_chunks=subseg_chunks)
        self.live = self.seg.live  # gate mode: the forward's tile flags of q * cumulative decay

    def run(self, timers: Optional[dict] = None):
        """One step.  ``timers`` optionally maps "fwd", "cum", "scan", "corr" to KernelTimers."""
        o, states = self.seg.run(timers)
        return o, states[:, :, -1]


def device_step(q, k, v, decay, s_recv, *, mode: str, chunk: int = 64, gate_norm: float = 16.0,
                subseg_chunks: int = 0, subseg: int = 0):
    """Returns (o, s_out) of one device that receives s_recv (None = zero)."""
    return DeviceStep(q, k, v, decay, s_recv, mode=mode, chunk=chunk, gate_norm=gate_norm,
                      subseg_chunks=subseg_chunks, subseg=subseg).run()


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
        self.qd = torch.empty_like(q) if mode == "gate" else None  # q times its cumulative decay
        self.live = _tile_flags(B, H, L, nseg, dev) if mode == "gate" else None

    def run(self, timers: Optional[dict] = None):
        """One pass.  ``timers`` optionally maps "fwd", "cum", "scan", "corr" to KernelTimers."""
        P = self.nseg
        t = timers or {}
        _forward(self, self.s_in, self.states, self.totals, P, t)
        la_state_scan(self.states, self.totals if self.mode != "none" else None, self.states, timer=t.get("scan"))
        if P > 1:
            _correct(self, self.states[:, :, : P - 1], P, 1, t)
        return self.o, self.states


def segmented_forward(q, k, v, decay, s_in, *, mode: str, nseg: int, chunk: int = 64, gate_norm: float = 16.0,
                      subseg_chunks: int = 0):
    """Returns (o, out_states [B,H,P,dk,dv]); out_states[:, :, -1] is the final state."""
    return SegmentedForward(q, k, v, decay, s_in, mode=mode, nseg=nseg, chunk=chunk, gate_norm=gate_norm,
                            subseg_chunks=subseg_chunks).run()
