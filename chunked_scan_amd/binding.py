"""ctypes binding of liblachunk.so (C ABI in include/la_chunk.h).

Argument marshalling only: tensors are checked (device, dtype, layout, shape), outputs are
allocated when not given, the ``la_shape`` struct is filled in, and the call is enqueued on the
current torch stream.  Every step of the computation runs in the HIP kernels of the library;
there is no CPU or PyTorch fallback, and calling any function without the built library raises.

Per-segment state arrays ([B,H,P,dk,dv]) and segment-total arrays ([B,H,P,dk]) may be strided
views whose (b,h) blocks are evenly spaced -- e.g. slot 1 of a [B,H,2,dk,dv] scan buffer -- and
are passed as a base pointer plus the ``state_stride`` / ``total_stride`` of the C ABI.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LACHUNK_LIB names another build of the same library (the host-sanitized build of build.py's
# build_sanitized()).
LIB_PATH = os.environ.get("LACHUNK_LIB") or os.path.join(_HERE, "liblachunk.so")

LA_F32, LA_BF16 = 0, 1
MODES = {"none": 0, "head": 1, "gate": 2}
STATUS = {0: "LA_OK", -1: "LA_ERR_NULL", -2: "LA_ERR_SHAPE", -3: "LA_ERR_DTYPE", -4: "LA_ERR_ALIAS",
          -5: "LA_ERR_UNSUPPORTED", -6: "LA_ERR_LAUNCH", -7: "LA_ERR_DECAY", -8: "LA_ERR_WORKSPACE",
          -9: "LA_ERR_TIMEOUT"}
NOALLOC_SCRATCH_BYTES = 32 << 20  # LA_NOALLOC_SCRATCH_BYTES of la_chunk.h
EXPORTS = ("la_chunk_fwd", "la_chunk_fwd_noalloc", "la_chunk_fwd_decayed", "la_chunk_bwd", "la_chunk_bwd_states", "la_state_scan", "la_state_correct", "la_state_correct_live",
           "la_cumdecay", "la_trim_workspace", "la_chain_status", "la_set_chain_spin_limit", "la_status_str", "la_supported",
           "la_version")


TRACE_MAX = 16


class Trace(ctypes.Structure):
    """la_trace: caller-created HIP events the library records around each kernel it enqueues."""
    _fields_ = [("start", ctypes.c_void_p * TRACE_MAX), ("stop", ctypes.c_void_p * TRACE_MAX),
                ("capacity", ctypes.c_int32), ("count", ctypes.c_int32), ("name", ctypes.c_char_p * TRACE_MAX)]


class Shape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("L", ctypes.c_int64),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("nseg", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("decay_mode", ctypes.c_int32),
        ("gate_norm", ctypes.c_float), ("seg_begin", ctypes.c_int32), ("state_stride", ctypes.c_int64),
        ("total_stride", ctypes.c_int64), ("subseg_chunks", ctypes.c_int32), ("fwd_schedule", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
        ("trace", ctypes.POINTER(Trace)),
    ]


class KernelTimer:
    """Per-kernel HIP-event timing through la_trace.  ``attach(shape)`` hooks a call; after the
    stream is synchronised ``harvest()`` returns [(kernel name, ms)] for the last hooked call."""

    def __init__(self, capacity: int = TRACE_MAX):
        self.events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(capacity)]
        for a, b in self.events:  # torch creates the HIP event on first record
            a.record()
            b.record()
        torch.cuda.synchronize()
        self.trace = Trace()
        self.trace.capacity = capacity
        for i, (a, b) in enumerate(self.events):
            self.trace.start[i] = a.cuda_event
            self.trace.stop[i] = b.cuda_event

    def harvest(self):
        return [(self.trace.name[i].decode(), self.events[i][0].elapsed_time(self.events[i][1]))
                for i in range(self.trace.count)]


class LaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblachunk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                               "g.build()'` (hipcc, gfx950). There is no fallback path.")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.POINTER(Shape)
        L.la_chunk_fwd.argtypes = [P, P, P, P, P, P, P, S, ctypes.c_int32]
        L.la_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, S, ctypes.c_int32]
        L.la_chunk_fwd_decayed.argtypes = [P, P, P, P, P, P, P, P, P, P, S, ctypes.c_int32]
        L.la_chunk_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, S, ctypes.c_int32]
        L.la_chunk_bwd_states.argtypes = [P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int64, P, P, P, P, P, P, P, S,
                                          ctypes.c_int32]
        L.la_state_correct_live.argtypes = [P, P, P, P, P, S]
        L.la_state_scan.argtypes = [P, P, ctypes.c_int32, P, S]
        L.la_state_correct.argtypes = [P, P, P, P, S]
        L.la_cumdecay.argtypes = [P, P, P, S]
        L.la_supported.argtypes = [S, ctypes.c_int32]
        L.la_status_str.argtypes = [ctypes.c_int]
        L.la_status_str.restype = ctypes.c_char_p
        L.la_trim_workspace.argtypes = []
        L.la_chain_status.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
        L.la_set_chain_spin_limit.argtypes = [ctypes.c_int32]
        for f in (L.la_chunk_fwd, L.la_chunk_fwd_noalloc, L.la_chunk_fwd_decayed, L.la_trim_workspace, L.la_state_scan, L.la_state_correct,
                  L.la_state_correct_live, L.la_cumdecay, L.la_supported, L.la_version, L.la_chain_status,
                  L.la_set_chain_spin_limit):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise LaError(fn, status, lib().la_status_str(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None, contiguous=True):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _bh_stride(t: torch.Tensor, name: str, inner: int) -> int:
    """Stride between (b,h) blocks of a [B,H,P,...] view whose per-(b,h) block of P*inner
    elements is dense and whose (b,h) blocks are evenly spaced; 0 when the whole view is dense."""
    if t.is_contiguous():
        return 0
    B, H, P = t.shape[:3]
    dense_tail = list(torch.empty(t.shape[2:], device="meta").stride())
    if list(t.stride()[2:]) != dense_tail:
        raise ValueError(f"{name}: each (b,h) block must be dense")
    s1 = t.stride(1) if H > 1 else t.stride(0) // max(H, 1)
    if B > 1 and t.stride(0) != H * s1:
        raise ValueError(f"{name}: (b,h) blocks must be evenly spaced")
    if s1 < P * inner:
        raise ValueError(f"{name}: (b,h) blocks overlap")
    return s1


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def mode_code(mode: Optional[str], decay: Optional[torch.Tensor]) -> int:
    if mode is None:
        mode = "none" if decay is None else ("head" if decay.dim() == 1 else "gate")
    return MODES[mode]


def make_shape(B, H, L, dk, dv, *, nseg=1, dtype=LA_BF16, mode=0, gate_norm=16.0, seg_begin=0,
               state_stride=0, total_stride=0, subseg_chunks=0, fwd_schedule=0, stream=None, timer=None) -> Shape:
    s = Shape(B, H, L, dk, dv, nseg, dtype, dtype, mode, gate_norm, seg_begin, state_stride,
              total_stride, subseg_chunks, fwd_schedule, stream)
    if timer is not None:
        s.trace = ctypes.pointer(timer.trace)
    return s


def la_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: Optional[torch.Tensor] = None,
                 s_in: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                 s_out: Optional[torch.Tensor] = None, *, mode: Optional[str] = None, nseg: int = 1,
                 chunk: int = 64, gate_norm: float = 16.0, subseg_chunks: int = 0, want_state: bool = True,
                 schedule: str = "auto", stream=None, timer=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise forward.  q, k [B,H,L,dk], v [B,H,L,dv] (f32 or bf16); decay None / [H] / [B,H,L,dk];
    s_in [B,H,dk,dv] f32 or None.  Returns (o [B,H,L,dv], s_out [B,H,nseg,dk,dv] f32 or None);
    s_out may be a view with evenly spaced dense (b,h) blocks.  schedule: "auto" (the library's
    choice), "passes" or "chained" (la_shape.fwd_schedule 0 / 1 / 2)."""
    return _chunk_fwd("la_chunk_fwd", q, k, v, decay, s_in, o, s_out, mode, nseg, chunk, gate_norm, subseg_chunks,
                      want_state, stream, timer, schedule)


def la_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: Optional[torch.Tensor] = None,
                         s_in: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                         s_out: Optional[torch.Tensor] = None, *, mode: Optional[str] = None, nseg: int = 1,
                         chunk: int = 64, gate_norm: float = 16.0, subseg_chunks: int = 0, want_state: bool = True,
                         schedule: str = "auto", stream=None, timer=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """la_chunk_fwd whose workspace is the library's fixed device array (the library allocates
    nothing).  Pass o (and s_out, or want_state=False) to keep the whole call free of allocations:
    the outputs this wrapper creates when they are not given come from torch's allocator."""
    return _chunk_fwd("la_chunk_fwd_noalloc", q, k, v, decay, s_in, o, s_out, mode, nseg, chunk, gate_norm,
                      subseg_chunks, want_state, stream, timer, schedule)


SCHEDULES = {"auto": 0, "passes": 1, "chained": 2}


def _chunk_fwd(fn, q, k, v, decay, s_in, o, s_out, mode, nseg, chunk, gate_norm, subseg_chunks, want_state, stream,
               timer, schedule="auto"):
    if schedule not in SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(SCHEDULES)}, not {schedule!r}")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    _dev(q, "q")
    _dev(k, "k", q.dtype, (B, H, L, dk))
    _dev(v, "v", q.dtype, (B, H, L, dv))
    m = mode_code(mode, decay)
    if decay is not None:
        _dev(decay, "decay", torch.float32)
    if s_in is not None:
        _dev(s_in, "s_in", torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    _dev(o, "o", q.dtype, (B, H, L, dv))
    if s_out is None and want_state:
        s_out = torch.empty((B, H, nseg, dk, dv), dtype=torch.float32, device=q.device)
    stride = 0
    if s_out is not None:
        _dev(s_out, "s_out", torch.float32, (B, H, nseg, dk, dv), contiguous=False)
        stride = _bh_stride(s_out, "s_out", dk * dv)
    shp = make_shape(B, H, L, dk, dv, nseg=nseg, dtype=_dtype_code(q), mode=m, gate_norm=gate_norm,
                     state_stride=stride, subseg_chunks=subseg_chunks, fwd_schedule=SCHEDULES[schedule],
                     stream=_stream(stream), timer=timer)
    _check(fn, getattr(lib(), fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(s_in), _ptr(o), _ptr(s_out),
                                  ctypes.byref(shp), chunk))
    return o, s_out


def la_chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, d_o: torch.Tensor,
                 decay: Optional[torch.Tensor] = None, s_in: Optional[torch.Tensor] = None,
                 ds_out: Optional[torch.Tensor] = None, *, mode: Optional[str] = None, nseg: int = 1,
                 chunk: int = 64, gate_norm: float = 16.0, want_decay: bool = True, want_ds_in: bool = True,
                 dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                 dv: Optional[torch.Tensor] = None, subseg_chunks: int = 0, s_sub: Optional[torch.Tensor] = None,
                 sub_len: int = 0, stream=None, timer=None):
    """Backward of la_chunk_fwd.  d_o [B,H,L,dv] (q's dtype) and ds_out [B,H,nseg,dk,dv] f32 or None are
    the loss's derivatives with respect to o and to each segment's final state.  Returns
    (dq, dk, dv, d_decay, ds_in): dq, dk [B,H,L,dk] and dv [B,H,L,dv] in q's dtype; d_decay f32 [H]
    (head decay: with respect to lambda_h) or [B,H,L,dk] (gate: with respect to g) or None; ds_in
    f32 [B,H,nseg,dk,dv] with respect to each segment's initial state, or None.
    With ``s_sub`` (f32 [B,H,nseg*nsub,dk,dv] or a view whose last three dims are dense, e.g. the
    device step's scan buffer without its last entry) the states entering every sub-segment of
    ``sub_len`` tokens are taken from it (la_chunk_bwd_states) instead of being recomputed."""
    B, H, L, dkk = q.shape
    dvv = v.shape[-1]
    _dev(q, "q")
    _dev(k, "k", q.dtype, (B, H, L, dkk))
    _dev(v, "v", q.dtype, (B, H, L, dvv))
    _dev(d_o, "d_o", q.dtype, (B, H, L, dvv))
    m = mode_code(mode, decay)
    if decay is not None:
        _dev(decay, "decay", torch.float32)
    if s_in is not None:
        _dev(s_in, "s_in", torch.float32, (B, H, dkk, dvv))
    if ds_out is not None:
        _dev(ds_out, "ds_out", torch.float32, (B, H, nseg, dkk, dvv))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _dev(dq, "dq", q.dtype, (B, H, L, dkk))
    _dev(dk, "dk", q.dtype, (B, H, L, dkk))
    _dev(dv, "dv", q.dtype, (B, H, L, dvv))
    d_decay = None
    if want_decay and m != 0:
        d_decay = torch.empty(decay.shape, dtype=torch.float32, device=q.device)
    ds_in = torch.empty((B, H, nseg, dkk, dvv), dtype=torch.float32, device=q.device) if want_ds_in else None
    shp = make_shape(B, H, L, dkk, dvv, nseg=nseg, dtype=_dtype_code(q), mode=m, gate_norm=gate_norm,
                     subseg_chunks=subseg_chunks, stream=_stream(stream), timer=timer)
    if s_sub is None:
        _check("la_chunk_bwd", lib().la_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(s_in), _ptr(d_o),
                                                  _ptr(ds_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(d_decay),
                                                  _ptr(ds_in), ctypes.byref(shp), chunk))
    else:
        nsub = -(-(L // nseg) // sub_len) if sub_len > 0 else 0
        if (s_sub.dtype != torch.float32 or s_sub.device != q.device or s_sub.dim() != 5
                or s_sub.shape[:2] != (B, H) or s_sub.shape[2] < nseg * nsub or s_sub.shape[3:] != (dkk, dvv)
                or s_sub.stride()[2:] != (dkk * dvv, dvv, 1)):
            raise ValueError("s_sub: float32 [B, H, >= nseg * nsub, dk, dv] with dense states on q's device")
        bh_stride = s_sub.stride(1) if H > 1 else (s_sub.stride(0) if B > 1 else 0)
        if B > 1 and H > 1 and s_sub.stride(0) != H * bh_stride:
            raise ValueError("s_sub: the (b, h) blocks must be evenly spaced")
        _check("la_chunk_bwd_states", lib().la_chunk_bwd_states(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(s_in), _ptr(s_sub), sub_len, bh_stride,
            _ptr(d_o), _ptr(ds_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(d_decay), _ptr(ds_in), ctypes.byref(shp),
            chunk))
    return dq, dk, dv, d_decay, ds_in


def la_chunk_fwd_decayed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: Optional[torch.Tensor] = None,
                         s_in: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                         s_out: Optional[torch.Tensor] = None, q_decayed: Optional[torch.Tensor] = None,
                         total: Optional[torch.Tensor] = None, tile_live: Optional[torch.Tensor] = None, *,
                         mode: Optional[str] = None, nseg: int = 1, chunk: int = 64, gate_norm: float = 16.0,
                         subseg_chunks: int = 0, want_state: bool = True, want_q_decayed: bool = True,
                         want_total: bool = True, want_tile_live: bool = False, stream=None, timer=None):
    """la_chunk_fwd plus q_decayed [B,H,L,dk] (q times its cumulative decay from the segment start,
    q's dtype), total [B,H,nseg,dk] f32 (each segment's total decay; may be a view with evenly
    spaced dense (b,h) blocks) and tile_live [B,H,nseg,ceil(L/nseg/64)] int32 (0: the 64-token tile
    of q_decayed is exactly zero; with tile_live, a q_decayed passed in keeps its old contents on
    such tiles).  Returns (o, s_out, q_decayed, total, tile_live); unrequested ones are None."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    _dev(q, "q")
    _dev(k, "k", q.dtype, (B, H, L, dk))
    _dev(v, "v", q.dtype, (B, H, L, dv))
    m = mode_code(mode, decay)
    if decay is not None:
        _dev(decay, "decay", torch.float32)
    if s_in is not None:
        _dev(s_in, "s_in", torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    _dev(o, "o", q.dtype, (B, H, L, dv))
    if s_out is None and want_state:
        s_out = torch.empty((B, H, nseg, dk, dv), dtype=torch.float32, device=q.device)
    stride = 0
    if s_out is not None:
        _dev(s_out, "s_out", torch.float32, (B, H, nseg, dk, dv), contiguous=False)
        stride = _bh_stride(s_out, "s_out", dk * dv)
    if q_decayed is None and want_q_decayed:
        # with tile flags the library leaves the rows of tiles flagged zero unwritten (they would be
        # zero); an array created here starts at zero so that it holds the full q * cum
        q_decayed = torch.zeros_like(q) if (tile_live is not None or want_tile_live) else torch.empty_like(q)
    if q_decayed is not None:
        _dev(q_decayed, "q_decayed", q.dtype, (B, H, L, dk))
    if total is None and want_total:
        total = torch.empty((B, H, nseg, dk), dtype=torch.float32, device=q.device)
    tstride = 0
    if total is not None:
        _dev(total, "total", torch.float32, (B, H, nseg, dk), contiguous=False)
        tstride = _bh_stride(total, "total", dk)
    ntile = (L // nseg + 63) // 64 if nseg else 0
    if tile_live is None and want_tile_live:
        tile_live = torch.empty((B, H, nseg, ntile), dtype=torch.int32, device=q.device)
    if tile_live is not None:
        _dev(tile_live, "tile_live", torch.int32, (B, H, nseg, ntile))
    shp = make_shape(B, H, L, dk, dv, nseg=nseg, dtype=_dtype_code(q), mode=m, gate_norm=gate_norm,
                     state_stride=stride, total_stride=tstride, subseg_chunks=subseg_chunks, stream=_stream(stream),
                     timer=timer)
    _check("la_chunk_fwd_decayed", lib().la_chunk_fwd_decayed(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(s_in),
                                                              _ptr(o), _ptr(s_out), _ptr(q_decayed), _ptr(total),
                                                              _ptr(tile_live), ctypes.byref(shp), chunk))
    return o, s_out, q_decayed, total, tile_live


def la_state_scan(seg_states: torch.Tensor, seg_decay: Optional[torch.Tensor],
                  out_states: Optional[torch.Tensor] = None, *, stream=None, timer=None) -> torch.Tensor:
    """Inclusive scan over axis 2: seg_states [B,H,P,dk,dv] f32, seg_decay [B,H,P,dk] f32 (dense) or
    None (no decay).  out_states may be seg_states itself (in place)."""
    B, H, P, dk, dv = seg_states.shape
    _dev(seg_states, "seg_states", torch.float32)
    if seg_decay is not None:
        _dev(seg_decay, "seg_decay", torch.float32, (B, H, P, dk))
    if out_states is None:
        out_states = torch.empty_like(seg_states)
    _dev(out_states, "out_states", torch.float32, (B, H, P, dk, dv))
    shp = make_shape(B, H, 0, dk, dv, stream=_stream(stream), timer=timer)
    _check("la_state_scan", lib().la_state_scan(_ptr(seg_states), _ptr(seg_decay), P, _ptr(out_states),
                                                ctypes.byref(shp)))
    return out_states


def la_state_correct(q: torch.Tensor, cumdecay: Optional[torch.Tensor], s_recv: torch.Tensor, o: torch.Tensor, *,
                     mode: Optional[str] = None, nseg: int = 1, seg_begin: int = 0,
                     tile_live: Optional[torch.Tensor] = None, stream=None, timer=None) -> torch.Tensor:
    """o += (q * cum) @ s_recv[p - seg_begin] for segments p >= seg_begin, in place.
    cumdecay: None (none), [H] log-decay (head) or [B,H,L,dk] cumulative decay (gate).
    s_recv: f32 [B,H,nseg-seg_begin,dk,dv], possibly a view with evenly spaced dense (b,h) blocks.
    tile_live: int32 [B,H,nseg,ceil(L/nseg/64)] from la_chunk_fwd_decayed, or None; with it
    la_state_correct_live skips the tiles flagged zero (whose correction is exactly zero)."""
    B, H, L, dk = q.shape
    dv = o.shape[-1]
    _dev(q, "q")
    _dev(o, "o", q.dtype, (B, H, L, dv))
    if cumdecay is not None:
        _dev(cumdecay, "cumdecay", torch.float32)
    m = mode_code(mode, cumdecay)
    np_ = nseg - seg_begin
    _dev(s_recv, "s_recv", torch.float32, (B, H, np_, dk, dv), contiguous=False)
    stride = _bh_stride(s_recv, "s_recv", dk * dv)
    shp = make_shape(B, H, L, dk, dv, nseg=nseg, dtype=_dtype_code(q), mode=m, seg_begin=seg_begin,
                     state_stride=stride, stream=_stream(stream), timer=timer)
    if tile_live is None:
        _check("la_state_correct", lib().la_state_correct(_ptr(q), _ptr(cumdecay), _ptr(s_recv), _ptr(o),
                                                          ctypes.byref(shp)))
    else:
        _dev(tile_live, "tile_live", torch.int32, (B, H, nseg, (L // nseg + 63) // 64))
        _check("la_state_correct_live", lib().la_state_correct_live(_ptr(q), _ptr(cumdecay), _ptr(s_recv), _ptr(o),
                                                                    _ptr(tile_live), ctypes.byref(shp)))
    return o


def la_cumdecay(decay: Optional[torch.Tensor], B: int, H: int, L: int, dk: int, *, mode: Optional[str] = None,
                nseg: int = 1, gate_norm: float = 16.0, cum: Optional[torch.Tensor] = None,
                total: Optional[torch.Tensor] = None, want_cum: bool = True, want_total: bool = True,
                device=None, stream=None, timer=None) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Returns (cumdecay [B,H,L,dk] or None, total [B,H,nseg,dk] or None), both f32.  total may be a
    view with evenly spaced dense (b,h) blocks."""
    m = mode_code(mode, decay)
    dev = decay.device if decay is not None else (device or torch.device("cuda"))
    if decay is not None:
        _dev(decay, "decay", torch.float32)
    if cum is None and want_cum:
        cum = torch.empty((B, H, L, dk), dtype=torch.float32, device=dev)
    if cum is not None:
        _dev(cum, "cum", torch.float32, (B, H, L, dk))
    if total is None and want_total:
        total = torch.empty((B, H, nseg, dk), dtype=torch.float32, device=dev)
    tstride = 0
    if total is not None:
        _dev(total, "total", torch.float32, (B, H, nseg, dk), contiguous=False)
        tstride = _bh_stride(total, "total", dk)
    shp = make_shape(B, H, L, dk, dk, nseg=nseg, mode=m, gate_norm=gate_norm, total_stride=tstride,
                     stream=_stream(stream), timer=timer)
    _check("la_cumdecay", lib().la_cumdecay(_ptr(decay), _ptr(cum), _ptr(total), ctypes.byref(shp)))
    return cum, total


def la_trim_workspace() -> None:
    """Return the current device's unused workspace-pool memory to the device."""
    _check("la_trim_workspace", lib().la_trim_workspace())


def la_chain_status(clear: bool = True) -> int:
    """Synchronise the current device and return how many chained-forward waves gave up on a wait
    since the counter was last cleared (raises LaError(LA_ERR_TIMEOUT) when any did)."""
    n = ctypes.c_int64(0)
    st = lib().la_chain_status(1 if clear else 0, ctypes.byref(n))
    _check("la_chain_status", st)
    return n.value


def la_set_chain_spin_limit(limit: int) -> int:
    """Polls per flag before a chained wave gives up, for later launches; returns the previous value
    (a negative limit only reads it)."""
    return lib().la_set_chain_spin_limit(limit)
