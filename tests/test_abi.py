"""C-ABI checks that need no GPU: the library loads, exports every symbol include/la_chunk.h
declares, the struct layout matches, and argument validation returns the documented codes.

Only calls that fail validation are made here (validation happens on the host before any HIP
call); the pointers are fake addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from chunked_scan_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la_chunk.h")

OK, NULL, SHAPE, DTYPE, ALIAS, UNSUP, LAUNCH, DECAY, WORKSPACE, TIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("liblachunk.so is not built (run __graft_entry__.build())")
    return B.lib()


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(la_\w+)\s*\(", txt, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.la_version() >> 16 == 1
    for code in (OK, NULL, SHAPE, DTYPE, ALIAS, UNSUP, LAUNCH, DECAY, WORKSPACE, TIMEOUT):
        assert lib.la_status_str(code) and lib.la_status_str(code) != b"unknown status", code
        assert B.STATUS[code]
    assert lib.la_status_str(12345) == b"unknown status"


def test_chain_spin_limit_setting(lib):
    # host-side setting only: no launch, no device
    default = lib.la_set_chain_spin_limit(-1)
    assert default == 1 << 22
    assert lib.la_set_chain_spin_limit(7) == default
    assert lib.la_set_chain_spin_limit(-5) == 7  # negative: read only
    assert lib.la_set_chain_spin_limit(default) == 7


def test_shape_struct_layout():
    # offsets follow the C layout of la_shape in include/la_chunk.h
    assert B.Shape.dk.offset == 24 and B.Shape.gate_norm.offset == 48
    assert B.Shape.state_stride.offset == 56 and B.Shape.total_stride.offset == 64
    assert B.Shape.subseg_chunks.offset == 72
    assert B.Shape.stream.offset == 80 and B.Shape.trace.offset == 88 and ctypes.sizeof(B.Shape) == 96
    assert B.Trace.capacity.offset == 256 and B.Trace.name.offset == 264 and ctypes.sizeof(B.Trace) == 392


# fake device addresses, far apart, never dereferenced
Q, K, V, O, S_IN, S_OUT, DEC = (0x10000000000 * (i + 1) for i in range(7))


def fwd(lib, shp, q=Q, k=K, v=V, dec=None, s_in=None, o=O, s_out=S_OUT, chunk=64):
    P = ctypes.c_void_p
    return lib.la_chunk_fwd(P(q), P(k), P(v), P(dec), P(s_in), P(o), P(s_out), ctypes.byref(shp), chunk)


def shape(**kw):
    d = dict(B=1, H=2, L=128, dk=64, dv=64, nseg=1, dtype=B.LA_BF16, mode=0)
    d.update(kw)
    return B.make_shape(d.pop("B"), d.pop("H"), d.pop("L"), d.pop("dk"), d.pop("dv"), **d)


def test_fwd_validation(lib):
    assert lib.la_chunk_fwd(None, None, None, None, None, None, None, None, 64) == NULL
    assert fwd(lib, shape(L=-1)) == SHAPE
    assert fwd(lib, shape(B=-1)) == SHAPE
    assert fwd(lib, shape(nseg=0)) == SHAPE
    assert fwd(lib, shape(L=100, nseg=3)) == SHAPE          # L % nseg != 0
    assert fwd(lib, shape(dk=0)) == SHAPE
    assert fwd(lib, shape(dk=96)) == UNSUP
    assert fwd(lib, shape(dv=256)) == UNSUP                    # 256 only with dk = dv
    assert fwd(lib, shape(dk=256, dv=256), chunk=32) == UNSUP  # d = 256: 64-token chunks
    assert fwd(lib, shape(dk=256, dv=256, dtype=B.LA_F32)) == UNSUP
    assert fwd(lib, shape(dk=256, dv=256, mode=2), dec=DEC) == UNSUP  # no gate at d = 256
    assert lib.la_supported(ctypes.byref(shape(dk=256, dv=256, mode=1)), 64) == 1
    assert fwd(lib, shape(), chunk=0) == SHAPE
    assert fwd(lib, shape(), chunk=48) == UNSUP
    # 128-token chunks: bf16 with dk = dv in {32, 64}, and 128 without gate decay
    assert fwd(lib, shape(dk=128, dv=128, mode=2), dec=DEC, chunk=128) == UNSUP
    assert lib.la_supported(ctypes.byref(shape(dk=128, dv=128)), 128) == 1
    assert fwd(lib, shape(dtype=B.LA_F32), chunk=128) == UNSUP
    assert fwd(lib, shape(dk=64, dv=32), chunk=128) == UNSUP
    assert fwd(lib, shape(dk=16, dv=16), chunk=128) == UNSUP
    assert fwd(lib, shape(subseg_chunks=-1)) == SHAPE
    bad = shape()
    bad.in_dtype = 7
    bad.out_dtype = 7
    assert fwd(lib, bad) == DTYPE
    mixed = shape()
    mixed.out_dtype = B.LA_F32
    assert fwd(lib, mixed) == DTYPE
    assert fwd(lib, shape(mode=3)) == DECAY
    assert fwd(lib, shape(mode=2, gate_norm=0.0)) == DECAY
    assert fwd(lib, shape(mode=2, gate_norm=float("nan")), dec=DEC) == DECAY
    assert fwd(lib, shape(mode=0), dec=DEC) == DECAY           # none mode takes no decay
    assert fwd(lib, shape(mode=1)) == NULL                     # head mode needs lambda_h
    assert fwd(lib, shape(mode=2)) == NULL                     # gate mode needs g
    assert fwd(lib, shape(), q=0) == NULL
    assert fwd(lib, shape(), o=0) == NULL
    assert fwd(lib, shape(), o=Q + 64) == ALIAS                # o overlaps q
    assert fwd(lib, shape(), s_out=V) == ALIAS                 # s_out overlaps v
    assert fwd(lib, shape(), s_in=S_IN, s_out=S_IN + 16) == ALIAS
    assert fwd(lib, shape(), o=S_OUT) == ALIAS                 # o overlaps s_out
    assert fwd(lib, shape(B=1 << 40, H=1 << 20)) == SHAPE      # byte counts would overflow
    # empty problems validate and enqueue nothing
    assert fwd(lib, shape(B=0), q=0, k=0, v=0, o=0, s_out=0) == OK
    assert fwd(lib, shape(H=0), q=0, k=0, v=0, o=0, s_out=0) == OK


def test_supported(lib):
    assert lib.la_supported(ctypes.byref(shape()), 64) == 1
    assert lib.la_supported(ctypes.byref(shape(dk=128, dv=128)), 64) == 1
    assert lib.la_supported(ctypes.byref(shape(dtype=B.LA_F32, dk=16, dv=16)), 16) == 1
    assert lib.la_supported(ctypes.byref(shape(dk=256)), 64) == 0
    assert lib.la_supported(ctypes.byref(shape()), 128) == 1
    assert lib.la_supported(ctypes.byref(shape(dk=32, dv=32)), 128) == 1
    assert lib.la_supported(ctypes.byref(shape(dk=128, dv=128)), 128) == 1
    assert lib.la_supported(ctypes.byref(shape(dk=128, dv=128, mode=2)), 128) == 0
    assert lib.la_supported(ctypes.byref(shape(dtype=B.LA_F32)), 128) == 0
    assert lib.la_supported(ctypes.byref(shape()), 256) == 0
    assert lib.la_supported(None, 64) == 0


def test_scan_validation(lib):
    P = ctypes.c_void_p
    s = shape()
    assert lib.la_state_scan(P(Q), P(DEC), 4, P(S_OUT), None) == NULL
    assert lib.la_state_scan(P(Q), P(DEC), 0, P(S_OUT), ctypes.byref(s)) == SHAPE
    assert lib.la_state_scan(None, P(DEC), 4, P(S_OUT), ctypes.byref(s)) == NULL
    assert lib.la_state_scan(P(Q), P(DEC), 4, P(Q + 64), ctypes.byref(s)) == ALIAS   # partial overlap
    assert lib.la_state_scan(P(Q), P(S_OUT + 16), 4, P(S_OUT), ctypes.byref(s)) == ALIAS
    assert lib.la_state_scan(P(Q + 4), P(DEC), 4, P(S_OUT), ctypes.byref(s)) == UNSUP  # not 16-byte aligned
    assert lib.la_state_scan(P(Q), P(DEC), 4, P(S_OUT), ctypes.byref(shape(dv=6))) == UNSUP
    assert lib.la_state_scan(P(Q), P(DEC), 4, P(S_OUT), ctypes.byref(shape(B=0))) == OK


def test_correct_validation(lib):
    P = ctypes.c_void_p

    def call(shp, q=Q, cum=None, s=S_IN, o=O):
        return lib.la_state_correct(P(q), P(cum), P(s), P(o), ctypes.byref(shp))

    assert lib.la_state_correct(P(Q), None, P(S_IN), P(O), None) == NULL
    assert call(shape(seg_begin=2)) == SHAPE
    assert call(shape(seg_begin=-1)) == SHAPE
    assert call(shape(nseg=4, seg_begin=1, state_stride=64 * 64)) == SHAPE   # stride smaller than 3 states
    assert call(shape(mode=1)) == NULL
    assert call(shape(mode=0), cum=DEC) == DECAY
    assert call(shape(), o=Q + 2) == ALIAS
    assert call(shape(), s=O + 100) == ALIAS
    assert call(shape(), q=0) == NULL
    assert call(shape(seg_begin=1), q=0, s=0, o=0) == OK                   # nothing to correct
    mixed = shape()
    mixed.out_dtype = B.LA_F32
    assert call(mixed) == DTYPE


def test_cumdecay_validation(lib):
    P = ctypes.c_void_p
    assert lib.la_cumdecay(P(DEC), P(Q), P(K), None) == NULL
    assert lib.la_cumdecay(None, P(Q), P(K), ctypes.byref(shape(mode=1))) == NULL
    assert lib.la_cumdecay(P(DEC), P(Q), P(K), ctypes.byref(shape(mode=0))) == DECAY
    assert lib.la_cumdecay(P(DEC), P(DEC + 4), None, ctypes.byref(shape(mode=2))) == ALIAS
    assert lib.la_cumdecay(P(DEC), None, None, ctypes.byref(shape(mode=1))) == OK    # nothing requested


# more fake addresses for the backward's derivative arguments
DO, DSO, DQ, DK, DV, DDEC, DSIN = (0x10000000000 * (i + 8) for i in range(7))


def bwd(lib, shp, q=Q, k=K, v=V, dec=None, s_in=None, d_o=DO, ds_out=None, dq=DQ, dk=DK, dv=DV, d_dec=None,
        ds_in=None, chunk=64):
    P = ctypes.c_void_p
    return lib.la_chunk_bwd(P(q), P(k), P(v), P(dec), P(s_in), P(d_o), P(ds_out), P(dq), P(dk), P(dv), P(d_dec),
                            P(ds_in), ctypes.byref(shp), chunk)


def bwd_states(lib, shp, s_sub, sub_len, sub_stride=0, dq=DQ, chunk=64):
    P = ctypes.c_void_p
    return lib.la_chunk_bwd_states(P(Q), P(K), P(V), P(None), P(None), P(s_sub), sub_len, sub_stride, P(DO), P(None),
                                   P(dq), P(DK), P(DV), P(None), P(None), ctypes.byref(shp), chunk)


def test_bwd_states_validation(lib):
    SSUB = 0x10000000000 * 20
    shp = shape(L=512)  # B1 H2 d64 bf16: 2 sub-segments of 256 tokens per (b, h)
    assert bwd_states(lib, shp, None, 256) == NULL
    assert bwd_states(lib, shp, SSUB, 0) == SHAPE
    assert bwd_states(lib, shp, SSUB, -64) == SHAPE
    assert bwd_states(lib, shp, SSUB, 100) == SHAPE                    # not a multiple of the chunk
    assert bwd_states(lib, shp, SSUB, 256, sub_stride=-1) == SHAPE
    assert bwd_states(lib, shp, SSUB, 256, sub_stride=2 * 64 * 64 - 1) == SHAPE  # below one (b,h) block
    assert bwd_states(lib, shp, SSUB, 256, dq=SSUB + 64) == ALIAS       # dq overlaps the states
    assert bwd_states(lib, shape(L=512, dk=96), SSUB, 256) == UNSUP


def test_bwd_validation(lib):
    assert lib.la_chunk_bwd(*([None] * 12), None, 64) == NULL
    assert bwd(lib, shape(L=-1)) == SHAPE
    assert bwd(lib, shape(nseg=0)) == SHAPE
    assert bwd(lib, shape(L=100, nseg=3)) == SHAPE
    assert bwd(lib, shape(), chunk=0) == SHAPE
    assert bwd(lib, shape(), chunk=48) == UNSUP
    assert bwd(lib, shape(), chunk=128) == UNSUP  # 128-token chunks: forward only
    assert bwd(lib, shape(dk=96)) == UNSUP
    assert bwd(lib, shape(state_stride=64 * 64 - 1)) == SHAPE       # smaller than one segment's state
    assert bwd(lib, shape(subseg_chunks=-1)) == SHAPE
    mixed = shape()
    mixed.out_dtype = B.LA_F32
    assert bwd(lib, mixed) == DTYPE
    assert bwd(lib, shape(mode=3)) == DECAY
    assert bwd(lib, shape(mode=0), dec=DEC) == DECAY                # none mode takes no decay
    assert bwd(lib, shape(mode=0), d_dec=DDEC) == DECAY             # ... and returns no decay derivative
    assert bwd(lib, shape(mode=1)) == NULL                          # head mode needs lambda_h
    assert bwd(lib, shape(mode=2)) == NULL                          # gate mode needs g
    for arg in ("q", "k", "v", "d_o", "dq", "dk", "dv"):
        assert bwd(lib, shape(), **{arg: 0}) == NULL, arg
    assert bwd(lib, shape(), dq=Q + 64) == ALIAS                    # dq overlaps q
    assert bwd(lib, shape(), dv=DO) == ALIAS                        # dv overlaps d_o
    assert bwd(lib, shape(), dk=DV + 128) == ALIAS                  # two outputs overlap
    assert bwd(lib, shape(), ds_out=DSO, ds_in=DSO + 256) == ALIAS  # ds_in overlaps ds_out
    assert bwd(lib, shape(mode=1), dec=DEC, d_dec=DEC) == ALIAS     # d lambda overwrites lambda
    assert bwd(lib, shape(mode=2), dec=DEC, d_dec=DEC + 1024) == ALIAS
    assert bwd(lib, shape(), s_in=S_IN, ds_in=S_IN) == ALIAS
    # an empty problem validates and enqueues nothing
    assert bwd(lib, shape(B=0), q=0, k=0, v=0, d_o=0, dq=0, dk=0, dv=0) == OK


def test_trace_validation(lib):
    t = B.Trace()
    t.capacity = 17  # more than LA_TRACE_MAX_KERNELS
    s = shape()
    s.trace = ctypes.pointer(t)
    assert fwd(lib, s) == SHAPE
    t.capacity = 2  # events missing
    assert fwd(lib, s) == NULL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_noalloc_validation_and_workspace_bound(lib):
    P = ctypes.c_void_p

    def call(shp, chunk=64, dec=None):
        return lib.la_chunk_fwd_noalloc(P(Q), P(K), P(V), P(dec), None, P(O), P(S_OUT), ctypes.byref(shp), chunk)

    # the same validation as la_chunk_fwd, before anything else
    assert lib.la_chunk_fwd_noalloc(None, None, None, None, None, None, None, None, 64) == NULL
    assert call(shape(L=100, nseg=3)) == SHAPE
    assert call(shape(dk=96)) == UNSUP
    assert call(shape(), dec=DEC) == DECAY
    # one 64-token chunk per sub-segment over 16 heads x 16k tokens at d = 128 needs 255 x 16
    # sub-segment states of 64 KiB (+ decay vectors): far beyond the fixed workspace, rejected on
    # the host (nothing is enqueued, so no GPU is needed to see it)
    big = shape(H=16, L=16384, dk=128, dv=128, subseg_chunks=1)
    assert call(big) == WORKSPACE
    assert 255 * 16 * (128 * 128 + 128) * 4 > B.NOALLOC_SCRATCH_BYTES
    # 128-token chunks with one chunk per sub-segment: 127 x 64 states of 16 KiB at d = 64
    assert call(shape(H=64, L=16384, dk=64, dv=64, subseg_chunks=1), chunk=128) == WORKSPACE
