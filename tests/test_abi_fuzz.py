"""Seeded fuzz of the C-ABI's host-side argument checks: every entry point is called with shapes
drawn from a mix of ordinary and extreme field values (0, negative, 2^31 - 1, 2^40, 2^62, NaN
gate norms, huge strides), with distinct fake device addresses.

The checks must return a documented status and must not overflow or read out of bounds on the
way; the run under the host-sanitized build (test_sanitize.py) turns any undefined behaviour in
them (signed overflow, an invalid enum, a bad shift) into a failure.  A call whose arguments pass
validation goes on to HIP, which on a machine without a GPU returns LA_ERR_LAUNCH; the fake
addresses would be dereferenced on a GPU, so this module runs only where there is none.
"""
import ctypes
import os
import random

import pytest

from chunked_scan_amd import binding as B

pytestmark = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                reason="fake device addresses: runs only on a machine without a GPU")

OK, NULL, SHAPE, DTYPE, ALIAS, UNSUP, LAUNCH, DECAY, WORKSPACE = 0, -1, -2, -3, -4, -5, -6, -7, -8
CODES = {OK, NULL, SHAPE, DTYPE, ALIAS, UNSUP, LAUNCH, DECAY, WORKSPACE}

# fake device addresses, 2^40 apart, never dereferenced
A = [ctypes.c_void_p(0x10000000000 * (i + 1)) for i in range(16)]

I64 = [0, 1, 2, 3, 7, 64, 100, 128, 16384, -1, -(1 << 40), (1 << 31) - 1, 1 << 40, 1 << 62, (1 << 63) - 1, -(1 << 63)]
I32 = [0, 1, 2, 3, 16, 32, 64, 128, 256, -1, -64, (1 << 31) - 1, -(1 << 31)]
DIMS = [16, 32, 64, 128, 0, -1, 8, 256, 96, (1 << 31) - 1, -(1 << 31)]
NORMS = [16.0, 1.0, 0.0, -1.0, float("nan"), float("inf"), 1e-30, 1e30]


def _pick(rng, ordinary, extreme, p_extreme=0.3):
    return rng.choice(extreme) if rng.random() < p_extreme else rng.choice(ordinary)


def _random_shape(rng):
    s = B.Shape()
    s.B = _pick(rng, [1, 2, 4], I64)
    s.H = _pick(rng, [1, 2, 16], I64)
    s.nseg = _pick(rng, [1, 2, 4, 64], I32)
    s.L = _pick(rng, [64, 128, 256, 192, 16384], I64)
    if rng.random() < 0.5 and s.nseg > 0:
        s.L = s.nseg * _pick(rng, [64, 128, 65], I64, 0.1)
    s.dk = _pick(rng, [32, 64, 128], DIMS)
    s.dv = s.dk if rng.random() < 0.7 else _pick(rng, [32, 64, 128], DIMS)
    s.in_dtype = _pick(rng, [B.LA_BF16, B.LA_F32], [2, -1, 1 << 30])
    s.out_dtype = s.in_dtype if rng.random() < 0.8 else rng.choice([0, 1, 2, -5])
    s.decay_mode = _pick(rng, [0, 1, 2], [3, -1, 1 << 30])
    s.gate_norm = _pick(rng, [16.0], NORMS)
    s.seg_begin = _pick(rng, [0, 1], I32)
    s.state_stride = _pick(rng, [0], I64)
    s.total_stride = _pick(rng, [0], I64)
    s.subseg_chunks = _pick(rng, [0, 1, 4], I32)
    s.fwd_schedule = _pick(rng, [0, 1, 2], [3, -1, 1 << 30], 0.1)
    s.stream = None
    return s


def _calls(lib, s, rng):
    """(entry point, thunk) pairs for one shape; pointer arguments are fake addresses, some NULL."""
    P = ctypes.c_void_p
    sp = ctypes.byref(s)
    chunk = _pick(rng, [64, 128], [0, -64, 16, 32, 256, 100])
    P_ = _pick(rng, [1, 2, 17], I32)
    dec = A[6] if s.decay_mode in (1, 2) or rng.random() < 0.1 else None
    opt = lambda i: A[i] if rng.random() < 0.8 else None  # noqa: E731
    return [
        ("la_chunk_fwd", lambda: lib.la_chunk_fwd(A[0], A[1], A[2], dec, opt(3), A[4], opt(5), sp, chunk)),
        ("la_chunk_fwd_noalloc", lambda: lib.la_chunk_fwd_noalloc(A[0], A[1], A[2], dec, opt(3), A[4], opt(5), sp,
                                                                  chunk)),
        ("la_chunk_fwd_decayed", lambda: lib.la_chunk_fwd_decayed(A[0], A[1], A[2], dec, opt(3), A[4], opt(5),
                                                                  opt(7), opt(8), opt(9), sp, chunk)),
        ("la_state_scan", lambda: lib.la_state_scan(A[10], opt(11), P_, opt(12) or A[10], sp)),
        ("la_state_correct", lambda: lib.la_state_correct(A[0], opt(6), A[3], A[4], sp)),
        ("la_state_correct_live", lambda: lib.la_state_correct_live(A[0], opt(6), A[3], A[4], opt(9), sp)),
        ("la_cumdecay", lambda: lib.la_cumdecay(dec, opt(7), opt(8), sp)),
        ("la_chunk_bwd", lambda: lib.la_chunk_bwd(A[0], A[1], A[2], dec, opt(3), A[13], opt(14), A[7], A[8], A[9],
                                                  opt(11), opt(12), sp, chunk)),
        ("la_chunk_bwd_states", lambda: lib.la_chunk_bwd_states(
            A[0], A[1], A[2], dec, opt(3), opt(5), _pick(rng, [1, 4, 16], I32), _pick(rng, [0, 16384], I64),
            A[13], opt(14), A[7], A[8], A[9], opt(11), opt(12), sp, chunk)),
        ("la_supported", lambda: lib.la_supported(sp, chunk)),
    ]


@pytest.mark.parametrize("seed", range(4))
def test_validation_fuzz(seed):
    lib = B.lib()
    rng = random.Random(1000 + seed)
    seen = {}
    for _ in range(1500):
        s = _random_shape(rng)
        for name, call in _calls(lib, s, rng):
            r = call()
            if name == "la_supported":
                assert r in (0, 1)
                continue
            assert r in CODES, (name, r)
            seen.setdefault(name, set()).add(r)
    # every entry point rejected shapes for several reasons, and all but the one whose sub-segment
    # arguments are rarely consistent at random let some through to HIP
    for name in seen:
        if name != "la_chunk_bwd_states":
            assert LAUNCH in seen[name] or OK in seen[name], (name, seen[name])
        assert len(seen[name] - {OK, LAUNCH}) >= 2, (name, seen[name])


def test_supported_agrees_with_forward_validation():
    """la_supported(shape, chunk) is 1 exactly when la_chunk_fwd's validation passes, for
    distinct, non-NULL pointers (passing validation: LA_ERR_LAUNCH here, or LA_OK with no work)."""
    lib = B.lib()
    rng = random.Random(7)
    agree = 0
    for _ in range(3000):
        s = _random_shape(rng)
        chunk = _pick(rng, [64, 128], [0, -64, 16, 32, 256])
        dec = A[6] if s.decay_mode in (1, 2) else None
        r = lib.la_chunk_fwd(A[0], A[1], A[2], dec, None, A[4], A[5], ctypes.byref(s), chunk)
        sup = lib.la_supported(ctypes.byref(s), chunk)
        if r in (LAUNCH, OK):
            assert sup == 1, (r, s.B, s.H, s.L, s.dk, s.dv, s.nseg, s.in_dtype, s.decay_mode, chunk)
            agree += 1
        elif r in (SHAPE, UNSUP, DTYPE, DECAY):
            assert sup == 0, (r, s.B, s.H, s.L, s.dk, s.dv, s.nseg, s.in_dtype, s.decay_mode, chunk)
    assert agree > 50
