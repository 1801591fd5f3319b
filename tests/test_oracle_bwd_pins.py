"""Pins of the oracle's backward pass (``oracle.recurrence_bwd``) against things other than itself.

* Central finite differences of the forward oracle (itself pinned in test_oracle_pins.py) for a
  loss L = <W, o> + <Ws, s_out>: every input element, every mode.  L is affine in any single
  element of q, k, v or s_in, so a central difference with an exactly representable step is exact
  up to rounding; the decay parameters enter through exp / sigmoid, where a Richardson-extrapolated
  central difference is accurate to O(h^4).
* The no-decay closed form written with matrix products (a textbook route, no recurrence).
* Euler's identity for functions homogeneous of degree one: o is linear in q, and (o, s_out) are
  jointly linear in (k, s_in) and in (v, s_in), so <dq, q> = <W, o> and <dk, k> + <ds_in, s_in> =
  <dv, v> + <ds_in, s_in> = L.
* Segments are independent sequences: cutting one run in two must give the two runs' results.
* A hand-derived worked example (tests/golden/worked_example_backward_gate_half.txt), exact in binary.
A dropped term (the diagonal, the s_in path, the ds_out path), a decay applied on the wrong side
of the add, a transposed gradient or a wrong chain-rule factor fails at least one of these.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import GATE, HEAD, NONE

pytestmark = pytest.mark.filterwarnings("ignore")


def _grid(rng, shape, step=2.0 ** -6, scale=1.0):
    """Values on a grid of ``step``: x and x +- 2^-4 are exact in float32."""
    return (np.round(rng.standard_normal(shape) * scale / step) * step).astype(np.float32)


def _problem(seed, mode, B=1, H=2, L=6, dk=3, dv=2, nseg=1, with_s_in=True):
    rng = np.random.default_rng(seed)
    q, k = _grid(rng, (B, H, L, dk)), _grid(rng, (B, H, L, dk))
    v = _grid(rng, (B, H, L, dv))
    if mode == HEAD:
        decay = (-np.round(rng.uniform(0.05, 0.6, H) * 4096) / 4096).astype(np.float32)
    elif mode == GATE:
        decay = (np.round(rng.standard_normal((B, H, L, dk)) * 4096) / 4096).astype(np.float32)
    else:
        decay = None
    s_in = rng.standard_normal((B, H, dk, dv)) if with_s_in else None
    W = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    Ws = rng.standard_normal((B, H, nseg, dk, dv))
    return q, k, v, decay, s_in, W, Ws


def _loss(q, k, v, mode, decay, s_in, W, Ws, nseg):
    o, s_out = oracle.recurrence(q, k, v, mode, decay, s_in, nseg=nseg, threads=1)
    return float(np.sum(W.astype(np.float64) * o) + np.sum(Ws * s_out))


def _fd(f, x, idx, h):
    """Central difference of f with respect to element idx of x (a copy is perturbed)."""
    xp, xm = x.copy(), x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (f(xp) - f(xm)) / (2 * h)


@pytest.mark.parametrize("mode", [NONE, HEAD, GATE])
@pytest.mark.parametrize("nseg", [1, 2])
def test_bwd_matches_finite_differences(mode, nseg):
    q, k, v, decay, s_in, W, Ws = _problem(11 + mode + 7 * nseg, mode, nseg=nseg)
    dq, dk, dv, dd, ds_in = oracle.recurrence_bwd(q, k, v, W, mode, decay, s_in, Ws, nseg=nseg, threads=1)
    h = 2.0 ** -4
    checks = [
        (dq, q, lambda x: _loss(x, k, v, mode, decay, s_in, W, Ws, nseg)),
        (dk, k, lambda x: _loss(q, x, v, mode, decay, s_in, W, Ws, nseg)),
        (dv, v, lambda x: _loss(q, k, x, mode, decay, s_in, W, Ws, nseg)),
        (ds_in[:, :, 0], s_in, lambda x: _loss(q, k, v, mode, decay, x, W, Ws, nseg)),
    ]
    for grad, x, f in checks:
        fd = np.zeros(x.shape)
        for idx in np.ndindex(*x.shape):
            fd[idx] = _fd(f, x, idx, h)
        assert np.max(np.abs(fd - grad)) <= 1e-9 * max(1.0, np.max(np.abs(grad)))
    if mode != NONE:
        f = lambda x: _loss(q, k, v, mode, x, s_in, W, Ws, nseg)  # noqa: E731
        fd = np.zeros(decay.shape)
        for idx in np.ndindex(*decay.shape):
            d1, d2 = _fd(f, decay, idx, 2.0 ** -8), _fd(f, decay, idx, 2.0 ** -9)
            fd[idx] = (4 * d2 - d1) / 3  # Richardson: the h^2 term cancels
        assert np.max(np.abs(fd - dd)) <= 1e-7 * max(1.0, np.max(np.abs(dd)))


def test_bwd_ds_in_of_later_segments_is_the_state_derivative():
    """For segment p >= 1 the initial state is zero, but its derivative is what the backward state
    scan carries: adding a state X to segment 1's start changes L by <ds_in[1], X> exactly.  The
    perturbed run is written as the same recurrence with segment 1 started from X, i.e. a separate
    one-segment run over segment 1's tokens."""
    mode = GATE
    q, k, v, decay, s_in, W, Ws = _problem(3, mode, L=8, nseg=2)
    _, _, _, _, ds_in = oracle.recurrence_bwd(q, k, v, W, mode, decay, s_in, Ws, nseg=2, threads=1)
    half = slice(4, 8)
    rng = np.random.default_rng(9)
    X = rng.standard_normal(s_in.shape)

    def seg1_loss(x0):
        o, s_out = oracle.recurrence(q[:, :, half], k[:, :, half], v[:, :, half], mode, decay[:, :, half], x0,
                                     threads=1)
        return float(np.sum(W[:, :, half].astype(np.float64) * o) + np.sum(Ws[:, :, 1] * s_out[:, :, 0]))

    got = seg1_loss(X) - seg1_loss(np.zeros_like(X))
    assert abs(got - np.sum(ds_in[:, :, 1] * X)) <= 1e-10 * max(1.0, abs(got))


@pytest.mark.parametrize("nseg", [1, 2])
def test_bwd_no_decay_closed_form(nseg):
    """a = 1: o = tril(Q K^T) V + Q s_in and s_out = s_in + K^T V per segment, so
    dq = tril(W V^T) K + W s_in^T, dk = tril(W V^T)^T Q + V Ws^T, dv = tril(Q K^T)^T W + K Ws,
    ds_in = Q^T W + Ws (matrix products; s_in enters segment 0 only)."""
    rng = np.random.default_rng(21)
    B, H, L, dk, dv = 1, 2, 64, 8, 6
    q, k = _grid(rng, (B, H, L, dk)), _grid(rng, (B, H, L, dk))
    v, W = _grid(rng, (B, H, L, dv)), _grid(rng, (B, H, L, dv))
    s_in = rng.standard_normal((B, H, dk, dv))
    Ws = rng.standard_normal((B, H, nseg, dk, dv))
    dq, dkk, dvv, dd, ds_in = oracle.recurrence_bwd(q, k, v, W, NONE, None, s_in, Ws, nseg=nseg)
    assert dd is None
    Ls = L // nseg
    for b in range(B):
        for h in range(H):
            for p in range(nseg):
                sl = slice(p * Ls, (p + 1) * Ls)
                Q, K, V, Wo = (x[b, h, sl].astype(np.float64) for x in (q, k, v, W))
                Sin = s_in[b, h] if p == 0 else np.zeros((dk, dv))
                WV = np.tril(Wo @ V.T)
                np.testing.assert_allclose(dq[b, h, sl], WV @ K + Wo @ Sin.T, rtol=0, atol=1e-11)
                np.testing.assert_allclose(dkk[b, h, sl], WV.T @ Q + V @ Ws[b, h, p].T, rtol=0, atol=1e-11)
                np.testing.assert_allclose(dvv[b, h, sl], np.tril(Q @ K.T).T @ Wo + K @ Ws[b, h, p], rtol=0,
                                           atol=1e-11)
                np.testing.assert_allclose(ds_in[b, h, p], Q.T @ Wo + Ws[b, h, p], rtol=0, atol=1e-11)


@pytest.mark.parametrize("mode", [NONE, HEAD, GATE])
def test_bwd_euler_identities(mode):
    q, k, v, decay, s_in, W, Ws = _problem(31 + mode, mode, B=2, H=3, L=40, dk=5, dv=4)
    o, s_out = oracle.recurrence(q, k, v, mode, decay, s_in)
    dq, dk, dv, _, ds_in = oracle.recurrence_bwd(q, k, v, W, mode, decay, s_in, Ws)
    Lo = np.sum(W.astype(np.float64) * o)
    L = Lo + np.sum(Ws * s_out)
    si = np.sum(ds_in[:, :, 0] * s_in)
    tol = 1e-11 * (np.sum(np.abs(W.astype(np.float64) * o)) + np.sum(np.abs(Ws * s_out)))
    assert abs(np.sum(dq * q) - Lo) <= tol
    assert abs(np.sum(dk * k) + si - L) <= tol
    assert abs(np.sum(dv * v) + si - L) <= tol


@pytest.mark.parametrize("mode", [NONE, HEAD, GATE])
def test_bwd_segments_are_independent_runs(mode):
    """nseg = 2 is the same op sequence as two separate one-segment runs (s_in to the first only):
    bit-identical in fp64."""
    q, k, v, decay, s_in, W, Ws = _problem(41 + mode, mode, B=1, H=2, L=16, dk=4, dv=3, nseg=2)
    both = oracle.recurrence_bwd(q, k, v, W, mode, decay, s_in, Ws, nseg=2)
    for p, sl in enumerate((slice(0, 8), slice(8, 16))):
        dec = decay[:, :, sl] if mode == GATE else decay
        one = oracle.recurrence_bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], W[:, :, sl], mode, dec,
                                    s_in if p == 0 else None, Ws[:, :, p:p + 1])
        for a, b in zip(both[:3], one[:3]):
            assert np.array_equal(a[:, :, sl], b)
        assert np.array_equal(both[4][:, :, p], one[4][:, :, 0])
        if mode == GATE:
            assert np.array_equal(both[3][:, :, sl], one[3])
    if mode == HEAD:
        parts = [oracle.recurrence_bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], W[:, :, sl], mode, decay,
                                       s_in if p == 0 else None, Ws[:, :, p:p + 1])[3]
                 for p, sl in enumerate((slice(0, 8), slice(8, 16)))]
        assert np.array_equal(both[3], parts[0] + parts[1])


def test_golden_hand_backward_example():
    """Every derivative of the hand-worked two-token, 2 x 2 example, exactly."""
    rows = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example_backward_gate_half.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rows[key] = np.array([float(x) for x in vals])
    tok = lambda x: rows[x].reshape(1, 1, 2, 2).astype(np.float32)  # noqa: E731
    dq, dk, dv, dg, ds_in = oracle.recurrence_bwd(tok("q"), tok("k"), tok("v"), tok("d_o"), GATE,
                                                  np.zeros((1, 1, 2, 2), np.float32),
                                                  rows["s_in"].reshape(1, 1, 2, 2),
                                                  rows["ds_out"].reshape(1, 1, 1, 2, 2), gate_norm=1.0)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg)):
        assert np.array_equal(got.reshape(-1), rows[name]), name
    assert np.array_equal(ds_in.reshape(-1), rows["ds_in"])
