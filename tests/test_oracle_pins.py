"""Pins of the fp64 CPU oracle against things other than itself (CPU only).

Each test checks the oracle against a closed form, a brute-force formula written a different
way, a textbook routine (BLAS matmul), an exact hand-derived example, or an invariant that
the mathematics fixes.  They are chosen so that a plausible slip in the oracle (a dropped
term, decay applied after instead of before the add, the diagonal left out of the causal
mask, a transposed state, a wrong segment offset, a one-hop scan) fails at least one of them.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import GATE, HEAD, NONE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape, scale=1.0):
    # Values exactly representable in float32, as the oracle takes float inputs.
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _log_decay(mode, decay, B, H, L, dk, gate_norm=16.0):
    """log a_t[d] for every (b,h,t,d), computed in log space (softplus), not as the oracle does."""
    if mode == NONE:
        return np.zeros((B, H, L, dk))
    if mode == HEAD:
        lam = np.asarray(decay, np.float64)
        return np.broadcast_to(lam[None, :, None, None], (B, H, L, dk)).copy()
    g = np.asarray(decay, np.float64)
    # log sigmoid(g) = -log(1 + exp(-g)) = -logaddexp(0, -g)
    return -np.logaddexp(0.0, -g) / gate_norm


def _brute_force(q, k, v, mode, decay, s_in, gate_norm=16.0):
    """O(L^2) causal weighted attention: for every t and j <= t,
    o_t += sum_d q_t[d] k_j[d] exp(sum_{s=j+1..t} log a_s[d]) v_j, plus the decayed s_in term
    sum_d q_t[d] exp(sum_{s<=t} log a_s[d]) s_in[d,:].  Written from the unrolled recurrence."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    la = _log_decay(mode, decay, B, H, L, dk, gate_norm)
    cs = np.cumsum(la, axis=2)  # inclusive: cs[t] = sum_{s<=t} log a_s
    o = np.zeros((B, H, L, dv))
    s_out = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                for j in range(t + 1):
                    w = np.exp(cs[b, h, t] - cs[b, h, j])  # prod_{s=j+1..t} a_s
                    o[b, h, t] += np.dot(q[b, h, t] * k[b, h, j] * w, np.ones(dk)) * v[b, h, j]
                if s_in is not None:
                    o[b, h, t] += (q[b, h, t] * np.exp(cs[b, h, t])) @ s_in[b, h]
            for j in range(L):
                w = np.exp(cs[b, h, L - 1] - cs[b, h, j])
                s_out[b, h] += np.outer(k[b, h, j] * w, v[b, h, j])
            if s_in is not None:
                s_out[b, h] += np.exp(cs[b, h, L - 1])[:, None] * s_in[b, h]
    return o, s_out


def _rel(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / den


@pytest.mark.parametrize("mode", [NONE, HEAD, GATE])
def test_brute_force_tiny(mode):
    rng = np.random.default_rng(10 + mode)
    B, H, L, dk, dv = 2, 2, 19, 5, 4
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    decay = {NONE: None, HEAD: -np.array([0.05, 0.4], np.float32),
             GATE: _rand(rng, B, H, L, dk, scale=2.0)}[mode]
    s_in = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.recurrence(q, k, v, mode, decay, s_in, gate_norm=4.0)
    ob, sb = _brute_force(q, k, v, mode, decay, s_in, gate_norm=4.0)
    assert _rel(o, ob) < 1e-12
    assert _rel(s[:, :, 0], sb) < 1e-12


def test_golden_hand_example():
    rows = {}
    with open(os.path.join(GOLDEN, "worked_example_gate_half.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rows[key] = np.array([float(x) for x in vals])
    q = rows["q"].reshape(1, 1, 3, 2)
    k = rows["k"].reshape(1, 1, 3, 2)
    v = rows["v"].reshape(1, 1, 3, 2)
    s_in = rows["s_in"].reshape(1, 1, 2, 2)
    o, s = oracle.recurrence(q, k, v, GATE, np.zeros((1, 1, 3, 2), np.float32), s_in, gate_norm=1.0)
    assert np.array_equal(o.ravel(), rows["gate_half_o"])
    assert np.array_equal(s.ravel(), rows["gate_half_s_out"])
    o, s = oracle.recurrence(q, k, v, NONE, None, s_in)
    assert np.array_equal(o.ravel(), rows["none_o"])
    assert np.array_equal(s.ravel(), rows["none_s_out"])


def test_closed_form_no_decay():
    """a = 1: O = tril(Q K^T) V + Q s_in and S_out = s_in + K^T V (BLAS matmuls)."""
    rng = np.random.default_rng(1)
    B, H, L, dk, dv = 1, 3, 96, 8, 6
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    s_in = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.recurrence(q, k, v, NONE, None, s_in)
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    for h in range(H):
        ref = np.tril(Q[0, h] @ K[0, h].T) @ V[0, h] + Q[0, h] @ s_in[0, h]
        assert _rel(o[0, h], ref) < 1e-13
        assert _rel(s[0, h, 0], s_in[0, h] + K[0, h].T @ V[0, h]) < 1e-13


def test_closed_form_zero_decay():
    """a = 0 (log-decay -inf): each token sees only itself, o_t = (q_t . k_t) v_t, S_out = k_L v_L^T."""
    rng = np.random.default_rng(2)
    B, H, L, dk, dv = 1, 2, 17, 6, 5
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    s_in = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.recurrence(q, k, v, HEAD, np.full(H, -np.inf, np.float32), s_in)
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    ref = np.sum(Q * K, axis=-1, keepdims=True) * V
    assert _rel(o, ref) < 1e-14
    assert _rel(s[0, :, 0], np.einsum("hd,hc->hdc", K[0, :, -1], V[0, :, -1])) < 1e-14


def test_toeplitz_constant_scalar_decay():
    """Constant a: O = (tril(QK^T) * D) V + diag(a^t) Q s_in with D[t,j] = a^(t-j), t 1-based."""
    rng = np.random.default_rng(3)
    B, H, L, dk, dv = 1, 2, 80, 7, 5
    lam = np.array([-0.03, -0.3], np.float32)
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    s_in = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.recurrence(q, k, v, HEAD, lam, s_in)
    t = np.arange(1, L + 1, dtype=np.float64)
    for h in range(H):
        a = np.exp(np.float64(lam[h]))
        D = np.tril(a ** (t[:, None] - t[None, :]))
        Q, K, V = (x[0, h].astype(np.float64) for x in (q, k, v))
        ref = ((Q @ K.T) * D) @ V + (a ** t)[:, None] * (Q @ s_in[0, h])
        assert _rel(o[0, h], ref) < 1e-12
        sref = (K * (a ** (L - t))[:, None]).T @ V + a ** L * s_in[0, h]
        assert _rel(s[0, h, 0], sref) < 1e-12


def test_gate_power_of_sigmoid():
    """g = 0 gives a = 2^(-1/gate_norm) exactly as a power; compare with a scalar-decay run."""
    rng = np.random.default_rng(4)
    B, H, L, dk, dv = 1, 1, 40, 4, 3
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    o_g, s_g = oracle.recurrence(q, k, v, GATE, np.zeros((B, H, L, dk), np.float32), None, gate_norm=16.0)
    # Constant a = 2^(-1/16): closed-form Toeplitz with a plain power, no sigmoid involved.
    a = 2.0 ** (-1.0 / 16.0)
    t = np.arange(1, L + 1, dtype=np.float64)
    D = np.tril(a ** (t[:, None] - t[None, :]))
    Q, K, V = (x[0, 0].astype(np.float64) for x in (q, k, v))
    assert _rel(o_g[0, 0], ((Q @ K.T) * D) @ V) < 1e-13


def test_linearity_in_initial_state():
    rng = np.random.default_rng(5)
    B, H, L, dk, dv = 1, 2, 33, 6, 4
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    g = _rand(rng, B, H, L, dk)
    s1, s2 = rng.standard_normal((2, B, H, dk, dv))
    o1, _ = oracle.recurrence(q, k, v, GATE, g, s1)
    o2, _ = oracle.recurrence(q, k, v, GATE, g, s2)
    o12, _ = oracle.recurrence(q, k, v, GATE, g, s1 + s2)
    o0, _ = oracle.recurrence(q, k, v, GATE, g, None)
    assert _rel(o12 - o0, (o1 - o0) + (o2 - o0)) < 1e-12


@pytest.mark.parametrize("mode", [NONE, HEAD, GATE])
def test_split_resume_bit_identical(mode):
    """Running the first half, then the second half from the carried state, is the same op
    sequence as one pass, so the fp64 results must be bit-identical."""
    rng = np.random.default_rng(6 + mode)
    B, H, L, dk, dv = 2, 2, 64, 8, 8
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    dec = {NONE: None, HEAD: np.array([-0.1, -0.01], np.float32), GATE: _rand(rng, B, H, L, dk)}[mode]
    s_in = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.recurrence(q, k, v, mode, dec, s_in)
    h = L // 2
    d1 = None if dec is None or mode == HEAD else dec[:, :, :h]
    d2 = None if dec is None or mode == HEAD else dec[:, :, h:]
    if mode == HEAD:
        d1 = d2 = dec
    oa, sa = oracle.recurrence(q[:, :, :h], k[:, :, :h], v[:, :, :h], mode, d1, s_in)
    ob, sb = oracle.recurrence(q[:, :, h:], k[:, :, h:], v[:, :, h:], mode, d2, sa[:, :, 0])
    assert np.array_equal(np.concatenate([oa, ob], axis=2), o)
    assert np.array_equal(sb, s)


def _decomposed(q, k, v, mode, dec, s_in, P, scan=None):
    """ZeCO-style route: every segment from a zero state (segment 0 from s_in), an inclusive
    scan of the segment states, then the rank-dk output correction with the incoming state."""
    B, H, L, dk = q.shape
    o_loc, seg = oracle.recurrence(q, k, v, mode, dec, s_in, nseg=P)
    cum, tot = oracle.cumdecay(B, H, L, dk, mode, dec, nseg=P)
    out = (scan or oracle.state_scan)(seg, tot)
    o = oracle.state_correct(q, cum, out[:, :, :P - 1], o_loc, nseg=P, seg_begin=1)
    return o, out


def _one_hop_scan(seg_states, seg_decay):
    """A planted mistake: each segment folds in only its neighbour's *local* state, which is
    what the All-Scan pseudo-code does if taken literally (it forwards S_local instead of the
    accumulated state, referee_report.major_comments[3] of the ZeCO review page)."""
    out = seg_states.copy()
    out[:, :, 1:] += seg_decay[:, :, 1:, :, None] * seg_states[:, :, :-1]
    return out


@pytest.mark.parametrize("mode", [NONE, HEAD, GATE])
def test_segmented_scan_equals_one_pass(mode):
    rng = np.random.default_rng(20 + mode)
    B, H, P, Ls, dk, dv = 1, 2, 5, 12, 6, 5
    L = P * Ls
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    dec = {NONE: None, HEAD: np.array([-0.02, -0.2], np.float32), GATE: _rand(rng, B, H, L, dk)}[mode]
    s_in = rng.standard_normal((B, H, dk, dv))
    o1, s1 = oracle.recurrence(q, k, v, mode, dec, s_in)
    o, out = _decomposed(q, k, v, mode, dec, s_in, P)
    assert _rel(o, o1) < 1e-12
    assert _rel(out[:, :, -1], s1[:, :, 0]) < 1e-12
    # The literal one-hop reading loses state from segments more than one hop back.
    o_bad, out_bad = _decomposed(q, k, v, mode, dec, s_in, P, scan=_one_hop_scan)
    assert _rel(o_bad, o1) > 1e-3 or _rel(out_bad[:, :, -1], s1[:, :, 0]) > 1e-3


def test_cumdecay_closed_forms():
    B, H, L, dk, P = 1, 2, 60, 3, 3
    lam = np.array([-0.05, -0.5], np.float32)
    cum, tot = oracle.cumdecay(B, H, L, dk, HEAD, lam, nseg=P)
    tau = (np.arange(L) % (L // P) + 1).astype(np.float64)
    for h in range(H):
        ref = np.exp(np.float64(lam[h]) * tau)
        assert _rel(cum[0, h, :, 0], ref) < 1e-13
        assert _rel(tot[0, h, :, 1], np.full(P, np.exp(np.float64(lam[h]) * (L // P)))) < 1e-13
    rng = np.random.default_rng(7)
    g = _rand(rng, B, H, L, dk)
    cum, tot = oracle.cumdecay(B, H, L, dk, GATE, g, nseg=P)
    la = _log_decay(GATE, g, B, H, L, dk).reshape(B, H, P, L // P, dk)
    ref = np.exp(np.cumsum(la, axis=3)).reshape(B, H, L, dk)
    assert _rel(cum, ref) < 1e-13
    assert _rel(tot, np.exp(la.sum(axis=3))) < 1e-13
    cum, tot = oracle.cumdecay(B, H, L, dk, NONE, None, nseg=P)
    assert np.all(cum == 1.0) and np.all(tot == 1.0)


def test_state_scan_exact_cases():
    rng = np.random.default_rng(8)
    B, H, P, dk, dv = 2, 1, 7, 3, 4
    x = rng.integers(-5, 6, size=(B, H, P, dk, dv)).astype(np.float64)
    # a = 1 with integer states: an exact cumulative sum over segments.
    assert np.array_equal(oracle.state_scan(x, np.ones((B, H, P, dk))), np.cumsum(x, axis=2))
    # decay 0: no state crosses a segment boundary.
    assert np.array_equal(oracle.state_scan(x, np.zeros((B, H, P, dk))), x)
    # P = 1 is the identity.
    assert np.array_equal(oracle.state_scan(x[:, :, :1], rng.random((B, H, 1, dk))), x[:, :, :1])
    # per-row decay acts on rows (key dims) of the state, not on columns.
    lam = np.zeros((B, H, P, dk))
    lam[:, :, :, 0] = 2.0
    out = oracle.state_scan(x, lam)
    ref_row0 = np.zeros_like(x[:, :, 0, 0])
    for p in range(P):
        ref_row0 = 2.0 * ref_row0 + x[:, :, p, 0]
        assert np.array_equal(out[:, :, p, 0], ref_row0)
        assert np.array_equal(out[:, :, p, 1:], x[:, :, p, 1:])


def test_state_correct_cases():
    rng = np.random.default_rng(9)
    B, H, L, dk, dv = 1, 2, 20, 4, 3
    q = _rand(rng, B, H, L, dk)
    o = rng.standard_normal((B, H, L, dv))
    S = rng.standard_normal((B, H, 1, dk, dv))
    ones = np.ones((B, H, L, dk))
    got = oracle.state_correct(q, ones, S, o)
    assert _rel(got, o + np.einsum("bhtd,bhdc->bhtc", q.astype(np.float64), S[:, :, 0])) < 1e-14
    assert np.array_equal(oracle.state_correct(q, ones, np.zeros_like(S), o), o)
    # seg_begin skips earlier segments bit-exactly
    got = oracle.state_correct(q, ones, S, o, nseg=2, seg_begin=1)
    assert np.array_equal(got[:, :, :10], o[:, :, :10])


def test_gate_reset_tokens_restart_the_recurrence():
    """A gate of -inf gives a = sigmoid(-inf)^(1/16) = 0 exactly: at such a token every key dim's state
    forgets everything before it.  So with g = -inf on all key dims of token t0, the outputs from t0
    on and S_out equal a fresh run over tokens t0.. from a zero state (the prefix changes nothing),
    and g = -1e3 (sigmoid underflows to 0 in fp64) behaves the same.  With g = -inf on one key dim
    only, that dim's row of S_out is k_L[d] v_L (every earlier term of the row is cut)."""
    rng = np.random.default_rng(21)
    B, H, L, dk, dv, t0 = 1, 2, 50, 4, 3, 19
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    g = _rand(rng, B, H, L, dk)
    s_in = rng.standard_normal((B, H, dk, dv))
    for reset in (-np.inf, -1e3):
        gr = g.copy()
        gr[:, :, t0, :] = reset
        o, s = oracle.recurrence(q, k, v, GATE, gr, s_in, gate_norm=16.0)
        o2, s2 = oracle.recurrence(q[:, :, t0:].copy(), k[:, :, t0:].copy(), v[:, :, t0:].copy(), GATE,
                                   gr[:, :, t0:].copy(), None, gate_norm=16.0)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
        assert np.array_equal(o[:, :, t0:], o2) and np.array_equal(s, s2)
    # one dim reset on every token: its row of the state is the last token's k v only
    gd = g.copy()
    gd[..., 2] = -np.inf
    _, s = oracle.recurrence(q, k, v, GATE, gd, s_in, gate_norm=16.0)
    K, V = k.astype(np.float64), v.astype(np.float64)
    assert np.allclose(s[:, :, 0, 2, :], K[:, :, -1, 2, None] * V[:, :, -1, :], rtol=0, atol=1e-15)
