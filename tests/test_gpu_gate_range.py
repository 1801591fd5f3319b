"""Gate mode with decays far outside one chunk's factorisation range, against the fp64 oracle.

A few key dims of the raw gate g are set to extreme values among dims drawn N(0, 1):
  * g = -25 on every token: log a = -softplus(25)/16 ~ -1.56 per token, about -100 over a 64-token
    chunk (2^-144), beyond the 2^-96 one factorisation reference may span;
  * g = -1e3 on a random tenth of the tokens: log a ~ -62.5, below the kernels' per-token floor
    (e^-33), so these tokens reset the dim's state up to e^-33;
  * g = -inf on a few tokens: a = 0 exactly (the oracle's sigmoid is 0), a true reset;
  * ("dense" pattern) g = -inf on every token of one dim: every chunk needs two-token windows.
The oracle evaluates a = sigmoid(g)^(1/16) directly in fp64 (0 for g = -inf and, by underflow, for
g = -1e3), so the floor's effect (every pair weight moved by at most e^-33) is far below the bf16
bound.  Every output must be finite and within the usual bounds: 2e-2 of max|ref| (bf16), 1e-5
(fp32 path).
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_scan_amd import binding as lb
from chunked_scan_amd import pipeline
from chunked_scan_amd.inputs import WORKLOADS, make_grads, make_inputs

from gpu_util import ORC_MODE, TOL, host32, note, oracle_run, rel_err, to_dev

pytestmark = pytest.mark.gpu

W3 = WORKLOADS[3]


def _extreme(g: torch.Tensor, pattern: str, seed: int) -> torch.Tensor:
    """Overwrite some key dims of the gate tensor g [B,H,L,dk] (CPU) with extreme values."""
    gen = torch.Generator().manual_seed(seed)
    dk = g.shape[-1]
    g = g.clone()
    g[..., 1] = -25.0
    mask = torch.rand(g.shape[:-1], generator=gen) < 0.1
    g[..., 5][mask] = -1e3
    idx = torch.randint(0, g.shape[2], (4,), generator=gen)
    g[:, :, idx, 9 % dk] = -float("inf")
    if pattern == "dense":
        g[..., dk - 1] = -float("inf")
    return g


def _case(d, L, pattern, seed, B=1, H=2, dtype="bf16", s_in=True):
    w = W3.scaled(B=B, H=H, L=L, dk=d, dv=d, qkv_std=d ** -0.5, dtype=dtype, s_in_std=0.05 if s_in else 0.0,
                  seed=seed)
    inp = make_inputs(w, "cpu")
    inp["decay"] = _extreme(inp["decay"], pattern, seed)
    return w, inp


def _finite(*ts):
    for t in ts:
        if t is not None:
            assert torch.isfinite(t.float()).all(), "non-finite output"


@pytest.mark.parametrize("pattern", ["sparse", "dense"])
@pytest.mark.parametrize("d,chunk", [(128, 64), (64, 64), (32, 64), (64, 128), (32, 128)])
@pytest.mark.parametrize("nseg,subseg", [(1, 3), (1, 0), (2, 1)])
def test_gate_extreme_forward(pattern, d, chunk, nseg, subseg):
    """la_chunk_fwd on the matrix-core kernels: one piece, sub-segment split (the d = 128 kernel's
    state and output passes, each with its windowed redo), one-chunk sub-segments, two segments."""
    L = 64 * 9 + 17 if nseg == 1 else 2 * (64 * 5 + 10)
    w, inp = _case(d, L, pattern, seed=1000 + d + chunk + nseg + subseg)
    note(f"la_chunk_fwd gate extreme {pattern} d={d} chunk={chunk} L={L} nseg={nseg} subseg={subseg}")
    dd = to_dev(inp)
    o, s = lb.la_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode="gate", nseg=nseg, chunk=chunk,
                           subseg_chunks=subseg)
    torch.cuda.synchronize()
    _finite(o, s)
    o_ref, s_ref = oracle_run(inp, w, nseg=nseg)
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("pattern", ["sparse", "dense"])
@pytest.mark.parametrize("d", [128, 64, 32])
def test_gate_extreme_decayed(pattern, d):
    """la_chunk_fwd_decayed: q times the cumulative decay, the segments' total decays and the tile
    flags, with several sub-segments and two segments."""
    nseg, L = 2, 2 * (64 * 7 + 20)
    w, inp = _case(d, L, pattern, seed=1100 + d, B=2)
    note(f"la_chunk_fwd_decayed gate extreme {pattern} d={d} L={L} nseg={nseg}")
    dd = to_dev(inp)
    o, s, qd, tot, live = lb.la_chunk_fwd_decayed(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode="gate",
                                                  nseg=nseg, subseg_chunks=2, want_tile_live=True)
    o0, s0 = lb.la_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode="gate", nseg=nseg,
                             subseg_chunks=2)
    torch.cuda.synchronize()
    _finite(o, s, qd, tot)
    assert torch.equal(o, o0) and torch.equal(s, s0)
    o_ref, s_ref = oracle_run(inp, w, nseg=nseg)
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]
    cref, tref = oracle.cumdecay(w.B, w.H, w.L, w.dk, oracle.GATE, host32(inp["decay"]), nseg=nseg,
                                 gate_norm=w.gate_norm)
    ref = host32(inp["q"]).astype(np.float64) * cref
    got = qd.cpu().double().numpy()
    # one bf16 rounding on top of the fp32 cumulative decay; where the exact decay is 0 (a = 0) or
    # below the floor the kernel's value is at most e^-33 per floored token
    assert np.all(np.abs(got - ref) <= (2.0 ** -8 + 2e-4) * np.abs(ref) + 1e-13)
    t = tot.cpu().double().numpy()
    assert np.all(np.abs(t - tref) <= 2e-4 * np.abs(tref) + 1e-13)
    # a tile flagged zero holds exactly zero rows of q_decayed
    Ls = L // nseg
    qz = torch.nn.functional.pad(qd.reshape(w.B, w.H, nseg, Ls, d), (0, 0, 0, live.shape[-1] * 64 - Ls))
    nonzero = qz.reshape(w.B, w.H, nseg, -1, 64 * d).ne(0).any(-1)
    assert not torch.any(nonzero & (live == 0))


@pytest.mark.parametrize("pattern", ["sparse", "dense"])
@pytest.mark.parametrize("d", [128, 64, 32])
def test_gate_extreme_device_step(pattern, d):
    """The device step (sub-segment forward with q times the cumulative decay, the scan with S_recv,
    the correction on live tiles) against one oracle pass from S_recv."""
    w, inp = _case(d, 64 * 12 + 6, pattern, seed=1200 + d, B=2)  # 3 sub-segments of 258 tokens
    note(f"device step gate extreme {pattern} d={d} L={w.L}")
    dd = to_dev(inp)
    o, s = pipeline.device_step(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode="gate", subseg=3)
    torch.cuda.synchronize()
    _finite(o, s)
    o_ref, s_ref = oracle_run(inp, w)
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref[:, :, 0]) <= TOL["bf16"]


def _bwd(w, inp, nseg, subseg=0):
    gr = make_grads(w, nseg=nseg)
    dd, gg = to_dev(inp), to_dev(gr)
    got = lb.la_chunk_bwd(dd["q"], dd["k"], dd["v"], gg["d_o"], dd["decay"], dd["s_in"], gg["ds_out"], mode="gate",
                          nseg=nseg, chunk=64, subseg_chunks=subseg)
    torch.cuda.synchronize()
    s_in = host32(inp["s_in"])
    ref = oracle.recurrence_bwd(host32(inp["q"]), host32(inp["k"]), host32(inp["v"]), host32(gr["d_o"]), oracle.GATE,
                                host32(inp["decay"]), None if s_in is None else s_in.astype(np.float64),
                                host32(gr["ds_out"]).astype(np.float64), nseg=nseg, gate_norm=w.gate_norm)
    return got, ref


@pytest.mark.parametrize("pattern", ["sparse", "dense"])
@pytest.mark.parametrize("d", [128, 64, 32])
@pytest.mark.parametrize("nseg,subseg", [(1, 3), (2, 0)])
def test_gate_extreme_backward(pattern, d, nseg, subseg):
    """la_chunk_bwd on the matrix cores with the gate derivative: dq, dk, dv, dg and ds_in (every
    pass and its windowed redo; sub-segments, two segments)."""
    L = 64 * 7 + 9 if nseg == 1 else 2 * (64 * 4 + 6)
    w, inp = _case(d, L, pattern, seed=1300 + d + nseg)
    note(f"la_chunk_bwd gate extreme {pattern} d={d} L={L} nseg={nseg} subseg={subseg}")
    got, ref = _bwd(w, inp, nseg, subseg)
    for name, g, r in zip(("dq", "dk", "dv", "dg", "ds_in"), got, ref):
        _finite(g)
        err = rel_err(g, r)
        assert err <= TOL["bf16"], (name, err)


@pytest.mark.parametrize("pattern", ["sparse", "dense"])
def test_gate_extreme_fp32_path(pattern):
    """The fp32 forward and backward (other head dims and fp32 inputs) with the same gates: a = 0
    used to give -inf - -inf = NaN in their pair exponentials."""
    w, inp = _case(32, 64 * 3 + 11, pattern, seed=1400, dtype="f32")
    note(f"fp32 path gate extreme {pattern}")
    dd = to_dev(inp)
    o, s = lb.la_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode="gate")
    torch.cuda.synchronize()
    _finite(o, s)
    o_ref, s_ref = oracle_run(inp, w)
    assert rel_err(o, o_ref) <= TOL["f32"]
    assert rel_err(s, s_ref) <= TOL["f32"]
    got, ref = _bwd(w, inp, 1)
    for name, g, r in zip(("dq", "dk", "dv", "dg", "ds_in"), got, ref):
        _finite(g)
        err = rel_err(g, r)
        assert err <= (5e-5 if name == "dg" else TOL["f32"]), (name, err)


def test_gate_wide_redo_runs_only_when_needed():
    """The d = 128 kernels hand a unit to the windowed kernels only when one of its chunks is too wide:
    with ordinary gates the redo launches find nothing to do (results bit-identical to a second call),
    and the extreme gates' result does not depend on which sub-segments met wide chunks."""
    w, inp = _case(128, 64 * 16, "sparse", seed=1500)
    note("gate d=128 redo only when needed")
    dd = to_dev(inp)
    plain = to_dev(make_inputs(w, "cpu"))
    o1, s1 = lb.la_chunk_fwd(plain["q"], plain["k"], plain["v"], plain["decay"], None, mode="gate", subseg_chunks=4)
    o2, s2 = lb.la_chunk_fwd(plain["q"], plain["k"], plain["v"], plain["decay"], None, mode="gate", subseg_chunks=4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    # extreme gates on the first and the last sub-segment only: the middle ones stay on the fast path
    g = plain["decay"].clone()
    g[:, :, :64 * 4] = dd["decay"][:, :, :64 * 4]
    g[:, :, -64 * 4:] = dd["decay"][:, :, -64 * 4:]
    inp2 = dict(inp)
    inp2["decay"] = g.cpu()
    o, s = lb.la_chunk_fwd(plain["q"], plain["k"], plain["v"], g, None, mode="gate", subseg_chunks=4)
    torch.cuda.synchronize()
    _finite(o, s)
    w2 = w.scaled(s_in_std=0.0)
    inp2["s_in"] = None
    o_ref, s_ref = oracle_run(inp2, w2)
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]
