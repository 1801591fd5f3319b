"""GPU parity of the chained forward: la_chunk_fwd's single launch in which the sub-segments of a
segment hand their states on through flags (la_shape.fwd_schedule = 2; bf16, dk = dv = 128,
64-token chunks, no or head decay), against the fp64 oracle and against the separate passes
(fwd_schedule = 1).

The chained kernel's workgroups may see each other's flags at different times from run to run;
its result must not depend on that (every element's scan runs in one fixed order), so repeated
runs are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_scan_amd import binding as lb
from chunked_scan_amd.inputs import WORKLOADS, make_inputs

from gpu_util import TOL, host32, note, oracle_run, rel_err, to_dev

pytestmark = pytest.mark.gpu

W1, W2 = WORKLOADS[1], WORKLOADS[2]
DECAY = {"none": "none", "head": "head_pow2"}


def _fwd(d, w, schedule="chained", nseg=1, subseg=0, s_in=True, fn=lb.la_chunk_fwd):
    return fn(d["q"], d["k"], d["v"], d["decay"], d["s_in"] if s_in else None, mode=w.mode, nseg=nseg,
              chunk=64, subseg_chunks=subseg, schedule=schedule)


@pytest.mark.parametrize("mode", ["none", "head"])
@pytest.mark.parametrize("B,H,L,nseg,subseg,s_in", [(2, 3, 64 * 9 + 17, 1, 0, True), (1, 2, 64 * 16, 1, 1, True),
                                                    (1, 2, 64 * 23 + 40, 1, 2, False), (2, 2, 3 * 640, 3, 2, True),
                                                    (1, 1, 64 * 5, 1, 4, True), (1, 3, 130, 1, 1, True)])
def test_chain_matches_oracle_and_passes(mode, B, H, L, nseg, subseg, s_in):
    w = W2.scaled(B=B, H=H, L=L, decay=DECAY[mode], s_in_std=0.05, seed=3000 + L + subseg)
    note(f"chained forward mode={mode} B={B} H={H} L={L} nseg={nseg} subseg_chunks={subseg} s_in={s_in}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w, nseg=nseg, with_s_in=s_in)
    d = to_dev(inp)
    oc, sc = _fwd(d, w, "chained", nseg, subseg, s_in)
    op, sp = _fwd(d, w, "passes", nseg, subseg, s_in)
    torch.cuda.synchronize()
    for o, s, name in ((oc, sc, "chained"), (op, sp, "passes")):
        assert rel_err(o, o_ref) <= TOL["bf16"], name
        assert rel_err(s, s_ref) <= TOL["bf16"], name
    # the two schedules differ in rounding order only
    assert rel_err(oc, op.double().cpu().numpy()) <= 2e-2
    assert rel_err(sc, sp.double().cpu().numpy()) <= 1e-4


@pytest.mark.parametrize("mode", ["none", "head"])
def test_chain_long_lookback(mode):
    """64 sub-segments of one chunk each: the last waits on the longest chain of hand-offs."""
    w = W2.scaled(B=1, H=2, L=64 * 64, decay=DECAY[mode], s_in_std=0.05, seed=3100)
    note(f"chained forward, 64 one-chunk sub-segments, mode={mode}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    d = to_dev(inp)
    runs = [_fwd(d, w, subseg=1) for _ in range(3)]
    torch.cuda.synchronize()
    assert rel_err(runs[0][0], o_ref) <= TOL["bf16"]
    assert rel_err(runs[0][1], s_ref) <= TOL["bf16"]
    for o, s in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(s, runs[0][1])


def test_chain_integer_inputs_bit_exact():
    """Integer inputs whose every intermediate is exact (no decay): the chained result equals the
    exact result rounded once, whatever the hand-off order."""
    g = torch.Generator().manual_seed(3200)
    B, H, L, d = 1, 3, 64 * 11 + 9, 128
    note("chained forward, integer inputs, bit-exact")
    q, k, v = (torch.randint(-1, 2, (B, H, L, d), generator=g).to(torch.bfloat16) for _ in range(3))
    s_in = torch.randint(-8, 9, (B, H, d, d), generator=g).float()
    o_ref, s_ref = oracle.recurrence(host32(q), host32(k), host32(v), oracle.NONE, None, s_in.double().numpy())
    for subseg in (1, 2, 3):
        o, s = lb.la_chunk_fwd(q.cuda(), k.cuda(), v.cuda(), None, s_in.cuda(), mode="none", subseg_chunks=subseg,
                               schedule="chained")
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), torch.from_numpy(o_ref).to(torch.bfloat16)), subseg
        assert torch.equal(s.cpu().double(), torch.from_numpy(s_ref)), subseg


@pytest.mark.parametrize("wid", [1, 2])
def test_chain_full_size_repeatable(wid):
    """The benchmark's shapes (B1 / B2, H16, L16384, d128): ten chained calls are bit-identical, and
    sampled heads match the oracle over all 16384 tokens."""
    w = WORKLOADS[wid]
    note(f"chained forward at full size, workload {wid} {w.name}, 10 repeats")
    d = make_inputs(w, "cuda")
    timer = lb.KernelTimer(8)
    o0, s0 = lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode=w.mode, schedule="chained",
                             timer=timer)
    torch.cuda.synchronize()
    names = [n for n, _ in timer.harvest()]
    assert names == ["chunk_fwd_chain_reset", "chunk_fwd_chain_output_pass"], names  # no fallback to the passes
    for rep in range(9):
        o, s = _fwd(d, w)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(s, s0), rep
    for b, h in ((0, 0), (w.B - 1, 13)):
        sub = {key: (None if t is None else (t[h:h + 1] if key == "decay" else t[b:b + 1, h:h + 1]))
               for key, t in d.items()}
        ws = w.scaled(B=1, H=1)
        o_ref, s_ref = oracle_run({key: (None if t is None else t.cpu()) for key, t in sub.items()}, ws)
        assert rel_err(o0[b:b + 1, h:h + 1], o_ref) <= TOL["bf16"], (b, h)
        assert rel_err(s0[b:b + 1, h:h + 1], s_ref) <= TOL["bf16"], (b, h)


def test_chain_noalloc_and_graph_replay():
    """la_chunk_fwd_noalloc runs the same chained kernel from its fixed array (bit-identical), and a
    captured chained call replays bit-identically with eager work between the replays (its flag
    reset is a kernel, not a memset)."""
    w = W2.scaled(B=1, H=16, L=4096, s_in_std=0.05, seed=3300)
    note("chained forward: noalloc entry point and graph replay")
    d = to_dev(make_inputs(w, "cpu"))
    o_ref, s_ref = _fwd(d, w)
    o_na, s_na = _fwd(d, w, fn=lb.la_chunk_fwd_noalloc)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref) and torch.equal(s_na, s_ref)
    o = torch.empty_like(o_ref)
    s = torch.empty_like(s_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], d["s_in"], o, s, mode=w.mode, schedule="chained")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], d["s_in"], o, s, mode=w.mode, schedule="chained")
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(4):
        o.zero_()
        scratch.add_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref), rep


def test_chain_give_up_is_reported():
    """Failure handling, forced from the host: with a spin limit of 0 every chained wave that waits
    gives up at once.  The kernel still ends normally; the sub-segments after the first compute on
    NaN states; la_chain_status reports the give-ups as LA_ERR_TIMEOUT and clears the counter.  With
    the default limit the same call gives up nowhere and matches the passes."""
    w = W2.scaled(B=1, H=2, L=64 * 8, s_in_std=0.05, seed=3400)
    note("chained forward: forced give-up (spin limit 0) and its status")
    d = to_dev(make_inputs(w, "cpu"))
    assert lb.la_chain_status() == 0
    prev = lb.la_set_chain_spin_limit(0)
    try:
        o, s = _fwd(d, w, subseg=2)  # four sub-segments of 128 tokens
        with pytest.raises(lb.LaError) as err:
            lb.la_chain_status()
        assert err.value.status == -9
    finally:
        assert lb.la_set_chain_spin_limit(prev) == 0
    assert lb.la_chain_status() == 0  # cleared by the call that reported
    of = o.float()
    assert torch.isfinite(of[:, :, :128]).all()  # the first sub-segment starts from s_in
    assert torch.isnan(of[:, :, 128:]).all() and torch.isnan(s).all()
    oc, sc = _fwd(d, w, subseg=2)
    op, sp = _fwd(d, w, "passes", subseg=2)
    assert lb.la_chain_status() == 0
    assert rel_err(oc, op.double().cpu().numpy()) <= 2e-2
    assert rel_err(sc, sp.double().cpu().numpy()) <= 1e-4
