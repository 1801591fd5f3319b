"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Inputs are drawn on the device; only the sampled (b, h) sequences are copied to the host and
run through the fp64 oracle, whole (every token of those sequences is compared).
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_scan_amd import binding as lb
from chunked_scan_amd.inputs import WORKLOADS, make_inputs
from chunked_scan_amd.pipeline import DeviceStep, ExactStep, RecvFirstStep, SegmentedForward

from gpu_util import ORC_MODE, TOL, host32, note, rel_err

pytestmark = pytest.mark.gpu


def _sample_oracle(inp, w, pairs, with_s_in=True):
    """fp64 oracle on the sampled (b, h) sequences; returns (o_ref [n,L,dv], s_ref [n,dk,dv])."""
    idx_b = [b for b, _ in pairs]
    idx_h = [h for _, h in pairs]
    sel = lambda t: t[idx_b, idx_h].unsqueeze(0)  # noqa: E731  [1, n, L, d]
    q, k, v = (host32(sel(inp[x])) for x in ("q", "k", "v"))
    dec = inp["decay"]
    if w.mode == "head":
        dec = host32(dec[idx_h])
    elif w.mode == "gate":
        dec = host32(sel(dec))
    s_in = None
    if with_s_in and inp["s_in"] is not None:
        s_in = host32(sel(inp["s_in"])).astype(np.float64)
    o, s = oracle.recurrence(q, k, v, ORC_MODE[w.mode], dec, s_in, gate_norm=w.gate_norm)
    return o[0], s[0, :, 0]


@pytest.mark.parametrize("wid,pairs", [(1, [(0, 0), (0, 7), (0, 15)]),
                                       (2, [(0, 0), (1, 8), (1, 15)]),
                                       (3, [(0, 0), (2, 7), (3, 15)])])
def test_workload_device_step(wid, pairs):
    w = WORKLOADS[wid]
    note(f"workload {wid} {w.name}: device step at full size, sampled (b,h) {pairs}")
    inp = make_inputs(w, "cuda")
    step = DeviceStep(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"], mode=w.mode, chunk=w.chunk,
                      gate_norm=w.gate_norm)
    o, s_out = step.run()
    torch.cuda.synchronize()
    o_ref, s_ref = _sample_oracle(inp, w, pairs)
    for n, (b, h) in enumerate(pairs):
        assert rel_err(o[b, h], o_ref[n]) <= TOL["bf16"], (b, h)
        assert rel_err(s_out[b, h], s_ref[n]) <= TOL["bf16"], (b, h)
    # the exact form (one la_chunk_fwd from S_recv: the benchmark's headline step), with the
    # library's default schedule and, where it exists, the chained single launch
    for schedule in ("auto", "chained") if w.mode != "gate" else ("auto",):
        note(f"workload {wid}: exact step, schedule {schedule}")
        o2, s2 = ExactStep(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"], mode=w.mode, chunk=w.chunk,
                           gate_norm=w.gate_norm, schedule=schedule).run()
        torch.cuda.synchronize()
        for n, (b, h) in enumerate(pairs):
            assert rel_err(o2[b, h], o_ref[n]) <= TOL["bf16"], (schedule, b, h)
            assert rel_err(s2[b, h], s_ref[n]) <= TOL["bf16"], (schedule, b, h)
    # the decomposed form with S_recv taken in by the first sub-segment
    note(f"workload {wid}: decomposed step, first sub-segment from S_recv")
    o3, s3 = RecvFirstStep(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"], mode=w.mode, chunk=w.chunk,
                           gate_norm=w.gate_norm).run()
    torch.cuda.synchronize()
    for n, (b, h) in enumerate(pairs):
        assert rel_err(o3[b, h], o_ref[n]) <= TOL["bf16"], ("recv_first", b, h)
        assert rel_err(s3[b, h], s_ref[n]) <= TOL["bf16"], ("recv_first", b, h)


def test_workload4_segmented_1M():
    w = WORKLOADS[4]
    heads = [0, 15]
    note(f"workload 4 {w.name}: {w.nseg}-segment pipeline over {w.L} tokens, sampled heads {heads}")
    inp = make_inputs(w, "cuda")
    seg = SegmentedForward(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"], mode=w.mode, nseg=w.nseg,
                           chunk=w.chunk)
    o, states = seg.run()
    torch.cuda.synchronize()
    note("workload 4: one-pass GPU run over the whole sequence")
    o1, s1 = lb.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"], mode=w.mode)
    torch.cuda.synchronize()
    note("workload 4: oracle on the sampled heads")
    o_ref, s_ref = _sample_oracle(inp, w, [(0, h) for h in heads])
    for n, h in enumerate(heads):
        assert rel_err(o[0, h], o_ref[n]) <= TOL["bf16"], h
        assert rel_err(states[0, h, -1], s_ref[n]) <= TOL["bf16"], h
        assert rel_err(o1[0, h], o_ref[n]) <= TOL["bf16"], h
        assert rel_err(s1[0, h, 0], s_ref[n]) <= TOL["bf16"], h
    # segmented vs one-pass GPU results over all heads
    assert rel_err(states[:, :, -1], s1[:, :, 0].double().cpu().numpy()) <= TOL["bf16"]
    for h in range(w.H):
        assert rel_err(o[0, h], o1[0, h].double().cpu().numpy()) <= TOL["bf16"], h


def test_workload0_bench_configuration():
    """The tiny fp32 workload through the device step, against the oracle (all of it)."""
    w = WORKLOADS[0]
    note(f"workload 0 {w.name}")
    inp = make_inputs(w, "cpu")
    d = {k: (None if t is None else t.cuda()) for k, t in inp.items()}
    o, s = DeviceStep(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode=w.mode, chunk=w.chunk).run()
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence(host32(inp["q"]), host32(inp["k"]), host32(inp["v"]), oracle.HEAD,
                                     host32(inp["decay"]), host32(inp["s_in"]).astype(np.float64))
    assert rel_err(o, o_ref) <= TOL["f32"]
    assert rel_err(s, s_ref[:, :, 0]) <= TOL["f32"]
