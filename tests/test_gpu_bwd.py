"""GPU parity of the backward pass (la_chunk_bwd) against the fp64 oracle's token-by-token
derivatives (oracle.recurrence_bwd), on the same seeded inputs.

The kernels form the decay derivative in three ways: the fp32 path from q * dq - k * dk and reverse
running sums over the segment; the matrix-core path for a head decay pair by pair of tokens (with
dS/dlambda carried beside S); the matrix-core path for the gate per chunk, from rowsum(S * D) at the
chunk's start plus an in-chunk running sum of k * dk - q * dq.  The oracle takes it from the
definition (da_t = rowsum(G_t * S_{t-1}) and the chain rule), so these tests also check those
identities.  Sizes span several chunks, a ragged last chunk, both slicings of the state (dk, dv up
to 128) and two segments.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_scan_amd import binding as lb
from chunked_scan_amd import pipeline
from chunked_scan_amd.inputs import WORKLOADS, make_grads, make_inputs

from gpu_util import ORC_MODE, TOL, host32, note, rel_err, to_dev

pytestmark = pytest.mark.gpu

W0 = WORKLOADS[0]
# fp32 path: the decay derivative is formed from q dq - k dk, whose terms largely cancel (d lambda_h
# sums them (t - t0 + 1)-weighted over whole segments in fp64, the gate derivative takes reverse
# running sums in fp32); the ~1e-7 relative rounding of dq and dk is magnified by that cancellation:
# measured up to 7.4e-6 of max|ref| for d lambda_h at L = 192..2048 (1e-6 for the gate), hence 5e-5.
# bf16 inputs: the general bf16 bound (the matrix-core d lambda_h, summed pair by pair with bf16
# operands, measures about 1e-3).
TOL_DECAY = {"f32": 5e-5, "bf16": 2e-2}


def _case(mode, dtype, dk, dv, L, chunk, nseg, seed, B=2, H=2, s_in=True, ds_out=True):
    decay = {"none": "none", "head": "head_uniform", "gate": "gate"}[mode]
    w = W0.scaled(B=B, H=H, L=L, dk=dk, dv=dv, decay=decay, chunk=chunk, dtype=dtype, seed=seed,
                  qkv_std=1.0 / np.sqrt(dk), s_in_std=0.1 if s_in else 0.0)
    inp = make_inputs(w, "cpu")
    gr = make_grads(w, nseg=nseg, ds_out_std=1.0 if ds_out else 0.0)
    return w, inp, gr


def _oracle(w, inp, gr, nseg):
    s_in = host32(inp["s_in"])
    ds_out = host32(gr["ds_out"])
    return oracle.recurrence_bwd(host32(inp["q"]), host32(inp["k"]), host32(inp["v"]), host32(gr["d_o"]),
                                 ORC_MODE[w.mode], host32(inp["decay"]),
                                 None if s_in is None else s_in.astype(np.float64),
                                 None if ds_out is None else ds_out.astype(np.float64), nseg=nseg,
                                 gate_norm=w.gate_norm)


def _gpu(w, inp, gr, nseg, want_decay=True):
    d = to_dev(inp)
    g = to_dev(gr)
    out = lb.la_chunk_bwd(d["q"], d["k"], d["v"], g["d_o"], d["decay"], d["s_in"], g["ds_out"], mode=w.mode,
                          nseg=nseg, chunk=w.chunk, gate_norm=w.gate_norm, want_decay=want_decay)
    torch.cuda.synchronize()
    return out


def _compare(got, ref, dtype, mode):
    names = ("dq", "dk", "dv", "d_decay", "ds_in")
    for name, g, r in zip(names, got, ref):
        if name == "d_decay":
            if mode == "none":
                assert g is None and r is None
                continue
            if g is None:  # not requested
                continue
            err = rel_err(g, r)
            assert err <= TOL_DECAY[dtype], (name, err)
        else:
            err = rel_err(g, r)
            assert err <= TOL[dtype], (name, err)


@pytest.mark.parametrize("want_decay", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_bwd_head_decay_both_walks(d, want_decay):
    """bf16 head decay: the matrix-core passes take their factorised walks (dq on the forward's
    kernel; dk/dv's own unless d lambda_h is wanted, whose pair sums keep the per-pair weights) for
    heads with lambda C log2(e) >= -100 and the per-pair weights for stronger decays, both in one
    call (lambda = -1.0 and -1.6 straddle the bounds, -inf is a = 0); every derivative against the
    oracle (ragged length, several sub-segments), d lambda_h too when requested.  The lambda = -inf
    head is left out of d lambda_h: its derivative there is not defined."""
    lams = np.array([-1e-4, -0.02, -0.5, -1.0, -1.6, -3.0, 0.0, -np.inf], np.float32)
    if want_decay:
        lams = lams[:-1]
    w, inp, gr = _case("head", "bf16", d, d, 64 * 9 + 21, 64, 1, seed=880 + d, B=1, H=len(lams))
    inp["decay"] = torch.from_numpy(lams)
    note(f"la_chunk_bwd head decay both walks d={d} want_decay={want_decay} lambdas={lams.tolist()}")
    dd, g = to_dev(inp), to_dev(gr)
    got = lb.la_chunk_bwd(dd["q"], dd["k"], dd["v"], g["d_o"], dd["decay"], dd["s_in"], g["ds_out"], mode="head",
                          want_decay=want_decay, subseg_chunks=2)
    torch.cuda.synchronize()
    ref = _oracle(w, inp, gr, 1)
    for name, x, r in zip(("dq", "dk", "dv", "ds_in"), (got[0], got[1], got[2], got[4]),
                          (ref[0], ref[1], ref[2], ref[4])):
        for h in range(len(lams)):
            assert rel_err(x[:, h:h + 1], r[:, h:h + 1]) <= TOL["bf16"], (name, float(lams[h]))
    if want_decay:
        for h in range(len(lams)):
            assert abs(float(got[3][h]) - ref[3][h]) <= TOL_DECAY["bf16"] * max(1e-12, np.max(np.abs(ref[3]))), \
                float(lams[h])


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("dk,dv,L,chunk,nseg", [(16, 16, 200, 16, 1), (32, 64, 301, 32, 1), (64, 32, 130, 64, 2),
                                                 (128, 128, 160, 64, 1), (16, 128, 154, 32, 2)])
def test_bwd_fp32(mode, dk, dv, L, chunk, nseg):
    note(f"la_chunk_bwd fp32 mode={mode} dk={dk} dv={dv} L={L} chunk={chunk} nseg={nseg}")
    w, inp, gr = _case(mode, "f32", dk, dv, L, chunk, nseg, seed=300 + dk + L)
    _compare(_gpu(w, inp, gr, nseg), _oracle(w, inp, gr, nseg), "f32", mode)


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("d,L,nseg", [(128, 192, 1), (64, 256, 2), (32, 130, 1)])
def test_bwd_bf16(mode, d, L, nseg):
    note(f"la_chunk_bwd bf16 mode={mode} d={d} L={L} nseg={nseg}")
    w, inp, gr = _case(mode, "bf16", d, d, L, 64, nseg, seed=400 + d + L)
    _compare(_gpu(w, inp, gr, nseg), _oracle(w, inp, gr, nseg), "bf16", mode)


@pytest.mark.parametrize("mode", ["head", "gate"])
def test_bwd_without_optional_terms(mode):
    """No s_in, no ds_out, and the decay / ds_in outputs not requested."""
    note(f"la_chunk_bwd no s_in / ds_out, mode={mode}")
    w, inp, gr = _case(mode, "f32", 32, 32, 96, 32, 1, seed=77, s_in=False, ds_out=False)
    ref = _oracle(w, inp, gr, 1)
    d = to_dev(inp)
    g = to_dev(gr)
    dq, dk, dv, dd, ds_in = lb.la_chunk_bwd(d["q"], d["k"], d["v"], g["d_o"], d["decay"], None, None, mode=w.mode,
                                            chunk=32, want_decay=False, want_ds_in=False)
    torch.cuda.synchronize()
    assert dd is None and ds_in is None
    for got, r in zip((dq, dk, dv), ref[:3]):
        assert rel_err(got, r) <= TOL["f32"]


def test_bwd_empty_and_zero_length():
    """L = 0: ds_in = ds_out, the head-decay derivative is zero; B = 0: zero derivative."""
    note("la_chunk_bwd empty shapes")
    w, inp, gr = _case("head", "f32", 16, 16, 0, 16, 2, seed=5)
    out = _gpu(w, inp, gr, 2)
    assert torch.equal(out[4].cpu(), gr["ds_out"])
    assert torch.count_nonzero(out[3]) == 0
    w, inp, gr = _case("head", "f32", 16, 16, 32, 16, 1, seed=6, B=0)
    out = _gpu(w, inp, gr, 1)
    assert out[3].shape == (2,) and torch.count_nonzero(out[3]) == 0


def test_bwd_chunk_invariance():
    """The chunk length changes the rounding order only."""
    note("la_chunk_bwd chunk 16 / 32 / 64 agree")
    w, inp, gr = _case("gate", "f32", 32, 32, 192, 64, 1, seed=88)
    ref = _oracle(w, inp, gr, 1)
    for c in (16, 32, 64):
        d = to_dev(inp)
        g = to_dev(gr)
        got = lb.la_chunk_bwd(d["q"], d["k"], d["v"], g["d_o"], d["decay"], d["s_in"], g["ds_out"], mode="gate",
                              chunk=c, gate_norm=w.gate_norm)
        torch.cuda.synchronize()
        _compare(got, ref, "f32", "gate")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("L,nseg,H", [(192, 1, 2), (1000, 1, 2), (2048, 2, 2), (640, 1, 3)])
def test_bwd_bf16_matrix_core_subsegments(mode, L, nseg, H, d):
    """bf16, d = 32 / 64 / 128, chunk 64, with no decay, a fixed head decay or a fixed gate (no decay
    derivative requested) runs on the matrix-core kernels, which split each segment into sub-segments
    (state passes, scans of the state and of its derivative, output passes): lengths that give one or
    several sub-segments and a ragged last chunk.  Gate mode there stages q 2^{B}, k 2^{-B} and
    k 2^{B_last - B} per chunk (B the in-chunk cumulative log2-decay per key dim)."""
    note(f"la_chunk_bwd bf16 d={d} matrix-core mode={mode} L={L} nseg={nseg} H={H}")
    w, inp, gr = _case(mode, "bf16", d, d, L, 64, nseg, seed=500 + L + H + d, B=1, H=H)
    got = _gpu(w, inp, gr, nseg, want_decay=False)
    assert got[3] is None
    _compare(got, _oracle(w, inp, gr, nseg), "bf16", mode)


@pytest.mark.parametrize("d,L,nseg,B", [(128, 192, 1, 1), (128, 1000, 1, 1), (128, 2048, 2, 2), (128, 4096, 1, 1),
                                        (64, 1000, 1, 1), (64, 2048, 2, 2), (32, 1000, 1, 1), (32, 640, 1, 2)])
def test_bwd_bf16_matrix_core_head_decay_derivative(d, L, nseg, B):
    """d lambda_h on the matrix-core path (bf16): summed pair by pair with dS/dlambda carried beside S,
    composed across sub-segments; one or several sub-segments, two segments, two batches."""
    note(f"la_chunk_bwd bf16 d={d} head decay derivative L={L} nseg={nseg} B={B}")
    w, inp, gr = _case("head", "bf16", d, d, L, 64, nseg, seed=600 + L + d, B=B, H=3)
    got = _gpu(w, inp, gr, nseg)
    ref = _oracle(w, inp, gr, nseg)
    print(f"  d_decay rel err {rel_err(got[3], ref[3]):.2e}")
    _compare(got, ref, "bf16", "head")


@pytest.mark.parametrize("d,L,nseg,B", [(128, 192, 1, 1), (128, 1000, 1, 1), (128, 2048, 2, 2), (128, 4096, 1, 1),
                                        (64, 1000, 1, 1), (64, 2048, 2, 2), (32, 1000, 1, 1), (32, 640, 1, 2)])
def test_bwd_bf16_matrix_core_gate_derivative(d, L, nseg, B):
    """dg on the matrix-core path (bf16): per chunk, rowsum(S (.) D) at the chunk's start plus the
    in-chunk running sum of k (.) dk - q (.) dq; one or several sub-segments, two segments, two
    batches, ragged last chunks."""
    note(f"la_chunk_bwd bf16 d={d} gate derivative L={L} nseg={nseg} B={B}")
    w, inp, gr = _case("gate", "bf16", d, d, L, 64, nseg, seed=700 + L + d, B=B, H=3)
    got = _gpu(w, inp, gr, nseg)
    ref = _oracle(w, inp, gr, nseg)
    print(f"  d_decay rel err {rel_err(got[3], ref[3]):.2e}")
    _compare(got, ref, "bf16", "gate")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_gate_strong_decay(dtype):
    """Gate mode on the fp32 path factorises e^{B_i - B_j} into q e^{B} and k e^{-B} per chunk unless a
    chunk's decay sum for one of the workgroup's key dims is below -80: here key dims 0..3 of every
    head decay by about -2.5 per token (g = -40), so their slice keeps the per-pair exponentials, and
    the other slices factorise."""
    note(f"la_chunk_bwd gate with strong decay on some key dims, {dtype}")
    w, inp, gr = _case("gate", dtype, 64, 32, 200, 64, 1, seed=91)
    inp["decay"][..., :4] = -40.0
    _compare(_gpu(w, inp, gr, 1), _oracle(w, inp, gr, 1), dtype, "gate")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_matrix_core_gate_strong_decay_within_range(d):
    """Key dims 0..7 here decay by about -0.875 per token (g = -14), -56 over a chunk (2^-80.8),
    the others as drawn: still inside the span one factorisation reference covers (2^-96), so every
    chunk stays in one piece; every derivative, dg included, against the oracle (wider decays:
    test_gpu_gate_range.py)."""
    note(f"la_chunk_bwd bf16 d={d} matrix-core gate, chunk decay sums near -56 on 8 key dims")
    w, inp, gr = _case("gate", "bf16", d, d, 300, 64, 1, seed=93 + d, B=1, H=2)
    inp["decay"][..., :8] = -14.0
    got = _gpu(w, inp, gr, 1)
    ref = _oracle(w, inp, gr, 1)
    print(f"  d_decay rel err {rel_err(got[3], ref[3]):.2e}")
    _compare(got, ref, "bf16", "gate")


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("subseg_chunks", [1, 3, 0])
def test_bwd_matrix_core_subsegment_length(mode, subseg_chunks):
    """The sub-segment length of the matrix-core backward changes the rounding order only: one chunk
    per sub-segment (G = 71 here, so every scan of the backward, the d lambda_h ones included, runs
    over more than 64 entries), three chunks, and the automatic choice, each against the oracle with
    the decay derivative."""
    note(f"la_chunk_bwd bf16 d=64 mode={mode} subseg_chunks={subseg_chunks}")
    w, inp, gr = _case(mode, "bf16", 64, 64, 64 * 70 + 5, 64, 1, seed=800 + subseg_chunks, B=1, H=2)
    d = to_dev(inp)
    g = to_dev(gr)
    got = lb.la_chunk_bwd(d["q"], d["k"], d["v"], g["d_o"], d["decay"], d["s_in"], g["ds_out"], mode=w.mode,
                          chunk=64, gate_norm=w.gate_norm, subseg_chunks=subseg_chunks)
    torch.cuda.synchronize()
    _compare(got, _oracle(w, inp, gr, 1), "bf16", mode)


def _sub_states(w, inp, nseg, sub_len):
    """The exact state entering every sub-segment of sub_len tokens of every segment (oracle, fp64,
    stored fp32): [B, H, nseg * nsub, dk, dv]."""
    Ls = w.L // nseg
    nsub = -(-Ls // sub_len)
    q, k, v = host32(inp["q"]), host32(inp["k"]), host32(inp["v"])
    dec = host32(inp["decay"])
    out = np.zeros((w.B, w.H, nseg * nsub, w.dk, w.dv), np.float32)
    for p in range(nseg):
        s_in = host32(inp["s_in"]).astype(np.float64) if (p == 0 and inp["s_in"] is not None) else None
        for j in range(1, nsub):
            sl = slice(p * Ls, p * Ls + j * sub_len)
            dj = None if dec is None else (dec[:, :, sl] if w.mode == "gate" else dec)
            _, so = oracle.recurrence(q[:, :, sl], k[:, :, sl], v[:, :, sl], ORC_MODE[w.mode], dj, s_in,
                                      gate_norm=w.gate_norm)
            out[:, :, p * nsub + j] = so[:, :, 0]
    return torch.from_numpy(out)


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("d,L,nseg,sub_len", [(128, 1000, 1, 256), (64, 2 * 700, 2, 192), (32, 1300, 1, 320)])
def test_bwd_with_forward_states(mode, d, L, nseg, sub_len):
    """la_chunk_bwd_states: the states entering the sub-segments are given (here the oracle's exact
    ones), so the matrix-core backward splits at them and runs no forward state pass; every
    derivative, the decay's included, against the oracle; ragged last sub-segments."""
    note(f"la_chunk_bwd_states bf16 d={d} mode={mode} L={L} nseg={nseg} sub_len={sub_len}")
    w, inp, gr = _case(mode, "bf16", d, d, L, 64, nseg, seed=1000 + L + d, B=2, H=2)
    s_sub = _sub_states(w, inp, nseg, sub_len).cuda()
    dd = to_dev(inp)
    g = to_dev(gr)
    got = lb.la_chunk_bwd(dd["q"], dd["k"], dd["v"], g["d_o"], dd["decay"], dd["s_in"], g["ds_out"], mode=w.mode,
                          nseg=nseg, chunk=64, gate_norm=w.gate_norm, s_sub=s_sub, sub_len=sub_len)
    torch.cuda.synchronize()
    _compare(got, _oracle(w, inp, gr, nseg), "bf16", mode)


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
def test_bwd_after_device_step(mode):
    """Training order on one device: the device step (local forward, scan with S_recv, correction),
    then the backward with the step's own scan buffer as the sub-segment states and S_recv as s_in,
    against the oracle's derivatives of the recurrence started from S_recv."""
    note(f"device step then la_chunk_bwd_states, bf16 d=128 mode={mode}")
    w, inp, gr = _case(mode, "bf16", 128, 128, 2048, 64, 1, seed=1100, B=1, H=3)
    dd = to_dev(inp)
    g = to_dev(gr)
    step = pipeline.DeviceStep(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode=w.mode, chunk=64,
                               gate_norm=w.gate_norm, subseg=4)
    step.run()
    timer = lb.KernelTimer()
    got = lb.la_chunk_bwd(dd["q"], dd["k"], dd["v"], g["d_o"], dd["decay"], dd["s_in"], g["ds_out"], mode=w.mode,
                          chunk=64, gate_norm=w.gate_norm, s_sub=step.states[:, :, 0:4], sub_len=512, timer=timer)
    torch.cuda.synchronize()
    names = [n for n, _ in timer.harvest()]
    assert "chunk_bwd_dq" in names and "chunk_bwd_dq_state_pass" not in names, names
    _compare(got, _oracle(w, inp, gr, 1), "bf16", mode)


@pytest.mark.parametrize("dtype,d,L,sub_len", [("f32", 32, 300, 128), ("bf16", 128, 500, 512), ("bf16", 64, 256, 1024)])
def test_bwd_with_forward_states_unused(dtype, d, L, sub_len):
    """la_chunk_bwd_states where the states are not needed: the fp32 path (no sub-segment split), and
    one sub-segment covering the whole segment; the results are la_chunk_bwd's, against the oracle."""
    note(f"la_chunk_bwd_states, states unused: {dtype} d={d} L={L} sub_len={sub_len}")
    w, inp, gr = _case("gate", dtype, d, d, L, 64, 1, seed=1200 + L, B=1, H=2)
    s_sub = _sub_states(w, inp, 1, sub_len).cuda()
    dd = to_dev(inp)
    g = to_dev(gr)
    got = lb.la_chunk_bwd(dd["q"], dd["k"], dd["v"], g["d_o"], dd["decay"], dd["s_in"], g["ds_out"], mode=w.mode,
                          chunk=64, gate_norm=w.gate_norm, s_sub=s_sub, sub_len=sub_len)
    torch.cuda.synchronize()
    _compare(got, _oracle(w, inp, gr, 1), dtype, "gate")


def test_bwd_pass_structure():
    """Which passes run (la_trace names), several sub-segments: with d lambda_h the d lambda state
    pass's scanned S serves the dq output pass (no dq state pass); held fixed, the dq passes build
    their own; with dg the dk/dv passes run before the dq passes and dg comes last."""
    note("la_chunk_bwd pass structure, bf16 d=64 L=2048")

    def names(mode, want):
        w, inp, gr = _case(mode, "bf16", 64, 64, 2048, 64, 1, seed=1300, B=1, H=2)
        dd, g = to_dev(inp), to_dev(gr)
        timer = lb.KernelTimer()
        lb.la_chunk_bwd(dd["q"], dd["k"], dd["v"], g["d_o"], dd["decay"], dd["s_in"], g["ds_out"], mode=w.mode,
                        chunk=64, gate_norm=w.gate_norm, want_decay=want, timer=timer)
        torch.cuda.synchronize()
        return [n for n, _ in timer.harvest()]

    n = names("head", True)
    assert "chunk_bwd_dlam_state_pass" in n and "chunk_bwd_dq_state_pass" not in n, n
    assert n.index("chunk_bwd_dlam_state_pass") < n.index("chunk_bwd_dq"), n
    n = names("head", False)
    assert "chunk_bwd_dq_state_pass" in n and "chunk_bwd_dlam_state_pass" not in n, n
    n = names("gate", True)
    assert n.index("chunk_bwd_dkdv") < n.index("chunk_bwd_dq") < n.index("chunk_bwd_dg"), n


def test_concurrent_streams_bit_identical():
    """Two different problems on two streams at once (forward with internal sub-segments, then the
    backward with the decay derivative, both drawing workspace from the stream-ordered pool) give
    bit for bit what each gives alone."""
    note("la_chunk_fwd + la_chunk_bwd on two streams concurrently, bf16 d=128 head decay")
    cases = [_case("head", "bf16", 128, 128, 3000, 64, 1, seed=1400 + i, B=1, H=2) for i in range(2)]
    devs = [(to_dev(inp), to_dev(gr), w) for w, inp, gr in cases]

    def run(d, g, w):
        o, s_out = lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode=w.mode, chunk=64)
        grads = lb.la_chunk_bwd(d["q"], d["k"], d["v"], g["d_o"], d["decay"], d["s_in"], g["ds_out"], mode=w.mode,
                                chunk=64)
        return (o, s_out) + tuple(grads)

    alone = []
    for d, g, w in devs:
        alone.append(run(d, g, w))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        together = []
        for (d, g, w), st in zip(devs, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                together.append(run(d, g, w))
        torch.cuda.synchronize()
        for a, b in zip(alone, together):
            for x, y in zip(a, b):
                assert torch.equal(x, y)
