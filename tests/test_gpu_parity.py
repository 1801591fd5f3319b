"""GPU parity: every C-ABI call against the fp64 CPU oracle on the same seeded inputs.

Sizes here are ones the oracle finishes in seconds while still spanning several chunks,
several internal sub-segments and a ragged tail.  Full-size workloads are covered in
test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_scan_amd import binding as lb
from chunked_scan_amd import pipeline
from chunked_scan_amd.inputs import WORKLOADS, make_inputs

from gpu_util import ORC_MODE, TOL, host32, note, oracle_run, rel_err, to_dev

pytestmark = pytest.mark.gpu

W0, W2, W3 = WORKLOADS[0], WORKLOADS[2], WORKLOADS[3]


def _fwd(inp, w, nseg=1, chunk=None, subseg=0, s_in=True):
    return lb.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"] if s_in else None,
                           mode=w.mode, nseg=nseg, chunk=chunk or w.chunk, gate_norm=w.gate_norm,
                           subseg_chunks=subseg)


def test_workload0_tiny_fp32():
    note("workload 0 (tiny fp32, head decay, s_in), la_chunk_fwd direct")
    w = W0
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    d = to_dev(inp)
    o, s = _fwd(d, w)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["f32"]
    assert rel_err(s, s_ref) <= TOL["f32"]
    note("workload 0 device step (local + combine + correct)")
    o2, s2 = pipeline.device_step(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode=w.mode, chunk=w.chunk)
    torch.cuda.synchronize()
    assert rel_err(o2, o_ref) <= TOL["f32"]
    assert rel_err(s2, s_ref[:, :, 0]) <= TOL["f32"]


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("dk,dv,L,chunk", [(16, 16, 200, 16), (32, 64, 301, 32), (64, 32, 130, 64),
                                            (128, 128, 160, 64), (16, 128, 77, 32)])
def test_generic_fp32(mode, dk, dv, L, chunk):
    decay = {"none": "none", "head": "head_uniform", "gate": "gate"}[mode]
    w = W0.scaled(B=2, H=2, L=L, dk=dk, dv=dv, decay=decay, chunk=chunk, seed=100 + dk + L)
    note(f"generic fp32 mode={mode} dk={dk} dv={dv} L={L} chunk={chunk}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    o, s = _fwd(to_dev(inp), w)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["f32"]
    assert rel_err(s, s_ref) <= TOL["f32"]


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("L,subseg", [(64 * 9 + 17, 0), (64 * 12, 3), (64 * 7, 1), (33, 0), (64 * 20 + 5, 8)])
def test_bf16_d128(mode, L, subseg):
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    w = W2.scaled(B=2, H=3, L=L, decay=decay, s_in_std=0.05, seed=200 + L + subseg)
    note(f"bf16 d128 chunk64 mode={mode} L={L} subseg_chunks={subseg}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    o, s = _fwd(to_dev(inp), w, subseg=subseg)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("L,subseg", [(64 * 9 + 17, 0), (64 * 12, 3), (33, 0), (64 * 20 + 5, 8)])
def test_bf16_small_heads(mode, d, L, subseg):
    """bf16 MFMA path for dk = dv = 32 and 64 (chunk 64): ragged last chunks, the intra-GPU split
    (state pass, sub-segment scan, output pass) and a sequence shorter than one chunk."""
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    w = W2.scaled(B=2, H=3, L=L, dk=d, dv=d, decay=decay, s_in_std=0.05, seed=500 + d + L + subseg)
    note(f"bf16 d{d} chunk64 mode={mode} L={L} subseg_chunks={subseg}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    o, s = _fwd(to_dev(inp), w, subseg=subseg)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("d", [32, 64])
def test_device_step_small_heads(mode, d):
    """The device step (G sub-segments, one scan, one correction) at dk = dv = 32 and 64."""
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    w = W2.scaled(B=2, H=3, L=768, dk=d, dv=d, decay=decay, s_in_std=0.05, seed=600 + d)
    note(f"device step bf16 d{d} mode={mode}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    dv = to_dev(inp)
    o, s = pipeline.device_step(dv["q"], dv["k"], dv["v"], dv["decay"], dv["s_in"], mode=w.mode, subseg=3)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref[:, :, 0]) <= TOL["bf16"]


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
def test_bf16_generic_other_dims(mode):
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    w = W2.scaled(B=1, H=2, L=300, dk=64, dv=32, decay=decay, chunk=32, s_in_std=0.05, seed=7)
    note(f"bf16 generic dk=64 dv=32 chunk=32 mode={mode}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    o, s = _fwd(to_dev(inp), w)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
def test_segmented_nseg(mode):
    """la_chunk_fwd with nseg > 1 treats segments as independent sequences."""
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    w = W2.scaled(B=1, H=2, L=6 * 200, decay=decay, s_in_std=0.05, seed=31)
    note(f"la_chunk_fwd nseg=6 mode={mode}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w, nseg=6)
    o, s = _fwd(to_dev(inp), w, nseg=6)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segmented_pipeline_equals_one_pass(mode, dtype):
    """The P-segment pipeline (local pass, state scan, correction) reproduces the one-pass
    recurrence over the whole sequence: outputs and the final state."""
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    dk = 128 if dtype == "bf16" else 32
    w = W2.scaled(B=1, H=2, L=8 * 192, dk=dk, dv=dk, dtype=dtype, decay=decay, s_in_std=0.05, seed=41)
    note(f"segmented pipeline P=8 mode={mode} dtype={dtype}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w, nseg=1)
    d = to_dev(inp)
    o, states = pipeline.segmented_forward(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode=w.mode, nseg=8)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert rel_err(o, o_ref) <= tol
    assert rel_err(states[:, :, -1], s_ref[:, :, 0]) <= tol


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("L,subseg", [(700, 0), (768, 1), (768, 3), (64 * 12, 12)])
def test_device_step_combine(mode, L, subseg):
    """G sub-segments from zero + one scan over [S_recv, S_loc...] + one correction pass == one
    pass from S_recv (G = 1: local pass, two-entry scan, correction; G = 12: one-chunk
    sub-segments; L = 700 chooses G = 2 with ragged chunks)."""
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    w = W2.scaled(B=2, H=2, L=L, decay=decay, s_in_std=0.05, seed=51 + L + subseg)
    note(f"device step combine mode={mode} L={L} subseg={subseg}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    d = to_dev(inp)
    o, s = pipeline.device_step(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode=w.mode, subseg=subseg)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref[:, :, 0]) <= TOL["bf16"]


# P spans every launch shape: the vector scan in one, four and eight parts (P <= 8, <= 20, <= 40,
# each edge and a partial block of columns: dk x dv = 480 or 1152), the four-part scalar scan
# (<= 64), the batched chain (longer)
@pytest.mark.parametrize("P,dk,dv", [(1, 64, 32), (4, 64, 32), (5, 32, 36), (8, 64, 32), (9, 20, 24), (13, 64, 32),
                                     (16, 64, 32), (17, 20, 24), (20, 64, 32), (21, 20, 24), (33, 128, 128),
                                     (40, 64, 32), (41, 64, 32), (64, 20, 24), (100, 64, 32)])
def test_state_scan_matches_oracle(P, dk, dv):
    note(f"la_state_scan random P={P} dk={dk} dv={dv}")
    g = torch.Generator().manual_seed(5)
    B, H = 2, 3
    x = torch.randn((B, H, P, dk, dv), generator=g)
    lam = torch.rand((B, H, P, dk), generator=g)
    ref = oracle.state_scan(x.double().numpy(), lam.double().numpy())
    out = lb.la_state_scan(x.cuda(), lam.cuda())
    torch.cuda.synchronize()
    assert rel_err(out, ref) <= 1e-6
    xi = x.cuda().clone()
    lb.la_state_scan(xi, lam.cuda(), xi)  # in place
    torch.cuda.synchronize()
    assert torch.equal(xi, out)
    # integer states with unit decay: an exact running sum
    xint = torch.randint(-8, 9, (B, H, P, dk, dv), generator=g).float()
    out = lb.la_state_scan(xint.cuda(), torch.ones((B, H, P, dk)).cuda())
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.cumsum(xint, dim=2))
    # no decay (NULL seg_decay) is the same running sum
    out = lb.la_state_scan(xint.cuda(), None)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.cumsum(xint, dim=2))


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64), ("bf16", 32), ("bf16", 64)])
def test_state_correct_matches_oracle(mode, dtype, dk):
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    P = 3
    w = W2.scaled(B=2, H=2, L=P * 150, dk=dk, dv=dk, dtype=dtype, decay=decay, s_in_std=0.05, seed=61)
    note(f"la_state_correct mode={mode} dtype={dtype} dk={dk}")
    inp = make_inputs(w, "cpu")
    g = torch.Generator().manual_seed(62)
    s_recv = torch.randn((w.B, w.H, P - 1, dk, dk), generator=g) * 0.05
    o0 = (torch.randn((w.B, w.H, w.L, dk), generator=g) * 0.1).to(inp["q"].dtype)
    cum_ref, _ = oracle.cumdecay(w.B, w.H, w.L, dk, ORC_MODE[w.mode], host32(inp["decay"]), nseg=P,
                                 gate_norm=w.gate_norm)
    ref = oracle.state_correct(host32(inp["q"]), cum_ref, s_recv.double().numpy(), host32(o0), nseg=P, seg_begin=1)
    d = to_dev(inp)
    cum = None
    if w.mode == "gate":
        cum, _ = lb.la_cumdecay(d["decay"], w.B, w.H, w.L, dk, mode="gate", nseg=P, want_total=False)
    elif w.mode == "head":
        cum = d["decay"]
    o = o0.cuda()
    lb.la_state_correct(d["q"], cum, s_recv.cuda(), o, mode=w.mode, nseg=P, seg_begin=1)
    torch.cuda.synchronize()
    assert rel_err(o, ref) <= TOL[dtype]
    # segment 0 is untouched bit-for-bit
    assert torch.equal(o[:, :, :150].cpu(), o0[:, :, :150])
    # a zero incoming state leaves the outputs bit-identical (the reviewers' S_recv = 0 ablation)
    o2 = o0.cuda()
    lb.la_state_correct(d["q"], cum, torch.zeros_like(s_recv).cuda(), o2, mode=w.mode, nseg=P, seg_begin=1)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu(), o0)


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
def test_state_correct_many_tiles_per_workgroup(mode):
    """bf16 d=128 correction with about five 64-token tiles per workgroup: ragged segments (2565
    tokens), incoming states that change inside a workgroup's range, and (head mode) decays that
    underflow to exactly zero part-way through a segment, whose tokens must stay bit-identical."""
    H, P, Ls, d = 4, 9, 2565, 128
    L = P * Ls
    note(f"la_state_correct many tiles mode={mode} H={H} P={P} Ls={Ls}")
    g = torch.Generator().manual_seed(63)
    q = torch.randn((1, H, L, d), generator=g).bfloat16()
    o0 = (torch.randn((1, H, L, d), generator=g) * 0.1).bfloat16()
    s_recv = torch.randn((1, H, P - 1, d, d), generator=g) * 0.05
    if mode == "head":
        decay = torch.tensor([0.0, -1e-3, -0.05, -0.5])  # the last two reach exactly zero in fp32
    elif mode == "gate":
        decay = torch.randn((1, H, L, d), generator=g) + 3.0
    else:
        decay = None
    cum_ref, _ = oracle.cumdecay(1, H, L, d, ORC_MODE[mode], None if decay is None else decay.numpy(), nseg=P)
    ref = oracle.state_correct(host32(q), cum_ref, s_recv.double().numpy(), host32(o0), nseg=P, seg_begin=1)
    cum = None
    if mode == "gate":
        cum, _ = lb.la_cumdecay(decay.cuda(), 1, H, L, d, mode="gate", nseg=P, want_total=False)
    elif mode == "head":
        cum = decay.cuda()
    o = o0.cuda()
    lb.la_state_correct(q.cuda(), cum, s_recv.cuda(), o, mode=mode, nseg=P, seg_begin=1)
    torch.cuda.synchronize()
    o = o.cpu()
    assert rel_err(o, ref) <= TOL["bf16"]
    assert torch.equal(o[:, :, :Ls], o0[:, :, :Ls])
    if mode == "head":
        # tokens whose factor exp(lambda * tau) is exactly zero in fp32 keep their bits
        tau = torch.arange(1, Ls + 1, dtype=torch.float32)
        for h in (2, 3):
            dead = torch.exp(decay[h] * tau) == 0
            assert dead.any()
            for p in range(1, P):
                seg = o[0, h, p * Ls:(p + 1) * Ls]
                assert torch.equal(seg[dead], o0[0, h, p * Ls:(p + 1) * Ls][dead]), (h, p)


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
def test_cumdecay_matches_oracle(mode):
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    P = 4
    w = W2.scaled(B=2, H=3, L=P * 700, dk=64, dv=64, decay=decay, seed=71)
    note(f"la_cumdecay mode={mode}")
    inp = make_inputs(w, "cpu")
    cref, tref = oracle.cumdecay(w.B, w.H, w.L, w.dk, ORC_MODE[w.mode], host32(inp["decay"]), nseg=P,
                                 gate_norm=w.gate_norm)
    cum, tot = lb.la_cumdecay(to_dev(inp)["decay"], w.B, w.H, w.L, w.dk, mode=w.mode, nseg=P, device="cuda")
    torch.cuda.synchronize()
    # per element relative error (values span many decades)
    c = cum.cpu().double().numpy()
    assert np.max(np.abs(c - cref) / np.maximum(np.abs(cref), 1e-30)) < 2e-4
    t = tot.cpu().double().numpy()
    assert np.max(np.abs(t - tref) / np.maximum(np.abs(tref), 1e-30)) < 2e-4


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("path,L,nseg,subseg", [("bf16_d128", 64 * 9 + 17, 1, 3), ("bf16_d128", 6 * 200, 6, 0),
                                                ("bf16_d128", 64 * 20, 2, 2), ("f32_d32", 3 * 150, 3, 0),
                                                ("bf16_d64", 64 * 9 + 17, 1, 3)])
def test_chunk_fwd_decayed(mode, path, L, nseg, subseg):
    """la_chunk_fwd_decayed: o and s_out exactly as la_chunk_fwd; q_decayed = q * cumdecay and total
    = each segment's decay against the oracle.  In gate mode with bf16 d=128 the forward's loaders
    emit them (several sub-segments, a ragged last chunk); elsewhere the separate pass does."""
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    bf = path.startswith("bf16")
    dk = int(path.split("_d")[1])
    w = W2.scaled(B=2, H=3, L=L, dk=dk, dv=dk, dtype="bf16" if bf else "f32", decay=decay, s_in_std=0.05,
                  seed=300 + L + nseg)
    note(f"la_chunk_fwd_decayed {path} mode={mode} L={L} nseg={nseg} subseg_chunks={subseg}")
    inp = make_inputs(w, "cpu")
    d = to_dev(inp)
    kw = dict(mode=w.mode, nseg=nseg, gate_norm=w.gate_norm, subseg_chunks=subseg)
    o0, s0 = lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], d["s_in"], **kw)
    o, s, qd, tot, live = lb.la_chunk_fwd_decayed(d["q"], d["k"], d["v"], d["decay"], d["s_in"], want_tile_live=True,
                                                  **kw)
    # each optional output alone
    _, _, qd_only, none_tot, _ = lb.la_chunk_fwd_decayed(d["q"], d["k"], d["v"], d["decay"], d["s_in"],
                                                         want_total=False, **kw)
    _, _, none_qd, tot_only, _ = lb.la_chunk_fwd_decayed(d["q"], d["k"], d["v"], d["decay"], d["s_in"],
                                                         want_q_decayed=False, **kw)
    _, _, _, _, live_only = lb.la_chunk_fwd_decayed(d["q"], d["k"], d["v"], d["decay"], d["s_in"],
                                                    want_q_decayed=False, want_total=False, want_tile_live=True, **kw)
    torch.cuda.synchronize()
    assert none_tot is None and none_qd is None
    assert torch.equal(o, o0) and torch.equal(s, s0)
    assert torch.equal(qd_only, qd) and torch.equal(tot_only, tot) and torch.equal(live_only, live)
    # with tile flags, the rows of a tile flagged zero are left as they were (a sentinel here), the
    # others are written exactly as without flags
    sentinel = torch.full_like(d["q"], float("nan"))
    _, _, qd_s, _, live_s = lb.la_chunk_fwd_decayed(d["q"], d["k"], d["v"], d["decay"], d["s_in"], q_decayed=sentinel,
                                                    want_tile_live=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(live_s, live)
    Ls = L // nseg
    pad = live.shape[-1] * 64 - Ls
    tiles = lambda x: torch.nn.functional.pad(x.reshape(w.B, w.H, nseg, Ls, dk).float(), (0, 0, 0, pad)).reshape(  # noqa: E731
        w.B, w.H, nseg, -1, 64 * dk)
    ts, tq = tiles(qd_s), tiles(qd_only)
    livem = (live != 0)[..., None].expand_as(ts)
    assert torch.equal(ts[livem], tq[livem])
    assert torch.all(torch.isnan(ts[~livem]) | (ts[~livem] == 0))
    # a tile flagged zero holds exactly zero rows of q_decayed
    qz = torch.nn.functional.pad(qd.reshape(w.B, w.H, nseg, Ls, dk), (0, 0, 0, live.shape[-1] * 64 - Ls))
    nonzero = qz.reshape(w.B, w.H, nseg, -1, 64 * dk).ne(0).any(-1)
    assert not torch.any(nonzero & (live == 0))
    cref, tref = oracle.cumdecay(w.B, w.H, w.L, w.dk, ORC_MODE[w.mode], host32(inp["decay"]), nseg=nseg,
                                 gate_norm=w.gate_norm)
    ref = host32(inp["q"]).astype(np.float64) * cref
    got = qd.cpu().double().numpy()
    if mode == "none":
        assert torch.equal(qd, d["q"])
    # one rounding to the storage dtype on top of the fp32 cumulative decay's own error; values
    # that fall below the fp32 normal range may flush to zero
    rnd = 2.0 ** -8 if bf else 2.0 ** -23
    assert np.all(np.abs(got - ref) <= (rnd + 2e-4) * np.abs(ref) + 1e-35)
    t = tot.cpu().double().numpy()
    assert np.max(np.abs(t - tref) / np.maximum(np.abs(tref), 1e-30)) < 2e-4


@pytest.mark.parametrize("H", [5, 70])
def test_state_correct_head_live_ranges(H):
    """Head-decay correction lists only tiles with a nonzero cumulative decay and balances the
    workgroups over them: heads with no live tile at all (a = 0, lambda = -inf), heads that never
    underflow (lambda = 0) and everything between, with more heads than a wave has lanes (70) and
    fewer (5).  Tokens whose decay is exactly zero keep O bit-identical."""
    B, P, Ls, d = 2, 3, 640 + 17, 128
    L = P * Ls
    note(f"la_state_correct head live ranges H={H}")
    g = torch.Generator().manual_seed(64 + H)
    q = torch.randn((B, H, L, d), generator=g).bfloat16()
    o0 = (torch.randn((B, H, L, d), generator=g) * 0.1).bfloat16()
    s_recv = torch.randn((B, H, P - 1, d, d), generator=g) * 0.05
    decay = -torch.rand(H, generator=g) * 0.6
    decay[0] = 0.0
    decay[1] = float("-inf")
    decay[H // 2] = float("-inf")
    decay[H - 1] = -2.0
    cum_ref, _ = oracle.cumdecay(B, H, L, d, ORC_MODE["head"], decay.numpy(), nseg=P)
    ref = oracle.state_correct(host32(q), cum_ref, s_recv.double().numpy(), host32(o0), nseg=P, seg_begin=1)
    o = o0.cuda()
    lb.la_state_correct(q.cuda(), decay.cuda(), s_recv.cuda(), o, mode="head", nseg=P, seg_begin=1)
    torch.cuda.synchronize()
    o = o.cpu()
    assert rel_err(o, ref) <= TOL["bf16"]
    dead = torch.from_numpy(cum_ref.reshape(B, H, L, d)[..., 0] == 0)
    assert torch.equal(o[dead], o0[dead])
    assert torch.equal(o[:, :, :Ls], o0[:, :, :Ls])


@pytest.mark.parametrize("pattern", ["none_live", "one_live", "last_segment", "sparse", "segment_starts"])
def test_state_correct_live_any_pattern(pattern):
    """la_state_correct_live skips the tiles flagged dead inside each workgroup's range of tiles;
    any pattern of live tiles -- none, a single one, all in the last segment, scattered, or
    clustered at each segment's start as a decay leaves them -- gives O bit-identical to
    la_state_correct over q whose rows are zero on the dead tiles."""
    B, H, nseg, seg_begin, Ls, d = 2, 8, 3, 1, 4096 + 40, 128
    L, tps = nseg * Ls, (Ls + 63) // 64
    note(f"la_state_correct_live pattern={pattern} B={B} H={H} nseg={nseg} Ls={Ls}")
    rng = np.random.default_rng(77)
    live = np.zeros((B, H, nseg, tps), np.int32)
    if pattern == "one_live":
        live[1, 5, 2, 17] = 1
    elif pattern == "last_segment":
        live[:, :, nseg - 1, :] = 1
    elif pattern == "sparse":
        live[:, :, seg_begin:, :] = rng.random((B, H, nseg - seg_begin, tps)) < 0.07
    elif pattern == "segment_starts":
        for b in range(B):
            for h in range(H):
                live[b, h, :, :rng.integers(0, tps + 1)] = 1
    g = torch.Generator().manual_seed(78)
    q = (torch.randn((B, H, L, d), generator=g) * 0.1).to(torch.bfloat16)
    rows = np.repeat(live, 64, axis=-1)[..., :Ls].reshape(B, H, L)
    q[torch.from_numpy(rows == 0)] = 0
    o = (torch.randn((B, H, L, d), generator=g) * 0.1).to(torch.bfloat16).cuda()
    s_recv = (torch.randn((B, H, nseg - seg_begin, d, d), generator=g) * 0.05).cuda()
    qd, flags = q.cuda(), torch.from_numpy(live).cuda()
    o1, o2 = o.clone(), o.clone()
    lb.la_state_correct(qd, None, s_recv, o1, mode="none", nseg=nseg, seg_begin=seg_begin)
    lb.la_state_correct(qd, None, s_recv, o2, mode="none", nseg=nseg, seg_begin=seg_begin, tile_live=flags)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    if pattern != "none_live" and live[:, :, seg_begin:].any():
        assert not torch.equal(o2, o)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("nseg,seg_begin", [(1, 0), (2, 1)])
def test_state_correct_live_skips_dead_tiles(nseg, seg_begin, d):
    """Gate decay over 4096-token segments: the cumulative decay underflows after ~1.7k tokens, so
    la_chunk_fwd_decayed flags later tiles zero (d = 128: the forward's loaders, from several
    internal sub-segments; d = 64: the separate three-pass computation), and
    la_state_correct_live, which skips them, gives O bit-identical to la_state_correct."""
    w = W3.scaled(B=1, H=2, L=4096 * nseg, dk=d, dv=d, s_in_std=0.05, seed=401 + nseg)
    note(f"la_state_correct_live gate d={d} nseg={nseg} seg_begin={seg_begin}")
    inp = make_inputs(w, "cpu")
    d = to_dev(inp)
    o, _, qd, _, live = lb.la_chunk_fwd_decayed(d["q"], d["k"], d["v"], d["decay"], None, mode="gate", nseg=nseg,
                                                gate_norm=w.gate_norm, subseg_chunks=4, want_tile_live=True)
    g = torch.Generator().manual_seed(9)
    s_recv = (torch.randn((w.B, w.H, nseg - seg_begin, w.dk, w.dv), generator=g) * 0.05).cuda()
    o1, o2 = o.clone(), o.clone()
    lb.la_state_correct(qd, None, s_recv, o1, mode="none", nseg=nseg, seg_begin=seg_begin)
    lb.la_state_correct(qd, None, s_recv, o2, mode="none", nseg=nseg, seg_begin=seg_begin, tile_live=live)
    torch.cuda.synchronize()
    dead = int((live[:, :, seg_begin:] == 0).sum())
    assert dead > 0.3 * live[:, :, seg_begin:].numel(), dead
    assert torch.equal(o1, o2)
    # and against the oracle: the correction of q_decayed rows
    ref = oracle.state_correct(host32(qd).astype(np.float64), np.ones((w.B, w.H, w.L, w.dk)),
                               s_recv.cpu().double().numpy(), host32(o).astype(np.float64), nseg=nseg,
                               seg_begin=seg_begin)
    assert rel_err(o2, ref) <= TOL["bf16"]


@pytest.mark.parametrize("path", ["f32_d16", "bf16_d128"])
def test_integer_inputs_bit_exact(path):
    """a = 1, q, k, v in {-1, 0, 1}, integer s_in with |s_in| <= 8.  Every intermediate is an integer
    below 2^24 (and below 256 where the bf16 path rounds operands), so the GPU must reproduce the
    exact result, rounded once to the output dtype, whatever its summation order."""
    g = torch.Generator().manual_seed(81)
    if path == "f32_d16":
        B, H, L, d, dt = 1, 2, 1000, 16, torch.float32
    else:
        B, H, L, d, dt = 1, 2, 192, 128, torch.bfloat16
    note(f"integer bit-exact {path}")
    q, k, v = (torch.randint(-1, 2, (B, H, L, d), generator=g).to(dt) for _ in range(3))
    s_in = torch.randint(-8, 9, (B, H, d, d), generator=g).float()
    o_ref, s_ref = oracle.recurrence(host32(q), host32(k), host32(v), oracle.NONE, None, s_in.double().numpy())
    for subseg in (0, 1):
        o, s = lb.la_chunk_fwd(q.cuda(), k.cuda(), v.cuda(), None, s_in.cuda(), mode="none", subseg_chunks=subseg)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), torch.from_numpy(o_ref).to(dt)), subseg
        assert torch.equal(s.cpu().double(), torch.from_numpy(s_ref)), subseg


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_impulse_causality_and_determinism(dtype):
    """Changing token j leaves o_t bit-identical for every t < j; two runs are bit-identical."""
    dk = 128 if dtype == "bf16" else 32
    w = W2.scaled(B=1, H=2, L=1000, dk=dk, dv=dk, dtype=dtype, decay="head_pow2", seed=91)
    note(f"impulse/causality {dtype}")
    d = to_dev(make_inputs(w, "cpu"))
    o1, s1 = _fwd(d, w)
    o1b, s1b = _fwd(d, w)
    for j in (0, 63, 64, 65, 500, 999):
        d2 = {k: (None if t is None else t.clone()) for k, t in d.items()}
        for key in ("q", "k", "v"):
            d2[key][:, :, j] += 0.5
        o2, _ = _fwd(d2, w)
        torch.cuda.synchronize()
        assert torch.equal(o1[:, :, :j], o2[:, :, :j]), j
        assert not torch.equal(o1[:, :, j:], o2[:, :, j:]), j
    torch.cuda.synchronize()
    assert torch.equal(o1, o1b) and torch.equal(s1, s1b)


def test_chunk_and_split_invariance():
    """Chunk length and internal sub-segment length change rounding only."""
    w = W3.scaled(B=1, H=2, L=2048, dtype="f32", dk=32, dv=32, seed=95)
    note("chunk-size invariance fp32 gate")
    d = to_dev(make_inputs(w, "cpu"))
    outs = [_fwd(d, w, chunk=c)[0] for c in (16, 32, 64)]
    torch.cuda.synchronize()
    ref = outs[0].double().cpu().numpy()
    for o in outs[1:]:
        assert rel_err(o, ref) <= 1e-5
    w = W3.scaled(B=1, H=2, L=64 * 40, seed=96)
    note("sub-segment invariance bf16 gate d128")
    d = to_dev(make_inputs(w, "cpu"))
    o_ref, _ = oracle_run(make_inputs(w, "cpu"), w)
    for subseg in (0, 1, 2, 5, 40, 1000):
        o, _ = _fwd(d, w, subseg=subseg)
        torch.cuda.synchronize()
        assert rel_err(o, o_ref) <= TOL["bf16"], subseg
    o32, _ = _fwd(d, w, chunk=32)  # generic bf16 path
    torch.cuda.synchronize()
    assert rel_err(o32, o_ref) <= TOL["bf16"]


def test_edge_cases():
    note("edge cases: empty L, B=0, L < chunk, L=1, a=1 head, a=0 head")
    w = W2.scaled(B=2, H=2, L=0, s_in_std=0.05, seed=99)
    d = to_dev(make_inputs(w, "cpu"))
    o, s = _fwd(d, w, nseg=3)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(s[:, :, 0], d["s_in"]) and torch.all(s[:, :, 1:] == 0)
    w = W2.scaled(B=0, L=100, seed=99)
    d = to_dev(make_inputs(w, "cpu"))
    o, s = _fwd(d, w)
    assert o.numel() == 0
    for L in (1, 5, 63):
        w = W2.scaled(B=1, H=2, L=L, s_in_std=0.05, seed=100 + L)
        inp = make_inputs(w, "cpu")
        o_ref, s_ref = oracle_run(inp, w)
        o, s = _fwd(to_dev(inp), w)
        torch.cuda.synchronize()
        assert rel_err(o, o_ref) <= TOL["bf16"] and rel_err(s, s_ref) <= TOL["bf16"], L
    # head mode with lambda = 0 equals no decay; lambda = -inf gives a = 0
    w = W2.scaled(B=1, H=2, L=300, s_in_std=0.05, seed=111)
    inp = make_inputs(w, "cpu")
    d = to_dev(inp)
    for lam, ref_mode in ((0.0, "none"), (-float("inf"), "zero")):
        dec = torch.full((2,), lam, device="cuda")
        o, s = lb.la_chunk_fwd(d["q"], d["k"], d["v"], dec, d["s_in"], mode="head")
        torch.cuda.synchronize()
        dec_h = np.full(2, lam, np.float32)
        o_ref, s_ref = oracle.recurrence(host32(inp["q"]), host32(inp["k"]), host32(inp["v"]), oracle.HEAD, dec_h,
                                         host32(inp["s_in"]).astype(np.float64))
        assert rel_err(o, o_ref) <= TOL["bf16"], lam
        assert rel_err(s, s_ref) <= TOL["bf16"], lam


@pytest.mark.parametrize("subseg", [0, 1, 2, 3, 5])
def test_head_decay_both_walks(subseg):
    """d = 128 head decay: the output pass takes its factorised walk (the intra-chunk product on v
    scaled by the state update's weights, one scale per output row) while lambda (C - 1) log2(e)
    >= -100, and keeps per-pair factors for stronger decays; heads on both sides of that bound
    (lambda = -1.0 and -1.2 straddle it), with lambda = 0, -inf and the workload's weakest decay,
    in one launch, against the oracle (ragged length, several sub-segments, s_in).  The sub-segment
    lengths give walks of 1 to 5 chunks, so the factorised walk's loaders run every form of their
    loop (two chunks in flight, the peeled tail, walks shorter than four chunks)."""
    lams = np.array([-1e-4, -0.02, -0.5, -1.0, -1.2, -3.0, 0.0, -np.inf], np.float32)
    w = W2.scaled(B=1, H=len(lams), L=64 * 9 + 19, s_in_std=0.05, seed=777 + subseg)
    note(f"head decay both walks, d=128 subseg_chunks={subseg} lambdas={lams.tolist()}")
    inp = make_inputs(w, "cpu")
    inp["decay"] = torch.from_numpy(lams)
    d = to_dev(inp)
    o, s = lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode="head", subseg_chunks=subseg)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence(host32(inp["q"]), host32(inp["k"]), host32(inp["v"]), oracle.HEAD, lams,
                                     host32(inp["s_in"]).astype(np.float64))
    for h in range(len(lams)):
        assert rel_err(o[:, h:h + 1], o_ref[:, h:h + 1]) <= TOL["bf16"], lams[h]
        assert rel_err(s[:, h:h + 1], s_ref[:, h:h + 1]) <= TOL["bf16"], lams[h]


@pytest.mark.parametrize("mode", ["none", "head", "gate"])
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("L,nseg,subseg", [(128 * 9 + 17, 1, 0), (128 * 6, 1, 1), (128 * 7 + 40, 1, 3), (300, 1, 0),
                                           (2 * (128 * 4 + 70), 2, 2)])
def test_chunk128_small_heads(mode, d, L, nseg, subseg):
    """128-token chunks (bf16, d = 32 / 64, the matrix-core kernels' chunk-length variant): o and the
    segment states against the oracle; ragged tails, one chunk per sub-segment, several segments."""
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    w = W2.scaled(B=2, H=3, L=L, dk=d, dv=d, decay=decay, s_in_std=0.05, qkv_std=d ** -0.5, seed=900 + L + d)
    note(f"bf16 d{d} chunk128 mode={mode} L={L} nseg={nseg} subseg_chunks={subseg}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w, nseg=nseg)
    o, s = _fwd(to_dev(inp), w, nseg=nseg, chunk=128, subseg=subseg)
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("mode", ["head", "gate"])
@pytest.mark.parametrize("d", [32, 64])
def test_chunk128_decayed_and_device_step(mode, d):
    """128-token chunks through la_chunk_fwd_decayed (q_decayed, segment totals, 64-token tile flags:
    a tile flagged zero holds only zero rows) and through the device step, against the oracle."""
    decay = {"head": "head_pow2", "gate": "gate"}[mode]
    L, nseg = 3 * (128 * 5 + 33), 3
    w = W2.scaled(B=2, H=3, L=L, dk=d, dv=d, decay=decay, s_in_std=0.05, qkv_std=d ** -0.5, seed=950 + d)
    note(f"la_chunk_fwd_decayed / device step, bf16 d{d} chunk128 mode={mode}")
    inp = make_inputs(w, "cpu")
    dv_ = to_dev(inp)
    o, s, qd, tot, live = lb.la_chunk_fwd_decayed(dv_["q"], dv_["k"], dv_["v"], dv_["decay"], dv_["s_in"], mode=w.mode,
                                                  nseg=nseg, chunk=128, gate_norm=w.gate_norm, want_tile_live=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_run(inp, w, nseg=nseg)
    assert rel_err(o, o_ref) <= TOL["bf16"] and rel_err(s, s_ref) <= TOL["bf16"]
    Ls = L // nseg
    assert live.shape[-1] == (Ls + 63) // 64
    qz = torch.nn.functional.pad(qd.reshape(w.B, w.H, nseg, Ls, d), (0, 0, 0, live.shape[-1] * 64 - Ls))
    assert not torch.any(qz.reshape(w.B, w.H, nseg, -1, 64 * d).ne(0).any(-1) & (live == 0))
    cref, tref = oracle.cumdecay(w.B, w.H, w.L, d, ORC_MODE[w.mode], host32(inp["decay"]), nseg=nseg,
                                 gate_norm=w.gate_norm)
    ref = host32(inp["q"]).astype(np.float64) * cref
    assert np.all(np.abs(qd.cpu().double().numpy() - ref) <= (2.0 ** -8 + 2e-4) * np.abs(ref) + 1e-35)
    assert np.max(np.abs(tot.cpu().double().numpy() - tref) / np.maximum(np.abs(tref), 1e-30)) < 2e-4
    # device step: S_recv drawn, the whole sequence as one device's share
    w1 = w.scaled(L=128 * 12 + 64)
    inp1 = make_inputs(w1, "cpu")
    s_recv = torch.randn((w1.B, w1.H, d, d), generator=torch.Generator().manual_seed(5)) * 0.05
    d1 = to_dev(inp1)
    step = pipeline.DeviceStep(d1["q"], d1["k"], d1["v"], d1["decay"], s_recv.cuda(), mode=w1.mode, chunk=128,
                               gate_norm=w1.gate_norm)
    o1, s_out = step.run()
    torch.cuda.synchronize()
    inp1 = dict(inp1, s_in=s_recv)
    o1_ref, s1_ref = oracle_run(inp1, w1)
    assert rel_err(o1, o1_ref) <= TOL["bf16"]
    assert rel_err(s_out, s1_ref[:, :, 0]) <= TOL["bf16"]


@pytest.mark.parametrize("mode,form", [("none", "decomposed"), ("head", "decomposed"), ("gate", "decomposed"),
                                       ("none", "exact"), ("head", "exact"), ("gate", "exact")])
def test_device_step_graph_replay(mode, form):
    """The device step captured in a HIP graph (through torch.cuda.graph) and replayed several times,
    with eager work and synchronisations between the replays: every replay's O and outgoing state
    equal the eager step's bit for bit (the library enqueues kernels only: no memsets, no host sync).
    The warm-up leaves a kept workspace on the side stream; the captured calls allocate per call."""
    decay = {"none": "none", "head": "head_pow2", "gate": "gate"}[mode]
    w = W2.scaled(B=1, H=4, L=64 * 40, decay=decay, s_in_std=0.05, seed=1500)
    note(f"device step graph replay, bf16 d128 mode={mode} form={form}")
    d = to_dev(make_inputs(w, "cpu"))
    if form == "exact":
        step = pipeline.ExactStep(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode=w.mode, chunk=64,
                                  gate_norm=w.gate_norm)
    else:
        step = pipeline.DeviceStep(d["q"], d["k"], d["v"], d["decay"], d["s_in"], mode=w.mode, chunk=64,
                                   gate_norm=w.gate_norm, subseg=4)
    o_ref, s_ref = (x.clone() for x in step.run())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as graph capture asks
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g, s_g = step.run()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(4):
        step.o.zero_()  # eager work between the replays
        scratch.add_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref), rep
        assert torch.equal(s_g, s_ref), rep


def test_kept_workspace_grows_and_follows_streams():
    """The forward's workspace stays with its stream between calls: calls of growing and shrinking
    sizes on one stream, and calls on two streams in flight together, each give the result of the
    allocation-free forward (same kernels) bit for bit; so do the calls after la_trim_workspace."""
    note("kept workspace: sizes and streams")
    ws = [W2.scaled(B=1, H=h, L=L, decay="head_pow2", s_in_std=0.05, seed=2100 + L)
          for h, L in ((2, 64 * 6), (4, 64 * 40 + 17), (3, 64 * 20))]
    ins = [to_dev(make_inputs(w, "cpu")) for w in ws]

    def outs(w):
        return (torch.empty((w.B, w.H, w.L, w.dv), dtype=torch.bfloat16, device="cuda"),
                torch.empty((w.B, w.H, 1, w.dk, w.dv), dtype=torch.float32, device="cuda"))

    refs = []
    for w, d in zip(ws, ins):
        o, s_ = outs(w)
        lb.la_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["decay"], d["s_in"], o, s_, mode=w.mode)
        refs.append((o, s_))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rnd in range(2):
        plan = [(sa, 0), (sb, 1), (sa, 1), (sb, 2), (sa, 2), (sb, 0), (sa, 0)]
        res = [outs(ws[i]) for _, i in plan]
        torch.cuda.synchronize()
        for (st, i), (o, s_) in zip(plan, res):
            d = ins[i]
            lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], d["s_in"], o, s_, mode=ws[i].mode, stream=st)
        torch.cuda.synchronize()
        for n, ((st, i), (o, s_)) in enumerate(zip(plan, res)):
            assert torch.equal(o, refs[i][0]) and torch.equal(s_, refs[i][1]), (rnd, n)
        lb.la_trim_workspace()


def test_trim_workspace_between_calls():
    """la_trim_workspace hands the pool's unused memory back; the next calls obtain it again and
    give bit-identical results (forward with its sub-segment split, backward, gate cumulative decay)."""
    w = W3.scaled(B=1, H=4, L=4096, seed=77)
    note("la_trim_workspace between calls")
    d = to_dev(make_inputs(w, "cpu"))
    o1, s1 = lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], None, mode="gate")
    c1, t1 = lb.la_cumdecay(d["decay"], w.B, w.H, w.L, w.dk, mode="gate")
    torch.cuda.synchronize()
    lb.la_trim_workspace()
    o2, s2 = lb.la_chunk_fwd(d["q"], d["k"], d["v"], d["decay"], None, mode="gate")
    c2, t2 = lb.la_cumdecay(d["decay"], w.B, w.H, w.L, w.dk, mode="gate")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(c1, c2) and torch.equal(t1, t2)
