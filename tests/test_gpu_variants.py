"""GPU parity of the forward's head-dim and chunk-length variants on the dv-tiled matrix-core
kernel (chunk_fwd_tiled.hip): dk = dv = 256 with 64-token chunks (four 64-column value tiles per
sub-segment), and dk = dv = 128 with 128-token chunks; no decay and per-head decay, against the
fp64 oracle, with ragged lengths, several sub-segments and segments, s_in present or not.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from chunked_scan_amd import binding as lb
from chunked_scan_amd.inputs import WORKLOADS, make_inputs

from gpu_util import TOL, host32, note, oracle_run, rel_err, to_dev

pytestmark = pytest.mark.gpu

W2 = WORKLOADS[2]
DECAY = {"none": "none", "head": "head_pow2"}
VARIANTS = {"d256": (256, 64), "d128_c128": (128, 128)}


def _w(variant, mode, B, H, L, seed):
    d, _ = VARIANTS[variant]
    return W2.scaled(B=B, H=H, L=L, dk=d, dv=d, qkv_std=1.0 / math.sqrt(d), decay=DECAY[mode], s_in_std=0.05,
                     seed=seed)


@pytest.mark.parametrize("variant", ["d256", "d128_c128"])
@pytest.mark.parametrize("mode", ["none", "head"])
@pytest.mark.parametrize("B,H,L,nseg,subseg,s_in", [(1, 2, 64 * 9 + 17, 1, 0, True), (2, 1, 64 * 16, 1, 1, True),
                                                    (1, 3, 128 * 5 + 40, 1, 2, False), (2, 2, 3 * 384, 3, 0, True),
                                                    (1, 1, 40, 1, 0, True)])
def test_variant_matches_oracle(variant, mode, B, H, L, nseg, subseg, s_in):
    d, chunk = VARIANTS[variant]
    w = _w(variant, mode, B, H, L, seed=4000 + L + subseg + d)
    note(f"forward variant {variant} mode={mode} B={B} H={H} L={L} nseg={nseg} subseg={subseg} s_in={s_in}")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w, nseg=nseg, with_s_in=s_in)
    dd = to_dev(inp)
    timer = lb.KernelTimer(8)
    o, s = lb.la_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"] if s_in else None, mode=w.mode,
                           nseg=nseg, chunk=chunk, subseg_chunks=subseg, timer=timer)
    torch.cuda.synchronize()
    assert "chunk_fwd_tiled_output_pass" in [n for n, _ in timer.harvest()]
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref) <= TOL["bf16"]
    # the allocation-free entry point runs the same kernels from its fixed array
    o2, s2 = lb.la_chunk_fwd_noalloc(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"] if s_in else None,
                                     mode=w.mode, nseg=nseg, chunk=chunk, subseg_chunks=subseg)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(s, s2)


@pytest.mark.parametrize("variant", ["d256", "d128_c128"])
def test_variant_integer_inputs_bit_exact(variant):
    """a = 1, q, k, v in {-1, 0, 1}, integer s_in: every intermediate is an exact integer, so the
    outputs are the exact result rounded once, whatever the tiling and the sub-segment order."""
    d, chunk = VARIANTS[variant]
    g = torch.Generator().manual_seed(4100 + d)
    B, H, L = 1, 2, 2 * chunk * 3 + 9
    note(f"forward variant {variant}, integer inputs, bit-exact")
    q, k, v = (torch.randint(-1, 2, (B, H, L, d), generator=g).to(torch.bfloat16) for _ in range(3))
    s_in = torch.randint(-8, 9, (B, H, d, d), generator=g).float()
    o_ref, s_ref = oracle.recurrence(host32(q), host32(k), host32(v), oracle.NONE, None, s_in.double().numpy())
    for subseg in (0, 1, 2):
        o, s = lb.la_chunk_fwd(q.cuda(), k.cuda(), v.cuda(), None, s_in.cuda(), mode="none", chunk=chunk,
                               subseg_chunks=subseg)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), torch.from_numpy(o_ref).to(torch.bfloat16)), subseg
        assert torch.equal(s.cpu().double(), torch.from_numpy(s_ref)), subseg


@pytest.mark.parametrize("variant", ["d256", "d128_c128"])
def test_variant_full_size(variant):
    """B1 H16 L16384 with head decay (the state-size sweep's shape): two sampled heads against the
    oracle over every token, and two runs bit-identical."""
    d, chunk = VARIANTS[variant]
    w = WORKLOADS[1].scaled(dk=d, dv=d, qkv_std=1.0 / math.sqrt(d), decay="head_pow2", s_in_std=0.05, seed=4200 + d)
    note(f"forward variant {variant} at full size")
    dd = make_inputs(w, "cuda")
    o, s = lb.la_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode=w.mode, chunk=chunk)
    o2, s2 = lb.la_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode=w.mode, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(s, s2)
    for h in (0, 11):
        sub = {"q": dd["q"][:, h:h + 1], "k": dd["k"][:, h:h + 1], "v": dd["v"][:, h:h + 1],
               "decay": dd["decay"][h:h + 1], "s_in": dd["s_in"][:, h:h + 1]}
        o_ref, s_ref = oracle_run({key: t.cpu() for key, t in sub.items()}, w.scaled(H=1))
        assert rel_err(o[:, h:h + 1], o_ref) <= TOL["bf16"], h
        assert rel_err(s[:, h:h + 1], s_ref) <= TOL["bf16"], h


def test_variant_device_step_d256():
    """The exact device step at d = 256 (one la_chunk_fwd from S_recv) equals the oracle's one pass
    with S_recv as the initial state; the scan runs on 256 x 256 states."""
    w = _w("d256", "head", 1, 4, 64 * 24, seed=4300)
    note("device step d = 256")
    inp = make_inputs(w, "cpu")
    o_ref, s_ref = oracle_run(inp, w)
    from chunked_scan_amd.pipeline import ExactStep

    dd = to_dev(inp)
    o, s = ExactStep(dd["q"], dd["k"], dd["v"], dd["decay"], dd["s_in"], mode=w.mode, subseg_chunks=3).run()
    torch.cuda.synchronize()
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(s, s_ref[:, :, 0]) <= TOL["bf16"]
    assert np.isfinite(o.float().cpu().numpy()).all()
