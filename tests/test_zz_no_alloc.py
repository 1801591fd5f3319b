"""la_chunk_fwd_noalloc against la_chunk_fwd through the C ABI.

The allocation-free forward runs the same kernels with the same split into sub-segments, only its
workspace is the library's fixed device array, so its outputs must equal la_chunk_fwd's bit for bit.
Two calls in a row on the same device, the second on a smaller input, check that the array's
contents left by one call do not leak into the next.  The file is named to be collected last.
"""
import pytest
import torch

from chunked_scan_amd import binding as B
from chunked_scan_amd.inputs import WORKLOADS, make_inputs
from tests.gpu_util import note, oracle_run, rel_err, TOL

pytestmark = pytest.mark.gpu

# (workload index for the decay recipe, B, H, L, d, chunk): the first call of each pair is the larger
CASES = [
    ((2, 1, 4, 8192, 128, 64), (3, 1, 2, 2048, 128, 64)),
    ((3, 2, 2, 4096, 64, 64), (1, 1, 2, 1536, 64, 64)),
    ((2, 1, 4, 4096, 32, 128), (3, 1, 1, 1024, 32, 128)),
]


def _inputs(widx, Bn, H, L, d, seed):
    w = WORKLOADS[widx].scaled(B=Bn, H=H, L=L, dk=d, dv=d, qkv_std=d ** -0.5, seed=seed)
    return w, make_inputs(w, "cuda")


def _both(w, inp, chunk):
    s_in = inp["s_in"]
    o_ref, s_ref = B.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["decay"], s_in, mode=w.mode, chunk=chunk,
                                  gate_norm=w.gate_norm)
    o = torch.empty_like(o_ref)
    s_out = torch.empty_like(s_ref)
    B.la_chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["decay"], s_in, o, s_out, mode=w.mode, chunk=chunk,
                           gate_norm=w.gate_norm)
    torch.cuda.synchronize()
    return o_ref, s_ref, o, s_out


@pytest.mark.parametrize("pair", CASES, ids=["d128_head_then_gate", "d64_gate_then_none", "d32_c128_head_then_gate"])
def test_noalloc_equals_la_chunk_fwd_twice(pair):
    for n, (widx, Bn, H, L, d, chunk) in enumerate(pair):
        note(f"la_chunk_fwd_noalloc call {n}: workload {widx} B={Bn} H={H} L={L} d={d} chunk={chunk}")
        w, inp = _inputs(widx, Bn, H, L, d, seed=100 + n)
        o_ref, s_ref, o, s_out = _both(w, inp, chunk)
        assert torch.equal(o, o_ref), f"call {n}: O differs from la_chunk_fwd"
        assert torch.equal(s_out, s_ref), f"call {n}: S_out differs from la_chunk_fwd"
        if n == 1:  # the smaller call also against the oracle, at the bf16 bound
            ref_o, ref_s = oracle_run({k: (None if t is None else t.cpu()) for k, t in inp.items()}, w)
            assert rel_err(o, ref_o) <= TOL["bf16"]
            assert rel_err(s_out[:, :, 0], ref_s[:, :, 0]) <= TOL["bf16"]


def test_noalloc_rejects_oversized_split():
    # one chunk per sub-segment over 16 heads x 16k tokens needs ~270 MB of sub-segment states
    w = WORKLOADS[1]
    inp = make_inputs(w.scaled(B=1, H=16, L=16384, seed=7), "cuda")
    note("la_chunk_fwd_noalloc rejection: subseg_chunks=1 at B1 H16 L16384 d128")
    with pytest.raises(B.LaError) as ei:
        B.la_chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], None, None, mode="none", subseg_chunks=1)
    assert ei.value.status == -8
