"""GPU parity of the backward pass at the full workload sizes (B·H·16384 tokens, d = 128, bf16), in
the launch configuration the benchmark times (matrix-core kernels, 8 or 16 sub-segments).

The loss derivative d_o is drawn as usual but kept only on the last M tokens of every sequence
(1.5 chunks: a ragged window); ds_out is drawn in full.  The exact derivatives then follow from the
fp64 oracle on a sampled (b, h) without a whole-sequence backward: the oracle's forward over the
first L - M tokens gives the state S before the window, its backward over the window (from S, with
ds_out) gives dq, dk, dv there and G', the derivative with respect to S; every earlier token j has
G_j = a^{L-M-1-j} G' (no d_o before the window), so dk_j = G_j v_j, dv_j = G_j^T k_j, dq_j = 0 and
ds_in = a^{L-M} G'.  In gate mode the decay differs per token and key dim, so the oracle's backward
over the first L - M tokens with d_o = 0 and ds_out = G' gives those tokens' dk, dv, dg and ds_in.
Every token of the sampled sequences is compared.  The head-decay derivative is checked against its
definition as a sum over token pairs (numpy, fp64), over both batch entries.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_scan_amd import binding as lb
from chunked_scan_amd.inputs import WORKLOADS, make_grads, make_inputs

from gpu_util import ORC_MODE, TOL, host32, note, rel_err

pytestmark = pytest.mark.gpu

M = 96  # tokens at the end that carry a loss derivative


def _f64(t):
    return host32(t).astype(np.float64)


def _expected(inp, gr, d_o, w, b, h):
    """Exact dq, dk, dv [L, d] and ds_in [dk, dv] of sequence (b, h) (fp64)."""
    L = w.L
    q, k, v = (host32(inp[x][b, h]) for x in ("q", "k", "v"))
    gate = w.mode == "gate"
    lam = None if w.mode in ("none", "gate") else float(host32(inp["decay"])[h])
    win, pre = slice(L - M, L), slice(0, L - M)
    if w.mode == "none":
        dec_pre = dec_win = None
    elif gate:  # per-token gate [B, H, L, dk]
        g = host32(inp["decay"])[b:b + 1, h:h + 1]
        dec_pre, dec_win = g[:, :, pre], g[:, :, win]
    else:
        dec_pre = dec_win = host32(inp["decay"])[h:h + 1]
    s_in = None if inp["s_in"] is None else _f64(inp["s_in"][b, h])[None, None]
    # forward state before the window
    _, s_pre = oracle.recurrence(q[None, None, pre], k[None, None, pre], v[None, None, pre],
                                 ORC_MODE[w.mode], dec_pre, s_in, gate_norm=w.gate_norm)
    dqw, dkw, dvw, dgw, dsw = oracle.recurrence_bwd(
        q[None, None, win], k[None, None, win], v[None, None, win], host32(d_o[b, h])[None, None, win],
        ORC_MODE[w.mode], dec_win, s_pre[:, :, 0], _f64(gr["ds_out"][b, h])[None, None], gate_norm=w.gate_norm)
    G = dsw[0, 0, 0]  # derivative with respect to the state before the window
    if gate:
        _, dkp, dvp, dgp, dsp = oracle.recurrence_bwd(
            q[None, None, pre], k[None, None, pre], v[None, None, pre], np.zeros((1, 1, L - M, w.dv), np.float32),
            ORC_MODE[w.mode], dec_pre, s_in, G[None, None, None], gate_norm=w.gate_norm)
        dq = np.zeros((L, w.dk))
        dq[win] = dqw[0, 0]
        return (dq, np.concatenate([dkp[0, 0], dkw[0, 0]]), np.concatenate([dvp[0, 0], dvw[0, 0]]),
                dsp[0, 0, 0], np.concatenate([dgp[0, 0], dgw[0, 0]]))
    j = np.arange(L - M)
    f = np.ones(L - M) if lam is None else np.exp(lam * (L - M - 1 - j))
    dq = np.zeros((L, w.dk))
    dq[win] = dqw[0, 0]
    dk = np.concatenate([f[:, None] * (v[:L - M].astype(np.float64) @ G.T), dkw[0, 0]])
    dv = np.concatenate([f[:, None] * (k[:L - M].astype(np.float64) @ G), dvw[0, 0]])
    ds_in = (1.0 if lam is None else np.exp(lam * (L - M))) * G
    return dq, dk, dv, ds_in, None


def _dlambda_pairs(inp, gr, d_o, w, h):
    """d lambda_h from its definition: sum over b and token pairs j <= t of (t - j) a^{t-j}
    (q_t . k_j)(v_j . d_o_t), plus (t + 1) a^{t+1} q_t^T s_in d_o_t and <ds_out, dS_out / dlambda>
    (d_o is zero before the window)."""
    L = w.L
    lam = float(host32(inp["decay"])[h])
    total = 0.0
    for b in range(w.B):
        q, k, v, do = (_f64(x[b, h]) for x in (inp["q"], inp["k"], inp["v"], d_o))
        s_in = None if inp["s_in"] is None else _f64(inp["s_in"][b, h])
        for t in range(L - M, L):
            dist = t - np.arange(t + 1)
            total += np.sum(dist * np.exp(lam * dist) * (k[:t + 1] @ q[t]) * (v[:t + 1] @ do[t]))
            if s_in is not None:
                total += (t + 1) * np.exp(lam * (t + 1)) * (q[t] @ s_in @ do[t])
        dist = L - 1 - np.arange(L)
        dS = (k * (dist * np.exp(lam * dist))[:, None]).T @ v
        if s_in is not None:
            dS += L * np.exp(lam * L) * s_in
        total += np.sum(_f64(gr["ds_out"][b, h, 0]) * dS)
    return total


@pytest.mark.parametrize("wid,pairs,want_decay", [(1, [(0, 0), (0, 9)], False),
                                                  (2, [(0, 3), (1, 14)], False),
                                                  (2, [(1, 0), (0, 12)], True),
                                                  (3, [(0, 5), (3, 11)], False),
                                                  (3, [(2, 7), (1, 15)], True)])
def test_backward_full_size(wid, pairs, want_decay):
    w = WORKLOADS[wid]
    note(f"la_chunk_bwd full size, workload {wid} {w.name}, d_lambda={want_decay}, sampled (b,h) {pairs}")
    inp = make_inputs(w, "cuda")
    gr = make_grads(w, device="cuda")
    d_o = gr["d_o"].clone()
    d_o[:, :, :w.L - M] = 0
    dq, dk, dv, dd, ds_in = lb.la_chunk_bwd(inp["q"], inp["k"], inp["v"], d_o, inp["decay"], inp["s_in"],
                                            gr["ds_out"], mode=w.mode, chunk=w.chunk, want_decay=want_decay)
    torch.cuda.synchronize()
    for b, h in pairs:
        e_dq, e_dk, e_dv, e_ds, e_dg = _expected(inp, gr, d_o, w, b, h)
        assert rel_err(dq[b, h], e_dq) <= TOL["bf16"], ("dq", b, h)
        assert rel_err(dk[b, h], e_dk) <= TOL["bf16"], ("dk", b, h)
        assert rel_err(dv[b, h], e_dv) <= TOL["bf16"], ("dv", b, h)
        # ds_in is fp32; the derivative decayed over a whole segment can lie below fp32's range
        # (head 0: a^16288 = e^-509), where the correctly rounded value is zero
        assert rel_err(ds_in[b, h, 0], e_ds.astype(np.float32)) <= TOL["bf16"], ("ds_in", b, h)
        assert torch.count_nonzero(dq[b, h, :w.L - M]) == 0  # no loss derivative before the window
        if want_decay and w.mode == "gate":  # dg of every token of the sequence (oracle, fp64)
            err = rel_err(dd[b, h], e_dg)
            print(f"  dg ({b},{h}) rel err {err:.2e}")
            assert err <= TOL["bf16"], ("dg", b, h)
        elif want_decay:
            ref = _dlambda_pairs(inp, gr, d_o, w, h)
            got = float(dd[h])
            print(f"  d_lambda[{h}] gpu {got:.6e} pairs {ref:.6e}")
            assert abs(got - ref) <= TOL["bf16"] * abs(ref), h


@pytest.mark.parametrize("wid,b_list,h,want_decay", [(1, [0], 9, False),
                                                     (2, [0, 1], 14, True),
                                                     (3, [2], 7, True)])
def test_backward_full_size_dense_d_o(wid, b_list, h, want_decay):
    """The same sizes and launch configuration with d_o drawn on every token: the oracle's backward
    runs over the whole 16384-token sequence of every sampled (b, h) (its state trajectory kept
    whole, about 2 GB per sequence), and every token of dq, dk, dv (and dg) is compared, with
    ds_in.  Head decay: both batch entries of head h are sampled, so the oracle's d lambda_h is
    complete and is compared too."""
    w = WORKLOADS[wid]
    note(f"la_chunk_bwd full size, dense d_o, workload {wid} {w.name}, d_decay={want_decay}, b {b_list} h {h}")
    inp = make_inputs(w, "cuda")
    gr = make_grads(w, device="cuda")
    dq, dk, dv, dd, ds_in = lb.la_chunk_bwd(inp["q"], inp["k"], inp["v"], gr["d_o"], inp["decay"], inp["s_in"],
                                            gr["ds_out"], mode=w.mode, chunk=w.chunk, want_decay=want_decay)
    torch.cuda.synchronize()
    sel = lambda t: host32(t[b_list, h][:, None])  # noqa: E731  [nb, 1, ...]
    if w.mode == "none":
        dec = None
    elif w.mode == "gate":
        dec = sel(inp["decay"])
    else:
        dec = host32(inp["decay"])[h:h + 1]
    s_in = None if inp["s_in"] is None else sel(inp["s_in"]).astype(np.float64)
    e_dq, e_dk, e_dv, e_dd, e_ds = oracle.recurrence_bwd(
        sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(gr["d_o"]), ORC_MODE[w.mode], dec, s_in,
        host32(gr["ds_out"][b_list, h][:, None]).astype(np.float64), gate_norm=w.gate_norm, threads=len(b_list))
    for i, b in enumerate(b_list):
        for name, got, ref in (("dq", dq, e_dq), ("dk", dk, e_dk), ("dv", dv, e_dv)):
            err = rel_err(got[b, h], ref[i, 0])
            print(f"  {name} ({b},{h}) rel err {err:.2e}")
            assert err <= TOL["bf16"], (name, b, h, err)
        assert rel_err(ds_in[b, h, 0], e_ds[i, 0, 0].astype(np.float32)) <= TOL["bf16"], ("ds_in", b, h)
        if want_decay and w.mode == "gate":
            err = rel_err(dd[b, h], e_dd[i, 0])
            print(f"  dg ({b},{h}) rel err {err:.2e}")
            assert err <= TOL["bf16"], ("dg", b, h, err)
    if want_decay and w.mode == "head":
        got, ref = float(dd[h]), float(e_dd[0])
        print(f"  d_lambda[{h}] gpu {got:.6e} oracle {ref:.6e}")
        assert abs(got - ref) <= TOL["bf16"] * abs(ref), (h, got, ref)
