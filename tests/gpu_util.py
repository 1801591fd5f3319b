"""Helpers shared by the GPU parity tests: device copies, oracle calls, error metrics."""
import sys

import numpy as np
import torch

import oracle
from chunked_scan_amd.inputs import Workload

ORC_MODE = {"none": oracle.NONE, "head": oracle.HEAD, "gate": oracle.GATE}
# Tolerances on max|gpu - ref| / max|ref| per output tensor: a genuine fp32 path must meet 1e-5;
# bf16 inputs with fp32 state and fp32 accumulation must meet 2e-2.
TOL = {"f32": 1e-5, "bf16": 2e-2}


def note(msg: str) -> None:
    """Name the case about to run on the GPU, flushed first, so a fault can be attributed."""
    sys.stdout.write("\n[gpu case] " + msg + "\n")
    sys.stdout.flush()


def to_dev(inp: dict, device="cuda") -> dict:
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def host32(t):
    """Exact float32 numpy copy of a (bf16 or f32) tensor."""
    return None if t is None else t.detach().to("cpu", torch.float32).numpy()


def oracle_run(inp: dict, w: Workload, nseg: int = 1, with_s_in: bool = True):
    dec = host32(inp["decay"])
    s_in = host32(inp["s_in"]) if with_s_in and inp["s_in"] is not None else None
    return oracle.recurrence(host32(inp["q"]), host32(inp["k"]), host32(inp["v"]), ORC_MODE[w.mode], dec,
                             None if s_in is None else s_in.astype(np.float64), nseg=nseg, gate_norm=w.gate_norm)


def rel_err(got, ref) -> float:
    g = got.detach().to("cpu", torch.float64).numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    den = np.max(np.abs(r))
    if den == 0:
        return float(np.max(np.abs(g)))
    return float(np.max(np.abs(g - r)) / den)
