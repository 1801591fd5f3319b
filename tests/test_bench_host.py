"""Host-side logic of bench.py (no GPU): the one-GPU contract, the split plan it uses for byte
accounting, the per-token algorithmic bytes and the live-tile count of the head-decay correction."""
import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from chunked_scan_amd.inputs import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_split_plan_of_the_workloads():
    # about 256 workgroups at d = 128: G sub-segments of cps 64-token chunks per (b, h)
    assert bench.split_plan(WORKLOADS[1]) == (16, 16)
    assert bench.split_plan(WORKLOADS[2]) == (8, 32)
    assert bench.split_plan(WORKLOADS[3]) == (4, 64)
    # below d = 128 the target is 512; never fewer than four chunks per sub-segment
    assert bench.split_plan(WORKLOADS[1].scaled(dk=64, dv=64)) == (32, 8)
    assert bench.split_plan(WORKLOADS[1].scaled(L=64 * 10 + 3)) == (3, 4)


def test_algorithmic_bytes_per_token_head():
    w = WORKLOADS[1]
    by, fl = bench.algorithmic(w, 0)
    assert by == 2 * (128 + 128 + 128 + 128)  # q, k, v read and o written, bf16
    assert fl == 2 * 64 * 128 * 2 + 2 * 128 * 128 * 2
    assert bench.algorithmic(WORKLOADS[3], 4 * 128)[0] == by + 512  # plus the fp32 gate row


def test_live_correction_tokens_head_decay():
    # per head, the 64-token tiles whose cumulative decay at their first token is nonzero in fp32
    w = WORKLOADS[2].scaled(B=1, H=3, L=4096)
    lam = torch.tensor([-1.0, -0.02, 0.0])
    got = bench.live_correction_tokens(w, 4096, 2, {"decay": lam})
    want = 0
    for h in range(3):
        for t0 in range(0, 4096, 64):
            if np.float32(np.exp(np.float64(np.float32(lam[h].item())) * (t0 + 1))) != 0:
                want += min(64, 4096 - t0)
    assert got == w.B * want * 2
    # no decay: every token of every corrected segment
    w0 = WORKLOADS[1]
    assert bench.live_correction_tokens(w0, 1024, 3) == w0.B * w0.H * 1024 * 3
