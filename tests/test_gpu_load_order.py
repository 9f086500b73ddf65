"""The library loaded before torch in a fresh process still shares torch's HIP runtime
(a second runtime would drop the launches on torch's streams without an error)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, %r)
import deterministic_exact_top_amd as detk
detk.load_library()                      # before anything imports torch
detk.debug_set(detk.DETK_DEBUG_FAST, 0)  # (a call into the library before torch is used)
import numpy as np, torch
import oracle, workloads as W
wl = W.plateau_abs(B=3, L=4096, k=2048, name="load_order")
s = torch.from_numpy(wl.scores).cuda()
gi, gv = detk.topk_ragged(s, torch.from_numpy(wl.row_starts).cuda(), torch.from_numpy(wl.lengths).cuda(), wl.k,
                          max_len=wl.max_len)
torch.cuda.synchronize()
oi, ov = oracle.topk_ragged(wl.scores, wl.row_starts, wl.lengths, wl.k, wl.max_len)
ok = np.array_equal(gi.cpu().numpy(), oi) and np.array_equal(gv.cpu().numpy().view(np.uint32), ov)
print("same" if ok else "DIFFERENT")
sys.exit(0 if ok else 1)
"""


def test_library_loaded_before_torch():
    print("fresh process: library loaded before torch", flush=True)
    r = subprocess.run([sys.executable, "-c", SCRIPT % ROOT], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "same" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
