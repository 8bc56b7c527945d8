"""bifocal_decode_noalloc against bifocal_decode (needs an MI355X).

The allocation-free entry point runs the same kernels with the split
partials in the library's per-GPU scratch array instead of a workspace, so
its output must be bitwise the workspace call's. Two calls in a row, the
second smaller, so the second meets the first one's leftovers in the scratch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from rope_context_extension_bifocal_amd import bifocal as bfl
from rope_context_extension_bifocal_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _pair(B, Hq, Hkv, cap, Ns, mode, seed):
    q, kc, vc = (x.cuda() for x in wl.decode_inputs(B, Hq, Hkv, cap, 128, "bf16", seed))
    args = (q, kc, vc, Ns, 4096, 32768, 1e6, mode, 1 / math.sqrt(128))
    o_ws, l_ws = bfl.decode(*args, return_lse=True)
    o_na, l_na = bfl.decode_noalloc(*args, return_lse=True)
    torch.cuda.synchronize()
    return (q, kc, vc), (o_ws, l_ws), (o_na, l_na)


def test_noalloc_decode_is_the_workspace_decode_twice():
    print("[noalloc] call 1: B=2, 32/8 heads, N = 131073 and 40000, FI", flush=True)
    _, (o1, l1), (n1, m1) = _pair(2, 32, 8, 131073, [131073, 40000], "fi", 61)
    assert torch.equal(o1, n1) and torch.equal(l1, m1)
    print("[noalloc] call 2: B=1, 16/2 heads, N = 3000, PA (smaller)", flush=True)
    (q, kc, vc), (o2, l2), (n2, m2) = _pair(1, 16, 2, 3000, [3000], "pa", 62)
    assert torch.equal(o2, n2) and torch.equal(l2, m2)
    # and the decode tolerance against the oracle on the smaller call
    ref, _ = oracle.decode(q.float().cpu().numpy(), kc.float().cpu().numpy(),
                           vc.float().cpu().numpy(), [3000], 4096, 32768, 1e6, "pa",
                           1 / math.sqrt(128))
    d = np.abs(n2.float().cpu().numpy() - ref)
    print(f"[noalloc] small call vs oracle: max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
