"""GPU parity at the largest sizes exercised: one 1,048,576-token sequence
(prefill, s = 32 at w_pre = 32768) and a decode over 1,048,577 cached keys,
checked on sampled rows against the fp64 oracle at the usual bar (bf16
max-abs 2e-2, mean-abs 2e-3), with the discrimination check (error small next
to the gap to plain attention). Element offsets here pass 2^31 (q alone holds
2^30 elements, the packed V^T and k'' index past 2^28 rows), so a 32-bit
offset anywhere would show. Needs an MI355X.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from rope_context_extension_bifocal_amd import bifocal as bfl
from rope_context_extension_bifocal_amd import workloads as wl

pytestmark = pytest.mark.gpu

THETA = 1e6
SCALE = 1 / math.sqrt(128)
L = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()
    yield


def _check(gpu, ref, what):
    d = np.abs(np.asarray(gpu, np.float64) - ref)
    print(f"[{what}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, what


def test_prefill_1m_tokens_sampled():
    Hq, Hkv, w0, w_pre = 8, 2, 4096, 32768  # s = 32
    q, k, v = wl.prefill_inputs(Hq, Hkv, L, 128, "bf16", 601)
    o = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), [0, L], w0, w_pre, THETA, "fi", SCALE)
    torch.cuda.synchronize()
    rows = wl.sample_rows(L, 10, [0, w0 - 1, w0, w_pre, L // 2, L - 2, L - 1], seed=602)
    rows = np.asarray(rows)
    qs = q[:, torch.from_numpy(rows)].float().numpy()
    kf, vf = k.float().numpy(), v.float().numpy()
    ref, _ = oracle.prefill(qs, kf, vf, [0, L], w0, w_pre, THETA, "fi", SCALE, rows=rows,
                            gathered=True)
    og = o[:, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    _check(og, ref, "prefill 1M")
    far = rows >= w0
    plain, _ = oracle.prefill(qs, kf, vf, [0, L], 10**9, w_pre, THETA, "fi", SCALE, rows=rows,
                              gathered=True)
    err = np.linalg.norm(og[:, far] - ref[:, far])
    gap = np.linalg.norm(ref[:, far] - plain[:, far])
    print(f"[prefill 1M discrimination] err {err:.3e} gap-plain {gap:.3e}", flush=True)
    assert err <= 0.05 * gap


def test_decode_1m_keys():
    Hq, Hkv, N = 8, 2, L + 1
    q, kc, vc = wl.decode_inputs(1, Hq, Hkv, N, 128, "bf16", 603)
    o = bfl.decode(q.cuda(), kc.cuda(), vc.cuda(), [N], 4096, 32768, THETA, "pa", SCALE)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), [N], 4096,
                           32768, THETA, "pa", SCALE)
    _check(o.float().cpu().numpy(), ref, "decode 1M")
