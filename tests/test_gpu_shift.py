"""GPU parity of the band-edge continuity shift (long_mode flag BF_LONG_SHIFT:
the far query sits at phi(p) + w0 - phi(w0)) against the fp64 oracle, for
FI and PA, prefill and decode. Needs an MI355X. Tolerances as for the
bifocal calls: bf16 max-abs 2e-2 and mean-abs 2e-3, fp32 max-abs 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from rope_context_extension_bifocal_amd import bifocal as bfl
from rope_context_extension_bifocal_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()
    yield


def _check(gpu, ref, what, mx_tol=2e-2, mean_tol=2e-3):
    d = np.abs(np.asarray(gpu, np.float64) - ref)
    print(f"[{what}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= mx_tol and d.mean() <= mean_tol, what


@pytest.mark.parametrize("mode", ["fi+shift", "pa+shift"])
def test_shift_prefill_bf16(mode):
    lens = [700, 413, 129, 1]
    cu = wl.cu_seqlens(lens)
    q, k, v = wl.prefill_inputs(8, 2, cu[-1], 128, "bf16", 91)
    scale = 1 / math.sqrt(128)
    o, lse = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), cu, 64, 256, 1e6, mode, scale, return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), cu, 64,
                                    256, 1e6, mode, scale)
    _check(o.float().cpu().numpy(), o_ref, f"shift prefill {mode}")
    _check(lse.cpu().numpy(), lse_ref, f"shift lse {mode}")
    # the shift is not a no-op at these sizes: the unshifted oracle differs
    o_no, _ = oracle.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), cu, 64, 256,
                             1e6, mode.split("+")[0], scale)
    assert np.abs(o_no - o_ref).max() > 5e-2


@pytest.mark.parametrize("mode", ["fi+shift", "pa+shift"])
def test_shift_prefill_fp32_full(mode):
    c = wl.CONFIGS["tiny_fp32_s2"]
    L = c["lens"][0]
    q, k, v = wl.prefill_inputs(c["Hq"], c["Hkv"], L, 128, "fp32", c["seed"])
    scale = 1 / math.sqrt(128)
    o = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), [0, L], c["w0"], c["w_pre"], c["theta"], mode, scale)
    torch.cuda.synchronize()
    o_ref, _ = oracle.prefill(q.numpy(), k.numpy(), v.numpy(), [0, L], c["w0"], c["w_pre"],
                              c["theta"], mode, scale)
    d = np.abs(o.cpu().numpy().astype(np.float64) - o_ref)
    print(f"[shift fp32 {mode}] max-abs {d.max():.3e}", flush=True)
    assert d.max() <= 1e-4


def test_shift_prefill_128k_sampled():
    c = wl.CONFIGS["qwen3_8b_prefill_128k"]
    L = c["lens"][0]
    q, k, v = wl.prefill_inputs(c["Hq"], c["Hkv"], L, 128, "bf16", c["seed"])
    scale = 1 / math.sqrt(128)
    o = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), [0, L], c["w0"], c["w_pre"], c["theta"], "fi+shift",
                    scale)
    torch.cuda.synchronize()
    w0 = c["w0"]
    rows = wl.sample_rows(L, 24, [0, w0 - 1, w0, w0 + 1, c["w_pre"], L - 1], seed=92)
    o_ref, _ = oracle.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), [0, L], w0,
                              c["w_pre"], c["theta"], "fi+shift", scale, rows=rows)
    _check(o[:, torch.from_numpy(rows).cuda()].float().cpu().numpy(), o_ref, "shift prefill 128k")


@pytest.mark.parametrize("mode", ["fi+shift", "pa+shift"])
@pytest.mark.parametrize("N", [1000, 32769, 131073])
def test_shift_decode(N, mode):
    Hq, Hkv = 32, 8
    w0, w_pre = (64, 256) if N == 1000 else (4096, 32768)
    q, kc, vc = wl.decode_inputs(1, Hq, Hkv, N, 128, "bf16", 93)
    scale = 1 / math.sqrt(128)
    o = bfl.decode(q.cuda(), kc.cuda(), vc.cuda(), [N], w0, w_pre, 1e6, mode, scale)
    torch.cuda.synchronize()
    o_ref, _ = oracle.decode(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), [N], w0,
                             w_pre, 1e6, mode, scale)
    _check(o.float().cpu().numpy(), o_ref, f"shift decode {mode} N={N}")
