"""GPU parity of the band-only special case (long_mode "band": far pairs
dropped, sliding-window attention over the w0 most recent keys with original
RoPE, as in the sliding-window layers of a hybrid model) against the fp64
oracle. Needs an MI355X. Tolerances as for the bifocal calls: bf16 max-abs
2e-2 and mean-abs 2e-3, fp32 max-abs 1e-4.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()
    yield


def _check(gpu, ref, what, mx_tol=2e-2, mean_tol=2e-3):
    d = np.abs(np.asarray(gpu, np.float64) - ref)
    print(f"[{what}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= mx_tol and d.mean() <= mean_tol, what


@pytest.mark.parametrize("w0", [1, 64, 300, 5000])
def test_band_prefill_bf16(w0):
    lens = [700, 413, 1, 129]
    cu = wl.cu_seqlens(lens)
    Hq, Hkv = 8, 2
    q, k, v = wl.prefill_inputs(Hq, Hkv, cu[-1], 128, "bf16", 81)
    scale = 1 / math.sqrt(128)
    o, lse = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), cu, w0, 256, THETA, "band", scale,
                         return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), cu,
                                    w0, 256, THETA, "band", scale)
    _check(o.float().cpu().numpy(), o_ref, f"band prefill w0={w0}")
    _check(lse.cpu().numpy(), lse_ref, f"band lse w0={w0}", 2e-2, 2e-3)


@pytest.mark.parametrize("G", [1, 4, 16])
def test_band_prefill_gqa(G):
    lens = [333, 90]
    cu = wl.cu_seqlens(lens)
    q, k, v = wl.prefill_inputs(G, 1, cu[-1], 128, "bf16", 82)
    scale = 1 / math.sqrt(128)
    o = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), cu, 100, 64, THETA, "band", scale)
    torch.cuda.synchronize()
    o_ref, _ = oracle.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), cu, 100, 64,
                              THETA, "band", scale)
    _check(o.float().cpu().numpy(), o_ref, f"band prefill G={G}")


def test_band_prefill_fp32_full():
    c = wl.CONFIGS["tiny_fp32_s2"]
    L = c["lens"][0]
    q, k, v = wl.prefill_inputs(c["Hq"], c["Hkv"], L, 128, "fp32", c["seed"])
    scale = 1 / math.sqrt(128)
    o = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), [0, L], c["w0"], c["w_pre"], c["theta"], "band",
                    scale)
    torch.cuda.synchronize()
    o_ref, _ = oracle.prefill(q.numpy(), k.numpy(), v.numpy(), [0, L], c["w0"], c["w_pre"],
                              c["theta"], "band", scale)
    d = np.abs(o.cpu().numpy().astype(np.float64) - o_ref)
    print(f"[band fp32] max-abs {d.max():.3e}", flush=True)
    assert d.max() <= 1e-4


def test_band_prefill_128k_sampled():
    c = wl.CONFIGS["qwen3_8b_prefill_128k"]
    L = c["lens"][0]
    q, k, v = wl.prefill_inputs(c["Hq"], c["Hkv"], L, 128, "bf16", c["seed"])
    scale = 1 / math.sqrt(128)
    o = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), [0, L], c["w0"], c["w_pre"], c["theta"], "band",
                    scale)
    torch.cuda.synchronize()
    w0 = c["w0"]
    rows = wl.sample_rows(L, 24, [0, 1, w0 - 1, w0, w0 + 1, L - 2, L - 1], seed=83)
    o_ref, _ = oracle.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), [0, L], w0,
                              c["w_pre"], c["theta"], "band", scale, rows=rows)
    _check(o[:, torch.from_numpy(np.asarray(rows)).cuda()].float().cpu().numpy(), o_ref,
           "band prefill 128k")


@pytest.mark.parametrize("N,w0", [(1, 4096), (63, 16), (4097, 4096), (32769, 4096),
                                  (131073, 4096), (500, 5000)])
def test_band_decode(N, w0):
    Hq, Hkv = 32, 8
    cap = N + 7
    q, kc, vc = wl.decode_inputs(1, Hq, Hkv, cap, 128, "bf16", 84)
    scale = 1 / math.sqrt(128)
    o, lse = bfl.decode(q.cuda(), kc.cuda(), vc.cuda(), [N], w0, 32768, THETA, "band", scale,
                        return_lse=True)
    torch.cuda.synchronize()
    k0 = max(0, N - w0)  # only the window reaches the oracle
    o_ref, lse_ref = oracle.decode(q.float().numpy(), kc[:, :, :N].float().numpy(),
                                   vc[:, :, :N].float().numpy(), [N], w0, 32768, THETA, "band",
                                   scale)
    _check(o.float().cpu().numpy(), o_ref, f"band decode N={N} w0={w0} (keys {k0}..{N - 1})")
    _check(lse.cpu().numpy(), lse_ref, f"band decode lse N={N}")


def test_band_decode_mixed_batch():
    lens = [70, 1000, 2500]
    w0 = 256
    Hq, Hkv = 8, 2
    cap = max(lens)
    rng = torch.Generator().manual_seed(85)
    kc = torch.randn(3, Hkv, cap, 128, generator=rng).to(torch.bfloat16)
    vc = torch.randn(3, Hkv, cap, 128, generator=rng).to(torch.bfloat16)
    q = torch.randn(3, Hq, 128, generator=rng).to(torch.bfloat16)
    scale = 1 / math.sqrt(128)
    o = bfl.decode(q.cuda(), kc.cuda(), vc.cuda(), lens, w0, 4096, THETA, "band", scale)
    torch.cuda.synchronize()
    o_ref, _ = oracle.decode(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), lens, w0,
                             4096, THETA, "band", scale)
    _check(o.float().cpu().numpy(), o_ref, "band decode batch")
