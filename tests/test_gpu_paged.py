"""GPU tests of bifocal_decode_paged: decode over a paged KV cache (pages
[num_pages, Hkv, page_size, D], a device block table per sequence). The keys
are the same as in a contiguous cache, read in the same order, so the result
must be bitwise equal to bifocal_decode on the contiguous cache; it is also
compared with the fp64 oracle at the decode tolerance (bf16 max-abs 2e-2,
mean-abs 2e-3). Needs an MI355X.
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


def paginate(kc, vc, seqlens, page, seed, spare=3):
    """Scatter contiguous caches [B, Hkv, cap, D] into shuffled pages."""
    B, Hkv, cap, D = kc.shape
    need = [math.ceil(n / page) for n in seqlens]
    max_pages = max(need)
    total = sum(need) + spare
    perm = np.random.default_rng(seed).permutation(total)
    kp = torch.zeros((total, Hkv, page, D), dtype=kc.dtype, device=kc.device)
    vp = torch.zeros_like(kp)
    table = np.full((B, max_pages), -7, dtype=np.int32)  # unused entries hold junk
    nxt = 0
    for b in range(B):
        for p in range(need[b]):
            phys = int(perm[nxt])
            nxt += 1
            table[b, p] = phys
            lo, hi = p * page, min((p + 1) * page, cap)
            kp[phys, :, :hi - lo] = kc[b, :, lo:hi]
            vp[phys, :, :hi - lo] = vc[b, :, lo:hi]
    return kp, vp, torch.from_numpy(table).cuda()


@pytest.mark.parametrize("page", [16, 64, 256])
@pytest.mark.parametrize("mode", ["fi", "pa", "pa+shift", "band"])
def test_paged_equals_contiguous(page, mode):
    seqlens = [1, 15, 16, 17, 1000, 4097, 9001]
    B, Hq, Hkv = len(seqlens), 8, 2
    cap = max(seqlens) + 5
    q, kc, vc = wl.decode_inputs(B, Hq, Hkv, cap, 128, "bf16", 101)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    scale = 1 / math.sqrt(128)
    w0, w_pre = 256, 2048
    o_c, l_c = bfl.decode(q, kc, vc, seqlens, w0, w_pre, 1e6, mode, scale, return_lse=True)
    kp, vp, table = paginate(kc, vc, seqlens, page, seed=page)
    o_p, l_p = bfl.decode_paged(q, kp, vp, table, seqlens, w0, w_pre, 1e6, mode, scale,
                                return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c), (page, mode)
    o_ref, _ = oracle.decode(q.float().cpu().numpy(), kc.float().cpu().numpy(),
                             vc.float().cpu().numpy(), seqlens, w0, w_pre, 1e6, mode, scale)
    d = np.abs(o_p.float().cpu().numpy() - o_ref)
    print(f"[paged page={page} {mode}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3


@pytest.mark.parametrize("page", [16, 128])
def test_paged_128k(page):
    N, Hq, Hkv = 131073, 32, 8
    q, kc, vc = wl.decode_inputs(1, Hq, Hkv, N, 128, "bf16", 102)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    scale = 1 / math.sqrt(128)
    o_c = bfl.decode(q, kc, vc, [N], 4096, 32768, 1e6, "fi", scale)
    kp, vp, table = paginate(kc, vc, [N], page, seed=7)
    del kc, vc
    o_p = bfl.decode_paged(q, kp, vp, table, [N], 4096, 32768, 1e6, "fi", scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c)


def test_paged_validation():
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    for kw in [dict(seqlens=[65]), dict(seqlens=[0])]:  # more keys than 4 pages of 16 / none
        with pytest.raises(bfl.BifocalError):
            bfl.decode_paged(q, kp, kp, table, kw["seqlens"], 16, 64, 1e4, "fi", 0.1)
    kp24 = torch.zeros((4, 2, 24, 128), dtype=torch.bfloat16, device="cuda")  # not a power of two
    with pytest.raises(bfl.BifocalError):
        bfl.decode_paged(q, kp24, kp24, table, [10], 16, 64, 1e4, "fi", 0.1)


def test_paged_longest_wave_span():
    # 64 sequences x 8 KV heads of 16128 keys make the split rule choose
    # 4032-key chunks: each split's keys span 252 pages of 16, close to the
    # 256 page numbers a wave holds (four registers of 64 lanes)
    B, Hq, Hkv, N, page = 64, 8, 8, 16128, 16
    q, kc, vc = wl.decode_inputs(B, Hq, Hkv, N, 128, "bf16", 103)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    o_c = bfl.decode(q, kc, vc, [N] * B, 4096, 8192, 1e6, "pa", 0.088)
    per = N // page
    perm = torch.randperm(B * per, generator=torch.Generator().manual_seed(104)).cuda()
    kp = torch.empty((B * per, Hkv, page, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    kp[perm] = kc.view(B, Hkv, per, page, 128).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page, 128)
    vp[perm] = vc.view(B, Hkv, per, page, 128).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page, 128)
    del kc, vc
    o_p = bfl.decode_paged(q, kp, vp, perm.to(torch.int32).view(B, per), [N] * B, 4096, 8192, 1e6,
                           "pa", 0.088)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c)
