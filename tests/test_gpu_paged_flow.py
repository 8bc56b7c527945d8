"""GPU tests of the paged raw-input pre-steps (bifocal_rope_prefill_paged,
bifocal_rope_append_paged) and of a whole serving flow on a paged cache: raw
prompt -> pre-step into pages -> chunked prefill over the pages -> raw decode
token appended into the pages -> paged decode. The paged calls write and read
the same values as the contiguous ones, so every output must be bitwise the
contiguous flow's; the decode is also checked against the fp64 oracle on its
own rotation of the raw inputs (bf16 max-abs 2e-2, mean-abs 2e-3). Needs an
MI355X.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()
    yield


def page_pool(B, Hkv, max_len, page, seed, spare=3):
    """An empty shuffled pool for B sequences of up to max_len keys and its
    block table (junk in the spare entries)."""
    per = math.ceil(max_len / page)
    total = B * per + spare
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(total)[:B * per].astype(np.int32))
    table = torch.full((B, per + 2), -9, dtype=torch.int32)
    table[:, :per] = perm.view(B, per)
    kp = torch.zeros((total, Hkv, page, 128), dtype=torch.bfloat16, device="cuda")
    return kp, torch.zeros_like(kp), table.cuda()


def unpage(pages, table, B, n):
    """Pages -> contiguous [B, Hkv, n, D] through the block table."""
    page = pages.shape[2]
    per = math.ceil(n / page)
    out = pages[table[:, :per].long()]            # [B, per, Hkv, page, D]
    return out.permute(0, 2, 1, 3, 4).reshape(B, pages.shape[1], per * page, 128)[:, :, :n]


@pytest.mark.parametrize("page", [1, 16, 128])
def test_rope_prefill_paged_equals_contiguous(page):
    lens, pos0 = [300, 1, 129], [0, 77, 1000]
    cu = wl.cu_seqlens(lens)
    q, k, v = (x.cuda() for x in wl.prefill_inputs(4, 2, cu[-1], 128, "bf16", 401))
    cap = 1129
    kc = torch.zeros((3, 2, cap, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    qo_c, ko_c = bfl.rope_prefill(q, k, cu, THETA, v=v, k_cache=kc, v_cache=vc, pos0=pos0)
    kp, vp, table = page_pool(3, 2, cap, page, seed=page)
    qo_p, ko_p = bfl.rope_prefill_paged(q, k, v, cu, THETA, kp, vp, table, write_k=True, pos0=pos0)
    torch.cuda.synchronize()
    assert torch.equal(qo_p, qo_c) and torch.equal(ko_p, ko_c)
    assert torch.equal(unpage(kp, table, 3, cap), kc) and torch.equal(unpage(vp, table, 3, cap), vc)


@pytest.mark.parametrize("page", [1, 16, 256])
def test_rope_append_paged_equals_contiguous(page):
    seqlens = [1, 4097, 300, 131073]
    cap = 131073
    g = torch.Generator().manual_seed(402)
    qr = torch.randn(4, 8, 128, generator=g).to(torch.bfloat16).cuda()
    kr = torch.randn(4, 2, 128, generator=g).to(torch.bfloat16).cuda()
    vr = torch.randn(4, 2, 128, generator=g).to(torch.bfloat16).cuda()
    kc = torch.zeros((4, 2, cap, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q_c = bfl.rope_append(qr, kr, vr, kc, vc, seqlens, THETA)
    kp, vp, table = page_pool(4, 2, cap, page, seed=page + 1)
    q_p = bfl.rope_append_paged(qr, kr, vr, kp, vp, table, seqlens, THETA)
    torch.cuda.synchronize()
    assert torch.equal(q_p, q_c)
    for b, n in enumerate(seqlens):
        pg = table[b, (n - 1) // page].item()
        assert torch.equal(kp[pg, :, (n - 1) % page], kc[b, :, n - 1]), b
        assert torch.equal(vp[pg, :, (n - 1) % page], vc[b, :, n - 1]), b
    assert int(torch.count_nonzero(kp)) == int(torch.count_nonzero(kc))  # nothing else written


@pytest.mark.parametrize("mode", ["fi", "pa+shift"])
def test_paged_serving_flow_equals_contiguous(mode):
    lens = [2500, 700]
    B, Hq, Hkv, w0, w_pre, page = 2, 8, 2, 256, 1024, 16
    cu = wl.cu_seqlens(lens)
    q, k, v = (x.cuda() for x in wl.prefill_inputs(Hq, Hkv, cu[-1], 128, "bf16", 403))
    g = torch.Generator().manual_seed(404)
    qt = torch.randn(B, Hq, 128, generator=g).to(torch.bfloat16).cuda()
    kt = torch.randn(B, Hkv, 128, generator=g).to(torch.bfloat16).cuda()
    vt = torch.randn(B, Hkv, 128, generator=g).to(torch.bfloat16).cuda()
    N = [n + 1 for n in lens]
    cap = max(N)
    # contiguous flow
    kc = torch.zeros((B, Hkv, cap, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q1, _ = bfl.rope_prefill(q, k, cu, THETA, v=v, k_cache=kc, v_cache=vc, write_k=False)
    o_pre_c = bfl.prefill_chunk(q1, kc, vc, cu, lens, w0, w_pre, THETA, mode, SCALE)
    qd = bfl.rope_append(qt, kt, vt, kc, vc, N, THETA)
    o_dec_c = bfl.decode(qd, kc, vc, N, w0, w_pre, THETA, mode, SCALE)
    # paged flow
    kp, vp, table = page_pool(B, Hkv, cap, page, seed=405)
    q1p, _ = bfl.rope_prefill_paged(q, k, v, cu, THETA, kp, vp, table)
    o_pre_p = bfl.prefill_chunk_paged(q1p, kp, vp, table, cu, lens, w0, w_pre, THETA, mode, SCALE)
    qdp = bfl.rope_append_paged(qt, kt, vt, kp, vp, table, N, THETA)
    o_dec_p = bfl.decode_paged(qdp, kp, vp, table, N, w0, w_pre, THETA, mode, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o_pre_p, o_pre_c) and torch.equal(o_dec_p, o_dec_c), mode
    # the decode step against the oracle on its own rotation of the raw inputs
    rq = oracle.rope_rows(qt.float().cpu().numpy()[:, :, None, :].transpose(1, 0, 2, 3).reshape(Hq, B, 128),
                          [n - 1 for n in N], THETA)  # [Hq, B, D]: token b at position N_b - 1
    kref = kc.float().cpu().numpy()
    vref = vc.float().cpu().numpy()
    o_ref, _ = oracle.decode(np.ascontiguousarray(rq.transpose(1, 0, 2)).astype(np.float32), kref,
                             vref, N, w0, w_pre, THETA, mode, SCALE)
    d = np.abs(o_dec_p.float().cpu().numpy() - o_ref)
    print(f"[paged flow {mode}] decode max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
