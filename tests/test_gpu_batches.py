"""GPU parity for batches of more than 64 sequences, which the library runs
as several launches of at most 64 sequences each (every launch gets its own
sequence table and offsets into the packed tensors, caches and workspace).
Each entry point is compared with the fp64 oracle at the usual bar (bf16
max-abs 2e-2, mean-abs 2e-3) over the whole batch. Needs an MI355X.
"""
import math
import re

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


def _check(gpu, ref, what):
    d = np.abs(np.asarray(gpu, np.float64) - ref)
    print(f"[{what}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, what


def _lens(n, lo, hi, seed):
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi, size=n)]


@pytest.mark.parametrize("mode", ["fi", "pa+shift", "band"])
def test_prefill_131_sequences(mode):
    lens = _lens(131, 1, 300, 201)
    cu = wl.cu_seqlens(lens)
    q, k, v = wl.prefill_inputs(4, 2, cu[-1], 128, "bf16", 202)
    o, lse = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), cu, 40, 64, THETA, mode, SCALE,
                         return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), cu,
                                    40, 64, THETA, mode, SCALE)
    _check(o.float().cpu().numpy(), o_ref, f"prefill 131 seqs {mode}")
    _check(lse.cpu().numpy(), lse_ref, f"prefill 131 seqs lse {mode}")


def test_chunk_100_sequences():
    Ns = _lens(100, 2, 400, 203)
    Lqs = [max(1, n // 3) for n in Ns]
    cu = wl.cu_seqlens(Lqs)
    cap = max(Ns) + 1
    q, _, _ = wl.prefill_inputs(4, 1, cu[-1], 128, "bf16", 204)
    _, kc, vc = wl.decode_inputs(len(Ns), 4, 1, cap, 128, "bf16", 205)
    o = bfl.prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), cu, Ns, 50, 64, THETA, "fi", SCALE)
    torch.cuda.synchronize()
    o_ref, _ = oracle.chunk(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), cu, Ns, 50,
                            64, THETA, "fi", SCALE)
    _check(o.float().cpu().numpy(), o_ref, "chunk 100 seqs")


def test_split_chunk_70_sequences(capfd, monkeypatch):
    # short chunks against 4K-8K-key caches: both launches (64 + 6 sequences)
    # split their keys, each merging its own token range
    monkeypatch.setenv("BIFOCAL_TRACE", "1")
    Ns = _lens(70, 4000, 8000, 217)
    Lqs = _lens(70, 1, 21, 218)
    cu = wl.cu_seqlens(Lqs)
    cap = max(Ns)
    q, _, _ = wl.prefill_inputs(4, 1, cu[-1], 128, "bf16", 219)
    _, kc, vc = wl.decode_inputs(len(Ns), 4, 1, cap, 128, "bf16", 220)
    o, lse = bfl.prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), cu, Ns, 512, 2048, THETA, "pa",
                               SCALE, return_lse=True)
    torch.cuda.synchronize()
    ks = [int(x) for x in re.findall(r"key_splits=(\d+)", capfd.readouterr().err)]
    print(f"[split chunk 70 seqs] key splits per launch {ks}", flush=True)
    assert len(ks) == 2 and min(ks) > 1
    o_ref, lse_ref = oracle.chunk(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), cu,
                                  Ns, 512, 2048, THETA, "pa", SCALE)
    _check(o.float().cpu().numpy(), o_ref, "split chunk 70 seqs")
    _check(lse.cpu().numpy(), lse_ref, "split chunk 70 seqs lse")


@pytest.mark.parametrize("mode", ["fi", "band"])
def test_decode_150_sequences(mode):
    Ns = _lens(150, 1, 3000, 206)
    q, kc, vc = wl.decode_inputs(len(Ns), 8, 2, max(Ns), 128, "bf16", 207)
    o, lse = bfl.decode(q.cuda(), kc.cuda(), vc.cuda(), Ns, 256, 512, THETA, mode, SCALE,
                        return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), Ns,
                                   256, 512, THETA, mode, SCALE)
    _check(o.float().cpu().numpy(), o_ref, f"decode 150 seqs {mode}")
    _check(lse.cpu().numpy(), lse_ref, f"decode 150 seqs lse {mode}")


def test_paged_decode_90_sequences():
    Ns = _lens(90, 1, 2000, 208)
    page = 32
    q, kc, vc = wl.decode_inputs(len(Ns), 8, 2, max(Ns), 128, "bf16", 209)
    need = [math.ceil(n / page) for n in Ns]
    perm = np.random.default_rng(210).permutation(sum(need))
    kp = torch.zeros((sum(need), 2, page, 128), dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    table = np.zeros((len(Ns), max(need)), dtype=np.int32)
    nxt = 0
    for b, n in enumerate(Ns):
        for pg in range(need[b]):
            phys = int(perm[nxt])
            nxt += 1
            table[b, pg] = phys
            lo, hi = pg * page, min((pg + 1) * page, n)
            kp[phys, :, :hi - lo] = kc[b, :, lo:hi]
            vp[phys, :, :hi - lo] = vc[b, :, lo:hi]
    o_p = bfl.decode_paged(q.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(table).cuda(), Ns, 256,
                           512, THETA, "pa", SCALE)
    o_c = bfl.decode(q.cuda(), kc.cuda(), vc.cuda(), Ns, 256, 512, THETA, "pa", SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c)
    o_ref, _ = oracle.decode(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), Ns, 256,
                             512, THETA, "pa", SCALE)
    _check(o_p.float().cpu().numpy(), o_ref, "paged decode 90 seqs")


def test_rope_prefill_and_append_100_sequences():
    lens = _lens(100, 1, 200, 211)
    cu = wl.cu_seqlens(lens)
    q, k, _ = wl.prefill_inputs(4, 2, cu[-1], 128, "bf16", 212)
    qo, ko = bfl.rope_prefill(q.cuda(), k.cuda(), cu, THETA)
    torch.cuda.synchronize()
    pos = oracle.packed_positions(cu)
    for got, raw in ((qo, q), (ko, k)):
        ref = oracle.rope_rows(raw.float().numpy(), pos, THETA)
        d = np.abs(got.float().cpu().numpy() - ref)
        print(f"[rope 100 seqs] max-abs {d.max():.3e}", flush=True)
        assert d.max() <= 2e-2
    # decode append for 100 sequences at their own positions
    Ns = _lens(100, 1, 500, 213)
    qr = torch.randn(100, 4, 128, generator=torch.Generator().manual_seed(214)).to(torch.bfloat16)
    kr = torch.randn(100, 2, 128, generator=torch.Generator().manual_seed(215)).to(torch.bfloat16)
    vr = torch.randn(100, 2, 128, generator=torch.Generator().manual_seed(216)).to(torch.bfloat16)
    kcache = torch.zeros((100, 2, 500, 128), dtype=torch.bfloat16, device="cuda")
    vcache = torch.zeros_like(kcache)
    qa = bfl.rope_append(qr.cuda(), kr.cuda(), vr.cuda(), kcache, vcache, Ns, THETA)
    torch.cuda.synchronize()
    for b in range(0, 100, 9):
        p = Ns[b] - 1
        rq = oracle.rope_rows(qr[b].float().numpy()[:, None, :], [p], THETA)[:, 0]
        rk = oracle.rope_rows(kr[b].float().numpy()[:, None, :], [p], THETA)[:, 0]
        assert np.abs(qa[b].float().cpu().numpy() - rq).max() <= 2e-2, b
        assert np.abs(kcache[b, :, p].float().cpu().numpy() - rk).max() <= 2e-2, b
        assert torch.equal(vcache[b, :, p].cpu(), vr[b]), b
