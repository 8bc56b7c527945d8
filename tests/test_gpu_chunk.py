"""GPU parity of bifocal_prefill_chunk: multi-token queries against a KV cache
(the last Lq_b of N_b positions, bottom-right causal) against the fp64 oracle,
bf16 max-abs 2e-2 / mean-abs 2e-3 and fp32 max-abs 1e-4. Cache slots past N_b
hold NaN, so a read of them would show. Identities: a chunk that is the whole
sequence is bitwise the one-shot bifocal_prefill (same engine, same work
split); chunk by chunk with s_len = the prompt length reproduces the one-shot
prefill. bifocal_prefill_chunk_paged (shuffled page pools of 1 to 256 keys per
page, junk in unused table entries) must be bitwise the contiguous call.
Short chunks against long caches split each work item's key tiles into
parts merged by their log-sum-exp; those launches are checked against the
oracle too, and the trace confirms that they split.
Needs an MI355X.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()
    yield


def _check(gpu, ref, what, mx_tol=2e-2, mean_tol=2e-3):
    d = np.abs(np.asarray(gpu, np.float64) - ref)
    print(f"[{what}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= mx_tol and d.mean() <= mean_tol, what


def chunk_inputs(Ns, Lqs, Hq, Hkv, cap, dtype, seed):
    """Caches [B, Hkv, cap, D] with N_b valid keys (NaN past them) and the
    packed queries of the chunks [Hq, sum Lq, D]."""
    B = len(Ns)
    q, kc, vc = wl.prefill_inputs(Hq, Hkv, sum(Lqs), 128, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.randn(B, Hkv, cap, 128, generator=g).to(tdt)
    vc = torch.randn(B, Hkv, cap, 128, generator=g).to(tdt)
    for b, N in enumerate(Ns):
        kc[b, :, N:] = float("nan")
        vc[b, :, N:] = float("nan")
    return q, kc, vc


@pytest.mark.parametrize("mode", ["fi", "pa", "pa+shift", "fi+shift", "band"])
def test_chunk_matches_oracle(mode):
    Ns = [1000, 4097, 700, 2500, 129, 64]
    Lqs = [300, 1, 700, 37, 64, 33]
    Hq, Hkv, cap = 8, 2, 4200
    cu = wl.cu_seqlens(Lqs)
    q, kc, vc = chunk_inputs(Ns, Lqs, Hq, Hkv, cap, "bf16", 91)
    scale = 1 / math.sqrt(128)
    w0, w_pre = 256, 512
    o, lse = bfl.prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), cu, Ns, w0, w_pre, THETA, mode,
                               scale, return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.chunk(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), cu, Ns,
                                  w0, w_pre, THETA, mode, scale)
    _check(o.float().cpu().numpy(), o_ref, f"chunk {mode}")
    _check(lse.cpu().numpy(), lse_ref, f"chunk lse {mode}")


def test_chunk_fp32():
    Ns, Lqs = [900, 300], [200, 300]
    cu = wl.cu_seqlens(Lqs)
    q, kc, vc = chunk_inputs(Ns, Lqs, 4, 1, 1000, "fp32", 92)
    scale = 1 / math.sqrt(128)
    o = bfl.prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), cu, Ns, 100, 256, THETA, "fi", scale)
    torch.cuda.synchronize()
    o_ref, _ = oracle.chunk(q.numpy(), kc.numpy(), vc.numpy(), cu, Ns, 100, 256, THETA, "fi", scale)
    d = np.abs(o.cpu().numpy().astype(np.float64) - o_ref)
    print(f"[chunk fp32] max-abs {d.max():.3e}", flush=True)
    assert d.max() <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_whole_sequence_chunk_is_bitwise_prefill(dtype):
    # Lq = N: qpos = 0 and the work split of the one-shot prefill, keys read
    # from the cache layout instead of the packed one
    lens = [700, 413, 1, 129]
    cu = wl.cu_seqlens(lens)
    Hq, Hkv, cap = 8, 2, 720
    q, k, v = wl.prefill_inputs(Hq, Hkv, cu[-1], 128, dtype, 93)
    kc = torch.full((4, Hkv, cap, 128), float("nan"), dtype=k.dtype)
    vc = torch.full_like(kc, float("nan"))
    for b, L in enumerate(lens):
        kc[b, :, :L] = k[:, cu[b]:cu[b + 1]]
        vc[b, :, :L] = v[:, cu[b]:cu[b + 1]]
    scale = 1 / math.sqrt(128)
    for mode in ["fi", "pa+shift", "band"]:
        o_p, l_p = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), cu, 64, 256, THETA, mode, scale,
                               return_lse=True)
        o_c, l_c = bfl.prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), cu, lens, 64, 256, THETA, mode,
                                     scale, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p), (dtype, mode)


@pytest.mark.parametrize("mode", ["fi", "pa"])
def test_chunked_prefill_reproduces_one_shot(mode):
    # a 3000-token prompt in three uneven chunks, each appended to the cache
    # before its call, with s_len = 3000: every row is the one-shot row
    L, Hq, Hkv, w0, w_pre = 3000, 8, 2, 300, 700
    q, k, v = wl.prefill_inputs(Hq, Hkv, L, 128, "bf16", 94)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = 1 / math.sqrt(128)
    o_one = bfl.prefill(qd, kd, vd, [0, L], w0, w_pre, THETA, mode, scale)
    kc = torch.full((1, Hkv, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    outs = []
    t = 0
    for n in [777, 1500, 723]:
        kc[0, :, t:t + n] = kd[:, t:t + n]
        vc[0, :, t:t + n] = vd[:, t:t + n]
        outs.append(bfl.prefill_chunk(qd[:, t:t + n].contiguous(), kc, vc, [0, n], [t + n], w0,
                                      w_pre, THETA, mode, scale, s_len=[L]))
        t += n
    o_ch = torch.cat(outs, dim=1)
    torch.cuda.synchronize()
    o_ref, _ = oracle.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), [0, L], w0,
                              w_pre, THETA, mode, scale)
    _check(o_ch.float().cpu().numpy(), o_ref, f"chunked prefill {mode}")
    d = (o_ch.float() - o_one.float()).abs()
    print(f"[chunked vs one-shot {mode}] max-abs {d.max().item():.3e}", flush=True)
    assert d.max().item() <= 1.6e-2


def test_single_query_chunk_matches_decode():
    Ns = [1, 63, 4097, 20000]
    Hq, Hkv, cap = 32, 8, 20000
    q, kc, vc = chunk_inputs(Ns, [1] * 4, Hq, Hkv, cap, "bf16", 95)
    scale = 1 / math.sqrt(128)
    qc = q.cuda()
    o_c = bfl.prefill_chunk(qc, kc.cuda(), vc.cuda(), [0, 1, 2, 3, 4], Ns, 4096, 8192, THETA, "fi",
                            scale)
    o_d = bfl.decode(qc.transpose(0, 1).contiguous(), kc.cuda(), vc.cuda(), Ns, 4096, 8192, THETA,
                     "fi", scale)
    torch.cuda.synchronize()
    o_ref, _ = oracle.decode(q.transpose(0, 1).float().numpy(), kc.float().numpy(),
                             vc.float().numpy(), Ns, 4096, 8192, THETA, "fi", scale)
    _check(o_c.transpose(0, 1).float().cpu().numpy(), o_ref, "single-query chunk")
    _check(o_d.float().cpu().numpy(), o_ref, "decode")


@pytest.mark.parametrize("mode", ["fi", "pa"])
def test_chunk_4k_at_128k_sampled(mode):
    # the last 4096 queries of a 131072-token sequence (Qwen3-8B shape, s = 4)
    c = wl.CONFIGS["qwen3_8b_prefill_128k"]
    N, Lq = c["lens"][0], 4096
    Hq, Hkv = c["Hq"], c["Hkv"]
    q, kc, vc = chunk_inputs([N], [Lq], Hq, Hkv, N, "bf16", 96)
    scale = 1 / math.sqrt(128)
    o = bfl.prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), [0, Lq], [N], c["w0"], c["w_pre"],
                          c["theta"], mode, scale)
    torch.cuda.synchronize()
    rows = wl.sample_rows(Lq, 20, [0, 1, 31, 32, 4094, 4095], seed=97)
    qs, kf, vf = q[:, rows].float().numpy(), kc.float().numpy(), vc.float().numpy()
    o_ref, _ = oracle.chunk(qs, kf, vf, [0, Lq], [N], c["w0"], c["w_pre"], c["theta"], mode, scale,
                            rows=rows, gathered=True)
    og = o[:, torch.from_numpy(np.asarray(rows)).cuda()].float().cpu().numpy()
    _check(og, o_ref, f"chunk 4k at 128k {mode}")
    # discrimination, as for the one-shot 128K prefill: every sampled row has
    # far pairs; the error must be small next to the gap to plain attention
    # (no correction) and to the other long mode
    err = np.linalg.norm(og - o_ref)
    plain, _ = oracle.chunk(qs, kf, vf, [0, Lq], [N], 10**9, c["w_pre"], c["theta"], mode, scale,
                            rows=rows, gathered=True)
    other, _ = oracle.chunk(qs, kf, vf, [0, Lq], [N], c["w0"], c["w_pre"], c["theta"],
                            "pa" if mode == "fi" else "fi", scale, rows=rows, gathered=True)
    gap_plain, gap_mode = np.linalg.norm(o_ref - plain), np.linalg.norm(o_ref - other)
    print(f"[chunk 128k discrimination {mode}] err {err:.3e} gap-plain {gap_plain:.3e} "
          f"gap-other-mode {gap_mode:.3e}", flush=True)
    assert err <= 0.05 * gap_plain
    assert err <= 0.25 * gap_mode


def test_chunk_is_deterministic():
    Ns, Lqs = [5000, 3000], [1000, 2048]
    cu = wl.cu_seqlens(Lqs)
    q, kc, vc = chunk_inputs(Ns, Lqs, 16, 4, 5000, "bf16", 98)
    args = (q.cuda(), kc.cuda(), vc.cuda(), cu, Ns, 512, 1024, THETA, "pa", 0.088)
    a = bfl.prefill_chunk(*args)
    b = bfl.prefill_chunk(*args)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def paginate(kc, vc, seqlens, page, seed, spare=3):
    """Scatter caches [B, Hkv, cap, D] (on the GPU) into a shuffled page pool
    [pages, Hkv, page, D]; unused block-table entries hold junk."""
    B, Hkv, cap, D = kc.shape
    need = [math.ceil(n / page) for n in seqlens]
    total = sum(need) + spare
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(total)).to(kc.device)
    kp = torch.zeros((total, Hkv, page, D), dtype=kc.dtype, device=kc.device)
    vp = torch.zeros_like(kp)
    table = torch.full((B, max(need) + 2), -5, dtype=torch.int32, device=kc.device)
    nxt = 0
    for b in range(B):
        n, pgs = seqlens[b], need[b]
        phys = perm[nxt:nxt + pgs]
        nxt += pgs
        table[b, :pgs] = phys.to(torch.int32)
        for src, dst in ((kc, kp), (vc, vp)):
            x = torch.zeros((Hkv, pgs * page, D), dtype=kc.dtype, device=kc.device)
            x[:, :n] = src[b, :, :n]
            dst[phys] = x.view(Hkv, pgs, page, D).permute(1, 0, 2, 3)
    return kp, vp, table


@pytest.mark.parametrize("page", [1, 16, 64, 256])
@pytest.mark.parametrize("mode", ["fi", "pa+shift", "band"])
def test_paged_chunk_equals_contiguous(page, mode):
    Ns = [1000, 4097, 700, 2500, 129, 64]
    Lqs = [300, 1, 700, 37, 64, 33]
    cu = wl.cu_seqlens(Lqs)
    q, kc, vc = chunk_inputs(Ns, Lqs, 8, 2, 4200, "bf16", 99)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    scale = 1 / math.sqrt(128)
    o_c, l_c = bfl.prefill_chunk(q, kc, vc, cu, Ns, 256, 512, THETA, mode, scale, return_lse=True)
    kp, vp, table = paginate(kc, vc, Ns, page, seed=page)
    del kc, vc
    o_p, l_p = bfl.prefill_chunk_paged(q, kp, vp, table, cu, Ns, 256, 512, THETA, mode, scale,
                                       return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c), (page, mode)


def test_paged_chunk_fp32_and_s_len():
    Ns, Lqs = [900, 300], [200, 300]
    cu = wl.cu_seqlens(Lqs)
    q, kc, vc = chunk_inputs(Ns, Lqs, 4, 1, 1000, "fp32", 100)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    scale = 1 / math.sqrt(128)
    o_c = bfl.prefill_chunk(q, kc, vc, cu, Ns, 100, 256, THETA, "pa", scale, s_len=[3000, 300])
    kp, vp, table = paginate(kc, vc, Ns, 32, seed=5)
    o_p = bfl.prefill_chunk_paged(q, kp, vp, table, cu, Ns, 100, 256, THETA, "pa", scale,
                                  s_len=[3000, 300])
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c)
    o_ref, _ = oracle.chunk(q.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy(), cu, Ns, 100, 256,
                            THETA, "pa", scale, s_len=[3000, 300])
    d = np.abs(o_p.cpu().numpy().astype(np.float64) - o_ref)
    print(f"[paged chunk fp32] max-abs {d.max():.3e}", flush=True)
    assert d.max() <= 1e-4


def test_paged_chunk_4k_at_128k():
    c = wl.CONFIGS["qwen3_8b_prefill_128k"]
    N, Lq = c["lens"][0], 4096
    q, kc, vc = chunk_inputs([N], [Lq], c["Hq"], c["Hkv"], N, "bf16", 101)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    scale = 1 / math.sqrt(128)
    o_c = bfl.prefill_chunk(q, kc, vc, [0, Lq], [N], c["w0"], c["w_pre"], c["theta"], "fi", scale)
    kp, vp, table = paginate(kc, vc, [N], 16, seed=6)
    del kc, vc
    o_p = bfl.prefill_chunk_paged(q, kp, vp, table, [0, Lq], [N], c["w0"], c["w_pre"], c["theta"],
                                  "fi", scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c)


def _key_splits(capfd):
    return [int(x) for x in re.findall(r"key_splits=(\d+)", capfd.readouterr().err)]


@pytest.mark.parametrize("mode", ["fi", "pa", "pa+shift", "fi+shift", "band"])
def test_short_chunks_split_keys_match_oracle(mode, capfd, monkeypatch):
    # three short chunks against caches of 9K-20K keys: 16 work items, so the
    # launch splits each item's key tiles and merges the parts
    monkeypatch.setenv("BIFOCAL_TRACE", "1")
    Ns, Lqs = [20000, 9000, 12345], [64, 33, 100]
    Hq, Hkv, cap = 8, 2, 20000
    w0, w_pre = (6000 if mode == "band" else 1024), 4096  # s = 5, 3, 4
    cu = wl.cu_seqlens(Lqs)
    q, kc, vc = chunk_inputs(Ns, Lqs, Hq, Hkv, cap, "bf16", 111)
    scale = 1 / math.sqrt(128)
    o, lse = bfl.prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), cu, Ns, w0, w_pre, THETA, mode,
                               scale, return_lse=True)
    torch.cuda.synchronize()
    ks = _key_splits(capfd)
    print(f"[split chunk {mode}] key splits {ks}", flush=True)
    assert ks and max(ks) > 1
    qf, kf, vf = q.float().numpy(), kc.float().numpy(), vc.float().numpy()
    o_ref, lse_ref = oracle.chunk(qf, kf, vf, cu, Ns, w0, w_pre, THETA, mode, scale)
    og = o.float().cpu().numpy()
    _check(og, o_ref, f"split chunk {mode}")
    _check(lse.cpu().numpy(), lse_ref, f"split chunk lse {mode}")
    # the merge must not hide a wrong branch: the error is small next to the
    # gap to plain causal attention over the same keys
    plain, _ = oracle.chunk(qf, kf, vf, cu, Ns, 10**9, w_pre, THETA, "fi", scale)
    err, gap = np.linalg.norm(og - o_ref), np.linalg.norm(o_ref - plain)
    print(f"[split chunk {mode} discrimination] err {err:.3e} gap-plain {gap:.3e}", flush=True)
    assert err <= 0.05 * gap


def test_split_chunk_is_deterministic_and_paged_equal(capfd, monkeypatch):
    monkeypatch.setenv("BIFOCAL_TRACE", "1")
    Ns, Lqs = [30000, 17000], [128, 40]
    Hq, Hkv, cap = 16, 4, 30000
    cu = wl.cu_seqlens(Lqs)
    q, kc, vc = chunk_inputs(Ns, Lqs, Hq, Hkv, cap, "bf16", 112)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    args = (cu, Ns, 2048, 8192, THETA, "pa+shift", 0.088)
    a, la = bfl.prefill_chunk(q, kc, vc, *args, return_lse=True)
    b, lb = bfl.prefill_chunk(q, kc, vc, *args, return_lse=True)
    kp, vp, table = paginate(kc, vc, Ns, 16, seed=113)
    c, lc = bfl.prefill_chunk_paged(q, kp, vp, table, *args, return_lse=True)
    torch.cuda.synchronize()
    ks = _key_splits(capfd)
    assert ks and min(ks) > 1, ks
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert torch.equal(c, a) and torch.equal(lc, la)


@pytest.mark.parametrize("mode", ["fi", "pa"])
def test_chunk_512_at_128k_split_sampled(mode, capfd, monkeypatch):
    # the last 512 queries of a 131072-token sequence (Qwen3-8B shape, s = 4):
    # 128 work items, split four ways
    monkeypatch.setenv("BIFOCAL_TRACE", "1")
    c = wl.CONFIGS["qwen3_8b_prefill_128k"]
    N, Lq = c["lens"][0], 512
    Hq, Hkv = c["Hq"], c["Hkv"]
    q, kc, vc = chunk_inputs([N], [Lq], Hq, Hkv, N, "bf16", 114)
    scale = 1 / math.sqrt(128)
    o = bfl.prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), [0, Lq], [N], c["w0"], c["w_pre"],
                          c["theta"], mode, scale)
    torch.cuda.synchronize()
    ks = _key_splits(capfd)
    print(f"[chunk 512 at 128k {mode}] key splits {ks}", flush=True)
    assert ks and max(ks) > 1
    rows = wl.sample_rows(Lq, 16, [0, 1, 31, 32, 510, 511], seed=115)
    qs, kf, vf = q[:, rows].float().numpy(), kc.float().numpy(), vc.float().numpy()
    o_ref, _ = oracle.chunk(qs, kf, vf, [0, Lq], [N], c["w0"], c["w_pre"], c["theta"], mode, scale,
                            rows=rows, gathered=True)
    og = o[:, torch.from_numpy(np.asarray(rows)).cuda()].float().cpu().numpy()
    _check(og, o_ref, f"chunk 512 at 128k {mode}")
    err = np.linalg.norm(og - o_ref)
    plain, _ = oracle.chunk(qs, kf, vf, [0, Lq], [N], 10**9, c["w_pre"], c["theta"], mode, scale,
                            rows=rows, gathered=True)
    other, _ = oracle.chunk(qs, kf, vf, [0, Lq], [N], c["w0"], c["w_pre"], c["theta"],
                            "pa" if mode == "fi" else "fi", scale, rows=rows, gathered=True)
    gap_plain, gap_mode = np.linalg.norm(o_ref - plain), np.linalg.norm(o_ref - other)
    print(f"[chunk 512 discrimination {mode}] err {err:.3e} gap-plain {gap_plain:.3e} "
          f"gap-other-mode {gap_mode:.3e}", flush=True)
    assert err <= 0.05 * gap_plain
    assert err <= 0.25 * gap_mode


def test_chunk_workspace_without_partials_runs_unsplit(capfd, monkeypatch):
    # the partials take 516 bytes per (split, query head, query token) at the
    # end of the workspace; a workspace short of all 8 splits' partials holds
    # the base layout but no split, so the call must run unsplit
    monkeypatch.setenv("BIFOCAL_TRACE", "1")
    Ns, Lqs = [20000, 9000, 12345], [64, 33, 100]
    Hq, Hkv, cap = 8, 2, 20000
    cu = wl.cu_seqlens(Lqs)
    q, kc, vc = chunk_inputs(Ns, Lqs, Hq, Hkv, cap, "bf16", 116)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    scale = 1 / math.sqrt(128)
    full = bfl.chunk_workspace_bytes(len(Ns), cu[-1], sum(Ns), Hq, Hkv)
    small = full - 8 * Hq * cu[-1] * 516
    outs = []
    for nbytes in (full, small):
        ws = bfl.alloc_workspace(nbytes, "cuda")
        outs.append(bfl.prefill_chunk(q, kc, vc, cu, Ns, 1024, 4096, THETA, "fi", scale,
                                      workspace=ws))
    torch.cuda.synchronize()
    ks = _key_splits(capfd)
    print(f"[chunk workspace] key splits with the full / the small workspace: {ks}", flush=True)
    assert len(ks) == 2 and ks[0] > 1 and ks[1] == 1
    o_ref, _ = oracle.chunk(q.float().cpu().numpy(), kc.float().cpu().numpy(),
                            vc.float().cpu().numpy(), cu, Ns, 1024, 4096, THETA, "fi", scale)
    for o, what in zip(outs, ("split", "unsplit")):
        _check(o.float().cpu().numpy(), o_ref, f"chunk workspace {what}")
