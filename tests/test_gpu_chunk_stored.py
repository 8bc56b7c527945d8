"""bifocal_prefill_chunk_stored on the GPU (needs an MI355X).

The chunk store keeps k''_j = R(theta_m (phi(j) - j)) k'_j and V^T of the
cache between calls [ai-feeds.com summary, "关键模块" item 3: the correction
rotation of cached keys; mufans.github.io wiki, Jet-Long Dynamic RoPE,
"可执行建议": prompt caching]. The stored values are the ones
bifocal_prefill_chunk forms for the whole cache on every call, so each call
must be bitwise the stateless chunk call (o and lse); that call is checked
against the fp64 oracle in test_gpu_chunk.py, and one stored call here is
checked against the oracle too. Stores start filled with NaN, so a read of
an entry the library has not written shows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from rope_context_extension_bifocal_amd import bifocal as bfl
from rope_context_extension_bifocal_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)
THETA = 1e6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()


def _caches(B, Hkv, cap, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    kc = torch.randn(B, Hkv, cap, 128, generator=g).to(dtype).cuda()
    vc = torch.randn(B, Hkv, cap, 128, generator=g).to(dtype).cuda()
    return kc, vc


def _queries(Hq, Lqs, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(Hq, sum(Lqs), 128, generator=g).to(dtype).cuda()


def _nan_store(kc):
    st = bfl.ChunkStore(kc)
    st.buf.fill_(255)  # all-ones bytes: NaN in bf16 and fp32
    return st


def _walk(kc, vc, store, chunks, Hq, w0, w_pre, mode, s_len, seed):
    """Calls over per-sequence chunk lists (one chunk per sequence and call),
    each stored call against the stateless one, o and lse bitwise."""
    B = len(chunks)
    ends = [0] * B
    for i in range(len(chunks[0])):
        Lqs = [c[i] for c in chunks]
        ends = [e + n for e, n in zip(ends, Lqs)]
        q = _queries(Hq, Lqs, kc.dtype, seed + i)
        cu = wl.cu_seqlens(Lqs)
        ref, lref = bfl.prefill_chunk(q, kc, vc, cu, ends, w0, w_pre, THETA, mode, SCALE,
                                      s_len=s_len, return_lse=True)
        got, lgot = bfl.prefill_chunk_stored(q, kc, vc, store, cu, ends, w0, w_pre, THETA, mode,
                                             SCALE, s_len=s_len, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(lgot, lref), (mode, i, ends)
        for b in range(B):
            assert store.keys[b] == ends[b]
            assert store.s[b] == bfl.s_of_L(s_len[b] if s_len else ends[b], w_pre)
    return ends


@pytest.mark.parametrize("mode", ["fi", "pa", "fi+shift", "pa+shift"])
def test_stored_chunks_equal_chunk(mode):
    # two prompts of 2900 and 2500 tokens in six chunks each, s fixed by
    # s_len (5 and 4); the first call has no far pair at all (N <= w0), so
    # only the store's prep sees those keys before later calls read them
    Hq, Hkv, w0, w_pre = 8, 2, 300, 700
    kc, vc = _caches(2, Hkv, 2944, torch.bfloat16, 120)
    store = _nan_store(kc)
    chunks = [[200, 197, 1000, 1, 700, 802], [100, 900, 64, 700, 36, 700]]
    _walk(kc, vc, store, chunks, Hq, w0, w_pre, mode, [2900, 2500], 121)


def test_stored_chunks_s_change_and_rollback():
    # no s_len: s = s(N) grows as the chunks pass multiples of w_pre, and each
    # change empties the store; then cache positions from 1700 on are
    # rewritten, the store is cut back to them, and the chunk is redone
    Hq, Hkv, w0, w_pre = 16, 4, 256, 512
    kc, vc = _caches(1, Hkv, 2400, torch.bfloat16, 122)
    store = _nan_store(kc)
    ends = _walk(kc, vc, store, [[300, 200, 13, 500, 511, 1, 300]], Hq, w0, w_pre, "fi", None, 123)
    assert ends == [1825]
    g = torch.Generator().manual_seed(124)
    kc[0, :, 1700:] = torch.randn(Hkv, 700, 128, generator=g).to(torch.bfloat16).cuda()
    vc[0, :, 1700:] = torch.randn(Hkv, 700, 128, generator=g).to(torch.bfloat16).cuda()
    store.reset(keys=1700)
    q = _queries(Hq, [200], torch.bfloat16, 125)
    ref = bfl.prefill_chunk(q, kc, vc, [0, 200], [1900], w0, w_pre, THETA, "fi", SCALE)
    got = bfl.prefill_chunk_stored(q, kc, vc, store, [0, 200], [1900], w0, w_pre, THETA, "fi",
                                   SCALE)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert store.keys[0] == 1900 and store.s[0] == 4


def test_stored_chunks_fp32():
    Hq, Hkv, w0, w_pre = 4, 1, 128, 256
    kc, vc = _caches(2, Hkv, 1100, torch.float32, 126)
    store = _nan_store(kc)
    _walk(kc, vc, store, [[300, 5, 400, 64], [64, 700, 1, 300]], Hq, w0, w_pre, "pa+shift",
          [1100, 1100], 127)


def test_stored_chunks_batch_of_70():
    # more sequences than one launch takes (64): two launch groups, each with
    # its part of the store; lengths and chunk sizes differ per sequence
    B, Hq, Hkv, w0, w_pre = 70, 8, 2, 128, 512
    kc, vc = _caches(B, Hkv, 1600, torch.bfloat16, 128)
    store = _nan_store(kc)
    chunks = [[40 + 3 * b, 200 + (7 * b) % 300, 1 + b % 5] for b in range(B)]
    _walk(kc, vc, store, chunks, Hq, w0, w_pre, "fi", [1600] * B, 129)


def test_stored_chunk_matches_oracle():
    # one stored call after the store was filled, against the fp64 oracle
    Hq, Hkv, w0, w_pre, N, Lq = 8, 2, 200, 600, 1900, 150
    kc, vc = _caches(1, Hkv, N, torch.bfloat16, 130)
    store = _nan_store(kc)
    q0 = _queries(Hq, [400], torch.bfloat16, 131)
    bfl.prefill_chunk_stored(q0, kc, vc, store, [0, 400], [N - Lq], w0, w_pre, THETA, "pa", SCALE,
                             s_len=[N])
    q = _queries(Hq, [Lq], torch.bfloat16, 132)
    o, lse = bfl.prefill_chunk_stored(q, kc, vc, store, [0, Lq], [N], w0, w_pre, THETA, "pa",
                                      SCALE, s_len=[N], return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.chunk(q.float().cpu().numpy(), kc.float().cpu().numpy(),
                                  vc.float().cpu().numpy(), [0, Lq], [N], w0, w_pre, THETA, "pa",
                                  SCALE, s_len=[N])
    d = np.abs(o.float().cpu().numpy() - o_ref)
    dl = np.abs(lse.cpu().numpy() - lse_ref)
    print(f"[stored chunk vs oracle] max-abs {d.max():.3e} mean-abs {d.mean():.3e} "
          f"lse max-abs {dl.max():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3 and dl.max() <= 2e-2


def test_stored_chunk_512_at_128k():
    # the chunk leg of the bench: the last 512 queries of a 131072-key cache
    # (Qwen3-8B shape, s = 4), after a call that filled the store up to 130560
    c = wl.CONFIGS["qwen3_8b_prefill_128k"]
    N, Lq, Hq, Hkv = c["lens"][0], 512, c["Hq"], c["Hkv"]
    kc, vc = _caches(1, Hkv, N, torch.bfloat16, 133)
    store = _nan_store(kc)
    args = (c["w0"], c["w_pre"], c["theta"], "fi", SCALE)
    q0 = _queries(Hq, [Lq], torch.bfloat16, 134)
    bfl.prefill_chunk_stored(q0, kc, vc, store, [0, Lq], [N - Lq], *args, s_len=[N])
    q = _queries(Hq, [Lq], torch.bfloat16, 135)
    ref, lref = bfl.prefill_chunk(q, kc, vc, [0, Lq], [N], *args, s_len=[N], return_lse=True)
    got, lgot = bfl.prefill_chunk_stored(q, kc, vc, store, [0, Lq], [N], *args, s_len=[N],
                                         return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(got, ref) and torch.equal(lgot, lref)
    assert store.keys[0] == N and store.s[0] == 4


def _paginate(kc, vc, page, seed, spare=3):
    """Shuffled page pool [B * per + spare, Hkv, page, D] of the caches (the
    spare pages hold NaN) and its block table [B, per]."""
    B, Hkv, cap, D = kc.shape
    per = cap // page
    n = B * per + spare
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(seed))[:B * per].cuda()
    kp = torch.full((n, Hkv, page, D), float("nan"), dtype=kc.dtype, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    kp[perm] = kc.view(B, Hkv, per, page, D).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page, D)
    vp[perm] = vc.view(B, Hkv, per, page, D).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page, D)
    return kp, vp, perm.to(torch.int32).view(B, per)


@pytest.mark.parametrize("page", [1, 16, 64, 256])
def test_stored_paged_chunks_equal_paged_chunk(page):
    # the two-prompt walk over a shuffled page pool: every call bitwise the
    # stateless paged call and the contiguous stored call on the same keys
    Hq, Hkv, w0, w_pre = 8, 2, 300, 700
    kc, vc = _caches(2, Hkv, 3072, torch.bfloat16, 140)
    kp, vp, table = _paginate(kc, vc, page, 141)
    sp = bfl.ChunkStore(kp, batch=2, max_pages_per_seq=table.shape[1])
    sc = bfl.ChunkStore(kc)
    sp.buf.fill_(255)
    sc.buf.fill_(255)
    chunks = [[200, 197, 1000, 1, 700, 802], [100, 900, 64, 700, 36, 700]]
    ends = [0, 0]
    args = (w0, w_pre, THETA, "pa+shift", SCALE)
    for i in range(len(chunks[0])):
        Lqs = [c[i] for c in chunks]
        ends = [e + n for e, n in zip(ends, Lqs)]
        q = _queries(Hq, Lqs, torch.bfloat16, 142 + i)
        cu = wl.cu_seqlens(Lqs)
        ref, lref = bfl.prefill_chunk_paged(q, kp, vp, table, cu, ends, *args, s_len=[2900, 2500],
                                            return_lse=True)
        got, lgot = bfl.prefill_chunk_stored_paged(q, kp, vp, table, sp, cu, ends, *args,
                                                   s_len=[2900, 2500], return_lse=True)
        gc, lgc = bfl.prefill_chunk_stored(q, kc, vc, sc, cu, ends, *args, s_len=[2900, 2500],
                                           return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(lgot, lref), (page, i)
        assert torch.equal(gc, ref) and torch.equal(lgc, lref), (page, i)
        assert list(sp.keys) == ends and list(sp.s) == list(sc.s)


def test_stored_paged_chunk_s_change_and_rollback():
    # s = s(N) changes as the prompt grows (each change empties the store and
    # the call rotates and gathers from key 0), then a rollback over rewritten
    # pages; 16-key pages
    Hq, Hkv, w0, w_pre = 16, 4, 256, 512
    kc, vc = _caches(1, Hkv, 2400, torch.bfloat16, 143)
    kp, vp, table = _paginate(kc, vc, 16, 144)
    st = bfl.ChunkStore(kp, batch=1, max_pages_per_seq=table.shape[1])
    st.buf.fill_(255)
    n = 0
    for i, lq in enumerate([300, 200, 13, 500, 511, 1, 300]):
        n += lq
        q = _queries(Hq, [lq], torch.bfloat16, 145 + i)
        ref = bfl.prefill_chunk_paged(q, kp, vp, table, [0, lq], [n], w0, w_pre, THETA, "fi", SCALE)
        got = bfl.prefill_chunk_stored_paged(q, kp, vp, table, st, [0, lq], [n], w0, w_pre, THETA,
                                             "fi", SCALE)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), n
        assert st.keys[0] == n and st.s[0] == bfl.s_of_L(n, w_pre)
    # rewrite the pages from position 1696 on, cut the store back, redo
    g = torch.Generator().manual_seed(146)
    pages = table[0, 1696 // 16:].long()
    kp[pages] = torch.randn(len(pages), Hkv, 16, 128, generator=g).to(torch.bfloat16).cuda()
    vp[pages] = torch.randn(len(pages), Hkv, 16, 128, generator=g).to(torch.bfloat16).cuda()
    st.reset(keys=1696)
    q = _queries(Hq, [200], torch.bfloat16, 147)
    ref = bfl.prefill_chunk_paged(q, kp, vp, table, [0, 200], [1900], w0, w_pre, THETA, "fi", SCALE)
    got = bfl.prefill_chunk_stored_paged(q, kp, vp, table, st, [0, 200], [1900], w0, w_pre, THETA,
                                         "fi", SCALE)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_stored_paged_chunk_512_at_128k():
    # the last 512 queries of the 131072-key Qwen3-8B-shaped cache over 16-key
    # pages, after a call that filled the store up to 130560
    c = wl.CONFIGS["qwen3_8b_prefill_128k"]
    N, Lq, Hq, Hkv = c["lens"][0], 512, c["Hq"], c["Hkv"]
    kc, vc = _caches(1, Hkv, N, torch.bfloat16, 148)
    kp, vp, table = _paginate(kc, vc, 16, 149, spare=0)
    del kc, vc
    st = bfl.ChunkStore(kp, batch=1, max_pages_per_seq=table.shape[1])
    st.buf.fill_(255)
    args = (c["w0"], c["w_pre"], c["theta"], "pa", SCALE)
    q0 = _queries(Hq, [Lq], torch.bfloat16, 150)
    bfl.prefill_chunk_stored_paged(q0, kp, vp, table, st, [0, Lq], [N - Lq], *args, s_len=[N])
    q = _queries(Hq, [Lq], torch.bfloat16, 151)
    ref, lref = bfl.prefill_chunk_paged(q, kp, vp, table, [0, Lq], [N], *args, s_len=[N],
                                        return_lse=True)
    got, lgot = bfl.prefill_chunk_stored_paged(q, kp, vp, table, st, [0, Lq], [N], *args,
                                               s_len=[N], return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(got, ref) and torch.equal(lgot, lref)


def test_stored_paged_chunks_fp32():
    # fp32 over 16-key pages: the fp32 kernel reads k' of the packed copy only
    # for tiles with a local pair, which start at or above the copy's first key
    Hq, Hkv, w0, w_pre = 4, 1, 128, 256
    kc, vc = _caches(2, Hkv, 1152, torch.float32, 152)
    kp, vp, table = _paginate(kc, vc, 16, 153)
    st = bfl.ChunkStore(kp, batch=2, max_pages_per_seq=table.shape[1])
    st.buf.fill_(255)
    ends = [0, 0]
    for i, Lqs in enumerate([[300, 64], [5, 700], [400, 1], [64, 300]]):
        ends = [e + n for e, n in zip(ends, Lqs)]
        q = _queries(Hq, Lqs, torch.float32, 154 + i)
        cu = wl.cu_seqlens(Lqs)
        args = (w0, w_pre, THETA, "pa+shift", SCALE)
        ref, lref = bfl.prefill_chunk_paged(q, kp, vp, table, cu, ends, *args, s_len=[1100, 1100],
                                            return_lse=True)
        got, lgot = bfl.prefill_chunk_stored_paged(q, kp, vp, table, st, cu, ends, *args,
                                                   s_len=[1100, 1100], return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(lgot, lref), i


def test_stored_paged_chunks_batch_of_70():
    # 70 sequences over a shuffled 16-key page pool: two launch groups, each
    # with its rows of the block table, its part of the store and of the key axis
    B, Hq, Hkv, w0, w_pre = 70, 8, 2, 128, 512
    kc, vc = _caches(B, Hkv, 1600, torch.bfloat16, 170)
    kp, vp, table = _paginate(kc, vc, 16, 171)
    st = bfl.ChunkStore(kp, batch=B, max_pages_per_seq=table.shape[1])
    st.buf.fill_(255)
    chunks = [[40 + 3 * b, 200 + (7 * b) % 300, 1 + b % 5] for b in range(B)]
    ends = [0] * B
    for i in range(3):
        Lqs = [c[i] for c in chunks]
        ends = [e + n for e, n in zip(ends, Lqs)]
        q = _queries(Hq, Lqs, torch.bfloat16, 172 + i)
        cu = wl.cu_seqlens(Lqs)
        args = (w0, w_pre, THETA, "fi", SCALE)
        ref = bfl.prefill_chunk_paged(q, kp, vp, table, cu, ends, *args, s_len=[1600] * B)
        got = bfl.prefill_chunk_stored_paged(q, kp, vp, table, st, cu, ends, *args, s_len=[1600] * B)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), i
        assert list(st.keys) == ends
