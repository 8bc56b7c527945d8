"""bifocal_decode_stored on the GPU (needs an MI355X).

The far-key store keeps k'' = R(theta_m (phi(j) - j)) k'_j of far keys
between decode steps [ai-feeds.com summary, "关键模块" item 3: the correction
rotation of cached keys]. The stored values are the ones bifocal_decode forms
on the fly, so every step must be bitwise the stateless decode; the stateless
decode itself is checked against the fp64 oracle in test_gpu_parity.py, and
one step here is checked against the oracle too.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()


@pytest.mark.parametrize("mode", ["fi", "pa", "fi+shift", "pa+shift"])
def test_stored_steps_equal_decode(mode):
    # 32 / 8 heads, w0 = 256, w_pre = 1024: s(N) = 2 up to N = 2048 and 3 from
    # 2049 on, so the walk refills the store once; then a rollback to 2070 keys
    # with the positions from 1809 on counted as rewritten
    B, Hq, Hkv, cap, w0, w_pre, theta = 2, 32, 8, 2304, 256, 1024, 1e4
    q, kc, vc = (x.cuda() for x in wl.decode_inputs(B, Hq, Hkv, cap, 128, "bf16", 71))
    store = bfl.DecodeStore(kc)
    store.k2.fill_(float("nan"))  # nothing the store has not written may be read
    steps = [2030, 2031, 2047, 2048, 2049, 2050, 2066, 2100, 2070]
    for i, n in enumerate(steps):
        lens = [n, n - 37]
        if n == 2070:
            store.reset(keys=n - w0 - 5)
        ref = bfl.decode(q, kc, vc, lens, w0, w_pre, theta, mode, SCALE)
        got = bfl.decode_stored(q, kc, vc, store, lens, w0, w_pre, theta, mode, SCALE)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (mode, n)
        for b, nb in enumerate(lens):
            s = bfl.s_of_L(nb, w_pre)
            assert store.s[b] == s
            assert store.keys[b] == (nb - w0 if s > 1 else 0)


def test_stored_batch_mixed_state():
    # one sequence without far keys (s = 1), one with a store made for another
    # s (ignored), one whose count exceeds its far keys (clamped), one fresh
    B, Hq, Hkv, cap, w0, w_pre, theta = 4, 16, 4, 9216, 512, 4096, 1e6
    q, kc, vc = (x.cuda() for x in wl.decode_inputs(B, Hq, Hkv, cap, 128, "bf16", 72))
    lens = [3000, 9000, 8200, 4500]
    store = bfl.DecodeStore(kc)
    warm = bfl.decode_stored(q, kc, vc, store, lens, w0, w_pre, theta, "pa", SCALE)
    torch.cuda.synchronize()
    assert list(store.s) == [1, 3, 3, 2] and list(store.keys) == [0, 8488, 7688, 3988]
    store.s[1] = 2           # as if made for another s: read nothing back
    store.keys[2] = 9000     # more than the far keys of 8200
    store.keys[3] = 0        # fresh
    ref = bfl.decode(q, kc, vc, lens, w0, w_pre, theta, "pa", SCALE)
    got = bfl.decode_stored(q, kc, vc, store, lens, w0, w_pre, theta, "pa", SCALE)
    torch.cuda.synchronize()
    assert torch.equal(got, ref) and torch.equal(warm, ref)


def test_stored_matches_oracle():
    B, Hq, Hkv, cap, w0, w_pre, theta = 1, 8, 2, 3000, 128, 1024, 1e4
    q, kc, vc = wl.decode_inputs(B, Hq, Hkv, cap, 128, "bf16", 73)
    N = 2999
    store = bfl.DecodeStore(kc.cuda())
    kcg, vcg, qg = kc.cuda(), vc.cuda(), q.cuda()
    bfl.decode_stored(qg, kcg, vcg, store, [N - 40], w0, w_pre, theta, "fi", SCALE)  # fills most of it
    got = bfl.decode_stored(qg, kcg, vcg, store, [N], w0, w_pre, theta, "fi", SCALE)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), [N], w0,
                           w_pre, theta, "fi", SCALE)
    d = np.abs(got.float().cpu().numpy() - ref)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3


def test_stored_128k():
    # the bench's decode layer: a fresh store (every far key rotated and
    # written), then a full one (every far key read back)
    B, Hq, Hkv, N = 1, 32, 8, 131073
    q, kc, vc = (x.cuda() for x in wl.decode_inputs(B, Hq, Hkv, N, 128, "bf16", 40))
    store = bfl.DecodeStore(kc)
    ref = bfl.decode(q, kc, vc, [N], 4096, 32768, 1e6, "fi", SCALE)
    a = bfl.decode_stored(q, kc, vc, store, [N], 4096, 32768, 1e6, "fi", SCALE)
    b = bfl.decode_stored(q, kc, vc, store, [N], 4096, 32768, 1e6, "fi", SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a, ref) and torch.equal(b, ref)
    assert store.keys[0] == N - 4096 and store.s[0] == 5


@pytest.mark.parametrize("page", [16, 64])
def test_stored_paged_equals_contiguous(page):
    # the same two-sequence walk over a shuffled page pool: bitwise the
    # contiguous stored decode and the stateless paged decode at every step
    B, Hq, Hkv, cap, w0, w_pre, theta = 2, 32, 8, 2304, 256, 1024, 1e4
    q, kc, vc = (x.cuda() for x in wl.decode_inputs(B, Hq, Hkv, cap, 128, "bf16", 74))
    per = cap // page
    perm = torch.randperm(B * per, generator=torch.Generator().manual_seed(75)).cuda()
    kp = torch.empty((B * per, Hkv, page, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    kp[perm] = kc.view(B, Hkv, per, page, 128).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page, 128)
    vp[perm] = vc.view(B, Hkv, per, page, 128).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page, 128)
    table = perm.to(torch.int32).view(B, per)
    sc, sp = bfl.DecodeStore(kc), bfl.DecodeStore(kp, batch=B)
    sp.k2.fill_(float("nan"))
    for n in [2030, 2031, 2048, 2049, 2050, 2100]:
        lens = [n, n - 21]
        ref = bfl.decode_paged(q, kp, vp, table, lens, w0, w_pre, theta, "pa+shift", SCALE)
        got_c = bfl.decode_stored(q, kc, vc, sc, lens, w0, w_pre, theta, "pa+shift", SCALE)
        got_p = bfl.decode_stored_paged(q, kp, vp, table, sp, lens, w0, w_pre, theta, "pa+shift",
                                        SCALE)
        torch.cuda.synchronize()
        assert torch.equal(got_p, ref) and torch.equal(got_c, ref), n
        assert list(sp.keys) == list(sc.keys) and list(sp.s) == list(sc.s)


def test_stored_batch_of_70():
    # more sequences than one launch takes (64): the counters of every group
    # are kept; lengths spread over s = 1 .. 3
    B, Hq, Hkv, cap, w0, w_pre, theta = 70, 8, 2, 2560, 128, 1024, 1e4
    q, kc, vc = (x.cuda() for x in wl.decode_inputs(B, Hq, Hkv, cap, 128, "bf16", 76))
    lens = [100 + 35 * b for b in range(B)]
    store = bfl.DecodeStore(kc)
    for step in range(3):
        cur = [n + step for n in lens]
        ref = bfl.decode(q, kc, vc, cur, w0, w_pre, theta, "fi", SCALE)
        got = bfl.decode_stored(q, kc, vc, store, cur, w0, w_pre, theta, "fi", SCALE)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), step
        for b, n in enumerate(cur):
            s = bfl.s_of_L(n, w_pre)
            assert store.s[b] == s and store.keys[b] == (n - w0 if s > 1 and n > w0 else 0)
