"""bf16 discrimination of the two long-branch modes on the GPU (needs an MI355X).

Frequency interpolation and position aliasing are distinct results
[ai-feeds.com summary, "实验 / 关键发现", ablation bullet: the two
long-branch strategies]. On N(0,1) inputs they differ by little next to the
bf16 rounding of q'', k'' and P, so these tests use the structured input S2
(tests/structured.py): one high-frequency rotary pair per KV group and values
that are Fourier features at that pair's frequency, on which the two modes
and plain attention differ by about a third of |o| or more.

Each test runs one entry point through the C-ABI in both modes and requires,
on rows with far pairs:
  * the bf16 tolerance against the fp64 oracle on the same bf16 inputs;
  * |gpu - oracle| <= 0.05 |oracle - plain attention|;
  * |gpu - oracle| <= 0.05 |oracle - oracle in the other mode|;
and checks on the oracle side that the other mode sits at >= 0.5 of the plain
gap, so that a kernel computing the wrong mode could not pass. Rows are taken
at the first position of an aliasing group (i = 0 mod s), where the query's
scaled position is the same in both modes and the modes differ through the
keys alone.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from rope_context_extension_bifocal_amd import bifocal as bfl
from structured import s2_inputs

pytestmark = pytest.mark.gpu

L, THETA, W_PRE, W0 = 8192, 1e4, 3000, 256  # s(8192) = s(8191) = 3
SCALE = 1 / math.sqrt(128)
OTHER = {"fi": "pa", "pa": "fi"}


@pytest.fixture(scope="module")
def s2():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()
    q, k, v = s2_inputs(L, THETA)
    return (q, k, v), tuple(x.float().numpy() for x in (q, k, v))


def _rows(lo, hi, n, seed):
    s = oracle.s_of_L(L, W_PRE)
    cand = np.arange(lo + (-lo) % s, hi, s)
    rows = np.random.default_rng(seed).choice(cand, size=min(n, len(cand)), replace=False)
    return np.sort(np.unique(np.append(rows, cand[-1])))


def _bars(tag, og, ref, other, plain):
    d = np.abs(og - ref)
    err = np.linalg.norm(og - ref)
    gap_plain = np.linalg.norm(ref - plain)
    gap_other = np.linalg.norm(ref - other)
    power = gap_other / gap_plain
    print(f"[{tag}] max-abs {d.max():.3e} mean-abs {d.mean():.3e} err {err:.3e} "
          f"gap-plain {gap_plain:.3e} gap-other {gap_other:.3e} err/gap-plain {err / gap_plain:.4f} "
          f"err/gap-other {err / gap_other:.4f} other-mode/plain (oracle) {power:.3f}", flush=True)
    assert power >= 0.5, "the input does not separate the modes"
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert err <= 0.05 * gap_plain
    assert err <= 0.05 * gap_other


@pytest.mark.parametrize("mode", ["fi", "pa"])
def test_s2_prefill_separates_modes(s2, mode):
    (q, k, v), (qf, kf, vf) = s2
    o = bfl.prefill(q.cuda(), k.cuda(), v.cuda(), [0, L], W0, W_PRE, THETA, mode, SCALE)
    torch.cuda.synchronize()
    rows = _rows(2048, L, 48, 1)
    og = o[:, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref, _ = oracle.prefill(qf, kf, vf, [0, L], W0, W_PRE, THETA, mode, SCALE, rows=rows)
    other, _ = oracle.prefill(qf, kf, vf, [0, L], W0, W_PRE, THETA, OTHER[mode], SCALE, rows=rows)
    plain, _ = oracle.prefill(qf, kf, vf, [0, L], 10**9, W_PRE, THETA, mode, SCALE, rows=rows)
    _bars(f"S2 prefill {mode}", og, ref, other, plain)


@pytest.mark.parametrize("mode", ["fi", "pa"])
@pytest.mark.parametrize("paged", [False, True])
def test_s2_decode_separates_modes(s2, mode, paged):
    # the query at position N - 1 = 8190 over the N = 8191 cached keys
    (q, k, v), (qf, kf, vf) = s2
    N = L - 1
    qd = q[:, N - 1].unsqueeze(0).contiguous()
    kc, vc = k[:, :N].unsqueeze(0).contiguous(), v[:, :N].unsqueeze(0).contiguous()
    if paged:  # 16-key pages in reversed order
        pg = 16
        npg = -(-N // pg)
        def pool(x):
            xp = torch.zeros((x.shape[1], npg * pg, 128), dtype=x.dtype)
            xp[:, :N] = x[0]
            return xp.view(x.shape[1], npg, pg, 128).transpose(0, 1).flip(0).contiguous()
        table = torch.arange(npg - 1, -1, -1, dtype=torch.int32)[None].cuda()
        o = bfl.decode_paged(qd.cuda(), pool(kc).cuda(), pool(vc).cuda(), table, [N], W0, W_PRE,
                             THETA, mode, SCALE)
    else:
        o = bfl.decode(qd.cuda(), kc.cuda(), vc.cuda(), [N], W0, W_PRE, THETA, mode, SCALE)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    args = (qd.float().numpy(), kc.float().numpy(), vc.float().numpy(), [N])
    ref, _ = oracle.decode(*args, W0, W_PRE, THETA, mode, SCALE)
    other, _ = oracle.decode(*args, W0, W_PRE, THETA, OTHER[mode], SCALE)
    plain, _ = oracle.decode(*args, 10**9, W_PRE, THETA, mode, SCALE)
    _bars(f"S2 decode{' paged' if paged else ''} {mode}", og, ref, other, plain)


@pytest.mark.parametrize("mode", ["fi", "pa"])
def test_s2_chunk_separates_modes(s2, mode):
    # the last 600 queries (positions 7591 .. 8190) against the 8191 cached
    # keys: a short chunk, so the launch splits its key tiles and merges the
    # parts by log-sum-exp
    (q, k, v), (qf, kf, vf) = s2
    N, Lq = L - 1, 600
    qc = q[:, N - Lq:N].contiguous()
    kc, vc = k[:, :N].unsqueeze(0).contiguous(), v[:, :N].unsqueeze(0).contiguous()
    o = bfl.prefill_chunk(qc.cuda(), kc.cuda(), vc.cuda(), [0, Lq], [N], W0, W_PRE, THETA, mode,
                          SCALE)
    torch.cuda.synchronize()
    pos = _rows(N - Lq, N, 48, 2)
    rows = pos - (N - Lq)
    og = o[:, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    args = (qc.float().numpy(), kc.float().numpy(), vc.float().numpy(), [0, Lq], [N])
    ref, _ = oracle.chunk(*args, W0, W_PRE, THETA, mode, SCALE, rows=rows)
    other, _ = oracle.chunk(*args, W0, W_PRE, THETA, OTHER[mode], SCALE, rows=rows)
    plain, _ = oracle.chunk(*args, 10**9, W_PRE, THETA, mode, SCALE, rows=rows)
    _bars(f"S2 chunk {mode}", og, ref, other, plain)
