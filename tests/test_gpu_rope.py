"""GPU parity of the raw-input pre-step (original RoPE of raw q / k and the
KV-cache append) against the fp64 CPU oracle, and of the raw-input flow
(pre-step, then bifocal prefill / decode) end to end. Needs an MI355X.

Element-wise bar: the kernel rotates in fp32 with fp64 angles and rounds once;
the oracle rotates in fp64. bf16 outputs must equal the oracle's value rounded
to bf16 within one bf16 ulp plus the fp32 rotation error (2^-20 of the pair's
input size), and almost all bit-equal; fp32 outputs within 2e-6 of the input
scale. End-to-end: the attention tolerances (bf16 max-abs
2e-2, mean-abs 2e-3).
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


def _bf16_round(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _pair_mag(x):
    """|x_m| + |x_(m+64)| at every element of the rotary pair (fp64 numpy)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    s = a[..., :64] + a[..., 64:]
    return np.concatenate([s, s], axis=-1)


def _check_rot_bf16(got, ref64, raw, what):
    """got: bf16 tensor (cpu); ref64: the oracle's fp64 values; raw: the input
    rows. Bound per element: one bf16 ulp of the result plus the fp32
    rotation's own error, a few fp32 ulps of the pair's input size (where
    x cos - y sin cancels, that is more than an ulp of the small result)."""
    ref = _bf16_round(ref64)
    g = got.float().numpy()
    r = ref.float().numpy()
    equal = float(np.mean(g == r))
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 7), 0.0)
    bound = ulp + 2.0 ** -20 * _pair_mag(raw)
    worst = float(np.max(np.abs(g - r) - bound))
    print(f"[{what}] bit-equal {equal:.5f}, worst excess over the bound {worst:.2e}", flush=True)
    assert worst <= 0.0 and equal >= 0.999, what


def _check_rot_f32(got, ref64, scale, what):
    d = float(np.abs(got.numpy().astype(np.float64) - ref64).max())
    print(f"[{what}] max-abs {d:.3e}", flush=True)
    assert d <= 2e-6 * scale, what


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rope_prefill_matches_oracle(dtype):
    lens = [700, 413, 64, 1]
    cu = wl.cu_seqlens(lens)
    q, k, _ = wl.prefill_inputs(8, 2, cu[-1], 128, dtype, 71)
    qo, ko = bfl.rope_prefill(q.cuda(), k.cuda(), cu, THETA)
    torch.cuda.synchronize()
    pos = oracle.packed_positions(cu)
    rq = oracle.rope_rows(q.float().numpy(), pos, THETA)
    rk = oracle.rope_rows(k.float().numpy(), pos, THETA)
    if dtype == "bf16":
        _check_rot_bf16(qo.cpu(), rq, q.float().numpy(), "rope q bf16")
        _check_rot_bf16(ko.cpu(), rk, k.float().numpy(), "rope k bf16")
    else:
        scale = float(max(q.abs().max(), k.abs().max()))
        _check_rot_f32(qo.cpu(), rq, scale, "rope q fp32")
        _check_rot_f32(ko.cpu(), rk, scale, "rope k fp32")


def test_rope_prefill_128k_positions_sampled():
    # one 131072-token sequence: angles up to 1.3e5 rad, checked on sampled
    # tokens that include the first and the last
    T = 131072
    q, k, _ = wl.prefill_inputs(2, 1, T, 128, "bf16", 72)
    qo, ko = bfl.rope_prefill(q.cuda(), k.cuda(), [0, T], THETA)
    torch.cuda.synchronize()
    rng = np.random.default_rng(72)
    rows = np.unique(np.concatenate([[0, 1, 4095, 4096, T - 2, T - 1], rng.integers(0, T, 250)]))
    ri = torch.from_numpy(rows)
    rq = oracle.rope_rows(q[:, ri].float().numpy(), rows, THETA)
    rk = oracle.rope_rows(k[:, ri].float().numpy(), rows, THETA)
    _check_rot_bf16(qo[:, ri.cuda()].cpu(), rq, q[:, ri].float().numpy(), "rope q 128k")
    _check_rot_bf16(ko[:, ri.cuda()].cpu(), rk, k[:, ri].float().numpy(), "rope k 128k")


def test_rope_prefill_in_place_and_cache_fill():
    lens = [300, 1, 129]
    cu = wl.cu_seqlens(lens)
    q, k, v = wl.prefill_inputs(4, 2, cu[-1], 128, "bf16", 73)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    qo, ko = bfl.rope_prefill(qd, kd, cu, THETA)  # out of place, the reference
    cap = 320
    sentinel = 7.0
    kc = torch.full((3, 2, cap, 128), sentinel, dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, sentinel)
    q_in, k_in = qd.clone(), kd.clone()
    q2, k2 = bfl.rope_prefill(q_in, k_in, cu, THETA, v=vd, k_cache=kc, v_cache=vc, q_out=q_in,
                              k_out=k_in)
    torch.cuda.synchronize()
    assert q2.data_ptr() == q_in.data_ptr() and torch.equal(q_in, qo) and torch.equal(k_in, ko)
    for b, L in enumerate(lens):
        t0 = cu[b]
        assert torch.equal(kc[b, :, :L], ko[:, t0:t0 + L]), b
        assert torch.equal(vc[b, :, :L], vd[:, t0:t0 + L]), b
        assert bool((kc[b, :, L:] == sentinel).all()) and bool((vc[b, :, L:] == sentinel).all()), b
    # cache only (no packed k output) writes the same cache
    kc2 = torch.full_like(kc, sentinel)
    vc2 = torch.full_like(kc, sentinel)
    _, none = bfl.rope_prefill(qd, kd, cu, THETA, v=vd, k_cache=kc2, v_cache=vc2, write_k=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(kc2, kc) and torch.equal(vc2, vc)


def test_rope_append_matches_oracle():
    seqlens = [1, 4097, 131073]
    cap, Hq, Hkv = 131073, 4, 2
    rng = torch.Generator().manual_seed(74)
    qr = torch.randn(3, Hq, 128, generator=rng).to(torch.bfloat16)
    kr = torch.randn(3, Hkv, 128, generator=rng).to(torch.bfloat16)
    vr = torch.randn(3, Hkv, 128, generator=rng).to(torch.bfloat16)
    sentinel = -3.0
    kc = torch.full((3, Hkv, cap, 128), sentinel, dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, sentinel)
    qo = bfl.rope_append(qr.cuda(), kr.cuda(), vr.cuda(), kc, vc, seqlens, THETA)
    torch.cuda.synchronize()
    for b, N in enumerate(seqlens):
        p = N - 1
        rq = oracle.rope_rows(qr[b].float().numpy()[:, None, :], [p], THETA)[:, 0]
        rk = oracle.rope_rows(kr[b].float().numpy()[:, None, :], [p], THETA)[:, 0]
        _check_rot_bf16(qo[b].cpu(), rq, qr[b].float().numpy(), f"append q N={N}")
        _check_rot_bf16(kc[b, :, p].cpu(), rk, kr[b].float().numpy(), f"append k N={N}")
        assert torch.equal(vc[b, :, p].cpu(), vr[b]), b
        for other in (p - 1, p + 1):
            if 0 <= other < cap:
                assert bool((kc[b, :, other] == sentinel).all()) and bool((vc[b, :, other] == sentinel).all())


@pytest.mark.parametrize("mode", ["fi", "pa"])
def test_raw_input_prefill_end_to_end(mode):
    # raw q / k -> pre-step -> bifocal prefill, against the oracle on the
    # oracle's own rotation of the same raw inputs (rounded to bf16 as the
    # kernels store it)
    lens = [1500, 700]
    cu = wl.cu_seqlens(lens)
    Hq, Hkv, w0, w_pre = 8, 2, 128, 512
    q, k, v = wl.prefill_inputs(Hq, Hkv, cu[-1], 128, "bf16", 75)
    qo, ko = bfl.rope_prefill(q.cuda(), k.cuda(), cu, THETA)
    scale = 1 / math.sqrt(128)
    o = bfl.prefill(qo, ko, v.cuda(), cu, w0, w_pre, THETA, mode, scale)
    torch.cuda.synchronize()
    pos = oracle.packed_positions(cu)
    rq = _bf16_round(oracle.rope_rows(q.float().numpy(), pos, THETA)).float().numpy()
    rk = _bf16_round(oracle.rope_rows(k.float().numpy(), pos, THETA)).float().numpy()
    o_ref, _ = oracle.prefill(rq, rk, v.float().numpy(), cu, w0, w_pre, THETA, mode, scale)
    d = np.abs(o.float().cpu().numpy() - o_ref)
    print(f"[raw prefill {mode}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3


@pytest.mark.parametrize("mode", ["fi", "pa"])
def test_raw_input_decode_flow(mode):
    # prefill of L raw tokens fills the cache, one raw decode token is
    # appended, bifocal decode runs the step; reference: the oracle on its own
    # rotation of the whole raw sequence
    L, Hq, Hkv, cap, w0, w_pre = 3000, 8, 2, 4096, 128, 1024
    N = L + 1
    q, k, v = wl.prefill_inputs(Hq, Hkv, N, 128, "bf16", 76)  # token N - 1 is the decode token
    kc = torch.zeros((1, Hkv, cap, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    bfl.rope_prefill(qd[:, :L].contiguous(), kd[:, :L].contiguous(), [0, L], THETA,
                     v=vd[:, :L].contiguous(), k_cache=kc, v_cache=vc, write_k=False)
    q_new = qd[:, L].contiguous()[None]  # [1, Hq, D]
    k_new = kd[:, L].contiguous()[None]
    v_new = vd[:, L].contiguous()[None]
    q_rot = bfl.rope_append(q_new, k_new, v_new, kc, vc, [N], THETA)
    scale = 1 / math.sqrt(128)
    o = bfl.decode(q_rot, kc, vc, [N], w0, w_pre, THETA, mode, scale)
    torch.cuda.synchronize()
    pos = np.arange(N)
    rq = _bf16_round(oracle.rope_rows(q.float().numpy(), pos, THETA)).float().numpy()
    rk = _bf16_round(oracle.rope_rows(k.float().numpy(), pos, THETA)).float().numpy()
    kc_ref = np.zeros((1, Hkv, N, 128), np.float32)
    kc_ref[0] = rk
    vc_ref = v.float().numpy()[None]
    o_ref, _ = oracle.decode(rq[:, N - 1][None], kc_ref, vc_ref, [N], w0, w_pre, THETA, mode, scale)
    d = np.abs(o.float().cpu().numpy() - o_ref)
    print(f"[raw decode {mode}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3


def test_rope_prefill_start_positions_and_cache_rows():
    # pos0 moves each sequence's positions (a chunk after a cached prefix);
    # the cache rows written are pos0 .. pos0 + L - 1 and nothing else
    lens, pos0 = [300, 1, 129], [0, 4096, 131000]
    cu = wl.cu_seqlens(lens)
    q, k, v = wl.prefill_inputs(4, 2, cu[-1], 128, "bf16", 77)
    cap = 131129 + 3
    sentinel = 5.0
    kc = torch.full((3, 2, cap, 128), sentinel, dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, sentinel)
    qo, ko = bfl.rope_prefill(q.cuda(), k.cuda(), cu, THETA, v=v.cuda(), k_cache=kc, v_cache=vc,
                              pos0=pos0)
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(L) + p0 for L, p0 in zip(lens, pos0)])
    _check_rot_bf16(qo.cpu(), oracle.rope_rows(q.float().numpy(), pos, THETA), q.float().numpy(),
                    "rope q at start positions")
    _check_rot_bf16(ko.cpu(), oracle.rope_rows(k.float().numpy(), pos, THETA), k.float().numpy(),
                    "rope k at start positions")
    for b, (L, p0) in enumerate(zip(lens, pos0)):
        assert torch.equal(kc[b, :, p0:p0 + L], ko[:, cu[b]:cu[b + 1]]), b
        assert torch.equal(vc[b, :, p0:p0 + L].cpu(), v[:, cu[b]:cu[b + 1]]), b
        untouched = torch.ones(cap, dtype=torch.bool)
        untouched[p0:p0 + L] = False
        assert bool((kc[b][:, untouched] == sentinel).all()), b
        assert bool((vc[b][:, untouched] == sentinel).all()), b


@pytest.mark.parametrize("mode", ["fi", "pa"])
def test_raw_input_chunked_prefill_flow(mode):
    # a 3000-token raw prompt: the first 2000 tokens through the pre-step into
    # the cache, then the last 1000 as a chunk (pre-step at position 2000,
    # cache fill, bifocal_prefill_chunk); reference: the oracle's rows
    # 2000 .. 2999 of a one-shot prefill on its own rotation of the raw inputs
    N, P, Hq, Hkv, w0, w_pre = 3000, 2000, 8, 2, 128, 512
    q, k, v = wl.prefill_inputs(Hq, Hkv, N, 128, "bf16", 78)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kc = torch.zeros((1, Hkv, N, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    bfl.rope_prefill(qd[:, :P].contiguous(), kd[:, :P].contiguous(), [0, P], THETA,
                     v=vd[:, :P].contiguous(), k_cache=kc, v_cache=vc, write_k=False)
    q_chunk, _ = bfl.rope_prefill(qd[:, P:].contiguous(), kd[:, P:].contiguous(), [0, N - P], THETA,
                                  v=vd[:, P:].contiguous(), k_cache=kc, v_cache=vc, write_k=False,
                                  pos0=[P])
    scale = 1 / math.sqrt(128)
    o = bfl.prefill_chunk(q_chunk, kc, vc, [0, N - P], [N], w0, w_pre, THETA, mode, scale)
    torch.cuda.synchronize()
    pos = np.arange(N)
    rq = _bf16_round(oracle.rope_rows(q.float().numpy(), pos, THETA)).float().numpy()
    rk = _bf16_round(oracle.rope_rows(k.float().numpy(), pos, THETA)).float().numpy()
    o_ref, _ = oracle.prefill(rq, rk, v.float().numpy(), [0, N], w0, w_pre, THETA, mode, scale,
                              rows=np.arange(P, N))
    d = np.abs(o.float().cpu().numpy() - o_ref)
    print(f"[raw chunked prefill {mode}] max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
