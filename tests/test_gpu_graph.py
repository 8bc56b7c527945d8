"""GPU test: a decode step (raw-input append, then bifocal decode, contiguous
and paged) captured into a HIP graph through torch.cuda.CUDAGraph. The library
launches kernels only (no allocation, no memset) on the caller's stream, with
caller-owned workspaces, so the step can be captured once and replayed. Each
replay runs after eager work and a synchronisation, on inputs the host has
changed in place, and must be bitwise the eager call on the same inputs.
Needs an MI355X.
"""
import math

import pytest
import torch

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


@pytest.mark.parametrize("paged", [False, True])
def test_decode_step_graph_replays_match_eager(paged):
    B, Hq, Hkv, cap, page = 2, 32, 8, 40000, 64
    N = [32769, 5000]  # the new token's position is N - 1
    _, kc, vc = wl.decode_inputs(B, Hq, Hkv, cap, 128, "bf16", 501)
    kc, vc = kc.cuda(), vc.cuda()
    if paged:
        per = cap // page
        perm = torch.randperm(B * per, generator=torch.Generator().manual_seed(502)).cuda()
        table = perm.to(torch.int32).view(B, per)
        kp = torch.empty((B * per, Hkv, page, 128), dtype=torch.bfloat16, device="cuda")
        vp = torch.empty_like(kp)
        kp[perm] = kc.view(B, Hkv, per, page, 128).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page, 128)
        vp[perm] = vc.view(B, Hkv, per, page, 128).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page, 128)
        kcache, vcache = kp, vp
    else:
        kcache, vcache = kc, vc
    g = torch.Generator(device="cuda").manual_seed(503)
    q_raw = torch.randn(B, Hq, 128, generator=g, device="cuda").to(torch.bfloat16)
    k_raw = torch.randn(B, Hkv, 128, generator=g, device="cuda").to(torch.bfloat16)
    v_raw = torch.randn(B, Hkv, 128, generator=g, device="cuda").to(torch.bfloat16)
    q_rot = torch.empty_like(q_raw)
    o = torch.empty_like(q_raw)
    ws = bfl.alloc_workspace(bfl.workspace_bytes(bfl.BF_PHASE_DECODE, B, max(N), Hq, Hkv), "cuda")

    def step():
        if paged:
            bfl.rope_append_paged(q_raw, k_raw, v_raw, kcache, vcache, table, N, THETA, q_out=q_rot)
            bfl.decode_paged(q_rot, kcache, vcache, table, N, 4096, 8192, THETA, "fi", SCALE, out=o,
                             workspace=ws)
        else:
            bfl.rope_append(q_raw, k_raw, v_raw, kcache, vcache, N, THETA, q_out=q_rot)
            bfl.decode(q_rot, kcache, vcache, N, 4096, 8192, THETA, "fi", SCALE, out=o, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        # new raw inputs in place, some eager work, then the replay
        q_raw.copy_(torch.randn(B, Hq, 128, generator=g, device="cuda").to(torch.bfloat16))
        k_raw.copy_(torch.randn(B, Hkv, 128, generator=g, device="cuda").to(torch.bfloat16))
        v_raw.copy_(torch.randn(B, Hkv, 128, generator=g, device="cuda").to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_graph = o.clone()
        step()  # eager on the same inputs (the append rewrites the same cache rows)
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o), (paged, r)
