"""Work scheduling of the bf16 prefill kernel (needs an MI355X).

A launch of 1024 or more work items runs on persistent workgroups that claim
their items from per-XCD queues; a smaller launch runs one workgroup per item.
Which workgroup runs an item must not change the item's arithmetic, so a
batched launch (claimed items) is bitwise the same sequences launched one at a
time (2048 tokens x 8 KV heads = 512 items each: one workgroup per item), and
repeated batched launches are bitwise equal. The per-sequence results are
checked against the fp64 oracle in test_gpu_parity.py.
"""
import math

import pytest
import torch

from rope_context_extension_bifocal_amd import bifocal as bfl
from rope_context_extension_bifocal_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    bfl.lib()


@pytest.mark.parametrize("mode", ["fi", "pa+shift", "band"])
def test_batched_launch_equals_per_sequence_launches(mode):
    # 12 prompts of 2048 tokens (s = 2), 32 / 8 heads: 12 x 64 x 8 = 6144 items
    B, L, Hq, Hkv, w0, w_pre = 12, 2048, 32, 8, 512, 1024
    cu = wl.cu_seqlens([L] * B)
    q, k, v = (x.cuda() for x in wl.prefill_inputs(Hq, Hkv, cu[-1], 128, "bf16", 160))
    o, lse = bfl.prefill(q, k, v, cu, w0, w_pre, 1e6, mode, SCALE, return_lse=True)
    for b in range(B):
        sl = slice(cu[b], cu[b + 1])
        ob, lb = bfl.prefill(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                             [0, L], w0, w_pre, 1e6, mode, SCALE, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o[:, sl], ob) and torch.equal(lse[:, sl], lb), (mode, b)


def test_batched_launch_is_deterministic():
    B, L, Hq, Hkv = 64, 2048, 32, 8
    cu = wl.cu_seqlens([L] * B)
    q, k, v = (x.cuda() for x in wl.prefill_inputs(Hq, Hkv, cu[-1], 128, "bf16", 161))
    a = bfl.prefill(q, k, v, cu, 4096, 1024, 1e6, "fi", SCALE)
    b = bfl.prefill(q, k, v, cu, 4096, 1024, 1e6, "fi", SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
