"""Seeded synthetic workloads for bifocal attention.

This module only draws random numbers and fixes shapes. It holds none of the
method's arithmetic (no RoPE, no s(L), no attention). The library tests, the
benchmark and the CPU oracle's callers all take their inputs from here, so
both sides of every parity check see the same bytes.

Value law: Q, K, V ~ N(0, 1), drawn in fp32 from a CPU torch.Generator in the
order Q, K, V and then rounded to the working dtype (round-to-nearest-even for
bf16). Because N(0, 1) vectors are rotation invariant in law, the samples are
used directly as the original-RoPE (cache form) q' and k'.

The shapes are those of Qwen3 attention layers (1.7B: 16 query / 8 KV heads;
4B and 8B: 32 / 8; head_dim 128) at the context lengths the pages evaluate
(up to 128K). They stand in for the RULER / HELMET-RAG / PG-19 inputs the
pages measure on, which need weights and datasets this project does not use.
"""
import math

import numpy as np
import torch

# Each entry is one workload of the benchmark / parity suite.
CONFIGS = {
    "tiny_fp32_s2": dict(
        dtype="fp32", Hq=2, Hkv=1, D=128, lens=[2048], w_pre=1024, w0=256,
        theta=1e4, modes=["fi"], seed=1),
    "qwen3_1p7b_prefill_32k_s1": dict(
        dtype="bf16", Hq=16, Hkv=8, D=128, lens=[32768], w_pre=32768, w0=4096,
        theta=1e6, modes=["fi"], seed=2),
    "qwen3_8b_prefill_128k": dict(
        dtype="bf16", Hq=32, Hkv=8, D=128, lens=[131072], w_pre=32768, w0=4096,
        theta=1e6, modes=["fi", "pa"], seed=3),
    "qwen3_8b_decode": dict(
        dtype="bf16", Hq=32, Hkv=8, D=128, cache_lens=[4096, 32768, 131072],
        w_pre=32768, w0=4096, theta=1e6, modes=["fi", "pa"], seed=40),
    "qwen3_4b_ragged_prefill": dict(
        dtype="bf16", Hq=32, Hkv=8, D=128, n_seqs=8, len_lo=4096, len_hi=131072,
        w_pre=32768, w0=4096, theta=1e6, modes=["fi"], seed=5),
}

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}


def ragged_lengths(n_seqs=8, lo=4096, hi=131072, seed=5):
    """Log-uniform sequence lengths in [lo, hi], seeded."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(lo), math.log(hi), size=n_seqs)
    return [int(min(max(int(math.floor(math.exp(x))), lo), hi)) for x in u]


def cu_seqlens(lens):
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + int(L))
    return cu


def _randn(gen, shape, dtype):
    out = torch.empty(shape, dtype=TORCH_DTYPES[dtype])
    # draw per leading index to bound the fp32 staging memory
    for h in range(shape[0]):
        out[h] = torch.randn(shape[1:], generator=gen, dtype=torch.float32).to(out.dtype)
    return out


def prefill_inputs(Hq, Hkv, T, D=128, dtype="bf16", seed=0):
    """Packed prefill inputs on the CPU: q [Hq,T,D], k [Hkv,T,D], v [Hkv,T,D]."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    q = _randn(gen, (Hq, T, D), dtype)
    k = _randn(gen, (Hkv, T, D), dtype)
    v = _randn(gen, (Hkv, T, D), dtype)
    return q, k, v


def decode_inputs(B, Hq, Hkv, cap, D=128, dtype="bf16", seed=0):
    """Decode inputs on the CPU: q [B,Hq,D], k_cache / v_cache [B,Hkv,cap,D]."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((B, Hq, D), generator=gen, dtype=torch.float32).to(TORCH_DTYPES[dtype])
    kc = torch.empty((B, Hkv, cap, D), dtype=TORCH_DTYPES[dtype])
    vc = torch.empty((B, Hkv, cap, D), dtype=TORCH_DTYPES[dtype])
    for b in range(B):
        kc[b] = _randn(gen, (Hkv, cap, D), dtype)
    for b in range(B):
        vc[b] = _randn(gen, (Hkv, cap, D), dtype)
    return q, kc, vc


def sample_rows(L, n, edges, seed):
    """A seeded sorted set of query rows of one sequence of length L: the
    given edge rows (clipped to [0, L)) plus n uniform draws."""
    rng = np.random.default_rng(seed)
    picked = set(int(e) for e in edges if 0 <= int(e) < L)
    if n > 0:
        picked.update(int(x) for x in rng.integers(0, L, size=n))
    return np.array(sorted(picked), dtype=np.int64)
