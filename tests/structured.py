"""Structured inputs for the discrimination checks (test data only).

S2: the raw query and key vectors of KV group g are nonzero on one rotary
pair m*_g only, where the pair turns by theta_m* ~ 1 rad per position. The
given q', k' carry original RoPE at their positions, so every score is
scale * a_q * a_k * cos(theta_m* dpos + tau) with dpos = i - j (local pair),
(i - j) / s (frequency interpolation) or floor(i / s) - floor(j / s)
(position aliasing). The values are Fourier features at integer multiples of
theta_m* (and at theta_m* / s), so the output sums the attention weights
with phases theta_m* j: interpolation puts the weight peaks at positions
whose phases line up, aliasing spreads each peak over a group of s keys with
different phases, and plain attention lines them up at other distances. The
three results then differ by a large fraction of |o| instead of averaging
out.
"""
import math

import numpy as np
import torch

S2_FREQS = (1.0, 2.0, 3.0, 1.0 / 3.0, 2.0 / 3.0)


def s2_inputs(L, theta, mstars=(0, 1), a_q=(1.0, 0.9, 1.0, 0.8), tau=(0.0, 0.0, 0.3, 0.0),
              score_amp=24.0, D=128):
    """bf16 q' [Hq, L, D], k' / v [Hkv, L, D] with Hkv = len(mstars),
    Hq = Hkv * len(a_q); query head h of group g has amplitude factor
    a_q[h % G] and phase offset tau[h % G]; the largest score is score_amp."""
    scale = 1 / math.sqrt(D)
    a = math.sqrt(score_amp / scale)
    G = len(a_q)
    Hkv = len(mstars)
    pos = np.arange(L, dtype=np.float64)
    q = np.zeros((Hkv * G, L, D))
    k = np.zeros((Hkv, L, D))
    v = np.zeros((Hkv, L, D))
    for g, ms in enumerate(mstars):
        th = theta ** (-2.0 * ms / D)
        k[g, :, ms], k[g, :, ms + D // 2] = a * np.cos(pos * th), a * np.sin(pos * th)
        for hh in range(G):
            h = g * G + hh
            q[h, :, ms] = a * a_q[hh] * np.cos(pos * th + tau[hh])
            q[h, :, ms + D // 2] = a * a_q[hh] * np.sin(pos * th + tau[hh])
        for n, f in enumerate(S2_FREQS):
            v[g, :, 2 * n] = np.cos(f * th * pos)
            v[g, :, 2 * n + 1] = np.sin(f * th * pos)
    bf = lambda x: torch.from_numpy(x).to(torch.float32).to(torch.bfloat16)
    return bf(q), bf(k), bf(v)
