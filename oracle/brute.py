"""Brute-force bifocal attention for tiny inputs (test infrastructure only).

A second, independent statement of the per-pair definition, used to pin the
C oracle. Every pair (i, j) is scored on its own with explicit 2x2 rotation
matrices, one per rotary pair, built from the angle pos * theta_m:

* local pair (i - j < w0): the dot product of the given q'_i and k'_j,
  which already carry original RoPE [ai-feeds.com summary, "方法 / 关键模块"
  item 1: the window of size w0 keeps unmodified RoPE];
* far pair: both vectors are taken back to their raw form with the inverse
  rotation at their own positions, then rotated to the scaled positions
  phi(p) = p / s or floor(p / s) [same item; "实验 / 关键发现", the two
  long-branch strategies], with s = max(1, ceil(L / w_pre)) [promo script,
  storyboard scene-2].

Softmax is evaluated per row over j <= i in fp64. Meant for L <= 64.
"""
import math

import numpy as np


def _rot2(angle):
    c, s = math.cos(angle), math.sin(angle)
    return np.array([[c, -s], [s, c]], dtype=np.float64)


def _rotate(x, pos, theta):
    """Apply original RoPE at (real) position pos with explicit 2x2 matrices;
    pair m couples coordinates m and m + D/2."""
    D = x.shape[0]
    H = D // 2
    y = np.empty(D, dtype=np.float64)
    for m in range(H):
        freq = theta ** (-2.0 * m / D)
        pair = np.array([x[m], x[m + H]], dtype=np.float64)
        r = _rot2(pos * freq) @ pair
        y[m], y[m + H] = r[0], r[1]
    return y


def scaled_factor(L, w_pre):
    s = 1
    while L > s * w_pre:          # smallest s >= 1 with L <= s * w_pre
        s += 1
    return s


def brute_prefill(q, k, v, w0, w_pre, theta, mode, scale):
    """One sequence: q [Hq,L,D], k/v [Hkv,L,D] (any float dtype).
    Returns (o [Hq,L,D], lse [Hq,L]) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, L, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    s = scaled_factor(L, w_pre)

    def phi(p):
        return p / s if mode == "fi" else float(p // s)

    o = np.zeros((Hq, L, D))
    lse = np.zeros((Hq, L))
    for h in range(Hq):
        hk = h // G
        for i in range(L):
            scores = []
            for j in range(i + 1):
                if i - j < w0:
                    sc = scale * float(q[h, i] @ k[hk, j])
                else:
                    qr = _rotate(q[h, i], -i, theta)
                    kr = _rotate(k[hk, j], -j, theta)
                    sc = scale * float(_rotate(qr, phi(i), theta) @ _rotate(kr, phi(j), theta))
                scores.append(sc)
            sc = np.array(scores)
            mx = sc.max()
            w = np.exp(sc - mx)
            o[h, i] = (w[:, None] * v[hk, : i + 1]).sum(0) / w.sum()
            lse[h, i] = mx + math.log(w.sum())
    return o, lse
