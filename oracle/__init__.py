"""fp64 CPU oracle for Dynamic Bifocal RoPE attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the library or its binding.

Thin ctypes wrapper around oracle.c (the per-pair piecewise definition in
fp64, OpenMP over (head, row)). Inputs are numpy arrays; bf16 data should be
widened to float32 first (exact).
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")  # e.g. the AddressSanitizer build
        if not path:
            build(force=False)
            path = LIB
        lib = ctypes.CDLL(path)
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        p = ctypes.c_void_p
        lib.oracle_s_of_L.restype = i64
        lib.oracle_s_of_L.argtypes = [i64, i64]
        lib.oracle_phi.restype = f64
        lib.oracle_phi.argtypes = [i64, i64, i32]
        lib.oracle_rope_rotate.restype = None
        lib.oracle_rope_rotate.argtypes = [p, p, i64, f64, f64]
        lib.oracle_rope_rows.restype = ctypes.c_int
        lib.oracle_rope_rows.argtypes = [p, p, i64, i64, i64, p, f64]
        lib.oracle_pair_branch.restype = i32
        lib.oracle_pair_branch.argtypes = [i64, i64, i64]
        lib.oracle_prefill_rows.restype = ctypes.c_int
        lib.oracle_prefill_rows.argtypes = [p, p, p, p, i64, p, i64, i64, i64, i64, i64, i64,
                                            f64, i32, f64, i32, p, p]
        lib.oracle_chunk_rows.restype = ctypes.c_int
        lib.oracle_chunk_rows.argtypes = [p, p, p, p, p, p, i64, i64, p, i64, i64, i64, i64, i64,
                                          i64, f64, i32, f64, p, p]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64, i64, f64, i32,
                                      f64, p, p]
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# band: far pairs dropped (sliding window w0); "+shift": band-edge continuity shift
MODES = {"fi": 0, "pa": 1, "band": 2, "fi+shift": 4, "pa+shift": 5}


def s_of_L(L, w_pre):
    return int(_load().oracle_s_of_L(int(L), int(w_pre)))


def phi(p, s, mode):
    return float(_load().oracle_phi(int(p), int(s), MODES[mode]))


def pair_branch(i, j, w0):
    """1 = local (original RoPE), 2 = far (scaled RoPE), 0 = causally masked."""
    return int(_load().oracle_pair_branch(int(i), int(j), int(w0)))


def rope_rotate(x, pos, theta):
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    y = np.empty_like(x)
    _load().oracle_rope_rotate(_ptr(x), _ptr(y), x.shape[-1], float(pos), float(theta))
    return y


def rope_rows(x, positions, theta):
    """Original RoPE of raw rows: x [H,T,D] (row (h, t) a token at
    positions[t]) -> fp64 [H,T,D] rotated by positions[t] * theta_m."""
    x = _f32(x)
    H, T, D = x.shape
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
    assert pos.shape == (T,)
    y = np.empty((H, T, D), dtype=np.float64)
    rc = _load().oracle_rope_rows(_ptr(x), _ptr(y), H, T, D, _ptr(pos), float(theta))
    if rc != 0:
        raise ValueError(f"oracle_rope_rows failed: {rc}")
    return y


def packed_positions(cu_seqlens):
    """Sequence-relative position of every packed token (restarts per sequence)."""
    cu = [int(c) for c in cu_seqlens]
    return np.concatenate([np.arange(cu[b + 1] - cu[b], dtype=np.int64) for b in range(len(cu) - 1)])


def prefill(q, k, v, cu_seqlens, w0, w_pre, theta, mode, scale, rows=None, variant=0,
            gathered=False):
    """Bifocal prefill at query rows `rows` (global packed token indices; all
    rows when None).  q [Hq,T,D] (or [Hq,R,D] already gathered at `rows` when
    gathered=True), k/v [Hkv,T,D].  Returns fp64 (o [Hq,R,D], lse [Hq,R]).
    variant 1 evaluates the inclusion-exclusion partials."""
    k = _f32(k)
    v = _f32(v)
    q = np.asarray(q)
    Hq, _, D = q.shape
    T = k.shape[1]
    Hkv = k.shape[0]
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    B = cu.shape[0] - 1
    if rows is None:
        rows = np.arange(T, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    q_rows = _f32(q) if gathered else _f32(q[:, rows, :])
    R = rows.shape[0]
    o = np.empty((Hq, R, D), dtype=np.float64)
    lse = np.empty((Hq, R), dtype=np.float64)
    rc = _load().oracle_prefill_rows(_ptr(q_rows), _ptr(k), _ptr(v), _ptr(cu), B, _ptr(rows), R,
                                     Hq, Hkv, D, int(w0), int(w_pre), float(theta), MODES[mode],
                                     float(scale), int(variant), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_prefill_rows failed: {rc}")
    return o, lse


def decode(q, k_cache, v_cache, seqlens, w0, w_pre, theta, mode, scale):
    """Bifocal single-token decode.  q [B,Hq,D], caches [B,Hkv,cap,D],
    seqlens[b] = number of valid keys including the new token.  Returns fp64
    (o [B,Hq,D], lse [B,Hq])."""
    q = _f32(q)
    k_cache = _f32(k_cache)
    v_cache = _f32(v_cache)
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int64))
    o = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = _load().oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sl), B, cap, Hq, Hkv,
                               D, int(w0), int(w_pre), float(theta), MODES[mode], float(scale),
                               _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_decode failed: {rc}")
    return o, lse


def chunk(q, k_cache, v_cache, cu_q, seqlens, w0, w_pre, theta, mode, scale, s_len=None,
          rows=None, gathered=False):
    """Multi-token queries over a KV cache (chunked prefill).  q [Hq,Tq,D]
    packed by cu_q (or [Hq,R,D] already gathered at `rows` when gathered=True),
    caches [B,Hkv,cap,D] with seqlens[b] keys; the queries of b are its last
    positions seqlens[b] - Lq_b .. seqlens[b] - 1, s = s(s_len[b]) (default
    seqlens[b]).  Returns fp64 (o [Hq,R,D], lse [Hq,R])."""
    k_cache = _f32(k_cache)
    v_cache = _f32(v_cache)
    q = np.asarray(q)
    Hq, _, D = q.shape
    B, Hkv, cap = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    cu = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int64))
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int64))
    sll = None if s_len is None else np.ascontiguousarray(np.asarray(s_len, dtype=np.int64))
    if rows is None:
        rows = np.arange(int(cu[-1]), dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    q_rows = _f32(q) if gathered else _f32(q[:, rows, :])
    R = rows.shape[0]
    o = np.empty((Hq, R, D), dtype=np.float64)
    lse = np.empty((Hq, R), dtype=np.float64)
    rc = _load().oracle_chunk_rows(_ptr(q_rows), _ptr(k_cache), _ptr(v_cache), _ptr(cu), _ptr(sl),
                                   _ptr(sll) if sll is not None else None, B, cap, _ptr(rows), R,
                                   Hq, Hkv, D, int(w0), int(w_pre), float(theta), MODES[mode],
                                   float(scale), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_chunk_rows failed: {rc}")
    return o, lse


def threads():
    """OpenMP threads the oracle will use (OMP_NUM_THREADS or all cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    return int(env) if env else os.cpu_count()
