"""Python binding of libbifocal (ctypes). Argument marshalling only.

Every step of the computation runs in the HIP kernels of libbifocal.so; this
module allocates outputs and workspaces through PyTorch (device memory and
streams are the only things PyTorch provides) and passes raw pointers to the
C-ABI entry points declared in include/bifocal.h. There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""
import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# BIFOCAL_LIB selects another build of the same library (e.g. the
# AddressSanitizer build of the host code for CPU-side test runs)
LIB_PATH = os.environ.get("BIFOCAL_LIB") or os.path.join(_PKG, "libbifocal.so")

BF_OK, BF_ERR_INVALID_ARG, BF_ERR_UNSUPPORTED, BF_ERR_WORKSPACE, BF_ERR_HIP = 0, -1, -2, -3, -4
BF_DTYPE_BF16, BF_DTYPE_FP32 = 0, 1
BF_LONG_FI, BF_LONG_PA, BF_LONG_NONE, BF_LONG_SHIFT = 0, 1, 2, 4
BF_PHASE_PREFILL, BF_PHASE_DECODE = 0, 1
# band: far pairs dropped; "+shift": band-edge continuity shift of the far query
LONG_MODES = {"fi": BF_LONG_FI, "pa": BF_LONG_PA, "band": BF_LONG_NONE,
              "fi+shift": BF_LONG_FI | BF_LONG_SHIFT, "pa+shift": BF_LONG_PA | BF_LONG_SHIFT}
_DTYPES = {torch.bfloat16: BF_DTYPE_BF16, torch.float32: BF_DTYPE_FP32}

EXPORTED = ("bifocal_s_of_L", "bifocal_workspace_bytes", "bifocal_prefill", "bifocal_decode",
            "bifocal_chunk_workspace_bytes", "bifocal_prefill_chunk", "bifocal_prefill_chunk_paged",
            "bifocal_decode_paged", "plain_attention_ref_gpu", "bifocal_rope_prefill", "bifocal_rope_append",
            "bifocal_rope_prefill_paged", "bifocal_rope_append_paged",
            "bifocal_test_pair_map", "bifocal_last_error", "bifocal_decode_noalloc",
            "bifocal_test_angles", "bifocal_decode_stored", "bifocal_decode_stored_paged",
            "bifocal_chunk_store_bytes", "bifocal_prefill_chunk_stored",
            "bifocal_prefill_chunk_stored_paged")

_lib = None


class BifocalError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libbifocal error {code}: {msg}")
        self.code = code


def lib():
    """Load libbifocal.so (built in-tree); raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python -m rope_context_extension_bifocal_amd.csrc.build")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
        L.bifocal_s_of_L.restype = i64
        L.bifocal_s_of_L.argtypes = [i64, i64]
        L.bifocal_workspace_bytes.restype = sz
        L.bifocal_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32, i32]
        L.bifocal_prefill.restype = ctypes.c_int
        L.bifocal_prefill.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i64, i64, f64,
                                      i32, f32, p, sz, p]
        L.bifocal_chunk_workspace_bytes.restype = sz
        L.bifocal_chunk_workspace_bytes.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32]
        L.bifocal_prefill_chunk_paged.restype = ctypes.c_int
        L.bifocal_prefill_chunk_paged.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32,
                                                  i32, i32, i32, i64, i64, f64, i32, f32, p, sz, p]
        L.bifocal_chunk_store_bytes.restype = sz
        L.bifocal_chunk_store_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.bifocal_prefill_chunk_stored.restype = ctypes.c_int
        L.bifocal_prefill_chunk_stored.argtypes = [p, p, p, p, sz, p, p, p, p, p, p, p, i32, i32,
                                                   i32, i32, i32, i32, i64, i64, f64, i32, f32, p,
                                                   sz, p]
        L.bifocal_prefill_chunk_stored_paged.restype = ctypes.c_int
        L.bifocal_prefill_chunk_stored_paged.argtypes = [p, p, p, p, sz, p, p, p, p, p, p, p, p, i32,
                                                         i32, i32, i32, i32, i32, i32, i32, i64, i64,
                                                         f64, i32, f32, p, sz, p]
        L.bifocal_prefill_chunk.restype = ctypes.c_int
        L.bifocal_prefill_chunk.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                            i64, i64, f64, i32, f32, p, sz, p]
        L.bifocal_decode.restype = ctypes.c_int
        L.bifocal_decode.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64, i64,
                                     f64, i32, f32, p, sz, p]
        L.bifocal_decode_stored.restype = ctypes.c_int
        L.bifocal_decode_stored.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                            i64, i64, f64, i32, f32, p, sz, p]
        L.bifocal_decode_stored_paged.restype = ctypes.c_int
        L.bifocal_decode_stored_paged.argtypes = [p, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32,
                                                  i32, i32, i32, i32, i64, i64, f64, i32, f32, p,
                                                  sz, p]
        L.bifocal_decode_noalloc.restype = ctypes.c_int
        L.bifocal_decode_noalloc.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64,
                                             i64, f64, i32, f32, p]
        L.bifocal_decode_paged.restype = ctypes.c_int
        L.bifocal_decode_paged.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                           i32, i64, i64, f64, i32, f32, p, sz, p]
        L.plain_attention_ref_gpu.restype = ctypes.c_int
        L.plain_attention_ref_gpu.argtypes = [i32, p, p, p, p, p, p, i32, i32, i32, i32, i32,
                                              i32, f32, p, sz, p]
        L.bifocal_rope_prefill.restype = ctypes.c_int
        L.bifocal_rope_prefill.argtypes = [p, p, p, p, p, p, p, i32, p, p, i32, i32, i32, i32,
                                           i32, f64, p]
        L.bifocal_rope_prefill_paged.restype = ctypes.c_int
        L.bifocal_rope_prefill_paged.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, p, p, i32,
                                                 i32, i32, i32, i32, f64, p]
        L.bifocal_rope_append_paged.restype = ctypes.c_int
        L.bifocal_rope_append_paged.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, p, i32, i32, i32,
                                                i32, i32, f64, p]
        L.bifocal_rope_append.restype = ctypes.c_int
        L.bifocal_rope_append.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f64,
                                          p]
        L.bifocal_test_pair_map.restype = ctypes.c_int
        L.bifocal_test_pair_map.argtypes = [i64, i64, i64, i32, p, p, p]
        L.bifocal_test_angles.restype = ctypes.c_int
        L.bifocal_test_angles.argtypes = [i32, p, i32, i64, i64, i64, f64, i32, p, p]
        L.bifocal_last_error.restype = ctypes.c_char_p
        L.bifocal_last_error.argtypes = []
        _lib = L
    return _lib


def _check(rc):
    if rc != BF_OK:
        raise BifocalError(rc, lib().bifocal_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _i32_array(vals):
    arr = (ctypes.c_int32 * len(vals))(*[int(x) for x in vals])
    return arr


def s_of_L(L, w_pre):
    return int(lib().bifocal_s_of_L(int(L), int(w_pre)))


def workspace_bytes(phase, batch, tokens, n_heads_q, n_heads_kv, head_dim=128,
                    dtype=torch.bfloat16):
    return int(lib().bifocal_workspace_bytes(int(phase), int(batch), int(tokens), int(n_heads_q),
                                             int(n_heads_kv), int(head_dim), _DTYPES[dtype]))


def alloc_workspace(nbytes, device):
    """Device workspace (256-byte aligned: the caching allocator aligns to 512)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _scale(softmax_scale, D):
    return float(softmax_scale) if softmax_scale is not None else 1.0 / math.sqrt(D)


def prefill(q, k, v, cu_seqlens, w0, w_pre, rope_theta, long_mode="fi", softmax_scale=None,
            return_lse=False, out=None, lse=None, workspace=None, stream=None):
    """Bifocal causal prefill. q [Hq,T,D], k/v [Hkv,T,D] on the GPU (bf16 or fp32),
    cu_seqlens a host list [B+1]. Returns o (and lse [Hq,T] fp32)."""
    Hq, T, D = q.shape
    Hkv = k.shape[0]
    B = len(cu_seqlens) - 1
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(BF_PHASE_PREFILL, B, T, Hq, Hkv, D, q.dtype),
                                    q.device)
    cu = _i32_array(cu_seqlens)
    _check(lib().bifocal_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), cu, B, Hq, Hkv,
                                 D, _DTYPES[q.dtype], int(w0), int(w_pre), float(rope_theta),
                                 LONG_MODES[long_mode], _scale(softmax_scale, D), _ptr(workspace),
                                 workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def chunk_workspace_bytes(batch, q_tokens, kv_tokens, n_heads_q, n_heads_kv, head_dim=128,
                          dtype=torch.bfloat16, paged=False):
    return int(lib().bifocal_chunk_workspace_bytes(int(batch), int(q_tokens), int(kv_tokens),
                                                   int(n_heads_q), int(n_heads_kv), int(head_dim),
                                                   _DTYPES[dtype], int(bool(paged))))


def prefill_chunk(q, k_cache, v_cache, cu_q, seqlens, w0, w_pre, rope_theta, long_mode="fi",
                  softmax_scale=None, s_len=None, return_lse=False, out=None, lse=None,
                  workspace=None, stream=None):
    """Multi-token queries against a KV cache (chunked prefill). q [Hq,Tq,D]
    packed by cu_q (host list [B+1]); caches [B,Hkv,cap,D] holding seqlens[b]
    keys, the chunk's own last; the queries of b sit at positions
    seqlens[b] - Lq_b .. seqlens[b] - 1. s from s_len[b] (default seqlens[b])."""
    Hq, Tq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    B = len(cu_q) - 1
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(chunk_workspace_bytes(B, Tq, sum(int(n) for n in seqlens), Hq,
                                                          Hkv, D, q.dtype), q.device)
    cu = _i32_array(cu_q)
    sl = _i32_array(seqlens)
    sls = _i32_array(s_len) if s_len is not None else None
    _check(lib().bifocal_prefill_chunk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse),
                                       cu, sl, sls, B, cap, Hq, Hkv, D, _DTYPES[q.dtype], int(w0),
                                       int(w_pre), float(rope_theta), LONG_MODES[long_mode],
                                       _scale(softmax_scale, D), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def chunk_store_bytes(batch, cache_capacity, n_heads_kv, head_dim=128, dtype=torch.bfloat16):
    return lib().bifocal_chunk_store_bytes(batch, cache_capacity, n_heads_kv, head_dim,
                                           _DTYPES[dtype])


class ChunkStore:
    """Caller-kept state of prefill_chunk_stored for one cache [B,Hkv,cap,D]
    (or, for prefill_chunk_stored_paged, a page pool [pages,Hkv,page,D] with
    `batch` and `max_pages_per_seq` given): an opaque device buffer holding
    k'' and V^T of the cache positions and, per sequence, how many keys it
    holds (keys) and for which s (s). The library updates keys and s."""

    def __init__(self, k_cache, batch=None, max_pages_per_seq=None):
        if batch is None:
            B, Hkv, cap, D = k_cache.shape
        else:  # a page pool: capacity = pages per sequence x page size
            B, Hkv, D = int(batch), k_cache.shape[1], k_cache.shape[3]
            cap = int(max_pages_per_seq) * k_cache.shape[2]
        n = chunk_store_bytes(B, cap, Hkv, D, k_cache.dtype)
        if n == 0:
            raise ValueError("no chunk store for a cache of shape %s" % (tuple(k_cache.shape),))
        self.buf = torch.empty(n, dtype=torch.uint8, device=k_cache.device)
        self.keys = (ctypes.c_int32 * B)()
        self.s = (ctypes.c_int32 * B)()

    def reset(self, b=None, keys=0):
        """Forget stored keys from `keys` on (all sequences, or sequence b),
        e.g. after rewriting cache positions from `keys` on."""
        for i in (range(len(self.keys)) if b is None else [b]):
            self.keys[i] = min(self.keys[i], int(keys))


def prefill_chunk_stored(q, k_cache, v_cache, store, cu_q, seqlens, w0, w_pre, rope_theta,
                         long_mode="fi", softmax_scale=None, s_len=None, return_lse=False,
                         out=None, lse=None, workspace=None, stream=None):
    """prefill_chunk with a ChunkStore: k'' and V^T are formed only for the
    keys the store does not hold yet. Bitwise prefill_chunk when both run with
    their default workspaces (the same key splits); the default here holds
    q'' and the split partials only."""
    Hq, Tq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    B = len(cu_q) - 1
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(chunk_workspace_bytes(B, Tq, Tq, Hq, Hkv, D, q.dtype), q.device)
    cu = _i32_array(cu_q)
    sl = _i32_array(seqlens)
    sls = _i32_array(s_len) if s_len is not None else None
    _check(lib().bifocal_prefill_chunk_stored(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(store.buf), store.buf.numel(), _ptr(o),
        _ptr(lse), cu, sl, sls, store.keys, store.s, B, cap, Hq, Hkv, D, _DTYPES[q.dtype], int(w0),
        int(w_pre), float(rope_theta), LONG_MODES[long_mode], _scale(softmax_scale, D),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def prefill_chunk_stored_paged(q, k_pages, v_pages, block_table, store, cu_q, seqlens, w0, w_pre,
                               rope_theta, long_mode="fi", softmax_scale=None, s_len=None,
                               return_lse=False, out=None, lse=None, workspace=None, stream=None):
    """prefill_chunk_paged with a ChunkStore (made with batch and
    max_pages_per_seq); bitwise prefill_chunk_paged with the same workspace
    size (both defaults are the same)."""
    Hq, Tq, D = q.shape
    Hkv, page = k_pages.shape[1], k_pages.shape[2]
    num_pages = k_pages.shape[0]
    B = len(cu_q) - 1
    maxp = block_table.shape[1]
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(chunk_workspace_bytes(B, Tq, sum(int(n) for n in seqlens), Hq,
                                                          Hkv, D, q.dtype, paged=True), q.device)
    cu = _i32_array(cu_q)
    sl = _i32_array(seqlens)
    sls = _i32_array(s_len) if s_len is not None else None
    _check(lib().bifocal_prefill_chunk_stored_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(store.buf), store.buf.numel(), _ptr(o),
        _ptr(lse), _ptr(block_table), cu, sl, sls, store.keys, store.s, B, page, maxp, num_pages, Hq,
        Hkv, D, _DTYPES[q.dtype], int(w0), int(w_pre), float(rope_theta), LONG_MODES[long_mode],
        _scale(softmax_scale, D), _ptr(workspace), workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def prefill_chunk_paged(q, k_pages, v_pages, block_table, cu_q, seqlens, w0, w_pre, rope_theta,
                        long_mode="fi", softmax_scale=None, s_len=None, return_lse=False, out=None,
                        lse=None, workspace=None, stream=None):
    """prefill_chunk over a paged cache: pages [num_pages,Hkv,page,D] and a
    device int32 block table [B,max_pages]."""
    Hq, Tq, D = q.shape
    num_pages, Hkv, page = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    B = len(cu_q) - 1
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(chunk_workspace_bytes(B, Tq, sum(int(n) for n in seqlens), Hq,
                                                          Hkv, D, q.dtype, paged=True), q.device)
    cu = _i32_array(cu_q)
    sl = _i32_array(seqlens)
    sls = _i32_array(s_len) if s_len is not None else None
    _check(lib().bifocal_prefill_chunk_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o),
                                             _ptr(lse), _ptr(block_table), cu, sl, sls, B, page,
                                             block_table.shape[1], num_pages, Hq, Hkv, D,
                                             _DTYPES[q.dtype], int(w0), int(w_pre),
                                             float(rope_theta), LONG_MODES[long_mode],
                                             _scale(softmax_scale, D), _ptr(workspace),
                                             workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def plain_prefill(q, k, v, cu_seqlens, softmax_scale=None, return_lse=False, out=None, lse=None,
                  workspace=None, stream=None):
    """Plain causal attention on the same engine (bifocal features compiled out)."""
    Hq, T, D = q.shape
    Hkv = k.shape[0]
    B = len(cu_seqlens) - 1
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(BF_PHASE_PREFILL, B, T, Hq, Hkv, D, q.dtype),
                                    q.device)
    cu = _i32_array(cu_seqlens)
    _check(lib().plain_attention_ref_gpu(BF_PHASE_PREFILL, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                         _ptr(lse), cu, B, 0, Hq, Hkv, D, _DTYPES[q.dtype],
                                         _scale(softmax_scale, D), _ptr(workspace),
                                         workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def decode(q, k_cache, v_cache, seqlens, w0, w_pre, rope_theta, long_mode="fi",
           softmax_scale=None, return_lse=False, out=None, lse=None, workspace=None, stream=None):
    """Bifocal single-token decode. q [B,Hq,D], caches [B,Hkv,cap,D] bf16 on the GPU,
    seqlens a host list [B] (valid keys including the new token's)."""
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(BF_PHASE_DECODE, B, max(seqlens), Hq, Hkv, D,
                                                    q.dtype), q.device)
    sl = _i32_array(seqlens)
    _check(lib().bifocal_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), sl, B,
                                cap, Hq, Hkv, D, _DTYPES[q.dtype], int(w0), int(w_pre),
                                float(rope_theta), LONG_MODES[long_mode],
                                _scale(softmax_scale, D), _ptr(workspace), workspace.numel(),
                                _stream(stream)))
    return (o, lse) if return_lse else o


class DecodeStore:
    """Caller-kept state of decode_stored for one cache: the far-key store k2
    (the cache's shape: [B,Hkv,cap,D], or a page pool [pages,Hkv,page,D] with
    `batch` given) and, per sequence, how many keys it holds (keys) and for
    which s (s). The library updates keys and s."""

    def __init__(self, k_cache, batch=None):
        self.k2 = torch.empty_like(k_cache)
        B = k_cache.shape[0] if batch is None else int(batch)  # a page pool needs `batch`
        self.keys = (ctypes.c_int32 * B)()
        self.s = (ctypes.c_int32 * B)()

    def reset(self, b=None, keys=0):
        """Forget stored keys from `keys` on (all sequences, or sequence b),
        e.g. after rewriting cache positions from `keys` on."""
        for i in (range(len(self.keys)) if b is None else [b]):
            self.keys[i] = min(self.keys[i], int(keys))


def decode_stored(q, k_cache, v_cache, store, seqlens, w0, w_pre, rope_theta, long_mode="fi",
                  softmax_scale=None, return_lse=False, out=None, lse=None, workspace=None,
                  stream=None):
    """bifocal_decode reading the k'' of far keys from a DecodeStore and
    adding the ones it forms; bitwise the result of decode()."""
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(BF_PHASE_DECODE, B, max(seqlens), Hq, Hkv, D,
                                                    q.dtype), q.device)
    sl = _i32_array(seqlens)
    _check(lib().bifocal_decode_stored(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(store.k2), _ptr(o),
                                       _ptr(lse), sl, store.keys, store.s, B, cap, Hq, Hkv, D,
                                       _DTYPES[q.dtype], int(w0), int(w_pre), float(rope_theta),
                                       LONG_MODES[long_mode], _scale(softmax_scale, D),
                                       _ptr(workspace), workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def decode_stored_paged(q, k_pages, v_pages, block_table, store, seqlens, w0, w_pre, rope_theta,
                        long_mode="fi", softmax_scale=None, return_lse=False, out=None, lse=None,
                        workspace=None, stream=None):
    """decode_stored over a paged cache; `store` is a DecodeStore made from
    k_pages (its k2 is a page pool under the same block table)."""
    B, Hq, D = q.shape
    num_pages, Hkv, page = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(BF_PHASE_DECODE, B, max(seqlens), Hq, Hkv, D,
                                                    q.dtype), q.device)
    sl = _i32_array(seqlens)
    _check(lib().bifocal_decode_stored_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(store.k2), _ptr(o), _ptr(lse), _ptr(block_table),
        sl, store.keys, store.s, B, page, block_table.shape[1], num_pages, Hq, Hkv, D,
        _DTYPES[q.dtype], int(w0), int(w_pre), float(rope_theta), LONG_MODES[long_mode],
        _scale(softmax_scale, D), _ptr(workspace), workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def decode_noalloc(q, k_cache, v_cache, seqlens, w0, w_pre, rope_theta, long_mode="fi",
                   softmax_scale=None, return_lse=False, out=None, lse=None, stream=None):
    """bifocal_decode without a workspace: the library's own per-GPU scratch
    holds the split partials (calls that overlap on one GPU race). Pass `out`
    (and `lse`) to allocate nothing on this side either."""
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    sl = _i32_array(seqlens)
    _check(lib().bifocal_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse),
                                        sl, B, cap, Hq, Hkv, D, _DTYPES[q.dtype], int(w0),
                                        int(w_pre), float(rope_theta), LONG_MODES[long_mode],
                                        _scale(softmax_scale, D), _stream(stream)))
    return (o, lse) if return_lse else o


def decode_paged(q, k_pages, v_pages, block_table, seqlens, w0, w_pre, rope_theta, long_mode="fi",
                 softmax_scale=None, return_lse=False, out=None, lse=None, workspace=None,
                 stream=None):
    """Bifocal decode over a paged cache: pages [num_pages,Hkv,page,D] bf16,
    block_table a device int32 tensor [B,max_pages]."""
    B, Hq, D = q.shape
    num_pages, Hkv, page = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(BF_PHASE_DECODE, B, max(seqlens), Hq, Hkv, D,
                                                    q.dtype), q.device)
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    sl = _i32_array(seqlens)
    _check(lib().bifocal_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o), _ptr(lse),
                                      _ptr(block_table), sl, B, page, block_table.shape[1],
                                      num_pages, Hq, Hkv, D, _DTYPES[q.dtype], int(w0), int(w_pre),
                                      float(rope_theta), LONG_MODES[long_mode],
                                      _scale(softmax_scale, D), _ptr(workspace), workspace.numel(),
                                      _stream(stream)))
    return (o, lse) if return_lse else o


def plain_decode(q, k_cache, v_cache, seqlens, softmax_scale=None, return_lse=False, out=None,
                 lse=None, workspace=None, stream=None):
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(BF_PHASE_DECODE, B, max(seqlens), Hq, Hkv, D,
                                                    q.dtype), q.device)
    sl = _i32_array(seqlens)
    _check(lib().plain_attention_ref_gpu(BF_PHASE_DECODE, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(o), _ptr(lse), sl, B, cap, Hq, Hkv, D,
                                         _DTYPES[q.dtype], _scale(softmax_scale, D),
                                         _ptr(workspace), workspace.numel(), _stream(stream)))
    return (o, lse) if return_lse else o


def rope_prefill(q_raw, k_raw, cu_seqlens, rope_theta, v=None, k_cache=None, v_cache=None,
                 q_out=None, k_out=None, write_k=True, pos0=None, stream=None):
    """Original RoPE on raw packed q [Hq,T,D] and k [Hkv,T,D] at sequence-relative
    positions, starting at pos0[b] (default 0; a chunk after a cached prefix
    starts at the prefix length). With k_cache / v_cache [B,Hkv,cap,D] (and v
    [Hkv,T,D]) the rotated keys and the values are also written to the cache at
    those positions. Returns (q', k') (k' is None when write_k is False and a
    cache is given)."""
    Hq, T, D = q_raw.shape
    Hkv = k_raw.shape[0]
    B = len(cu_seqlens) - 1
    qo = q_out if q_out is not None else torch.empty_like(q_raw)
    ko = k_out if k_out is not None else (torch.empty_like(k_raw) if write_k or k_cache is None
                                          else None)
    cap = k_cache.shape[2] if k_cache is not None else 0
    cu = _i32_array(cu_seqlens)
    p0 = _i32_array(pos0) if pos0 is not None else None
    _check(lib().bifocal_rope_prefill(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(qo), _ptr(ko),
                                      _ptr(k_cache), _ptr(v_cache), cap, cu, p0, B, Hq, Hkv, D,
                                      _DTYPES[q_raw.dtype], float(rope_theta), _stream(stream)))
    return qo, ko


def rope_append(q_raw, k_raw, v_new, k_cache, v_cache, seqlens, rope_theta, q_out=None,
                stream=None):
    """One decode step's raw q [B,Hq,D] and new k, v [B,Hkv,D]: q' at position
    seqlens[b] - 1 is returned, k' and v go to the caches at that position."""
    B, Hq, D = q_raw.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    qo = q_out if q_out is not None else torch.empty_like(q_raw)
    sl = _i32_array(seqlens)
    _check(lib().bifocal_rope_append(_ptr(q_raw), _ptr(k_raw), _ptr(v_new), _ptr(qo),
                                     _ptr(k_cache), _ptr(v_cache), sl, B, cap, Hq, Hkv, D,
                                     _DTYPES[q_raw.dtype], float(rope_theta), _stream(stream)))
    return qo


def rope_prefill_paged(q_raw, k_raw, v, cu_seqlens, rope_theta, k_pages, v_pages, block_table,
                       q_out=None, k_out=None, write_k=False, pos0=None, stream=None):
    """rope_prefill with the cache fill going to a paged cache (pages
    [num_pages,Hkv,page,D], device int32 block table [B,max_pages])."""
    Hq, T, D = q_raw.shape
    Hkv = k_raw.shape[0]
    B = len(cu_seqlens) - 1
    qo = q_out if q_out is not None else torch.empty_like(q_raw)
    ko = k_out if k_out is not None else (torch.empty_like(k_raw) if write_k else None)
    cu = _i32_array(cu_seqlens)
    p0 = _i32_array(pos0) if pos0 is not None else None
    _check(lib().bifocal_rope_prefill_paged(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(qo), _ptr(ko),
                                            _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                            k_pages.shape[2], block_table.shape[1], k_pages.shape[0],
                                            cu, p0, B, Hq, Hkv, D, _DTYPES[q_raw.dtype],
                                            float(rope_theta), _stream(stream)))
    return qo, ko


def rope_append_paged(q_raw, k_raw, v_new, k_pages, v_pages, block_table, seqlens, rope_theta,
                      q_out=None, stream=None):
    """rope_append into a paged cache."""
    B, Hq, D = q_raw.shape
    Hkv = k_raw.shape[1]
    qo = q_out if q_out is not None else torch.empty_like(q_raw)
    sl = _i32_array(seqlens)
    _check(lib().bifocal_rope_append_paged(_ptr(q_raw), _ptr(k_raw), _ptr(v_new), _ptr(qo),
                                           _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                           k_pages.shape[2], block_table.shape[1], k_pages.shape[0],
                                           sl, B, Hq, Hkv, D, _DTYPES[q_raw.dtype],
                                           float(rope_theta), _stream(stream)))
    return qo


def test_pair_map(L, w0, w_pre, long_mode="fi", device="cuda", fill=-1):
    """The bf16 tile kernel's pair classification (1 local, 2 far, 3 both, 0
    neither; `fill` where no wave covers the pair) and the prep pass's
    (phi(p) - p) * s numerators (test hook)."""
    br = torch.full((L, L), fill, dtype=torch.int8, device=device)
    num = torch.empty((L,), dtype=torch.int64, device=device)
    _check(lib().bifocal_test_pair_map(int(L), int(w0), int(w_pre), LONG_MODES[long_mode],
                                       _ptr(br), _ptr(num), _stream(None)))
    torch.cuda.synchronize()
    return br, num


def test_angles(which, positions, L, w0, w_pre, rope_theta, long_mode="fi", device="cuda"):
    """fp32 (cos, sin) [n, 64, 2] the kernels rotate with at `positions`
    (which: 0 prefill queries, 1 prefill keys, 2 decode keys of an L-key call,
    3 decode queries at position p of a (p + 1)-key call) (test hook)."""
    pos = (ctypes.c_int64 * len(positions))(*[int(x) for x in positions])
    cs = torch.empty((len(positions), 64, 2), dtype=torch.float32, device=device)
    _check(lib().bifocal_test_angles(int(which), pos, len(positions), int(L), int(w0), int(w_pre),
                                     float(rope_theta), LONG_MODES[long_mode], _ptr(cs),
                                     _stream(None)))
    torch.cuda.synchronize()
    return cs
