/*
 * libbifocal -- Dynamic Bifocal RoPE attention for AMD MI355X (gfx950).
 *
 * What is computed (Jet-Long, arXiv 2607.07740, as described on the pages):
 *   - s(L) = max(1, ceil(L / w_pre)), one factor per sequence of length L
 *     [Jet-Long promo script (papers.ananclaw.com), section 4 storyboard,
 *      scene-2 formula; ai-feeds.com summary, "方法 / 关键模块" item 2].
 *   - For a query at position i and a key at position j <= i of the same
 *     sequence, the pair is LOCAL when i - j < w0 and is scored with the
 *     model's original RoPE; otherwise it is FAR and is scored with RoPE at
 *     the scaled positions phi(p): p / s (frequency interpolation) or
 *     floor(p / s) (position aliasing) [ai-feeds.com summary, "关键模块"
 *     item 1 and "关键发现", ablation bullet].
 *   - Softmax over j <= i with every pair counted once: the inclusion-
 *     exclusion merge of the full scaled branch, minus its local band, plus
 *     the band under original RoPE [seventnews.com (FR), fusion paragraph].
 *   - Inputs q, k are the cache form: they already carry original RoPE at
 *     their absolute positions. The far branch is reached by a correction
 *     rotation R(theta_m * (phi(p) - p)) applied on the fly to cached keys
 *     and to the query [ai-feeds.com summary, "关键模块" item 3].
 * Rotary pairs are half-split (m, m + D/2), theta_m = rope_theta^(-2m/D).
 *
 * Conventions for every entry point:
 *   - Tensors are caller-owned DEVICE memory and must stay valid until the
 *     work enqueued on `stream` completes. Host arrays (cu_seqlens_host,
 *     seqlens_host, ...) are read, and the counters of the far-key and
 *     chunk stores (store_keys_host, store_s_host) written, before the call
 *     returns.
 *   - All work is enqueued on `stream` (a hipStream_t, NULL = default
 *     stream). The library never synchronises and keeps no state between
 *     calls except a thread-local error string.
 *   - Scratch memory lives only in the caller's `workspace` (device memory,
 *     256-byte aligned, at least bifocal_workspace_bytes(...) bytes); its
 *     contents on entry do not matter. Calls that run concurrently need
 *     distinct workspaces.
 *   - Every argument is validated before the first HIP call: on any error
 *     nothing is launched and outputs are untouched.
 *   - Returns BF_OK (0) or a negative code; bifocal_last_error() explains.
 *   - Output is bitwise reproducible for the same inputs and device.
 */
#ifndef BIFOCAL_H
#define BIFOCAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define BF_OK 0
#define BF_ERR_INVALID_ARG (-1) /* null pointer, non-positive size, Hq % Hkv != 0,
                                   w0 < 0, w_pre < 1, bad lengths, theta <= 1, bad enum */
#define BF_ERR_UNSUPPORTED (-2) /* head_dim != 128, fp32 decode */
#define BF_ERR_WORKSPACE (-3)   /* workspace NULL, too small or misaligned */
#define BF_ERR_HIP (-4)         /* a HIP launch failed; see bifocal_last_error() */

/* element types of q, k, v, o (and the caches) */
#define BF_DTYPE_BF16 0
#define BF_DTYPE_FP32 1

/* long-branch position map phi(p) */
#define BF_LONG_FI 0 /* frequency interpolation: phi(p) = p / s */
#define BF_LONG_PA 1 /* position aliasing:       phi(p) = floor(p / s) */
#define BF_LONG_SHIFT 4 /* flag, OR-ed into BF_LONG_FI / BF_LONG_PA: band-edge continuity
                           shift. The far query sits at phi(p) + w0 - phi(w0) (keys stay at
                           phi(j)). A far pair at distance exactly w0 then sees relative
                           position w0, as the band does one step closer: for FI always,
                           for PA when s divides w0 or the key is at position 0 (otherwise
                           floor(i/s) - floor((i-w0)/s) may differ from floor(w0/s) by one)
                           [seventnews.com (FR), fusion paragraph: the correction re-aligns
                           the phases of the two branches]. Off by default. */
#define BF_LONG_NONE 2 /* band only: far pairs are dropped, i.e. sliding-window attention
                          over the w0 most recent keys with original RoPE (w0 >= 1; w_pre
                          unused), the sliding-window layers of a hybrid model */

/* phases for the workspace query and the plain reference */
#define BF_PHASE_PREFILL 0
#define BF_PHASE_DECODE 1

/*
 * s(L) = max(1, ceil(L / w_pre)) in 64-bit integers; -1 if L < 1 or
 * w_pre < 1. Host only. [promo script, storyboard scene-2 formula]
 */
int64_t bifocal_s_of_L(int64_t L, int64_t w_pre);

/*
 * Workspace bytes needed by bifocal_prefill / bifocal_decode /
 * plain_attention_ref_gpu for the given phase and sizes.
 *   PREFILL: `tokens` = total packed tokens T = cu_seqlens[batch].
 *   DECODE:  `tokens` = the largest seqlens[b] of the call.
 * The same figure covers both the bifocal and the plain call of a phase.
 * PREFILL holds 256 bytes of work-item counters (launches of 1024 or more
 * work items run persistent workgroups that claim their items), V^T (padded
 * per sequence to 64 keys), the corrected queries q'' and the corrected keys
 * k'' in the input dtype: about
 * (Hq + 2 Hkv) x T x head_dim elements, 1.5 GiB for a 131072-token bf16
 * prefill with 32 query / 8 KV heads (k'' and q'' are formed once per call
 * instead of on every re-read of a key tile). DECODE holds the split
 * partials: batch x Hq x S x 520 bytes, S = max(129, ceil(tokens / 4032) + 1),
 * 2.1 MB for one 131073-key sequence with 32 query heads.
 * Returns 0 for invalid arguments.
 */
size_t bifocal_workspace_bytes(int32_t phase, int32_t batch, int64_t tokens, int32_t n_heads_q,
                               int32_t n_heads_kv, int32_t head_dim, int32_t dtype);

/*
 * Causal bifocal prefill over a packed ragged batch.
 *   q, o : [n_heads_q,  T, head_dim]   dtype (bf16 or fp32), head-major,
 *                                      head_dim contiguous
 *   k, v : [n_heads_kv, T, head_dim]   same dtype
 *   lse  : [n_heads_q, T] fp32 natural-log row log-sum-exp, or NULL
 *   cu_seqlens_host : host int32 [batch + 1], cu[0] = 0, strictly
 *          increasing; sequence b is tokens cu[b] .. cu[b+1]-1, its
 *          positions restart at 0 and it gets its own s(L_b).
 *   w0 >= 0 local window (w0 = 0: every pair far; w0 >= L: plain RoPE),
 *   w_pre >= 1 pretrained window, rope_theta > 1 RoPE base,
 *   long_mode BF_LONG_FI or BF_LONG_PA (either with BF_LONG_SHIFT OR-ed
 *   in), or BF_LONG_NONE for the band-only special case (needs w0 >= 1),
 *   softmax_scale > 0 (both branches).
 * Query head h reads KV head h / (n_heads_q / n_heads_kv).
 * [ai-feeds.com summary, "方法": inputs are L and the pretrained RoPE
 *  configuration, the output is the attention output of the sequence;
 *  "关键发现": the two long-branch strategies; band only: ai-feeds.com
 *  summary, "核心洞察" third bullet, and seventnews.com (FR), "Généralisation
 *  aux architectures d'attention hybrides": sliding-window and global
 *  attention layers coexist in hybrid models]
 */
int bifocal_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_host, int32_t batch, int32_t n_heads_q,
                    int32_t n_heads_kv, int32_t head_dim, int32_t dtype, int64_t w0,
                    int64_t w_pre, double rope_theta, int32_t long_mode, float softmax_scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes of bifocal_prefill_chunk (paged = 0) and
 * bifocal_prefill_chunk_paged (paged = 1): q_tokens = cu_q[batch] (the packed
 * queries), kv_tokens = the sum of seqlens[b] (the keys the call reads).
 * For bf16 chunks too short to fill the GPU with work items (fewer than
 * about 1024 query rows per KV head group), the size includes room for up to
 * 8 key splits per item: partial outputs (fp32) and their log-sum-exp,
 * 516 bytes per (split, query head, query token).
 * Returns 0 for invalid arguments (also kv_tokens < q_tokens).
 */
size_t bifocal_chunk_workspace_bytes(int32_t batch, int64_t q_tokens, int64_t kv_tokens,
                                     int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                                     int32_t dtype, int32_t paged);

/*
 * Multi-token queries against a KV cache (chunked prefill, a prompt suffix
 * after a cached prefix, speculative verification): the queries of sequence b
 * are its LAST Lq_b positions, N_b - Lq_b .. N_b - 1, and attend causally
 * (bottom-right aligned) to the N_b keys in the cache, the chunk's own keys
 * included (append them first, e.g. with bifocal_rope_prefill). Each row is
 * the bifocal_prefill row at its position, with s = s(s_len_host[b]) (or
 * s(N_b) when s_len_host is NULL: the length seen so far, as decode does).
 *   q, o             : [n_heads_q, Tq, head_dim] dtype, packed as in
 *                      bifocal_prefill, Tq = cu_q_host[batch]
 *   k_cache, v_cache : [batch, n_heads_kv, cache_capacity, head_dim] dtype,
 *                      ORIGINAL RoPE at their positions; entries past N_b
 *                      are never used
 *   lse              : [n_heads_q, Tq] fp32 or NULL
 *   cu_q_host        : host int32 [batch + 1], cu_q[0] = 0, strictly
 *                      increasing (Lq_b = cu_q[b+1] - cu_q[b] >= 1)
 *   seqlens_host     : host int32 [batch], Lq_b <= N_b <= cache_capacity
 *   s_len_host       : host int32 [batch] or NULL; s_len[b] >= N_b (pass
 *                      the full prompt length to reproduce a one-shot
 *                      bifocal_prefill of that prompt chunk by chunk)
 *   workspace        : bifocal_chunk_workspace_bytes(batch, Tq, sum N_b, ..., 0)
 * Other arguments as bifocal_prefill (bf16 or fp32; every long_mode).
 * With Lq_b = N_b and s_len = NULL this is bifocal_prefill of the cached
 * sequences; with Lq_b = 1 it is bifocal_decode.
 * Key splits (bf16): when a launch has too few work items (row blocks x KV
 * heads) for the GPU, each item's key tiles are split into up to 8 parts,
 * run as separate workgroups, and merged by their log-sum-exp (a second
 * kernel) before O and lse are written. The split count follows from the
 * shapes and from the workspace: a workspace that holds the base layout but
 * not the partials runs unsplit. Split results are deterministic but not
 * bitwise those of an unsplit call (the merge rounds differently).
 * [mufans.github.io wiki, Jet-Long Dynamic RoPE, "可执行建议": pairing the
 *  method with prompt caching; ai-feeds.com summary, "关键模块" item 3: the
 *  correction rotation applied to cached keys]
 */
int bifocal_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* o,
                          float* lse, const int32_t* cu_q_host, const int32_t* seqlens_host,
                          const int32_t* s_len_host, int32_t batch, int32_t cache_capacity,
                          int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t dtype,
                          int64_t w0, int64_t w_pre, double rope_theta, int32_t long_mode,
                          float softmax_scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * bifocal_prefill_chunk over a PAGED KV cache: the same computation and
 * arguments, with the cache split into fixed-size pages.
 *   k_pages, v_pages : [num_pages, n_heads_kv, page_size, head_dim] dtype
 *   block_table      : DEVICE int32 [batch, max_pages_per_seq]; keys
 *                      p * page_size .. (p + 1) * page_size - 1 of sequence b
 *                      are in page block_table[b][p] (entries clamped to
 *                      [0, num_pages - 1]; only pages holding keys below N_b
 *                      are read)
 *   page_size        : a power of two, 1 <= page_size <= 2^20
 *   seqlens_host     : Lq_b <= N_b <= max_pages_per_seq * page_size
 *   workspace        : bifocal_chunk_workspace_bytes(..., paged = 1)
 * The keys are gathered once per call into a packed copy in the workspace,
 * so the result is bitwise that of bifocal_prefill_chunk on a contiguous
 * cache holding the same keys (each call given the workspace size its
 * bifocal_chunk_workspace_bytes returns, so that both split the same way).
 */
int bifocal_prefill_chunk_paged(const void* q, const void* k_pages, const void* v_pages, void* o,
                                float* lse, const int32_t* block_table, const int32_t* cu_q_host,
                                const int32_t* seqlens_host, const int32_t* s_len_host,
                                int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                                int32_t num_pages, int32_t n_heads_q, int32_t n_heads_kv,
                                int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                                double rope_theta, int32_t long_mode, float softmax_scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the store of bifocal_prefill_chunk_stored for `batch` sequences
 * of a cache with cache_capacity keys (max_pages_per_seq * page_size for the
 * paged form) and n_heads_kv KV heads (k'' and V^T of
 * every cache position, padded to 64 keys). Returns 0 for invalid arguments
 * and when 64 sequences x n_heads_kv x cache_capacity (rounded up to 64)
 * exceed 2^31 - 1 key rows.
 */
size_t bifocal_chunk_store_bytes(int32_t batch, int32_t cache_capacity, int32_t n_heads_kv,
                                 int32_t head_dim, int32_t dtype);

/*
 * bifocal_prefill_chunk with a caller-kept store of the per-key operands the
 * call would otherwise rebuild for the whole cache: k''_j = R(theta_m (phi(j)
 * - j)) k'_j, which depends only on j and s, and V^T. A call then forms them
 * only for the keys appended since the store was filled, so successive
 * chunks of one long prompt (s fixed by s_len) cost what their new keys
 * cost [mufans.github.io wiki, Jet-Long Dynamic RoPE, "可执行建议": pairing
 * the method with prompt caching; ai-feeds.com summary, "关键模块" item 3:
 * the correction rotation of cached keys; item 2: s from the length].
 *   store            : device, caller-owned, 256-byte aligned, at least
 *                      bifocal_chunk_store_bytes(batch, cache_capacity, ...)
 *                      bytes; its contents are the library's (opaque)
 *   store_bytes      : its size
 *   store_keys_host  : host int32 [batch], in/out: the store holds keys
 *                      0 .. P_b - 1 of sequence b for s = store_s_host[b]
 *   store_s_host     : host int32 [batch], in/out (start both at 0)
 *   workspace        : bifocal_chunk_workspace_bytes(batch, Tq, Tq, ..., 0)
 *                      suffices (q'' and the key-split partials only); the
 *                      split count follows the workspace as for
 *                      bifocal_prefill_chunk
 * Other arguments as bifocal_prefill_chunk on a contiguous cache, long_mode
 * FI or PA with or without BF_LONG_SHIFT; band-only (BF_LONG_NONE) returns
 * BF_ERR_UNSUPPORTED. If store_s_host[b] != s(s_len_b) (s(N_b) without
 * s_len) the store of sequence b counts as empty. The call forms k'' of keys
 * min(P_b, N_b) .. N_b - 1 and V^T from that key's 64-key tile on; after it
 * has been queued, store_keys_host[b] = N_b and store_s_host[b] = s. The
 * result is bitwise that of bifocal_prefill_chunk given a workspace of the
 * same size. The store belongs to one cache, long_mode and rope_theta: after
 * rewriting cache positions below P_b, lower store_keys_host[b] to the first
 * rewritten position; after changing the mode or rope_theta, set it to 0.
 * Validation errors leave outputs, store and both host arrays untouched.
 */
int bifocal_prefill_chunk_stored(const void* q, const void* k_cache, const void* v_cache,
                                 void* store, size_t store_bytes, void* o, float* lse,
                                 const int32_t* cu_q_host, const int32_t* seqlens_host,
                                 const int32_t* s_len_host, int32_t* store_keys_host,
                                 int32_t* store_s_host, int32_t batch, int32_t cache_capacity,
                                 int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                                 int32_t dtype, int64_t w0, int64_t w_pre, double rope_theta,
                                 int32_t long_mode, float softmax_scale, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * bifocal_prefill_chunk_stored over a PAGED KV cache: the arguments of
 * bifocal_prefill_chunk_paged plus the store and host arrays of
 * bifocal_prefill_chunk_stored. The store is sized by
 * bifocal_chunk_store_bytes(batch, max_pages_per_seq * page_size, ...) and
 * indexed by sequence and position (not by page). The call still gathers
 * into the workspace's packed copy the keys its local pass reads: from the
 * window start of the chunk's first query on (64-aligned; every key when s
 * = 1), plus any key without a stored k''.
 *   workspace        : bifocal_chunk_workspace_bytes(..., paged = 1), as for
 *                      bifocal_prefill_chunk_paged
 * The result is bitwise that of bifocal_prefill_chunk_paged given a workspace
 * of the same size (and of bifocal_prefill_chunk_stored on a contiguous cache
 * holding the same keys). Validation errors leave outputs, store and both
 * host arrays untouched.
 */
int bifocal_prefill_chunk_stored_paged(const void* q, const void* k_pages, const void* v_pages,
                                       void* store, size_t store_bytes, void* o, float* lse,
                                       const int32_t* block_table, const int32_t* cu_q_host,
                                       const int32_t* seqlens_host, const int32_t* s_len_host,
                                       int32_t* store_keys_host, int32_t* store_s_host,
                                       int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                                       int32_t num_pages, int32_t n_heads_q, int32_t n_heads_kv,
                                       int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                                       double rope_theta, int32_t long_mode, float softmax_scale,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Single-token bifocal decode over a KV cache (bf16 only).
 *   q, o             : [batch, n_heads_q, head_dim] bf16
 *   k_cache, v_cache : [batch, n_heads_kv, cache_capacity, head_dim] bf16,
 *                      keys stored with ORIGINAL RoPE at their positions
 *   lse              : [batch, n_heads_q] fp32 or NULL
 *   seqlens_host     : host int32 [batch], 1 <= N_b <= cache_capacity,
 *                      the number of valid keys INCLUDING the new token's
 *                      own (already appended); the query sits at position
 *                      N_b - 1 and s = s(N_b).
 * Result equals the last row of bifocal_prefill over the same N_b tokens;
 * long_mode BF_LONG_NONE reads only the keys N_b - w0 .. N_b - 1.
 * [promo script, voice-over: single-batch generation; ai-feeds.com summary,
 *  "关键模块" item 3: the correction rotation applied to cached keys]
 */
int bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                   const int32_t* seqlens_host, int32_t batch, int32_t cache_capacity,
                   int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t dtype,
                   int64_t w0, int64_t w_pre, double rope_theta, int32_t long_mode,
                   float softmax_scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bifocal_decode with a caller-kept store of corrected far keys, so that a
 * decode step rotates only the keys that became far since the store was
 * filled. The correction of key j, R(theta_m (phi(j) - j)), depends on j and
 * s alone, and s = s(N_b) stays the same over w_pre steps, so k'' of a far
 * key can be kept between steps [ai-feeds.com summary, "关键模块" item 3: the
 * correction rotation of cached keys; item 2: s from the length].
 *   k2_store         : [batch, n_heads_kv, cache_capacity, head_dim] bf16,
 *                      device, caller-owned, the layout of k_cache
 *   store_keys_host  : host int32 [batch], in/out: keys 0 .. P_b - 1 of
 *                      sequence b in k2_store hold k'' for s = store_s_host[b]
 *   store_s_host     : host int32 [batch], in/out (start both at 0)
 * Other arguments as bifocal_decode, long_mode FI or PA (with or without
 * BF_LONG_SHIFT); band-only (BF_LONG_NONE) returns BF_ERR_UNSUPPORTED.
 * If store_s_host[b] != s(N_b) the store of sequence b is treated as empty.
 * Far keys below min(P_b, N_b - w0), rounded down to a multiple of 16, are
 * read from k2_store; every other far key is rotated from k_cache and its k''
 * written to k2_store. When the call has been queued it sets
 * store_keys_host[b] = max(0, N_b - w0) (0 when s = 1) and store_s_host[b] =
 * s(N_b): the store as the stream leaves the call. The result is bitwise that
 * of bifocal_decode (the stored k'' are the values it forms on the fly). The
 * store belongs to one cache, long_mode and rope_theta: after rewriting cache
 * positions below P_b (a rollback), lower store_keys_host[b] to the first
 * rewritten position; after changing the mode or rope_theta, set it to 0.
 * Validation errors leave outputs and both host arrays untouched.
 */
int bifocal_decode_stored(const void* q, const void* k_cache, const void* v_cache, void* k2_store,
                          void* o, float* lse, const int32_t* seqlens_host, int32_t* store_keys_host,
                          int32_t* store_s_host, int32_t batch, int32_t cache_capacity,
                          int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t dtype,
                          int64_t w0, int64_t w_pre, double rope_theta, int32_t long_mode,
                          float softmax_scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * bifocal_decode_stored over a PAGED KV cache: the arguments of
 * bifocal_decode_paged plus the store of bifocal_decode_stored, which is a
 * page pool of its own with the shape of k_pages, addressed through the same
 * block_table ([num_pages, n_heads_kv, page_size, head_dim] bf16, device,
 * caller-owned). Result bitwise that of bifocal_decode_paged (and of
 * bifocal_decode_stored on a contiguous cache holding the same keys).
 */
int bifocal_decode_stored_paged(const void* q, const void* k_pages, const void* v_pages,
                                void* k2_pages, void* o, float* lse, const int32_t* block_table,
                                const int32_t* seqlens_host, int32_t* store_keys_host,
                                int32_t* store_s_host, int32_t batch, int32_t page_size,
                                int32_t max_pages_per_seq, int32_t num_pages, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t head_dim, int32_t dtype, int64_t w0,
                                int64_t w_pre, double rope_theta, int32_t long_mode,
                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * bifocal_decode without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, layouts, result (bitwise) and
 * validation as bifocal_decode, minus workspace / workspace_bytes. The split
 * partials live in a scratch array the library holds in device memory, 32 MiB
 * per GPU it runs on, kept until the process ends; a call whose partials
 * would not fit (batch x n_heads_q x splits x 520 bytes, splits = max(129,
 * ceil(max N / 4032) + 1)) returns BF_ERR_UNSUPPORTED before any HIP call.
 * The array is the current device's: `stream` must belong to it. Every call
 * on one GPU shares that GPU's array, so calls that overlap on one GPU (other
 * streams, other threads) race; serialise them. The call allocates nothing.
 */
int bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                           float* lse, const int32_t* seqlens_host, int32_t batch,
                           int32_t cache_capacity, int32_t n_heads_q, int32_t n_heads_kv,
                           int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                           double rope_theta, int32_t long_mode, float softmax_scale,
                           void* stream);

/*
 * bifocal_decode over a PAGED KV cache: the same computation and arguments as
 * bifocal_decode, with the cache split into fixed-size pages.
 *   k_pages, v_pages : [num_pages, n_heads_kv, page_size, head_dim] bf16
 *   block_table      : DEVICE int32 [batch, max_pages_per_seq]; keys
 *                      p * page_size .. (p + 1) * page_size - 1 of sequence b
 *                      are in page block_table[b][p] (entries are clamped to
 *                      [0, num_pages - 1]; only the pages that hold keys the
 *                      call reads need valid entries)
 *   page_size        : a power of two, 16 <= page_size <= 2^20
 *   seqlens_host     : as bifocal_decode, 1 <= N_b <= max_pages_per_seq *
 *                      page_size
 * The workspace is bifocal_workspace_bytes(BF_PHASE_DECODE, ...) as for the
 * contiguous call, and the result is bitwise the same as bifocal_decode on a
 * contiguous cache holding the same keys.
 */
int bifocal_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o,
                         float* lse, const int32_t* block_table, const int32_t* seqlens_host,
                         int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                         int32_t num_pages, int32_t n_heads_q, int32_t n_heads_kv,
                         int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                         double rope_theta, int32_t long_mode, float softmax_scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Plain causal softmax attention on the same (original-RoPE) q and k, run by
 * the same engine with the bifocal features compiled out: the reference for
 * the bifocal overhead and for the s = 1 identity.
 *   phase BF_PHASE_PREFILL: layouts and lens_host as bifocal_prefill
 *          (lens_host = cu_seqlens [batch + 1]; cache_capacity ignored);
 *   phase BF_PHASE_DECODE: layouts and lens_host as bifocal_decode
 *          (lens_host = seqlens [batch]).
 */
int plain_attention_ref_gpu(int32_t phase, const void* q, const void* k, const void* v, void* o,
                            float* lse, const int32_t* lens_host, int32_t batch,
                            int32_t cache_capacity, int32_t n_heads_q, int32_t n_heads_kv,
                            int32_t head_dim, int32_t dtype, float softmax_scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Raw-input pre-step for prefill: the model's ORIGINAL RoPE applied to raw
 * (position-free) q and k, giving the q', k' that bifocal_prefill (or, with
 * start positions, bifocal_prefill_chunk) takes, and optionally the KV-cache
 * fill for a following bifocal_decode / bifocal_prefill_chunk.
 *   q_raw, q_out : [n_heads_q,  T, head_dim]  dtype (bf16 or fp32)
 *   k_raw, k_out : [n_heads_kv, T, head_dim]  same dtype; k_out may be NULL
 *                  when k_cache is given
 *   cu_seqlens_host : as bifocal_prefill; token t of sequence b is rotated
 *                  at position P_b + t - cu[b]
 *   pos0_host    : host int32 [batch] start positions P_b >= 0, or NULL for
 *                  0 (a chunk that continues a cached prefix starts at the
 *                  prefix length)
 *   k_cache, v_cache, v : if k_cache is not NULL, k' and v of sequence b are
 *                  also written to k_cache / v_cache [batch, n_heads_kv,
 *                  cache_capacity, head_dim] at positions P_b .. P_b + L_b - 1
 *                  (P_b + L_b <= cache_capacity); v is [n_heads_kv, T, head_dim].
 * q_out may be q_raw and k_out may be k_raw (in place); no other buffers may
 * overlap. theta_m = rope_theta^(-2m/D), half-split pairs (m, m + D/2); the
 * angle is formed in fp64, the rotation in fp32. No workspace.
 * [mufans.github.io wiki, Jet-Long Dynamic RoPE, "关键实现 / 推理流程": the
 *  flow starts by computing RoPE for the input tokens; ai-feeds.com summary,
 *  "关键模块" item 3: cached keys carry original RoPE]
 */
int bifocal_rope_prefill(const void* q_raw, const void* k_raw, const void* v, void* q_out,
                         void* k_out, void* k_cache, void* v_cache, int32_t cache_capacity,
                         const int32_t* cu_seqlens_host, const int32_t* pos0_host, int32_t batch,
                         int32_t n_heads_q,
                         int32_t n_heads_kv, int32_t head_dim, int32_t dtype, double rope_theta,
                         void* stream);

/*
 * Raw-input pre-step for one decode step: the new token of sequence b sits at
 * position p_b = seqlens_host[b] - 1.
 *   q_raw, q_out : [batch, n_heads_q, head_dim]; q_out = R(p_b theta) q_raw
 *                  (may be q_raw: in place)
 *   k_raw, v_new : [batch, n_heads_kv, head_dim]; R(p_b theta) k_raw and
 *                  v_new are written to k_cache / v_cache [batch, n_heads_kv,
 *                  cache_capacity, head_dim] at position p_b
 *   1 <= seqlens_host[b] <= cache_capacity.
 * bifocal_decode with the same seqlens then runs the step. Same rotation and
 * references as bifocal_rope_prefill. No workspace.
 */
int bifocal_rope_append(const void* q_raw, const void* k_raw, const void* v_new, void* q_out,
                        void* k_cache, void* v_cache, const int32_t* seqlens_host, int32_t batch,
                        int32_t cache_capacity, int32_t n_heads_q, int32_t n_heads_kv,
                        int32_t head_dim, int32_t dtype, double rope_theta, void* stream);

/*
 * The two pre-steps above with the cache PAGED, as bifocal_decode_paged and
 * bifocal_prefill_chunk_paged read it:
 *   k_pages, v_pages : [num_pages, n_heads_kv, page_size, head_dim] dtype;
 *                      position p of sequence b goes to page
 *                      block_table[b][p / page_size], row p % page_size
 *   block_table      : DEVICE int32 [batch, max_pages_per_seq] (entries
 *                      clamped to [0, num_pages - 1])
 *   page_size        : a power of two, 1 <= page_size <= 2^20
 * Positions must stay below max_pages_per_seq * page_size. Everything else
 * (layouts, start positions, in-place use, rounding) as the contiguous calls.
 */
int bifocal_rope_prefill_paged(const void* q_raw, const void* k_raw, const void* v, void* q_out,
                               void* k_out, void* k_pages, void* v_pages, const int32_t* block_table,
                               int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                               const int32_t* cu_seqlens_host, const int32_t* pos0_host,
                               int32_t batch, int32_t n_heads_q, int32_t n_heads_kv,
                               int32_t head_dim, int32_t dtype, double rope_theta, void* stream);
int bifocal_rope_append_paged(const void* q_raw, const void* k_raw, const void* v_new, void* q_out,
                              void* k_pages, void* v_pages, const int32_t* block_table,
                              int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                              const int32_t* seqlens_host, int32_t batch, int32_t n_heads_q,
                              int32_t n_heads_kv, int32_t head_dim, int32_t dtype,
                              double rope_theta, void* stream);

/*
 * Test hook: the bf16 prefill tile kernel's own pair classification for one
 * sequence of length L (L <= 4096, query positions 0 .. L - 1, the work items
 * of GQA groups of 4 query heads: 32 query positions each). For every
 * (32-row item, 64-key tile) one wave takes the item's far-pass and
 * local-pass tile ranges and applies both passes' per-element masks to a
 * tile, exactly as the tile loop does, and reports how each pair it covers
 * would be scored:
 *   branch_out : device int8 [L * L], row-major (i, j); 1 = by the local pass
 *                (original RoPE), 2 = by the far pass (scaled RoPE), 3 = by
 *                both (never correct), 0 = by neither (j > i, or a pair
 *                band-only attention drops). Entries the kernel never covers
 *                (tiles past an item's last key) keep the caller's value.
 *                With s(L) = 1 the two branches coincide and the kernel
 *                scores every causal pair locally.
 *   phi_num_out: device int64 [L], the prep pass's (phi(p) - p) * s: -p (s - 1)
 *                for FI, (floor(p / s) - p) s for PA, both exact integers
 *                (unused, may be NULL, for BF_LONG_NONE).
 * long_mode: BF_LONG_FI, BF_LONG_PA or BF_LONG_NONE (s(L) computed on the
 * host from w_pre, as for bifocal_prefill).
 * [ai-feeds.com summary, "关键模块" items 1 and 3: the local window and the
 *  correction of far keys]
 */
int bifocal_test_pair_map(int64_t L, int64_t w0, int64_t w_pre, int32_t long_mode,
                          int8_t* branch_out, int64_t* phi_num_out, void* stream);

/*
 * Test hook: the fp32 (cos, sin) pairs the kernels rotate with, for up to
 * 128 positions given on the host, written to cs_out (device float
 * [n_pos][64][2], rotary pair m = theta_m = rope_theta^(-2m/128)):
 *   which 0: prefill queries at the positions of a sequence of length L
 *            (the prep pass's angle theta_m (phi(p) - p), plus
 *            theta_m (w0 - phi(w0)) with BF_LONG_SHIFT);
 *   which 1: prefill keys (the same without the shift);
 *   which 2: decode keys of a call with N = L keys, through the split
 *            kernel's angle addition (per-step base rotation times the
 *            offset-table rotation, with its incremental divmod tracking);
 *   which 3: decode queries at position p (a call with N = p + 1 keys).
 * s = s(L) (s(p + 1) for which 3); long_mode BF_LONG_FI or BF_LONG_PA, with
 * BF_LONG_SHIFT for the queries' continuity shift.
 * [ai-feeds.com summary, "关键模块" item 3: the correction rotation]
 */
int bifocal_test_angles(int32_t which, const int64_t* positions_host, int32_t n_pos, int64_t L,
                        int64_t w0, int64_t w_pre, double rope_theta, int32_t long_mode,
                        float* cs_out, void* stream);

/* Thread-local description of the last error (empty string after success). */
const char* bifocal_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BIFOCAL_H */
