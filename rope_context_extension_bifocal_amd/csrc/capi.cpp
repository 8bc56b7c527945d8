// libbifocal C-ABI: argument validation, the s(L) schedule, per-launch
// sequence tables, workspace carving and kernel launches. Host code only; the
// kernels live in prefill.hip, decode.hip and rope.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "bifocal.h"
#include "bf_common.h"

namespace bf {
hipError_t launch_correction_prep(int dtype, const PrepParams& pp, const SeqTable& st,
                                  const ThetaTable& tt, hipStream_t stream);
hipError_t launch_vt_transpose(int dtype, const VtParams& vp, const SeqTable& st,
                               hipStream_t stream);
hipError_t launch_prefill_main(int dtype, bool bifocal, bool band, const PrefillParams& pp,
                               const SeqTable& st, int grid, hipStream_t stream);
hipError_t launch_chunk_combine(const PrefillParams& pp, int tok_begin, int n_tok,
                                hipStream_t stream);
hipError_t launch_pair_map(long long L, long long w0, long long s, int mode, int8_t* br,
                           long long* dphi_num, hipStream_t stream);
hipError_t launch_prep_angles(const AngleProbe& a, const ThetaTable& tt, float* cs,
                              hipStream_t stream);
hipError_t launch_decode_angles(const AngleProbe& a, const ThetaTable& tt, int which, float* cs,
                                hipStream_t stream);
size_t decode_workspace_bytes(int batch, long long max_len, int Hq);
size_t decode_noalloc_capacity();
int decode_noalloc_scratch(hipStream_t stream, void** out, std::string& err);
struct PagedCache {
  const int* block_table;
  int page_size;
  int max_pages;
  int num_pages;
};
struct DecodeStore {
  void* k2;
  int32_t* keys;
  int32_t* s;
};
int run_decode(bool bifocal, const void* q, const void* kc, const void* vc, void* o, float* lse,
               const int32_t* seqlens, int batch, int cap, int Hq, int Hkv, long long w0,
               long long w_pre, double theta, int mode, float scale, void* ws, size_t ws_bytes,
               hipStream_t stream, std::string& err, long long window, const PagedCache* paged,
               bool validate_only = false, const DecodeStore* store = nullptr);
int run_rope_prefill(const void* q, const void* k, const void* v, void* q_out, void* k_out,
                     void* k_cache, void* v_cache, int cap, const int32_t* cu, const int32_t* pos0,
                     const PagedKV& pk, int batch, int Hq, int Hkv, int dtype, double theta,
                     hipStream_t stream, std::string& err);
int run_rope_append(const void* q, const void* k, const void* v, void* q_out, void* k_cache,
                    void* v_cache, int cap, const int32_t* seqlens, const PagedKV& pk, int batch,
                    int Hq, int Hkv, int dtype, double theta, hipStream_t stream, std::string& err);
}  // namespace bf

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool trace_on() {
  const char* e = getenv("BIFOCAL_TRACE");
  return e && e[0] == '1';
}

bool forced_launch_failure() {
  const char* e = getenv("BIFOCAL_TEST_FAIL_LAUNCH");
  return e && e[0] == '1';
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_size(int dtype) { return dtype == BF_DTYPE_BF16 ? 2 : 4; }

bf::ThetaTable theta_table(double rope_theta) {
  bf::ThetaTable tt;
  for (int m = 0; m < bf::kPairs; ++m)
    tt.th[m] = std::pow(rope_theta, -2.0 * (double)m / (double)bf::kHeadDim);
  return tt;
}

// Geometry of the prefill launch for a given element type and GQA group size.
struct PrefillGeom {
  int hpw, n_hsub, P_wg;
};

PrefillGeom prefill_geom(int dtype, int G) {
  PrefillGeom g;
  g.hpw = std::gcd(G, 4);
  g.n_hsub = G / g.hpw;
  const int rows = dtype == BF_DTYPE_BF16 ? bf::kWaveRowsBf16 : bf::kWaveRowsF32;
  const int waves = dtype == BF_DTYPE_BF16 ? bf::kWavesPerGroupBf16 : bf::kWavesPerGroupF32;
  g.P_wg = rows * waves / g.hpw;
  return g;
}

struct PrefillWs {
  size_t ctr_off, vt_off, q2_off, k2_off, kc_off, base, po_off, pl_off, total;
};

// Workspace of Tq packed queries against Tk keys (a one-shot prefill has
// Tk = Tq = T): 256 bytes of work-item counters, V^T padded per sequence,
// q'', k'', for a paged key source the
// packed copy of the keys (Tk_copy of them, by default Tk; base ends here),
// and for `splits` > 1 key splits their partial O (fp32) and log2-sum-exp.
PrefillWs prefill_ws_layout(int batch, long long Tq, long long Tk, int Hq, int Hkv, int dtype,
                            bool paged = false, int splits = 1, long long Tk_copy = -1) {
  const size_t es = elem_size(dtype);
  const size_t tpad_bound = (size_t)Tk + 63u * (size_t)batch;
  PrefillWs w;
  w.ctr_off = 0;
  w.vt_off = 256;
  w.q2_off = w.vt_off + align256((size_t)Hkv * bf::kHeadDim * tpad_bound * es);
  w.k2_off = w.q2_off + align256((size_t)Hq * (size_t)Tq * bf::kHeadDim * es);
  w.kc_off = w.k2_off + align256((size_t)Hkv * (size_t)Tk * bf::kHeadDim * es);
  if (Tk_copy < 0) Tk_copy = Tk;
  w.base = w.kc_off + (paged ? align256((size_t)Hkv * (size_t)Tk_copy * bf::kHeadDim * es) : 0);
  const size_t rows = splits > 1 ? (size_t)splits * Hq * (size_t)Tq : 0;
  w.po_off = w.base;
  w.pl_off = w.po_off + align256(rows * bf::kHeadDim * sizeof(float));
  w.total = w.pl_off + align256(rows * sizeof(float));
  return w;
}

// The 512 workgroup slots of the part: two prefill workgroups on each of 256 CUs.
constexpr long long kPrefillSlots = 512;

// Largest key-split count a chunk launch of Tq queries may use: a chunk is
// split only while its work items fill at most two rounds of the slots, so
// the count is bounded by the fewest items Tq queries can make (one
// sequence). fp32 launches are not split.
int chunk_split_cap(long long Tq, int Hq, int Hkv, int dtype) {
  if (dtype != BF_DTYPE_BF16 || Hkv < 1 || Hq % Hkv) return 1;
  const PrefillGeom geo = prefill_geom(dtype, Hq / Hkv);
  const long long wmin = (long long)Hkv * geo.n_hsub * ((Tq + geo.P_wg - 1) / geo.P_wg);
  return (int)std::max(1LL, std::min<long long>(bf::kMaxKeySplits, 2 * kPrefillSlots / std::max(1LL, wmin)));
}

// Key splits of one launch: W workgroups whose items visit about `visits`
// key tiles each. k splits make ceil(W k / slots) rounds of visits / k tiles
// plus a fixed cost of about 6 tile times per workgroup (prologue, the last
// P V, the partial's store); the cheapest k up to `cap` wins, with at least
// 32 tiles per split.
int pick_key_splits(long long W, double visits, int cap) {
  int best = 1;
  double best_cost = -1.0;
  for (int k = 1; k <= cap; ++k) {
    if (k > 1 && visits / k < 32.0) break;
    const double rounds = (double)((W * k + kPrefillSlots - 1) / kPrefillSlots);
    const double cost = rounds * (visits / k + 6.0);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = k;
    }
  }
  return best;
}

int check_common(int Hq, int Hkv, int head_dim, int dtype) {
  if (Hq < 1 || Hkv < 1) return fail(BF_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(BF_ERR_INVALID_ARG, "n_heads_q %% n_heads_kv != 0 (%d, %d)", Hq, Hkv);
  if (dtype != BF_DTYPE_BF16 && dtype != BF_DTYPE_FP32)
    return fail(BF_ERR_INVALID_ARG, "dtype must be BF_DTYPE_BF16 or BF_DTYPE_FP32 (got %d)", dtype);
  if (head_dim != bf::kHeadDim) return fail(BF_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  return BF_OK;
}

int check_bifocal_knobs(long long w0, long long w_pre, double theta, int mode) {
  if (w0 < 0) return fail(BF_ERR_INVALID_ARG, "w0 must be >= 0 (got %lld)", w0);
  if (w_pre < 1) return fail(BF_ERR_INVALID_ARG, "w_pre must be >= 1 (got %lld)", w_pre);
  if (!(theta > 1.0) || !std::isfinite(theta))
    return fail(BF_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  const int base = mode & ~BF_LONG_SHIFT;
  if (base != BF_LONG_FI && base != BF_LONG_PA && base != BF_LONG_NONE)
    return fail(BF_ERR_INVALID_ARG, "long_mode must be BF_LONG_FI or BF_LONG_PA (optionally with "
                "BF_LONG_SHIFT) or BF_LONG_NONE (got %d)", mode);
  if (base == BF_LONG_NONE && (mode & BF_LONG_SHIFT))
    return fail(BF_ERR_INVALID_ARG, "BF_LONG_SHIFT has no meaning for band-only attention");
  if (base == BF_LONG_NONE && w0 < 1)
    return fail(BF_ERR_INVALID_ARG, "band-only attention (BF_LONG_NONE) needs w0 >= 1");
  return BF_OK;
}

int check_scale(float scale) {
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(BF_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  return BF_OK;
}

// One launch description shared by the one-shot prefill and the chunk of
// queries against a KV cache: sequence b has Lq_b = cu[b+1] - cu[b] packed
// queries at positions qpos[b] .. qpos[b] + Lq_b - 1 and N_b = qpos[b] + Lq_b
// keys at K / V rows h * k_hstride + kbase[b] + j; s comes from slen[b].
struct RowsJob {
  bool bifocal = false;
  const void *q = nullptr, *k = nullptr, *v = nullptr;
  void* o = nullptr;
  float* lse = nullptr;
  std::vector<int> cu, qpos;
  std::vector<long long> kbase, slen;
  long long k_hstride = 0, k_rows = 0;
  bf::PagedKV pk{nullptr, 0, 0, 0};  // paged K / V source (block table of the whole batch)
  int batch = 0, Hq = 0, Hkv = 0, dtype = 0;
  long long w0 = 0, w_pre = 1;
  double theta = 10000.0;
  int mode = 0;
  float scale = 1.f;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t stream = nullptr;
  int split_cap = 1;  // key splits allowed (chunk launches; the workspace may cap it further)
  // caller-kept store of k'' and V^T (chunk launches over a contiguous cache),
  // or null: k'' at rows (b * Hkv + h) * store_cap64 + j, V^T from byte
  // store_vt_off in tiles (b * Hkv + h) * store_cap64 / 64 + t; the call forms
  // them for keys kfirst[b] .. N_b - 1 only (V^T from kfirst[b]'s tile on)
  char* store = nullptr;
  long long store_cap64 = 0;
  size_t store_vt_off = 0;
  std::vector<int> kfirst;
};

// Validation of the arguments both paths share; tensors checked by the caller.
int check_rows_common(bool bifocal, int batch, int Hq, int Hkv, int head_dim, int dtype,
                      long long w0, long long w_pre, double theta, int mode, float scale) {
  if (batch < 1) return fail(BF_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  int rc = check_common(Hq, Hkv, head_dim, dtype);
  if (rc) return rc;
  if (bifocal && (rc = check_bifocal_knobs(w0, w_pre, theta, mode))) return rc;
  return check_scale(scale);
}

// Query-key pairs a sequence scores: Lq queries at positions qpos .. qpos +
// Lq - 1, each seeing every key up to its own position, or only the nearest
// band of them when band >= 0 (band-only attention, band = w0).
double scored_pairs(long long qpos, long long Lq, long long band) {
  if (band < 0) return (double)Lq * qpos + 0.5 * (double)Lq * (Lq + 1);
  const long long a = std::min(Lq, std::max(0LL, band - qpos - 1));  // rows seeing < band keys
  return (double)a * (qpos + 1) + 0.5 * (double)a * (a - 1) + (double)(Lq - a) * band;
}

int run_rows(RowsJob& j) {
  const int batch = j.batch, Hq = j.Hq, Hkv = j.Hkv, dtype = j.dtype;
  const bool bifocal = j.bifocal;
  long long Tq = j.cu[batch], Tk = 0;
  const bool band_mode = bifocal && (j.mode & ~BF_LONG_SHIFT) == BF_LONG_NONE;
  std::vector<int> kcu(batch + 1, 0), vt_off(batch + 1, 0), vt_t0(batch, 0);
  for (int b = 0; b < batch; ++b) {
    const long long N = (long long)j.qpos[b] + (j.cu[b + 1] - j.cu[b]);
    kcu[b + 1] = (int)(kcu[b] + N);
    // band only: no query of the sequence reaches a key below qpos - w0 + 1,
    // so V^T (and a paged gather) start at that key's tile
    if (band_mode) vt_t0[b] = (int)(std::max(0LL, (long long)j.qpos[b] - j.w0 + 1) / bf::kKeyTile);
    const long long tiles = (N + bf::kKeyTile - 1) / bf::kKeyTile - vt_t0[b];
    vt_off[b + 1] = vt_off[b] + (int)tiles * bf::kKeyTile;
  }
  Tk = kcu[batch];
  const bool paged = j.pk.block_table != nullptr;
  const bool stored = j.store != nullptr;
  const long long Tk_ws = stored ? 0 : Tk;  // a store holds k'' and V^T: none in the workspace
  // with a store, the prep's key axis of sequence b holds keys ax0[b] ..
  // N_b - 1 (at acu[b] ..): those without a stored k'' and, for a paged
  // source, also every key the local pass reads (from the window start of
  // the chunk's first query on), which go to the packed copy
  std::vector<int> ax0(batch, 0), acu(batch + 1, 0);
  if (stored) {
    for (int b = 0; b < batch; ++b) {
      const long long N = kcu[b + 1] - kcu[b];
      const long long s = std::max<long long>(1, bifocal_s_of_L(j.slen[b], j.w_pre));
      const long long win = s > 1 ? std::max(0LL, (long long)j.qpos[b] - j.w0 + 1) : 0;
      const long long kc0 = win / bf::kKeyTile * bf::kKeyTile;
      ax0[b] = (int)(paged ? std::min<long long>(j.kfirst[b], kc0) : j.kfirst[b]);
      acu[b + 1] = acu[b] + (int)(N - ax0[b]);
    }
  }
  const long long Tk_copy = stored ? acu[batch] : Tk;  // rows of the packed copy (paged)
  const PrefillWs wl = prefill_ws_layout(batch, Tq, Tk_ws, Hq, Hkv, dtype, paged, 1, Tk_copy);
  if (!j.ws) return fail(BF_ERR_WORKSPACE, "workspace is null");
  if ((uintptr_t)j.ws & 255u) return fail(BF_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const bool shift = bifocal && (j.mode & BF_LONG_SHIFT);
  const int mode = j.mode & ~BF_LONG_SHIFT;
  const bool band_only = bifocal && mode == BF_LONG_NONE;
  const size_t need = paged ? wl.base : bifocal && !band_only ? wl.kc_off : wl.q2_off;
  if (j.ws_bytes < need)
    return fail(BF_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", j.ws_bytes, need);
  // key splits the workspace has room for (partials after the base layout)
  int split_cap = dtype == BF_DTYPE_BF16 ? std::max(1, std::min(j.split_cap, bf::kMaxKeySplits)) : 1;
  while (split_cap > 1 &&
         prefill_ws_layout(batch, Tq, Tk_ws, Hq, Hkv, dtype, paged, split_cap, Tk_copy).total > j.ws_bytes)
    --split_cap;

  const int G = Hq / Hkv;
  const PrefillGeom geo = prefill_geom(dtype, G);
  const int Tpad = vt_off[batch];
  const bf::ThetaTable tt = theta_table(bifocal ? j.theta : 10000.0);
  char* wsb = (char*)j.ws;

  // Plan every launch group (at most kMaxSeqPerLaunch sequences each) before
  // the first launch, so that an argument a later group rejects leaves
  // nothing enqueued and the outputs untouched.
  struct Group {
    bf::SeqTable st;
    bf::PrefillParams pp;
    bf::PagedKV pk;
    bool any_far;
    long long grid;
  };
  std::vector<Group> groups;
  for (int b0 = 0; b0 < batch; b0 += bf::kMaxSeqPerLaunch) {
    const int nb = std::min(bf::kMaxSeqPerLaunch, batch - b0);
    groups.emplace_back();
    Group& gr = groups.back();
    bf::SeqTable& st = gr.st;
    std::memset(&st, 0, sizeof st);
    st.n = nb;
    bool any_far = false;
    int total_items = 0;
    double work[bf::kMaxSeqPerLaunch], visit_sum = 0.0;
    for (int i = 0; i <= nb; ++i) {
      st.cu[i] = j.cu[b0 + i];
      st.kcu[i] = kcu[b0 + i];
      st.vt_off[i] = vt_off[b0 + i];
    }
    for (int i = 0; i < nb; ++i) st.vt_t0[i] = vt_t0[b0 + i];
    for (int i = 0; i < nb; ++i) {
      const long long Lq = j.cu[b0 + i + 1] - j.cu[b0 + i];
      const long long N = j.qpos[b0 + i] + Lq;
      const long long s = bifocal && !band_only ? bifocal_s_of_L(j.slen[b0 + i], j.w_pre) : 1;
      if (s < 1 || s > (1LL << 30))
        return fail(BF_ERR_INVALID_ARG, "s(L) of sequence %d is %lld, outside [1, 2^30]", b0 + i, s);
      st.s[i] = (int)s;
      st.qpos[i] = j.qpos[b0 + i];
      // a paged source is gathered into the packed copy, which the tile
      // kernel then reads like packed keys (with a store, from key ax0 on)
      st.kbase[i] = paged ? (stored ? (long long)acu[b0 + i] - ax0[b0 + i] : kcu[b0 + i]) : j.kbase[b0 + i];
      // far pairs to score (bifocal) or to drop (band only): the last query
      // (position N - 1) reaches back past the window
      if ((s > 1 || band_only) && j.w0 < N) any_far = true;
      st.nrb[i] = (int)((Lq + geo.P_wg - 1) / geo.P_wg);
      total_items += st.nrb[i];
      // key tiles a row block visits: all N keys, or only its window (band only)
      const long long span = band_only ? std::min(N, j.w0 + geo.P_wg + bf::kKeyTile) : N;
      visit_sum += (double)st.nrb[i] * (double)((span + bf::kKeyTile - 1) / bf::kKeyTile);
      work[i] = scored_pairs(j.qpos[b0 + i], Lq, band_only ? j.w0 : -1);
    }
    gr.any_far = any_far;
    // work order: sequences with the most scored pairs first (ties in batch
    // order), each one's row blocks as one run of ranks
    std::iota(st.order, st.order + nb, 0);
    std::stable_sort(st.order, st.order + nb, [&](int a, int b) { return work[a] > work[b]; });
    st.ioff[0] = 0;
    for (int i = 0; i < nb; ++i) st.ioff[i + 1] = st.ioff[i] + st.nrb[st.order[i]];
    gr.pk = j.pk;  // the block-table rows of this group's sequences
    if (paged) gr.pk.block_table += (size_t)b0 * gr.pk.max_pages;
    bf::PrefillParams& pp = gr.pp;
    pp.q = j.q;
    pp.k = paged ? (const void*)(wsb + wl.kc_off) : j.k;
    pp.q2 = wsb + wl.q2_off;
    pp.k2 = wsb + wl.k2_off;
    pp.vt = wsb + wl.vt_off;
    pp.o = j.o;
    pp.lse = j.lse;
    pp.w0 = j.w0;
    pp.scale_log2 = j.scale * 1.4426950408889634f;
    pp.k_hstride = paged ? Tk_copy : j.k_hstride;
    pp.k_rows = paged ? (long long)Hkv * Tk_copy : j.k_rows;
    pp.T = (int)Tq;
    pp.Tk = (int)Tk;
    pp.Tpad = Tpad;
    pp.Hq = Hq;
    pp.Hkv = Hkv;
    pp.G = G;
    pp.hpw = geo.hpw;
    pp.n_hsub = geo.n_hsub;
    pp.P_wg = geo.P_wg;
    pp.total_items = total_items;
    const long long wgs = (long long)Hkv * geo.n_hsub * total_items;
    pp.nks = split_cap > 1 ? pick_key_splits(wgs, visit_sum / total_items, split_cap) : 1;
    pp.part_o = pp.nks > 1 ? (float*)(wsb + wl.po_off) : nullptr;
    pp.part_lse = pp.nks > 1 ? (float*)(wsb + prefill_ws_layout(batch, Tq, Tk_ws, Hq, Hkv, dtype, paged, pp.nks,
                                                                  Tk_copy).pl_off)
                             : nullptr;
    pp.k2_rows = (long long)Hkv * Tk;
    pp.vt_rows = (long long)Hkv * Tpad;
    if (stored) {
      // this group's sequences in the store: k'' and V^T of (i, h) at
      // rows / columns (i * Hkv + h) * cap64 from the group's first sequence
      const size_t seq_bytes = (size_t)Hkv * j.store_cap64 * bf::kHeadDim * elem_size(dtype);
      pp.k2 = j.store + (size_t)b0 * seq_bytes;
      pp.vt = j.store + j.store_vt_off + (size_t)b0 * seq_bytes;
      pp.Tk = (int)j.store_cap64;
      pp.Tpad = (int)j.store_cap64;
      pp.k2_rows = pp.vt_rows = (long long)nb * Hkv * j.store_cap64;
    }
    gr.grid = wgs * pp.nks;
    // a bf16 launch of two rounds of workgroups or more runs on persistent
    // workgroups that claim their work items from per-XCD queues (see
    // claim_item): the XCDs run at slightly different speeds, and a static
    // split leaves the faster ones idle for up to a few percent of a long
    // launch; short items also skip the workgroup turnover. Same box, bitwise
    // the same output: 128K 120.4 against 121.7-123.3 ms, 64 x 2048 prompts
    // 2.49-2.50 against 2.52-2.53 ms, 16 x 8192 7.96-7.98 against 8.06-8.13 ms.
    pp.item_ctr = dtype == BF_DTYPE_BF16 && gr.grid >= 2 * kPrefillSlots ? (int*)(wsb + wl.ctr_off) : nullptr;
    if (gr.grid > 0x7fffffffLL)
      return fail(BF_ERR_INVALID_ARG, "launch grid of sequences %d..%d too large (%lld workgroups)", b0,
                  b0 + nb - 1, gr.grid);
    pp.n_items = (int)gr.grid;
    if (pp.item_ctr) gr.grid = kPrefillSlots;  // persistent workgroups, two per CU
  }
  if (forced_launch_failure()) return fail(BF_ERR_HIP, "launch failure forced by BIFOCAL_TEST_FAIL_LAUNCH");

  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const Group& gr = groups[gi];
    const bf::SeqTable& st = gr.st;
    const bf::PrefillParams& pp = gr.pp;
    const int b0 = (int)gi * bf::kMaxSeqPerLaunch, nb = st.n;
    hipError_t e = hipSuccess;
    if (!stored) {
      bf::VtParams vp{j.v, wsb + wl.vt_off, gr.pk, j.k_hstride, Tpad, Hkv, 0};
      e = bf::launch_vt_transpose(dtype, vp, st, j.stream);
      if (e != hipSuccess) return fail(BF_ERR_HIP, "vt_transpose launch: %s", hipGetErrorString(e));
      if ((bifocal && gr.any_far && !band_only) || paged) {
        // band-only or s = 1 sequences get no rotation: the prep only gathers
        bf::PrepParams prep{j.q, j.k, wsb + wl.q2_off, wsb + wl.k2_off, paged ? wsb + wl.kc_off : nullptr, gr.pk,
                            j.k_hstride, (int)Tq, (int)Tk, Hq, Hkv, mode, shift ? 1 : 0, j.w0, 0, {}, {}};
        e = bf::launch_correction_prep(dtype, prep, st, tt, j.stream);
        if (e != hipSuccess) return fail(BF_ERR_HIP, "correction_prep launch: %s", hipGetErrorString(e));
      }
    } else {
      // V^T of the tiles from each sequence's first new key on (the tile of
      // kfirst is redone whole: its keys past the old length were zero)
      bf::SeqTable sv = st;
      sv.vt_off[0] = 0;
      for (int i = 0; i < nb; ++i) {
        const int N = st.kcu[i + 1] - st.kcu[i];
        sv.vt_t0[i] = j.kfirst[b0 + i] / bf::kKeyTile;
        sv.vt_off[i + 1] = sv.vt_off[i] + ((N + bf::kKeyTile - 1) / bf::kKeyTile - sv.vt_t0[i]) * bf::kKeyTile;
      }
      if (sv.vt_off[nb] > 0) {
        bf::VtParams vp{j.v, const_cast<void*>(pp.vt), gr.pk, j.k_hstride, 0, Hkv,
                        (int)(j.store_cap64 / bf::kKeyTile)};
        e = bf::launch_vt_transpose(dtype, vp, sv, j.stream);
        if (e != hipSuccess) return fail(BF_ERR_HIP, "vt_transpose launch: %s", hipGetErrorString(e));
      }
      // q'' of the chunk and k'' of keys kfirst .. N - 1 into the store, for
      // every sequence with s > 1 (also one whose keys are all local yet:
      // the store then holds its far keys for later calls); a paged source
      // also gathers keys ax0 .. N - 1 into the packed copy
      bf::SeqTable sp = st;
      for (int i = 0; i <= nb; ++i) sp.kcu[i] = acu[b0 + i];
      bf::PrepParams prep{j.q, j.k, wsb + wl.q2_off, const_cast<void*>(pp.k2), paged ? wsb + wl.kc_off : nullptr,
                          gr.pk, j.k_hstride, (int)Tq, (int)Tk_copy, Hq, Hkv, mode, shift ? 1 : 0, j.w0,
                          (int)j.store_cap64, {}, {}};
      for (int i = 0; i < nb; ++i) {
        prep.kfirst[i] = ax0[b0 + i];
        prep.krot[i] = j.kfirst[b0 + i];
      }
      e = bf::launch_correction_prep(dtype, prep, sp, tt, j.stream);
      if (e != hipSuccess) return fail(BF_ERR_HIP, "correction_prep launch: %s", hipGetErrorString(e));
    }
    // a store: the main kernel finds k'' and V^T of sequence i at
    // (i * Hkv + h) * cap64 rows and columns of the group's part of it
    bf::SeqTable sm;
    if (stored) {
      sm = st;
      for (int i = 0; i <= nb; ++i) sm.kcu[i] = sm.vt_off[i] = (int)(i * Hkv * j.store_cap64);
      for (int i = 0; i < nb; ++i) sm.vt_t0[i] = 0;
    }
    if (trace_on())
      fprintf(stderr, "[bifocal] prefill %s dtype=%d seqs=%d..%d grid=%lld P_wg=%d hpw=%d n_hsub=%d s0=%d qpos0=%d w0=%lld key_splits=%d\n",
              band_only ? "band-only" : bifocal ? "bifocal" : "plain", dtype, b0, b0 + nb - 1, gr.grid, geo.P_wg, geo.hpw,
              geo.n_hsub, st.s[0], st.qpos[0], j.w0, pp.nks);
    e = bf::launch_prefill_main(dtype, bifocal && gr.any_far, band_only && gr.any_far, pp, stored ? sm : st,
                                (int)gr.grid, j.stream);
    if (e != hipSuccess) return fail(BF_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    if (pp.nks > 1) {
      e = bf::launch_chunk_combine(pp, st.cu[0], st.cu[nb] - st.cu[0], j.stream);
      if (e != hipSuccess) return fail(BF_ERR_HIP, "chunk combine launch: %s", hipGetErrorString(e));
    }
  }
  g_err.clear();
  return BF_OK;
}

// A paged cache as the C-ABI passes it: pages [num_pages][Hkv][page_size][D].
struct ChunkPages {
  const int32_t* block_table;  // device [batch][max_pages]
  int page_size, max_pages, num_pages;
};

// Validates a paged cache; sets the kernels' description and the most keys a
// sequence's pages hold.
int check_pages(const ChunkPages& pg, bf::PagedKV& pk, long long& hold) {
  const int ps = pg.page_size;
  if (ps < 1 || ps > (1 << 20) || (ps & (ps - 1)))
    return fail(BF_ERR_INVALID_ARG, "page_size must be a power of two in [1, 2^20] (got %d)", ps);
  if (pg.max_pages < 1 || pg.num_pages < 1)
    return fail(BF_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
  if (!pg.block_table || ((uintptr_t)pg.block_table & 3u))
    return fail(BF_ERR_INVALID_ARG, "block_table must be a non-null 4-byte aligned device pointer");
  int lg = 0;
  while ((1 << lg) < ps) ++lg;
  pk = bf::PagedKV{pg.block_table, lg, pg.max_pages, pg.num_pages};
  hold = (long long)pg.max_pages * ps;
  return BF_OK;
}

// Shared prefill path of bifocal_prefill and the plain reference.
int run_prefill(bool bifocal, const void* q, const void* k, const void* v, void* o, float* lse,
                const int32_t* cu, int batch, int Hq, int Hkv, int head_dim, int dtype,
                long long w0, long long w_pre, double theta, int mode, float scale, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !cu) return fail(BF_ERR_INVALID_ARG, "null tensor or cu_seqlens pointer");
  int rc = check_rows_common(bifocal, batch, Hq, Hkv, head_dim, dtype, w0, w_pre, theta, mode, scale);
  if (rc) return rc;
  if (cu[0] != 0) return fail(BF_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  for (int b = 0; b < batch; ++b)
    if (cu[b + 1] <= cu[b])
      return fail(BF_ERR_INVALID_ARG, "cu_seqlens must be strictly increasing (b=%d: %d -> %d)", b, cu[b], cu[b + 1]);
  const long long T = cu[batch];
  if (T + 63LL * batch > (1LL << 31) - 1) return fail(BF_ERR_INVALID_ARG, "too many tokens (%lld)", T);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BF_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && ((uintptr_t)lse & 3u)) return fail(BF_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  RowsJob j;
  j.bifocal = bifocal;
  j.q = q; j.k = k; j.v = v; j.o = o; j.lse = lse;
  j.cu.assign(cu, cu + batch + 1);
  j.qpos.assign(batch, 0);
  j.kbase.resize(batch);
  j.slen.resize(batch);
  for (int b = 0; b < batch; ++b) {
    j.kbase[b] = cu[b];
    j.slen[b] = cu[b + 1] - cu[b];
  }
  j.k_hstride = T;
  j.k_rows = (long long)Hkv * T;
  j.batch = batch; j.Hq = Hq; j.Hkv = Hkv; j.dtype = dtype;
  j.w0 = w0; j.w_pre = w_pre; j.theta = theta; j.mode = mode; j.scale = scale;
  j.ws = ws; j.ws_bytes = ws_bytes; j.stream = stream;
  return run_rows(j);
}


// The caller-kept k'' / V^T store of bifocal_prefill_chunk_stored: `bytes`
// of device memory and two host arrays of per-sequence state.
struct ChunkStore {
  void* buf;
  size_t bytes;
  int32_t* keys;  // in/out: keys 0 .. keys[b] - 1 of sequence b are held ...
  int32_t* s;     // ... for s = s[b]
};

// Bytes of a chunk store: k'' [batch][Hkv][cap64][D], then (256-aligned) V^T
// [batch][Hkv][cap64 / 64][D][64], cap64 = cap rounded up to 64. 0 when a
// launch group's offsets (64 sequences x Hkv x cap64) would not fit an int.
size_t chunk_store_bytes(int batch, long long cap, int Hkv, int dtype) {
  if (batch < 1 || cap < 1 || Hkv < 1) return 0;
  const long long cap64 = (cap + bf::kKeyTile - 1) / bf::kKeyTile * bf::kKeyTile;
  if ((long long)std::min(batch, bf::kMaxSeqPerLaunch) * Hkv * cap64 > 0x7fffffffLL) return 0;
  const size_t region = align256((size_t)batch * Hkv * cap64 * bf::kHeadDim * elem_size(dtype));
  return 2 * region;
}

// Chunk of queries against a KV cache [B][Hkv][cap][D] (bifocal_prefill_chunk)
// or a paged cache (bifocal_prefill_chunk_paged: pages != null, cap = the
// most keys a sequence's pages hold); with `store`, k'' and V^T are kept
// between calls (bifocal_prefill_chunk_stored and its paged form).
int run_chunk(const void* q, const void* kc, const void* vc, void* o, float* lse,
              const int32_t* cu_q, const int32_t* seqlens, const int32_t* s_len, int batch,
              int cap, int Hq, int Hkv, int head_dim, int dtype, long long w0, long long w_pre,
              double theta, int mode, float scale, void* ws, size_t ws_bytes, hipStream_t stream,
              const ChunkPages* pages = nullptr, const ChunkStore* store = nullptr) {
  if (!q || !kc || !vc || !o || !cu_q || !seqlens)
    return fail(BF_ERR_INVALID_ARG, "null tensor, cu_q or seqlens pointer");
  int rc = check_rows_common(true, batch, Hq, Hkv, head_dim, dtype, w0, w_pre, theta, mode, scale);
  if (rc) return rc;
  bf::PagedKV pk{nullptr, 0, 0, 0};
  if (pages) {
    long long hold = 0;
    if ((rc = check_pages(*pages, pk, hold))) return rc;
    cap = (int)std::min<long long>(hold, 0x7fffffffLL);
  }
  if (cap < 1) return fail(BF_ERR_INVALID_ARG, "cache_capacity must be >= 1 (got %d)", cap);
  if (cu_q[0] != 0) return fail(BF_ERR_INVALID_ARG, "cu_q[0] must be 0 (got %d)", cu_q[0]);
  long long Tk = 0;
  for (int b = 0; b < batch; ++b) {
    const int Lq = cu_q[b + 1] - cu_q[b];
    if (Lq < 1) return fail(BF_ERR_INVALID_ARG, "cu_q must be strictly increasing (b=%d: %d -> %d)", b, cu_q[b], cu_q[b + 1]);
    if (seqlens[b] < Lq || seqlens[b] > cap)
      return fail(BF_ERR_INVALID_ARG, "seqlens[%d] = %d must lie in [chunk length %d, %s %d]", b, seqlens[b],
                  Lq, pages ? "max_pages_per_seq * page_size" : "cache_capacity", cap);
    if (s_len && s_len[b] < seqlens[b])
      return fail(BF_ERR_INVALID_ARG, "s_len[%d] = %d is below seqlens[%d] = %d", b, s_len[b], b, seqlens[b]);
    Tk += seqlens[b];
  }
  if (Tk + 63LL * batch > (1LL << 31) - 1) return fail(BF_ERR_INVALID_ARG, "too many keys (%lld)", Tk);
  if (!pages && (long long)batch * Hkv * cap > (1LL << 40)) return fail(BF_ERR_INVALID_ARG, "cache too large");
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(o))
    return fail(BF_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  if (lse && ((uintptr_t)lse & 3u)) return fail(BF_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  size_t store_need = 0;
  if (store) {
    if ((mode & ~BF_LONG_SHIFT) == BF_LONG_NONE)
      return fail(BF_ERR_UNSUPPORTED, "band-only attention (long_mode NONE) has no k'' to store");
    if (!store->buf || ((uintptr_t)store->buf & 255u))
      return fail(BF_ERR_INVALID_ARG, "store must be a non-null 256-byte aligned device pointer");
    if (!store->keys || !store->s)
      return fail(BF_ERR_INVALID_ARG, "store_keys_host and store_s_host must be non-null");
    store_need = chunk_store_bytes(batch, cap, Hkv, dtype);
    if (store_need == 0)
      return fail(BF_ERR_UNSUPPORTED, "store of 64 sequences x %d KV heads x %d keys exceeds 2^31 rows", Hkv, cap);
    if (store->bytes < store_need)
      return fail(BF_ERR_WORKSPACE, "store too small: %zu bytes given, %zu needed", store->bytes, store_need);
    for (int b = 0; b < batch; ++b)
      if (store->keys[b] < 0)
        return fail(BF_ERR_INVALID_ARG, "store_keys_host[%d] = %d is negative", b, store->keys[b]);
  }
  RowsJob j;
  j.bifocal = true;
  j.q = q; j.k = kc; j.v = vc; j.o = o; j.lse = lse;
  j.cu.assign(cu_q, cu_q + batch + 1);
  j.qpos.resize(batch);
  j.kbase.resize(batch);
  j.slen.resize(batch);
  for (int b = 0; b < batch; ++b) {
    j.qpos[b] = seqlens[b] - (cu_q[b + 1] - cu_q[b]);
    j.kbase[b] = (long long)b * Hkv * cap;
    j.slen[b] = s_len ? s_len[b] : seqlens[b];
  }
  j.k_hstride = cap;
  j.k_rows = (long long)batch * Hkv * cap;
  j.pk = pk;
  j.batch = batch; j.Hq = Hq; j.Hkv = Hkv; j.dtype = dtype;
  j.w0 = w0; j.w_pre = w_pre; j.theta = theta; j.mode = mode; j.scale = scale;
  j.ws = ws; j.ws_bytes = ws_bytes; j.stream = stream;
  j.split_cap = chunk_split_cap(j.cu[batch], Hq, Hkv, dtype);
  std::vector<int> s_of(batch, 1);
  if (store) {
    j.store = (char*)store->buf;
    j.store_cap64 = (cap + bf::kKeyTile - 1) / bf::kKeyTile * bf::kKeyTile;
    j.store_vt_off = store_need / 2;
    j.kfirst.resize(batch);
    for (int b = 0; b < batch; ++b) {
      // an s outside [1, 2^30] is rejected by run_rows before any launch
      s_of[b] = (int)std::min<long long>(bifocal_s_of_L(j.slen[b], w_pre), 1LL << 30);
      j.kfirst[b] = store->s[b] == s_of[b] ? std::min(store->keys[b], seqlens[b]) : 0;
    }
  }
  rc = run_rows(j);
  if (rc == BF_OK && store)
    for (int b = 0; b < batch; ++b) {
      store->keys[b] = seqlens[b];
      store->s[b] = s_of[b];
    }
  return rc;
}

int rope_prefill_impl(const void* q_raw, const void* k_raw, const void* v, void* q_out,
                      void* k_out, void* k_cache, void* v_cache, int cache_capacity,
                      const int32_t* cu, const int32_t* pos0, int batch, int n_heads_q,
                      int n_heads_kv, int head_dim, int dtype, double rope_theta, void* stream,
                      const ChunkPages* pages) {
  int rc = check_common(n_heads_q, n_heads_kv, head_dim, dtype);
  if (rc) return rc;
  bf::PagedKV pk{nullptr, 0, 0, 0};
  if (pages && k_cache) {
    long long hold = 0;
    if ((rc = check_pages(*pages, pk, hold))) return rc;
    cache_capacity = (int)std::min<long long>(hold, 0x7fffffffLL);
  }
  if (!q_raw || !k_raw || !q_out || !cu) return fail(BF_ERR_INVALID_ARG, "null tensor or cu_seqlens pointer");
  if (!k_out && !k_cache) return fail(BF_ERR_INVALID_ARG, "k_out and k_cache are both NULL");
  if (k_cache && (!v_cache || !v)) return fail(BF_ERR_INVALID_ARG, "k_cache given without v_cache and v");
  if (!(rope_theta > 1.0) || !std::isfinite(rope_theta))
    return fail(BF_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (batch < 1) return fail(BF_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  if (cu[0] != 0) return fail(BF_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  long long max_end = 0;  // largest P_b + L_b
  for (int b = 0; b < batch; ++b) {
    if (cu[b + 1] <= cu[b])
      return fail(BF_ERR_INVALID_ARG, "cu_seqlens must be strictly increasing (b=%d: %d -> %d)", b, cu[b], cu[b + 1]);
    const long long p0 = pos0 ? pos0[b] : 0;
    if (p0 < 0) return fail(BF_ERR_INVALID_ARG, "pos0[%d] = %lld must be >= 0", b, p0);
    const long long end = p0 + (cu[b + 1] - cu[b]);
    if (end > 0x7fffffffLL) return fail(BF_ERR_INVALID_ARG, "positions of sequence %d exceed 2^31 - 1", b);
    max_end = std::max(max_end, end);
  }
  if (k_cache && max_end > cache_capacity)
    return fail(BF_ERR_INVALID_ARG, "a sequence reaches position %lld, beyond %s %d", max_end - 1,
                pages ? "max_pages_per_seq * page_size" : "cache_capacity", cache_capacity);
  if (!aligned16(q_raw) || !aligned16(k_raw) || !aligned16(q_out) || (k_out && !aligned16(k_out)) ||
      (k_cache && (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(v))))
    return fail(BF_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (forced_launch_failure()) return fail(BF_ERR_HIP, "launch failure forced by BIFOCAL_TEST_FAIL_LAUNCH");
  std::string err;
  rc = bf::run_rope_prefill(q_raw, k_raw, v, q_out, k_out, k_cache, v_cache, cache_capacity, cu, pos0, pk,
                            batch, n_heads_q, n_heads_kv, dtype, rope_theta, (hipStream_t)stream, err);
  if (rc) return fail(rc, "%s", err.c_str());
  g_err.clear();
  return BF_OK;
}

int rope_append_impl(const void* q_raw, const void* k_raw, const void* v_new, void* q_out,
                     void* k_cache, void* v_cache, const int32_t* seqlens, int batch,
                     int cache_capacity, int n_heads_q, int n_heads_kv, int head_dim, int dtype,
                     double rope_theta, void* stream, const ChunkPages* pages) {
  int rc = check_common(n_heads_q, n_heads_kv, head_dim, dtype);
  if (rc) return rc;
  bf::PagedKV pk{nullptr, 0, 0, 0};
  if (pages) {
    long long hold = 0;
    if ((rc = check_pages(*pages, pk, hold))) return rc;
    cache_capacity = (int)std::min<long long>(hold, 0x7fffffffLL);
  }
  if (!q_raw || !k_raw || !v_new || !q_out || !k_cache || !v_cache || !seqlens)
    return fail(BF_ERR_INVALID_ARG, "null tensor or seqlens pointer");
  if (!(rope_theta > 1.0) || !std::isfinite(rope_theta))
    return fail(BF_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (batch < 1 || cache_capacity < 1) return fail(BF_ERR_INVALID_ARG, "batch and cache_capacity must be >= 1");
  for (int b = 0; b < batch; ++b)
    if (seqlens[b] < 1 || seqlens[b] > cache_capacity)
      return fail(BF_ERR_INVALID_ARG, "seqlens[%d] = %d out of [1, %s]", b, seqlens[b],
                  pages ? "max_pages_per_seq * page_size" : "cache_capacity");
  if (!aligned16(q_raw) || !aligned16(k_raw) || !aligned16(v_new) || !aligned16(q_out) ||
      !aligned16(k_cache) || !aligned16(v_cache))
    return fail(BF_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (forced_launch_failure()) return fail(BF_ERR_HIP, "launch failure forced by BIFOCAL_TEST_FAIL_LAUNCH");
  std::string err;
  rc = bf::run_rope_append(q_raw, k_raw, v_new, q_out, k_cache, v_cache, cache_capacity, seqlens, pk,
                           batch, n_heads_q, n_heads_kv, dtype, rope_theta, (hipStream_t)stream, err);
  if (rc) return fail(rc, "%s", err.c_str());
  g_err.clear();
  return BF_OK;
}

}  // namespace

extern "C" {

int64_t bifocal_s_of_L(int64_t L, int64_t w_pre) {
  if (L < 1 || w_pre < 1) return -1;
  const int64_t q = L / w_pre + (L % w_pre != 0 ? 1 : 0);  // ceil(L / w_pre), no overflow
  return q < 1 ? 1 : q;
}

size_t bifocal_workspace_bytes(int32_t phase, int32_t batch, int64_t tokens, int32_t n_heads_q,
                               int32_t n_heads_kv, int32_t head_dim, int32_t dtype) {
  if (batch < 1 || tokens < 1 || n_heads_q < 1 || n_heads_kv < 1 || head_dim != bf::kHeadDim)
    return 0;
  if (dtype != BF_DTYPE_BF16 && dtype != BF_DTYPE_FP32) return 0;
  if (phase == BF_PHASE_PREFILL)
    return prefill_ws_layout(batch, tokens, tokens, n_heads_q, n_heads_kv, dtype).total;
  if (phase == BF_PHASE_DECODE) return bf::decode_workspace_bytes(batch, tokens, n_heads_q);
  return 0;
}

int bifocal_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_host, int32_t batch, int32_t n_heads_q,
                    int32_t n_heads_kv, int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                    double rope_theta, int32_t long_mode, float softmax_scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return run_prefill(true, q, k, v, o, lse, cu_seqlens_host, batch, n_heads_q, n_heads_kv,
                     head_dim, dtype, w0, w_pre, rope_theta, long_mode, softmax_scale, workspace,
                     workspace_bytes, (hipStream_t)stream);
}

size_t bifocal_chunk_workspace_bytes(int32_t batch, int64_t q_tokens, int64_t kv_tokens,
                                     int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                                     int32_t dtype, int32_t paged) {
  if (batch < 1 || q_tokens < 1 || kv_tokens < q_tokens || n_heads_q < 1 || n_heads_kv < 1 ||
      head_dim != bf::kHeadDim)
    return 0;
  if (dtype != BF_DTYPE_BF16 && dtype != BF_DTYPE_FP32) return 0;
  return prefill_ws_layout(batch, q_tokens, kv_tokens, n_heads_q, n_heads_kv, dtype, paged != 0,
                           chunk_split_cap(q_tokens, n_heads_q, n_heads_kv, dtype)).total;
}

int bifocal_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* o,
                          float* lse, const int32_t* cu_q_host, const int32_t* seqlens_host,
                          const int32_t* s_len_host, int32_t batch, int32_t cache_capacity,
                          int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t dtype,
                          int64_t w0, int64_t w_pre, double rope_theta, int32_t long_mode,
                          float softmax_scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return run_chunk(q, k_cache, v_cache, o, lse, cu_q_host, seqlens_host, s_len_host, batch,
                   cache_capacity, n_heads_q, n_heads_kv, head_dim, dtype, w0, w_pre, rope_theta,
                   long_mode, softmax_scale, workspace, workspace_bytes, (hipStream_t)stream);
}

int bifocal_prefill_chunk_paged(const void* q, const void* k_pages, const void* v_pages, void* o,
                                float* lse, const int32_t* block_table, const int32_t* cu_q_host,
                                const int32_t* seqlens_host, const int32_t* s_len_host,
                                int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                                int32_t num_pages, int32_t n_heads_q, int32_t n_heads_kv,
                                int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                                double rope_theta, int32_t long_mode, float softmax_scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const ChunkPages pg{block_table, page_size, max_pages_per_seq, num_pages};
  return run_chunk(q, k_pages, v_pages, o, lse, cu_q_host, seqlens_host, s_len_host, batch, 1,
                   n_heads_q, n_heads_kv, head_dim, dtype, w0, w_pre, rope_theta, long_mode,
                   softmax_scale, workspace, workspace_bytes, (hipStream_t)stream, &pg);
}

int bifocal_prefill_chunk_stored_paged(const void* q, const void* k_pages, const void* v_pages,
                                       void* store, size_t store_bytes, void* o, float* lse,
                                       const int32_t* block_table, const int32_t* cu_q_host,
                                       const int32_t* seqlens_host, const int32_t* s_len_host,
                                       int32_t* store_keys_host, int32_t* store_s_host,
                                       int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                                       int32_t num_pages, int32_t n_heads_q, int32_t n_heads_kv,
                                       int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                                       double rope_theta, int32_t long_mode, float softmax_scale,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  const ChunkPages pg{block_table, page_size, max_pages_per_seq, num_pages};
  const ChunkStore cs{store, store_bytes, store_keys_host, store_s_host};
  return run_chunk(q, k_pages, v_pages, o, lse, cu_q_host, seqlens_host, s_len_host, batch, 1,
                   n_heads_q, n_heads_kv, head_dim, dtype, w0, w_pre, rope_theta, long_mode,
                   softmax_scale, workspace, workspace_bytes, (hipStream_t)stream, &pg, &cs);
}

size_t bifocal_chunk_store_bytes(int32_t batch, int32_t cache_capacity, int32_t n_heads_kv,
                                 int32_t head_dim, int32_t dtype) {
  if (head_dim != bf::kHeadDim || (dtype != BF_DTYPE_BF16 && dtype != BF_DTYPE_FP32)) return 0;
  return chunk_store_bytes(batch, cache_capacity, n_heads_kv, dtype);
}

int bifocal_prefill_chunk_stored(const void* q, const void* k_cache, const void* v_cache,
                                 void* store, size_t store_bytes, void* o, float* lse,
                                 const int32_t* cu_q_host, const int32_t* seqlens_host,
                                 const int32_t* s_len_host, int32_t* store_keys_host,
                                 int32_t* store_s_host, int32_t batch, int32_t cache_capacity,
                                 int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                                 int32_t dtype, int64_t w0, int64_t w_pre, double rope_theta,
                                 int32_t long_mode, float softmax_scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const ChunkStore cs{store, store_bytes, store_keys_host, store_s_host};
  return run_chunk(q, k_cache, v_cache, o, lse, cu_q_host, seqlens_host, s_len_host, batch,
                   cache_capacity, n_heads_q, n_heads_kv, head_dim, dtype, w0, w_pre, rope_theta,
                   long_mode, softmax_scale, workspace, workspace_bytes, (hipStream_t)stream,
                   nullptr, &cs);
}

int bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                   const int32_t* seqlens_host, int32_t batch, int32_t cache_capacity,
                   int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t dtype,
                   int64_t w0, int64_t w_pre, double rope_theta, int32_t long_mode,
                   float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(n_heads_q, n_heads_kv, head_dim, dtype);
  if (rc) return rc;
  if ((rc = check_bifocal_knobs(w0, w_pre, rope_theta, long_mode))) return rc;
  if (dtype != BF_DTYPE_BF16) return fail(BF_ERR_UNSUPPORTED, "decode supports bf16 only");
  std::string err;
  // band only: the plain engine over the keys N - w0 .. N - 1 of each sequence
  const bool band_only = long_mode == BF_LONG_NONE;
  rc = bf::run_decode(!band_only, q, k_cache, v_cache, o, lse, seqlens_host, batch, cache_capacity,
                      n_heads_q, n_heads_kv, w0, w_pre, rope_theta, long_mode, softmax_scale,
                      workspace, workspace_bytes, (hipStream_t)stream, err, band_only ? w0 : 0, nullptr);
  if (rc) return fail(rc, "%s", err.c_str());
  g_err.clear();
  return BF_OK;
}

int bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                           float* lse, const int32_t* seqlens_host, int32_t batch,
                           int32_t cache_capacity, int32_t n_heads_q, int32_t n_heads_kv,
                           int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                           double rope_theta, int32_t long_mode, float softmax_scale,
                           void* stream) {
  int rc = check_common(n_heads_q, n_heads_kv, head_dim, dtype);
  if (rc) return rc;
  if ((rc = check_bifocal_knobs(w0, w_pre, rope_theta, long_mode))) return rc;
  if (dtype != BF_DTYPE_BF16) return fail(BF_ERR_UNSUPPORTED, "decode supports bf16 only");
  const bool band_only = long_mode == BF_LONG_NONE;
  std::string err;
  // every argument is checked (no HIP call) before the scratch is looked up
  rc = bf::run_decode(!band_only, q, k_cache, v_cache, o, lse, seqlens_host, batch, cache_capacity,
                      n_heads_q, n_heads_kv, w0, w_pre, rope_theta, long_mode, softmax_scale, nullptr, 0,
                      (hipStream_t)stream, err, band_only ? w0 : 0, nullptr, true);
  if (rc) return fail(rc, "%s", err.c_str());
  long long max_len = 0;
  for (int b = 0; b < batch; ++b) max_len = std::max<long long>(max_len, seqlens_host[b]);
  const size_t need = bf::decode_workspace_bytes(batch, max_len, n_heads_q);
  const size_t cap = bf::decode_noalloc_capacity();
  if (need > cap)
    return fail(BF_ERR_UNSUPPORTED, "this call needs %zu bytes of decode scratch; the allocation-free "
                "entry point holds %zu (fewer sequences or query heads per call, or bifocal_decode "
                "with a workspace)", need, cap);
  void* ws = nullptr;
  if ((rc = bf::decode_noalloc_scratch((hipStream_t)stream, &ws, err))) return fail(rc, "%s", err.c_str());
  rc = bf::run_decode(!band_only, q, k_cache, v_cache, o, lse, seqlens_host, batch, cache_capacity,
                      n_heads_q, n_heads_kv, w0, w_pre, rope_theta, long_mode, softmax_scale, ws, cap,
                      (hipStream_t)stream, err, band_only ? w0 : 0, nullptr);
  if (rc) return fail(rc, "%s", err.c_str());
  g_err.clear();
  return BF_OK;
}

int bifocal_decode_stored(const void* q, const void* k_cache, const void* v_cache, void* k2_store,
                          void* o, float* lse, const int32_t* seqlens_host, int32_t* store_keys_host,
                          int32_t* store_s_host, int32_t batch, int32_t cache_capacity,
                          int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t dtype,
                          int64_t w0, int64_t w_pre, double rope_theta, int32_t long_mode,
                          float softmax_scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int rc = check_common(n_heads_q, n_heads_kv, head_dim, dtype);
  if (rc) return rc;
  if ((rc = check_bifocal_knobs(w0, w_pre, rope_theta, long_mode))) return rc;
  if (dtype != BF_DTYPE_BF16) return fail(BF_ERR_UNSUPPORTED, "decode supports bf16 only");
  if (long_mode == BF_LONG_NONE)
    return fail(BF_ERR_UNSUPPORTED, "band-only decode has no far keys to store (use bifocal_decode)");
  const bf::DecodeStore st{k2_store, store_keys_host, store_s_host};
  std::string err;
  rc = bf::run_decode(true, q, k_cache, v_cache, o, lse, seqlens_host, batch, cache_capacity,
                      n_heads_q, n_heads_kv, w0, w_pre, rope_theta, long_mode, softmax_scale,
                      workspace, workspace_bytes, (hipStream_t)stream, err, 0, nullptr, false, &st);
  if (rc) return fail(rc, "%s", err.c_str());
  g_err.clear();
  return BF_OK;
}

int bifocal_decode_stored_paged(const void* q, const void* k_pages, const void* v_pages,
                                void* k2_pages, void* o, float* lse, const int32_t* block_table,
                                const int32_t* seqlens_host, int32_t* store_keys_host,
                                int32_t* store_s_host, int32_t batch, int32_t page_size,
                                int32_t max_pages_per_seq, int32_t num_pages, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t head_dim, int32_t dtype, int64_t w0,
                                int64_t w_pre, double rope_theta, int32_t long_mode,
                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                void* stream) {
  int rc = check_common(n_heads_q, n_heads_kv, head_dim, dtype);
  if (rc) return rc;
  if ((rc = check_bifocal_knobs(w0, w_pre, rope_theta, long_mode))) return rc;
  if (dtype != BF_DTYPE_BF16) return fail(BF_ERR_UNSUPPORTED, "decode supports bf16 only");
  if (long_mode == BF_LONG_NONE)
    return fail(BF_ERR_UNSUPPORTED, "band-only decode has no far keys to store (use bifocal_decode_paged)");
  const bf::PagedCache pc{block_table, page_size, max_pages_per_seq, num_pages};
  const bf::DecodeStore st{k2_pages, store_keys_host, store_s_host};
  std::string err;
  rc = bf::run_decode(true, q, k_pages, v_pages, o, lse, seqlens_host, batch, 1, n_heads_q,
                      n_heads_kv, w0, w_pre, rope_theta, long_mode, softmax_scale, workspace,
                      workspace_bytes, (hipStream_t)stream, err, 0, &pc, false, &st);
  if (rc) return fail(rc, "%s", err.c_str());
  g_err.clear();
  return BF_OK;
}

int bifocal_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o,
                         float* lse, const int32_t* block_table, const int32_t* seqlens_host,
                         int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                         int32_t num_pages, int32_t n_heads_q, int32_t n_heads_kv,
                         int32_t head_dim, int32_t dtype, int64_t w0, int64_t w_pre,
                         double rope_theta, int32_t long_mode, float softmax_scale,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(n_heads_q, n_heads_kv, head_dim, dtype);
  if (rc) return rc;
  if ((rc = check_bifocal_knobs(w0, w_pre, rope_theta, long_mode))) return rc;
  if (dtype != BF_DTYPE_BF16) return fail(BF_ERR_UNSUPPORTED, "decode supports bf16 only");
  const bf::PagedCache pc{block_table, page_size, max_pages_per_seq, num_pages};
  std::string err;
  const bool band_only = long_mode == BF_LONG_NONE;
  rc = bf::run_decode(!band_only, q, k_pages, v_pages, o, lse, seqlens_host, batch, 1, n_heads_q,
                      n_heads_kv, w0, w_pre, rope_theta, long_mode, softmax_scale, workspace,
                      workspace_bytes, (hipStream_t)stream, err, band_only ? w0 : 0, &pc);
  if (rc) return fail(rc, "%s", err.c_str());
  g_err.clear();
  return BF_OK;
}

int plain_attention_ref_gpu(int32_t phase, const void* q, const void* k, const void* v, void* o,
                            float* lse, const int32_t* lens_host, int32_t batch,
                            int32_t cache_capacity, int32_t n_heads_q, int32_t n_heads_kv,
                            int32_t head_dim, int32_t dtype, float softmax_scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (phase == BF_PHASE_PREFILL)
    return run_prefill(false, q, k, v, o, lse, lens_host, batch, n_heads_q, n_heads_kv, head_dim,
                       dtype, 0, 1, 10000.0, 0, softmax_scale, workspace, workspace_bytes,
                       (hipStream_t)stream);
  if (phase != BF_PHASE_DECODE) return fail(BF_ERR_INVALID_ARG, "phase must be PREFILL or DECODE (got %d)", phase);
  int rc = check_common(n_heads_q, n_heads_kv, head_dim, dtype);
  if (rc) return rc;
  if (dtype != BF_DTYPE_BF16) return fail(BF_ERR_UNSUPPORTED, "decode supports bf16 only");
  std::string err;
  rc = bf::run_decode(false, q, k, v, o, lse, lens_host, batch, cache_capacity, n_heads_q,
                      n_heads_kv, 0, 1, 10000.0, 0, softmax_scale, workspace, workspace_bytes,
                      (hipStream_t)stream, err, 0, nullptr);
  if (rc) return fail(rc, "%s", err.c_str());
  g_err.clear();
  return BF_OK;
}

int bifocal_test_pair_map(int64_t L, int64_t w0, int64_t w_pre, int32_t long_mode,
                          int8_t* branch_out, int64_t* phi_num_out, void* stream) {
  if (L < 1 || L > 4096) return fail(BF_ERR_INVALID_ARG, "test_pair_map needs 1 <= L <= 4096");
  if (long_mode & BF_LONG_SHIFT) return fail(BF_ERR_INVALID_ARG, "test_pair_map takes FI, PA or band only");
  int rc = check_bifocal_knobs(w0, w_pre, 10000.0, long_mode);
  if (rc) return rc;
  if (!branch_out || (!phi_num_out && long_mode != BF_LONG_NONE))
    return fail(BF_ERR_INVALID_ARG, "null output pointer");
  if (forced_launch_failure()) return fail(BF_ERR_HIP, "launch failure forced by BIFOCAL_TEST_FAIL_LAUNCH");
  const long long s = long_mode == BF_LONG_NONE ? 1 : bifocal_s_of_L(L, w_pre);
  hipError_t e = bf::launch_pair_map(L, w0, s, long_mode, branch_out, (long long*)phi_num_out,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(BF_ERR_HIP, "pair_map launch: %s", hipGetErrorString(e));
  g_err.clear();
  return BF_OK;
}

int bifocal_test_angles(int32_t which, const int64_t* positions_host, int32_t n_pos, int64_t L,
                        int64_t w0, int64_t w_pre, double rope_theta, int32_t long_mode,
                        float* cs_out, void* stream) {
  if (which < 0 || which > 3) return fail(BF_ERR_INVALID_ARG, "which must be 0..3 (got %d)", which);
  if (n_pos < 1 || n_pos > bf::kProbeMax)
    return fail(BF_ERR_INVALID_ARG, "n_pos must be in [1, %d] (got %d)", bf::kProbeMax, n_pos);
  if (!positions_host || !cs_out) return fail(BF_ERR_INVALID_ARG, "null pointer");
  const int base = long_mode & ~BF_LONG_SHIFT;
  if (base != BF_LONG_FI && base != BF_LONG_PA)
    return fail(BF_ERR_INVALID_ARG, "long_mode must be FI or PA (optionally with the shift)");
  int rc = check_bifocal_knobs(w0, w_pre, rope_theta, long_mode);
  if (rc) return rc;
  if (L < 1 || L > (1LL << 31)) return fail(BF_ERR_INVALID_ARG, "L must be in [1, 2^31]");
  bf::AngleProbe a;
  std::memset(&a, 0, sizeof a);
  a.n = n_pos;
  a.mode = base;
  a.shift = (long_mode & BF_LONG_SHIFT) ? 1 : 0;
  a.query = which == 0 ? 1 : 0;
  a.w0 = w0;
  a.N = L;
  for (int i = 0; i < n_pos; ++i) {
    const long long p = positions_host[i];
    if (p < 0 || (which != 3 && p >= L) || p + 1 > (1LL << 31))
      return fail(BF_ERR_INVALID_ARG, "position %lld out of range", p);
    a.pos[i] = p;
    const long long s = bifocal_s_of_L(which == 3 ? p + 1 : L, w_pre);
    if (s > (1LL << 30)) return fail(BF_ERR_INVALID_ARG, "s(L) out of range");
    a.s[i] = s;
  }
  if (forced_launch_failure()) return fail(BF_ERR_HIP, "launch failure forced by BIFOCAL_TEST_FAIL_LAUNCH");
  const bf::ThetaTable tt = theta_table(rope_theta);
  const hipError_t e = which <= 1 ? bf::launch_prep_angles(a, tt, cs_out, (hipStream_t)stream)
                                  : bf::launch_decode_angles(a, tt, which, cs_out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BF_ERR_HIP, "angle probe launch: %s", hipGetErrorString(e));
  g_err.clear();
  return BF_OK;
}

int bifocal_rope_prefill(const void* q_raw, const void* k_raw, const void* v, void* q_out,
                         void* k_out, void* k_cache, void* v_cache, int32_t cache_capacity,
                         const int32_t* cu, const int32_t* pos0, int32_t batch, int32_t n_heads_q,
                         int32_t n_heads_kv, int32_t head_dim, int32_t dtype, double rope_theta,
                         void* stream) {
  return rope_prefill_impl(q_raw, k_raw, v, q_out, k_out, k_cache, v_cache, cache_capacity, cu, pos0,
                           batch, n_heads_q, n_heads_kv, head_dim, dtype, rope_theta, stream, nullptr);
}

int bifocal_rope_prefill_paged(const void* q_raw, const void* k_raw, const void* v, void* q_out,
                               void* k_out, void* k_pages, void* v_pages, const int32_t* block_table,
                               int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                               const int32_t* cu, const int32_t* pos0, int32_t batch,
                               int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                               int32_t dtype, double rope_theta, void* stream) {
  if (!k_pages) return fail(BF_ERR_INVALID_ARG, "k_pages is NULL");
  const ChunkPages pg{block_table, page_size, max_pages_per_seq, num_pages};
  return rope_prefill_impl(q_raw, k_raw, v, q_out, k_out, k_pages, v_pages, 0, cu, pos0, batch,
                           n_heads_q, n_heads_kv, head_dim, dtype, rope_theta, stream, &pg);
}

int bifocal_rope_append(const void* q_raw, const void* k_raw, const void* v_new, void* q_out,
                        void* k_cache, void* v_cache, const int32_t* seqlens, int32_t batch,
                        int32_t cache_capacity, int32_t n_heads_q, int32_t n_heads_kv,
                        int32_t head_dim, int32_t dtype, double rope_theta, void* stream) {
  return rope_append_impl(q_raw, k_raw, v_new, q_out, k_cache, v_cache, seqlens, batch, cache_capacity,
                          n_heads_q, n_heads_kv, head_dim, dtype, rope_theta, stream, nullptr);
}

int bifocal_rope_append_paged(const void* q_raw, const void* k_raw, const void* v_new, void* q_out,
                              void* k_pages, void* v_pages, const int32_t* block_table,
                              int32_t page_size, int32_t max_pages_per_seq, int32_t num_pages,
                              const int32_t* seqlens, int32_t batch, int32_t n_heads_q,
                              int32_t n_heads_kv, int32_t head_dim, int32_t dtype,
                              double rope_theta, void* stream) {
  const ChunkPages pg{block_table, page_size, max_pages_per_seq, num_pages};
  return rope_append_impl(q_raw, k_raw, v_new, q_out, k_pages, v_pages, seqlens, batch, 1, n_heads_q,
                          n_heads_kv, head_dim, dtype, rope_theta, stream, &pg);
}

const char* bifocal_last_error(void) { return g_err.c_str(); }

}  // extern "C"
