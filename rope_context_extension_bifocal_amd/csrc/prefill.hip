// Bifocal RoPE attention, causal prefill on gfx950 (CDNA4).
//
// Kernels:
//   correction_prep_kernel  far-branch copies q'' = R(Delta(i)) q', k'' = R(Delta(j)) k'
//                           with Delta_m(p) = theta_m * (phi(p) - p), angles in fp64
//                           (and, for a paged key source, the packed copy of k')
//                           [ai-feeds.com summary, "关键模块" item 3: correction
//                            rotation of cached keys so that long-range keys meet
//                            the query at the scaled positions]
//   vt_transpose_*_kernel   V -> V^T, each sequence padded to a multiple of 64 keys
//
// The queries of a launch are packed rows; row r of sequence b sits at
// position qpos[b] + r (0 for a one-shot prefill, N - Lq for a chunk of
// queries against a KV cache) and sees keys 0 .. qpos[b] + r. Keys come from a
// packed tensor or a cache (SeqTable: k_hstride, kbase).
//   prefill_bf16_kernel     MFMA 32x32x16 bf16 tile loop, one online softmax
//   prefill_f32_kernel      the same loop on MFMA 32x32x2 f32 for fp32 inputs
//   pair_map_kernel         test hook: the device pair rule and position map
//
// Tile loop [ai-feeds.com summary, "关键模块" items 1 and 3; seventnews.com (FR),
// fusion paragraph]: every causal pair is either local (i - j < w0: original
// RoPE, q' . k') or far (q'' . k''). In the bf16 kernel the far branch and the
// local branch run as two passes over their own key-tile ranges, sharing one
// online-softmax state; the fp32 kernel visits the tiles once in ascending
// order and, on a tile holding both kinds, computes both score blocks and
// picks per element. Either way each pair enters the softmax exactly once and
// the scaled-branch work over the band that the inclusion-exclusion merge
// would subtract again is never done.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "bf_common.h"

namespace bf {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;  // 8 packed bf16
typedef __attribute__((ext_vector_type(4))) unsigned int du32x4;

// ----------------------------------------------------------------- helpers
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Local-window rule for one causal pair [ai-feeds.com summary, "关键模块" item 1].
__device__ __forceinline__ bool pair_is_local(long long i, long long j, long long w0) {
  return i - j < w0;
}

// (phi(p) - p) * s as an exact integer: FI phi = p / s gives -p (s - 1);
// PA phi = floor(p / s) gives (floor(p / s) - p) * s.
__device__ __forceinline__ long long corr_num(long long p, long long s, int mode) {
  return mode == 1 ? (p / s - p) * s : -p * (s - 1);
}

// MFMA row r of a 32-row key block -> key index inside the block. Chosen so
// that the 32x32 accumulator register r of lane half h holds key
// 16 * (r / 8) + 8 * h + r % 8, i.e. 8 consecutive keys per lane half for
// every 8 consecutive registers: the P operand of the PV product then lines
// up with 16-byte reads of a V^T row.
__device__ __forceinline__ int key_of_mfma_row(int r) {
  const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
  return ((a >> 1) << 4) | (h << 3) | ((a & 1) << 2) | b;
}

__device__ __forceinline__ int key_of_acc(int r, int hl) {  // key of acc register r
  return ((r >> 3) << 4) | (hl << 3) | (r & 7);
}

// Work item of a workgroup: ranks run over the sequences in the host's work
// order (order[i] owns ranks ioff[i] .. ioff[i + 1] - 1) and, inside a
// sequence, over its row blocks last (heaviest) first. The workgroups that
// run at the same time then mostly share one sequence's keys, which the XCD's
// L2 serves, and the lightest items come last.
// The lookup is wave-parallel: lane i loads ioff[i + 1], ioff[i] and
// order[i] (one memory round trip), a ballot counts the sequences that start
// at or below the rank, and that count selects the entries by lane reads.
// (A search would chain one load per step at the start of every workgroup.)
__device__ __forceinline__ void decode_item(const SeqTable& st, int rank, int& b, int& rb) {
  static_assert(kMaxSeqPerLaunch == 64, "one table entry per lane");
  const int lane = threadIdx.x & 63;
  const int next = st.ioff[lane + 1];  // start of sequence lane + 1 in the order
  const int own = st.ioff[lane], ord = st.order[lane];
  const int pos = __popcll(__ballot(lane + 1 < st.n && next <= rank));
  b = __builtin_amdgcn_readlane(ord, pos);
  rb = st.nrb[b] - 1 - (rank - __builtin_amdgcn_readlane(own, pos));
}

// ----------------------------------------------------------------- prep
// One thread per (token, group of E = 16 / sizeof(T) rotary pairs): it forms
// the E angles once and applies them to the token's row in every head,
// reading and writing 16 bytes of each half of the row (pairs m0 .. m0 + E - 1
// and m0 + 64 ..). blockIdx.y = 0 rotates the queries (positions qpos[b] +
// row), 1 the keys (positions 0 .. N_b - 1, read from the K layout, written
// packed). The angle is formed in fp64 from an exact integer numerator, so it
// stays accurate at 128K positions (theta_0 * p ~ 1e5 rad), and is applied in
// fp32.
template <typename T>
struct Chunk16 {  // 16 bytes of T as floats
  static constexpr int E = 16 / (int)sizeof(T);
  float x[E];
  __device__ __forceinline__ void load(const T* p) {
    const uint4 u = *(const uint4*)p;
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      x[0] = __uint_as_float(u.x);
      x[1] = __uint_as_float(u.y);
      x[2] = __uint_as_float(u.z);
      x[3] = __uint_as_float(u.w);
    }
  }
  __device__ __forceinline__ void store(T* p) const {
    uint4 u;
    if constexpr (sizeof(T) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)f32_to_bf16(x[2 * i]) | ((uint32_t)f32_to_bf16(x[2 * i + 1]) << 16);
      u = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      u = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                     __float_as_uint(x[3]));
    }
    *(uint4*)p = u;
  }
};

// Row (in elements / kHeadDim) of key j of launch sequence b, KV head h, in a
// K / V source: the SeqTable layout, or pages through the block table.
__device__ __forceinline__ long long kv_row(const PagedKV& pk, const SeqTable& st,
                                            long long k_hstride, int Hkv, int b, int h,
                                            long long j) {
  if (pk.block_table == nullptr) return (long long)h * k_hstride + st.kbase[b] + j;
  int pg = pk.block_table[(size_t)b * pk.max_pages + (j >> pk.page_log2)];
  pg = min(max(pg, 0), pk.num_pages - 1);
  return (((long long)pg * Hkv + h) << pk.page_log2) + (j & ((1LL << pk.page_log2) - 1));
}

// Sequence of packed token tok along offsets cu[0 .. n]: the last b with
// cu[b] <= tok.
__device__ __forceinline__ int seq_of_tok(const int* cu, int n, int tok) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= tok) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Correction angle of the prep pass: (phi(pos) - pos) * s as an exact
// integer, plus for queries with the band-edge continuity shift
// (w0 - phi(w0)) * s = w0 (s - 1) (FI) or (w0 - floor(w0 / s)) s (PA); the
// angle theta_m * num / s is formed in fp64 and rounded to fp32 cos / sin.
__device__ __forceinline__ long long prep_num(long long pos, long long s, int mode, bool query,
                                              int shift, long long w0) {
  long long num = corr_num(pos, s, mode);
  if (query && shift) num += mode == 1 ? (w0 - w0 / s) * s : w0 * (s - 1);
  return num;
}
__device__ __forceinline__ void prep_cos_sin(double th_m, double ratio, float& c, float& sn) {
  double sd, cd;
  sincos(th_m * ratio, &sd, &cd);
  c = (float)cd;
  sn = (float)sd;
}

template <typename T>
__global__ __launch_bounds__(256) void correction_prep_kernel(PrepParams p, SeqTable st,
                                                              ThetaTable tt) {
  constexpr int E = Chunk16<T>::E;   // pairs per thread
  constexpr int TPR = kPairs / E;    // threads per token
  constexpr int TOK = 256 / TPR;     // tokens per workgroup
  const bool keys = blockIdx.y == 1;
  const int* cu = keys ? st.kcu : st.cu;
  const int tok = cu[0] + blockIdx.x * TOK + (int)threadIdx.x / TPR;
  const int m0 = ((int)threadIdx.x % TPR) * E;
  if (tok >= cu[st.n]) return;
  const int b = seq_of_tok(cu, st.n, tok);
  const int s = st.s[b];
  const long long row = tok - cu[b] + (keys ? p.kfirst[b] : 0);
  // s = 1: no far branch for this sequence; a store already holds the k'' of
  // its keys below krot
  const bool rot = s > 1 && !(keys && p.k2_cap > 0 && row < p.krot[b]);
  const bool copy = keys && p.kcopy != nullptr;  // paged keys: gather the packed copy
  if (!rot && !copy) return;
  if (keys && row < (long long)st.vt_t0[b] * kKeyTile) return;  // key no window reaches
  float c[E], sn[E];
  if (rot) {
    const long long pos = keys ? row : st.qpos[b] + row;
    const long long num = prep_num(pos, s, p.long_mode, !keys, p.shift, p.w0);
    const double ratio = (double)num / (double)s;
#pragma unroll
    for (int e = 0; e < E; ++e) prep_cos_sin(tt.th[m0 + e], ratio, c[e], sn[e]);
  }
  const int nh = keys ? p.Hkv : p.Hq;
  for (int h = 0; h < nh; ++h) {
    const T* src;
    T* dst;
    if (keys) {
      src = (const T*)p.k + kv_row(p.pk, st, p.k_hstride, p.Hkv, b, h, row) * kHeadDim;
      dst = (T*)p.k2 + (p.k2_cap > 0 ? ((size_t)b * p.Hkv + h) * p.k2_cap + row
                                     : (size_t)h * p.Tk + tok) * kHeadDim;
    } else {
      src = (const T*)p.q + ((size_t)h * p.T + tok) * kHeadDim;
      dst = (T*)p.q2 + ((size_t)h * p.T + tok) * kHeadDim;
    }
    if (copy) {  // 16-byte copies of both halves, unconverted
      T* cp = (T*)p.kcopy + ((size_t)h * p.Tk + tok) * kHeadDim;
      *(uint4*)(cp + m0) = *(const uint4*)(src + m0);
      *(uint4*)(cp + kPairs + m0) = *(const uint4*)(src + kPairs + m0);
    }
    if (!rot) continue;
    Chunk16<T> x0, x1, y0, y1;
    x0.load(src + m0);
    x1.load(src + kPairs + m0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      y0.x[e] = x0.x[e] * c[e] - x1.x[e] * sn[e];
      y1.x[e] = x1.x[e] * c[e] + x0.x[e] * sn[e];
    }
    y0.store(dst + m0);
    y1.store(dst + kPairs + m0);
  }
}

// V (the layout of K) -> V^T in 64-key tiles: tile t (global over the padded
// key axis, sequence b owns tiles vt_off[b] / 64 ..) of KV head h is the
// contiguous block vt[(h * Tpad / 64 + t) * D * 64 ..], laid out
// [head dim][64 keys]. Keys past a sequence's length are zero.
// Sequence of the padded V^T column c: the last b with vt_off[b] <= c.
__device__ __forceinline__ int seq_of_vt(const SeqTable& st, int c) {
  int lo = 0, hi = st.n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (st.vt_off[mid] <= c) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Destination tile of padded column c (key p0 of sequence b, KV head h): the
// packed axis, or the store's tile of (b, h, p0 / 64).
__device__ __forceinline__ size_t vt_tile_index(const VtParams& p, int b, int h, int c, int p0) {
  return p.store_tiles > 0 ? ((size_t)b * p.Hkv + h) * p.store_tiles + p0 / kKeyTile
                           : (size_t)h * (p.Tpad / kKeyTile) + c / kKeyTile;
}

// fp32 V^T: one 256-thread workgroup per (64-key tile, KV head), through LDS.
__global__ __launch_bounds__(256) void vt_transpose_f32_kernel(VtParams p, SeqTable st) {
  __shared__ float tile[kKeyTile][kHeadDim + 1];
  __shared__ long long rows[kKeyTile];  // V row of each key of the tile, -1 past the end
  const int c = st.vt_off[0] + blockIdx.x * kKeyTile;
  const int h = blockIdx.y;
  const int b = seq_of_vt(st, c);
  const int p0 = c - st.vt_off[b] + st.vt_t0[b] * kKeyTile;  // first key of the tile
  const int L = st.kcu[b + 1] - st.kcu[b];
  if (threadIdx.x < kKeyTile) {
    const int j = p0 + threadIdx.x;
    rows[threadIdx.x] = j < L ? kv_row(p.pk, st, p.k_hstride, p.Hkv, b, h, j) : -1;
  }
  __syncthreads();
  const float* v = (const float*)p.v;
  for (int e = threadIdx.x; e < kKeyTile * kHeadDim; e += 256) {
    const int r = e / kHeadDim, d = e % kHeadDim;
    const long long vr = rows[r];
    tile[r][d] = vr >= 0 ? v[(size_t)vr * kHeadDim + d] : 0.f;
  }
  __syncthreads();
  float* vt = (float*)p.vt + vt_tile_index(p, b, h, c, p0) * (kHeadDim * kKeyTile);
  for (int e = threadIdx.x; e < kKeyTile * kHeadDim; e += 256) {
    const int d = e / kKeyTile, r = e % kKeyTile;
    vt[d * kKeyTile + r] = tile[r][d];
  }
}

// bf16 V^T: one 128-thread workgroup per (64-key tile, KV head), no LDS for
// the data. Thread t moves the block of keys 8 kb .. 8 kb + 7 and head dims
// 8 db .. 8 db + 7 (kb = t % 8, db = t / 8): eight 16-byte reads (one per
// key), a transpose in registers, and eight 16-byte writes (one per head
// dim, 8 keys each). Each read or write instruction of a wave then covers
// whole 128-byte lines: 8 keys x 128 bytes of V, or 8 full V^T rows.
__global__ __launch_bounds__(128) void vt_transpose_bf16_kernel(VtParams p, SeqTable st) {
  __shared__ long long rows[kKeyTile];  // V row of each key of the tile, -1 past the end
  const int c = st.vt_off[0] + blockIdx.x * kKeyTile;
  const int h = blockIdx.y;
  const int b = seq_of_vt(st, c);
  const int p0 = c - st.vt_off[b] + st.vt_t0[b] * kKeyTile;  // first key of the tile
  const int L = st.kcu[b + 1] - st.kcu[b];
  if (threadIdx.x < kKeyTile) {
    const int j = p0 + threadIdx.x;
    rows[threadIdx.x] = j < L ? kv_row(p.pk, st, p.k_hstride, p.Hkv, b, h, j) : -1;
  }
  __syncthreads();
  const int kb = threadIdx.x & 7, db = threadIdx.x >> 3;
  const uint16_t* v = (const uint16_t*)p.v;
  uint32_t in[8][4];  // key 8 kb + k: head dims 8 db + 2 w (low half) and + 1 (high half)
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const long long vr = rows[kb * 8 + k];
    uint4 x = make_uint4(0, 0, 0, 0);
    if (vr >= 0) x = *(const uint4*)(v + (size_t)vr * kHeadDim + db * 8);
    in[k][0] = x.x;
    in[k][1] = x.y;
    in[k][2] = x.z;
    in[k][3] = x.w;
  }
  uint16_t* vt = (uint16_t*)p.vt + vt_tile_index(p, b, h, c, p0) * (kHeadDim * kKeyTile);
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // head dim 8 db + i: keys 8 kb .. 8 kb + 7, two per word
    uint32_t w[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint32_t x = in[2 * a][i >> 1], y = in[2 * a + 1][i >> 1];
      w[a] = (i & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
    }
    *(uint4*)(vt + (size_t)(db * 8 + i) * kKeyTile + kb * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ----------------------------------------------------------------- main
// Shared work-item geometry of both element types.
// Rows index the packed queries of the sequence (0 .. L - 1); the query of
// row r sits at position qp + r and sees keys 0 .. qp + r.
struct Item {
  int kvh, hq, b, tok0, L, qp, R0, r0, nkt, split;
  long long w0;
};

template <bool BIFOCAL, bool BAND>
__device__ __forceinline__ Item make_item(const PrefillParams& p, const SeqTable& st, int wave,
                                          int wave_rows, int id) {
  Item it;
  it.kvh = id % p.Hkv;
  const int r1 = id / p.Hkv;
  const int hsub = r1 % p.n_hsub;
  const int r2 = r1 / p.n_hsub;
  // key split in the high bits: the workgroups in flight together then share
  // one key range
  it.split = r2 / p.total_items;
  const int rank = r2 - it.split * p.total_items;
  int rb;
  decode_item(st, rank, it.b, rb);
  it.tok0 = st.cu[it.b];
  it.L = st.cu[it.b + 1] - it.tok0;
  it.qp = st.qpos[it.b];
  // s = 1 means the far branch equals the local one: treat every pair as local;
  // band-only attention keeps the window whatever s is
  it.w0 = (BIFOCAL && (BAND || st.s[it.b] > 1)) ? p.w0 : (1LL << 62);
  const int hw = wave % p.hpw, pw = wave / p.hpw;
  it.hq = it.kvh * p.G + hsub * p.hpw + hw;
  it.R0 = rb * p.P_wg;
  it.r0 = it.R0 + pw * wave_rows;
  const int wg_end = it.qp + min(it.R0 + p.P_wg, it.L);  // keys < wg_end
  it.nkt = (wg_end + kKeyTile - 1) / kKeyTile;
  return it;
}

// Next work item of a persistent workgroup (PrefillParams::item_ctr): queue r
// holds the item ids r, r + 8, r + 16, ... below n, in that order, which
// with the KV head in the low bits of the id is one KV head's work, heaviest
// first. A workgroup takes the next id of its own XCD's queue, so each XCD's
// L2 still serves one KV head, and once that queue is empty the next id of
// the following queues: XCDs that run faster take over the last items of
// slower ones instead of idling. A failed claim means that queue is empty
// for good; -1 when every queue is.
__device__ __forceinline__ int claim_item(int* ctr, int n) {
  const int xcc = (int)__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7;  // XCC_ID
  for (int i = 0; i < 8; ++i) {
    const int r = (xcc + i) & 7;
    const int len = (n - r + 7) >> 3;
    if (len <= 0) continue;
    const int k = atomicAdd(ctr + r, 1);
    if (k < len) return r + 8 * k;
  }
  return -1;
}

// Key-tile ranges of the two passes for a workgroup's query positions
// R0 .. Rl: the far pass visits tiles [0, far_end) (a far pair needs a key
// j <= Rl - w0), the local pass [loc_b, nkt) (a local pair needs j > R0 - w0).
// w0 is the effective window (2^62 when every pair is local).
template <bool BIFOCAL, bool BAND>
__device__ __forceinline__ void pass_ranges(long long R0, long long Rl, int nkt, long long w0,
                                            int& far_end, int& loc_b) {
  far_end = (BIFOCAL && !BAND && Rl - w0 >= 0) ? min(nkt, (int)((Rl - w0) / kKeyTile) + 1) : 0;
  loc_b = nkt;
  if (w0 > 0) {
    const long long first = R0 - w0 + 1;  // smallest key with a local pair
    loc_b = first <= 0 ? 0 : (int)min((long long)nkt, first / kKeyTile);
  }
}

// Tile needs, for the whole workgroup (query positions R0 .. R0 + P_wg - 1)
// and keys c0 .. c0 + 63: any far pair / any local pair.
template <bool BIFOCAL>
__device__ __forceinline__ void tile_needs(long long R0, long long P_wg, long long c0,
                                           long long w0, bool& need_far, bool& need_loc) {
  need_far = BIFOCAL && (R0 + P_wg - 1 - c0 >= w0);
  need_loc = !BIFOCAL || (w0 > 0 && R0 - (c0 + kKeyTile - 1) < w0);
}

__device__ __forceinline__ void online_softmax_rescale(float& m_run, float& l_run, float mx,
                                                       float scale_log2, float& mbase,
                                                       float& alpha) {
  const float mnew = fmaxf(m_run, mx * scale_log2);
  mbase = (mnew == -INFINITY) ? 0.f : mnew;
  alpha = __builtin_amdgcn_exp2f(m_run - mbase);
  m_run = mnew;
}

// --------------------------------------------------------------- bf16
// Workgroup: 4 waves; wave = (query head, 32 query positions). The G query
// heads of one KV group share every staged K/V tile. Scores are formed as
// S^T = K Q^T on MFMA 32x32x16 blocks (keys x queries) and the output as
// O^T += V^T P^T (head dims x queries); a lane owns one query column, so a row
// max needs one exchange with the other lane half and the row sum none until
// the end.
//
// The far branch and the local branch run as two passes over their own tile
// ranges with one online-softmax state: the far pass (q'' . k'' on every tile
// that holds a far pair, local pairs masked out) leaves its partial
// (m, l, O) in place, and the local pass (q' . k' on every tile that holds a
// band pair, far pairs masked out) continues from it. Carrying the state over
// is the log-sum-exp merge of the two branch partials, so every causal pair is
// counted once and the scaled-branch work over the band is never done. Only
// the one or two tiles at the window edge are visited by both passes.
//
// Two 4-wave workgroups share a CU, so each SIMD runs two independent waves
// whose softmax (VALU) and matrix (MFMA) phases overlap. K and V^T tiles (64
// keys) are staged by direct global->LDS loads one tile ahead (two-slot
// rings); within a tile the MFMA operands are read from LDS two MFMA steps
// ahead of their use. The O accumulator is rescaled only when a row max grows
// by more than 2^8: numerator and denominator share the same stale max, so
// the result is unchanged, and probabilities stay below 2^8.
constexpr float kRescaleLog2 = 8.f;
constexpr int kSlot = 1024;  // 16-byte chunks per staged 64 x 128 bf16 tile
constexpr int kBf16Waves = 4;
constexpr int kStageIters = kSlot / (64 * kBf16Waves);  // 1 KiB loads per wave per tile

struct WaveRows {
  int r0;  // first query row of the wave (sequence-relative)
  int p0;  // its position (r0 + qpos)
  int L;   // query rows of the sequence
  int w0;  // local window, clamped to 2^30 (s = 1 or the plain engine: all local)
};

struct RowState {
  float m_used;  // stale row max in scaled log2 units (-inf: no key yet)
  float l_part;  // this lane half's share of the row sum
  float alpha;   // pending factor for the O accumulator
  bool rescale;  // (wave-uniform) alpha differs from 1
};

// apply a pending rescale of the O accumulator
__device__ __forceinline__ void apply_rescale(RowState& rs, f32x16 (&oacc)[4]) {
  if (rs.rescale) {
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= rs.alpha;
    rs.alpha = 1.f;
    rs.rescale = false;
  }
}

// LDS byte addresses of MFMA operand fragments. Both swizzles XOR the chunk
// index with lane bits only, so the address of k-step t is one v_xad of a
// lane base: base + ((step bits) ^ lane swizzle). The lane swizzle is made
// opaque at each use so that the compiler recomputes the per-step addresses
// (one instruction each) instead of holding all of them in registers.
struct FragAddr {
  uint32_t k_base, k_sw;  // K tile: row key_of_mfma_row(li), chunk (2 t + hl) ^ (row % 16)
  uint32_t v_base, v_sw;  // V^T tile: head dim li (+ 32 db), chunk (4 jb + 2 u + hl) ^ ((li / 2) % 8)
};

// k_base / v_base are absolute LDS byte addresses of slot 0 of the K / V^T
// rings; other slots and the second 32-key block are immediate offsets.
__device__ __forceinline__ FragAddr frag_addr(int li, int hl, const uint4* sK, const uint4* sV) {
  FragAddr fa;
  const int row0 = key_of_mfma_row(li), sk = row0 & 15;
  fa.k_base = (uint32_t)(uintptr_t)sK + (uint32_t)(row0 * 256 + ((hl ^ sk) & 1) * 16);
  fa.k_sw = (uint32_t)((sk & 14) * 16);
  const int sv = (li >> 1) & 7;
  fa.v_base = (uint32_t)(uintptr_t)sV + (uint32_t)(li * 128 + ((hl ^ sv) & 1) * 16);
  fa.v_sw = (uint32_t)((sv & 6) * 16);
  return fa;
}

__device__ __forceinline__ bf16x8 lds_at(uint32_t addr) {
  const du32x4 v = *(const __attribute__((address_space(3))) du32x4*)addr;
  return __builtin_bit_cast(bf16x8, v);
}

// Waits for all outstanding LDS reads. Written with the builtin (not inline
// asm) so that the compiler's wait insertion knows the reads are complete.
// Explicit waits are used in the tile loops because after a direct
// global->LDS load the compiler only emits full LDS waits anyway (those do not
// wait for the direct loads themselves); placing them before the next operand
// batch is issued keeps that batch in flight.
__device__ __forceinline__ void lds_reads_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// QK^T of one tile: S[blk] (keys 32 blk .. 32 blk + 31 x the wave's 32
// queries). K operands are read in batches of four, one batch ahead of their
// MFMAs, with one full LDS wait per batch (see lds_reads_done).
__device__ __forceinline__ void qk_tile(uint32_t slot_off, const bf16x8 (&q)[8], FragAddr fa,
                                        f32x16 (&S)[2]) {
  asm volatile("" : "+v"(fa.k_sw));
  bf16x8 fr[16];
  auto load = [&](int i) {  // MFMA i: k-step t = i / 2, key block blk = i % 2
    const int t = i >> 1, blk = i & 1;
    fr[i] = lds_at((((uint32_t)(32 * t) ^ fa.k_sw) + fa.k_base) + slot_off + blk * (32 * 256));
  };
  S[0] = f32x16{};
  S[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < 4; ++i) load(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    lds_reads_done();
    if (b < 3) {
#pragma unroll
      for (int j = 0; j < 4; ++j) load(4 * b + 4 + j);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * b + j;
      S[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], q[i >> 1], S[i & 1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Mask a tile (keys c0 .. c0 + 63) for a pass: the far pass keeps pairs with
// i - j >= w0, the local pass keeps 0 <= i - j < w0.
template <bool FAR>
__device__ __forceinline__ void mask_tile(f32x16 (&S)[2], const WaveRows& wr, int c0, int li,
                                          int hl) {
  const int dmax = wr.p0 + 31 - c0;
  const int dmin = wr.p0 - (c0 + 63);
  const bool full = FAR ? (dmin >= wr.w0) : (dmin >= 0 && dmax < wr.w0);
  if (full) return;
  const int base = wr.p0 + li - c0 - 8 * hl;  // i - j = base - 32 jb - 16 (r / 8) - r % 8
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = base - 32 * jb - 16 * (r >> 3) - (r & 7);
      const bool keep = FAR ? (d >= wr.w0) : (d >= 0 && d < wr.w0);
      if (!keep) S[jb][r] = -INFINITY;
    }
}

__device__ __forceinline__ void pv_tile(uint32_t slot_off, const u32x4 (&P)[2][2], FragAddr fa,
                                        f32x16 (&oacc)[4]) {
  asm volatile("" : "+v"(fa.v_sw));
  bf16x8 a[4][2][2];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t off = ((uint32_t)(64 * jb + 32 * u) ^ fa.v_sw) + fa.v_base;
#pragma unroll
      for (int db = 0; db < 4; ++db) a[db][jb][u] = lds_at(off + slot_off + db * 32 * 128);
    }
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[db][jb][u], __builtin_bit_cast(bf16x8, P[jb][u]),
                                                           oacc[db], 0, 0, 0);
  // operands two MFMAs ahead
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int i = 0; i < 14; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier that waits for this wave's LDS reads but not for its
// outstanding global->LDS loads (those are waited for explicitly).
__device__ __forceinline__ void slot_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// Per-lane byte offsets of the direct global -> LDS staging, fixed for a pass
// (16 bytes per lane, 1 KiB per wave instruction, kStageIters instructions per
// wave, tile and operand). LDS chunk p of a K tile holds key row p / 16 and
// swizzled column (p % 16) ^ (row % 16); chunk p of a V^T tile holds head dim
// d = p / 8 and key chunk (p % 8) ^ ((d / 2) % 8). Both swizzles keep the 16
// lanes of one LDS read cycle on distinct banks.
struct StageOffsets {
  uint32_t k;  // byte offset inside a 64-key K tile of instruction 0 (key row = offset / 256)
  uint32_t v;  // byte offset inside a V^T tile of instruction 0
};
// Instruction i of a wave covers chunks p + 256 i: the swizzled column does
// not depend on i (row % 16 and (d / 2) % 8 only see the wave and lane bits),
// so instruction i is instruction 0 moved by 4 KiB.
constexpr uint32_t kStageStride = 4096;

__device__ __forceinline__ StageOffsets stage_offsets(int wave, int lane) {
  StageOffsets so;
  const int p = wave * 64 + lane;
  const int row = p >> 4, col = (p & 15) ^ (row & 15);
  so.k = (uint32_t)(row * kHeadDim + col * 8) * 2u;
  const int d = p >> 3, vc = (p & 7) ^ ((d >> 1) & 7);
  so.v = (uint32_t)(d * kKeyTile + vc * 8) * 2u;
  return so;
}

// A wave-uniform pointer, held in scalar registers (the loads below then use
// a scalar base plus a 32-bit per-lane offset).
__device__ __forceinline__ const char* scalar_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// Direct global -> LDS staging of one 64-key tile through a buffer resource
// whose base is the tile start and whose size runs to the end of the tensor:
// instruction i of a wave reads 1 KiB at lane offset (fixed per pass) + 4 KiB
// i. Base and size sit in scalar registers, so a load costs no vector
// arithmetic. K rows past a sequence's last key read whatever the next rows of
// the K tensor hold (the next tokens of a packed tensor, or cache slots past
// N): every score of such a key is replaced by -inf before use, and reads past
// the tensor end return zeros (buffer range check). V^T tiles are zero-padded
// per sequence, so P = 0 never meets a non-finite value.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* tile, const char* end) {
  const long long left = (long long)(end - tile);
  const int n = (int)(left < 0 ? 0 : left < 0x7fffffffLL ? left : 0x7fffffffLL);
  return __builtin_amdgcn_make_buffer_rsrc((void*)tile, (short)0, n, 0x00020000);
}

__device__ __forceinline__ void b2lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      uint4* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           soff, 0, 0);
}

struct KStage {
  uint32_t off[kStageIters];  // lane byte offsets of the K loads inside a tile (range-checked)
};

__device__ __forceinline__ KStage k_stage_offsets(const StageOffsets& so) {
  KStage ks;
#pragma unroll
  for (int i = 0; i < kStageIters; ++i) ks.off[i] = so.k + i * kStageStride;
  return ks;
}

__device__ __forceinline__ void stage_k(uint4* slot, __amdgpu_buffer_rsrc_t r, const KStage& ks,
                                        int wave) {
#pragma unroll
  for (int i = 0; i < kStageIters; ++i) b2lds(r, ks.off[i], 0, slot + (kBf16Waves * i + wave) * 64);
}

__device__ __forceinline__ void stage_v(uint4* slot, __amdgpu_buffer_rsrc_t r, uint32_t so_v, int wave) {
#pragma unroll
  for (int i = 0; i < kStageIters; ++i)
    b2lds(r, so_v, i * kStageStride, slot + (kBf16Waves * i + wave) * 64);
}

// Row max over the two lane halves that hold one query row: one cross-half
// lane swap (no LDS round trip). max3 of the value and both swap results is
// the row max whichever half each result comes from.
__device__ __forceinline__ float row_max_halves(float m) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(m, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Softmax of one tile's (already masked) scores: row max, lazy rescale
// decision, probabilities (bf16) and row sum. Branch-free, so that it can
// share a scheduling region with the next tile's QK MFMAs: the decision to
// move the stale max is a wave-wide ballot applied with selects (when nothing
// moves, alpha = exp2(0) = 1 exactly).
__device__ __forceinline__ void softmax_tile(f32x16 (&S)[2], float sc, RowState& rs,
                                             u32x4 (&P)[2][2]) {
  float m = -INFINITY;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) m = fmaxf(fmaxf(m, S[jb][r]), S[jb][r + 1]);
  m = row_max_halves(m) * sc;
  // a new row max more than 2^8 above the stale one moves the stale max; the
  // factor for the O accumulator is left to the next matrix slot
  const bool grow = __any(m > rs.m_used + kRescaleLog2);
  const float mn = grow ? fmaxf(rs.m_used, m) : rs.m_used;
  const float alpha = (rs.m_used == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(rs.m_used - mn);
  rs.l_part *= alpha;
  rs.alpha *= alpha;
  rs.rescale = rs.rescale || grow;
  rs.m_used = mn;
  const float mb = (mn == -INFINITY) ? 0.f : mn;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float sum = rs.l_part;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(S[jb][8 * u + e], sc, -mb));
      P[jb][u] = __builtin_bit_cast(u32x4, v);
      // the row sum adds the same bf16-rounded probabilities the P V product uses
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {v[e], v[e + 1]};
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
      }
    }
  rs.l_part = sum;
}

constexpr int kRing = 2;  // K and V^T ring slots per workgroup

// P V of tile t - 1 (probabilities Pp) and the softmax of tile t (scores S ->
// Pn) in an instruction order fixed by sched_barrier: each of the 16 MFMA
// slots carries a piece of the softmax (row max over slots 0-3, the rescale
// decision in slot 4, then two or four probabilities per slot). V^T operands
// are read in batches of four, one batch ahead. O picks up P V of tile t - 1
// here; a rescale the softmax decides is applied by the caller afterwards,
// before P V of tile t.
__device__ __forceinline__ void pv_softmax(uint32_t slot_off, const u32x4 (&Pp)[2][2],
                                           FragAddr fa, f32x16 (&oacc)[4], const f32x16 (&S)[2],
                                           float sc, RowState& rs, u32x4 (&Pn)[2][2]) {
  asm volatile("" : "+v"(fa.v_sw));
  bf16x8 fr[16];
  auto load = [&](int pi) {  // MFMA slot pi: key half jb, step u, head-dim block db
    const int jb = pi >> 3, u = (pi >> 2) & 1, db = pi & 3;
    fr[pi] = lds_at((((uint32_t)(64 * jb + 32 * u) ^ fa.v_sw) + fa.v_base) + slot_off + db * (32 * 128));
  };
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float m = -INFINITY, mb = 0.f, sum = 0.f;
  // probabilities of score pair q (0..15): S[jb][r], S[jb][r + 1], r = 2 q % 16
  auto prob_pair = [&](int qp) {
    const int idx = 2 * qp, jb = idx >> 4, r = idx & 15, u = r >> 3, w = (r & 7) >> 1;
    const float x0 = __builtin_amdgcn_exp2f(fmaf(S[jb][r], sc, -mb));
    const float x1 = __builtin_amdgcn_exp2f(fmaf(S[jb][r + 1], sc, -mb));
    const bf16x2 pr = {(__bf16)x0, (__bf16)x1};
    Pn[jb][u][w] = __builtin_bit_cast(unsigned int, pr);
    sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);  // row sum of the bf16 P V uses
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) load(i);
  __builtin_amdgcn_sched_barrier(0);
  // While a wave is in this region the SIMD's arbiter prefers it: its MFMAs
  // and softmax slices then interleave tightly, and the other wave of the
  // SIMD (in its QK^T or barrier phase) fills the gaps.
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if ((i & 3) == 0) {  // batch i / 4 has landed; send the next batch
      lds_reads_done();
      if (i + 4 < 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) load(i + 4 + j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      const int jb = i >> 3, u = (i >> 2) & 1, db = i & 3;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], __builtin_bit_cast(bf16x8, Pp[jb][u]),
                                                         oacc[db], 0, 0, 0);
    }
    if (i < 4) {  // row max, 8 scores per slot (a chain of 3-input maxima)
      const int jb = i >> 1, r = (i & 1) * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) m = fmaxf(fmaxf(m, S[jb][r + e]), S[jb][r + e + 1]);
    } else {
      if (i == 4) {  // row max over both lane halves, lazy rescale decision
        m = row_max_halves(m) * sc;
        const bool grow = __any(m > rs.m_used + kRescaleLog2);
        const float mn = grow ? fmaxf(rs.m_used, m) : rs.m_used;
        const float alpha = (rs.m_used == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(rs.m_used - mn);
        rs.l_part *= alpha;
        rs.alpha *= alpha;
        rs.rescale = rs.rescale || grow;
        rs.m_used = mn;
        mb = (mn == -INFINITY) ? 0.f : mn;
        sum = rs.l_part;
      }
      // pairs 0..7 two per slot in slots 4..7, pairs 8..15 one per slot in slots 8..15
      if (i < 8) {
        prob_pair(2 * (i - 4));
        prob_pair(2 * (i - 4) + 1);
      } else {
        prob_pair(i);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  rs.l_part = sum;
}

// One pass (far or local) of a wave over tiles [ktb, kte), software-pipelined:
// iteration t runs P V of tile t - 1 together with the softmax of tile t
// (pv_softmax), then QK^T of tile t + 1. K tiles are staged two tiles ahead of
// their QK^T and V^T tiles one tile ahead of their P V, in two-slot rings
// (slot = (t - ktb) % 2). Tiles from kte_w on hold no causal pair of this
// wave's rows: there it only stages and takes part in the barriers. vt0 + t
// tiles is the sequence's V^T tile t of this KV head (for t >= ktb).
template <bool FAR>
__device__ __forceinline__ void run_pass(const uint16_t* qsrc, const uint16_t* ksrc,
                                         const uint16_t* vt0, const char* kend, const char* vend,
                                         int ktb, int kte,
                                         const WaveRows& wr, float sc, int wave, int lane,
                                         uint4* sK, uint4* sV, RowState& rs,
                                         f32x16 (&oacc)[4]) {
  const int li = lane & 31, hl = lane >> 5;
  // The tile range is wave-uniform but derives from sequence-table entries
  // that the compiler sees as per-lane values; held in scalar registers, the
  // tile addresses and buffer descriptors below are formed by scalar
  // arithmetic instead of a per-load loop over the lanes' values.
  ktb = __builtin_amdgcn_readfirstlane(ktb);
  kte = __builtin_amdgcn_readfirstlane(kte);
  bf16x8 qf[8];
  {
    const int row = wr.r0 + li;
    const bool ok = row < wr.L;
    const int rowc = ok ? row : wr.L - 1;  // in-bounds address, value zeroed below
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint4 v = *(const uint4*)(qsrc + (size_t)rowc * kHeadDim + (2 * t + hl) * 8);
      if (!ok) v = make_uint4(0, 0, 0, 0);
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // tiles with a causal pair of this wave: c0 <= p0 + 31, none if r0 >= L
  const int kte_w = wr.r0 >= wr.L ? ktb : min(kte, (wr.p0 + 31) / kKeyTile + 1);
  const StageOffsets so = stage_offsets(wave, lane);
  const KStage ks = k_stage_offsets(so);
  const FragAddr fa = frag_addr(li, hl, sK, sV);
  constexpr int kTileBytes = kHeadDim * kKeyTile * 2;
  const char* kb0 = scalar_ptr(ksrc);
  const char* vb0 = scalar_ptr(vt0);
  auto stage_k_t = [&](uint4* slot, int t) {
    const char* tile = kb0 + (size_t)t * kTileBytes;
    stage_k(slot, tile_rsrc(tile, kend), ks, wave);
  };
  auto stage_v_t = [&](uint4* slot, int t) {
    const char* tile = vb0 + (size_t)t * kTileBytes;
    stage_v(slot, tile_rsrc(tile, vend), so.v, wave);
  };
  uint4* const sK0 = sK;
  uint4* const sK1 = sK + kSlot;
  uint4* const sV0 = sV;
  uint4* const sV1 = sV + kSlot;

  slot_barrier();  // LDS of a previous pass is no longer read
  stage_k_t(sK0, ktb);
  if (ktb + 1 < kte) stage_k_t(sK1, ktb + 1);
  wait_vmem_all();
  slot_barrier();
  f32x16 S[2];
  constexpr uint32_t kSlotBytes = kSlot * 16;
  if (ktb < kte_w) qk_tile(0, qf, fa, S);

  // iteration t (ring slot parity E = (t - ktb) & 1): S holds the scores of
  // tile t (then receives tile t + 1); Pp the probabilities of tile t - 1, Pn
  // receives those of tile t
  auto step = [&](int t, auto parity, u32x4 (&Pp)[2][2], u32x4 (&Pn)[2][2]) {
    constexpr int E = decltype(parity)::value;
    uint4* const k_this = E ? sK1 : sK0;  // K(t), refilled with K(t + 2)
    uint4* const v_this = E ? sV1 : sV0;  // V(t), staged now
    constexpr uint32_t k_next = E ? 0 : kSlotBytes;  // K(t + 1), ring offset
    constexpr uint32_t v_prev = E ? 0 : kSlotBytes;  // V(t - 1), ring offset
    wait_vmem_all();
    slot_barrier();  // K(t + 1), V(t - 1) landed for every wave; K(t) and V(t - 2) are no longer read
    if (t + 2 < kte) stage_k_t(k_this, t + 2);
    stage_v_t(v_this, t);
    const bool sm = t < kte_w, pv = t > ktb && t - 1 < kte_w, qk = t + 1 < kte_w;
    if (sm) {
      mask_tile<FAR>(S, wr, t * kKeyTile, li, hl);
      if (pv) pv_softmax(v_prev, Pp, fa, oacc, S, sc, rs, Pn);
      else softmax_tile(S, sc, rs, Pn);
    } else if (pv) {
      pv_tile(v_prev, Pp, fa, oacc);
    }
    apply_rescale(rs, oacc);
    if (qk) qk_tile(k_next, qf, fa, S);
  };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  u32x4 Pa[2][2], Pb[2][2];
  for (int t = ktb; t < kte; t += 2) {
    step(t, Even{}, Pa, Pb);
    if (t + 1 < kte) step(t + 1, Odd{}, Pb, Pa);
  }
  // P V of the last tile: P(t) sits in Pb when t - ktb is even
  wait_vmem_all();
  slot_barrier();
  const int tl = kte - 1;
  if (tl < kte_w) {
    if (((tl - ktb) & 1) == 0) pv_tile(0, Pb, fa, oacc);
    else pv_tile(kSlotBytes, Pa, fa, oacc);
  }
}

// One work item of the bf16 kernel (lanes whose query row is past the
// sequence return early from the epilogue only, after the last barrier).
template <bool BIFOCAL, bool BAND>
__device__ __forceinline__ void prefill_bf16_item(const PrefillParams& p, const SeqTable& st, int id,
                                                  uint4* smem) {
  uint4* sK = smem;                  // kRing slots
  uint4* sV = smem + kRing * kSlot;  // kRing slots
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int li = lane & 31, hl = lane >> 5;
  const Item it = make_item<BIFOCAL, BAND>(p, st, wave, kWaveRowsBf16, id);
  const WaveRows wr{it.r0, it.qp + it.r0, it.L, (int)min(it.w0, (long long)(1 << 30))};

  const uint16_t* qg = (const uint16_t*)p.q + ((size_t)it.hq * p.T + it.tok0) * kHeadDim;
  const uint16_t* kg =
      (const uint16_t*)p.k + ((size_t)it.kvh * p.k_hstride + st.kbase[it.b]) * kHeadDim;
  // V^T tile t of the sequence sits at vt0 + t tiles, t >= vt_t0 (the first
  // tile with a copy; the passes never go below it)
  const uint16_t* vt0 = (const uint16_t*)p.vt +
                        ((long long)it.kvh * (p.Tpad / kKeyTile) + st.vt_off[it.b] / kKeyTile -
                         st.vt_t0[it.b]) * (kHeadDim * kKeyTile);

  // ends of the K, K'' and V^T tensors (range limit of the staging loads)
  const char* k_end = (const char*)p.k + (size_t)p.k_rows * kHeadDim * 2;
  const char* k2_end = (const char*)p.k2 + (size_t)p.k2_rows * kHeadDim * 2;
  const char* vt_end = (const char*)p.vt + (size_t)p.vt_rows * kHeadDim * 2;

  RowState rs{-INFINITY, 0.f, 1.f, false};
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};

  // tile ranges of the two passes for the workgroup's query positions
  // R0 .. R0 + P_wg - 1
  const long long R0 = (long long)it.qp + it.R0, Rl = R0 + p.P_wg - 1;
  const long long w0 = it.w0;
  int far_end, loc_b;
  pass_ranges<BIFOCAL, BAND>(R0, Rl, it.nkt, w0, far_end, loc_b);
  // key split: part `split` of the nks takes visits [v0, v1) of the sequence
  // far tiles, then local tiles
  int far_b = 0, far_e = far_end, loc_e = it.nkt;
  if (p.nks > 1) {
    const int nv = far_end + (it.nkt - loc_b);
    const int v0 = (int)((long long)nv * it.split / p.nks);
    const int v1 = (int)((long long)nv * (it.split + 1) / p.nks);
    far_b = min(v0, far_end);
    far_e = min(v1, far_end);
    const int lb = loc_b + max(v0 - far_end, 0);
    loc_e = loc_b + max(v1 - far_end, 0);
    loc_b = lb;
  }
  if (far_b < far_e)
    run_pass<true>((const uint16_t*)p.q2 + ((size_t)it.hq * p.T + it.tok0) * kHeadDim,
                   (const uint16_t*)p.k2 + ((size_t)it.kvh * p.Tk + st.kcu[it.b]) * kHeadDim, vt0,
                   k2_end, vt_end, far_b, far_e, wr, p.scale_log2, wave, lane, sK, sV, rs, oacc);
  if (loc_b < loc_e)
    run_pass<false>(qg, kg, vt0, k_end, vt_end, loc_b, loc_e, wr, p.scale_log2, wave, lane, sK, sV,
                    rs, oacc);

  // epilogue: normalise, store O (bf16) and lse, or a key split's partial
  const int row = it.r0 + li;
  const float l = rs.l_part + __shfl_xor(rs.l_part, 32);
  if (p.nks > 1) {
    if (row >= it.L) return;
    // a split may hold no key of a row: O = 0 and lse = -inf then weigh
    // nothing in the merge
    const size_t prow = ((size_t)it.split * p.Hq + it.hq) * p.T + it.tok0 + row;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* po = p.part_o + prow * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hl;
        *(float4*)(po + d) = make_float4(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv,
                                         oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      }
    if (hl == 0) p.part_lse[prow] = l > 0.f ? rs.m_used + __log2f(l) : -INFINITY;
    return;
  }
  // the wave's 32 rows are one 8 KiB block of O: they go through the K ring
  // (no longer read after the last QK^T) and out as row-contiguous 16-byte
  // stores; in LDS, 16-byte chunk c of row r sits at chunk c ^ (r % 16)
  char* lds = (char*)sK + wave * 8192;
  const float inv = row < it.L ? 1.f / l : 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16(oacc[db][4 * g + 0] * inv) |
            ((uint32_t)f32_to_bf16(oacc[db][4 * g + 1] * inv) << 16);
      w.y = (uint32_t)f32_to_bf16(oacc[db][4 * g + 2] * inv) |
            ((uint32_t)f32_to_bf16(oacc[db][4 * g + 3] * inv) << 16);
      *(uint2*)(lds + li * 256 + (((4 * db + g) ^ (li & 15)) << 4) + (hl << 3)) = w;
    }
  uint16_t* og = (uint16_t*)p.o + ((size_t)it.hq * p.T + it.tok0 + it.r0) * kHeadDim;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = 4 * i + (lane >> 4), cc = lane & 15;
    const uint4 v = *(const uint4*)(lds + rr * 256 + ((cc ^ (rr & 15)) << 4));
    if (it.r0 + rr < it.L) *(uint4*)(og + (size_t)rr * kHeadDim + cc * 8) = v;
  }
  if (p.lse && hl == 0 && row < it.L)
    p.lse[(size_t)it.hq * p.T + it.tok0 + row] = (rs.m_used + __log2f(l)) * 0.69314718055994530942f;
}

// Workgroup w runs work item w, or, with claim counters, workgroups loop
// over the items they claim until every queue is empty (see claim_item).
template <bool BIFOCAL, bool BAND>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillParams p, SeqTable st) {
  extern __shared__ uint4 smem[];
  __shared__ int s_item;
  int id = blockIdx.x;
  for (;;) {
    if (p.item_ctr) {
      __syncthreads();  // every wave has read the previous item's id
      if (threadIdx.x == 0) s_item = claim_item(p.item_ctr, p.n_items);
      __syncthreads();
      id = __builtin_amdgcn_readfirstlane(s_item);
      if (id < 0) return;
    }
    prefill_bf16_item<BIFOCAL, BAND>(p, st, id, smem);
    if (!p.item_ctr) return;
  }
}

// --------------------------------------------------------------- fp32
// Same loop with fp32 operands on MFMA 32x32x2 f32: one 32-row query block per
// wave; k-step t contracts head dims t (lanes 0-31) and 64 + t (lanes 32-63).
__device__ __forceinline__ void qk_f32(const uint4* __restrict__ sk, const float (&q)[64], int li,
                                       int hl, f32x16 (&S)[2]) {
  S[0] = f32x16{};
  S[1] = f32x16{};
  const int row0 = key_of_mfma_row(li), row1 = 32 + row0;
#pragma unroll
  for (int tc = 0; tc < 16; ++tc) {
    const int ch = 16 * hl + tc;
    const float4 a0 = __builtin_bit_cast(float4, sk[row0 * 32 + (ch ^ (row0 & 31))]);
    const float4 a1 = __builtin_bit_cast(float4, sk[row1 * 32 + (ch ^ (row1 & 31))]);
    S[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.x, q[4 * tc + 0], S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.x, q[4 * tc + 0], S[1], 0, 0, 0);
    S[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.y, q[4 * tc + 1], S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.y, q[4 * tc + 1], S[1], 0, 0, 0);
    S[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.z, q[4 * tc + 2], S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.z, q[4 * tc + 2], S[1], 0, 0, 0);
    S[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.w, q[4 * tc + 3], S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.w, q[4 * tc + 3], S[1], 0, 0, 0);
  }
}

template <bool BIFOCAL, bool BAND>
__global__ __launch_bounds__(256, 1) void prefill_f32_kernel(PrefillParams p, SeqTable st) {
  extern __shared__ uint4 smem[];
  uint4* sK = smem;                            // [64][32 x 16 B]
  uint4* sK2 = smem + 2048;
  uint4* sV = smem + (BIFOCAL && !BAND ? 4096 : 2048);  // [128][16 x 16 B] (no K'' slot without a far branch)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hl = lane >> 5;
  const Item it = make_item<BIFOCAL, BAND>(p, st, wave, kWaveRowsF32, blockIdx.x);
  const long long w0 = it.w0;

  const float* qg = (const float*)p.q + ((size_t)it.hq * p.T + it.tok0) * kHeadDim;
  const float* kg = (const float*)p.k + ((size_t)it.kvh * p.k_hstride + st.kbase[it.b]) * kHeadDim;
  const float* q2g = BIFOCAL ? (const float*)p.q2 + ((size_t)it.hq * p.T + it.tok0) * kHeadDim : nullptr;
  const float* k2g =
      BIFOCAL ? (const float*)p.k2 + ((size_t)it.kvh * p.Tk + st.kcu[it.b]) * kHeadDim : nullptr;
  const int nk = it.qp + it.L;   // keys of the sequence
  const int p0 = it.qp + it.r0;  // position of the wave's first row
  const float* vt0 = (const float*)p.vt +
                     ((long long)it.kvh * (p.Tpad / kKeyTile) + st.vt_off[it.b] / kKeyTile -
                      st.vt_t0[it.b]) * (kHeadDim * kKeyTile);

  float qf[64], qf2[64];
  {
    const int row = it.r0 + li;
    const bool ok = row < it.L;
    const bool ok2 = ok && w0 < nk && !BAND;  // corrected queries exist only with far pairs
    const int rowc = ok ? row : it.L - 1;
#pragma unroll
    for (int tc = 0; tc < 16; ++tc) {
      const size_t off = (size_t)rowc * kHeadDim + 64 * hl + 4 * tc;
      float4 a = *(const float4*)(qg + off);
      if (!ok) a = make_float4(0, 0, 0, 0);
      qf[4 * tc] = a.x; qf[4 * tc + 1] = a.y; qf[4 * tc + 2] = a.z; qf[4 * tc + 3] = a.w;
      if constexpr (BIFOCAL) {
        float4 c = make_float4(0, 0, 0, 0);
        if (ok2) c = *(const float4*)(q2g + off);
        qf2[4 * tc] = c.x; qf2[4 * tc + 1] = c.y; qf2[4 * tc + 2] = c.z; qf2[4 * tc + 3] = c.w;
      }
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  const uint4 zero4 = make_uint4(0, 0, 0, 0);

  for (int kt = st.vt_t0[it.b]; kt < it.nkt; ++kt) {  // tiles below vt_t0 hold no pair of these rows
    const int c0 = kt * kKeyTile;
    bool cf, cl;
    tile_needs<BIFOCAL>((long long)it.qp + it.R0, p.P_wg, c0, w0, cf, cl);
    if (BAND) cf = false;  // far pairs are dropped, never scored
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 5, col = c & 31;
      const bool ok = c0 + row < nk;
      const size_t off = (size_t)min(c0 + row, nk - 1) * kHeadDim + col * 4;
      if (cl) {
        uint4 kv = *(const uint4*)(kg + off);
        if (!ok) kv = zero4;
        sK[row * 32 + (col ^ (row & 31))] = kv;
      }
      if constexpr (BIFOCAL)
        if (cf) {
          uint4 kv = *(const uint4*)(k2g + off);
          if (!ok) kv = zero4;
          sK2[row * 32 + (col ^ (row & 31))] = kv;
        }
      const int d = c >> 4, vc = c & 15;
      sV[d * 16 + (vc ^ (d & 15))] =
          *(const uint4*)(vt0 + (size_t)kt * (kHeadDim * kKeyTile) + d * kKeyTile + vc * 4);
    }
    __syncthreads();

    const bool wave_skip = (it.r0 >= it.L) || (c0 > p0 + kWaveRowsF32 - 1);
    if (wave_skip) continue;
    const long long dmax = (long long)p0 + kWaveRowsF32 - 1 - c0;
    const long long dmin = (long long)p0 - (c0 + kKeyTile - 1);
    const bool has_far = BIFOCAL && dmax >= w0;
    const bool has_loc = !BIFOCAL || (w0 > 0 && dmin < w0);
    constexpr bool band_only = BIFOCAL && BAND;
    if (band_only && !has_loc) continue;  // every pair of the tile is dropped

    f32x16 S[2];
    if (BIFOCAL && has_far && !band_only) qk_f32(sK2, qf2, li, hl, S);
    else qk_f32(sK, qf, li, hl, S);
    const long long i = p0 + li;
    if (band_only && has_far) {  // drop the far pairs of a mixed tile
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const long long j = c0 + 32 * jb + key_of_acc(r, hl);
          if (!pair_is_local(i, j, w0)) S[jb][r] = -INFINITY;
        }
    } else if (BIFOCAL && has_far && has_loc) {
      f32x16 Sl[2];
      qk_f32(sK, qf, li, hl, Sl);
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const long long j = c0 + 32 * jb + key_of_acc(r, hl);
          if (pair_is_local(i, j, w0)) S[jb][r] = Sl[jb][r];
        }
    }
    if (dmin < 0) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const long long j = c0 + 32 * jb + key_of_acc(r, hl);
          if (j > i) S[jb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[jb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float mbase, alpha;
    online_softmax_rescale(m_run, l_run, mx, p.scale_log2, mbase, alpha);
    float rs = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(S[jb][r], p.scale_log2, -mbase));
        S[jb][r] = e;
        rs += e;
      }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
    // O^T += V^T P^T; register r of lane half hl is key 32 jb + key_of_acc(r, hl)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + li;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {  // registers 4g .. 4g+3
          const int key = 32 * jb + key_of_acc(4 * g, hl);
          const int ch = key >> 2;
          const float4 a = __builtin_bit_cast(float4, sV[d * 16 + (ch ^ (d & 15))]);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, S[jb][4 * g + 0], oacc[db], 0, 0, 0);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, S[jb][4 * g + 1], oacc[db], 0, 0, 0);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, S[jb][4 * g + 2], oacc[db], 0, 0, 0);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, S[jb][4 * g + 3], oacc[db], 0, 0, 0);
        }
    }
  }

  const int row = it.r0 + li;
  if (row >= it.L) return;
  float* og = (float*)p.o + ((size_t)it.hq * p.T + it.tok0) * kHeadDim;
  const float inv = 1.f / l_run;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * hl;
      *(float4*)(og + (size_t)row * kHeadDim + d) =
          make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                      oacc[db][4 * g + 3] * inv);
    }
  if (p.lse && hl == 0)
    p.lse[(size_t)it.hq * p.T + it.tok0 + row] = (m_run + __log2f(l_run)) * 0.69314718055994530942f;
}

// --------------------------------------------------------------- test hooks
// The bf16 tile kernel's own classification for one sequence of length L
// (query positions 0 .. L - 1, GQA groups of 4 heads: 32-row work items):
// wave (row block rb, key tile kt) takes the pass tile ranges of its item
// (pass_ranges) and runs mask_tile of both passes on a zero tile, exactly as
// the tile loop does, and writes for every causal pair it covers
//   1: scored by the local pass, 2: scored by the far pass,
//   3: scored by both (an error), 0: scored by neither.
// Pairs the kernel never visits keep what the caller put there.
template <bool BAND>
__global__ __launch_bounds__(64) void pair_map_kernel(long long L, long long w0_eff, int8_t* br) {
  const int rb = blockIdx.x, kt = blockIdx.y, lane = threadIdx.x;
  const int li = lane & 31, hl = lane >> 5;
  const long long R0 = 32LL * rb, Rl = min(R0 + 31, L - 1);
  const int nkt = (int)((Rl + 1 + kKeyTile - 1) / kKeyTile);
  if (kt >= nkt) return;
  int far_end, loc_b;
  pass_ranges<true, BAND>(R0, R0 + 31, nkt, w0_eff, far_end, loc_b);
  const WaveRows wr{(int)R0, (int)R0, (int)L, (int)min(w0_eff, (long long)(1 << 30))};
  f32x16 Sf[2], Sl[2];
  Sf[0] = Sf[1] = Sl[0] = Sl[1] = f32x16{};
  mask_tile<true>(Sf, wr, kt * kKeyTile, li, hl);
  mask_tile<false>(Sl, wr, kt * kKeyTile, li, hl);
  const long long i = R0 + li;
  if (i >= L) return;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const long long j = (long long)kt * kKeyTile + 32 * jb + key_of_acc(r, hl);
      if (j >= L) continue;
      const bool far = kt < far_end && Sf[jb][r] != -INFINITY;
      const bool loc = kt >= loc_b && kt < nkt && Sl[jb][r] != -INFINITY;
      br[i * L + j] = (int8_t)((far ? 2 : 0) + (loc ? 1 : 0));
    }
}

// The prep pass's (phi(p) - p) * s numerators for p < L.
__global__ void phi_num_kernel(long long L, long long s, int mode, long long* dphi_num) {
  for (long long pidx = blockIdx.x * (long long)blockDim.x + threadIdx.x; pidx < L;
       pidx += (long long)gridDim.x * blockDim.x)
    dphi_num[pidx] = prep_num(pidx, s, mode, false, 0, 0);
}

// The prep pass's fp32 cos / sin of the correction angle for given positions:
// block = position, thread = rotary pair; cs [n][64][2].
__global__ __launch_bounds__(64) void prep_angle_kernel(AngleProbe a, ThetaTable tt, float* cs) {
  const int n = blockIdx.x, m = threadIdx.x;
  const long long num = prep_num(a.pos[n], a.s[n], a.mode, a.query != 0, a.shift, a.w0);
  float c, sn;
  prep_cos_sin(tt.th[m], (double)num / (double)a.s[n], c, sn);
  cs[((size_t)n * kPairs + m) * 2] = c;
  cs[((size_t)n * kPairs + m) * 2 + 1] = sn;
}

// --------------------------------------------------------------- launchers
hipError_t launch_correction_prep(int dtype, const PrepParams& pp, const SeqTable& st,
                                  const ThetaTable& tt, hipStream_t stream) {
  const int tq = st.cu[st.n] - st.cu[0], tk = st.kcu[st.n] - st.kcu[0];
  const int tok_per_wg = 256 / (kPairs / (dtype == 0 ? 8 : 4));
  const dim3 grid((max(tq, tk) + tok_per_wg - 1) / tok_per_wg, 2);
  if (dtype == 0)
    hipLaunchKernelGGL(correction_prep_kernel<uint16_t>, grid, dim3(256), 0, stream, pp, st, tt);
  else
    hipLaunchKernelGGL(correction_prep_kernel<float>, grid, dim3(256), 0, stream, pp, st, tt);
  return hipGetLastError();
}

hipError_t launch_vt_transpose(int dtype, const VtParams& vp, const SeqTable& st,
                               hipStream_t stream) {
  dim3 grid((st.vt_off[st.n] - st.vt_off[0]) / kKeyTile, vp.Hkv);
  if (dtype == 0)
    hipLaunchKernelGGL(vt_transpose_bf16_kernel, grid, dim3(128), 0, stream, vp, st);
  else
    hipLaunchKernelGGL(vt_transpose_f32_kernel, grid, dim3(256), 0, stream, vp, st);
  return hipGetLastError();
}

// Merge of the key splits of a chunk launch: one thread per (query head,
// row, 8 head dims) weighs the parts' normalised O by 2^(lse_s - max lse) and
// writes bf16 O (and lse, natural log) like the unsplit kernel.
__global__ __launch_bounds__(256) void chunk_combine_kernel(PrefillParams p, int tok_begin,
                                                            int n_tok) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int g = (int)(gid & 15);  // head dims 8 g .. 8 g + 7
  const long long hr = gid >> 4;
  if (hr >= (long long)p.Hq * n_tok) return;
  const int h = (int)(hr / n_tok);
  const int tok = tok_begin + (int)(hr - (long long)h * n_tok);
  const size_t plane = (size_t)p.Hq * p.T;  // rows per split
  const size_t r = (size_t)h * p.T + tok;
  float lse[kMaxKeySplits];
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxKeySplits; ++s) {
    lse[s] = s < p.nks ? p.part_lse[s * plane + r] : -INFINITY;
    mx = fmaxf(mx, lse[s]);
  }
  const float mb = mx == -INFINITY ? 0.f : mx;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxKeySplits; ++s) {
    if (s < p.nks) {
      const float w = __builtin_amdgcn_exp2f(lse[s] - mb);  // 0 for a split without keys
      const float* po = p.part_o + (s * plane + r) * kHeadDim + 8 * g;
      const float4 a = *(const float4*)po, b = *(const float4*)(po + 4);
      acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
      acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
      wsum += w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint32_t wd[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    wd[e] = (uint32_t)f32_to_bf16(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[2 * e + 1] * inv) << 16);
  *(uint4*)((uint16_t*)p.o + r * kHeadDim + 8 * g) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  if (p.lse && g == 0) p.lse[r] = (mb + __log2f(wsum)) * 0.69314718055994530942f;
}

hipError_t launch_chunk_combine(const PrefillParams& pp, int tok_begin, int n_tok,
                                hipStream_t stream) {
  const long long threads = (long long)pp.Hq * n_tok * 16;
  const int grid = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(chunk_combine_kernel, dim3(grid), dim3(256), 0, stream, pp, tok_begin, n_tok);
  return hipGetLastError();
}

template <typename K>
static hipError_t launch_with_lds(K kernel, int grid, int threads, size_t lds, hipStream_t stream,
                                  const PrefillParams& pp, const SeqTable& st) {
  hipError_t e = hipFuncSetAttribute((const void*)kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, stream, pp, st);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void zero_item_ctr_kernel(int* ctr) {
  if (threadIdx.x < 8) ctr[threadIdx.x] = 0;
}

hipError_t launch_prefill_main(int dtype, bool bifocal, bool band, const PrefillParams& pp,
                               const SeqTable& st, int grid, hipStream_t stream) {
  if (pp.item_ctr) {  // the claim counters start at zero (a fill kernel, not a memset)
    hipLaunchKernelGGL(zero_item_ctr_kernel, dim3(1), dim3(64), 0, stream, pp.item_ctr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dtype == 0) {
    const int th = 64 * kBf16Waves;
    const size_t lds = 2 * kRing * kSlot * sizeof(uint4);
    if (band) return launch_with_lds(prefill_bf16_kernel<true, true>, grid, th, lds, stream, pp, st);
    if (bifocal) return launch_with_lds(prefill_bf16_kernel<true, false>, grid, th, lds, stream, pp, st);
    return launch_with_lds(prefill_bf16_kernel<false, false>, grid, th, lds, stream, pp, st);
  }
  if (band) return launch_with_lds(prefill_f32_kernel<true, true>, grid, 256, 2 * 32768, stream, pp, st);
  if (bifocal) return launch_with_lds(prefill_f32_kernel<true, false>, grid, 256, 3 * 32768, stream, pp, st);
  return launch_with_lds(prefill_f32_kernel<false, false>, grid, 256, 2 * 32768, stream, pp, st);
}

hipError_t launch_pair_map(long long L, long long w0, long long s, int mode, int8_t* br,
                           long long* dphi_num, hipStream_t stream) {
  // the tile kernel treats every pair as local when s = 1 (both branches coincide)
  const bool band = mode == 2;
  const long long w0_eff = (band || s > 1) ? w0 : (1LL << 62);
  const dim3 grid((unsigned)((L + 31) / 32), (unsigned)((L + kKeyTile - 1) / kKeyTile));
  if (band) hipLaunchKernelGGL(pair_map_kernel<true>, grid, dim3(64), 0, stream, L, w0_eff, br);
  else hipLaunchKernelGGL(pair_map_kernel<false>, grid, dim3(64), 0, stream, L, w0_eff, br);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || band) return e;
  hipLaunchKernelGGL(phi_num_kernel, dim3(16), dim3(256), 0, stream, L, s, mode, dphi_num);
  return hipGetLastError();
}

hipError_t launch_prep_angles(const AngleProbe& a, const ThetaTable& tt, float* cs,
                              hipStream_t stream) {
  hipLaunchKernelGGL(prep_angle_kernel, dim3(a.n), dim3(64), 0, stream, a, tt, cs);
  return hipGetLastError();
}

}  // namespace bf
