// Bifocal RoPE attention, single-token decode over a KV cache on gfx950.
//
// decode_split_kernel: workgroup = (batch b, KV head, split of C keys). The
//   split's keys and values are streamed from HBM once. Keys farther than w0
//   from the query (position N - 1) get the correction rotation
//   R(theta_m * (phi(j) - j)) in registers right after they are loaded, keys
//   inside the window are used as cached [ai-feeds.com summary, "关键模块"
//   item 3: rotation of cached keys; item 1: the w0 window keeps original
//   RoPE]. The query gets the same correction at its own position. Scores use
//   MFMA 16x16x32 (queries as columns), P V uses MFMA 16x16x16, with one
//   online softmax state per query and wave; at the end the waves are merged
//   and the split writes its (m, l, acc) partial. Instantiated for a
//   contiguous or a paged cache, and with non-temporal K / V loads for
//   launches that stream more than the MALL could keep.
// decode_combine_kernel: log-sum-exp merge of the splits of each query head.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <type_traits>

#include "bifocal.h"
#include "bf_common.h"

namespace bf {

typedef __attribute__((ext_vector_type(8))) __bf16 dbf16x8;
typedef __attribute__((ext_vector_type(4))) short ds16x4;
typedef __attribute__((ext_vector_type(4))) float df32x4;
typedef __attribute__((ext_vector_type(2))) float df32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 dbf16x2;

constexpr int kDecBlock = 64;    // keys per streamed block
constexpr int kDecMaxG = 16;     // query heads per KV head the kernel supports

struct DecodeParams {
  const uint16_t* q;    // [B][Hq][D]
  const uint16_t* kc;   // [B][Hkv][cap][D], or pages [num_pages][Hkv][page][D]
  const uint16_t* vc;   // same layout as kc
  uint16_t* k2;         // far-key store (contiguous cache only): k'' of each far key, layout of kc
  const int* block_table;  // paged cache: [B][max_pages] page of each page-sized key block
  float* part_m;        // [B][Hq][S]  running max (log2 domain, scaled)
  float* part_l;        // [B][Hq][S]
  float* part_acc;      // [B][Hq][S][D]
  uint16_t* o;          // [B][Hq][D]
  float* lse;           // [B][Hq] or null
  long long cap;
  long long w0;
  float scale_log2;
  int Hq, Hkv, G, S;
  int mode;   // 0 = FI, 1 = PA
  int shift;  // 1: the query gets the band-edge continuity shift w0 - phi(w0)
  int max_pages;  // paged cache: row length of block_table
  int num_pages;  // paged cache: pages in the pool (page numbers are clamped below it)
  int page_log2;  // paged cache: log2 of the page size (keys per page, >= 16)
};

struct DecodeSeqs {
  int n;
  int N[kMaxSeqPerLaunch];       // valid keys (query at N - 1)
  int s[kMaxSeqPerLaunch];       // s(N)
  int nsplit[kMaxSeqPerLaunch];
  int chunk[kMaxSeqPerLaunch];   // keys per split (multiple of 64)
  int kstart[kMaxSeqPerLaunch];  // first key read, a multiple of 16 (steps never cross a page)
  int kmin[kMaxSeqPerLaunch];    // first key that counts: 0, or N - w0 for band-only attention
  int stored[kMaxSeqPerLaunch];  // far-key store: keys 0 .. stored - 1 hold k'' (a multiple of 16)
};

__device__ __forceinline__ float dbf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t df2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ long long dcorr_num(long long p, long long s, int mode) {
  return mode == 1 ? (p / s - p) * s : -p * (s - 1);
}

constexpr double kInv2Pi = 0.15915494309189533577;

// cos / sin of an angle given in turns (fp64): the reduction to one turn is
// done in fp64 (angles reach ~1e5 rad at 128K keys), the reduced fraction goes
// through the hardware sin / cos, which take their input in turns.
__device__ __forceinline__ void turn_cos_sin(double turns, float& c, float& sn) {
  const float fr = (float)(turns - rint(turns));
  sn = __builtin_amdgcn_sinf(fr);
  c = __builtin_amdgcn_cosf(fr);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((df32x2){lo, hi}, dbf16x2));
}

// a wave-uniform pointer forced into scalar registers, so that loads use the
// scalar-base + 32-bit vector-offset addressing form
__device__ __forceinline__ const char* dscalar_ptr(const void* ptr) {
  const uint64_t v = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// 16-byte global load at a base plus a 32-bit offset (loaded as a native
// vector: copying the uint4 struct through a reference would go back to a
// generic pointer and a flat load)
typedef __attribute__((ext_vector_type(4))) unsigned int du32x4;
__device__ __forceinline__ uint4 gload16(const char* base, uint32_t off) {
  const du32x4 v = *(const __attribute__((address_space(1))) du32x4*)(base + off);
  return __builtin_bit_cast(uint4, v);
}

// The same load marked non-temporal: the line is streamed through the caches
// instead of being kept. Every K / V byte of a call is read once, so keeping
// the lines only evicts others; when the cache is larger than the MALL that
// costs bandwidth (the lines could not have stayed resident anyway).
template <bool NT>
__device__ __forceinline__ uint4 kvload16(const char* base, uint32_t off) {
  const auto* ptr = (const __attribute__((address_space(1))) du32x4*)(base + off);
  if constexpr (NT) return __builtin_bit_cast(uint4, __builtin_nontemporal_load(ptr));
  else return __builtin_bit_cast(uint4, *ptr);
}

// x holds elements (m, m + 1), y holds (m + 64, m + 65): rotate both pairs,
// returning the new x and writing the new y.
__device__ __forceinline__ uint32_t rot_word(uint32_t x, uint32_t y, float c0, float s0, float c1,
                                             float s1, uint32_t& y_out) {
  const float a0 = __uint_as_float(x << 16), a1 = __uint_as_float(x & 0xffff0000u);
  const float b0 = __uint_as_float(y << 16), b1 = __uint_as_float(y & 0xffff0000u);
  y_out = pack_bf16x2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
  return pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
}

// Pieces of the far-key correction angle, shared by the split kernel and the
// angle test kernel (reading: angle addition over a 16-key step, see below).
// Base angle of a step starting at key jb, in turns per unit theta_m
// (multiplied by theta_m / 2pi by the caller): phi(jb) - jb, where
// q_pa = floor(jb / s) for position aliasing.
__device__ __forceinline__ double dec_step_base(int mode, long long q_pa, long long jb, long long s,
                                                double inv_s) {
  return mode == 1 ? (double)(q_pa - jb) : (double)(-jb * (s - 1)) * inv_s;
}
// Offset-table row of key jb + n16 (r_pa = jb mod s): n16 for FI,
// n16 - floor((r_pa + n16) / s) for PA (a float divide corrected by one either way).
__device__ __forceinline__ int dec_offset_row(int mode, int r_pa, int n16, int s_i, float inv_s_f) {
  if (mode != 1) return n16;
  const int x = r_pa + n16;
  int qd = (int)((float)x * inv_s_f);
  if ((qd + 1) * s_i <= x) ++qd;
  if (qd * s_i > x) --qd;
  return n16 - qd;
}
// Offset-table entry of row idx for pair m: rotation by -theta_m idx kappa,
// kappa = (s - 1) / s (FI) or 1 (PA).
__device__ __forceinline__ void dec_offset_cos_sin(double th_m, int idx, double kappa, float& c,
                                                   float& sn) {
  turn_cos_sin(-th_m * kInv2Pi * (double)idx * kappa, c, sn);
}
// Rotation of a key: the step's base rotation (bc, bs) times the offset (tc, ts).
__device__ __forceinline__ void dec_compose(float bc, float bs, float tc, float ts, float& c,
                                            float& sn) {
  c = bc * tc - bs * ts;
  sn = bs * tc + bc * ts;
}
// (q_pa, r_pa) = divmod(step start, s), advanced by add_q s + add_r keys
// (0 <= add_r < s).
__device__ __forceinline__ void dec_advance(long long& q_pa, int& r_pa, int add_q, int add_r,
                                            int s_i) {
  q_pa += add_q;
  r_pa += add_r;
  if (r_pa >= s_i) {
    r_pa -= s_i;
    ++q_pa;
  }
}
// Query angle numerator in turns per unit theta_m: (phi(N - 1) - (N - 1)),
// plus w0 - phi(w0) with the band-edge continuity shift.
__device__ __forceinline__ double dec_query_base(int mode, int shift, long long N, long long s,
                                                 long long w0) {
  const long long qsh = !shift ? 0 : mode == 1 ? (w0 - w0 / s) * s : w0 * (s - 1);
  return (double)(dcorr_num(N - 1, s, mode) + qsh) / (double)s;
}

// ------------------------------------------------------------------ kernels
// Split kernel: workgroup = (batch b, KV head, split of `chunk` keys). The 4
// waves take the split's 16-key steps in turn (step st of wave w is the
// split's step 4 st + w), each with its own softmax state, so the workgroup
// reads one contiguous stream of K and one of V; otherwise the waves run
// independently. (Each wave streaming its own quarter of the split made four
// times as many streams and read about 3 % slower.) Both K and V go straight
// from HBM into registers, already in the MFMA operand layouts (no LDS
// staging):
//   - K: lane (key n16, group g4) holds head-dim chunks 4 t + g4 (t = 0..3) of
//     its key, the A operand of MFMA 16x16x32 for S^T = K Q^T. Both halves
//     (m, m + 64) of every rotary pair sit in the same lane, so the correction
//     rotation of far keys is done in place;
//   - V: lane (n16, g4) holds chunk n16 (head dims 8 n16 .. 8 n16 + 7) of keys
//     4 g4 + q (q = 0..3); each quarter-wave reads whole 256-byte rows. P V
//     uses the head-dim order d = 8 row + block, so these four registers feed
//     the 8 MFMA 16x16x16 of the step after byte permutes only;
//   - three register slots: a step's K is reloaded with the step three
//     ahead as soon as QK^T has read it, its V after P V, so two to three
//     steps are in flight.
// The G query heads of the KV group are the MFMA columns (columns >= G are
// zero queries whose results are dropped).
//
// Correction angles of far keys by angle addition. For a step starting at key
// jb, key jb + n has phi(jb + n) - (jb + n) = [phi(jb) - jb] + e, where
//   FI: e = -n (s - 1) / s                         (idx = n)
//   PA: e = floor((r + n) / s) - n, r = jb mod s   (idx = n - floor((r + n) / s))
// so e = -idx * kappa with idx in [0, 16) and kappa = (s - 1) / s (FI) or 1 (PA).
// Per step each lane m computes the base rotation of theta_m [phi(jb) - jb]
// (one fp64 reduction per pair for the whole wave), the 16 x 64 rotations by
// theta_m e are a per-workgroup table, and a key's rotation is the product of
// the two (cos / sin addition formulas).
constexpr int kDecWaves = 4;
constexpr int kDecStep = 16;  // keys per wave step
constexpr int kDecRing = 3;   // register slots per wave
constexpr int kDecTRow = 66;  // padded float2 row of the offset table (conflict-free reads)
constexpr float kDecRescaleLog2 = 8.f;
constexpr int kDecPageRegs = 4;  // page-number registers per lane: 256 pages per split

// LDS layout (bytes). Prologue / loop: Q' and Q'' [2][16][128] bf16, offset
// table [16][66] float2, per-wave base rows [4][64] float2. After the loop the
// same memory holds the 4-wave merge: m [4][16], l [4][16], acc [4][16][128].
constexpr int kDecLdsQ = 0;
constexpr int kDecLdsT = kDecLdsQ + 2 * kDecMaxG * kHeadDim * 2;
constexpr int kDecLdsB = kDecLdsT + kDecStep * kDecTRow * 8;
constexpr int kDecLdsLoop = kDecLdsB + kDecWaves * kPairs * 8;
constexpr int kDecLdsMerge = (2 * kDecWaves * kDecMaxG + kDecWaves * kDecMaxG * kHeadDim) * 4;
constexpr int kDecLds = kDecLdsLoop > kDecLdsMerge ? kDecLdsLoop : kDecLdsMerge;

// Workgroup barrier after ds_write-only LDS traffic, with a compiler memory
// barrier; unlike __syncthreads it does not wait for the K / V prefetches
// already in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// STORE (bifocal): the far keys below ds.stored[b] are read as k'' from p.k2
// (the layout of p.kc: a contiguous cache, or a page pool under the same
// block table) and used as loaded; every other far key is rotated as usual
// and its k'' written to p.k2, so after the call p.k2 holds k'' of all far
// keys (a later call with the same s reads them back).
template <bool BIFOCAL, bool PAGED, bool NT, bool STORE = false>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeParams p, DecodeSeqs ds,
                                                              ThetaTable tt) {
  static_assert(!STORE || BIFOCAL, "the far-key store serves the bifocal decode");
  __shared__ uint4 smem[kDecLds / 16];
  uint4* sQ = smem + kDecLdsQ / 16;

  const int b = blockIdx.z, kvh = blockIdx.y, sp = blockIdx.x;
  if (sp >= ds.nsplit[b]) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const long long N = ds.N[b];
  const int s_i = ds.s[b];
  const long long s = s_i;
  const long long w0 = (BIFOCAL && s > 1) ? p.w0 : (1LL << 62);
  const long long far_lim = N - w0;  // keys j < far_lim are far
  const int chunk = ds.chunk[b];
  const long long k_begin = ds.kstart[b] + (long long)sp * chunk;
  const long long k_end = min(N, k_begin + chunk);
  const long long kw0 = k_begin, kw1 = k_end;
  const int tsteps = kw1 > kw0 ? (int)((kw1 - kw0 + kDecStep - 1) / kDecStep) : 0;
  const int ns = tsteps > wave ? (tsteps - wave + kDecWaves - 1) / kDecWaves : 0;  // this wave's steps
  const bool split_far = BIFOCAL && k_begin < far_lim;

  // split-local key indexing: key kw0 + jl, jl in [0, nl); step st of this
  // wave starts at jl = 16 (4 st + wave); byte offsets fit 32 bits
  const int nl = ns > 0 ? (int)(kw1 - kw0) : 0;
  auto jl_of = [&](int st) { return (st * kDecWaves + wave) * kDecStep; };
  const int far_l = (int)max(-1LL, min(far_lim - kw0, (long long)(chunk + kDecStep)));
  // keys below kmin (the band-only window start, rounded down to kstart) are masked
  const int lo_l = (int)max(0LL, min((long long)ds.kmin[b] - kw0, (long long)(chunk + kDecStep)));
  const char* kwb;
  const char* vwb;
  char* k2wb = nullptr;  // far-key store at the split's first key (STORE)
  // steps with jl + 16 <= st_l read k'' from the store (STORE)
  const int st_l = STORE ? (int)max(0LL, min((long long)ds.stored[b] - kw0, (long long)(chunk + kDecStep))) : 0;
  int first_page = 0, pg[kDecPageRegs] = {};
  if constexpr (!PAGED) {
    const size_t hoff = ((size_t)b * p.Hkv + kvh) * (size_t)p.cap * kHeadDim;
    const size_t koff = (size_t)(ns > 0 ? kw0 : 0) * kHeadDim;
    kwb = dscalar_ptr(p.kc + hoff + koff);
    vwb = dscalar_ptr(p.vc + hoff + koff);
    if constexpr (STORE) k2wb = (char*)dscalar_ptr(p.k2 + hoff + koff);
  } else {
    // the pages the split's keys live in, page i of the split in lane i % 64
    // of register i / 64 (a split spans at most 4032 / 16 + 1 = 253 pages),
    // read once; each step picks its page by register and lane
    kwb = dscalar_ptr(p.kc);
    vwb = dscalar_ptr(p.vc);
    if constexpr (STORE) k2wb = (char*)dscalar_ptr(p.k2);
    if (ns > 0) {
      first_page = (int)(kw0 >> p.page_log2);
      const int last_page = (int)((kw1 - 1) >> p.page_log2);
#pragma unroll
      for (int g = 0; g < kDecPageRegs; ++g)
        if (first_page + 64 * g + lane <= last_page)
          pg[g] = min(max(p.block_table[(size_t)b * p.max_pages + first_page + 64 * g + lane], 0),
                      p.num_pages - 1);
    }
  }
  uint4 kreg[kDecRing][4], vreg[kDecRing][4];
  // issue the loads of step st into register slot r, K first (needed first);
  // rows past the wave's last key re-read that key (their scores are masked).
  // Keys are addressed from kb / vb: the wave's first key (contiguous cache)
  // or the first key of the step's page block (paged cache, rel0 = 0).
  // (KV = 0: K, 1: V)
  // paged cache: the pool row of the first key of the step at split-local key j0
  // (a step never crosses a page: 16 | page size)
  auto page_row = [&](int j0) -> size_t {
    const long long key = kw0 + j0;
    const int pi = (int)(key >> p.page_log2) - first_page;  // wave-uniform, < 64 kDecPageRegs
    int page = __builtin_amdgcn_readlane(pg[0], pi & 63);
#pragma unroll
    for (int g = 1; g < kDecPageRegs; ++g) {
      const int pgg = __builtin_amdgcn_readlane(pg[g], pi & 63);
      page = (pi >> 6) == g ? pgg : page;
    }
    return (((size_t)page * p.Hkv + kvh) << p.page_log2) + (size_t)(key & ((1LL << p.page_log2) - 1));
  };
  auto issue_half = [&](int st, int r, auto kv) {
    constexpr int KV = decltype(kv)::value;
    const int j0 = jl_of(st);
    const char* kb = (STORE && j0 + kDecStep <= st_l) ? (const char*)k2wb : kwb;
    const char* vb = vwb;
    int rel0 = j0;
    if constexpr (PAGED) {
      const size_t row = page_row(j0);
      kb = dscalar_ptr(kb + row * (kHeadDim * 2));
      vb = dscalar_ptr(vb + row * (kHeadDim * 2));
      rel0 = 0;
    }
    // rows are clamped to the last key (a no-op except in the split's last
    // step), without a branch, so that every step issues the same loads
    if constexpr (KV == 0) {
      const uint32_t kk = (uint32_t)(min(j0 + n16, nl - 1) - j0 + rel0);
#pragma unroll
      for (int t = 0; t < 4; ++t) kreg[r][t] = kvload16<NT>(kb, kk * (kHeadDim * 2) + (4 * t + g4) * 16);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t kv = (uint32_t)(min(j0 + 4 * g4 + q, nl - 1) - j0 + rel0);
        vreg[r][q] = kvload16<NT>(vb, kv * (kHeadDim * 2) + n16 * 16);
      }
    }
  };
  using KHalf = std::integral_constant<int, 0>;
  using VHalf = std::integral_constant<int, 1>;
  auto issue = [&](int st, int r) {
    issue_half(st, r, KHalf{});
    issue_half(st, r, VHalf{});
  };

  // the query row and this lane's theta (every loop below over pairs has
  // m = lane) are loaded first, then the first three steps' K / V loads go out
  // before the prologue that needs them
  const double th_lane = BIFOCAL ? tt.th[lane] : 0.0;
  {
    const int qi = tid >> 4, c = tid & 15;
    uint4 v0 = make_uint4(0, 0, 0, 0);
    if (qi < p.G) v0 = gload16((const char*)p.q, (uint32_t)((((size_t)b * p.Hq + kvh * p.G + qi) * kHeadDim + c * 8) * 2));
    if (ns > 0) issue(0, 0);
    if (ns > 1) issue(1, 1);
    if (ns > 2) issue(2, 2);
    sQ[qi * 16 + c] = v0;
    sQ[kDecMaxG * 16 + qi * 16 + c] = v0;
  }
  float2* sT = (float2*)((char*)smem + kDecLdsT);
  float2* sBw = (float2*)((char*)smem + kDecLdsB) + wave * kPairs;
  // the offset table serves the far keys this split rotates (with a store:
  // those at or above its stored count)
  const bool rotates = split_far && (!STORE || min(k_end, far_lim) - kw0 > (long long)st_l);
  if (rotates) {
    // offset table: row idx, pair m = rotation by -theta_m * idx * kappa
    const double kappa = p.mode == 1 ? 1.0 : (double)(s - 1) / (double)s;
    for (int e = tid; e < kDecStep * kPairs; e += 256) {  // pair m = e % 64 = lane
      const int idx = e >> 6;
      float c, sn;
      dec_offset_cos_sin(th_lane, idx, kappa, c, sn);
      sT[idx * kDecTRow + lane] = make_float2(c, sn);
    }
  }
  lds_barrier();
  if (split_far) {
    // query angle numerator (phi(N - 1) - (N - 1)) s, plus (w0 - phi(w0)) s
    // with the band-edge continuity shift (w0 < N here, so no overflow)
    const double qn = dec_query_base(p.mode, p.shift, N, s, w0);
    float c, sn;
    turn_cos_sin(th_lane * kInv2Pi * qn, c, sn);
    for (int e = tid; e < p.G * kPairs; e += 256) {  // pair m = e % 64 = lane
      const int qi = e >> 6, m = lane;
      const uint16_t* row = (const uint16_t*)(sQ + qi * 16);
      const float x0 = dbf2f(row[m]), x1 = dbf2f(row[m + kPairs]);
      uint16_t* r2 = (uint16_t*)(sQ + kDecMaxG * 16 + qi * 16);
      r2[m] = df2bf(x0 * c - x1 * sn);
      r2[m + kPairs] = df2bf(x1 * c + x0 * sn);
    }
  }
  lds_barrier();
  // B operand of a step, read from LDS per step (Q' or Q''): lane (query n16,
  // group g4) holds head dims 32 t + 8 g4 .. +7
  auto q_operand = [&](bool corrected, dbf16x8 (&qo)[4]) {
    const uint4* src = sQ + (corrected ? kDecMaxG * 16 : 0) + n16 * 16 + g4;
#pragma unroll
    for (int t = 0; t < 4; ++t) qo[t] = __builtin_bit_cast(dbf16x8, src[4 * t]);
  };

  const double inv_s = 1.0 / (double)s;
  const float inv_s_f = 1.f / (float)s_i;
  const double th_turn = th_lane * kInv2Pi;  // this lane's pair m = lane
  // (q_pa, r_pa) = divmod(step start, s), advanced by 64 keys per step of this wave
  long long q_pa = 0;
  int r_pa = 0;
  if (BIFOCAL) {
    const long long k0 = kw0 + (long long)wave * kDecStep;  // this wave's first step
    q_pa = k0 / s;
    r_pa = (int)(k0 - q_pa * s);
  }
  constexpr int kAdv = kDecStep * kDecWaves;  // keys from one of this wave's steps to the next
  const int adv_q = kAdv / s_i, adv_r = kAdv % s_i;

  float m_used = -INFINITY, l_part = 0.f;
  df32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = df32x4{};

  // process step st from register slot r; REFILL 1: then load step st + 3
  // into the same slot (K as soon as QK^T has read it, V after P V),
  // REFILL 2: the same if step st + 3 exists
  auto process = [&](int st, int r, auto refill) {
    constexpr int REFILL = decltype(refill)::value;
    const bool more = REFILL == 1 || (REFILL == 2 && st + kDecRing < ns);
    const int jbl = jl_of(st);  // split-local first key of the step
    const bool any_far = BIFOCAL && jbl < far_l;
    const bool any_loc = !BIFOCAL || jbl + kDecStep - 1 >= far_l;
    uint4* kr = kreg[r];  // rotated in place
    df32x4 Sl = df32x4{};
    if (any_far && any_loc) {  // step straddles the window edge: local keys score with Q'
      dbf16x8 ql[4];
      q_operand(false, ql);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        Sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dbf16x8, kr[t]), ql[t], Sl, 0, 0, 0);
    }
    const bool stored = STORE && jbl + kDecStep <= st_l;  // k'' read from the store
    if (any_far && !stored) {
      // base rotation of the step, pair m = lane
      const long long jb = kw0 + jbl;
      const double qb = dec_step_base(p.mode, q_pa, jb, s, inv_s);
      float cb, sb;
      turn_cos_sin(th_turn * qb, cb, sb);
      sBw[lane] = make_float2(cb, sb);
      const int idx = dec_offset_row(p.mode, r_pa, n16, s_i, inv_s_f);
      if (jbl + n16 < far_l) {
        const float4* bq4 = (const float4*)sBw;
        const float4* tq4 = (const float4*)(sT + idx * kDecTRow);
        // rotary pairs (m, m + 64) = (element e of chunk 4 t + g4, same element of chunk 4 (t + 2) + g4)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          uint32_t* lo = (uint32_t*)&kr[t];
          uint32_t* hi = (uint32_t*)&kr[t + 2];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            // pairs m = 32 t + 8 g4 + 2 w and m + 1
            const float4 bq = bq4[16 * t + 4 * g4 + w];
            const float4 tq = tq4[16 * t + 4 * g4 + w];
            float c0, s0, c1, s1;
            dec_compose(bq.x, bq.y, tq.x, tq.y, c0, s0);
            dec_compose(bq.z, bq.w, tq.z, tq.w, c1, s1);
            uint32_t yo;
            lo[w] = rot_word(lo[w], hi[w], c0, s0, c1, s1, yo);
            hi[w] = yo;
          }
        }
        if constexpr (STORE) {  // this lane's key is far: keep its k'' (rows as loaded)
          if (jbl + n16 < nl) {
            char* wb = PAGED ? k2wb + page_row(jbl) * (kHeadDim * 2) : k2wb;
            const uint32_t row = (uint32_t)(PAGED ? n16 : jbl + n16) * (kHeadDim * 2);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              *(__attribute__((address_space(1))) du32x4*)(wb + row + (4 * t + g4) * 16) =
                  __builtin_bit_cast(du32x4, kr[t]);
          }
        }
      }
    }
    if (BIFOCAL) dec_advance(q_pa, r_pa, adv_q, adv_r, s_i);
    dbf16x8 qs[4];
    q_operand(any_far, qs);
    df32x4 S = df32x4{};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dbf16x8, kr[t]), qs[t], S, 0, 0, 0);
    if (REFILL != 0 && more) issue_half(st + kDecRing, r, KHalf{});
    if (any_far && any_loc) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (jbl + 4 * g4 + q >= far_l) S[q] = Sl[q];
    }
    // C layout: lane (query n16, g4) holds keys jbl + 4 g4 + q
    if (jbl + kDecStep > nl) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (jbl + 4 * g4 + q >= nl) S[q] = -INFINITY;
    }
    if (jbl < lo_l) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (jbl + 4 * g4 + q < lo_l) S[q] = -INFINITY;
    }
    // lazy rescale: the reference max of a query moves only when one of its
    // scores exceeds it by more than 2^8; the column max is needed only then
    float mx = fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3])) * p.scale_log2;
    if (__any(mx > m_used + kDecRescaleLog2)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m_used, mx);
      const float alpha = (m_used == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_used - mn);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
      m_used = mn;
    }
    const float mb = (m_used == -INFINITY) ? 0.f : m_used;
    float e[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      e[q] = __builtin_amdgcn_exp2f(fmaf(S[q], p.scale_log2, -mb));
      l_part += e[q];
    }
    const ds16x4 pb =
        __builtin_bit_cast(ds16x4, make_uint2(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])));
    // vreg[r][q]: key 4 g4 + q, head dims 8 n16 .. 8 n16 + 7
    const uint4* vr = vreg[r];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t w0q = ((const uint32_t*)&vr[0])[db >> 1], w1q = ((const uint32_t*)&vr[1])[db >> 1];
      const uint32_t w2q = ((const uint32_t*)&vr[2])[db >> 1], w3q = ((const uint32_t*)&vr[3])[db >> 1];
      const uint32_t sel = (db & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t x01 = __builtin_amdgcn_perm(w1q, w0q, sel), x23 = __builtin_amdgcn_perm(w3q, w2q, sel);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(ds16x4, make_uint2(x01, x23)), pb, oacc[db], 0, 0, 0);
    }
    if (REFILL != 0 && more) issue_half(st + kDecRing, r, VHalf{});
  };

  // steady state: every step refills its own slot with the step three ahead
  // (no branches, so the compiler's load-counter waits stay exact); the last
  // steps drain
  using Refill = std::integral_constant<int, 1>;
  using RefillIfAny = std::integral_constant<int, 2>;
  int st = 0;
  for (; st + 2 * kDecRing <= ns; st += kDecRing) {
    process(st, 0, Refill{});
    process(st + 1, 1, Refill{});
    process(st + 2, 2, Refill{});
  }
#pragma unroll
  for (int u = 0; u < 2 * kDecRing - 1; ++u) {
    const int cur = st + u;
    if (cur < ns) process(cur, u % kDecRing, RefillIfAny{});
  }

  // ---- merge the 4 waves, write the split's partial
  const float lsum = l_part + __shfl_xor(l_part, 16);
  const float ltot = lsum + __shfl_xor(lsum, 32);  // column total over the wave's keys
  __syncthreads();
  float* mw = (float*)smem;                 // [4][16]
  float* lw = mw + kDecWaves * kDecMaxG;    // [4][16]
  float* ow = lw + kDecWaves * kDecMaxG;    // [4][16][128]
  if (g4 == 0) {
    mw[wave * kDecMaxG + n16] = m_used;
    lw[wave * kDecMaxG + n16] = ltot;
  }
  // oacc[db][q] is O^T row (4 g4 + q) of block db = head dim 8 (4 g4 + q) + db, query n16
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ow[(wave * kDecMaxG + n16) * kHeadDim + 8 * (4 * g4 + q) + db] = oacc[db][q];
  __syncthreads();
  for (int e = tid; e < p.G * kHeadDim; e += 256) {
    const int qi = e >> 7, d = e & 127;
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mt = fmaxf(mt, mw[w * kDecMaxG + qi]);
    const float mbt = (mt == -INFINITY) ? 0.f : mt;
    float acc = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(mw[w * kDecMaxG + qi] - mbt);
      acc += f * ow[(w * kDecMaxG + qi) * kHeadDim + d];
      lt += f * lw[w * kDecMaxG + qi];
    }
    const size_t row = ((size_t)b * p.Hq + kvh * p.G + qi) * p.S + sp;
    p.part_acc[row * kHeadDim + d] = acc;
    if (d == 0) {
      p.part_m[row] = mt;
      p.part_l[row] = lt;
    }
  }
}

// Log-sum-exp merge of the splits. Workgroup = (query head, batch, quarter
// of the head dims). Thread t owns float4 d4 = t % 8 of the quarter for the
// splits t / 8 + 32 k: it loads their partial rows, maxima and row sums up
// front (the first 160 splits; more are read in a loop), so the merge costs
// one memory round trip plus two barriers: one for the maximum over all
// splits, one for the sums over the 32 split groups (three lane swaps inside
// a wave, then four LDS entries).
constexpr int kDecMaxSplits = 1088;
constexpr int kCombGroups = 32;  // split groups per workgroup
constexpr int kCombHold = 5;     // 32 x 5 = 160 splits held in registers
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p, DecodeSeqs ds) {
  __shared__ float red[8];
  __shared__ float4 part4[4][8];  // per-wave sums of the weighted rows
  const int b = blockIdx.y, h = blockIdx.x, dq = blockIdx.z, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int ns = ds.nsplit[b];
  const size_t row0 = ((size_t)b * p.Hq + h) * p.S;
  const int d4 = t & 7, grp = t >> 3;
  const int dcol = 32 * dq + 4 * d4;  // first head dim of this thread's float4
  float4 hold[kCombHold];
  float mi[kCombHold], li[kCombHold];
#pragma unroll
  for (int k = 0; k < kCombHold; ++k) {
    const int i = grp + kCombGroups * k;
    const size_t r = row0 + min(i, ns - 1);
    const float4 v = *(const float4*)(p.part_acc + r * kHeadDim + dcol);
    const float m = p.part_m[r], l = p.part_l[r];
    hold[k] = i < ns ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    mi[k] = i < ns ? m : -INFINITY;
    li[k] = i < ns ? l : 0.f;
  }
  float mloc = fmaxf(fmaxf(fmaxf(mi[0], mi[1]), fmaxf(mi[2], mi[3])), mi[4]);
  for (int i = grp + kCombGroups * kCombHold; i < ns; i += kCombGroups)
    mloc = fmaxf(mloc, p.part_m[row0 + i]);
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  const float mt = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float mbt = (mt == -INFINITY) ? 0.f : mt;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
#pragma unroll
  for (int k = 0; k < kCombHold; ++k) {
    const float w = __builtin_amdgcn_exp2f(mi[k] - mbt);  // 0 for absent splits
    acc.x += w * hold[k].x;
    acc.y += w * hold[k].y;
    acc.z += w * hold[k].z;
    acc.w += w * hold[k].w;
    lsum += w * li[k];
  }
  for (int i = grp + kCombGroups * kCombHold; i < ns; i += kCombGroups) {
    const float4 v = *(const float4*)(p.part_acc + (row0 + i) * kHeadDim + dcol);
    const float w = __builtin_amdgcn_exp2f(p.part_m[row0 + i] - mbt);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
    lsum += w * p.part_l[row0 + i];
  }
  // sums over the split groups: the lanes 8 g + d4 of a wave hold groups
  // 8 wave + g (every d4 lane carries the same row sum)
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o);
    acc.y += __shfl_xor(acc.y, o);
    acc.z += __shfl_xor(acc.z, o);
    acc.w += __shfl_xor(acc.w, o);
    lsum += __shfl_xor(lsum, o);
  }
  if (lane < 8) part4[wave][lane] = acc;
  if (lane == 0) red[4 + wave] = lsum;
  __syncthreads();
  if (t < 8) {
    const float4 a0 = part4[0][t], a1 = part4[1][t], a2 = part4[2][t], a3 = part4[3][t];
    const float4 a = make_float4((a0.x + a1.x) + (a2.x + a3.x), (a0.y + a1.y) + (a2.y + a3.y),
                                 (a0.z + a1.z) + (a2.z + a3.z), (a0.w + a1.w) + (a2.w + a3.w));
    const float lt = (red[4] + red[5]) + (red[6] + red[7]);
    const float inv = 1.f / lt;
    uint16_t* o = p.o + ((size_t)b * p.Hq + h) * kHeadDim + 32 * dq + 4 * t;
    uint2 w;
    w.x = (uint32_t)df2bf(a.x * inv) | ((uint32_t)df2bf(a.y * inv) << 16);
    w.y = (uint32_t)df2bf(a.z * inv) | ((uint32_t)df2bf(a.w * inv) << 16);
    *(uint2*)o = w;
    if (p.lse && t == 0 && dq == 0)
      p.lse[(size_t)b * p.Hq + h] = (mt + __log2f(lt)) * 0.69314718055994530942f;
  }
}

// ------------------------------------------------------------------ test hook
// The fp32 cos / sin the split kernel rotates with, for given positions:
// which = 2: the key at a.pos[n] of a call with s = a.s[n], through the
//   kernel's own angle addition (a split whose first key is the multiple of
//   1024 below the key, the divmod tracking of the wave that takes the key's
//   step, the step's base rotation, the offset-table row and the product of
//   the two);
// which = 3: the query at a.pos[n] (N = pos + 1 keys, s = a.s[n]).
// Block = position, thread = rotary pair; cs [n][64][2].
__global__ __launch_bounds__(64) void decode_angle_kernel(AngleProbe a, ThetaTable tt, int which,
                                                          float* cs) {
  const int n = blockIdx.x, m = threadIdx.x;
  const long long pos = a.pos[n], s = a.s[n];
  const int s_i = (int)s;
  float c, sn;
  if (which == 3) {
    turn_cos_sin(tt.th[m] * kInv2Pi * dec_query_base(a.mode, a.shift, pos + 1, s, a.w0), c, sn);
  } else {
    const long long kw0 = (pos / 1024) * 1024, jb = pos & ~15LL;
    const long long k0 = kw0 + (jb - kw0) / kDecStep % kDecWaves * kDecStep;  // the wave's first step
    long long q_pa = k0 / s;
    int r_pa = (int)(k0 - q_pa * s);
    constexpr int kAdv = kDecStep * kDecWaves;
    for (long long j = k0; j < jb; j += kAdv) dec_advance(q_pa, r_pa, kAdv / s_i, kAdv % s_i, s_i);
    float cb, sb, tc, ts;
    turn_cos_sin(tt.th[m] * kInv2Pi * dec_step_base(a.mode, q_pa, jb, s, 1.0 / (double)s), cb, sb);
    const int idx = dec_offset_row(a.mode, r_pa, (int)(pos - jb), s_i, 1.f / (float)s_i);
    dec_offset_cos_sin(tt.th[m], idx, a.mode == 1 ? 1.0 : (double)(s - 1) / (double)s, tc, ts);
    dec_compose(cb, sb, tc, ts, c, sn);
  }
  cs[((size_t)n * kPairs + m) * 2] = c;
  cs[((size_t)n * kPairs + m) * 2 + 1] = sn;
}

hipError_t launch_decode_angles(const AngleProbe& a, const ThetaTable& tt, int which, float* cs,
                                hipStream_t stream) {
  hipLaunchKernelGGL(decode_angle_kernel, dim3(a.n), dim3(64), 0, stream, a, tt, which, cs);
  return hipGetLastError();
}

// ------------------------------------------------------------------ host side
// Split geometry. The chip holds kDecTargetWgs split workgroups at once (two
// per CU of the 256 CUs: one round). For N keys of a sequence in a launch of
// `per` (sequence, KV head) groups the split count is the one that minimises
// rounds x (chunk + a fixed per-workgroup cost), over splits of 256 to
// kDecMaxChunk keys (at most kDecMaxTargetSplits splits unless the cap needs
// more), with the keys spread evenly; a last split of under a quarter chunk
// rides along without a round of its own. The bounds are build-time
// overridable for tuning.
#ifndef BF_DEC_TARGET_WGS
#define BF_DEC_TARGET_WGS 512
#endif
#ifndef BF_DEC_MAX_CHUNK
#define BF_DEC_MAX_CHUNK 4032
#endif
constexpr long long kDecTargetWgs = BF_DEC_TARGET_WGS;
constexpr long long kDecMaxChunk = BF_DEC_MAX_CHUNK;
// K + V bytes of a launch from which its loads are non-temporal (a quarter of
// the 256 MB MALL: smaller caches can stay resident between calls)
constexpr long long kDecStreamBytes = 64LL << 20;
constexpr long long kDecMaxTargetSplits = 128;
constexpr long long kDecMinChunk = 256;  // fewer keys per split cost more than they save
constexpr long long kDecWgCost = 256;    // fixed cost of a split workgroup, in keys
static_assert(kDecMaxChunk % kDecBlock == 0, "chunk must be a multiple of 64 keys");
static_assert(kDecMaxChunk / 16 + 1 <= 64 * kDecPageRegs,
              "a split's pages of 16 keys must fit the kernel's page-number registers");

static long long decode_target_splits(int batch, int Hkv) {
  return (long long)batch * Hkv;  // (sequence, KV head) groups sharing the launch
}

static int decode_chunk(long long N, long long per) {
  const long long need = (N + kDecMaxChunk - 1) / kDecMaxChunk;  // splits the cap forces
  long long most = (N + kDecMinChunk - 1) / kDecMinChunk;
  if (most > kDecMaxTargetSplits) most = kDecMaxTargetSplits;
  if (most < need) most = need;
  long long best_c = kDecMaxChunk, best_cost = -1;
  for (long long sp = need; sp <= most; ++sp) {
    long long c = (N + sp - 1) / sp;
    c = ((c + kDecBlock - 1) / kDecBlock) * kDecBlock;
    if (c > kDecMaxChunk) continue;
    const long long nsp = (N + c - 1) / c;
    const long long rem = N - (nsp - 1) * c;              // keys of the last split
    const long long heavy = nsp - (rem * 4 < c ? 1 : 0);  // a short last split rides along
    const long long rounds = (per * heavy + kDecTargetWgs - 1) / kDecTargetWgs;
    const long long cost = rounds * (c + kDecWgCost);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_c = c;
    }
  }
  return (int)best_c;
}

static int decode_splits(long long N, long long target) {
  const long long c = decode_chunk(N, target);
  return (int)((N + c - 1) / c);
}

// Upper bound of decode_splits over all lengths <= max_len and every target
// (splits <= target unless the chunk is capped at kDecMaxChunk).
static int decode_split_bound(long long max_len) {
  const long long a = (max_len + kDecMaxChunk - 1) / kDecMaxChunk + 1;
  return (int)(a > kDecMaxTargetSplits + 1 ? a : kDecMaxTargetSplits + 1);
}

struct DecodeWs {
  size_t m_off, l_off, acc_off, total;
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static DecodeWs decode_ws_layout(int batch, long long max_len, int Hq) {
  const size_t S = (size_t)decode_split_bound(max_len);
  DecodeWs w;
  w.m_off = 0;
  w.l_off = al256((size_t)batch * Hq * S * 4);
  w.acc_off = w.l_off + al256((size_t)batch * Hq * S * 4);
  w.total = w.acc_off + al256((size_t)batch * Hq * S * kHeadDim * 4);
  return w;
}

size_t decode_workspace_bytes(int batch, long long max_len, int Hq) {
  return decode_ws_layout(batch, max_len, Hq).total;
}

// A paged cache: pages [num_pages][Hkv][page_size][D]; sequence b's keys
// p * page_size .. (p + 1) * page_size - 1 live in page block_table[b][p].
struct PagedCache {
  const int* block_table;  // device [batch][max_pages], or null: contiguous cache
  int page_size;           // keys per page: a power of two >= 16
  int max_pages;           // row length of block_table
  int num_pages;           // pages in the pool
};

// A caller-kept far-key store (bifocal_decode_stored): k2 has the layout of
// the contiguous cache; keys 0 .. keys[b] - 1 of sequence b hold k'' for
// s = s[b]. Both host arrays are updated when the launch has been queued.
struct DecodeStore {
  void* k2;
  int32_t* keys;
  int32_t* s;
};

// ------------------------------------------------------------------ allocation-free decode
// Scratch for bifocal_decode_noalloc: the split partials (m, l, acc) live in
// this file-scope device array instead of a caller workspace. Each GPU the
// library runs on holds its own copy until the process ends; every call on
// that GPU shares it, so calls that overlap on one GPU race. The split kernel
// writes every partial the combine kernel reads, so no clearing is needed.
// Host code never passes the array's name to a kernel: it uses the device
// address hipGetSymbolAddress returns for the current device, looked up once
// per device and kept below.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices];  // per device: the device address of `scratch`
}  // namespace

size_t decode_noalloc_capacity() { return kNoAllocScratchBytes; }

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
int decode_noalloc_scratch(hipStream_t stream, void** out, std::string& err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    err = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return BF_ERR_HIP;
  }
  if (stream != nullptr) {  // the scratch used is the current device's
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) {
      err = std::string("hipStreamGetDevice: ") + hipGetErrorString(e);
      return BF_ERR_HIP;
    }
    if ((int)sdev != dev) {
      err = "stream belongs to device " + std::to_string((int)sdev) + ", the current device is " +
            std::to_string(dev);
      return BF_ERR_INVALID_ARG;
    }
  }
  if (dev < 0 || dev >= kScratchMaxDevices) {
    err = "device index " + std::to_string(dev) + " beyond the " + std::to_string(kScratchMaxDevices) +
          " devices the allocation-free decode tracks";
    return BF_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return BF_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BF_OK;
}

int run_decode(bool bifocal, const void* q, const void* kc, const void* vc, void* o, float* lse,
               const int32_t* seqlens, int batch, int cap, int Hq, int Hkv, long long w0,
               long long w_pre, double theta, int mode, float scale, void* ws, size_t ws_bytes,
               hipStream_t stream, std::string& err, long long window, const PagedCache* paged,
               bool validate_only, const DecodeStore* store) {
  auto bad = [&](int code, const std::string& m) { err = m; return code; };
  if (!q || !kc || !vc || !o || !seqlens) return bad(BF_ERR_INVALID_ARG, "null tensor or seqlens pointer");
  if (store) {
    if (!bifocal || window > 0)
      return bad(BF_ERR_UNSUPPORTED, "the far-key store serves FI / PA decode");
    if (!store->k2 || ((uintptr_t)store->k2 & 15u))
      return bad(BF_ERR_INVALID_ARG, "k2_store must be a non-null 16-byte aligned device pointer");
    if (!store->keys || !store->s) return bad(BF_ERR_INVALID_ARG, "null store_keys or store_s pointer");
    for (int b = 0; b < batch; ++b)
      if (store->keys[b] < 0 || store->s[b] < 0)
        return bad(BF_ERR_INVALID_ARG, "store_keys[" + std::to_string(b) + "] and store_s[" +
                                           std::to_string(b) + "] must be >= 0");
  }
  int page_log2 = 0;
  if (paged) {
    if (!paged->block_table || ((uintptr_t)paged->block_table & 3u))
      return bad(BF_ERR_INVALID_ARG, "block_table must be a non-null 4-byte aligned device pointer");
    const int ps = paged->page_size;
    if (ps < kDecStep || (ps & (ps - 1)) != 0 || ps > (1 << 20))
      return bad(BF_ERR_INVALID_ARG, "page_size must be a power of two in [16, 2^20] (got " + std::to_string(ps) + ")");
    while ((1 << page_log2) < ps) ++page_log2;
    if (paged->max_pages < 1 || paged->num_pages < 1)
      return bad(BF_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
    if ((long long)paged->max_pages * ps > 0x7fffffffLL)
      return bad(BF_ERR_INVALID_ARG, "max_pages_per_seq x page_size exceeds 2^31 - 1 keys");
    cap = paged->max_pages * ps;  // keys a sequence can hold
  }
  if (batch < 1 || cap < 1) return bad(BF_ERR_INVALID_ARG, "batch and cache_capacity must be >= 1");
  if (!(scale > 0.f) || !(scale < 1e30f)) return bad(BF_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  const int G = Hq / Hkv;
  if (G > kDecMaxG) return bad(BF_ERR_UNSUPPORTED, "decode supports at most 16 query heads per KV head");
  if (((uintptr_t)q | (uintptr_t)kc | (uintptr_t)vc | (uintptr_t)o) & 15u)
    return bad(BF_ERR_INVALID_ARG, "q, caches and o must be 16-byte aligned");
  if (lse && ((uintptr_t)lse & 3u)) return bad(BF_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  long long max_len = 0;
  for (int b = 0; b < batch; ++b) {
    if (seqlens[b] < 1 || seqlens[b] > cap)
      return bad(BF_ERR_INVALID_ARG, "seqlens[" + std::to_string(b) + "] out of [1, cache_capacity]");
    if (seqlens[b] > max_len) max_len = seqlens[b];
  }
  if (decode_split_bound(max_len) > kDecMaxSplits)
    return bad(BF_ERR_UNSUPPORTED, "decode supports at most " + std::to_string(kDecMaxSplits - 1) +
                                       " x " + std::to_string(kDecMaxChunk) + " keys per sequence");
  const DecodeWs wl = decode_ws_layout(batch, max_len, Hq);
  if (validate_only) return BF_OK;  // every argument but the workspace checked
  if (!ws) return bad(BF_ERR_WORKSPACE, "workspace is null");
  if ((uintptr_t)ws & 255u) return bad(BF_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < wl.total)
    return bad(BF_ERR_WORKSPACE, "workspace too small: " + std::to_string(ws_bytes) + " given, " +
                                     std::to_string(wl.total) + " needed");
  const char* ff = getenv("BIFOCAL_TEST_FAIL_LAUNCH");
  if (ff && ff[0] == '1') return bad(BF_ERR_HIP, "launch failure forced by BIFOCAL_TEST_FAIL_LAUNCH");

  ThetaTable tt;
  for (int m = 0; m < kPairs; ++m) tt.th[m] = pow(theta, -2.0 * (double)m / (double)kHeadDim);
  char* wsb = (char*)ws;
  DecodeParams dp;
  dp.cap = cap;
  dp.w0 = w0;
  dp.scale_log2 = scale * 1.4426950408889634f;
  dp.Hq = Hq;
  dp.Hkv = Hkv;
  dp.G = G;
  dp.S = decode_split_bound(max_len);
  dp.block_table = paged ? paged->block_table : nullptr;
  dp.max_pages = paged ? paged->max_pages : 0;
  dp.num_pages = paged ? paged->num_pages : 0;
  dp.page_log2 = page_log2;
  dp.shift = (mode & BF_LONG_SHIFT) ? 1 : 0;
  dp.mode = mode & ~BF_LONG_SHIFT;
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = batch - b0 < kMaxSeqPerLaunch ? batch - b0 : kMaxSeqPerLaunch;
    const long long target = decode_target_splits(nb, Hkv);
    DecodeSeqs ds;
    ds.n = nb;
    int max_split = 0;
    long long kv_bytes = 0;  // K and V bytes the launch reads
    for (int i = 0; i < nb; ++i) {
      const long long N = seqlens[b0 + i];
      ds.N[i] = (int)N;
      long long s = 1;
      if (bifocal) s = N / w_pre + (N % w_pre != 0 ? 1 : 0);
      ds.s[i] = (int)(s < 1 ? 1 : s);
      // a window (band-only attention) reads keys N - window .. N - 1 only,
      // from the multiple of 16 at or below N - window on (the rest masked)
      const long long kmin = window > 0 && N > window ? N - window : 0;
      const long long k0 = kmin & ~15LL;
      ds.kmin[i] = (int)kmin;
      ds.kstart[i] = (int)k0;
      ds.chunk[i] = decode_chunk(N - k0, target);
      ds.nsplit[i] = decode_splits(N - k0, target);
      if (ds.nsplit[i] > max_split) max_split = ds.nsplit[i];
      // far keys are 0 .. N - w0 - 1 (none when s = 1); the store's k'' count
      // only when it was made with this s, rounded down to whole 16-key steps
      const long long far_n = ds.s[i] > 1 && N > w0 ? N - w0 : 0;
      ds.stored[i] = 0;
      if (store && store->s[b0 + i] == ds.s[i])
        ds.stored[i] = (int)(std::min<long long>(store->keys[b0 + i], far_n) & ~15LL);
      kv_bytes += (N - k0) * Hkv * kHeadDim * 2 * 2;
    }
    dp.q = (const uint16_t*)q + (size_t)b0 * Hq * kHeadDim;
    // contiguous: the launch's first sequence; paged: the page pool, rows of
    // the block table from the launch's first sequence on
    dp.kc = (const uint16_t*)kc + (paged ? 0 : (size_t)b0 * Hkv * cap * kHeadDim);
    dp.vc = (const uint16_t*)vc + (paged ? 0 : (size_t)b0 * Hkv * cap * kHeadDim);
    dp.k2 = store ? (uint16_t*)store->k2 + (paged ? 0 : (size_t)b0 * Hkv * cap * kHeadDim) : nullptr;
    if (paged) dp.block_table = paged->block_table + (size_t)b0 * paged->max_pages;
    dp.o = (uint16_t*)o + (size_t)b0 * Hq * kHeadDim;
    dp.lse = lse ? lse + (size_t)b0 * Hq : nullptr;
    dp.part_m = (float*)(wsb + wl.m_off) + (size_t)b0 * Hq * dp.S;
    dp.part_l = (float*)(wsb + wl.l_off) + (size_t)b0 * Hq * dp.S;
    dp.part_acc = (float*)(wsb + wl.acc_off) + (size_t)b0 * Hq * dp.S * kHeadDim;
    if (getenv("BIFOCAL_TRACE") && getenv("BIFOCAL_TRACE")[0] == '1')
      fprintf(stderr, "[bifocal] decode %s seqs=%d..%d N0=%d s0=%d splits=%d chunk=%d\n",
              bifocal ? "bifocal" : "plain", b0, b0 + nb - 1, ds.N[0], ds.s[0], ds.nsplit[0], ds.chunk[0]);
    dim3 grid(max_split, Hkv, nb);
    // non-temporal K / V loads unless the launch reads little enough that
    // its cache could stay resident in the 256 MB MALL between calls
    const bool nt = kv_bytes >= kDecStreamBytes;
    auto kern = store ? (paged ? (nt ? decode_split_kernel<true, true, true, true> : decode_split_kernel<true, true, false, true>)
                               : (nt ? decode_split_kernel<true, false, true, true> : decode_split_kernel<true, false, false, true>))
              : bifocal ? (paged ? (nt ? decode_split_kernel<true, true, true> : decode_split_kernel<true, true, false>)
                                 : (nt ? decode_split_kernel<true, false, true> : decode_split_kernel<true, false, false>))
                        : (paged ? (nt ? decode_split_kernel<false, true, true> : decode_split_kernel<false, true, false>)
                                 : (nt ? decode_split_kernel<false, false, true> : decode_split_kernel<false, false, false>));
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, dp, ds, tt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return bad(BF_ERR_HIP, std::string("decode split launch: ") + hipGetErrorString(e));
    hipLaunchKernelGGL(decode_combine_kernel, dim3(Hq, nb, kHeadDim / 32), dim3(256), 0, stream, dp, ds);
    e = hipGetLastError();
    if (e != hipSuccess) return bad(BF_ERR_HIP, std::string("decode combine launch: ") + hipGetErrorString(e));
    if (store)  // the store as the stream leaves this launch: k'' of every far key for s
      for (int i = 0; i < nb; ++i) {
        const long long N = ds.N[i];
        store->keys[b0 + i] = ds.s[i] > 1 && N > w0 ? (int32_t)(N - w0) : 0;
        store->s[b0 + i] = ds.s[i];
      }
  }
  return BF_OK;
}

}  // namespace bf
