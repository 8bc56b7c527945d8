// Raw-input pre-step on gfx950: the model's original RoPE applied to raw
// (position-free) q and k, and the KV-cache append of k' and v. The pages'
// flow starts by computing RoPE for the current positions, and cached keys
// carry original RoPE [mufans.github.io knowledge-base wiki, Jet-Long
// Dynamic RoPE, "关键实现 / 推理流程", first step; ai-feeds.com summary,
// "关键模块" item 3]; these kernels produce exactly the inputs
// bifocal_prefill / bifocal_decode take.
//
// Rotation (half-split pairs, theta_m = rope_theta^(-2m/D)):
//   x'[m]      = x[m] cos(p theta_m) - x[m + 64] sin(p theta_m)
//   x'[m + 64] = x[m + 64] cos(p theta_m) + x[m] sin(p theta_m)
// The angle p * theta_m is formed in fp64 (it reaches 2e9 rad at theta_0 = 1
// and p near 2^31) and reduced to [-pi, pi] in fp64 by Cody and Waite's
// method (2 pi split into a double and a correction); the reduced angle's
// cosine / sine are taken in fp32, and the rotation runs in fp32, rounded
// once to the storage type.
//
// Layout of the work: 8 lanes per (token, chunk of head rows), lane u holding
// pairs 8u .. 8u + 7 (elements 8u .. 8u + 7 and their partners 64 + 8u ..),
// so a row moves as 16-byte (bf16) or 32-byte (fp32) pieces. The
// head rows of a token are the Hq query rows, then the Hkv key rows. With
// many tokens one group takes all of a token's rows (one angle set serves
// every head); with few (a decode step) each row gets its own group, so the
// step costs one memory round trip. A group loads four rows before it stores
// any (outputs either are their inputs or do not overlap them), keeping four
// loads in flight per lane.
#include <hip/hip_runtime.h>

#include <string>

#include "bifocal.h"
#include "bf_common.h"

namespace bf {

struct RopeParams {
  const void* q;     // raw queries, row (h, t) at q + (h * q_hs + t * q_ts) elements
  const void* k;     // raw keys, same for (h, t) with k_hs / k_ts
  const void* v;     // values copied to the cache (may be null when no cache)
  void* q_out;       // rotated queries, same layout as q
  void* k_out;       // rotated keys, same layout as k (may be null: cache only)
  void* k_cache;     // [B][Hkv][cap][D], pages [num_pages][Hkv][page][D], or null
  void* v_cache;     // same layout as k_cache
  PagedKV pk;        // block_table non-null: the caches are paged (rows of this launch)
  long long q_hs, q_ts;  // element strides of q / q_out: per head, per token
  long long k_hs, k_ts;  // element strides of k / k_out / v: per head, per token
  long long cap;         // cache capacity (tokens)
  int n_tok;             // tokens of the launch
  int Hq, Hkv;
  int rows_per_group;    // head rows per 8-lane group (Hq + Hkv: a whole token)
  int groups_per_tok;    // ceil((Hq + Hkv) / rows_per_group)
};

// Token t of a launch: its sequence b and position; prefill tokens are packed
// (cu offsets; sequence b's positions run from pos0[b]), decode tokens are one
// per sequence at position N_b - 1.
struct RopeSeqs {
  int n;                          // sequences in the launch
  int cu[kMaxSeqPerLaunch + 1];   // prefill: token offsets; decode: unused
  int pos0[kMaxSeqPerLaunch];     // decode: position of sequence b's token; prefill: its first token's
  int decode;                     // 1: token t is sequence t at pos0[t]
};

__device__ __forceinline__ uint32_t rope_bf16(float f) {  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// cos / sin of an angle a (rad, fp64): a - k 2 pi with k = rint(a / 2 pi), the
// product k 2 pi taken in two fused steps (2 pi = kTwoPiHi + kTwoPiLo), so
// the reduced angle is accurate to ~1e-16 rad relative to a; then fp32
// sincosf on [-pi, pi].
constexpr double kInvTwoPi = 0.15915494309189533577;
constexpr double kTwoPiHi = 6.283185307179586232;    // 2 pi rounded to fp64
constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2 pi - kTwoPiHi
__device__ __forceinline__ void rope_cos_sin(double a, float& c, float& s) {
  const double k = rint(a * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, a);
  r = fma(-k, kTwoPiLo, r);
  sincosf((float)r, &s, &c);
}

// eight consecutive elements of a row, as loaded and stored
template <typename T>
struct Oct;
template <>
struct Oct<uint16_t> {
  typedef uint4 V;
  __device__ static void unpack(V v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static V pack(const float (&f)[8]) {
    return make_uint4(rope_bf16(f[0]) | (rope_bf16(f[1]) << 16), rope_bf16(f[2]) | (rope_bf16(f[3]) << 16),
                      rope_bf16(f[4]) | (rope_bf16(f[5]) << 16), rope_bf16(f[6]) | (rope_bf16(f[7]) << 16));
  }
};
struct F8 {
  float4 a, b;
};
template <>
struct Oct<float> {
  typedef F8 V;
  __device__ static void unpack(V v, float (&f)[8]) {
    f[0] = v.a.x; f[1] = v.a.y; f[2] = v.a.z; f[3] = v.a.w;
    f[4] = v.b.x; f[5] = v.b.y; f[6] = v.b.z; f[7] = v.b.w;
  }
  __device__ static V pack(const float (&f)[8]) {
    return F8{make_float4(f[0], f[1], f[2], f[3]), make_float4(f[4], f[5], f[6], f[7])};
  }
};

// Loads and stores of one 8-element piece, optionally non-temporal: a large
// pre-step streams every byte once (each input read once, each output written
// once), and keeping those lines in the caches only evicts others.
typedef __attribute__((ext_vector_type(4))) unsigned int ru32x4;
typedef __attribute__((ext_vector_type(4))) float rf32x4;
template <bool NT, typename E>
__device__ __forceinline__ E ld_piece(const E* p) {
  if constexpr (NT) return __builtin_nontemporal_load((const __attribute__((address_space(1))) E*)p);
  else return *(const __attribute__((address_space(1))) E*)p;
}
template <bool NT, typename E>
__device__ __forceinline__ void st_piece(E* p, E v) {
  if constexpr (NT) __builtin_nontemporal_store(v, (__attribute__((address_space(1))) E*)p);
  else *(__attribute__((address_space(1))) E*)p = v;
}
template <bool NT>
__device__ __forceinline__ uint4 ld_oct(const uint4* p) {
  return __builtin_bit_cast(uint4, ld_piece<NT>((const ru32x4*)p));
}
template <bool NT>
__device__ __forceinline__ F8 ld_oct(const F8* p) {
  const rf32x4* q = (const rf32x4*)p;
  return F8{__builtin_bit_cast(float4, ld_piece<NT>(q)), __builtin_bit_cast(float4, ld_piece<NT>(q + 1))};
}
template <bool NT>
__device__ __forceinline__ void st_oct(uint4* p, uint4 v) {
  st_piece<NT>((ru32x4*)p, __builtin_bit_cast(ru32x4, v));
}
template <bool NT>
__device__ __forceinline__ void st_oct(F8* p, F8 v) {
  rf32x4* q = (rf32x4*)p;
  st_piece<NT>(q, __builtin_bit_cast(rf32x4, v.a));
  st_piece<NT>(q + 1, __builtin_bit_cast(rf32x4, v.b));
}

template <typename T, bool NT>
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p, RopeSeqs sq, ThetaTable tt) {
  typedef typename Oct<T>::V V;
  constexpr int kBatch = 4;  // rows loaded before the first store
  const long long g = (long long)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int u = threadIdx.x & 7;
  if (g >= (long long)p.n_tok * p.groups_per_tok) return;
  const int t = (int)(g / p.groups_per_tok);
  const int r0 = (int)(g % p.groups_per_tok) * p.rows_per_group;
  const int r1 = min(p.Hq + p.Hkv, r0 + p.rows_per_group);
  int b, pos;
  if (sq.decode) {
    b = t;
    pos = sq.pos0[t];
  } else {
    b = 0;
    while (b + 1 < sq.n && t >= sq.cu[b + 1]) ++b;
    pos = sq.pos0[b] + t - sq.cu[b];
  }
  // cos / sin of pairs 8u .. 8u + 7 at this position
  float c[8], s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) rope_cos_sin((double)pos * tt.th[8 * u + e], c[e], s[e]);
  auto rotate = [&](V lo_v, V hi_v, V& lo_o, V& hi_o) {
    float lo[8], hi[8], ro[8], rh[8];
    Oct<T>::unpack(lo_v, lo);
    Oct<T>::unpack(hi_v, hi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ro[e] = lo[e] * c[e] - hi[e] * s[e];
      rh[e] = hi[e] * c[e] + lo[e] * s[e];
    }
    lo_o = Oct<T>::pack(ro);
    hi_o = Oct<T>::pack(rh);
  };
  // element offset of lane u's low piece inside a row; the high piece is 64 on
  const int e_lo = 8 * u, e_hi = kPairs + 8 * u;
  // element offset of head row j (query rows first, then key rows)
  auto row_off = [&](int j) {
    return j < p.Hq ? j * p.q_hs + (long long)t * p.q_ts
                    : (j - p.Hq) * p.k_hs + (long long)t * p.k_ts;
  };
  const bool cache = p.k_cache != nullptr;
  for (int j0 = r0; j0 < r1; j0 += kBatch) {
    V lo[kBatch], hi[kBatch], vlo[kBatch], vhi[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = j0 + i;
      if (j < r1) {
        const T* src = (const T*)(j < p.Hq ? p.q : p.k) + row_off(j);
        lo[i] = ld_oct<NT>((const V*)(src + e_lo));
        hi[i] = ld_oct<NT>((const V*)(src + e_hi));
        if (cache && j >= p.Hq) {
          const T* vs = (const T*)p.v + row_off(j);
          vlo[i] = ld_oct<NT>((const V*)(vs + e_lo));
          vhi[i] = ld_oct<NT>((const V*)(vs + e_hi));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = j0 + i;
      if (j >= r1) break;
      V lo_o, hi_o;
      rotate(lo[i], hi[i], lo_o, hi_o);
      const long long r = row_off(j);
      if (j < p.Hq) {
        T* dst = (T*)p.q_out + r;
        st_oct<NT>((V*)(dst + e_lo), lo_o);
        st_oct<NT>((V*)(dst + e_hi), hi_o);
        continue;
      }
      if (p.k_out) {
        T* dst = (T*)p.k_out + r;
        st_oct<NT>((V*)(dst + e_lo), lo_o);
        st_oct<NT>((V*)(dst + e_hi), hi_o);
      }
      if (cache) {
        const int h = j - p.Hq;
        long long crow;  // cache row of (sequence b, KV head h, position pos)
        if (p.pk.block_table != nullptr) {
          int pg = p.pk.block_table[(size_t)b * p.pk.max_pages + (pos >> p.pk.page_log2)];
          pg = min(max(pg, 0), p.pk.num_pages - 1);
          crow = (((long long)pg * p.Hkv + h) << p.pk.page_log2) + (pos & ((1 << p.pk.page_log2) - 1));
        } else {
          crow = ((long long)b * p.Hkv + h) * p.cap + pos;
        }
        const long long cr = crow * kHeadDim;
        T* kc = (T*)p.k_cache + cr;
        T* vc = (T*)p.v_cache + cr;
        st_oct<NT>((V*)(kc + e_lo), lo_o);
        st_oct<NT>((V*)(kc + e_hi), hi_o);
        st_oct<NT>((V*)(vc + e_lo), vlo[i]);
        st_oct<NT>((V*)(vc + e_hi), vhi[i]);
      }
    }
  }
}

static hipError_t launch_rope(int dtype, RopeParams p, const RopeSeqs& sq,
                              const ThetaTable& tt, hipStream_t stream) {
  // rows per group: about 262144 groups per launch (four rounds of the 256
  // CUs x 256 groups a launch holds), a whole token per group at most
  const int rows = p.Hq + p.Hkv;
  const long long rpg = (long long)rows * p.n_tok / 262144;
  p.rows_per_group = (int)(rpg < 1 ? 1 : (rpg > rows ? rows : rpg));
  p.groups_per_tok = (rows + p.rows_per_group - 1) / p.rows_per_group;
  const long long groups = (long long)p.n_tok * p.groups_per_tok;
  const int grid = (int)((groups + 31) / 32);
  // non-temporal when the launch moves at least 64 MB (a quarter of the
  // 256 MB MALL); a small step's outputs may still be cached for the next call
  const long long moved = (long long)rows * p.n_tok * kHeadDim * (dtype == 0 ? 2 : 4) * 2;
  const bool nt = moved >= (64LL << 20);
  if (dtype == 0) {
    if (nt) hipLaunchKernelGGL((rope_kernel<uint16_t, true>), dim3(grid), dim3(256), 0, stream, p, sq, tt);
    else hipLaunchKernelGGL((rope_kernel<uint16_t, false>), dim3(grid), dim3(256), 0, stream, p, sq, tt);
  } else {
    if (nt) hipLaunchKernelGGL((rope_kernel<float, true>), dim3(grid), dim3(256), 0, stream, p, sq, tt);
    else hipLaunchKernelGGL((rope_kernel<float, false>), dim3(grid), dim3(256), 0, stream, p, sq, tt);
  }
  return hipGetLastError();
}

// Prefill layout [H][T][D]: one launch per group of kMaxSeqPerLaunch
// sequences; sequence b's tokens sit at positions P_b .. P_b + L_b - 1
// (P_b = pos0[b], 0 when pos0 is null), and the cache (if any) is
// [batch][Hkv][cap][D] with those tokens at those positions.
int run_rope_prefill(const void* q, const void* k, const void* v, void* q_out, void* k_out,
                     void* k_cache, void* v_cache, int cap, const int32_t* cu, const int32_t* pos0,
                     const PagedKV& pk, int batch, int Hq,
                     int Hkv, int dtype, double theta, hipStream_t stream, std::string& err) {
  ThetaTable tt;
  for (int m = 0; m < kPairs; ++m) tt.th[m] = pow(theta, -2.0 * (double)m / (double)kHeadDim);
  const size_t es = dtype == 0 ? 2 : 4;
  const long long T = cu[batch];
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = batch - b0 < kMaxSeqPerLaunch ? batch - b0 : kMaxSeqPerLaunch;
    RopeSeqs sq;
    sq.n = nb;
    sq.decode = 0;
    for (int i = 0; i <= nb; ++i) sq.cu[i] = cu[b0 + i] - cu[b0];
    for (int i = 0; i < nb; ++i) sq.pos0[i] = pos0 ? pos0[b0 + i] : 0;
    const long long t0 = cu[b0];
    RopeParams p;
    p.q = (const char*)q + t0 * kHeadDim * es;
    p.k = (const char*)k + t0 * kHeadDim * es;
    p.v = v ? (const char*)v + t0 * kHeadDim * es : nullptr;
    p.q_out = (char*)q_out + t0 * kHeadDim * es;
    p.k_out = k_out ? (char*)k_out + t0 * kHeadDim * es : nullptr;
    const bool paged = pk.block_table != nullptr;
    p.k_cache = !k_cache ? nullptr : paged ? k_cache : (char*)k_cache + (size_t)b0 * Hkv * cap * kHeadDim * es;
    p.v_cache = !v_cache ? nullptr : paged ? v_cache : (char*)v_cache + (size_t)b0 * Hkv * cap * kHeadDim * es;
    p.pk = pk;
    if (paged) p.pk.block_table += (size_t)b0 * pk.max_pages;
    p.q_hs = T * kHeadDim;
    p.q_ts = kHeadDim;
    p.k_hs = T * kHeadDim;
    p.k_ts = kHeadDim;
    p.cap = cap;
    p.n_tok = cu[b0 + nb] - cu[b0];
    p.Hq = Hq;
    p.Hkv = Hkv;
    const hipError_t e = launch_rope(dtype, p, sq, tt, stream);
    if (e != hipSuccess) {
      err = std::string("rope launch: ") + hipGetErrorString(e);
      return BF_ERR_HIP;
    }
  }
  return BF_OK;
}

// Decode layout: q [batch][Hq][D], k / v [batch][Hkv][D], one token per
// sequence at position seqlens[b] - 1, appended to [batch][Hkv][cap][D].
int run_rope_append(const void* q, const void* k, const void* v, void* q_out, void* k_cache,
                    void* v_cache, int cap, const int32_t* seqlens, const PagedKV& pk, int batch,
                    int Hq, int Hkv,
                    int dtype, double theta, hipStream_t stream, std::string& err) {
  ThetaTable tt;
  for (int m = 0; m < kPairs; ++m) tt.th[m] = pow(theta, -2.0 * (double)m / (double)kHeadDim);
  const size_t es = dtype == 0 ? 2 : 4;
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = batch - b0 < kMaxSeqPerLaunch ? batch - b0 : kMaxSeqPerLaunch;
    RopeSeqs sq;
    sq.n = nb;
    sq.decode = 1;
    for (int i = 0; i <= nb; ++i) sq.cu[i] = 0;
    for (int i = 0; i < nb; ++i) sq.pos0[i] = seqlens[b0 + i] - 1;
    RopeParams p;
    p.q = (const char*)q + (size_t)b0 * Hq * kHeadDim * es;
    p.k = (const char*)k + (size_t)b0 * Hkv * kHeadDim * es;
    p.v = (const char*)v + (size_t)b0 * Hkv * kHeadDim * es;
    p.q_out = (char*)q_out + (size_t)b0 * Hq * kHeadDim * es;
    p.k_out = nullptr;
    const bool paged = pk.block_table != nullptr;
    p.k_cache = paged ? k_cache : (char*)k_cache + (size_t)b0 * Hkv * cap * kHeadDim * es;
    p.v_cache = paged ? v_cache : (char*)v_cache + (size_t)b0 * Hkv * cap * kHeadDim * es;
    p.pk = pk;
    if (paged) p.pk.block_table += (size_t)b0 * pk.max_pages;
    p.q_hs = kHeadDim;
    p.q_ts = (long long)Hq * kHeadDim;
    p.k_hs = kHeadDim;
    p.k_ts = (long long)Hkv * kHeadDim;
    p.cap = cap;
    p.n_tok = nb;
    p.Hq = Hq;
    p.Hkv = Hkv;
    const hipError_t e = launch_rope(dtype, p, sq, tt, stream);
    if (e != hipSuccess) {
      err = std::string("rope append launch: ") + hipGetErrorString(e);
      return BF_ERR_HIP;
    }
  }
  return BF_OK;
}

}  // namespace bf
