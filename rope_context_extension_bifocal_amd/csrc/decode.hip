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
//   and the split writes its (m, l, acc) partial.
// decode_combine_kernel: log-sum-exp merge of the splits of each query head.
#include <hip/hip_runtime.h>

#include <string>

#include "bifocal.h"
#include "bf_common.h"

namespace bf {

typedef __attribute__((ext_vector_type(8))) __bf16 dbf16x8;
typedef __attribute__((ext_vector_type(4))) short ds16x4;
typedef __attribute__((ext_vector_type(4))) float df32x4;

constexpr int kDecBlock = 64;    // keys per streamed block
constexpr int kDecMaxG = 16;     // query heads per KV head the kernel supports
constexpr int kDecVRow = 136;    // padded LDS row of V (elements)

struct DecodeParams {
  const uint16_t* q;    // [B][Hq][D]
  const uint16_t* kc;   // [B][Hkv][cap][D]
  const uint16_t* vc;   // [B][Hkv][cap][D]
  float* part_m;        // [B][Hq][S]  running max (log2 domain, scaled)
  float* part_l;        // [B][Hq][S]
  float* part_acc;      // [B][Hq][S][D]
  uint16_t* o;          // [B][Hq][D]
  float* lse;           // [B][Hq] or null
  long long cap;
  long long w0;
  float scale_log2;
  int Hq, Hkv, G, S;
  int mode;
};

struct DecodeSeqs {
  int n;
  int N[kMaxSeqPerLaunch];       // valid keys (query at N - 1)
  int s[kMaxSeqPerLaunch];       // s(N)
  int nsplit[kMaxSeqPerLaunch];
  int chunk[kMaxSeqPerLaunch];   // keys per split (multiple of 64)
};

__device__ __forceinline__ float dbf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t df2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ long long dcorr_num(long long p, long long s, int mode) {
  return mode == 1 ? (p / s - p) * s : -p * (s - 1);
}

// cos / sin of theta_m * (phi(p) - p): the angle and its reduction to one
// turn are done in fp64 (exact integer numerator, ~1e5 rad at 128K), the
// reduced turn fraction goes through the hardware sin / cos (input in turns).
__device__ __forceinline__ void corr_cos_sin(double th, long long num, long long s, float& c,
                                             float& sn) {
  const double turns = th * ((double)num / (double)s) * 0.15915494309189533577;
  const float fr = (float)(turns - rint(turns));
  sn = __builtin_amdgcn_sinf(fr);
  c = __builtin_amdgcn_cosf(fr);
}

// ------------------------------------------------------------------ kernels
// Split kernel: workgroup = (batch b, KV head, split of `chunk` keys). Each of
// the 4 waves streams its own contiguous quarter of the split in 16-key steps,
// independently of the other waves:
//   - the 16 keys' K rows go straight into registers, laid out as the A
//     operand of MFMA 16x16x32 (lane = key n16, head-dim chunks 4 t + g4), so
//     both halves (m, m + 64) of every rotary pair sit in the same lane and the
//     correction rotation of far keys is done in place;
//   - the 16 keys' V rows go by direct global->LDS loads into a wave-private
//     ring; P V uses the head-dim order d = 8 row + block so that one 16-byte
//     LDS read per key feeds all 8 output blocks;
//   - loads run two steps ahead of compute.
// The G query heads of the KV group are the MFMA columns (columns >= G are
// zero queries whose results are dropped).
constexpr int kDecWaves = 4;
constexpr int kDecStep = 16;  // keys per wave step
constexpr int kDecRing = 3;   // V ring slots per wave (two steps in flight)
constexpr float kDecRescaleLog2 = 8.f;

__device__ __forceinline__ void dec_wait_vm(int outstanding_steps) {
  // loads complete in issue order; each step issues 8 vector-memory operations
  if (outstanding_steps >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (outstanding_steps == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool BIFOCAL>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeParams p, DecodeSeqs ds,
                                                              ThetaTable tt) {
  // LDS: V rings [4 waves][3 slots][16 keys x 16 chunks] | Q' and Q'' [2][16][16 chunks]
  __shared__ uint4 smem[kDecWaves * kDecRing * 256 + 2 * kDecMaxG * 16];
  uint4* sQ = smem + kDecWaves * kDecRing * 256;

  const int b = blockIdx.z, kvh = blockIdx.y, sp = blockIdx.x;
  if (sp >= ds.nsplit[b]) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const long long N = ds.N[b];
  const long long s = ds.s[b];
  const long long w0 = (BIFOCAL && s > 1) ? p.w0 : (1LL << 62);
  const long long far_lim = N - w0;  // keys j < far_lim are far
  const int chunk = ds.chunk[b];
  const long long k_begin = (long long)sp * chunk;
  const long long k_end = min(N, k_begin + chunk);
  const int per = chunk / kDecWaves;  // multiple of 16
  const long long kw0 = k_begin + (long long)wave * per;
  const long long kw1 = min(k_end, kw0 + per);
  const int ns = kw1 > kw0 ? (int)((kw1 - kw0 + kDecStep - 1) / kDecStep) : 0;

  // ---- queries: Q' as given, Q'' = R(Delta(N - 1)) Q'; rows >= G are zero
  {
    const int qi = tid >> 4, c = tid & 15;
    uint4 v0 = make_uint4(0, 0, 0, 0);
    if (qi < p.G) v0 = *(const uint4*)(p.q + ((size_t)b * p.Hq + kvh * p.G + qi) * kHeadDim + c * 8);
    sQ[qi * 16 + c] = v0;
    sQ[kDecMaxG * 16 + qi * 16 + c] = v0;
  }
  __syncthreads();
  if (BIFOCAL && far_lim > 0) {
    for (int e = tid; e < p.G * kPairs; e += 256) {
      const int qi = e >> 6, m = e & 63;
      double sd, cd;
      sincos(tt.th[m] * ((double)dcorr_num(N - 1, s, p.mode) / (double)s), &sd, &cd);
      const float c = (float)cd, sn = (float)sd;
      const uint16_t* row = (const uint16_t*)(sQ + qi * 16);
      const float x0 = dbf2f(row[m]), x1 = dbf2f(row[m + kPairs]);
      uint16_t* r2 = (uint16_t*)(sQ + kDecMaxG * 16 + qi * 16);
      r2[m] = df2bf(x0 * c - x1 * sn);
      r2[m + kPairs] = df2bf(x1 * c + x0 * sn);
    }
  }
  __syncthreads();
  dbf16x8 qf[4], qf2[4];  // B operand: lane (query n16, group g4), head dims 32 t + 8 g4 .. +7
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    qf[t] = __builtin_bit_cast(dbf16x8, sQ[n16 * 16 + 4 * t + g4]);
    qf2[t] = __builtin_bit_cast(dbf16x8, sQ[kDecMaxG * 16 + n16 * 16 + 4 * t + g4]);
  }

  const uint16_t* kbase = p.kc + ((size_t)b * p.Hkv + kvh) * (size_t)p.cap * kHeadDim;
  const uint16_t* vbase = p.vc + ((size_t)b * p.Hkv + kvh) * (size_t)p.cap * kHeadDim;
  uint4* vring = smem + wave * (kDecRing * 256);
  const double inv_s = 1.0 / (double)s;

  float m_used = -INFINITY, l_part = 0.f;
  df32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = df32x4{};

  uint4 kreg[kDecRing][4];
  // issue the loads of step st into ring slot r: V rows first, then this lane's K row
  auto issue = [&](int st, int r) {
    const long long j0 = kw0 + (long long)st * kDecStep;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long long key = min(j0 + 4 * i + (lane >> 4), kw1 - 1);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(vbase + (size_t)key * kHeadDim + (lane & 15) * 8),
          (__attribute__((address_space(3))) void*)(vring + r * 256 + i * 64), 16, 0, 0);
    }
    const long long key = min(j0 + n16, kw1 - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      kreg[r][t] = *(const uint4*)(kbase + (size_t)key * kHeadDim + (4 * t + g4) * 8);
  };

  auto process = [&](int st, int r) {
    const long long jb = kw0 + (long long)st * kDecStep;
    const bool any_far = BIFOCAL && jb < far_lim;
    const bool any_loc = !BIFOCAL || jb + kDecStep - 1 >= far_lim;
    uint4 kr[4] = {kreg[r][0], kreg[r][1], kreg[r][2], kreg[r][3]};
    const long long j = jb + n16;  // this lane's A-operand key
    if (any_far && j < far_lim) {
      // rotary pairs (m, m + 64) = (element e of chunk 4 t + g4, same element of chunk 4 (t + 2) + g4)
      const double qn = (double)dcorr_num(j, s, p.mode) * inv_s;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t* lo = (uint32_t*)&kr[t];
        uint32_t* hi = (uint32_t*)&kr[t + 2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int m0 = 32 * t + 8 * g4 + 2 * w;
          const double tu0 = tt.th[m0] * qn * 0.15915494309189533577;
          const double tu1 = tt.th[m0 + 1] * qn * 0.15915494309189533577;
          const float f0 = (float)(tu0 - rint(tu0)), f1 = (float)(tu1 - rint(tu1));
          const float c0 = __builtin_amdgcn_cosf(f0), s0 = __builtin_amdgcn_sinf(f0);
          const float c1 = __builtin_amdgcn_cosf(f1), s1 = __builtin_amdgcn_sinf(f1);
          const float a0 = __uint_as_float(lo[w] << 16), a1 = __uint_as_float(lo[w] & 0xffff0000u);
          const float b0 = __uint_as_float(hi[w] << 16), b1 = __uint_as_float(hi[w] & 0xffff0000u);
          lo[w] = (uint32_t)df2bf(a0 * c0 - b0 * s0) | ((uint32_t)df2bf(a1 * c1 - b1 * s1) << 16);
          hi[w] = (uint32_t)df2bf(b0 * c0 + a0 * s0) | ((uint32_t)df2bf(b1 * c1 + a1 * s1) << 16);
        }
      }
    }
    df32x4 S = df32x4{};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dbf16x8, kr[t]),
                                                  any_far ? qf2[t] : qf[t], S, 0, 0, 0);
    if (any_far && any_loc) {  // step straddles the window edge: local keys score with Q'
      df32x4 Sl = df32x4{};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        Sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dbf16x8, kreg[r][t]), qf[t],
                                                     Sl, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (jb + 4 * g4 + q >= far_lim) S[q] = Sl[q];
    }
    // C layout: lane (query n16, g4) holds keys jb + 4 g4 + q
    if (jb + kDecStep > kw1) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (jb + 4 * g4 + q >= kw1) S[q] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx *= p.scale_log2;
    if (__any(mx > m_used + kDecRescaleLog2)) {
      const float mn = fmaxf(m_used, mx);
      const float alpha = (m_used == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_used - mn);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
      m_used = mn;
    }
    const float mb = (m_used == -INFINITY) ? 0.f : m_used;
    ds16x4 pb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float e = __builtin_amdgcn_exp2f(fmaf(S[q], p.scale_log2, -mb));
      l_part += e;
      pb[q] = (short)df2bf(e);
    }
    // V rows of keys 4 g4 + q, chunk n16 (head dims 8 n16 .. 8 n16 + 7)
    uint4 vr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) vr[q] = vring[r * 256 + (4 * g4 + q) * 16 + n16];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t w0q = ((const uint32_t*)&vr[0])[db >> 1], w1q = ((const uint32_t*)&vr[1])[db >> 1];
      const uint32_t w2q = ((const uint32_t*)&vr[2])[db >> 1], w3q = ((const uint32_t*)&vr[3])[db >> 1];
      const uint32_t sel = (db & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t x01 = __builtin_amdgcn_perm(w1q, w0q, sel), x23 = __builtin_amdgcn_perm(w3q, w2q, sel);
      ds16x4 a;
      a[0] = (short)(x01 & 0xffff);
      a[1] = (short)(x01 >> 16);
      a[2] = (short)(x23 & 0xffff);
      a[3] = (short)(x23 >> 16);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, oacc[db], 0, 0, 0);
    }
  };

  if (ns > 0) issue(0, 0);
  if (ns > 1) issue(1, 1);
  for (int st = 0; st < ns; st += kDecRing) {
#pragma unroll
    for (int u = 0; u < kDecRing; ++u) {
      const int cur = st + u;
      if (cur < ns) {
        if (cur + 2 < ns) issue(cur + 2, (u + 2) % kDecRing);
        dec_wait_vm(min(2, ns - 1 - cur));
        process(cur, u);
      }
    }
  }

  // ---- merge the 4 waves (V rings reused), write the split's partial
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

// One workgroup per (query head, batch): log-sum-exp merge of the splits.
// Split weights are computed once into LDS; each thread then sums a strided
// subset of splits for one float4 of head dims and the subsets are added.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p, DecodeSeqs ds) {
  __shared__ float wgt[1088];
  __shared__ float red[256];
  __shared__ float4 part4[8][32];
  const int b = blockIdx.y, h = blockIdx.x, t = threadIdx.x;
  const int ns = ds.nsplit[b];
  const size_t row0 = ((size_t)b * p.Hq + h) * p.S;
  float mloc = -INFINITY;
  for (int i = t; i < ns; i += 256) mloc = fmaxf(mloc, p.part_m[row0 + i]);
  red[t] = mloc;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (t < k) red[t] = fmaxf(red[t], red[t + k]);
    __syncthreads();
  }
  const float mt = red[0];
  const float mbt = (mt == -INFINITY) ? 0.f : mt;
  __syncthreads();
  float lloc = 0.f;
  for (int i = t; i < ns; i += 256) {
    const float w = __builtin_amdgcn_exp2f(p.part_m[row0 + i] - mbt);
    wgt[i] = w;
    lloc += w * p.part_l[row0 + i];
  }
  red[t] = lloc;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (t < k) red[t] += red[t + k];
    __syncthreads();
  }
  const float lt = red[0];
  const int d4 = t & 31, grp = t >> 5;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int i = grp; i < ns; i += 8) {
    const float4 v = *(const float4*)(p.part_acc + (row0 + i) * kHeadDim + 4 * d4);
    const float w = wgt[i];
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  part4[grp][d4] = acc;
  __syncthreads();
  if (t < 32) {
    float4 a = part4[0][t];
#pragma unroll
    for (int g = 1; g < 8; ++g) {
      a.x += part4[g][t].x;
      a.y += part4[g][t].y;
      a.z += part4[g][t].z;
      a.w += part4[g][t].w;
    }
    const float inv = 1.f / lt;
    uint16_t* o = p.o + ((size_t)b * p.Hq + h) * kHeadDim + 4 * t;
    uint2 w;
    w.x = (uint32_t)df2bf(a.x * inv) | ((uint32_t)df2bf(a.y * inv) << 16);
    w.y = (uint32_t)df2bf(a.z * inv) | ((uint32_t)df2bf(a.w * inv) << 16);
    *(uint2*)o = w;
    if (p.lse && t == 0) p.lse[(size_t)b * p.Hq + h] = (mt + __log2f(lt)) * 0.69314718055994530942f;
  }
}

// ------------------------------------------------------------------ host side
// Keys per split: about 128 splits per sequence, 64..1024 keys each.
static int decode_chunk(long long N) {
  long long c = (N + 127) / 128;
  c = ((c + kDecBlock - 1) / kDecBlock) * kDecBlock;
  if (c < kDecBlock) c = kDecBlock;
  if (c > 1024) c = 1024;
  return (int)c;
}

int decode_splits(long long N) { return (int)((N + decode_chunk(N) - 1) / decode_chunk(N)); }

static int decode_split_bound(long long max_len) {
  const long long a = (max_len + 1023) / 1024 + 1;
  return (int)(a > 129 ? a : 129);
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

int run_decode(bool bifocal, const void* q, const void* kc, const void* vc, void* o, float* lse,
               const int32_t* seqlens, int batch, int cap, int Hq, int Hkv, long long w0,
               long long w_pre, double theta, int mode, float scale, void* ws, size_t ws_bytes,
               hipStream_t stream, std::string& err) {
  auto bad = [&](int code, const std::string& m) { err = m; return code; };
  if (!q || !kc || !vc || !o || !seqlens) return bad(BF_ERR_INVALID_ARG, "null tensor or seqlens pointer");
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
  if (decode_split_bound(max_len) > 1088)
    return bad(BF_ERR_UNSUPPORTED, "decode supports caches of at most 1088 x 1024 keys");
  const DecodeWs wl = decode_ws_layout(batch, max_len, Hq);
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
  dp.mode = mode;
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = batch - b0 < kMaxSeqPerLaunch ? batch - b0 : kMaxSeqPerLaunch;
    DecodeSeqs ds;
    ds.n = nb;
    int max_split = 0;
    for (int i = 0; i < nb; ++i) {
      const long long N = seqlens[b0 + i];
      ds.N[i] = (int)N;
      long long s = 1;
      if (bifocal) s = N / w_pre + (N % w_pre != 0 ? 1 : 0);
      ds.s[i] = (int)(s < 1 ? 1 : s);
      ds.chunk[i] = decode_chunk(N);
      ds.nsplit[i] = decode_splits(N);
      if (ds.nsplit[i] > max_split) max_split = ds.nsplit[i];
    }
    dp.q = (const uint16_t*)q + (size_t)b0 * Hq * kHeadDim;
    dp.kc = (const uint16_t*)kc + (size_t)b0 * Hkv * cap * kHeadDim;
    dp.vc = (const uint16_t*)vc + (size_t)b0 * Hkv * cap * kHeadDim;
    dp.o = (uint16_t*)o + (size_t)b0 * Hq * kHeadDim;
    dp.lse = lse ? lse + (size_t)b0 * Hq : nullptr;
    dp.part_m = (float*)(wsb + wl.m_off) + (size_t)b0 * Hq * dp.S;
    dp.part_l = (float*)(wsb + wl.l_off) + (size_t)b0 * Hq * dp.S;
    dp.part_acc = (float*)(wsb + wl.acc_off) + (size_t)b0 * Hq * dp.S * kHeadDim;
    if (getenv("BIFOCAL_TRACE") && getenv("BIFOCAL_TRACE")[0] == '1')
      fprintf(stderr, "[bifocal] decode %s seqs=%d..%d N0=%d s0=%d splits=%d chunk=%d\n",
              bifocal ? "bifocal" : "plain", b0, b0 + nb - 1, ds.N[0], ds.s[0], ds.nsplit[0], ds.chunk[0]);
    dim3 grid(max_split, Hkv, nb);
    if (bifocal)
      hipLaunchKernelGGL(decode_split_kernel<true>, grid, dim3(256), 0, stream, dp, ds, tt);
    else
      hipLaunchKernelGGL(decode_split_kernel<false>, grid, dim3(256), 0, stream, dp, ds, tt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return bad(BF_ERR_HIP, std::string("decode split launch: ") + hipGetErrorString(e));
    hipLaunchKernelGGL(decode_combine_kernel, dim3(Hq, nb), dim3(256), 0, stream, dp, ds);
    e = hipGetLastError();
    if (e != hipSuccess) return bad(BF_ERR_HIP, std::string("decode combine launch: ") + hipGetErrorString(e));
  }
  return BF_OK;
}

}  // namespace bf
