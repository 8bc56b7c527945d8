// Bifocal RoPE attention, single-token decode over a KV cache on gfx950.
//
// decode_split_kernel: workgroup = (batch b, KV head, split of C keys). The
//   split's keys and values are streamed from HBM once, 64 keys at a time.
//   Keys farther than w0 from the query (position N - 1) get the correction
//   rotation R(theta_m * (phi(j) - j)) in registers before they are staged in
//   LDS, keys inside the window are used as cached [ai-feeds.com summary,
//   "关键模块" item 3: rotation of cached keys; item 1: the w0 window keeps
//   original RoPE]. The query gets the same correction at its own position.
//   Each of the 4 waves scores 16 keys of a block for all G query heads of
//   the KV group (MFMA 16x16x32, queries as columns), keeps one online
//   softmax state per query, and accumulates O^T with MFMA 16x16x16. At the
//   end the waves are merged and the split writes (m, l, acc) partials.
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

template <bool BIFOCAL>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p, DecodeSeqs ds,
                                                           ThetaTable tt) {
  // LDS: K block [64][16 x 16 B] swizzled | V block [64][136] bf16 | Q' and Q'' [2][16][16 x 16 B]
  __shared__ uint4 smem[1024 + (kDecBlock * kDecVRow * 2) / 16 + 2 * kDecMaxG * 16];
  uint4* sK = smem;
  uint16_t* sV = (uint16_t*)(smem + 1024);
  uint4* sQ = smem + 1024 + (kDecBlock * kDecVRow * 2) / 16;

  const int b = blockIdx.z, kvh = blockIdx.y, sp = blockIdx.x;
  if (sp >= ds.nsplit[b]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const long long N = ds.N[b];
  const long long s = ds.s[b];
  const long long w0 = (BIFOCAL && s > 1) ? p.w0 : (1LL << 62);
  const long long far_lim = N - w0;  // keys j < far_lim are far
  const long long k_begin = (long long)sp * ds.chunk[b];
  const long long k_end = min(N, k_begin + ds.chunk[b]);

  // ---- queries: Q' as given, Q'' = R(Delta(N - 1)) Q'; rows >= G are zero
  {
    const int qi = tid >> 4, c = tid & 15;  // 16 rows x 16 chunks
    uint4 v0 = make_uint4(0, 0, 0, 0);
    if (qi < p.G) v0 = *(const uint4*)(p.q + ((size_t)b * p.Hq + kvh * p.G + qi) * kHeadDim + c * 8);
    sQ[qi * 16 + c] = v0;
    sQ[kDecMaxG * 16 + qi * 16 + c] = v0;
  }
  __syncthreads();
  if (BIFOCAL && far_lim > 0) {
    // thread (qi, m): 256 threads cover 4 queries x 64 pairs per pass
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

  float m_run = -INFINITY, l_run = 0.f;
  df32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = df32x4{};

  const uint16_t* kbase = p.kc + ((size_t)b * p.Hkv + kvh) * (size_t)p.cap * kHeadDim;
  const uint16_t* vbase = p.vc + ((size_t)b * p.Hkv + kvh) * (size_t)p.cap * kHeadDim;
  const int kk = tid >> 2, q4 = tid & 3;  // staging: key row kk, chunks q4 + 4i

  for (long long kb = k_begin; kb < k_end; kb += kDecBlock) {
    // ---- stage: load this thread's 4 key chunks and 4 value chunks
    const long long j = kb + kk;
    const bool valid = j < k_end;
    uint4 kv[4], vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = q4 + 4 * i;
      kv[i] = valid ? *(const uint4*)(kbase + (size_t)j * kHeadDim + c * 8) : make_uint4(0, 0, 0, 0);
      vv[i] = valid ? *(const uint4*)(vbase + (size_t)j * kHeadDim + c * 8) : make_uint4(0, 0, 0, 0);
    }
    if (BIFOCAL && valid && j < far_lim) {
      // chunk pairs (q4, q4 + 8) and (q4 + 4, q4 + 12) hold rotary pairs (m, m + 64)
      const long long num = dcorr_num(j, s, p.mode);
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        uint32_t* lo = (uint32_t*)&kv[hp];
        uint32_t* hi = (uint32_t*)&kv[hp + 2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int m0 = 8 * (q4 + 4 * hp) + 2 * w;
          float c0, s0, c1, s1;
          corr_cos_sin(tt.th[m0], num, s, c0, s0);
          corr_cos_sin(tt.th[m0 + 1], num, s, c1, s1);
          const float a0 = __uint_as_float(lo[w] << 16), a1 = __uint_as_float(lo[w] & 0xffff0000u);
          const float b0 = __uint_as_float(hi[w] << 16), b1 = __uint_as_float(hi[w] & 0xffff0000u);
          const float ra0 = a0 * c0 - b0 * s0, rb0 = b0 * c0 + a0 * s0;
          const float ra1 = a1 * c1 - b1 * s1, rb1 = b1 * c1 + a1 * s1;
          lo[w] = (uint32_t)df2bf(ra0) | ((uint32_t)df2bf(ra1) << 16);
          hi[w] = (uint32_t)df2bf(rb0) | ((uint32_t)df2bf(rb1) << 16);
        }
      }
    }
    __syncthreads();  // previous block's LDS reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = q4 + 4 * i;
      sK[kk * 16 + (c ^ (kk & 15))] = kv[i];
      *(uint4*)(sV + kk * kDecVRow + c * 8) = vv[i];
    }
    __syncthreads();

    // ---- wave: 16 keys kb + 16 wave .. +15
    const long long jw = kb + 16 * wave;
    if (jw < k_end) {
      const int krow = 16 * wave + n16;  // A operand row of this lane
      df32x4 S = df32x4{};
      const bool any_far = BIFOCAL && jw < far_lim;
      const bool any_loc = !BIFOCAL || jw + 15 >= far_lim;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const dbf16x8 a = __builtin_bit_cast(dbf16x8, sK[krow * 16 + ((4 * t + g4) ^ (krow & 15))]);
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, any_far ? qf2[t] : qf[t], S, 0, 0, 0);
      }
      if (any_far && any_loc) {  // block straddles the window edge: local keys use Q'
        df32x4 Sl = df32x4{};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const dbf16x8 a = __builtin_bit_cast(dbf16x8, sK[krow * 16 + ((4 * t + g4) ^ (krow & 15))]);
          Sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[t], Sl, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (jw + 4 * g4 + r >= far_lim) S[r] = Sl[r];
      }
      // C layout: lane (query n16, g4) holds keys jw + 4 g4 + r
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (jw + 4 * g4 + r >= k_end) S[r] = -INFINITY;
      float mx = fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m_run, mx * p.scale_log2);
      const float mbase = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mbase);
      m_run = mnew;
      float rs = 0.f;
      ds16x4 pb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(S[r], p.scale_log2, -mbase));
        rs += e;
        pb[r] = (short)df2bf(e);
      }
      rs += __shfl_xor(rs, 16);
      rs += __shfl_xor(rs, 32);
      l_run = l_run * alpha + rs;
      // O^T += V^T P^T: A = V^T rows d = 16 db + n16, keys 16 wave + 4 g4 + r
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 16 * db + n16;
        ds16x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = (short)sV[(16 * wave + 4 * g4 + r) * kDecVRow + d];
        oacc[db] *= alpha;
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- merge the 4 waves (LDS reused), write the split's partial
  __syncthreads();
  float* mw = (float*)smem;                 // [4][16]
  float* lw = mw + 4 * kDecMaxG;            // [4][16]
  float* ow = lw + 4 * kDecMaxG;            // [4][16][128]
  if (g4 == 0) {
    mw[wave * kDecMaxG + n16] = m_run;
    lw[wave * kDecMaxG + n16] = l_run;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      ow[(wave * kDecMaxG + n16) * kHeadDim + 16 * db + 4 * g4 + r] = oacc[db][r];
  __syncthreads();
  for (int e = tid; e < p.G * kHeadDim; e += 256) {
    const int qi = e >> 7, d = e & 127;
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mt = fmaxf(mt, mw[w * kDecMaxG + qi]);
    const float mb = (mt == -INFINITY) ? 0.f : mt;
    float acc = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(mw[w * kDecMaxG + qi] - mb);
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

// One workgroup per (query head, batch): LSE merge of the splits.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeParams p, DecodeSeqs ds) {
  const int b = blockIdx.y, h = blockIdx.x, d = threadIdx.x;
  const int ns = ds.nsplit[b];
  const size_t row0 = ((size_t)b * p.Hq + h) * p.S;
  float mt = -INFINITY;
  for (int i = 0; i < ns; ++i) mt = fmaxf(mt, p.part_m[row0 + i]);
  const float mb = (mt == -INFINITY) ? 0.f : mt;
  float acc = 0.f, lt = 0.f;
  for (int i = 0; i < ns; ++i) {
    const float f = __builtin_amdgcn_exp2f(p.part_m[row0 + i] - mb);
    acc += f * p.part_acc[(row0 + i) * kHeadDim + d];
    lt += f * p.part_l[row0 + i];
  }
  p.o[((size_t)b * p.Hq + h) * kHeadDim + d] = df2bf(acc / lt);
  if (p.lse && d == 0) p.lse[(size_t)b * p.Hq + h] = (mt + __log2f(lt)) * 0.69314718055994530942f;
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
    hipLaunchKernelGGL(decode_combine_kernel, dim3(Hq, nb), dim3(128), 0, stream, dp, ds);
    e = hipGetLastError();
    if (e != hipSuccess) return bad(BF_ERR_HIP, std::string("decode combine launch: ") + hipGetErrorString(e));
  }
  return BF_OK;
}

}  // namespace bf
