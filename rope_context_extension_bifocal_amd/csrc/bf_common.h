// Shared between the HIP kernels and the host-side launch code of libbifocal.
// Plain structs passed by value as kernel arguments (well under the 4 KiB
// kernel-argument limit), so a launch needs no host-to-device copy.
#pragma once
#include <stdint.h>

namespace bf {

constexpr int kHeadDim = 128;     // the only head_dim the kernels are built for
constexpr int kPairs = kHeadDim / 2;
constexpr int kMaxSeqPerLaunch = 64;
constexpr int kKeyTile = 64;      // keys per K/V tile (prefill) and V^T padding unit
constexpr int kWaveRowsBf16 = 32; // query positions per wave, bf16 prefill
constexpr int kWaveRowsF32 = 32;  // query positions per wave, fp32 prefill
constexpr int kWavesPerGroupBf16 = 4;  // waves per bf16 prefill workgroup (256 lanes)
constexpr int kWavesPerGroupF32 = 4;   // waves per fp32 prefill workgroup (256 lanes)

// Per-launch description of up to kMaxSeqPerLaunch packed sequences.
struct SeqTable {
  int n;                              // sequences in this launch
  int cu[kMaxSeqPerLaunch + 1];       // token offsets into the packed T axis
  int vt_off[kMaxSeqPerLaunch + 1];   // 64-aligned offsets into the padded V^T axis
  int s[kMaxSeqPerLaunch];            // s(L_b) (1 = no far branch)
  int nrb[kMaxSeqPerLaunch];          // query row blocks of the sequence
};

// theta_m = rope_theta^(-2m/D) for the 64 rotary pairs, fp64.
struct ThetaTable {
  double th[kPairs];
};

struct PrefillParams {
  const void* q;    // [Hq][T][D]   original-RoPE queries
  const void* k;    // [Hkv][T][D]  original-RoPE keys
  const void* q2;   // [Hq][T][D]   corrected queries (far branch), workspace
  const void* k2;   // [Hkv][T][D]  corrected keys (far branch), workspace
  const void* vt;   // [Hkv][D][Tpad] values, transposed and 64-padded per sequence
  void* o;          // [Hq][T][D]
  float* lse;       // [Hq][T] or null
  long long w0;     // local window (ignored by the plain engine)
  float scale_log2; // softmax_scale * log2(e)
  int T, Tpad;
  int Hq, Hkv, G;
  int hpw;          // query heads per workgroup
  int n_hsub;       // workgroups per (KV head, row block) = G / hpw
  int P_wg;         // query positions per workgroup
  int total_items;  // row blocks over all sequences of the launch
  int max_nrb;
};

struct PrepParams {
  const void* q;  // [Hq][T][D]
  const void* k;  // [Hkv][T][D]
  void* q2;       // [Hq][T][D]
  void* k2;       // [Hkv][T][D]
  int T, Hq, Hkv;
  int long_mode;  // 0 = FI, 1 = PA
  int shift;      // 1: queries get the band-edge continuity shift w0 - phi(w0)
  long long w0;
};

struct VtParams {
  const void* v;  // [Hkv][T][D]
  void* vt;       // [Hkv][D][Tpad]
  int T, Tpad, Hkv;
};

}  // namespace bf
