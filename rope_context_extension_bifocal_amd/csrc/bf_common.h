// Shared between the HIP kernels and the host-side launch code of libbifocal.
// Plain structs passed by value as kernel arguments (well under the 4 KiB
// kernel-argument limit), so a launch needs no host-to-device copy.
#pragma once
#include <stdint.h>

namespace bf {

constexpr int kHeadDim = 128;     // the only head_dim the kernels are built for
constexpr int kPairs = kHeadDim / 2;
constexpr int kMaxSeqPerLaunch = 64;
constexpr int kMaxKeySplits = 8;  // key splits of a chunk launch (prefill_bf16_kernel)
constexpr int kKeyTile = 64;      // keys per K/V tile (prefill) and V^T padding unit
constexpr int kWaveRowsBf16 = 32; // query positions per wave, bf16 prefill
constexpr int kWaveRowsF32 = 32;  // query positions per wave, fp32 prefill
constexpr int kWavesPerGroupBf16 = 4;  // waves per bf16 prefill workgroup (256 lanes)
constexpr int kWavesPerGroupF32 = 4;   // waves per fp32 prefill workgroup (256 lanes)

// Per-launch description of up to kMaxSeqPerLaunch sequences. Queries are
// packed along the T axis (q, o, lse, q''); keys are read from a K / V tensor
// whose row of key j, KV head h, sequence b is h * k_hstride + kbase[b] + j
// (a packed [Hkv][T][D] tensor: k_hstride = T, kbase = cu; a KV cache
// [B][Hkv][cap][D]: k_hstride = cap, kbase = b * Hkv * cap). A one-shot
// prefill has qpos = 0 and keys = queries; a chunk of queries against a cache
// has its first query at position qpos = N - Lq.
struct SeqTable {
  int n;                              // sequences in this launch
  int cu[kMaxSeqPerLaunch + 1];       // query token offsets into the packed T axis
  int kcu[kMaxSeqPerLaunch + 1];      // key offsets into the packed k'' axis (Tk); keys of b: kcu[b+1]-kcu[b]
  int vt_off[kMaxSeqPerLaunch + 1];   // 64-aligned offsets into the padded V^T axis
  int vt_t0[kMaxSeqPerLaunch];        // first key tile with a V^T copy: 0, or for band-only chunks
                                      // the first tile any query's window reaches
  int qpos[kMaxSeqPerLaunch];         // position of the sequence's first query row
  int order[kMaxSeqPerLaunch];        // sequences in work order (most scored pairs first)
  int ioff[kMaxSeqPerLaunch + 1];     // first work-item rank of order[i]; ioff[n] = all row blocks
  long long kbase[kMaxSeqPerLaunch];  // K / V row offset of the sequence's key 0
  int s[kMaxSeqPerLaunch];            // s(L_b) (1 = no far branch)
  int nrb[kMaxSeqPerLaunch];          // query row blocks of the sequence
};

// theta_m = rope_theta^(-2m/D) for the 64 rotary pairs, fp64.
struct ThetaTable {
  double th[kPairs];
};

struct PrefillParams {
  const void* q;    // [Hq][T][D]   original-RoPE queries
  const void* k;    // original-RoPE keys, rows h * k_hstride + kbase[b] + j
  const void* q2;   // [Hq][T][D]   corrected queries (far branch), workspace
  const void* k2;   // [Hkv][Tk][D] corrected keys (far branch), workspace
  const void* vt;   // [Hkv][D][Tpad] values, transposed and 64-padded per sequence
  void* o;          // [Hq][T][D]
  float* lse;       // [Hq][T] or null
  long long w0;     // local window (ignored by the plain engine)
  float scale_log2; // softmax_scale * log2(e)
  long long k_hstride;  // K rows between KV heads
  long long k_rows;     // rows of the whole K tensor (range limit of the loads)
  long long k2_rows;    // rows of the k'' tensor (range limit): Hkv * Tk, or a store's
  long long vt_rows;    // head-dim rows x 64 keys of V^T (range limit): Hkv * Tpad, or a store's
  int T, Tk, Tpad;
  int Hq, Hkv, G;
  int hpw;          // query heads per workgroup
  int n_hsub;       // workgroups per (KV head, row block) = G / hpw
  int P_wg;         // query positions per workgroup
  int total_items;  // row blocks over the launch's sequences
  // key splits (bf16 only): nks > 1 splits each work item's tile visits into
  // nks parts; part s writes its normalised O and log2-sum-exp to
  // part_o [nks][Hq][T][D] and part_lse [nks][Hq][T] instead of o / lse
  int nks;
  float* part_o;
  float* part_lse;
  // null: workgroup w runs work item w. Otherwise 8 counters, zeroed before
  // the launch, and fewer workgroups than items: each workgroup claims the
  // next item of its XCD's queue (the items whose id is the XCD's index mod
  // 8, in id order) and, once that queue is empty, of the other queues, until
  // all n_items are taken
  int* item_ctr;
  int n_items;
};

// A paged K / V source: pages [num_pages][Hkv][page][D], key j of sequence
// b in page block_table[b * max_pages + j / page] (entries clamped to the pool).
struct PagedKV {
  const int* block_table;  // null: the K / V layout of SeqTable (h * k_hstride + kbase[b] + j)
  int page_log2, max_pages, num_pages;
};

struct PrepParams {
  const void* q;  // [Hq][T][D]
  const void* k;  // rows h * k_hstride + kbase[b] + j, or pages (pk)
  void* q2;       // [Hq][T][D]
  void* k2;       // [Hkv][Tk][D], or with k2_cap > 0 a store [n][Hkv][k2_cap][D]
  void* kcopy;    // [Hkv][Tk][D] packed copy of the keys (paged source only), else null
  PagedKV pk;
  long long k_hstride;
  int T, Tk, Hq, Hkv;
  int long_mode;  // 0 = FI, 1 = PA
  int shift;      // 1: queries get the band-edge continuity shift w0 - phi(w0)
  long long w0;
  // k2_cap > 0: k'' of key j of sequence b (of the launch) goes to row
  // (b * Hkv + h) * k2_cap + j of the store, the packed key axis (kcu) holds
  // only keys kfirst[b] .. N_b - 1 (all of them copied when kcopy is set), and
  // only keys from krot[b] on are rotated (the store holds the ones below);
  // k2_cap = 0: the packed layout, kfirst 0
  int k2_cap;
  int kfirst[kMaxSeqPerLaunch];
  int krot[kMaxSeqPerLaunch];
};

struct VtParams {
  const void* v;  // rows h * k_hstride + kbase[b] + j (the layout of K), or pages (pk)
  void* vt;       // [Hkv][D][Tpad], or with store_tiles > 0 a store [n][Hkv][store_tiles][D][64]
  PagedKV pk;
  long long k_hstride;
  int Tpad, Hkv;
  int store_tiles;  // > 0: tile t of sequence b (of the launch), KV head h, goes to store
                    // tile (b * Hkv + h) * store_tiles + t
};

// Kernel arguments stay within 4 KiB.
static_assert(sizeof(PrepParams) + sizeof(SeqTable) + sizeof(ThetaTable) <= 4096, "prep arguments");
static_assert(sizeof(PrefillParams) + sizeof(SeqTable) <= 4096, "prefill arguments");

// Positions whose correction angles a test hook reports (at most kProbeMax).
constexpr int kProbeMax = 128;
struct AngleProbe {
  int n;
  int mode;   // 0 = FI, 1 = PA
  int shift;  // band-edge continuity shift (queries)
  int query;  // prefill: 1 = query angles, 0 = key angles
  long long w0;
  long long N;               // decode: keys of the call (s = s(N) for key angles)
  long long pos[kProbeMax];  // positions
  long long s[kProbeMax];    // s of each position's call
};

}  // namespace bf
