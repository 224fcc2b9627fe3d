// Launch interface between the host sequencing code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moba_plan.h"

namespace moba {

// Gate over one query chunk: positions [t0, t0 + cnt) of batch entry bb.
struct GateArgs {
  const void* q;
  const float* mu;       // [batch, hkv, n, D] block means (mean gate)
  const float* lohi;     // [batch, hkv, n, 2, D] block key min / max (min/max gate)
  const uint16_t* mu3;   // the bf16 path's MFMA tile images of the summaries, or null
  int32_t minmax;        // 1: the min/max gate, 0: the mean gate
  int32_t* sel;          // row (h, t) at sel + h * sel_stride_h + (t - sel_pos_base) * topk
  int64_t sel_stride_h;
  int64_t sel_pos_base;
  int32_t* hist;         // [hkv, gate_wg, n] rows per block per work-group, or null
  int64_t seqlen, n, t0, cnt, gate_wg;
  int32_t hq, hkv, block, topk, kp, causal, g, gate_t, bb;
};

// Row lists of one chunk: list (hk, i) holds the (row, slot) pairs whose row
// chose block i as a non-own block.
struct DispatchArgs {
  const int32_t* sel;    // as GateArgs
  int64_t sel_stride_h;
  int64_t sel_pos_base;
  int32_t* hist;         // in: per-WG counts; out: per-WG start inside the list
  int32_t* count;        // [hkv * n]
  int32_t* listoff;      // [hkv * n + 1]
  int32_t* tiles;        // [0] = number of tiles, [8 + 2 t] = list id, [9 + 2 t] = first entry
  int32_t* entries;      // local_row * kp + slot
  int64_t n, t0, cnt, gate_wg;
  int32_t hq, hkv, block, topk, kp, causal, g, gate_t, tile_rows;
};

// Attention over one list tile (non-own blocks, no mask).
struct PastArgs {
  const void* q;         // whole q, [batch, seqlen, hq, D]
  const void* k;
  const void* v;
  const int32_t* tiles;
  const int32_t* count;
  const int32_t* listoff;
  const int32_t* entries;
  uint16_t* part_o;      // normalised partial outputs, bf16 (layout in attn_bf16.hip)
  float* part_lse;       // their log2-domain log-sum-exp of the scaled logits
  int64_t part_rows;     // row capacity of one slot plane (chunk positions x hq)
  const uint16_t* kimg;  // K slice images [batch, hkv, seqlen / 64, 64 x 128], or null
  const uint16_t* vimg;  // V^T slice images, same shape
  int64_t seqlen, n, t0;
  int32_t hq, hkv, block, kp, g, bb, max_tiles, tile_rows;
  float scale_log2;      // log2(e) / sqrt(D)
};

// Own block (causal) + merge of the partials, writes out.
struct OwnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const uint16_t* part_o;  // partial outputs written by the past-block kernel
  const float* part_lse;
  int64_t part_rows;
  const uint16_t* kimg;    // K / V^T slice images, or null
  const uint16_t* vimg;
  float* lse;              // [batch, hq, seqlen] row log-sum-exp (natural log), or null
  int64_t seqlen, n, t0, cnt;
  int32_t hq, hkv, block, kp, g, own_t, bb, causal;
  int32_t rows;            // 128-row tiles read from K and V rows (block a multiple of 32)
  float scale_log2;
};

// fp32 path: one wave per query row, reading the row's selection directly.
struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* out;
  const int32_t* sel;
  int64_t sel_stride_h;
  int64_t sel_pos_base;
  int64_t seqlen, t0, cnt;
  float* lse;            // [batch, hq, seqlen] row log-sum-exp (natural log), or null
  int32_t hq, hkv, d, block, topk, causal, g, bb;
  float scale_log2;
};

// Decode (one new query per sequence against its cache); the limits are in
// moba_plan.h.
struct DecodeArgs {
  const void* q;           // [batch, hq, d]
  const void* k;           // [batch, lmax, hkv, d]
  const void* v;
  float* mu;               // [batch, hkv, nmax, d] means of the complete blocks (the merge
                           // writes the mean of an own block the new token completes)
  const int32_t* lens;     // [batch] cached positions, the new token included
  int32_t* sel;            // [batch, hq, topk]
  float* sc;               // [batch, hq, nmax] gate scores
  int32_t* uni;            // [batch * hkv, U] the group's chosen blocks, ascending
  int32_t* uslot;          // [batch * hkv, U, g] slot of a union entry in each head's row, or -1
  int32_t* ucount;         // [batch * hkv] union sizes
  float* po;               // [batch, hq, topk, nchunk, d] unnormalised partial outputs
  float* pml;              // [batch, hq, topk, nchunk, 2] partial max (base 2) and sum
  float* ksum;             // [batch * hkv, nchunk, d] key column sums of a completed own block
  void* out;               // [batch, hq, d]
  int64_t batch, lmax, nmax;
  int32_t hq, hkv, g, d, block, topk, U, nchunk;
  float scale_log2;
};
// stage 0: gate + top-k + union; 1: chunk attention; 2: merge
int launch_decode_stage(const DecodeArgs& a, int dtype, int stage, hipStream_t stream);
// Block means of every complete block of the cache.
int launch_decode_means(const void* k, const int32_t* lens, float* mu, int dtype, int64_t batch, int64_t lmax,
                        int64_t nmax, int hkv, int d, int block, hipStream_t stream);

// Backward (bf16, head dim 128).  Rows are (batch, position, query head),
// row index (b * seqlen + t) * hq + h.
struct BwdArgs {
  const void* q;           // [batch, seqlen, hq, 128] bf16
  const void* k;           // [batch, seqlen, hkv, 128]
  const void* v;
  const void* dout;        // like q
  const float* lse2;       // [rows] row log-sum-exp of the scaled logits, base 2
  const float* delta;      // [rows] dout . out
  // query-chunk dispatch (dq): as DispatchArgs, 256-row tiles
  const int32_t* tiles;
  const int32_t* count;
  const int32_t* listoff;
  const int32_t* entries;
  // whole-sequence lists (dk, dv)
  const int32_t* count_f;
  const int32_t* listoff_f;
  const int32_t* entries_f;
  const uint16_t* kimg;    // K in the K slice-image layout
  const uint16_t* vkimg;   // V in the K slice-image layout
  const uint16_t* kvimg;   // K in the V^T slice-image layout
  float* dq_part;          // [chunk rows, kps, 128] per (row, slot) dq contributions
  void* dq;                // [batch, seqlen, hq, 128] bf16
  void* dk;                // [batch, seqlen, hkv, 128] bf16
  void* dv;
  int64_t seqlen, n, t0, cnt;
  int32_t hq, hkv, block, kp, kps, g, bb, causal;
  float scale_log2;        // log2(e) / sqrt(D)
  float scale;             // 1 / sqrt(D)
};
// delta = rowsum(dout * out) and lse2 = lse * log2(e), all rows.
int launch_bwd_prep(const void* out, const void* dout, const float* lse, float* lse2, float* delta, int64_t batch,
                    int64_t seqlen, int hq, hipStream_t stream);
// dq contributions of one query chunk: the chunk's list tiles (max_tiles
// work-groups) and, causal, its own blocks; then their sum into dq.
int launch_bwd_dq(const BwdArgs& a, int64_t max_tiles, hipStream_t stream);
// dk and dv of all keys of batch entry a.bb.
int launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
// Per gate-work-group list counts from a given selection (the gate's side
// output when the gate has not run), then the dispatch.
int launch_dispatch_from_sel(const DispatchArgs& a, hipStream_t stream);

// K and V^T images of all 64-key slices (bf16 path, seqlen % 64 == 0).
int launch_kv_image(const void* k, const void* v, int64_t batch, int64_t seqlen, int hkv, uint16_t* kimg,
                    uint16_t* vimg, hipStream_t stream);

int launch_meanpool(const void* k, int dtype, int64_t batch, int64_t seqlen, int hkv, int d, int block,
                    float* mu, hipStream_t stream);
int launch_gate(const GateArgs& a, int dtype, int d, hipStream_t stream);
// Block means split into three bf16 parts, as the gate's MFMA tile images.
int launch_mu_split(const float* mu, int64_t batch, int64_t n, int hkv, uint16_t* mu3, hipStream_t stream);
// Block key max and min (bf16 values) as the min/max gate's MFMA tile images.
int launch_mm_split(const float* lohi, int64_t batch, int64_t n, int hkv, uint16_t* mu3, hipStream_t stream);
// Element-wise min / max of each block's keys: lohi [batch, hkv, n, 2, d].
int launch_minmaxpool(const void* k, int dtype, int64_t batch, int64_t seqlen, int hkv, int d, int block,
                      float* lohi, hipStream_t stream);
int launch_dispatch(const DispatchArgs& a, hipStream_t stream);
int launch_attn_past(const PastArgs& a, hipStream_t stream);
int launch_attn_own(const OwnArgs& a, hipStream_t stream);
int launch_attn_f32(const F32Args& a, hipStream_t stream);

}  // namespace moba
