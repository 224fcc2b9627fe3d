// Host-side validation and workspace planning (no HIP calls).
#include "moba_plan.h"

#include <algorithm>

#include "../../include/moba.h"

namespace moba {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int make_plan(const Shape& s, Plan* p, int64_t max_chunk_blocks, bool allow_image) {
  if (!p) return MOBA_ERR_NULL;
  if (s.dtype != MOBA_DTYPE_F32 && s.dtype != MOBA_DTYPE_BF16) return MOBA_ERR_DTYPE;
  if (s.batch < 1 || s.seqlen < 1 || s.hq < 1 || s.hkv < 1 || s.block < 1 || s.d < 1)
    return MOBA_ERR_SHAPE;
  if (s.dtype == MOBA_DTYPE_BF16 && s.d != 128) return MOBA_ERR_HEAD_DIM;
  if (s.dtype == MOBA_DTYPE_F32 && s.d != 64 && s.d != 128) return MOBA_ERR_HEAD_DIM;
  // no padding is defined for a ragged last block: reject it
  if (s.seqlen % s.block != 0) return MOBA_ERR_SEQ_NOT_DIVISIBLE;
  if (s.hq % s.hkv != 0) return MOBA_ERR_GQA;
  if (s.hq / s.hkv > kMaxGroup) return MOBA_ERR_GQA;
  if (s.topk < 1) return MOBA_ERR_TOPK;

  Plan q{};
  q.s = s;
  q.n = s.seqlen / s.block;
  // grid z carries the batch
  if (s.batch > 65535) return MOBA_ERR_SHAPE;
  q.keff = (int32_t)std::min<int64_t>(s.topk, q.n);
  q.kp = s.causal ? q.keff - 1 : q.keff;
  q.g = s.hq / s.hkv;
  // candidates the gate ranks: past blocks (at most n-1) or all n blocks
  const int64_t cand = s.causal ? q.n - 1 : q.n;
  q.selective = q.kp < cand;

  // index arithmetic bounds: the rows of one batch entry (positions x heads)
  // and row * slot products stay in int32 range; tested by division, before
  // any product of the sizes is formed
  if (s.seqlen > (int64_t(1) << 31) / s.hq) return MOBA_ERR_SHAPE;

  q.gate_t = std::max(1, kGateRows / q.g);

  // per (row, past block) pair: the normalised partial o in bf16 plus its lse in fp32
  const uint64_t per_block_partial =
      (uint64_t)s.block * s.hq * (uint64_t)std::max(q.kp, 0) * (uint64_t)(s.d * 2 + 4);
  if (q.kp == 0) {
    q.chunk_blocks = q.n;
  } else {
    q.chunk_blocks = (int64_t)std::max<uint64_t>(1, kPartialCapBytes / per_block_partial);
    q.chunk_blocks = std::min<int64_t>(q.chunk_blocks, q.n);
  }
  {
    // the count table: KV heads x blocks x ceil(chunk positions / gate_t)
    // int32 entries, kept within kHistCapBytes (one block per chunk at least)
    const uint64_t per_wg = (uint64_t)s.hkv * (uint64_t)q.n * sizeof(int32_t);
    const uint64_t max_wg = kHistCapBytes / per_wg;
    const int64_t cb = (int64_t)(max_wg * (uint64_t)q.gate_t / (uint64_t)s.block);
    q.chunk_blocks = std::max<int64_t>(1, std::min<int64_t>(q.chunk_blocks, cb));
  }
  if (max_chunk_blocks < 0) return MOBA_ERR_SHAPE;
  if (max_chunk_blocks > 0) q.chunk_blocks = std::min<int64_t>(q.chunk_blocks, max_chunk_blocks);
  const int64_t chunk_pos = q.chunk_blocks * s.block;
  q.gate_wg = (chunk_pos + q.gate_t - 1) / q.gate_t;
  q.max_pairs = chunk_pos * s.hq * (int64_t)q.kp;
  if (q.max_pairs >= (int64_t(1) << 31)) return MOBA_ERR_SHAPE;
  const int64_t lists = (int64_t)s.hkv * q.n;
  // long lists: 384-row tiles over the K/V slice images (bf16, whole slices),
  // else 256; short lists: 128
  q.tile_rows = (q.max_pairs / lists >= kLargeTileMinRows) ? kTileRowsLarge : kTileRowsSmall;
  if (allow_image && q.tile_rows == kTileRowsLarge && s.dtype == MOBA_DTYPE_BF16 && s.block % kSliceKeys == 0)
    q.tile_rows = kTileRowsImage;
  q.max_tiles = (q.max_pairs + q.tile_rows - 1) / q.tile_rows + lists;
  q.max_tiles = (q.max_tiles + 7) / 8 * 8;

  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  q.off_mu = take((size_t)s.batch * s.hkv * q.n * s.d * sizeof(float));
  q.off_sel = take((size_t)s.hq * chunk_pos * s.topk * sizeof(int32_t));
  q.off_hist = take((size_t)s.hkv * q.gate_wg * q.n * sizeof(int32_t));
  q.off_count = take((size_t)lists * sizeof(int32_t));
  q.off_listoff = take((size_t)(lists + 1) * sizeof(int32_t));
  q.off_tiles = take((size_t)(2 * q.max_tiles + 8) * sizeof(int32_t));
  q.off_entries = take((size_t)std::max<int64_t>(q.max_pairs, 1) * sizeof(int32_t));
  q.off_part_o = take((size_t)std::max<int64_t>(q.max_pairs, 1) * s.d * sizeof(uint16_t));
  q.off_part_lse = take((size_t)std::max<int64_t>(q.max_pairs, 1) * sizeof(float));
  // K and V^T slice images for the 384-row past-block tiles:
  // [batch, hkv, seqlen / 64, 64 x 128] bf16 each, as large as K and V
  // (and for the own-block kernel alone when no past block is chosen and the
  // blocks are long, e.g. block_size = seqlen: dense causal attention)
  q.kv_image = allow_image && s.dtype == MOBA_DTYPE_BF16 && s.block % kSliceKeys == 0 &&
               (q.kp > 0 ? q.tile_rows == kTileRowsImage : s.block >= kOwnImageMinBlock);
  // own-block tiles: 128 rows from K and V rows in 32-key slices (three
  // work-groups per CU) when the block allows it; where the slice images
  // exist, only with past blocks and blocks of at least kOwnRowsMinBlock
  // keys (dense attention and short blocks run faster in 256-row tiles from
  // the images)
  q.own_rows = s.dtype == MOBA_DTYPE_BF16 && s.block % kRowSliceKeys == 0 &&
               (!q.kv_image || (q.kp > 0 && s.block >= kOwnRowsMinBlock));
  q.own_t = std::max(1, (q.own_rows ? kOwnRowsSmall : kOwnRows) / q.g);
  const size_t img = q.kv_image ? (size_t)s.batch * s.hkv * s.seqlen * s.d * sizeof(uint16_t) : 0;
  q.off_kimg = take(img);
  q.off_vimg = take(img);
  // bf16 gate: block means split into three bf16 parts, per tile of 32 blocks
  const size_t mu3 = s.dtype == MOBA_DTYPE_BF16 && q.selective
                         ? (size_t)s.batch * s.hkv * ((q.n + kGateTile - 1) / kGateTile) * kGateTile * 3 * s.d * 2
                         : 0;
  q.off_mu3 = take(mu3);
  // min/max gate: the element-wise key min and max per block, fp32
  q.off_lohi = take((size_t)s.batch * s.hkv * q.n * 2 * s.d * sizeof(float));
  q.total = off;
  *p = q;
  return MOBA_OK;
}

// The largest chunk (at most the default one) whose workspace fits, or 0.
static int64_t largest_fitting_chunk(const Shape& s, size_t ws_bytes, int64_t hi, bool allow_image, Plan* best) {
  Plan cand{};
  if (make_plan(s, &cand, 1, allow_image) != MOBA_OK || cand.total > ws_bytes) return 0;
  *best = cand;
  int64_t lo = 1;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (make_plan(s, &cand, mid, allow_image) == MOBA_OK && cand.total <= ws_bytes) {
      lo = mid;
      *best = cand;
    } else {
      hi = mid - 1;
    }
  }
  return lo;
}

int plan_for_workspace(const Shape& s, size_t ws_bytes, Plan* p) {
  Plan def{};
  const int st = make_plan(s, &def);
  if (st != MOBA_OK) return st;
  if (def.total <= ws_bytes) {
    *p = def;
    return MOBA_OK;
  }
  // the workspace grows with the chunk: the largest chunk that fits, with
  // the slice images if any chunk fits with them
  Plan best{};
  if (largest_fitting_chunk(s, ws_bytes, def.chunk_blocks, true, &best) > 0 ||
      largest_fitting_chunk(s, ws_bytes, def.chunk_blocks, false, &best) > 0) {
    *p = best;
    return MOBA_OK;
  }
  return MOBA_ERR_WORKSPACE;
}

// Decode: sizes, limits and the workspace carve-up.
int make_decode_plan(int64_t batch, int64_t lmax, int32_t hq, int32_t hkv, int32_t d, int32_t dtype, int32_t block,
                     int32_t topk, DecodePlan* p) {
  if (dtype != MOBA_DTYPE_F32 && dtype != MOBA_DTYPE_BF16) return MOBA_ERR_DTYPE;
  if (batch < 1 || lmax < 1 || hq < 1 || hkv < 1 || block < 1 || d < 1) return MOBA_ERR_SHAPE;
  if (dtype == MOBA_DTYPE_BF16 && d != 128) return MOBA_ERR_HEAD_DIM;
  if (dtype == MOBA_DTYPE_F32 && d != 64 && d != 128) return MOBA_ERR_HEAD_DIM;
  if (hq % hkv != 0 || hq / hkv > kDecodeMaxGroup) return MOBA_ERR_GQA;
  if (topk < 1 || topk > kDecodeMaxTopk) return MOBA_ERR_TOPK;
  if (lmax % block != 0) return MOBA_ERR_SEQ_NOT_DIVISIBLE;
  DecodePlan q{};
  q.nmax = lmax / block;
  q.g = hq / hkv;
  q.U = q.g * topk;
  q.nchunk = (block + kDecodeChunk - 1) / kDecodeChunk;
  // grid limits: (batch * hkv, nchunk, U), (hkv, batch), (hq, batch)
  if (q.nmax > kDecodeMaxBlocks || batch > 65535 || q.nchunk > 65535 || batch * hkv > (int64_t(1) << 31) - 1 ||
      lmax > (int64_t(1) << 31) - 1)
    return MOBA_ERR_SHAPE;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const size_t rows = (size_t)batch * hq;
  q.off_sc = take(rows * q.nmax * sizeof(float));
  q.off_uni = take((size_t)batch * hkv * q.U * sizeof(int32_t));
  q.off_uslot = take((size_t)batch * hkv * q.U * q.g * sizeof(int32_t));
  q.off_ucount = take((size_t)batch * hkv * sizeof(int32_t));
  q.off_sel = take(rows * topk * sizeof(int32_t));
  q.off_po = take(rows * topk * q.nchunk * (size_t)d * sizeof(float));
  q.off_pml = take(rows * topk * q.nchunk * 2 * sizeof(float));
  q.off_ksum = take((size_t)batch * hkv * q.nchunk * (size_t)d * sizeof(float));
  q.total = off;
  *p = q;
  return MOBA_OK;
}

int make_bwd_plan(const Shape& s, BwdPlan* out) {
  BwdPlan b{};
  const int st = make_plan(s, &b.p);
  if (st != MOBA_OK) return st;
  if (s.dtype != MOBA_DTYPE_BF16) return MOBA_ERR_DTYPE;  // the backward runs on bf16 MFMA
  if (s.block % 64 != 0) return MOBA_ERR_SHAPE;            // whole 64-key slices
  const Plan& p = b.p;
  b.kps = p.kp + (s.causal ? 1 : 0);
  const int64_t S = s.seqlen, rows = s.batch * S * s.hq, lists = (int64_t)s.hkv * p.n;
  // the whole-sequence dk/dv lists hold one int32 entry (row * kp + slot) per
  // (row, past block) pair of a batch entry, and their offsets are int32
  if (S * s.hq * (int64_t)std::max(p.kp, 1) >= (int64_t(1) << 31)) return MOBA_ERR_SHAPE;
  b.gate_wg_f = (S + p.gate_t - 1) / p.gate_t;
  b.max_tiles_f = ((S * s.hq * (int64_t)std::max(p.kp, 0) + 255) / 256 + lists + 7) / 8 * 8;
  const uint64_t per_block = (uint64_t)s.block * s.hq * b.kps * 128 * 4;
  int64_t cb = (int64_t)std::max<uint64_t>(1, kBwdPartialCapBytes / per_block);
  cb = std::min<int64_t>(cb, p.n);
  b.chunk = cb * s.block;
  b.gate_wg_c = (b.chunk + p.gate_t - 1) / p.gate_t;
  b.max_tiles_c = ((b.chunk * s.hq * (int64_t)std::max(p.kp, 0) + 255) / 256 + lists + 7) / 8 * 8;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const size_t img = (size_t)s.batch * S * s.hkv * 128 * 2;
  b.off_lse2 = take(rows * 4);
  b.off_delta = take(rows * 4);
  b.off_kimg = take(img);
  b.off_vtmp = take(img);
  b.off_vkimg = take(img);
  b.off_kvimg = take(img);
  b.off_hist_f = take((size_t)lists * b.gate_wg_f * 4);
  b.off_count_f = take((size_t)lists * 4);
  b.off_listoff_f = take((size_t)(lists + 1) * 4);
  b.off_tiles_f = take((size_t)(8 + 2 * b.max_tiles_f) * 4);
  b.off_entries_f = take((size_t)S * s.hq * std::max(p.kp, 1) * 4);
  b.off_hist_c = take((size_t)lists * b.gate_wg_c * 4);
  b.off_count_c = take((size_t)lists * 4);
  b.off_listoff_c = take((size_t)(lists + 1) * 4);
  b.off_tiles_c = take((size_t)(8 + 2 * b.max_tiles_c) * 4);
  b.off_entries_c = take((size_t)b.chunk * s.hq * std::max(p.kp, 1) * 4);
  b.off_dqp = take((size_t)b.chunk * s.hq * b.kps * 128 * 4);
  b.total = off;
  *out = b;
  return MOBA_OK;
}

}  // namespace moba
