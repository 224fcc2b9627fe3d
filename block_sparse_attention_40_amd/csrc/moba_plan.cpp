// Host-side validation and workspace planning (no HIP calls).
#include "moba_plan.h"

#include <algorithm>

#include "../../include/moba.h"

namespace moba {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int make_plan(const Shape& s, Plan* p) {
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
  // per-block counters live in LDS (32 KiB at most); grid z carries the batch
  if (q.n > 8192 || s.batch > 65535) return MOBA_ERR_SHAPE;
  q.keff = (int32_t)std::min<int64_t>(s.topk, q.n);
  q.kp = s.causal ? q.keff - 1 : q.keff;
  q.g = s.hq / s.hkv;
  // candidates the gate ranks: past blocks (at most n-1) or all n blocks
  const int64_t cand = s.causal ? q.n - 1 : q.n;
  q.selective = q.kp < cand;
  if (q.selective && q.kp > MOBA_MAX_SELECTIVE_TOPK) return MOBA_ERR_TOPK;

  // index arithmetic bounds: rows and row*slot products stay in int32 range
  const int64_t rows_total = s.batch * s.seqlen * (int64_t)s.hq;
  if (s.seqlen > (int64_t(1) << 31) / s.hq || rows_total <= 0) return MOBA_ERR_SHAPE;

  q.gate_t = std::max(1, kGateRows / q.g);
  q.own_t = std::max(1, kOwnRows / q.g);

  // per (row, past block) pair: the normalised partial o in bf16 plus its lse in fp32
  const uint64_t per_block_partial =
      (uint64_t)s.block * s.hq * (uint64_t)std::max(q.kp, 0) * (uint64_t)(s.d * 2 + 4);
  if (q.kp == 0) {
    q.chunk_blocks = q.n;
  } else {
    q.chunk_blocks = (int64_t)std::max<uint64_t>(1, kPartialCapBytes / per_block_partial);
    q.chunk_blocks = std::min<int64_t>(q.chunk_blocks, q.n);
  }
  const int64_t chunk_pos = q.chunk_blocks * s.block;
  q.gate_wg = (chunk_pos + q.gate_t - 1) / q.gate_t;
  q.max_pairs = chunk_pos * s.hq * (int64_t)q.kp;
  if (q.max_pairs >= (int64_t(1) << 31)) return MOBA_ERR_SHAPE;
  const int64_t lists = (int64_t)s.hkv * q.n;
  // long lists: 384-row tiles over the K/V slice images (bf16, whole slices),
  // else 256; short lists: 128
  q.tile_rows = (q.max_pairs / lists >= kLargeTileMinRows) ? kTileRowsLarge : kTileRowsSmall;
  if (q.tile_rows == kTileRowsLarge && s.dtype == MOBA_DTYPE_BF16 && s.block % kSliceKeys == 0)
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
  q.kv_image = s.dtype == MOBA_DTYPE_BF16 && s.block % kSliceKeys == 0 &&
               (q.kp > 0 ? q.tile_rows == kTileRowsImage : s.block >= kOwnImageMinBlock);
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

}  // namespace moba
