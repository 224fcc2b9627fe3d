// Host-side argument validation and workspace planning for the MoBA forward.
// Pure C++ (no HIP calls), so it is exercised by the CPU tests as well.
#pragma once

#include <cstddef>
#include <cstdint>

namespace moba {

// Rows of one gate work-group (threads; one query row per thread).
constexpr int kGateRows = 256;
// Query rows of one past-block attention tile: 4, 8 or 12 waves x 32 rows,
// the larger when the per-block row lists are long; 12 waves (three per
// SIMD) when the tile reads the K/V slice images (bf16, whole 64-key slices).
constexpr int kTileRowsSmall = 128;
constexpr int kTileRowsLarge = 256;
constexpr int kTileRowsImage = 384;
// Mean list length from which the large tile is used.
constexpr int64_t kLargeTileMinRows = 2048;
// Query rows of one own-block attention tile (8 waves x 32 rows).
constexpr int kOwnRows = 256;
// Largest query-head group (num_q_heads / num_kv_heads) the tiles support.
constexpr int kMaxGroup = 128;
// Blocks per tile of the bf16 gate's score MFMAs.
constexpr int kGateTile = 32;
// Block size from which the own-block kernel alone (no past blocks) reads
// K and V through the slice images.
constexpr int64_t kOwnImageMinBlock = 1024;
// Keys per K / V^T image slice (the attention kernels' LDS slice).
constexpr int kSliceKeys = 64;
// Upper bound on the partial-result buffer of one query chunk (bf16 o + fp32 lse).
constexpr uint64_t kPartialCapBytes = 8ull << 30;

struct Shape {
  int64_t batch, seqlen;
  int32_t hq, hkv, d, dtype, block, topk, causal;
};

struct Plan {
  Shape s;
  int64_t n;            // number of blocks
  int32_t keff;         // min(topk, n)
  int32_t kp;           // past slots per row: keff - 1 (causal) or keff (non-causal)
  int32_t g;            // query heads per KV head
  int32_t gate_t;       // query positions per gate work-group
  int32_t own_t;        // query positions per own-block tile
  int32_t tile_rows;    // rows per past-block attention tile
  int64_t chunk_blocks; // query blocks processed per chunk
  int64_t gate_wg;      // gate work-groups per KV head per chunk
  int64_t max_pairs;    // (row, past block) pairs in one chunk, upper bound
  int64_t max_tiles;    // attention tiles in one chunk, upper bound (multiple of 8)
  bool selective;       // whether the gate has to score and rank blocks
  bool kv_image;        // K and V are re-laid out per 64-key slice for direct LDS loads (bf16, block % 64 == 0)
  // workspace layout (byte offsets, 256-aligned)
  size_t off_mu, off_sel, off_hist, off_count, off_listoff, off_tiles, off_entries;
  size_t off_part_o, off_part_lse, off_kimg, off_vimg, off_mu3, off_lohi, total;
};

// Validate `s` and fill `p`.  Returns a moba_status code.
int make_plan(const Shape& s, Plan* p);

}  // namespace moba
