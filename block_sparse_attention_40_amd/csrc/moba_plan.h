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
// Query rows of one own-block attention tile: 8 waves x 32 rows, or 4 waves
// x 32 rows when the tile reads K and V rows in 32-key slices (bf16, no
// slice images, block a multiple of 32), three work-groups per CU.
constexpr int kOwnRows = 256;
constexpr int kOwnRowsSmall = 128;
// Keys per LDS slice of the kernels that read K and V rows directly.
constexpr int kRowSliceKeys = 32;
// Block size from which the own-block tiles read K and V rows even where the
// slice images exist (with past blocks): measured 4 % faster on the own block
// at 1M (block 4096) and 1 % at 128K (block 512), 2.5 % slower at block 128.
constexpr int64_t kOwnRowsMinBlock = 512;
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
// Per-block row counters that one dispatch pass keeps in LDS (32 KiB); with
// more blocks the gate leaves the counting to the dispatch, which makes one
// pass over the selection per range of this many blocks.
constexpr int64_t kDispatchRange = 8192;
// Upper bound on the per-(list, gate work-group) count table of one chunk
// (KV heads x blocks x gate work-groups, int32): it grows with the chunk times
// the number of blocks, so many-block shapes take shorter chunks.
constexpr uint64_t kHistCapBytes = 2ull << 30;

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
  bool own_rows;        // own-block tiles of 128 rows from K and V rows (else 256 rows, from the images or through registers)
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

// Decode (one new query per sequence against its cache).
constexpr int kDecodeMaxGroup = 16;     // query heads per KV head
constexpr int kDecodeMaxTopk = 64;
constexpr int kDecodeMaxBlocks = 16384;  // cache capacity in blocks
constexpr int kDecodeChunk = 512;        // keys per attention work-group (8 steps of 64)

// Decode: sizes, limits and the workspace carve-up.
struct DecodePlan {
  int64_t nmax;
  int32_t g, U, nchunk;
  size_t off_sc, off_uni, off_uslot, off_ucount, off_sel, off_po, off_pml, off_ksum, total;
};
int make_decode_plan(int64_t batch, int64_t lmax, int32_t hq, int32_t hkv, int32_t d, int32_t dtype, int32_t block,
                     int32_t topk, DecodePlan* p);

// Backward: sizes and the workspace carve-up (bf16, head dim 128).
constexpr uint64_t kBwdPartialCapBytes = 2ull << 30;  // per-chunk dq contributions

// Validate `s` and fill `p`.  max_chunk_blocks > 0 caps the query blocks per
// chunk (0: the default, partials of one chunk within kPartialCapBytes);
// allow_image = false never re-lays K and V out as slice images.  Returns a
// moba_status code.
int make_plan(const Shape& s, Plan* p, int64_t max_chunk_blocks = 0, bool allow_image = true);

// The plan with the largest query chunk whose workspace fits in ws_bytes
// (the default plan when it fits); without the K/V slice images when no plan
// with them fits.  MOBA_ERR_WORKSPACE when even one query block per chunk
// does not fit.
int plan_for_workspace(const Shape& s, size_t ws_bytes, Plan* p);

struct BwdPlan {
  Plan p;
  int32_t kps;              // dq slots per row: kp past + 1 own (causal)
  int64_t gate_wg_f;        // rows-per-work-group units of the whole sequence
  int64_t max_tiles_f;
  int64_t chunk;            // query positions per dq chunk (whole blocks)
  int64_t gate_wg_c, max_tiles_c;
  size_t off_lse2, off_delta, off_kimg, off_vtmp, off_vkimg, off_kvimg;
  size_t off_hist_f, off_count_f, off_listoff_f, off_tiles_f, off_entries_f;
  size_t off_hist_c, off_count_c, off_listoff_c, off_tiles_c, off_entries_c, off_dqp, total;
};
int make_bwd_plan(const Shape& s, BwdPlan* out);

}  // namespace moba
