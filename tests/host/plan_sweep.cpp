// Sweep of the host-side planners of the MoBA library (forward, forward with
// a given workspace, backward, decode) over shapes that include the overflow
// edges of their size arithmetic.  tests/test_host_sanitizers.py builds it
// with g++ -fsanitize=address,undefined (UndefinedBehaviorSanitizer aborts on
// signed overflow, misaligned access and the like) and runs it; it exits 0
// when every accepted plan is self-consistent.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../block_sparse_attention_40_amd/csrc/moba_plan.h"
#include "../../include/moba.h"

using namespace moba;

static long g_checked = 0, g_accepted = 0, g_fail = 0;

#define CHECK(c, ...)                                                  \
  do {                                                                 \
    if (!(c)) {                                                        \
      ++g_fail;                                                        \
      std::fprintf(stderr, "FAIL %s:%d %s: ", __FILE__, __LINE__, #c); \
      std::fprintf(stderr, __VA_ARGS__);                               \
      std::fprintf(stderr, "\n");                                      \
    }                                                                  \
  } while (0)

static void describe(const Shape& s, char* buf, size_t n) {
  std::snprintf(buf, n, "b=%lld S=%lld hq=%d hkv=%d d=%d dt=%d B=%d k=%d c=%d", (long long)s.batch,
                (long long)s.seqlen, s.hq, s.hkv, s.d, s.dtype, s.block, s.topk, s.causal);
}

// Offsets of one workspace layout: 256-aligned, within the total, ascending.
static void check_offsets(const std::vector<size_t>& offs, size_t total, const char* what, const char* d) {
  size_t prev = 0;
  for (size_t o : offs) {
    CHECK(o % 256 == 0, "%s %s offset %zu not 256-aligned", what, d, o);
    CHECK(o >= prev, "%s %s offsets out of order", what, d);
    CHECK(o <= total, "%s %s offset %zu beyond total %zu", what, d, o, total);
    prev = o;
  }
}

static void check_plan(const Shape& s, const Plan& p, const char* d) {
  CHECK(p.n >= 1 && p.n * (int64_t)s.block == s.seqlen, "%s n", d);
  CHECK(p.chunk_blocks >= 1 && p.chunk_blocks <= p.n, "%s chunk_blocks %lld", d, (long long)p.chunk_blocks);
  CHECK(p.keff >= 1 && p.keff <= s.topk && p.keff <= p.n, "%s keff", d);
  CHECK(p.kp >= 0 && p.kp <= p.keff, "%s kp", d);
  CHECK(p.max_pairs >= 0 && p.max_pairs < (int64_t(1) << 31), "%s max_pairs", d);
  CHECK(p.tile_rows == kTileRowsSmall || p.tile_rows == kTileRowsLarge || p.tile_rows == kTileRowsImage,
        "%s tile_rows %d", d, p.tile_rows);
  CHECK(p.tile_rows != kTileRowsImage || (p.kv_image && s.block % kSliceKeys == 0), "%s image tiles without images",
        d);
  CHECK(p.max_tiles % 8 == 0 && p.max_tiles >= (p.max_pairs + p.tile_rows - 1) / p.tile_rows, "%s max_tiles", d);
  CHECK(p.gate_wg >= 1, "%s gate_wg", d);
  // the per-(list, gate work-group) count table fits its region and its cap
  const uint64_t table = (uint64_t)s.hkv * (uint64_t)p.gate_wg * (uint64_t)p.n * 4;
  CHECK(p.off_count - p.off_hist >= table, "%s count table region", d);
  CHECK(table <= kHistCapBytes || p.chunk_blocks == 1, "%s count table %llu above the cap", d,
        (unsigned long long)table);
  check_offsets({p.off_mu, p.off_sel, p.off_hist, p.off_count, p.off_listoff, p.off_tiles, p.off_entries,
                 p.off_part_o, p.off_part_lse, p.off_kimg, p.off_vimg, p.off_mu3, p.off_lohi},
                p.total, "fwd", d);
  // the regions the kernels index: entries and partials hold max_pairs pairs
  CHECK(p.off_part_o - p.off_entries >= (size_t)p.max_pairs * 4, "%s entries region", d);
  CHECK(p.off_part_lse - p.off_part_o >= (size_t)p.max_pairs * s.d * 2, "%s partial region", d);
}

static void sweep_forward(const Shape& s) {
  char d[256];
  describe(s, d, sizeof d);
  ++g_checked;
  Plan p{};
  if (make_plan(s, &p) != MOBA_OK) return;
  ++g_accepted;
  check_plan(s, p, d);
  // the smallest plan, and plans for workspaces between it and the default
  Plan lo{};
  CHECK(make_plan(s, &lo, 1, false) == MOBA_OK, "%s smallest plan refused", d);
  check_plan(s, lo, d);
  CHECK(lo.total <= p.total, "%s smallest plan larger than the default", d);
  int64_t prev_chunk = 0;
  for (int f = 0; f <= 8; ++f) {
    const size_t ws = lo.total + (size_t)((double)(p.total - lo.total) * f / 8.0);
    Plan q{};
    const int st = plan_for_workspace(s, ws, &q);
    CHECK(st == MOBA_OK, "%s workspace %zu refused", d, ws);
    if (st != MOBA_OK) continue;
    check_plan(s, q, d);
    CHECK(q.total <= ws, "%s plan needs %zu > workspace %zu", d, q.total, ws);
    CHECK(q.chunk_blocks >= prev_chunk || q.kv_image, "%s chunk shrank as the workspace grew", d);
    prev_chunk = q.chunk_blocks;
  }
  if (lo.total > 0) {
    Plan q{};
    CHECK(plan_for_workspace(s, lo.total - 1, &q) == MOBA_ERR_WORKSPACE, "%s below the smallest plan", d);
  }
  BwdPlan b{};
  if (make_bwd_plan(s, &b) == MOBA_OK) {
    check_offsets({b.off_lse2, b.off_delta, b.off_kimg, b.off_vtmp, b.off_vkimg, b.off_kvimg, b.off_hist_f,
                   b.off_count_f, b.off_listoff_f, b.off_tiles_f, b.off_entries_f, b.off_hist_c, b.off_count_c,
                   b.off_listoff_c, b.off_tiles_c, b.off_entries_c, b.off_dqp},
                  b.total, "bwd", d);
    CHECK(b.chunk >= s.block && b.chunk % s.block == 0 && b.chunk <= s.seqlen, "%s bwd chunk", d);
    CHECK(s.seqlen * s.hq * (int64_t)(b.p.kp > 0 ? b.p.kp : 1) < (int64_t(1) << 31), "%s bwd entries", d);
  }
}

static void sweep_decode(int64_t batch, int64_t lmax, int32_t hq, int32_t hkv, int32_t d_, int32_t dt, int32_t block,
                         int32_t topk) {
  char d[256];
  std::snprintf(d, sizeof d, "decode b=%lld L=%lld hq=%d hkv=%d d=%d dt=%d B=%d k=%d", (long long)batch,
                (long long)lmax, hq, hkv, d_, dt, block, topk);
  ++g_checked;
  DecodePlan p{};
  if (make_decode_plan(batch, lmax, hq, hkv, d_, dt, block, topk, &p) != MOBA_OK) return;
  ++g_accepted;
  CHECK(p.nmax * block == lmax && p.nmax <= kDecodeMaxBlocks, "%s nmax", d);
  check_offsets({p.off_sc, p.off_uni, p.off_uslot, p.off_ucount, p.off_sel, p.off_po, p.off_pml, p.off_ksum}, p.total,
                "decode", d);
}

int main() {
  const int64_t I64 = INT64_MAX;
  const int32_t I32 = INT32_MAX;
  const std::vector<int64_t> batches = {-1, 0, 1, 2, 65535, 65536, int64_t(1) << 40};
  const std::vector<int64_t> seqs = {-1,         0,           1,           16,      960, 1024, 8192, 32768,
                                     1 << 20,    int64_t(10) << 20, int64_t(1) << 31, int64_t(1) << 40, I64};
  const std::vector<int32_t> hqs = {-1, 0, 1, 4, 32, 128, 129, I32};
  const std::vector<int32_t> ds = {0, 64, 96, 128, I32};
  const std::vector<int32_t> blocks = {-1, 0, 1, 16, 64, 96, 128, 512, 4096, 40960, 1 << 30, I32};
  const std::vector<int32_t> topks = {-1, 0, 1, 3, 12, 33, 34, I32};
  for (int64_t b : batches)
    for (int64_t S : seqs)
      for (int32_t hq : hqs)
        for (int32_t hkv : {1, 8, 3})
          for (int32_t d : ds)
            for (int32_t dt : {0, 1, 7})
              for (int32_t B : blocks)
                for (int32_t k : topks)
                  for (int32_t c : {0, 1}) sweep_forward(Shape{b, S, hq, hkv, d, dt, B, k, c});
  for (int64_t b : {int64_t(-1), int64_t(1), int64_t(8), int64_t(65536)})
    for (int64_t L : {int64_t(0), int64_t(4096), int64_t(1) << 20, int64_t(1) << 31, I64})
      for (int32_t hq : {1, 32, 34, I32})
        for (int32_t hkv : {1, 2, 8})
          for (int32_t d : {64, 128})
            for (int32_t dt : {0, 1})
              for (int32_t B : {-1, 0, 64, 512, 4096, I32})
                for (int32_t k : {0, 1, 12, 64, 65}) sweep_decode(b, L, hq, hkv, d, dt, B, k);
  std::printf("checked %ld shapes, %ld accepted, %ld failures\n", g_checked, g_accepted, g_fail);
  return g_fail ? 1 : 0;
}
