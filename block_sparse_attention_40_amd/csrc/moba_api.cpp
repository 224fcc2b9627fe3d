// C ABI of the MoBA forward: validation, workspace carving and launch
// sequencing on the caller's stream.  No device allocation, no host sync.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/moba.h"
#include "moba_kernels.h"
#include "moba_plan.h"

using namespace moba;

namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// ---- measurement support: events around each launch, work per stage ----
struct ProfRec {
  int stage;
  hipEvent_t a, b;
  double work;
};
struct Profiler {
  bool on = false;
  std::mutex mu;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler g_prof;

// Brackets one launch (or a short sequence of launches of one stage).
struct StageScope {
  int stage;
  hipStream_t s;
  double work;
  hipEvent_t a = nullptr;
  StageScope(int stage_, hipStream_t s_, double work_) : stage(stage_), s(s_), work(work_) {
    if (g_prof.on) {
      std::lock_guard<std::mutex> lk(g_prof.mu);
      a = g_prof.get();
      if (a) (void)hipEventRecord(a, s);
    }
  }
  ~StageScope() {
    if (!a) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    hipEvent_t b = g_prof.get();
    if (!b) return;
    (void)hipEventRecord(b, s);
    g_prof.recs.push_back(ProfRec{stage, a, b, work});
  }
};

// Sum over query positions [t0, t0 + cnt) of the past blocks a row attends.
double past_blocks_sum(const Plan& p, int64_t t0, int64_t cnt) {
  const int64_t B = p.s.block;
  double tot = 0;
  for (int64_t jb = t0 / B; jb < (t0 + cnt) / B; ++jb)
    tot += (double)B * (double)(p.s.causal ? (jb < p.kp ? jb : p.kp) : p.kp);
  return tot;
}

// moba_attn_fwd_noalloc's fixed scratch.  In host code `scratch` names a
// host-side stand-in, not the device array: the device address comes from
// hipGetSymbolAddress, once per device (each GPU holds its own copy of the
// array, at its own address, until the process ends).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[MOBA_NOALLOC_SCRATCH_BYTES];

namespace {

// The scratch of the current device (which `stream` must belong to).
int scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOBA_ERR_HIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return MOBA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOBA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOBA_OK;
}

float scale_log2_for(int d) {
  // log2(e) / sqrt(D): the softmax scale 1/sqrt(D) folded into base-2 exponentials
  return (float)(1.4426950408889634 / std::sqrt((double)d));
}

}  // namespace

extern "C" {

int moba_version(void) { return 100; }

int moba_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = on != 0;
  return MOBA_OK;
}

int moba_profile_read(double* ms, int64_t* launches, double* work, int32_t n) {
  if (!ms || !launches || !work) return MOBA_ERR_NULL;
  if (n < 0 || n > MOBA_NUM_STAGES) return MOBA_ERR_SHAPE;
  for (int i = 0; i < n; ++i) { ms[i] = 0; launches[i] = 0; work[i] = 0; }
  std::lock_guard<std::mutex> lk(g_prof.mu);
  int status = MOBA_OK;
  for (const ProfRec& r : g_prof.recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      status = MOBA_ERR_HIP;
    if (r.stage < n) {
      ms[r.stage] += t;
      launches[r.stage] += 1;
      work[r.stage] += r.work;
    }
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  return status;
}

const char* moba_status_string(int status) {
  switch (status) {
    case MOBA_OK: return "ok";
    case MOBA_ERR_NULL: return "a required pointer is NULL";
    case MOBA_ERR_DTYPE: return "unknown dtype";
    case MOBA_ERR_HEAD_DIM: return "head_dim not supported for this dtype (bf16: 128; fp32: 64 or 128)";
    case MOBA_ERR_SEQ_NOT_DIVISIBLE: return "seqlen is not a multiple of block_size";
    case MOBA_ERR_TOPK: return "topk < 1 (decode: also topk above its maximum)";
    case MOBA_ERR_GQA: return "num_q_heads is not a multiple of num_kv_heads, or the group exceeds 128";
    case MOBA_ERR_WORKSPACE: return "workspace is NULL or too small (forward: below moba_workspace_bytes_chunked(..., 1))";
    case MOBA_ERR_HIP: return "a HIP call or kernel launch failed";
    case MOBA_ERR_SHAPE: return "non-positive or too large sizes";
    case MOBA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    default: return "unknown status";
  }
}

int moba_workspace_bytes(int64_t batch, int64_t seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, int32_t block_size, int32_t topk, int32_t causal,
                         size_t* bytes) {
  return moba_workspace_bytes_chunked(batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk,
                                      causal, 0, bytes);
}

int moba_workspace_bytes_chunked(int64_t batch, int64_t seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, int32_t block_size, int32_t topk, int32_t causal,
                                 int64_t max_chunk_blocks, size_t* bytes) {
  if (!bytes) return MOBA_ERR_NULL;
  Plan p;
  // one block per chunk: the smallest plan, without the K/V slice images
  const int st = make_plan(Shape{batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk,
                                 causal ? 1 : 0},
                           &p, max_chunk_blocks, max_chunk_blocks != 1);
  if (st != MOBA_OK) return st;
  *bytes = p.total;
  return MOBA_OK;
}

int moba_plan_info(int64_t batch, int64_t seqlen, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t dtype, int32_t block_size, int32_t topk, int32_t causal, size_t workspace_bytes,
                   int64_t* chunk_blocks, int32_t* tile_rows, int32_t* slice_images) {
  if (!chunk_blocks || !tile_rows || !slice_images) return MOBA_ERR_NULL;
  Plan p;
  const int st = plan_for_workspace(Shape{batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size,
                                          topk, causal ? 1 : 0},
                                    workspace_bytes, &p);
  if (st != MOBA_OK) return st;
  *chunk_blocks = p.chunk_blocks;
  *tile_rows = p.tile_rows;
  *slice_images = p.kv_image ? 1 : 0;
  return MOBA_OK;
}

}  // extern "C"

namespace {

// The forward behind moba_attn_fwd, moba_attn_fwd_gate and moba_attn_fwd_train.
int fwd_impl(const void* q, const void* k, const void* v, int64_t batch, int64_t seqlen, int32_t num_q_heads,
             int32_t num_kv_heads, int32_t head_dim, int32_t dtype, int32_t block_size, int32_t topk, int32_t causal,
             int32_t gate_kind, void* out, int32_t* sel_idx, float* lse, void* workspace, size_t workspace_bytes,
             void* stream) {
  if (gate_kind != MOBA_GATE_MEAN && gate_kind != MOBA_GATE_MINMAX) return MOBA_ERR_SHAPE;
  const bool minmax = gate_kind == MOBA_GATE_MINMAX;
  const Shape shape{batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk, causal ? 1 : 0};
  Plan p;
  int st = make_plan(shape, &p);
  if (st != MOBA_OK) return st;
  if (!q || !k || !v || !out) return MOBA_ERR_NULL;
  if (!workspace) return MOBA_ERR_WORKSPACE;
  // the query chunk is the largest whose workspace fits
  st = plan_for_workspace(shape, workspace_bytes, &p);
  if (st != MOBA_OK) return st;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(workspace) ||
      (sel_idx && (reinterpret_cast<uintptr_t>(sel_idx) & 3u)))
    return MOBA_ERR_ALIGN;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* mu = reinterpret_cast<float*>(ws + p.off_mu);
  int32_t* ws_sel = reinterpret_cast<int32_t*>(ws + p.off_sel);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + p.off_hist);
  int32_t* count = reinterpret_cast<int32_t*>(ws + p.off_count);
  int32_t* listoff = reinterpret_cast<int32_t*>(ws + p.off_listoff);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + p.off_tiles);
  int32_t* entries = reinterpret_cast<int32_t*>(ws + p.off_entries);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(ws + p.off_part_o);
  float* part_lse = reinterpret_cast<float*>(ws + p.off_part_lse);
  // one slot plane of the partials holds every row of a chunk
  const int64_t part_rows = p.kp > 0 ? p.max_pairs / p.kp : 0;
  const bool bf16 = dtype == MOBA_DTYPE_BF16;
  const float sl2 = scale_log2_for(head_dim);

  const double elt = bf16 ? 2.0 : 4.0;
  const double D = head_dim;
  float* lohi = reinterpret_cast<float*>(ws + p.off_lohi);
  // 1. block summaries of the keys (means, or min / max), all blocks of all
  // batch entries.  Only the gate's ranking reads them: when the top-k
  // covers every candidate block no row ranks, and they are not computed.
  if (p.selective) {
    StageScope sc(MOBA_STAGE_MEANPOOL, s,
                  (double)batch * seqlen * num_kv_heads * D * elt +
                      (double)batch * num_kv_heads * p.n * D * (minmax ? 8.0 : 4.0));
    if (minmax) {
      if (launch_minmaxpool(k, dtype, batch, seqlen, num_kv_heads, head_dim, block_size, lohi, s))
        return MOBA_ERR_HIP;
    } else if (launch_meanpool(k, dtype, batch, seqlen, num_kv_heads, head_dim, block_size, mu, s)) {
      return MOBA_ERR_HIP;
    }
  }
  // bf16 gate: the summaries as MFMA tile images (means split into three
  // bf16 parts; max and min as they are)
  uint16_t* mu3 = nullptr;
  if (bf16 && p.selective) {
    mu3 = reinterpret_cast<uint16_t*>(ws + p.off_mu3);
    StageScope sc(MOBA_STAGE_MEANPOOL, s, (double)batch * num_kv_heads * p.n * D * (minmax ? 8.0 + 4.0 : 4.0 + 6.0));
    if (minmax ? launch_mm_split(lohi, batch, p.n, num_kv_heads, mu3, s)
               : launch_mu_split(mu, batch, p.n, num_kv_heads, mu3, s))
      return MOBA_ERR_HIP;
  }

  uint16_t* kimg = p.kv_image ? reinterpret_cast<uint16_t*>(ws + p.off_kimg) : nullptr;
  uint16_t* vimg = p.kv_image ? reinterpret_cast<uint16_t*>(ws + p.off_vimg) : nullptr;
  if (kimg) {
    StageScope sc(MOBA_STAGE_KVLAYOUT, s, 4.0 * (double)batch * seqlen * num_kv_heads * D * elt);
    if (launch_kv_image(k, v, batch, seqlen, num_kv_heads, kimg, vimg, s)) return MOBA_ERR_HIP;
  }

  // 2.. per query chunk: gate, dispatch, past blocks, own block + merge
  for (int64_t bb = 0; bb < batch; ++bb) {
    for (int64_t jc = 0; jc < p.n; jc += p.chunk_blocks) {
      const int64_t nb = (jc + p.chunk_blocks <= p.n) ? p.chunk_blocks : p.n - jc;
      const int64_t t0 = jc * block_size, cnt = nb * block_size;
      const int64_t gate_wg = (cnt + p.gate_t - 1) / p.gate_t;
      int32_t* sel_base;
      int64_t sel_stride_h, sel_pos_base;
      if (sel_idx) {
        sel_base = sel_idx + bb * (int64_t)num_q_heads * seqlen * topk;
        sel_stride_h = seqlen * (int64_t)topk;
        sel_pos_base = 0;
      } else {
        sel_base = ws_sel;
        sel_stride_h = cnt * (int64_t)topk;
        sel_pos_base = t0;
      }
      const bool need_lists = bf16 && p.kp > 0;
      // the gate counts rows per block in LDS up to kDispatchRange blocks;
      // beyond, the dispatch counts them from the selection
      const bool gate_counts = need_lists && p.n <= kDispatchRange;

      GateArgs ga{};
      ga.q = q; ga.mu = mu; ga.lohi = lohi; ga.minmax = minmax ? 1 : 0; ga.mu3 = mu3; ga.sel = sel_base; ga.sel_stride_h = sel_stride_h; ga.sel_pos_base = sel_pos_base;
      ga.hist = gate_counts ? hist : nullptr;
      ga.seqlen = seqlen; ga.n = p.n; ga.t0 = t0; ga.cnt = cnt; ga.gate_wg = gate_wg;
      ga.hq = num_q_heads; ga.hkv = num_kv_heads; ga.block = block_size; ga.topk = topk; ga.kp = p.kp;
      ga.causal = causal ? 1 : 0; ga.g = p.g; ga.gate_t = p.gate_t; ga.bb = (int32_t)bb;
      {
        StageScope sc(MOBA_STAGE_GATE, s,
                      (double)cnt * num_q_heads * D * elt + (double)num_kv_heads * p.n * D * 4.0 +
                          (double)cnt * num_q_heads * topk * 4.0);
        if (launch_gate(ga, dtype, head_dim, s)) return MOBA_ERR_HIP;
      }
      const double past_rows = past_blocks_sum(p, t0, cnt) * num_q_heads;  // (row, past block) pairs
      const double own_keys = causal ? (double)nb * num_q_heads * (double)block_size * (block_size + 1) / 2.0 : 0.0;

      if (!bf16) {
        F32Args fa{};
        fa.q = static_cast<const float*>(q); fa.k = static_cast<const float*>(k);
        fa.v = static_cast<const float*>(v); fa.out = static_cast<float*>(out);
        fa.sel = sel_base; fa.sel_stride_h = sel_stride_h; fa.sel_pos_base = sel_pos_base;
        fa.seqlen = seqlen; fa.t0 = t0; fa.cnt = cnt; fa.hq = num_q_heads; fa.hkv = num_kv_heads;
        fa.d = head_dim; fa.block = block_size; fa.topk = topk; fa.causal = causal ? 1 : 0; fa.g = p.g;
        fa.bb = (int32_t)bb; fa.scale_log2 = sl2; fa.lse = lse;
        StageScope sc(MOBA_STAGE_F32, s, 4.0 * D * (past_rows * block_size + own_keys));
        if (launch_attn_f32(fa, s)) return MOBA_ERR_HIP;
        continue;
      }

      if (need_lists) {
        DispatchArgs da{};
        da.sel = sel_base; da.sel_stride_h = sel_stride_h; da.sel_pos_base = sel_pos_base;
        da.hist = hist; da.count = count; da.listoff = listoff; da.tiles = tiles; da.entries = entries;
        da.n = p.n; da.t0 = t0; da.cnt = cnt; da.gate_wg = gate_wg; da.hq = num_q_heads;
        da.hkv = num_kv_heads; da.block = block_size; da.topk = topk; da.kp = p.kp;
        da.causal = causal ? 1 : 0; da.g = p.g; da.gate_t = p.gate_t; da.tile_rows = p.tile_rows;
        {
          StageScope sc(MOBA_STAGE_DISPATCH, s, (double)cnt * num_q_heads * topk * 4.0 + past_rows * 4.0);
          if ((gate_counts ? launch_dispatch(da, s) : launch_dispatch_from_sel(da, s)) != 0) return MOBA_ERR_HIP;
        }

        PastArgs pa{};
        pa.q = q; pa.k = k; pa.v = v; pa.tiles = tiles; pa.count = count; pa.listoff = listoff;
        pa.entries = entries; pa.part_o = part_o; pa.part_lse = part_lse; pa.part_rows = part_rows;
        pa.seqlen = seqlen; pa.n = p.n;
        pa.t0 = t0; pa.hq = num_q_heads; pa.hkv = num_kv_heads; pa.block = block_size; pa.kp = p.kp;
        pa.g = p.g; pa.bb = (int32_t)bb; pa.max_tiles = (int32_t)p.max_tiles; pa.tile_rows = p.tile_rows;
        pa.scale_log2 = sl2; pa.kimg = kimg; pa.vimg = vimg;
        {
          StageScope sc(MOBA_STAGE_PAST, s, 4.0 * D * past_rows * block_size);
          if (launch_attn_past(pa, s)) return MOBA_ERR_HIP;
        }
      }

      OwnArgs oa{};
      oa.q = q; oa.k = k; oa.v = v; oa.out = out; oa.part_o = part_o; oa.part_lse = part_lse;
      oa.part_rows = part_rows;
      oa.seqlen = seqlen; oa.n = p.n; oa.t0 = t0; oa.cnt = cnt; oa.hq = num_q_heads; oa.hkv = num_kv_heads;
      oa.block = block_size; oa.kp = p.kp; oa.g = p.g; oa.own_t = p.own_t; oa.rows = p.own_rows ? 1 : 0; oa.bb = (int32_t)bb;
      oa.causal = causal ? 1 : 0; oa.scale_log2 = sl2; oa.kimg = kimg; oa.vimg = vimg; oa.lse = lse;
      {
        StageScope sc(MOBA_STAGE_OWN, s, 4.0 * D * own_keys);
        if (launch_attn_own(oa, s)) return MOBA_ERR_HIP;
      }
    }
  }
  return MOBA_OK;
}

}  // namespace

extern "C" {

int moba_attn_fwd(const void* q, const void* k, const void* v, int64_t batch, int64_t seqlen,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                  int32_t block_size, int32_t topk, int32_t causal, void* out, int32_t* sel_idx,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk, causal,
                  MOBA_GATE_MEAN, out, sel_idx, nullptr, workspace, workspace_bytes, stream);
}

int moba_attn_fwd_noalloc(const void* q, const void* k, const void* v, int64_t batch, int64_t seqlen,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                          int32_t block_size, int32_t topk, int32_t causal, void* out, int32_t* sel_idx,
                          void* stream) {
  // every check is host arithmetic and comes before the scratch is looked up
  const Shape shape{batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk, causal ? 1 : 0};
  Plan p;
  int st = make_plan(shape, &p);
  if (st != MOBA_OK) return st;
  if (!q || !k || !v || !out) return MOBA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) ||
      (sel_idx && (reinterpret_cast<uintptr_t>(sel_idx) & 3u)))
    return MOBA_ERR_ALIGN;
  st = plan_for_workspace(shape, MOBA_NOALLOC_SCRATCH_BYTES, &p);  // MOBA_ERR_WORKSPACE: beyond the scratch
  if (st != MOBA_OK) return st;
  void* ws = nullptr;
  st = scratch_for_current_device(reinterpret_cast<hipStream_t>(stream), &ws);
  if (st != MOBA_OK) return st;
  return fwd_impl(q, k, v, batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk, causal,
                  MOBA_GATE_MEAN, out, sel_idx, nullptr, ws, MOBA_NOALLOC_SCRATCH_BYTES, stream);
}

int moba_attn_fwd_gate(const void* q, const void* k, const void* v, int64_t batch, int64_t seqlen,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                       int32_t block_size, int32_t topk, int32_t causal, int32_t gate_kind, void* out,
                       int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk, causal,
                  gate_kind, out, sel_idx, nullptr, workspace, workspace_bytes, stream);
}

int moba_attn_fwd_train(const void* q, const void* k, const void* v, int64_t batch, int64_t seqlen,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                        int32_t block_size, int32_t topk, int32_t causal, void* out, int32_t* sel_idx, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!sel_idx || !lse) return MOBA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return MOBA_ERR_ALIGN;
  return fwd_impl(q, k, v, batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk, causal,
                  MOBA_GATE_MEAN, out, sel_idx, lse, workspace, workspace_bytes, stream);
}

int moba_meanpool(const void* k, int64_t batch, int64_t seqlen, int32_t num_kv_heads, int32_t head_dim,
                  int32_t dtype, int32_t block_size, float* mu, void* stream) {
  Plan p;
  const int st = make_plan(Shape{batch, seqlen, num_kv_heads, num_kv_heads, head_dim, dtype, block_size, 1, 1}, &p);
  if (st != MOBA_OK) return st;
  if (!k || !mu) return MOBA_ERR_NULL;
  if (misaligned(k) || misaligned(mu)) return MOBA_ERR_ALIGN;
  if (launch_meanpool(k, dtype, batch, seqlen, num_kv_heads, head_dim, block_size, mu,
                      reinterpret_cast<hipStream_t>(stream)))
    return MOBA_ERR_HIP;
  return MOBA_OK;
}

int moba_minmaxpool(const void* k, int64_t batch, int64_t seqlen, int32_t num_kv_heads, int32_t head_dim,
                    int32_t dtype, int32_t block_size, float* lohi, void* stream) {
  Plan p;
  const int st = make_plan(Shape{batch, seqlen, num_kv_heads, num_kv_heads, head_dim, dtype, block_size, 1, 1}, &p);
  if (st != MOBA_OK) return st;
  if (!k || !lohi) return MOBA_ERR_NULL;
  if (misaligned(k) || misaligned(lohi)) return MOBA_ERR_ALIGN;
  if (launch_minmaxpool(k, dtype, batch, seqlen, num_kv_heads, head_dim, block_size, lohi,
                        reinterpret_cast<hipStream_t>(stream)))
    return MOBA_ERR_HIP;
  return MOBA_OK;
}

int moba_gate(const void* q, const float* mu, int64_t batch, int64_t seqlen, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t dtype, int32_t block_size, int32_t topk,
              int32_t causal, int32_t* sel_idx, void* stream) {
  Plan p;
  const int st = make_plan(Shape{batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk,
                                 causal ? 1 : 0},
                           &p);
  if (st != MOBA_OK) return st;
  if (!q || !mu || !sel_idx) return MOBA_ERR_NULL;
  if (misaligned(q) || misaligned(mu) || (reinterpret_cast<uintptr_t>(sel_idx) & 3u)) return MOBA_ERR_ALIGN;
  for (int64_t bb = 0; bb < batch; ++bb) {
    GateArgs ga{};
    ga.q = q; ga.mu = mu; ga.sel = sel_idx + bb * (int64_t)num_q_heads * seqlen * topk;
    ga.sel_stride_h = seqlen * (int64_t)topk; ga.sel_pos_base = 0; ga.hist = nullptr;
    ga.seqlen = seqlen; ga.n = p.n; ga.t0 = 0; ga.cnt = seqlen; ga.gate_wg = (seqlen + p.gate_t - 1) / p.gate_t;
    ga.hq = num_q_heads; ga.hkv = num_kv_heads; ga.block = block_size; ga.topk = topk; ga.kp = p.kp;
    ga.causal = causal ? 1 : 0; ga.g = p.g; ga.gate_t = p.gate_t; ga.bb = (int32_t)bb;
    if (launch_gate(ga, dtype, head_dim, reinterpret_cast<hipStream_t>(stream))) return MOBA_ERR_HIP;
  }
  return MOBA_OK;
}

int moba_decode_workspace_bytes(int64_t batch, int64_t max_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, int32_t block_size, int32_t topk, size_t* bytes) {
  if (!bytes) return MOBA_ERR_NULL;
  DecodePlan p;
  const int st = make_decode_plan(batch, max_len, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk, &p);
  if (st != MOBA_OK) return st;
  *bytes = p.total;
  return MOBA_OK;
}

int moba_decode_fwd(const void* q, const void* k_cache, const void* v_cache, float* mu_cache,
                    const int32_t* cache_lens, int64_t batch, int64_t max_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype, int32_t block_size, int32_t topk,
                    void* out, int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream) {
  DecodePlan p;
  const int st = make_decode_plan(batch, max_len, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk, &p);
  if (st != MOBA_OK) return st;
  if (!q || !k_cache || !v_cache || !mu_cache || !cache_lens || !out) return MOBA_ERR_NULL;
  if (!workspace || workspace_bytes < p.total) return MOBA_ERR_WORKSPACE;
  if (misaligned(q) || misaligned(k_cache) || misaligned(v_cache) || misaligned(mu_cache) || misaligned(out) ||
      misaligned(workspace) || (reinterpret_cast<uintptr_t>(cache_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(sel_idx) & 3u))
    return MOBA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  DecodeArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.mu = mu_cache; a.lens = cache_lens;
  a.sel = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(ws + p.off_sel);
  a.sc = reinterpret_cast<float*>(ws + p.off_sc);
  a.uni = reinterpret_cast<int32_t*>(ws + p.off_uni);
  a.uslot = reinterpret_cast<int32_t*>(ws + p.off_uslot);
  a.ucount = reinterpret_cast<int32_t*>(ws + p.off_ucount);
  a.po = reinterpret_cast<float*>(ws + p.off_po);
  a.pml = reinterpret_cast<float*>(ws + p.off_pml);
  a.ksum = reinterpret_cast<float*>(ws + p.off_ksum);
  a.out = out;
  a.batch = batch; a.lmax = max_len; a.nmax = p.nmax;
  a.hq = num_q_heads; a.hkv = num_kv_heads; a.g = p.g; a.d = head_dim; a.block = block_size; a.topk = topk;
  a.U = p.U; a.nchunk = p.nchunk;
  a.scale_log2 = scale_log2_for(head_dim);
  // the bytes each stage reads depend on the cache lengths, which are device
  // data: the stages record no work figure
  // the mean of a block this token completes is formed by the attention and
  // merge kernels (for the next call's gate; this call's gate reads the
  // blocks before it)
  {
    StageScope sc(MOBA_STAGE_DECODE_GATE, s, 0.0);
    if (launch_decode_stage(a, dtype, 0, s)) return MOBA_ERR_HIP;
  }
  {
    StageScope sc(MOBA_STAGE_DECODE_ATTN, s, 0.0);
    if (launch_decode_stage(a, dtype, 1, s)) return MOBA_ERR_HIP;
  }
  {
    StageScope sc(MOBA_STAGE_DECODE_MERGE, s, 0.0);
    if (launch_decode_stage(a, dtype, 2, s)) return MOBA_ERR_HIP;
  }
  return MOBA_OK;
}

int moba_decode_means(const void* k_cache, const int32_t* cache_lens, int64_t batch, int64_t max_len,
                      int32_t num_kv_heads, int32_t head_dim, int32_t dtype, int32_t block_size, float* mu_cache,
                      void* stream) {
  DecodePlan p;
  const int st = make_decode_plan(batch, max_len, num_kv_heads, num_kv_heads, head_dim, dtype, block_size, 1, &p);
  if (st != MOBA_OK) return st;
  if (!k_cache || !cache_lens || !mu_cache) return MOBA_ERR_NULL;
  if (misaligned(k_cache) || misaligned(mu_cache) || (reinterpret_cast<uintptr_t>(cache_lens) & 3u))
    return MOBA_ERR_ALIGN;
  if (launch_decode_means(k_cache, cache_lens, mu_cache, dtype, batch, max_len, p.nmax, num_kv_heads, head_dim,
                          block_size, reinterpret_cast<hipStream_t>(stream)))
    return MOBA_ERR_HIP;
  return MOBA_OK;
}

int moba_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t dtype, int32_t block_size, int32_t topk, int32_t causal,
                             size_t* bytes) {
  if (!bytes) return MOBA_ERR_NULL;
  BwdPlan b;
  const int st = make_bwd_plan(Shape{batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk,
                                     causal ? 1 : 0},
                               &b);
  if (st != MOBA_OK) return st;
  *bytes = b.total;
  return MOBA_OK;
}

int moba_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  const int32_t* sel_idx, int64_t batch, int64_t seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t dtype, int32_t block_size, int32_t topk, int32_t causal, void* dq,
                  void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  BwdPlan b;
  const int st = make_bwd_plan(Shape{batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk,
                                     causal ? 1 : 0},
                               &b);
  if (st != MOBA_OK) return st;
  const Plan& p = b.p;
  if (!q || !k || !v || !out || !dout || !lse || !sel_idx || !dq || !dk || !dv) return MOBA_ERR_NULL;
  if (!workspace || workspace_bytes < b.total) return MOBA_ERR_WORKSPACE;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(dout) || misaligned(dq) ||
      misaligned(dk) || misaligned(dv) || misaligned(workspace) || (reinterpret_cast<uintptr_t>(lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(sel_idx) & 3u))
    return MOBA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  const int64_t S = seqlen, D = head_dim;
  float* lse2 = reinterpret_cast<float*>(ws + b.off_lse2);
  float* delta = reinterpret_cast<float*>(ws + b.off_delta);
  uint16_t* kimg = reinterpret_cast<uint16_t*>(ws + b.off_kimg);
  uint16_t* vtmp = reinterpret_cast<uint16_t*>(ws + b.off_vtmp);
  uint16_t* vkimg = reinterpret_cast<uint16_t*>(ws + b.off_vkimg);
  uint16_t* kvimg = reinterpret_cast<uint16_t*>(ws + b.off_kvimg);
  {
    StageScope sc(MOBA_STAGE_BWD_PREP, s, (double)batch * S * num_q_heads * D * 2.0 * 2.0 +
                                              4.0 * batch * S * num_kv_heads * D * 2.0 * 2.0);
    if (launch_bwd_prep(out, dout, lse, lse2, delta, batch, S, num_q_heads, s)) return MOBA_ERR_HIP;
    // K and V in both operand layouts: (K layout of K, V^T layout of V) and (K layout of V, V^T layout of K)
    if (launch_kv_image(k, v, batch, S, num_kv_heads, kimg, vtmp, s)) return MOBA_ERR_HIP;
    if (launch_kv_image(v, k, batch, S, num_kv_heads, vkimg, kvimg, s)) return MOBA_ERR_HIP;
  }
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.lse2 = lse2; a.delta = delta;
  a.kimg = kimg; a.vkimg = vkimg; a.kvimg = kvimg;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dq_part = reinterpret_cast<float*>(ws + b.off_dqp);
  a.seqlen = S; a.n = p.n; a.hq = num_q_heads; a.hkv = num_kv_heads; a.block = block_size; a.kp = p.kp;
  a.kps = b.kps; a.g = p.g; a.causal = causal ? 1 : 0;
  a.scale_log2 = scale_log2_for(head_dim);
  a.scale = (float)(1.0 / std::sqrt((double)head_dim));
  const double own_pairs_per_block = causal ? (double)num_q_heads * block_size * (block_size + 1) / 2.0 : 0.0;
  for (int64_t bb = 0; bb < batch; ++bb) {
    a.bb = (int32_t)bb;
    const int32_t* sel_b = sel_idx + bb * (int64_t)num_q_heads * S * topk;
    DispatchArgs da{};
    da.sel = sel_b; da.sel_stride_h = S * (int64_t)topk; da.sel_pos_base = 0;
    da.n = p.n; da.hq = num_q_heads; da.hkv = num_kv_heads; da.block = block_size; da.topk = topk; da.kp = p.kp;
    da.causal = causal ? 1 : 0; da.g = p.g; da.gate_t = p.gate_t; da.tile_rows = 256;
    // whole-sequence lists for dk / dv
    a.count_f = reinterpret_cast<int32_t*>(ws + b.off_count_f);
    a.listoff_f = reinterpret_cast<int32_t*>(ws + b.off_listoff_f);
    a.entries_f = reinterpret_cast<int32_t*>(ws + b.off_entries_f);
    if (p.kp > 0) {
      StageScope sc(MOBA_STAGE_DISPATCH, s, (double)S * num_q_heads * topk * 4.0 * 3.0);
      DispatchArgs df = da;
      df.hist = reinterpret_cast<int32_t*>(ws + b.off_hist_f);
      df.count = const_cast<int32_t*>(a.count_f);
      df.listoff = const_cast<int32_t*>(a.listoff_f);
      df.tiles = reinterpret_cast<int32_t*>(ws + b.off_tiles_f);
      df.entries = const_cast<int32_t*>(a.entries_f);
      df.t0 = 0; df.cnt = S; df.gate_wg = b.gate_wg_f;
      if (launch_dispatch_from_sel(df, s)) return MOBA_ERR_HIP;
    }
    {
      const double pairs = past_blocks_sum(p, 0, S) * num_q_heads * block_size + own_pairs_per_block * p.n;
      StageScope sc(MOBA_STAGE_BWD_DKDV, s, 8.0 * D * pairs);
      if (launch_bwd_dkdv(a, s)) return MOBA_ERR_HIP;
    }
    for (int64_t t0 = 0; t0 < S; t0 += b.chunk) {
      const int64_t cnt = std::min<int64_t>(b.chunk, S - t0);
      a.t0 = t0; a.cnt = cnt;
      a.tiles = reinterpret_cast<int32_t*>(ws + b.off_tiles_c);
      a.count = reinterpret_cast<int32_t*>(ws + b.off_count_c);
      a.listoff = reinterpret_cast<int32_t*>(ws + b.off_listoff_c);
      a.entries = reinterpret_cast<int32_t*>(ws + b.off_entries_c);
      if (p.kp > 0) {
        StageScope sc(MOBA_STAGE_DISPATCH, s, (double)cnt * num_q_heads * topk * 4.0 * 3.0);
        DispatchArgs dc = da;
        dc.hist = reinterpret_cast<int32_t*>(ws + b.off_hist_c);
        dc.count = const_cast<int32_t*>(a.count);
        dc.listoff = const_cast<int32_t*>(a.listoff);
        dc.tiles = const_cast<int32_t*>(a.tiles);
        dc.entries = const_cast<int32_t*>(a.entries);
        dc.t0 = t0; dc.cnt = cnt; dc.gate_wg = (cnt + p.gate_t - 1) / p.gate_t;
        if (launch_dispatch_from_sel(dc, s)) return MOBA_ERR_HIP;
      }
      const double pairs = past_blocks_sum(p, t0, cnt) * num_q_heads * block_size +
                           own_pairs_per_block * (double)(cnt / block_size);
      StageScope sc(MOBA_STAGE_BWD_DQ, s, 6.0 * D * pairs);
      if (launch_bwd_dq(a, p.kp > 0 ? b.max_tiles_c : 0, s)) return MOBA_ERR_HIP;
    }
  }
  return MOBA_OK;
}

}  // extern "C"
