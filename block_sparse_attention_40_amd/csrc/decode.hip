// Decode-time MoBA: one new query per sequence against its key/value cache.
//
// The new token of sequence b sits at position t = L_b - 1 of a cache holding
// L_b keys and values (its own included) and is routed exactly as prefill row
// t (report §2.2, §2.3): own block j = t / B cut at t, the best min(k-1, j) of
// the complete past blocks 0..j-1 by <q, mean key>, softmax over the union.
// The pages evaluate generation with full attention and name sparse decode as
// future work (report §4.4, §6.3); the rule above is the prefill rule at the
// last row.
//
// Kernels, in launch order:
//   decode_gate_kernel   one work-group per (KV head, sequence): scores of the
//                        group's queries against the cached block means,
//                        top-k per head, and the union of the group's chosen
//                        blocks (so a block chosen by several heads of the
//                        group is read from HBM once);
//   decode_attn_kernel   one work-group per (512-key chunk, union entry,
//                        sequence x KV head): streams the chunk's K and V
//                        through LDS once, in 64-key steps, and serves every
//                        head of the group that chose the block; writes an
//                        unnormalised partial (o, max, sum) per (head, slot,
//                        chunk), and the key column sums of an own block that
//                        the new token completes;
//   decode_merge_kernel  one wave per (head, sequence): merges the partials,
//                        and turns those column sums into the block's cached
//                        mean (the next step's gate reads it);
//   decode_means_kernel  the mean of every complete block (initialisation of
//                        the cache of means).
// HBM-bound: the chosen blocks' keys and values are the only large reads.
#include "moba_device.h"
#include "moba_kernels.h"

namespace moba {

constexpr int kGateRegKeys = 8;  // past blocks per lane held in registers (j <= 512)

namespace {

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, o), hi = __shfl_xor((uint32_t)(x >> 32), o);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    x = y > x ? y : x;
  }
  return x;
}
// Inclusive prefix sum over the 256 threads of a work-group.
__device__ __forceinline__ int block_incl_scan_256(int x, int* wtot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  for (int w = 0; w < wave; ++w) x += wtot[w];
  return x;
}

__device__ __forceinline__ void load2(const bf16raw* p, float& a, float& b) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  a = bf16lo(w);
  b = bf16hi(w);
}
__device__ __forceinline__ void load2(const float* p, float& a, float& b) {
  const float2 w = *reinterpret_cast<const float2*>(p);
  a = w.x;
  b = w.y;
}
__device__ __forceinline__ void store2(bf16raw* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}
__device__ __forceinline__ void store2(float* p, float a, float b) { *reinterpret_cast<float2*>(p) = float2{a, b}; }

__device__ __forceinline__ bool len_ok(int64_t L, int64_t lmax) { return L >= 1 && L <= lmax; }

}  // namespace

// ---------------------------------------------------------------------------
// Gate, top-k and the group's union.  grid (hkv, batch), 256 threads.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_gate_kernel(DecodeArgs a) {
  __shared__ float qs[kDecodeMaxGroup * D];              // the group's queries, fp32
  __shared__ int32_t srow[kDecodeMaxGroup * kDecodeMaxTopk];  // the group's sel rows
  __shared__ uint32_t bits[kDecodeMaxBlocks / 32];       // union bitmap over blocks 0..j
  __shared__ int wtot[4];
  const int hk = blockIdx.x;
  const int64_t bb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = a.g, topk = a.topk;
  const int64_t L = a.lens[bb];
  const bool ok = len_ok(L, a.lmax);
  const int64_t j = ok ? (L - 1) / a.block : 0;
  const int m = ok ? (int)(j < topk - 1 ? j : topk - 1) : 0;
  const bool rank = ok && m < j;  // some complete past block is left out
  const int64_t hq0 = bb * a.hq + (int64_t)hk * g;  // first query head row of the group

  for (int e = tid; e < g * D; e += 256) qs[e] = load_f32(reinterpret_cast<const T*>(a.q) + hq0 * D + e);
  __syncthreads();

  if (rank) {
    // s_i = <q, mu_i> for the complete past blocks, each mean read once for
    // the whole group
    const float* mu = a.mu + (bb * a.hkv + hk) * a.nmax * D;
    for (int64_t i = tid; i < j; i += 256) {
      float acc[kDecodeMaxGroup];
#pragma unroll
      for (int hh = 0; hh < kDecodeMaxGroup; ++hh) acc[hh] = 0.f;
      for (int d0 = 0; d0 < D; d0 += 4) {
        const f32x4 mv = *reinterpret_cast<const f32x4*>(mu + i * D + d0);
#pragma unroll
        for (int hh = 0; hh < kDecodeMaxGroup; ++hh) {
          if (hh < g) {
            const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + hh * D + d0);
            acc[hh] = __builtin_fmaf(qv[0], mv[0], acc[hh]);
            acc[hh] = __builtin_fmaf(qv[1], mv[1], acc[hh]);
            acc[hh] = __builtin_fmaf(qv[2], mv[2], acc[hh]);
            acc[hh] = __builtin_fmaf(qv[3], mv[3], acc[hh]);
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < kDecodeMaxGroup; ++hh)
        if (hh < g) a.sc[(hq0 + hh) * a.nmax + i] = acc[hh] != acc[hh] ? -__builtin_inff() : acc[hh];
    }
  }
  __syncthreads();

  // per head (one wave each): round r takes the largest key below round
  // r-1's; key = orderable score, then the lower block index
  for (int hh = wave; hh < g; hh += 4) {
    int32_t* row = srow + hh * kDecodeMaxTopk;
    if (!rank) {
      // no choice: every past block, then the own block (or nothing)
      for (int s = lane; s < topk; s += 64) row[s] = !ok ? -1 : (s < j ? s : (s == j ? (int32_t)j : -1));
      continue;
    }
    const float* sc = a.sc + (hq0 + hh) * a.nmax;
    uint64_t prev = ~0ull;
    uint32_t mine = 0xffffffffu;  // lane r keeps round r's block
    if (j <= 64 * kGateRegKeys) {
      // up to kGateRegKeys keys per lane, read once
      uint64_t kr[kGateRegKeys];
#pragma unroll
      for (int x = 0; x < kGateRegKeys; ++x) {
        const int64_t i = lane + 64 * x;
        kr[x] = i < j ? ((uint64_t)orderable(sc[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i) : 0ull;
      }
      for (int r = 0; r < m; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int x = 0; x < kGateRegKeys; ++x)
          if (kr[x] < prev && kr[x] > best) best = kr[x];
        best = wave_max_u64(best);
        prev = best;
        if (lane == r) mine = 0xffffffffu - (uint32_t)best;
      }
    } else {
      for (int r = 0; r < m; ++r) {
        uint64_t best = 0;
        for (int64_t i = lane; i < j; i += 64) {
          const uint64_t key = ((uint64_t)orderable(sc[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
          if (key < prev && key > best) best = key;
        }
        best = wave_max_u64(best);
        prev = best;
        if (lane == r) mine = 0xffffffffu - (uint32_t)best;
      }
    }
    // ascending order: lane r's position among the m chosen blocks
    int pos = 0;
    for (int r = 0; r < m; ++r) {
      const uint32_t o = __shfl(mine, r);
      pos += (o < mine) ? 1 : 0;
    }
    if (lane < m) row[pos] = (int32_t)mine;
    for (int s = m + lane; s < topk; s += 64) row[s] = (s == m) ? (int32_t)j : -1;
  }
  __syncthreads();

  for (int e = tid; e < g * topk; e += 256) {
    const int hh = e / topk, s = e % topk;
    a.sel[(hq0 + hh) * topk + s] = srow[hh * kDecodeMaxTopk + s];
  }

  // union of the group's chosen blocks, ascending: bitmap, then ranks
  const int64_t z = bb * a.hkv + hk;
  const int nw = ok ? (int)(j / 32 + 1) : 0;
  for (int w = tid; w < kDecodeMaxBlocks / 32; w += 256) bits[w] = 0u;
  for (int e = tid; e < a.U * g; e += 256) a.uslot[z * a.U * g + e] = -1;
  __syncthreads();
  for (int e = tid; e < g * topk; e += 256) {
    const int32_t v = srow[(e / topk) * kDecodeMaxTopk + e % topk];
    if (v >= 0) atomicOr(&bits[v >> 5], 1u << (v & 31));
  }
  __syncthreads();
  // thread tid owns words 2 tid and 2 tid + 1 (kDecodeMaxBlocks / 32 = 512)
  const int w0 = 2 * tid;
  const int c0 = w0 < nw ? __builtin_popcount(bits[w0]) : 0;
  const int c1 = w0 + 1 < nw ? __builtin_popcount(bits[w0 + 1]) : 0;
  const int incl = block_incl_scan_256(c0 + c1, wtot);
  __shared__ int wprefix[kDecodeMaxBlocks / 32];
  __shared__ int total_s;
  if (w0 < kDecodeMaxBlocks / 32) {
    wprefix[w0] = incl - c0 - c1;
    wprefix[w0 + 1] = incl - c1;
  }
  if (tid == 255) total_s = incl;
  __syncthreads();
  for (int e = tid; e < g * topk; e += 256) {
    const int hh = e / topk, s = e % topk;
    const int32_t v = srow[hh * kDecodeMaxTopk + s];
    if (v >= 0) {
      const int r = wprefix[v >> 5] + __builtin_popcount(bits[v >> 5] & ((1u << (v & 31)) - 1u));
      a.uni[z * a.U + r] = v;  // several heads may write the same value
      a.uslot[(z * a.U + r) * g + hh] = s;
    }
  }
  if (tid == 0) a.ucount[z] = total_s;
}

// ---------------------------------------------------------------------------
// Attention over one chunk (kDecodeChunk keys) of one union block for the
// heads of the group that chose it.  grid (batch * hkv, nchunk, U), 256
// threads.  The chunk is streamed in 64-key steps: step s + 1 is loaded into
// registers while step s is computed from LDS; an online softmax per head
// carries (max, sum, o) across steps.  When the block is the own block and
// the new token completes it, the work-group also writes the column sums of
// its keys, from which the merge forms the block's mean.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  constexpr int SUB = 64;                 // keys per step: one per lane
  constexpr int RB = D * (int)sizeof(T);  // bytes per cached row
  constexpr int RBK = RB + 16;            // K rows padded: conflict-free 16-byte row reads
  constexpr int UPR = RB / 16;            // 16-byte units per row
  constexpr int UPT = SUB * UPR / 256;    // units per thread and step, per tensor
  constexpr int NP = D / 2;               // dim pairs per head
  constexpr int PPT = kDecodeMaxGroup * NP / 256;  // (head, dim pair) slots per thread
  constexpr int CPT = 256 / D;            // threads per column of the key sums
  static_assert(UPT >= 1 && PPT >= 1 && CPT >= 1, "tile shape");
  static_assert(kDecodeChunk % SUB == 0, "whole steps per chunk");
  __shared__ __attribute__((aligned(16))) char ks[SUB * RBK];
  __shared__ __attribute__((aligned(16))) char vs[SUB * RB];
  __shared__ __attribute__((aligned(16))) float qs[kDecodeMaxGroup * D];
  __shared__ float ps[kDecodeMaxGroup * SUB];
  __shared__ float alpha_s[kDecodeMaxGroup];
  __shared__ float csum_s[256];
  __shared__ int hlist[kDecodeMaxGroup], hslot[kDecodeMaxGroup];
  __shared__ int nh_s;
  const int64_t z = blockIdx.x;
  const int c = blockIdx.y, u = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bb = z / a.hkv;
  const int hk = (int)(z % a.hkv);
  const int g = a.g;
  // independent loads first (u < U keeps uni in bounds even for an entry
  // past the union, whose value is then unused)
  const int ucount = a.ucount[z];
  const int64_t i = a.uni[z * a.U + u];
  const int64_t L = a.lens[bb];  // valid: ucount is 0 otherwise
  const int sl = (tid < g) ? a.uslot[(z * a.U + u) * g + tid] : -1;
  if (u >= ucount) return;  // uniform over the work-group
  const int64_t j = (L - 1) / a.block;
  const int64_t kend = (i == j) ? L : (i + 1) * a.block;
  const int64_t k0 = i * a.block + (int64_t)c * kDecodeChunk;
  const int nk = (int)(kend - k0 < kDecodeChunk ? kend - k0 : kDecodeChunk);
  if (nk <= 0) return;  // past the end of the block (or of the own block's keys)
  const int nsteps = (nk + SUB - 1) / SUB;
  const bool do_sum = (i == j) && (L % a.block == 0);

  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  u32x4 rk[UPT], rv[UPT];
  // rows past the chunk's end re-read its last row (kept in bounds and
  // branch-free, so the loads of a step issue back to back); they are not
  // stored
  auto load_step = [&](int s) {
    const int base = s * SUB;
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int e = tid + 256 * x, r = e / UPR, uo = e % UPR;
      const int rr = base + r < nk ? base + r : nk - 1;
      const int64_t off = ((bb * a.lmax + k0 + rr) * a.hkv + hk) * (int64_t)RB + uo * 16;
      rk[x] = *reinterpret_cast<const u32x4*>(kb + off);
      rv[x] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  };
  load_step(0);

  // the heads of the group that chose block i, compacted
  if (wave == 0) {
    const int s = sl;
    const uint64_t mask = __ballot(s >= 0);
    if (s >= 0) {
      const int r = __builtin_popcountll(mask & ((1ull << lane) - 1ull));
      hlist[r] = lane;
      hslot[r] = s;
    }
    if (lane == 0) nh_s = __builtin_popcountll(mask);
  }
  __syncthreads();
  const int nh = nh_s;
  const int64_t hq0 = bb * a.hq + (int64_t)hk * g;
  for (int e = tid; e < nh * D; e += 256)
    qs[e] = load_f32(reinterpret_cast<const T*>(a.q) + (hq0 + hlist[e / D]) * D + e % D) * a.scale_log2;

  float m_h[4], l_h[4];  // per head of this wave (heads wave, wave + 4, ...)
#pragma unroll
  for (int x = 0; x < 4; ++x) { m_h[x] = -__builtin_inff(); l_h[x] = 0.f; }
  float o0[PPT], o1[PPT];
#pragma unroll
  for (int x = 0; x < PPT; ++x) { o0[x] = 0.f; o1[x] = 0.f; }
  float csum = 0.f;

  for (int s = 0; s < nsteps; ++s) {
    const int nks = nk - s * SUB < SUB ? nk - s * SUB : SUB;
    __syncthreads();  // the previous step's LDS reads are done
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int e = tid + 256 * x, r = e / UPR, uo = e % UPR;
      if (r < nks) {
        *reinterpret_cast<u32x4*>(ks + r * RBK + uo * 16) = rk[x];
        *reinterpret_cast<u32x4*>(vs + r * RB + uo * 16) = rv[x];
      }
    }
    if (s + 1 < nsteps) load_step(s + 1);
    __syncthreads();

    // scores (lane = key, wave = head) and the online softmax update
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int hx = wave + 4 * x;
      if (hx < nh) {
        float sc = -__builtin_inff();
        if (lane < nks) {
          const char* kr = ks + lane * RBK;
          const float* qh = qs + hx * D;
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int d0 = 0; d0 < D; d0 += 8) {
            float kv[8];
            load8(reinterpret_cast<const T*>(kr) + d0, kv);
            const f32x4 qa = *reinterpret_cast<const f32x4*>(qh + d0);
            const f32x4 qb = *reinterpret_cast<const f32x4*>(qh + d0 + 4);
            s0 = __builtin_fmaf(qa[0], kv[0], s0);
            s1 = __builtin_fmaf(qa[1], kv[1], s1);
            s0 = __builtin_fmaf(qa[2], kv[2], s0);
            s1 = __builtin_fmaf(qa[3], kv[3], s1);
            s0 = __builtin_fmaf(qb[0], kv[4], s0);
            s1 = __builtin_fmaf(qb[1], kv[5], s1);
            s0 = __builtin_fmaf(qb[2], kv[6], s0);
            s1 = __builtin_fmaf(qb[3], kv[7], s1);
          }
          sc = s0 + s1;
        }
        const float mnew = __builtin_fmaxf(m_h[x], wave_max_f(sc));
        const float al = fast_exp2(m_h[x] - mnew);  // 0 on the first step
        const float p = lane < nks ? fast_exp2(sc - mnew) : 0.f;
        l_h[x] = l_h[x] * al + wave_sum_f(p);
        m_h[x] = mnew;
        ps[hx * SUB + lane] = p;
        if (lane == 0) alpha_s[hx] = al;
      }
    }
    if (do_sum) {
      // column sums of this step's keys: CPT threads per column
      const int col = tid % D, part = tid / D;
      for (int r = part; r < nks; r += CPT) csum += load_f32(reinterpret_cast<const T*>(ks + r * RBK) + col);
    }
    __syncthreads();

    // o = o * alpha + sum_x p_x v_x  (slot = head, dim pair)
#pragma unroll
    for (int x = 0; x < PPT; ++x) {
      const int e = tid + 256 * x;
      const int hx = e / NP, dp = e % NP;
      if (hx < nh) {
        const float al = alpha_s[hx];
        float a0 = o0[x] * al, a1 = o1[x] * al;
        const float* ph = ps + hx * SUB;
        for (int r = 0; r < nks; ++r) {
          float v0, v1;
          load2(reinterpret_cast<const T*>(vs + r * RB) + 2 * dp, v0, v1);
          a0 = __builtin_fmaf(ph[r], v0, a0);
          a1 = __builtin_fmaf(ph[r], v1, a1);
        }
        o0[x] = a0;
        o1[x] = a1;
      }
    }
  }

  // partials: o relative to the head's running max, the max (base 2) and the sum
#pragma unroll
  for (int x = 0; x < PPT; ++x) {
    const int e = tid + 256 * x;
    const int hx = e / NP, dp = e % NP;
    if (hx < nh) {
      const int64_t pidx = ((hq0 + hlist[hx]) * a.topk + hslot[hx]) * a.nchunk + c;
      store2(a.po + pidx * D + 2 * dp, o0[x], o1[x]);
    }
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int hx = wave + 4 * x;
    if (hx < nh && lane == 0) {
      const int64_t pidx = ((hq0 + hlist[hx]) * a.topk + hslot[hx]) * a.nchunk + c;
      store2(a.pml + pidx * 2, m_h[x], l_h[x]);
    }
  }
  if (do_sum) {
    csum_s[tid] = csum;
    __syncthreads();
    if (tid < D) {
      float t = 0.f;
      for (int p = 0; p < CPT; ++p) t += csum_s[p * D + tid];
      a.ksum[(z * a.nchunk + c) * D + tid] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of a head's partials (one pass, online rescaling).  grid (hq,
// batch), 64 threads (two dims each).  The group's first head also turns the
// key sums of a just-completed own block into its cached mean.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int64_t bb = blockIdx.y;
  const int lane = threadIdx.x;
  const bool act = 2 * lane < D;
  const int64_t row = bb * a.hq + h;
  T* out = reinterpret_cast<T*>(a.out) + row * D;
  const int64_t L = a.lens[bb];
  if (!len_ok(L, a.lmax)) {
    if (act) store2(out + 2 * lane, 0.f, 0.f);
    return;
  }
  const int64_t j = (L - 1) / a.block;
  const int32_t* sel = a.sel + row * a.topk;
  float m = -__builtin_inff(), l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < a.topk; ++s) {
    const int64_t i = sel[s];
    if (i < 0) continue;
    const int64_t len = ((i == j) ? L : (i + 1) * a.block) - i * a.block;
    const int nc = (int)((len + kDecodeChunk - 1) / kDecodeChunk);
    const int64_t p0 = (row * a.topk + s) * a.nchunk;
#pragma unroll 4
    for (int c = 0; c < nc; ++c) {
      const float2 ml = *reinterpret_cast<const float2*>(a.pml + (p0 + c) * 2);
      float2 po = float2{0.f, 0.f};
      if (act) po = *reinterpret_cast<const float2*>(a.po + (p0 + c) * D + 2 * lane);
      const float mn = __builtin_fmaxf(m, ml.x);
      const float wa = fast_exp2(m - mn), wb = fast_exp2(ml.x - mn);
      l = l * wa + ml.y * wb;
      o0 = o0 * wa + po.x * wb;
      o1 = o1 * wa + po.y * wb;
      m = mn;
    }
  }
  const float inv = 1.f / l;
  if (act) store2(out + 2 * lane, o0 * inv, o1 * inv);

  // the block this token completes joins the cached means
  const int hk = h / a.g;
  if (h % a.g == 0 && L % a.block == 0 && act) {
    const int nc = (int)((a.block + kDecodeChunk - 1) / kDecodeChunk);
    const int64_t z = bb * a.hkv + hk;
    float s0 = 0.f, s1 = 0.f;
    for (int c = 0; c < nc; ++c) {
      const float2 t = *reinterpret_cast<const float2*>(a.ksum + (z * a.nchunk + c) * D + 2 * lane);
      s0 += t.x;
      s1 += t.y;
    }
    const float inv_b = 1.f / (float)a.block;
    store2(a.mu + ((bb * a.hkv + hk) * a.nmax + j) * D + 2 * lane, s0 * inv_b, s1 * inv_b);
  }
}

// ---------------------------------------------------------------------------
// Block means of the cache: block blockIdx.x if it is complete.  grid
// (blocks, hkv, batch), 256 threads.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_means_kernel(const T* __restrict__ k, const int32_t* __restrict__ lens,
                                                           float* __restrict__ mu, int64_t lmax, int64_t nmax,
                                                           int hkv, int block) {
  constexpr int CU = D / 8;        // 8-dim units per row
  constexpr int R = 256 / CU;      // row groups
  __shared__ float red[256 * 8];
  const int hk = blockIdx.y;
  const int64_t bb = blockIdx.z;
  const int64_t L = lens[bb];
  if (!len_ok(L, lmax)) return;
  const int64_t i = blockIdx.x;
  if (i >= L / block) return;
  const int tid = threadIdx.x, cu = tid % CU, rg = tid / CU;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const T* base = k + ((bb * lmax + i * block) * hkv + hk) * (int64_t)D + cu * 8;
  for (int x = rg; x < block; x += R) {
    float kv[8];
    load8(base + (int64_t)x * hkv * D, kv);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += kv[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tid * 8 + e] = acc[e];
  __syncthreads();
  if (rg == 0) {
    for (int r = 1; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += red[(r * CU + cu) * 8 + e];
    float* dst = mu + ((bb * hkv + hk) * nmax + i) * D + cu * 8;
    const float inv = 1.f / (float)block;
    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D>
static void decode_launch_all(const DecodeArgs& a, hipStream_t st, int stage) {
  if (stage == 0)
    hipLaunchKernelGGL((decode_gate_kernel<T, D>), dim3((unsigned)a.hkv, (unsigned)a.batch), dim3(256), 0, st, a);
  else if (stage == 1)
    hipLaunchKernelGGL((decode_attn_kernel<T, D>), dim3((unsigned)(a.batch * a.hkv), (unsigned)a.nchunk, (unsigned)a.U),
                       dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)a.hq, (unsigned)a.batch), dim3(64), 0, st, a);
}

int launch_decode_stage(const DecodeArgs& a, int dtype, int stage, hipStream_t st) {
  if (dtype == 1)
    decode_launch_all<bf16raw, 128>(a, st, stage);
  else if (a.d == 64)
    decode_launch_all<float, 64>(a, st, stage);
  else
    decode_launch_all<float, 128>(a, st, stage);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_decode_means(const void* k, const int32_t* lens, float* mu, int dtype, int64_t batch, int64_t lmax,
                        int64_t nmax, int hkv, int d, int block, hipStream_t st) {
  const dim3 grid((unsigned)nmax, (unsigned)hkv, (unsigned)batch);
  if (dtype == 1)
    hipLaunchKernelGGL((decode_means_kernel<bf16raw, 128>), grid, dim3(256), 0, st, (const bf16raw*)k, lens, mu, lmax,
                       nmax, hkv, block);
  else if (d == 64)
    hipLaunchKernelGGL((decode_means_kernel<float, 64>), grid, dim3(256), 0, st, (const float*)k, lens, mu, lmax, nmax,
                       hkv, block);
  else
    hipLaunchKernelGGL((decode_means_kernel<float, 128>), grid, dim3(256), 0, st, (const float*)k, lens, mu, lmax,
                       nmax, hkv, block);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
