// MoBA gate (deep-dive report on MoBA, sections 2.2 and 2.3): fp32 scores
// s_i = <q, mu_i>, exclusion of future blocks, the forced own block, and a
// hard top-k with ties broken towards the lower block index.  Every form
// below chooses exactly the same set.
//
// gate_kernel (VALU; fp32 inputs and the stand-alone gate): one work-group
// handles `gate_t` consecutive query positions of one KV head and all query
// heads of its group (one row per thread), so the block means of that KV
// head are staged once in LDS (in slices of kMuSlice blocks) and read by
// every row with broadcast loads.  Each thread keeps its running top-m list
// in registers as 64-bit keys (orderable score << 32 | ~index): a larger key
// is a larger score, and between equal scores the lower block index, which
// is exactly the tie rule.  gate_rounds_kernel takes over when m exceeds
// one list of 32 (the cut-off score found in rounds, RoundState).
//
// gate_mfma_kernel (bf16 inputs): the scores on the matrix cores, the choice
// in one pass for short lists, in two passes (the m-th largest score, then
// the blocks above it and the lowest-index ties at it) for longer ones, and
// in rounds beyond 32.
//
// Besides sel_idx the kernels write, per work-group, how many of its rows
// chose each block (used to build the per-block row lists), stored as
// [KV head, block, work-group] so that each list's counts are contiguous;
// with more blocks than the dispatch's LDS counters hold the caller passes no
// count table and the dispatch counts the rows from sel_idx instead.
#include "moba_device.h"
#include "moba_kernels.h"
#include "moba_plan.h"

namespace moba {

constexpr int kMuSlice = 32;  // block means staged in LDS at a time

// fp32 score of one block for one row: q (registers) against the block's
// summary in LDS (D means, or D minima then D maxima); NaN ranks lowest.
template <int D, bool kMinMax>
__device__ __forceinline__ float gate_score(const float* qr, const float* mrow) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int d0 = 0; d0 < D; d0 += 4) {
    const f32x4 mv = *reinterpret_cast<const f32x4*>(mrow + d0);
    if constexpr (kMinMax) {
      // term d: max(q_d lo_d, q_d hi_d), each product rounded once (a per-d
      // select on the sign of q would keep 128 lane masks live across the
      // block loop)
      const f32x4 hv = *reinterpret_cast<const f32x4*>(mrow + D + d0);
      s0 += __builtin_fmaxf(qr[d0 + 0] * mv[0], qr[d0 + 0] * hv[0]);
      s1 += __builtin_fmaxf(qr[d0 + 1] * mv[1], qr[d0 + 1] * hv[1]);
      s2 += __builtin_fmaxf(qr[d0 + 2] * mv[2], qr[d0 + 2] * hv[2]);
      s3 += __builtin_fmaxf(qr[d0 + 3] * mv[3], qr[d0 + 3] * hv[3]);
    } else {
      s0 = __builtin_fmaf(qr[d0 + 0], mv[0], s0);
      s1 = __builtin_fmaf(qr[d0 + 1], mv[1], s1);
      s2 = __builtin_fmaf(qr[d0 + 2], mv[2], s2);
      s3 = __builtin_fmaf(qr[d0 + 3], mv[3], s3);
    }
  }
  float s = (s0 + s1) + (s2 + s3);
  if (s != s) s = -__builtin_inff();
  return s;
}

template <typename T, int D, int KCAP, bool kMinMax>
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
  // per block: D floats of the mean, or 2 D (min, then max) for min/max
  constexpr int SD = kMinMax ? 2 * D : D;
  extern __shared__ float smem[];
  float* mu_s = smem;                                       // [kMuSlice][SD]
  int* lhist = reinterpret_cast<int*>(smem + kMuSlice * SD);  // [n]
  const int tid = threadIdx.x;
  const int64_t w = blockIdx.x;
  const int hk = blockIdx.y;
  const int64_t n = a.n;
  const int g = a.g;

  if (a.hist)
    for (int64_t i = tid; i < n; i += 256) lhist[i] = 0;

  const int64_t pic = w * a.gate_t + tid / g;  // position inside the chunk
  const int h = hk * g + tid % g;
  const bool valid = tid < a.gate_t * g && pic < a.cnt;
  const int64_t t = a.t0 + pic;
  const int64_t j = t / a.block;
  const int64_t ncand = a.causal ? j : n;
  const int m = (int)(a.causal ? (j < a.kp ? j : a.kp) : a.kp);
  const bool rank = valid && m > 0 && (int64_t)m < ncand;

  // candidates any row of this work-group may have to score
  const int64_t last_pic = (w * a.gate_t + a.gate_t < a.cnt ? w * a.gate_t + a.gate_t : a.cnt) - 1;
  const int64_t wg_cand = a.causal ? (a.t0 + last_pic) / a.block : n;

  float qr[D];
  uint64_t ks[KCAP];
#pragma unroll
  for (int p = 0; p < KCAP; ++p) ks[p] = (p < KCAP - m) ? ~0ull : 0ull;

  const int any_rank = __syncthreads_or(rank ? 1 : 0);
  if (any_rank) {
    if (rank) {
      const T* qp = reinterpret_cast<const T*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * (int64_t)D;
#pragma unroll
      for (int d0 = 0; d0 < D; d0 += 8) load8(qp + d0, qr + d0);
    }
    const float* mu_h = (kMinMax ? a.lohi : a.mu) + ((int64_t)a.bb * a.hkv + hk) * n * SD;
    for (int64_t c0 = 0; c0 < wg_cand; c0 += kMuSlice) {
      const int64_t c1 = (c0 + kMuSlice < wg_cand) ? c0 + kMuSlice : wg_cand;
      __syncthreads();
      const int nel = (int)(c1 - c0) * SD;
      for (int e = tid * 4; e < nel; e += 256 * 4)
        *reinterpret_cast<f32x4*>(mu_s + e) = *reinterpret_cast<const f32x4*>(mu_h + c0 * SD + e);
      __syncthreads();
      if (rank) {
        const int64_t cend = ncand < c1 ? ncand : c1;
        for (int64_t i = c0; i < cend; ++i) {
          const float s = gate_score<D, kMinMax>(qr, mu_s + (i - c0) * SD);
          const uint64_t key = ((uint64_t)orderable(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
          if (key > ks[KCAP - 1]) {
            ks[KCAP - 1] = key;
#pragma unroll
            for (int p = KCAP - 1; p > 0; --p) {
              const uint64_t lo = ks[p], hi = ks[p - 1];
              const bool sw = lo > hi;
              ks[p] = sw ? hi : lo;
              ks[p - 1] = sw ? lo : hi;
            }
          }
        }
      }
    }
  }

  if (valid) {
    int32_t* row = a.sel + (int64_t)h * a.sel_stride_h + (t - a.sel_pos_base) * a.topk;
    int c = 0;
    if (rank) {
      // the m kept blocks sit in ks[KCAP-m .. KCAP-1]; emit them ascending
      uint32_t idx[KCAP];
#pragma unroll
      for (int p = 0; p < KCAP; ++p)
        idx[p] = (p >= KCAP - m) ? (0xffffffffu - (uint32_t)ks[p]) : 0xffffffffu;
#pragma unroll
      for (int pass = 0; pass < KCAP; ++pass) {
#pragma unroll
        for (int p = pass & 1; p + 1 < KCAP; p += 2) {
          const uint32_t x = idx[p], y = idx[p + 1];
          idx[p] = x < y ? x : y;
          idx[p + 1] = x < y ? y : x;
        }
      }
#pragma unroll
      for (int p = 0; p < KCAP; ++p) {
        if (p < m) {
          row[c++] = (int32_t)idx[p];
          if (a.hist) atomicAdd(&lhist[idx[p]], 1);
        }
      }
    } else if ((int64_t)m >= ncand) {
      // no more candidates than slots: every candidate is chosen
      for (int64_t i = 0; i < ncand; ++i) {
        row[c++] = (int32_t)i;
        if (a.hist) atomicAdd(&lhist[i], 1);
      }
    }
    if (a.causal) row[c++] = (int32_t)j;  // the own block, always kept
    for (; c < a.topk; ++c) row[c] = -1;
  }

  if (a.hist) {
    __syncthreads();
    int32_t* dst = a.hist + (int64_t)hk * n * a.gate_wg + w;  // [hkv, n, gate_wg]
    for (int64_t i = tid; i < n; i += 256) dst[i * a.gate_wg] = lhist[i];
  }
}

// ---------------------------------------------------------------------------
// bf16 path: scores on the matrix cores.
//
// Each fp32 block mean is split into three bf16 parts hi + mid + lo that add
// up to it exactly (hi = bf16(mu), mid = bf16(mu - hi), lo = mu - hi - mid,
// each step exact in fp32).  With bf16 queries every product q_d * part_d is
// exact in fp32, so <q, mu> = sum over the three parts of the MFMA dot
// products, accumulated in fp32: the same fp32 rounding model as the plain
// dot product over 3 D terms.
//
// Split means are stored per tile of 32 blocks as the LDS operand image
// [part][16-byte unit u of 8 d][block] (unit-major, so the 32 lanes that read
// 32 blocks of one unit hit every bank once), 24 KiB per tile.
// ---------------------------------------------------------------------------
constexpr int kMu3TileElems = 3 * 16 * kGateTile * 8;  // bf16 per tile image
static_assert(16 * kGateTile * 8 == 512 * 8, "the MFMA gate stages one part per 512 threads x 8 bf16");

__global__ __launch_bounds__(256) void mu_split_kernel(const float* __restrict__ mu, int64_t n, int hkv,
                                                       uint16_t* __restrict__ mu3) {
  const int64_t tile = blockIdx.x;
  const int hk = blockIdx.y;
  const int64_t bb = blockIdx.z;
  const int64_t ntile = (n + kGateTile - 1) / kGateTile;
  const float* src = mu + (bb * hkv + hk) * n * 128;
  uint16_t* dst = mu3 + ((bb * hkv + hk) * ntile + tile) * kMu3TileElems;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int pair = threadIdx.x + 256 * x;  // (unit, block) of the tile
    const int u = pair >> 5, blk = pair & 31;
    const int64_t i = tile * kGateTile + blk;
    float v[8];
    if (i < n) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(src + i * 128 + u * 8);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + i * 128 + u * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    uint32_t w[3][4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t h2 = pack_bf16x2(v[e], v[e + 1]);
      const float r0 = v[e] - bf16lo(h2), r1 = v[e + 1] - bf16hi(h2);
      const uint32_t m2 = pack_bf16x2(r0, r1);
      const uint32_t l2 = pack_bf16x2(r0 - bf16lo(m2), r1 - bf16hi(m2));
      w[0][e >> 1] = h2;
      w[1][e >> 1] = m2;
      w[2][e >> 1] = l2;
    }
#pragma unroll
    for (int part = 0; part < 3; ++part)
      *reinterpret_cast<u32x4*>(dst + ((part * 16 + u) * kGateTile + blk) * 8) =
          u32x4{w[part][0], w[part][1], w[part][2], w[part][3]};
  }
}

// Min/max gate on the matrix cores: max(q_d lo_d, q_d hi_d) = q+_d hi_d +
// q-_d lo_d with q+ = max(q, 0) and q- = min(q, 0), both exact in bf16; with
// bf16 keys, lo and hi are bf16 values, so the score is two exact-product
// dot products (2 D terms) accumulated in fp32.  Images as above with two
// parts: part 0 = hi (paired with q+), part 1 = lo (paired with q-).
__global__ __launch_bounds__(256) void mm_split_kernel(const float* __restrict__ lohi, int64_t n, int hkv,
                                                       uint16_t* __restrict__ mu3) {
  const int64_t tile = blockIdx.x;
  const int hk = blockIdx.y;
  const int64_t bb = blockIdx.z;
  const int64_t ntile = (n + kGateTile - 1) / kGateTile;
  const float* src = lohi + (bb * hkv + hk) * n * 256;
  uint16_t* dst = mu3 + ((bb * hkv + hk) * ntile + tile) * kMu3TileElems;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int pair = threadIdx.x + 256 * x;  // (unit, block) of the tile
    const int u = pair >> 5, blk = pair & 31;
    const int64_t i = tile * kGateTile + blk;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (i < n) {
        const float* row = src + i * 256 + (part == 0 ? 128 : 0) + u * 8;
        const f32x4 a = *reinterpret_cast<const f32x4*>(row);
        const f32x4 b = *reinterpret_cast<const f32x4*>(row + 4);
        w[0] = pack_bf16x2(a[0], a[1]);
        w[1] = pack_bf16x2(a[2], a[3]);
        w[2] = pack_bf16x2(b[0], b[1]);
        w[3] = pack_bf16x2(b[2], b[3]);
      }
      *reinterpret_cast<u32x4*>(dst + ((part * 16 + u) * kGateTile + blk) * 8) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

// q+ and q- of eight packed bf16: q+ keeps the halves whose sign bit is
// clear, q- those whose sign bit is set (the other halves become +0).
__device__ __forceinline__ void sign_split(u32x4 w, bf16x8& pos, bf16x8& neg) {
  u32x4 p, n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = ((w[i] >> 15) & 0x00010001u) * 0xffffu;  // 0xffff in each negative half
    n[i] = w[i] & m;
    p[i] = w[i] ^ n[i];
  }
  pos = __builtin_bit_cast(bf16x8, p);
  neg = __builtin_bit_cast(bf16x8, n);
}

// A value and the one lane l ^ 32 holds (v_permlane32_swap with both inputs
// the same value: lane l < 32 gets (x[l], x[l + 32]), lane l >= 32 gets
// (x[l - 32], x[l])); the two results are copied to scalars first.
__device__ __forceinline__ void pair_values_u(uint32_t x, uint32_t& u, uint32_t& v) {
  const auto pr = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const uint32_t r0 = pr[0], r1 = pr[1];
  u = r0;
  v = r1;
}
__device__ __forceinline__ void pair_values_f(float x, float& u, float& v) {
  uint32_t a, b;
  pair_values_u(__builtin_bit_cast(uint32_t, x), a, b);
  u = __builtin_bit_cast(float, a);
  v = __builtin_bit_cast(float, b);
}

// Insert a 64-bit key into a descending top list (ks[0] largest).
template <int KCAP>
__device__ __forceinline__ void topk_insert(uint64_t* ks, uint64_t key) {
  if (key > ks[KCAP - 1]) {
    ks[KCAP - 1] = key;
#pragma unroll
    for (int p = KCAP - 1; p > 0; --p) {
      const uint64_t lo = ks[p], hi = ks[p - 1];
      const bool sw = lo > hi;
      ks[p] = sw ? hi : lo;
      ks[p - 1] = sw ? lo : hi;
    }
  }
}

// The m-th largest of a row's candidate scores (m <= KCAP) and how many of
// them lie above it, from a descending list of the row's top KCAP scores.
template <int KCAP>
__device__ __forceinline__ void list_insert(float* tv, float x) {
  // tv sorted descending; with x inserted, entry p becomes the median of
  // (tv[p-1], tv[p], x) of the list before (x above tv[p-1]: tv[p-1]; x
  // between: x; x below tv[p]: tv[p]).  One v_med3_f32 per entry, from the
  // old values (highest index first, in place), and no chain between them.
#pragma unroll
  for (int p = KCAP - 1; p > 0; --p) tv[p] = __builtin_amdgcn_fmed3f(tv[p - 1], tv[p], x);
  tv[0] = __builtin_fmaxf(tv[0], x);
}

// Search for a row's m-th largest score T in rounds, for m beyond one list
// of KCAP.  Before a round, `acc` scores are known to lie above `hi` and the
// rest are not accounted for; the round lists the KCAP largest scores below
// `hi` (descending, -inf padded) and counts `eqc` scores equal to `hi`.  Then
// T is hi (when the acc + eqc scores at or above hi already reach m), or an
// entry of the list (when the rest of m fits in it), or the next round starts
// below the list's last entry.  `hi` falls strictly every round, so the
// search ends; it takes about m / KCAP rounds.  `above` is the number of
// scores above T.
struct RoundState {
  float hi;
  int acc;
  bool done;
  float thr;
  int above;
};
template <int KCAP>
__device__ __forceinline__ void round_update(RoundState& st, const float* tv, int eqc, int m) {
  if (st.done) return;
  const int at_or_above = st.acc + eqc;
  if (m <= at_or_above) {
    st.thr = st.hi;
    st.above = st.acc;
    st.done = true;
    return;
  }
  const int mp = m - at_or_above;  // still to find, below hi
  if (mp <= KCAP) {
    float thr = tv[0];
#pragma unroll
    for (int p = 1; p < KCAP; ++p)
      if (p < mp) thr = tv[p];
    int ab = at_or_above;
#pragma unroll
    for (int p = 0; p < KCAP; ++p)
      if (p < mp && tv[p] > thr) ++ab;
    st.thr = thr;
    st.above = ab;
    st.done = true;
  } else {
    const float hn = tv[KCAP - 1];
    int ab = at_or_above;
#pragma unroll
    for (int p = 0; p < KCAP; ++p)
      if (tv[p] > hn) ++ab;
    st.acc = ab;
    st.hi = hn;
  }
}

// Bits e (0..15) of a lane half's 16 scores of a 32-block score tile, placed
// at their block offsets inside the tile: score e of lane half lg is block
// 8 (e >> 2) + 4 lg + (e & 3).
__device__ __forceinline__ uint32_t spread_tile_bits(uint32_t m16, int lg) {
  const uint32_t x = (m16 & 0xfu) | ((m16 & 0xf0u) << 4) | ((m16 & 0xf00u) << 8) | ((m16 & 0xf000u) << 12);
  return x << (4 * lg);
}

// Lists of up to this many entries take the one-pass choice (a short 64-bit
// insertion list costs less than scoring every tile twice); longer lists take
// the two passes.
constexpr int kGateOnePassMaxKcap = 4;

// One work-group = 256 rows (gate_t positions x the group's heads of one KV
// head), 8 waves of 32 rows.  Per tile of 32 blocks a wave computes the
// 32 x 32 score tile S^T = Mu Q^T (24 MFMAs: 3 parts x 8 steps of 16 d);
// lane l then holds 16 of the 32 scores of row l % 32 (the other 16 are in
// lane l ^ 32).  The top-m choice is exact.  Short lists (KCAP at most
// kGateOnePassMaxKcap) keep 64-bit (score, index) keys in one pass; longer
// ones take two passes over the tiles:
//   1. every lane keeps the descending top-KCAP list of its scores (fp32
//      values only, one median-of-three per entry and score, no branch); the
//      two half-row lists are merged, and the row's m-th largest score T and
//      the number of its scores above T follow;
//   2. the tiles are scored again (the same MFMAs on the same operands give
//      the same fp32 scores) and a row keeps every block scoring above T and,
//      of those scoring exactly T, the lowest-index ones up to m: the tie
//      rule.  The kept blocks come out tile by tile in ascending order.
template <int KCAP, bool kMinMax, bool kRounds = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(KCAP <= 12 ? 4 : 1))) void gate_mfma_kernel(
    GateArgs a, const uint16_t* __restrict__ mu3) {
  constexpr int NPART = kMinMax ? 2 : 3;
  extern __shared__ __attribute__((aligned(16))) char gsm[];
  char* tbuf = gsm;                                          // 2 tile images
  int* lhist = reinterpret_cast<int*>(gsm + 2 * kMu3TileElems * 2);  // [n]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 5;
  const int64_t w = blockIdx.x;
  const int hk = blockIdx.y;
  const int64_t n = a.n;
  const int g = a.g;

  if (a.hist)
    for (int64_t i = tid; i < n; i += 512) lhist[i] = 0;

  const int r = wave * 32 + (lane & 31);
  const int64_t pic = w * a.gate_t + r / g;  // position inside the chunk
  const int h = hk * g + r % g;
  const bool valid = r < a.gate_t * g && pic < a.cnt;
  const int64_t t = a.t0 + (valid ? pic : 0);
  const int64_t j = t / a.block;
  const int64_t ncand = a.causal ? j : n;
  const int m = (int)(a.causal ? (j < a.kp ? j : a.kp) : a.kp);
  const bool rank = valid && m > 0 && (int64_t)m < ncand;

  const int64_t last_pic = (w * a.gate_t + a.gate_t < a.cnt ? w * a.gate_t + a.gate_t : a.cnt) - 1;
  const int64_t wg_cand = a.causal ? (a.t0 + last_pic) / a.block : n;
  const int64_t ntile = (n + kGateTile - 1) / kGateTile;
  const int64_t wg_tiles = (wg_cand + kGateTile - 1) / kGateTile;

  int32_t* row = a.sel + (int64_t)h * a.sel_stride_h + (t - a.sel_pos_base) * a.topk;
  int nout = 0;  // entries written to the row so far

  const int any_rank = __syncthreads_or(rank ? 1 : 0);
  if (any_rank) {
    bf16x8 qb[8];
    {
      const bf16raw* qp = reinterpret_cast<const bf16raw*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * 128;
#pragma unroll
      for (int s = 0; s < 8; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qp + lg * 8 + 16 * s);
    }
    const uint16_t* mt = mu3 + ((int64_t)a.bb * a.hkv + hk) * ntile * kMu3TileElems;
    const int aofs = (lg * 32 + (lane & 31)) * 16;  // this lane's A-operand unit (part 0, step 0)
    // one 16-byte unit per thread and part (512 threads x 8 bf16 = one part)
    u32x4 stg[NPART];
    auto load_tile = [&](int64_t c) {
#pragma unroll
      for (int x = 0; x < NPART; ++x)
        stg[x] = *reinterpret_cast<const u32x4*>(mt + c * kMu3TileElems + (tid + 512 * x) * 8);
    };
    auto store_tile = [&](char* dst) {
#pragma unroll
      for (int x = 0; x < NPART; ++x) *reinterpret_cast<u32x4*>(dst + (tid + 512 * x) * 16) = stg[x];
    };
    // this lane's 16 scores of tile c (LDS image cur), NaN ranked lowest
    auto score_tile = [&](const char* cur, float* sc) {
      f32x16 s0, s1;
#pragma unroll
      for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
      if constexpr (kMinMax) {
        // B operands q+ (with hi, part 0) and q- (with lo, part 1), formed
        // from q per tile: the opaque copy keeps the compiler from holding
        // all 16 of them live across the loop
#pragma unroll
        for (int st = 0; st < 8; st += 2) {
          u32x4 w0 = __builtin_bit_cast(u32x4, qb[st]), w1 = __builtin_bit_cast(u32x4, qb[st + 1]);
          asm volatile("" : "+v"(w0));
          asm volatile("" : "+v"(w1));
          bf16x8 p0, n0, p1, n1;
          sign_split(w0, p0, n0);
          sign_split(w1, p1, n1);
          const bf16x8 h0 = *reinterpret_cast<const bf16x8*>(cur + aofs + (2 * st) * 512);
          const bf16x8 h1 = *reinterpret_cast<const bf16x8*>(cur + aofs + (2 * st + 2) * 512);
          const bf16x8 l0 = *reinterpret_cast<const bf16x8*>(cur + aofs + (16 + 2 * st) * 512);
          const bf16x8 l1 = *reinterpret_cast<const bf16x8*>(cur + aofs + (16 + 2 * st + 2) * 512);
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h0, p0, s0, 0, 0, 0);
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h1, p1, s0, 0, 0, 0);
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l0, n0, s0, 0, 0, 0);
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l1, n1, s0, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int part = 0; part < NPART; ++part)
#pragma unroll
          for (int st = 0; st < 8; st += 2) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(cur + aofs + (part * 16 + 2 * st) * 512);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(cur + aofs + (part * 16 + 2 * st + 2) * 512);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[st], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[st + 1], s1, 0, 0, 0);
          }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = kMinMax ? s0[e] : s0[e] + s1[e];
        sc[e] = v != v ? -__builtin_inff() : v;
      }
    };
    // every tile of the work-group's candidates through LDS (double-buffered,
    // the next tile's loads in flight), `body(c, image)` on each
    auto for_each_tile = [&](auto&& body) {
      load_tile(0);
      store_tile(tbuf);
      __syncthreads();
      for (int64_t c = 0; c < wg_tiles; ++c) {
        char* cur = tbuf + (c & 1) * (kMu3TileElems * 2);
        if (c + 1 < wg_tiles) load_tile(c + 1);
        // the MFMAs run on the whole wave (wave-uniform branch)
        if (__any(rank && c * kGateTile < ncand)) body(c, cur);
        if (c + 1 < wg_tiles) store_tile(tbuf + ((c + 1) & 1) * (kMu3TileElems * 2));
        __syncthreads();
      }
    };
    auto is_cand = [&](int64_t c, int e) {
      const int64_t i = c * kGateTile + 8 * (e >> 2) + 4 * lg + (e & 3);
      return rank && i < ncand;
    };

    if constexpr (KCAP <= kGateOnePassMaxKcap) {
      // one pass: each lane keeps its top-KCAP 64-bit keys (orderable score
      // bits, then the complemented index, so equal scores rank the lower
      // index higher); the partner's list is merged in and the m kept
      // indices are emitted ascending
      uint64_t ks[KCAP];
#pragma unroll
      for (int p = 0; p < KCAP; ++p) ks[p] = (p < KCAP - m) ? ~0ull : 0ull;
      for_each_tile([&](int64_t c, const char* cur) {
        float sc[16];
        score_tile(cur, sc);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t i = c * kGateTile + 8 * (e >> 2) + 4 * lg + (e & 3);
          const uint64_t key = ((uint64_t)orderable(sc[e]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
          if (is_cand(c, e)) topk_insert<KCAP>(ks, key);
        }
      });
      uint64_t pk_[KCAP];
#pragma unroll
      for (int p = 0; p < KCAP; ++p) {
        uint32_t l0, l1, h0, h1;
        pair_values_u((uint32_t)ks[p], l0, l1);
        pair_values_u((uint32_t)(ks[p] >> 32), h0, h1);
        pk_[p] = lg ? (((uint64_t)h0 << 32) | l0) : (((uint64_t)h1 << 32) | l1);
      }
#pragma unroll
      for (int p = 0; p < KCAP; ++p)
        if (rank && p >= KCAP - m) topk_insert<KCAP>(ks, pk_[p]);
      if (rank && lg == 0) {
        uint32_t idx[KCAP];
#pragma unroll
        for (int p = 0; p < KCAP; ++p)
          idx[p] = (p >= KCAP - m) ? (0xffffffffu - (uint32_t)ks[p]) : 0xffffffffu;
#pragma unroll
        for (int pass = 0; pass < KCAP; ++pass) {
#pragma unroll
          for (int p = pass & 1; p + 1 < KCAP; p += 2) {
            const uint32_t x = idx[p], y = idx[p + 1];
            idx[p] = x < y ? x : y;
            idx[p + 1] = x < y ? y : x;
          }
        }
#pragma unroll
        for (int p = 0; p < KCAP; ++p) {
          if (p < m) {
            row[nout++] = (int32_t)idx[p];
            if (a.hist) atomicAdd(&lhist[idx[p]], 1);
          }
        }
      }
    } else {
      float thr;
      int above;
      if constexpr (!kRounds) {
        // pass 1: the row's m-th largest score
        float tv[KCAP];
#pragma unroll
        for (int p = 0; p < KCAP; ++p) tv[p] = -__builtin_inff();
        for_each_tile([&](int64_t c, const char* cur) {
          float sc[16];
          score_tile(cur, sc);
#pragma unroll
          for (int e = 0; e < 16; ++e) list_insert<KCAP>(tv, is_cand(c, e) ? sc[e] : -__builtin_inff());
        });
        {
          // merge the partner lane's list (lane l ^ 32 holds the row's other half)
          float pv[KCAP];
#pragma unroll
          for (int p = 0; p < KCAP; ++p) {
            float u, v;
            pair_values_f(tv[p], u, v);
            pv[p] = lg ? u : v;
          }
#pragma unroll
          for (int p = 0; p < KCAP; ++p) list_insert<KCAP>(tv, pv[p]);
        }
        thr = tv[0];
        above = 0;
#pragma unroll
        for (int p = 1; p < KCAP; ++p)
          if (p < m) thr = tv[p];
#pragma unroll
        for (int p = 0; p < KCAP; ++p)
          if (p < m && tv[p] > thr) ++above;
      } else {
        // m may exceed the list: rounds over the tiles (RoundState), the
        // loop uniform over the work-group (each round streams the tiles)
        RoundState rs{__builtin_inff(), 0, !rank, 0.f, 0};
        while (__syncthreads_or(rs.done ? 0 : 1)) {
          float tv[KCAP];
#pragma unroll
          for (int p = 0; p < KCAP; ++p) tv[p] = -__builtin_inff();
          int eqc = 0;
          for_each_tile([&](int64_t c, const char* cur) {
            float sc[16];
            score_tile(cur, sc);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const bool cd = !rs.done && is_cand(c, e);
              list_insert<KCAP>(tv, (cd && sc[e] < rs.hi) ? sc[e] : -__builtin_inff());
              eqc += (cd && sc[e] == rs.hi) ? 1 : 0;
            }
          });
          float pv[KCAP];
#pragma unroll
          for (int p = 0; p < KCAP; ++p) {
            float u, v;
            pair_values_f(tv[p], u, v);
            pv[p] = lg ? u : v;
          }
#pragma unroll
          for (int p = 0; p < KCAP; ++p) list_insert<KCAP>(tv, pv[p]);
          uint32_t e0, e1;
          pair_values_u((uint32_t)eqc, e0, e1);
          round_update<KCAP>(rs, tv, (int)(e0 + e1), m);
        }
        thr = rs.thr;
        above = rs.above;
      }
      int ties_left = m - above;  // blocks scoring exactly thr still to keep, lowest index first

      // pass 2: the kept blocks, ascending
      for_each_tile([&](int64_t c, const char* cur) {
        float sc[16];
        score_tile(cur, sc);
        uint32_t gt = 0u, eq = 0u;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool cand = is_cand(c, e);
          gt |= (cand && sc[e] > thr) ? (1u << e) : 0u;
          eq |= (cand && sc[e] == thr) ? (1u << e) : 0u;
        }
        // the row's 32-block masks of this tile, the same in both lanes
        uint32_t gu, gw, eu, ew;
        pair_values_u(spread_tile_bits(gt, lg), gu, gw);
        pair_values_u(spread_tile_bits(eq, lg), eu, ew);
        uint32_t keep = gu | gw;
        uint32_t ties = eu | ew;
        while (ties && ties_left > 0) {
          const uint32_t b = ties & (0u - ties);
          keep |= b;
          ties ^= b;
          --ties_left;
        }
        if (rank && lg == 0) {
          while (keep) {
            const int b = __builtin_ctz(keep);
            keep &= keep - 1u;
            const int32_t idx = (int32_t)(c * kGateTile + b);
            row[nout++] = idx;
            if (a.hist) atomicAdd(&lhist[idx], 1);
          }
        }
      });
    }
  }

  if (valid && lg == 0) {
    int c = nout;
    if (!rank && (int64_t)m >= ncand) {
      for (int64_t i = 0; i < ncand; ++i) {
        row[c++] = (int32_t)i;
        if (a.hist) atomicAdd(&lhist[i], 1);
      }
    }
    if (a.causal) row[c++] = (int32_t)j;  // the own block, always kept
    for (; c < a.topk; ++c) row[c] = -1;
  }

  if (a.hist) {
    __syncthreads();
    int32_t* dst = a.hist + (int64_t)hk * n * a.gate_wg + w;  // [hkv, n, gate_wg]
    for (int64_t i = tid; i < n; i += 512) dst[i * a.gate_wg] = lhist[i];
  }
}

// VALU gate for a selective top-m beyond one register list (m > 32, any
// input dtype): one row per thread as in gate_kernel, the block summaries
// staged through LDS in slices.  The row's m-th largest score T is found in
// rounds (RoundState: each round a pass over the row's blocks listing the 32
// largest scores below the previous threshold and counting those equal to
// it); a last pass keeps, in ascending block order, every block scoring above
// T and the lowest-index blocks scoring exactly T up to m.  Every pass
// computes the same fp32 scores (gate_score), so the passes agree.
template <typename T, int D, bool kMinMax>
__global__ __launch_bounds__(256) void gate_rounds_kernel(GateArgs a) {
  constexpr int SD = kMinMax ? 2 * D : D;
  constexpr int KCAP = 32;
  extern __shared__ float smem[];
  float* mu_s = smem;                                       // [kMuSlice][SD]
  int* lhist = reinterpret_cast<int*>(smem + kMuSlice * SD);  // [n]
  const int tid = threadIdx.x;
  const int64_t w = blockIdx.x;
  const int hk = blockIdx.y;
  const int64_t n = a.n;
  const int g = a.g;

  if (a.hist)
    for (int64_t i = tid; i < n; i += 256) lhist[i] = 0;

  const int64_t pic = w * a.gate_t + tid / g;  // position inside the chunk
  const int h = hk * g + tid % g;
  const bool valid = tid < a.gate_t * g && pic < a.cnt;
  const int64_t t = a.t0 + (valid ? pic : 0);
  const int64_t j = t / a.block;
  const int64_t ncand = a.causal ? j : n;
  const int m = (int)(a.causal ? (j < a.kp ? j : a.kp) : a.kp);
  const bool rank = valid && m > 0 && (int64_t)m < ncand;

  const int64_t last_pic = (w * a.gate_t + a.gate_t < a.cnt ? w * a.gate_t + a.gate_t : a.cnt) - 1;
  const int64_t wg_cand = a.causal ? (a.t0 + last_pic) / a.block : n;

  int32_t* row = a.sel + (int64_t)h * a.sel_stride_h + (t - a.sel_pos_base) * a.topk;
  int nout = 0;

  const int any_rank = __syncthreads_or(rank ? 1 : 0);
  if (any_rank) {
    float qr[D];
    if (rank) {
      const T* qp = reinterpret_cast<const T*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * (int64_t)D;
#pragma unroll
      for (int d0 = 0; d0 < D; d0 += 8) load8(qp + d0, qr + d0);
    }
    const float* mu_h = (kMinMax ? a.lohi : a.mu) + ((int64_t)a.bb * a.hkv + hk) * n * SD;
    // one pass over the work-group's candidate blocks: body(i, score) for
    // each candidate of each ranking row, in ascending i
    auto scan = [&](auto&& body) {
      for (int64_t c0 = 0; c0 < wg_cand; c0 += kMuSlice) {
        const int64_t c1 = (c0 + kMuSlice < wg_cand) ? c0 + kMuSlice : wg_cand;
        __syncthreads();
        const int nel = (int)(c1 - c0) * SD;
        for (int e = tid * 4; e < nel; e += 256 * 4)
          *reinterpret_cast<f32x4*>(mu_s + e) = *reinterpret_cast<const f32x4*>(mu_h + c0 * SD + e);
        __syncthreads();
        if (rank) {
          const int64_t cend = ncand < c1 ? ncand : c1;
          for (int64_t i = c0; i < cend; ++i) body(i, gate_score<D, kMinMax>(qr, mu_s + (i - c0) * SD));
        }
      }
    };
    RoundState rs{__builtin_inff(), 0, !rank, 0.f, 0};
    while (__syncthreads_or(rs.done ? 0 : 1)) {
      float tv[KCAP];
#pragma unroll
      for (int p = 0; p < KCAP; ++p) tv[p] = -__builtin_inff();
      int eqc = 0;
      scan([&](int64_t, float x) {
        if (!rs.done) {
          list_insert<KCAP>(tv, x < rs.hi ? x : -__builtin_inff());
          eqc += x == rs.hi ? 1 : 0;
        }
      });
      round_update<KCAP>(rs, tv, eqc, m);
    }
    int ties_left = m - rs.above;  // blocks scoring exactly T still to keep, lowest index first
    scan([&](int64_t i, float x) {
      const bool tie = x == rs.thr && ties_left > 0;
      if (x > rs.thr || tie) {
        ties_left -= tie ? 1 : 0;
        row[nout++] = (int32_t)i;
        if (a.hist) atomicAdd(&lhist[i], 1);
      }
    });
  }

  if (valid) {
    int c = nout;
    if (!rank && (int64_t)m >= ncand) {
      // no more candidates than slots: every candidate is chosen
      for (int64_t i = 0; i < ncand; ++i) {
        row[c++] = (int32_t)i;
        if (a.hist) atomicAdd(&lhist[i], 1);
      }
    }
    if (a.causal) row[c++] = (int32_t)j;  // the own block, always kept
    for (; c < a.topk; ++c) row[c] = -1;
  }

  if (a.hist) {
    __syncthreads();
    int32_t* dst = a.hist + (int64_t)hk * n * a.gate_wg + w;  // [hkv, n, gate_wg]
    for (int64_t i = tid; i < n; i += 256) dst[i * a.gate_wg] = lhist[i];
  }
}

template <typename T, int D, bool kMinMax>
static void launch_gate_kcap(const GateArgs& a, int kcap, size_t shmem, hipStream_t st, dim3 grid) {
  if (kcap <= 4)
    hipLaunchKernelGGL((gate_kernel<T, D, 4, kMinMax>), grid, dim3(256), shmem, st, a);
  else if (kcap <= 16)
    hipLaunchKernelGGL((gate_kernel<T, D, 16, kMinMax>), grid, dim3(256), shmem, st, a);
  else if (kcap <= 32)
    hipLaunchKernelGGL((gate_kernel<T, D, 32, kMinMax>), grid, dim3(256), shmem, st, a);
  else
    hipLaunchKernelGGL((gate_rounds_kernel<T, D, kMinMax>), grid, dim3(256), shmem, st, a);
}
template <typename T, int D>
static void launch_gate_valu(const GateArgs& a, int kcap, hipStream_t st, dim3 grid) {
  const size_t hist = a.hist ? (size_t)a.n * sizeof(int) : 0;
  if (a.minmax)
    launch_gate_kcap<T, D, true>(a, kcap, (size_t)kMuSlice * 2 * D * sizeof(float) + hist, st, grid);
  else
    launch_gate_kcap<T, D, false>(a, kcap, (size_t)kMuSlice * D * sizeof(float) + hist, st, grid);
}

template <bool kMinMax>
static void launch_gate_mfma(const GateArgs& a, int kc, size_t sh, hipStream_t st, dim3 grid) {
  // the list as short as the kept blocks allow: each entry a score may pass
  // costs a 64-bit compare-and-swap in the one-pass form
  if (kc <= 1)
    hipLaunchKernelGGL((gate_mfma_kernel<1, kMinMax>), grid, dim3(512), sh, st, a, a.mu3);
  else if (kc <= 2)
    hipLaunchKernelGGL((gate_mfma_kernel<2, kMinMax>), grid, dim3(512), sh, st, a, a.mu3);
  else if (kc <= 4)
    hipLaunchKernelGGL((gate_mfma_kernel<4, kMinMax>), grid, dim3(512), sh, st, a, a.mu3);
  else if (kc <= 8)
    hipLaunchKernelGGL((gate_mfma_kernel<8, kMinMax>), grid, dim3(512), sh, st, a, a.mu3);
  else if (kc <= 12)
    hipLaunchKernelGGL((gate_mfma_kernel<12, kMinMax>), grid, dim3(512), sh, st, a, a.mu3);
  else if (kc <= 16)
    hipLaunchKernelGGL((gate_mfma_kernel<16, kMinMax>), grid, dim3(512), sh, st, a, a.mu3);
  else if (kc <= 32)
    hipLaunchKernelGGL((gate_mfma_kernel<32, kMinMax>), grid, dim3(512), sh, st, a, a.mu3);
  else
    hipLaunchKernelGGL((gate_mfma_kernel<32, kMinMax, true>), grid, dim3(512), sh, st, a, a.mu3);
}

int launch_mm_split(const float* lohi, int64_t batch, int64_t n, int hkv, uint16_t* mu3, hipStream_t st) {
  hipLaunchKernelGGL(mm_split_kernel, dim3((unsigned)((n + kGateTile - 1) / kGateTile), (unsigned)hkv, (unsigned)batch),
                     dim3(256), 0, st, lohi, n, hkv, mu3);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mu_split(const float* mu, int64_t batch, int64_t n, int hkv, uint16_t* mu3, hipStream_t st) {
  hipLaunchKernelGGL(mu_split_kernel, dim3((unsigned)((n + kGateTile - 1) / kGateTile), (unsigned)hkv, (unsigned)batch),
                     dim3(256), 0, st, mu, n, hkv, mu3);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gate(const GateArgs& a, int dtype, int d, hipStream_t st) {
  dim3 grid((unsigned)a.gate_wg, (unsigned)a.hkv);
  if (dtype == 1 && a.mu3 && a.gate_t * a.g <= 256) {
    const size_t sh = (size_t)2 * kMu3TileElems * 2 + (a.hist ? (size_t)a.n * sizeof(int) : 0);
    const int kc = a.kp < 1 ? 1 : a.kp;
    if (a.minmax)
      launch_gate_mfma<true>(a, kc, sh, st, grid);
    else
      launch_gate_mfma<false>(a, kc, sh, st, grid);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int kcap = a.kp < 1 ? 1 : a.kp;
  if (dtype == 1) {
    launch_gate_valu<bf16raw, 128>(a, kcap, st, grid);
  } else if (d == 64) {
    launch_gate_valu<float, 64>(a, kcap, st, grid);
  } else {
    launch_gate_valu<float, 128>(a, kcap, st, grid);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
