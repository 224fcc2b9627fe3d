// Block-sparse attention of the MoBA forward on bf16 MFMA (gfx950).
//
// Deep-dive report on MoBA, section 3.2: the attention over the chosen blocks
// is split by the causal flag.  Past blocks lie wholly before the query (the
// gate never routes to a future block), so they need no mask; only the
// query's own block is causal.  Their partial softmax results are merged
// exactly with the log-sum-exp rule of online softmax.
//
//   attn_past_kernel: one work-group per tile of up to 128 (row, slot)
//       entries that all chose the same block i of the same KV head.  The
//       gathered query rows stay in registers; the block's keys and values
//       stream through LDS in 64-key slices.  Output per entry: the
//       normalised partial o (fp32) and its log2-domain log-sum-exp.
//   attn_own_kernel: one work-group per 128 query rows of one own block
//       (all query heads of a KV-head group together).  Causal attention over
//       the own block up to each query, then the merge of that row's
//       partials, then the bf16 output.
//
// Tile mathematics (per wave: 32 query rows, per step: 64 keys, D = 128):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = keys from LDS, B = the
//   queries' registers), so each lane owns one query and 16 of every 32 keys;
//   row max / sum need one cross-lane exchange with lane l ^ 32 only.
//   O^T += V^T P^T on the same instruction: P^T is fed straight from the
//   score registers (the key order inside each 16-key step is permuted to the
//   accumulator layout, and V^T is read from LDS in the same permuted order),
//   and V is stored transposed in LDS so those reads are 8-byte vectors.
//   exp2 with log2(e)/sqrt(D) folded into one scale.
#include "moba_device.h"
#include "moba_kernels.h"
#include "moba_plan.h"

namespace moba {

constexpr int HD = 128;           // head dim of the bf16 path
constexpr int KT = 64;            // keys per LDS slice
constexpr int KS_STRIDE = HD + 8; // bf16 per K row in LDS (272 B: conflict-free 16 B reads)
constexpr int VT_STRIDE = KT + 4; // bf16 per V^T row in LDS (136 B: conflict-free 8 B reads)

struct TileState {
  f32x16 o[4];    // O^T accumulators: d block x (32 d x 32 queries)
  float m;        // running max of the scaled logits (log2 domain)
  float l;        // this lane's share of the running sum
};

__device__ __forceinline__ void state_init(TileState& st) {
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[b][e] = 0.f;
  st.m = -__builtin_inff();
  st.l = 0.f;
}

// Load this lane's query row into the B-operand layout of S^T = K Q^T:
// step s holds d = (lane / 32) * 8 + 16 s .. + 7.
__device__ __forceinline__ void load_q_operand(const bf16raw* qrow, int lane, bf16x8* qb) {
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qb[s] = *reinterpret_cast<const bf16x8*>(qrow + (lane >> 5) * 8 + 16 * s);
}

// Stage keys [key0, key0 + KT) of one KV head into LDS (K row-major, V
// transposed).  Keys at or beyond key_end are zero-filled.
__device__ __forceinline__ void stage_kv(const bf16raw* __restrict__ k, const bf16raw* __restrict__ v,
                                         int64_t row_stride, int64_t key0, int64_t key_end,
                                         bf16raw* ks, bf16raw* vts) {
  const int tid = threadIdx.x;
  // K: 64 keys x 16 chunks of 8 bf16; 4 chunks per thread
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = tid + 256 * u;
    const int key = c >> 4, dc = c & 15;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key0 + key < key_end) val = *reinterpret_cast<const u32x4*>(k + (key0 + key) * row_stride + dc * 8);
    *reinterpret_cast<u32x4*>(ks + key * KS_STRIDE + dc * 8) = val;
  }
  // V: thread owns 4 consecutive keys x 8 consecutive d and writes them as
  // 8 rows of V^T (4 keys = 8 bytes each)
  {
    const int dc = tid & 15, kg = tid >> 4;
    u32x4 r[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int64_t key = key0 + kg * 4 + x;
      r[x] = (key < key_end) ? *reinterpret_cast<const u32x4*>(v + key * row_stride + dc * 8)
                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // d = dc*8 + 2w (low halves) and dc*8 + 2w + 1 (high halves)
      const uint32_t lo01 = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x07060302u);
      *reinterpret_cast<u32x2*>(vts + (dc * 8 + 2 * w) * VT_STRIDE + kg * 4) = u32x2{lo01, lo23};
      *reinterpret_cast<u32x2*>(vts + (dc * 8 + 2 * w + 1) * VT_STRIDE + kg * 4) = u32x2{hi01, hi23};
    }
  }
}

// One 64-key slice: scores, online softmax update, P V.  `masked(kr)` tells
// whether key kr (0..63 inside the slice) is invisible to this lane's query.
template <typename Mask>
__device__ __forceinline__ void attend_slice(const bf16raw* ks, const bf16raw* vts, const bf16x8* qb,
                                             TileState& st, float scale_log2, int lane, Mask masked) {
  const int lr = lane & 31, lg = lane >> 5;
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
    const bf16raw* krow = ks + (kb * 32 + lr) * KS_STRIDE + lg * 8;
#pragma unroll
    for (int step = 0; step < 8; ++step) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * step);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[step], s[kb], 0, 0, 0);
    }
  }
  // scale, mask, slice max (this lane's 32 keys, then the partner lane's)
  float mx = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = kb * 32 + 8 * (e >> 2) + lg * 4 + (e & 3);
      float x = s[kb][e] * scale_log2;
      if (masked(kr)) x = -__builtin_inff();
      s[kb][e] = x;
      mx = __builtin_fmaxf(mx, x);
    }
  mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = __builtin_fmaxf(st.m, mx);
  // all keys so far invisible: keep the state as it is
  const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  st.m = m_new;
  float psum = 0.f;
  uint32_t pk[2][8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = fast_exp2(s[kb][e] - m_use);
      const float p1 = fast_exp2(s[kb][e + 1] - m_use);
      psum += p0 + p1;
      pk[kb][e >> 1] = pack_bf16x2(p0, p1);
    }
  st.l = st.l * alpha + psum;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[b][e] *= alpha;
  // O^T[d][q] += sum_key V^T[d][key] P^T[key][q]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      u32x4 pw = {pk[kb][4 * hs + 0], pk[kb][4 * hs + 1], pk[kb][4 * hs + 2], pk[kb][4 * hs + 3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bf16raw* vrow = vts + (b * 32 + lr) * VT_STRIDE + kb * 32 + 16 * hs + lg * 4;
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vrow + 8);
        u32x4 vw = {v0[0], v0[1], v1[0], v1[1]};
        st.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pb, st.o[b], 0, 0, 0);
      }
    }
}

struct NoMask {
  __device__ __forceinline__ bool operator()(int) const { return false; }
};

struct TailMask {  // keys at or beyond `lim` (slice-relative) do not exist
  int lim;
  __device__ __forceinline__ bool operator()(int kr) const { return kr >= lim; }
};

struct CausalMask {  // key slice-relative kr is visible iff kr <= qpos (slice-relative)
  int qpos;
  __device__ __forceinline__ bool operator()(int kr) const { return kr > qpos; }
};

__global__ __launch_bounds__(256) void attn_past_kernel(PastArgs a) {
  __shared__ __attribute__((aligned(16))) bf16raw ks[KT * KS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16raw vts[HD * VT_STRIDE];
  // XCD-aware order: consecutive tiles of one list run on the same XCD
  const int32_t total = a.tiles[0];
  const int32_t per_xcd = (total + 7) >> 3;
  const int32_t loc = blockIdx.x >> 3;
  if (loc >= per_xcd) return;
  const int32_t tile = (int32_t)(blockIdx.x & 7) * per_xcd + loc;
  if (tile >= total) return;
  const int32_t L = a.tiles[8 + 2 * tile];
  const int32_t start = a.tiles[9 + 2 * tile];
  const int32_t end = a.listoff[L] + a.count[L];
  const int32_t cnt = (end - start) < kTileRows ? (end - start) : kTileRows;
  const int hk = (int)(L / a.n);
  const int64_t blk = L % a.n;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = wave * 32 + (lane & 31);
  const bool valid = r < cnt;
  const int32_t entry = a.entries[start + (valid ? r : 0)];
  const int64_t local_row = entry / a.kp;
  const int64_t pic = local_row / a.hq;
  const int h = (int)(local_row % a.hq);
  const int64_t t = a.t0 + pic;
  const bf16raw* qrow = reinterpret_cast<const bf16raw*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * HD;
  bf16x8 qb[8];
  load_q_operand(qrow, lane, qb);

  const int64_t row_stride = (int64_t)a.hkv * HD;
  const bf16raw* kbase = reinterpret_cast<const bf16raw*>(a.k) + (a.bb * a.seqlen) * row_stride + hk * HD;
  const bf16raw* vbase = reinterpret_cast<const bf16raw*>(a.v) + (a.bb * a.seqlen) * row_stride + hk * HD;
  const int64_t key_begin = blk * a.block, key_end = key_begin + a.block;

  TileState st;
  state_init(st);
  for (int64_t k0 = key_begin; k0 < key_end; k0 += KT) {
    __syncthreads();
    stage_kv(kbase, vbase, row_stride, k0, key_end, ks, vts);
    __syncthreads();
    if (key_end - k0 >= KT)
      attend_slice(ks, vts, qb, st, a.scale_log2, lane, NoMask{});
    else
      attend_slice(ks, vts, qb, st, a.scale_log2, lane, TailMask{(int)(key_end - k0)});
  }

  const float ltot = st.l + __shfl_xor(st.l, 32);
  if (valid) {
    const float inv = 1.f / ltot;
    float* dst = a.part_o + (int64_t)entry * HD;
    const int lg = lane >> 5;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 o4 = {st.o[b][4 * q4] * inv, st.o[b][4 * q4 + 1] * inv, st.o[b][4 * q4 + 2] * inv,
                    st.o[b][4 * q4 + 3] * inv};
        *reinterpret_cast<f32x4*>(dst + b * 32 + 8 * q4 + lg * 4) = o4;
      }
    if (lg == 0) a.part_lse[entry] = st.m + fast_log2(ltot);
  }
}

__global__ __launch_bounds__(256) void attn_own_kernel(OwnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16raw ks[KT * KS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16raw vts[HD * VT_STRIDE];
  const int64_t tiles_per_block = (a.block + a.own_t - 1) / a.own_t;
  const int64_t jl = blockIdx.x / tiles_per_block;        // block inside the chunk
  const int64_t p0 = (blockIdx.x % tiles_per_block) * a.own_t;  // first position inside the block
  const int hk = blockIdx.y;
  const int64_t cblk0 = a.t0 / a.block;
  const int64_t j = cblk0 + jl;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rr = wave * 32 + (lane & 31);
  const int64_t pos = p0 + rr / a.g;                      // position inside the block
  const int h = hk * a.g + rr % a.g;
  const bool valid = rr < a.own_t * a.g && pos < a.block;
  const int64_t pos_c = valid ? pos : p0;                 // clamp for loads
  const int h_c = valid ? h : hk * a.g;
  const int64_t t = j * a.block + pos_c;
  const bf16raw* qrow = reinterpret_cast<const bf16raw*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h_c) * HD;
  bf16x8 qb[8];
  load_q_operand(qrow, lane, qb);

  const int64_t row_stride = (int64_t)a.hkv * HD;
  const bf16raw* kbase = reinterpret_cast<const bf16raw*>(a.k) + (a.bb * a.seqlen) * row_stride + hk * HD;
  const bf16raw* vbase = reinterpret_cast<const bf16raw*>(a.v) + (a.bb * a.seqlen) * row_stride + hk * HD;

  TileState st;
  state_init(st);
  if (a.causal) {
    const int64_t last = (p0 + a.own_t < a.block ? p0 + a.own_t : a.block);  // keys [0, last) of the block
    const int64_t kb0 = j * a.block;
    for (int64_t k0 = 0; k0 < last; k0 += KT) {
      __syncthreads();
      stage_kv(kbase, vbase, row_stride, kb0 + k0, kb0 + last, ks, vts);
      __syncthreads();
      if (k0 + KT <= p0)
        attend_slice(ks, vts, qb, st, a.scale_log2, lane, NoMask{});
      else
        attend_slice(ks, vts, qb, st, a.scale_log2, lane, CausalMask{(int)(pos_c - k0)});
    }
  }

  // merge this row's partials (log-sum-exp rule), normalise, store bf16
  const float l_own = st.l + __shfl_xor(st.l, 32);
  const int64_t local_row = (j * a.block + pos_c - a.t0) * a.hq + h_c;
  const int64_t nslot = a.causal ? (j < a.kp ? j : a.kp) : a.kp;
  float M = st.m;
  for (int64_t s = 0; s < nslot; ++s) M = __builtin_fmaxf(M, a.part_lse[local_row * a.kp + s]);
  const float c_own = (st.m == -__builtin_inff()) ? 0.f : fast_exp2(st.m - M);
  float Lsum = l_own * c_own;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[b][e] *= c_own;
  const int lg = lane >> 5;
  for (int64_t s = 0; s < nslot; ++s) {
    const int64_t p = local_row * a.kp + s;
    const float w = fast_exp2(a.part_lse[p] - M);
    Lsum += w;
    const float* src = a.part_o + p * HD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 o4 = *reinterpret_cast<const f32x4*>(src + b * 32 + 8 * q4 + lg * 4);
#pragma unroll
        for (int x = 0; x < 4; ++x) st.o[b][4 * q4 + x] += w * o4[x];
      }
  }
  if (valid) {
    const float inv = 1.f / Lsum;
    bf16raw* dst = reinterpret_cast<bf16raw*>(a.out) + ((a.bb * a.seqlen + t) * a.hq + h) * HD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 w2 = {pack_bf16x2(st.o[b][4 * q4] * inv, st.o[b][4 * q4 + 1] * inv),
                    pack_bf16x2(st.o[b][4 * q4 + 2] * inv, st.o[b][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(dst + b * 32 + 8 * q4 + lg * 4) = w2;
      }
  }
}

int launch_attn_past(const PastArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(attn_past_kernel, dim3((unsigned)a.max_tiles), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_attn_own(const OwnArgs& a, hipStream_t st) {
  const int64_t tiles_per_block = (a.block + a.own_t - 1) / a.own_t;
  const int64_t nblk = a.cnt / a.block;
  hipLaunchKernelGGL(attn_own_kernel, dim3((unsigned)(nblk * tiles_per_block), (unsigned)a.hkv), dim3(256), 0, st,
                     a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
