// Block-sparse attention of the MoBA forward on bf16 MFMA (gfx950).
//
// Deep-dive report on MoBA, section 3.2: the attention over the chosen blocks
// is split by the causal flag.  Past blocks lie wholly before the query (the
// gate never routes to a future block), so they need no mask; only the
// query's own block is causal.  The partial softmax results are merged
// exactly with the log-sum-exp rule of online softmax.
//
//   attn_past_kernel<NW>: one work-group per tile of up to NW*32 (row, slot)
//       entries that all chose the same block i of the same KV head.  The
//       gathered query rows stay in registers; the block's keys and values
//       stream through LDS in 64-key slices.  Output per entry: the
//       normalised partial o (bf16) and its log2-domain log-sum-exp (fp32).
//   attn_own_kernel: one work-group per 256 query rows of one own block (all
//       query heads of a KV-head group together): causal attention over the
//       own block up to each query, with the row's partials folded into the
//       same online softmax as further groups of keys (their loads overlap
//       the slice loop), then the bf16 output.
//   attn_past_img_kernel: the past-block tiles of 384 rows, K and V read
//       from per-slice images laid out as LDS wants them (long lists).
//   attn_past_rows_kernel / attn_own_rows_kernel: 128-row tiles that load K
//       and V rows as they are straight into LDS in 32-key slices and read
//       the V^T operand with the transposing LDS load; three work-groups per
//       CU (the past blocks of short lists; the own block of most shapes).
//
// Work split inside a work-group: every wave owns 32 query rows; 4, 8 or 12
// waves share each K/V slice staged in LDS, and two or three waves per SIMD
// let one wave's softmax arithmetic overlap another's MFMAs.  Slices are
// loaded ahead while the current one is computed (into registers, or
// straight into a third LDS buffer on the direct-load paths), and one
// barrier per slice separates the buffer hand-over.
//
// Tile mathematics (per wave, per 64-key slice, D = 128):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = keys from LDS, B = the
//   queries' registers), so each lane owns one query and 16 of every 32 keys;
//   the row max needs one exchange with lane l ^ 32 and the row sum stays
//   split across the pair until the end.
//   O^T += V^T P^T on the same instruction: P^T is fed straight from the
//   score registers (inside each 16-key step the key order is permuted to the
//   accumulator layout, and V^T is read from LDS in the same permuted order),
//   V being stored transposed in LDS so those reads are 16-byte vectors.
//   The max is taken on raw scores; p = exp2(s * c - m) with
//   c = log2(e)/sqrt(D), one FMA and one exp2 per score.  The running max m
//   is only raised when a slice exceeds it by more than 2^8 (then the
//   accumulators are rescaled); otherwise p may reach 2^8, which fp32 sums
//   and bf16 P hold without loss of relative precision.
#include "moba_device.h"
#include "moba_kernels.h"
#include "moba_plan.h"

namespace moba {

constexpr int HD = 128;                    // head dim of the bf16 path
constexpr int KT = 64;                     // keys per LDS slice
constexpr int KS_STRIDE = HD + 8;          // bf16 per K row in LDS (272 B: conflict-free 16 B reads)
constexpr int VT_STRIDE = KT;              // bf16 per V^T row in LDS (128 B, see vt_index)
constexpr int KS_ELEMS = KT * KS_STRIDE;
constexpr int VT_ELEMS = HD * VT_STRIDE;
constexpr int BUF_ELEMS = KS_ELEMS + VT_ELEMS;   // one slice buffer, 33792 B
constexpr float kLazyRescale = 8.0f;       // log2 units
constexpr float kMInit = -1e30f;           // finite "minus infinity" for the running max

// V^T layout in LDS.  Inside every 16-key step the key bits 2 and 3 are
// swapped, so the 8 keys one MFMA lane needs (two groups of 4, 8 apart) form
// one 16-byte unit; rows are 128 bytes and the unit index of row d is XORed
// with ((d >> 3) ^ d) & 7.  Measured on gfx950 with the LDS bank-conflict
// counter, this keeps both the operand reads (16 consecutive rows, one unit
// each) and the transposing staging writes (rows 8 apart) close to
// conflict-free; padded rows without the XOR make the writes 9-32x slower.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 3) ^ d) & 7; }
__device__ __forceinline__ int vt_index(int d, int key) {
  const int pk = (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
  return d * VT_STRIDE + ((((pk >> 3) ^ vt_swz(d)) & 7) << 3) + (pk & 7);
}

// Per-thread registers that carry one slice from HBM to LDS.  K: 64 keys x
// 16 chunks of 16 bytes.  V: units of KPU consecutive keys x 8 consecutive d,
// written as 8 rows of V^T (KPU keys each).  Offsets inside a slice are fixed
// per thread; a slice is addressed by its first key only.
template <int NW>
struct KVStager {
  static constexpr int NT = NW * 64;
  static constexpr int KCH = 1024 / NT;     // K chunks per thread
  static constexpr int KPU = 1024 / NT;     // keys per V unit (one unit per thread)
  u32x4 kr[KCH];
  u32x4 vr[KPU];

  __device__ __forceinline__ static int k_key(int x) { return (int)(threadIdx.x + NT * x) >> 4; }
  __device__ __forceinline__ static int k_dc(int x) { return (int)(threadIdx.x + NT * x) & 15; }
  __device__ __forceinline__ static int v_key(int y) { return (int)(threadIdx.x >> 4) * KPU + y; }
  __device__ __forceinline__ static int v_dc() { return (int)threadIdx.x & 15; }

  // Slice of 64 keys starting at the row pointers k0p / v0p (row stride rs).
  // kClamp: rows at or beyond `avail` (a ragged last slice) repeat row
  // avail - 1; their scores are masked to -inf, so they carry weight 0.
  template <bool kClamp>
  __device__ __forceinline__ void load(const bf16raw* __restrict__ k0p, const bf16raw* __restrict__ v0p, int rs,
                                       int avail) {
#pragma unroll
    for (int x = 0; x < KCH; ++x) {
      int key = k_key(x);
      if (kClamp) key = key < avail ? key : avail - 1;
      kr[x] = *reinterpret_cast<const u32x4*>(k0p + key * rs + k_dc(x) * 8);
    }
#pragma unroll
    for (int y = 0; y < KPU; ++y) {
      int key = v_key(y);
      if (kClamp) key = key < avail ? key : avail - 1;
      vr[y] = *reinterpret_cast<const u32x4*>(v0p + key * rs + v_dc() * 8);
    }
  }

  __device__ __forceinline__ void store(bf16raw* buf) const {
    bf16raw* ks = buf;
    bf16raw* vts = buf + KS_ELEMS;
#pragma unroll
    for (int x = 0; x < KCH; ++x)
      *reinterpret_cast<u32x4*>(ks + k_key(x) * KS_STRIDE + k_dc(x) * 8) = kr[x];
    const int dc = v_dc(), kg = (int)threadIdx.x >> 4;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // V^T rows d = dc*8 + 2w (low bf16 of each word) and dc*8 + 2w + 1 (high bf16);
      // the KPU keys of a unit stay adjacent under the key-bit swap
      bf16raw* lo = vts + vt_index(dc * 8 + 2 * w, kg * KPU);
      bf16raw* hi = vts + vt_index(dc * 8 + 2 * w + 1, kg * KPU);
      if constexpr (KPU == 4) {
        const uint32_t lo01 = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vr[3][w], vr[2][w], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vr[3][w], vr[2][w], 0x07060302u);
        *reinterpret_cast<u32x2*>(lo) = u32x2{lo01, lo23};
        *reinterpret_cast<u32x2*>(hi) = u32x2{hi01, hi23};
      } else {
        *reinterpret_cast<uint32_t*>(lo) = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x05040100u);
        *reinterpret_cast<uint32_t*>(hi) = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x07060302u);
      }
    }
  }
};

// Softmax state and accumulators of one wave's 32 query rows.
struct WaveRows {
  bf16x8 qb[8];   // B operand of S^T: step s holds d = (lane/32)*8 + 16 s .. +7
  f32x16 o[4];    // O^T accumulators: d block (32 d x 32 queries)
  float m;        // running max of the scaled logits (log2 domain)
  float l;        // this lane's share of the running sum
};

__device__ __forceinline__ void rows_init(WaveRows& R) {
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) R.o[b][e] = 0.f;
  R.m = kMInit;
  R.l = 0.f;
}

__device__ __forceinline__ void load_q(const bf16raw* qrow, int lane, bf16x8* qb) {
#pragma unroll
  for (int s = 0; s < 8; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qrow + (lane >> 5) * 8 + 16 * s);
}

// Combine a value with the one held by lane l ^ 32 (the other half of the same
// query's keys) without going through LDS.  v_permlane32_swap(a, b) returns,
// for lane l < 32, (a[l], a[l + 32]) and for lane l >= 32, (b[l - 32], b[l]);
// with a = b = x every lane gets its own value and its partner's.  (The two
// results are copied to scalars before the bit cast: a bit cast applied to a
// vector element directly reads element 0.)
__device__ __forceinline__ void pair_values(float x, float& u, float& w) {
  const uint32_t xb = __builtin_bit_cast(uint32_t, x);
  const auto pr = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
  const uint32_t r0 = pr[0], r1 = pr[1];
  u = __builtin_bit_cast(float, r0);
  w = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float pair_max(float x) {
  float u, w;
  pair_values(x, u, w);
  return __builtin_fmaxf(u, w);
}
__device__ __forceinline__ float pair_sum(float x) {
  float u, w;
  pair_values(x, u, w);
  return u + w;
}

// Sum of the two bf16 halves of a packed word, accumulated into acc in fp32.
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// Partial results of one chunk, private to the two attention kernels.
// Rows are numbered in the own-block kernel's order,
//   orow = ((jl * hkv + hk) * block + pos) * g + gi
// for position pos of the chunk's block jl and query head hk * g + gi, so
// the 32 rows of an own-block wave are consecutive.  Slot s (the row's s-th
// past block) is a plane of `rows` partials (the chunk's row capacity): the
// partial o of (orow, s) is 256 contiguous bytes at (s * rows + orow) * 256,
// so a wave's 32 rows of one slot are one contiguous 8 KiB.  Inside a partial
// the d values are in the order the O^T accumulators hold them: lane half lg
// owns the 128 bytes at 128 lg, whose 16-byte unit x = 2 b + h holds
// d = 32 b + 8 q4 + 4 lg + i for q4 = 2h, 2h + 1 and i = 0..3.  A (row, slot)
// pair is written whole by one lane pair of the past-block kernel, so its
// cache lines are complete after one wave's stores.  The log-sum-exp of
// (orow, s) sits at s * rows + orow.
__device__ __forceinline__ int64_t partial_row(int64_t pic, int h, int64_t block, int hkv, int g) {
  const int64_t jl = pic / block;
  return ((jl * hkv + h / g) * block + (pic - jl * block)) * g + h % g;
}
__device__ __forceinline__ void store_partial(bf16raw* part_o, int64_t rows, int64_t orow, int64_t s, const f32x16* o,
                                              float inv, int lg) {
  u32x4* p = reinterpret_cast<u32x4*>(part_o) + (s * rows + orow) * 16 + 8 * lg;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 8 * h;  // accumulator elements of q4 = 2h, 2h + 1
      p[2 * b + h] = u32x4{pack_bf16x2(o[b][e] * inv, o[b][e + 1] * inv), pack_bf16x2(o[b][e + 2] * inv, o[b][e + 3] * inv),
                           pack_bf16x2(o[b][e + 4] * inv, o[b][e + 5] * inv), pack_bf16x2(o[b][e + 6] * inv, o[b][e + 7] * inv)};
    }
}
__device__ __forceinline__ void load_partial(const bf16raw* part_o, int64_t rows, int64_t orow, int64_t s, int lg,
                                             u32x4* v) {
  const u32x4* p = reinterpret_cast<const u32x4*>(part_o) + (s * rows + orow) * 16 + 8 * lg;
#pragma unroll
  for (int x = 0; x < 8; ++x) v[x] = p[x];
}
__device__ __forceinline__ void add_partial(const u32x4* v, float w, f32x16* o) {
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[b][8 * h + 2 * j] += w * bf16lo(v[2 * b + h][j]);
        o[b][8 * h + 2 * j + 1] += w * bf16hi(v[2 * b + h][j]);
      }
}

// Fold one partial (normalised o, log2-domain log-sum-exp) into a row's
// running softmax state as one more group of keys: its weight relative to
// the running max m is 2^(lse - m), and m is raised by the same lazy rule
// as for a slice of scores.  The weight enters the row sum once (lane half
// 0), since the two lanes of a row each hold half of the sum.
__device__ __forceinline__ void fold_partial(WaveRows& R, const u32x4* v, float lse, int lg) {
  const bool need = lse > R.m + kLazyRescale;
  if (__any(need)) {
    const float mn = need ? lse : R.m;
    const float alpha = need ? fast_exp2(R.m - mn) : 1.0f;
    R.m = mn;
    R.l *= alpha;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) R.o[b][e] *= alpha;
  }
  const float w = fast_exp2(lse - R.m);
  R.l += (lg == 0) ? w : 0.f;
  add_partial(v, w, R.o);
}

// Byte offsets of this lane's V^T operand units.  Row d = 32 b + lr holds
// unit (4 kb + 2 hs + lg) at position unit ^ vt_swz(d), and
// vt_swz(32 b + lr) = vt_swz(lr) ^ (4 (b & 1)); so the position is
// c ^ x with the compile-time c = (4 kb + 2 hs) ^ 4 (b & 1) and the lane's
// x = lg ^ vt_swz(lr).  VtOffsets keeps lr * 128 + 16 (c ^ x) for all 8 c;
// the row block b adds the immediate b * 32 * 128.
struct VtOffsets {
  int off[8];
  __device__ __forceinline__ void init(int lane) {
    const int lr = lane & 31, x = (lane >> 5) ^ vt_swz(lr);
#pragma unroll
    for (int c = 0; c < 8; ++c) off[c] = lr * VT_STRIDE * 2 + ((c ^ x) << 4);
  }
};
__host__ __device__ constexpr int vt_c(int b, int kb, int hs) { return (4 * kb + 2 * hs) ^ (4 * (b & 1)); }

// Slice-relative key index held in accumulator element e of 32-key block kb
// is key_of(kb, e) + 4 * (lane / 32); the masks take the lane term into
// their limit, so every test compares against a compile-time key.
__device__ __forceinline__ constexpr int key_of(int kb, int e) { return kb * 32 + 8 * (e >> 2) + (e & 3); }

// S^T for one 64-key slice: two 32-key blocks of 32 keys x 32 queries.
__device__ __forceinline__ void qk_slice(const bf16raw* buf, const bf16x8* qb, f32x16* s, int lane) {
  const bf16raw* krow0 = buf + (lane & 31) * KS_STRIDE + (lane >> 5) * 8;
#pragma unroll
  for (int e = 0; e < 16; ++e) { s[0][e] = 0.f; s[1][e] = 0.f; }
  bf16x8 ka[8], kb_[8];
#pragma unroll
  for (int step = 0; step < 8; ++step) {
    ka[step] = *reinterpret_cast<const bf16x8*>(krow0 + 16 * step);
    kb_[step] = *reinterpret_cast<const bf16x8*>(krow0 + 32 * KS_STRIDE + 16 * step);
  }
#pragma unroll
  for (int step = 0; step < 8; ++step) {
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[step], qb[step], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb_[step], qb[step], s[1], 0, 0, 0);
  }
}

// Online-softmax update with the scores of one slice; returns P^T as packed
// bf16 pairs (pk[kb][x] holds accumulator elements 2x and 2x+1 of block kb).
// masked(kc): key kc + 4 * (lane / 32) of the slice is invisible to this
// lane's query.
template <bool kMasked, typename Mask, int NKB = 2>
__device__ __forceinline__ void softmax_p(f32x16* s, WaveRows& R, float c, int lane, Mask masked, uint32_t (*pk)[8]) {
  const int lg = lane >> 5;
  float mx = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (kMasked && masked(key_of(kb, e))) s[kb][e] = -__builtin_inff();
      mx = __builtin_fmaxf(mx, s[kb][e]);
    }
  mx = pair_max(mx);
  const float mxs = mx * c;
  // The need to rescale is decided per row (lanes l and l^32 agree); rows
  // that do not need it multiply by exactly 1, so a row's rounding never
  // depends on the other rows sharing its wave.  The branch itself is
  // wave-uniform.
  const bool need = mxs > R.m + kLazyRescale;
  if (__any(need)) {
    const float mn = need ? __builtin_fmaxf(R.m, mxs) : R.m;
    const float alpha = need ? fast_exp2(R.m - mn) : 1.0f;
    R.m = mn;
    R.l *= alpha;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) R.o[b][e] *= alpha;
  }
  const float negm = -R.m;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s[kb][e], c, negm));
      const float p1 = fast_exp2(__builtin_fmaf(s[kb][e + 1], c, negm));
      pk[kb][e >> 1] = pack_bf16x2(p0, p1);
    }
  // the row sum adds the bf16 weights that P V actually uses; two partial
  // sums keep the dependency chains short
  float ps0 = 0.f, ps1 = 0.f;
  if constexpr (NKB == 2) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      ps0 = add_bf16_pair(pk[0][x], ps0);
      ps1 = add_bf16_pair(pk[1][x], ps1);
    }
  } else {
#pragma unroll
    for (int x = 0; x < 8; x += 2) {
      ps0 = add_bf16_pair(pk[0][x], ps0);
      ps1 = add_bf16_pair(pk[0][x + 1], ps1);
    }
  }
  R.l += ps0 + ps1;
}

// O^T[d][q] += sum_key V^T[d][key] P^T[key][q] for one slice.
__device__ __forceinline__ void pv_vt(const char* vtb, const uint32_t (*pk)[8], WaveRows& R, const VtOffsets& vo) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const u32x4 pw = {pk[kb][4 * hs], pk[kb][4 * hs + 1], pk[kb][4 * hs + 2], pk[kb][4 * hs + 3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        // keys kb*32 + 16 hs + 8 (e/4) + 4 lg + e%4, e = 0..7: one 16-byte unit
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vtb + vo.off[vt_c(b, kb, hs)] + b * 32 * VT_STRIDE * 2);
        R.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, R.o[b], 0, 0, 0);
      }
    }
}

__device__ __forceinline__ void pv(const bf16raw* buf, const uint32_t (*pk)[8], WaveRows& R, const VtOffsets& vo) {
  pv_vt(reinterpret_cast<const char*>(buf + KS_ELEMS), pk, R, vo);
}

template <bool kMasked, typename Mask>
__device__ __forceinline__ void softmax_pv(const bf16raw* buf, f32x16* s, WaveRows& R, const VtOffsets& vo,
                                           float c, int lane, Mask masked) {
  uint32_t pk[2][8];
  softmax_p<kMasked>(s, R, c, lane, masked, pk);
  pv(buf, pk, R, vo);
}

// One 64-key slice without pipelining (scores, softmax, P V).
template <bool kMasked, typename Mask>
__device__ __forceinline__ void attend_slice(const bf16raw* buf, WaveRows& R, const VtOffsets& vo, float c, int lane,
                                             Mask masked) {
  f32x16 s[2];
  qk_slice(buf, R.qb, s, lane);
  softmax_pv<kMasked>(buf, s, R, vo, c, lane, masked);
}

// Scores of the keys a mask hides become -inf (weight 0 after the softmax).
template <typename Mask, int NKB = 2>
__device__ __forceinline__ void mask_scores(f32x16* s, Mask masked) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (masked(key_of(kb, e))) s[kb][e] = -__builtin_inff();
}

struct NoMask {
  __device__ __forceinline__ bool operator()(int) const { return false; }
};
// Keys at or beyond `avail` (slice-relative) do not exist.
struct TailMask {
  int lim;  // avail - 4 * (lane / 32)
  __device__ __forceinline__ TailMask(int avail, int lane) : lim(avail - 4 * (lane >> 5)) {}
  __device__ __forceinline__ bool operator()(int kc) const { return kc >= lim; }
};
// Key kr (slice-relative) is visible iff kr <= qpos.
struct CausalMask {
  int lim;  // qpos - 4 * (lane / 32)
  __device__ __forceinline__ CausalMask(int qpos, int lane) : lim(qpos - 4 * (lane >> 5)) {}
  __device__ __forceinline__ bool operator()(int kc) const { return kc > lim; }
};

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_past_kernel(PastArgs a) {
  __shared__ __attribute__((aligned(16))) bf16raw smem[2 * BUF_ELEMS];
  constexpr int ROWS = NW * 32;
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
  const int32_t cnt = (end - start) < ROWS ? (end - start) : ROWS;
  const int hk = (int)(L / a.n);
  const int64_t blk = L % a.n;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  WaveRows R;
  const int r = wave * 32 + (lane & 31);
  const bool valid = r < cnt;
  const int32_t entry = a.entries[start + (valid ? r : 0)];
  {
    const int64_t local_row = entry / a.kp;
    const int64_t pic = local_row / a.hq;
    const int h = (int)(local_row % a.hq);
    const int64_t t = a.t0 + pic;
    load_q(reinterpret_cast<const bf16raw*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * HD, lane, R.qb);
  }
  rows_init(R);
  VtOffsets vo;
  vo.init(lane);

  const int rs = a.hkv * HD;
  const bf16raw* kblk = reinterpret_cast<const bf16raw*>(a.k) + ((a.bb * a.seqlen) + blk * a.block) * (int64_t)rs + hk * HD;
  const bf16raw* vblk = reinterpret_cast<const bf16raw*>(a.v) + ((a.bb * a.seqlen) + blk * a.block) * (int64_t)rs + hk * HD;
  // any block size: double-buffered slices (the loads of slice s+1 in
  // flight while slice s is computed), a ragged last slice masked
  const int nsl = (a.block + KT - 1) / KT;
  const int nfull = a.block / KT;
  KVStager<NW> st;
  auto fetch = [&](int sl) {
    const int64_t off = (int64_t)sl * KT * rs;
    if (sl < nfull)
      st.template load<false>(kblk + off, vblk + off, rs, KT);
    else
      st.template load<true>(kblk + off, vblk + off, rs, a.block - sl * KT);
  };
  fetch(0);
  st.store(smem);
  __syncthreads();
  for (int sl = 0; sl < nfull; ++sl) {
    if (sl + 1 < nsl) fetch(sl + 1);
    attend_slice<false>(smem + (sl & 1) * BUF_ELEMS, R, vo, a.scale_log2, lane, NoMask{});
    if (sl + 1 < nsl) st.store(smem + ((sl + 1) & 1) * BUF_ELEMS);
    __syncthreads();
  }
  if (nfull < nsl)
    attend_slice<true>(smem + (nfull & 1) * BUF_ELEMS, R, vo, a.scale_log2, lane, TailMask(a.block - nfull * KT, lane));

  const int lg = lane >> 5;
  const float ltot = pair_sum(R.l);
  if (valid) {
    // the normalised partial is a convex combination of value rows, so bf16
    // keeps it to 2^-9 of the largest |v|
    const int64_t local_row = entry / a.kp, slot = entry - local_row * a.kp;
    const int64_t orow = partial_row(local_row / a.hq, (int)(local_row % a.hq), a.block, a.hkv, a.g);
    store_partial(a.part_o, a.part_rows, orow, slot, R.o, 1.f / ltot, lg);
    if (lg == 0) a.part_lse[slot * a.part_rows + orow] = R.m + fast_log2(ltot);
  }
}

// ---------------------------------------------------------------------------
// Image path (block a whole number of 64-key slices).
//
// K and V are first re-laid out once per call into per-slice images: slice
// c of KV head hk is a 16 KiB K image and a 16 KiB V^T image, each exactly
// the LDS layout the MFMA operand reads want, stored contiguously.  Staging
// a slice is then a plain 16-byte copy per thread (no transposition on the
// way), and the operand reads need no per-read address arithmetic.
//
// Both images are unit-major: 16-byte unit u of row r sits at slot
// u * rows + r.  An operand read (32 lanes on 32 consecutive rows, same
// unit) then touches 16 consecutive slots per 16 lanes, i.e. all 64 banks
// once, and a lane's reads differ only by immediate offsets.
//   K image:   unit u = 8 consecutive d (u = 0..15) of key row r (0..63):
//              slot u * 64 + r.
//   V^T image: unit U = 4 kb + 2 hs + lg (0..7) of d row (0..127): slot
//              U * 128 + d, holding V[key][d] for the 8 keys
//              32 kb + 16 hs + 8 (e >> 2) + 4 lg + (e & 3), e = 0..7 (the
//              order in which P^T leaves the score accumulators).
// ---------------------------------------------------------------------------
constexpr int IMG_BYTES = KT * HD * 2;         // one K or V^T slice image, 16 KiB
constexpr int SLICE_BYTES = 2 * IMG_BYTES;     // K image + V^T image

__global__ __launch_bounds__(256) void kv_image_kernel(const bf16raw* __restrict__ k, const bf16raw* __restrict__ v,
                                                       int64_t seqlen, int hkv, uint16_t* __restrict__ kimg,
                                                       uint16_t* __restrict__ vimg) {
  __shared__ __attribute__((aligned(16))) bf16raw kt[KT * KS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16raw vt[KT * KS_STRIDE];
  const int64_t sl = blockIdx.x;
  const int hk = blockIdx.y;
  const int64_t bb = blockIdx.z;
  const int64_t rs = (int64_t)hkv * HD;
  const int64_t src = (bb * seqlen + sl * KT) * rs + hk * HD;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int u = threadIdx.x + 256 * x;  // 64 keys x 16 units of 8 d
    const int key = u >> 4, dc = u & 15;
    *reinterpret_cast<u32x4*>(kt + key * KS_STRIDE + dc * 8) = *reinterpret_cast<const u32x4*>(k + src + key * rs + dc * 8);
    *reinterpret_cast<u32x4*>(vt + key * KS_STRIDE + dc * 8) = *reinterpret_cast<const u32x4*>(v + src + key * rs + dc * 8);
  }
  __syncthreads();
  const int64_t img = ((bb * hkv + hk) * (seqlen / KT) + sl) * (KT * HD);
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int slot = threadIdx.x + 256 * x;
    // K image: slot = unit * 64 + key row
    const int kr = slot & 63, ku = slot >> 6;
    *reinterpret_cast<u32x4*>(kimg + img + slot * 8) = *reinterpret_cast<const u32x4*>(kt + kr * KS_STRIDE + ku * 8);
    // V^T image: slot = U * 128 + d
    const int d = slot & 127, U = slot >> 7;
    const int kbase = 32 * (U >> 2) + 16 * ((U >> 1) & 1) + 4 * (U & 1);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int k0 = kbase + 8 * (e >> 2) + (e & 3);
      w[e >> 1] = (uint32_t)vt[k0 * KS_STRIDE + d] | ((uint32_t)vt[(k0 + 1) * KS_STRIDE + d] << 16);
    }
    *reinterpret_cast<u32x4*>(vimg + img + slot * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// O^T += V^T P^T for one slice from a V^T image; vb = this lane's base
// (lg * 2048 + (lane & 31) * 16 bytes), everything else immediate.
__device__ __forceinline__ void pv_img(const char* vb, const uint32_t (*pk)[8], WaveRows& R) {
  bf16x8 va[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int kb = x >> 3, hs = (x >> 2) & 1, b = x & 3;
    va[x] = *reinterpret_cast<const bf16x8*>(vb + (4 * kb + 2 * hs) * 2048 + b * 512);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const u32x4 pw = {pk[kb][4 * hs], pk[kb][4 * hs + 1], pk[kb][4 * hs + 2], pk[kb][4 * hs + 3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        R.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[8 * kb + 4 * hs + b], pb, R.o[b], 0, 0, 0);
    }
  // operand reads four MFMAs ahead, as in qk_img
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int x = 0; x < 12; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// S^T = K Q^T for one slice from a K image; kb = this lane's base
// (lg * 1024 + (lane & 31) * 16 bytes).
__device__ __forceinline__ void qk_img(const char* kb, const bf16x8* qb, f32x16* s) {
  bf16x8 ka[8], kc[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    ka[st] = *reinterpret_cast<const bf16x8*>(kb + st * 2048);
    kc[st] = *reinterpret_cast<const bf16x8*>(kb + st * 2048 + 512);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) { s[0][e] = 0.f; s[1][e] = 0.f; }
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], qb[st], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[st], qb[st], s[1], 0, 0, 0);
  }
  // operand reads two steps ahead of the MFMAs: four reads, then one MFMA
  // per read, then the last four MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int x = 0; x < 12; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Registers that carry one slice of the K and V^T images from HBM to LDS:
// each thread moves 16-byte units tid + NT x of both 16 KiB images, loaded
// and stored at the same offset (the images already are the LDS layout).
template <int NW>
struct ImgStager {
  static constexpr int NT = NW * 64;
  static constexpr int NU = 1024 / NT;  // units per image per thread
  u32x4 kr[NU], vr[NU];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs) {
#pragma unroll
    for (int x = 0; x < NU; ++x) {
      const int u = (int)threadIdx.x + NT * x;
      kr[x] = *reinterpret_cast<const u32x4*>(ks + u * 8);
      vr[x] = *reinterpret_cast<const u32x4*>(vs + u * 8);
    }
  }
  __device__ __forceinline__ void store(char* buf) const {
#pragma unroll
    for (int x = 0; x < NU; ++x) {
      const int u = (int)threadIdx.x + NT * x;
      *reinterpret_cast<u32x4*>(buf + u * 16) = kr[x];
      *reinterpret_cast<u32x4*>(buf + IMG_BYTES + u * 16) = vr[x];
    }
  }
};

// Past-block tiles of 384 rows over a block that is a whole number of
// slices, from the K and V^T images.  12 waves (three per SIMD) run in step:
// per slice the scores, the softmax and P V, one barrier per slice.  The
// images go straight from HBM into LDS (global_load_lds, no registers on
// the way): the loads of slice s+2 are issued at the start of slice s into
// the third of three LDS buffers, so each has two slice iterations to
// arrive, and the barrier that ends slice s first waits until only the
// youngest slice's loads are in flight.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void attn_past_img_kernel(PastArgs a) {
  __shared__ __attribute__((aligned(16))) char lb0[SLICE_BYTES];
  __shared__ __attribute__((aligned(16))) char lb1[SLICE_BYTES];
  __shared__ __attribute__((aligned(16))) char lb2[SLICE_BYTES];
  constexpr int ROWS = NW * 32;
  const int32_t total = a.tiles[0];
  const int32_t per_xcd = (total + 7) >> 3;
  const int32_t loc = blockIdx.x >> 3;
  if (loc >= per_xcd) return;
  const int32_t tile = (int32_t)(blockIdx.x & 7) * per_xcd + loc;
  if (tile >= total) return;
  const int32_t L = a.tiles[8 + 2 * tile];
  const int32_t start = a.tiles[9 + 2 * tile];
  const int32_t end = a.listoff[L] + a.count[L];
  const int32_t cnt = (end - start) < ROWS ? (end - start) : ROWS;
  const int hk = (int)(L / a.n);
  const int64_t blk = L % a.n;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  WaveRows R;
  const int r = wave * 32 + (lane & 31);
  const bool valid = r < cnt;
  const int32_t entry = a.entries[start + (valid ? r : 0)];
  {
    const int64_t local_row = entry / a.kp;
    const int64_t pic = local_row / a.hq;
    const int h = (int)(local_row % a.hq);
    const int64_t t = a.t0 + pic;
    load_q(reinterpret_cast<const bf16raw*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * HD, lane, R.qb);
  }
  rows_init(R);

  const int nsl = a.block / KT;
  const int64_t img0 = (((int64_t)a.bb * a.hkv + hk) * (a.seqlen / KT) + blk * nsl) * (KT * HD);
  const uint16_t* kimg = a.kimg + img0;
  const uint16_t* vimg = a.vimg + img0;
  const int lg = lane >> 5;
  const int kofs = lg * 1024 + (lane & 31) * 16;
  const int vofs = lg * 2048 + (lane & 31) * 16;
  // past the last slice the loads repeat it, so every iteration issues the same loads
  auto src = [&](int sl) { return (int64_t)(sl < nsl ? sl : nsl - 1) * (KT * HD); };
  const float c = a.scale_log2;

  // The loads into LDS are written as inline asm, so the compiler neither
  // tracks them nor adds waits for them; the explicit wait before each
  // barrier (vmcnt: at most the youngest slice's loads in flight) and the
  // barrier publish a slice to every wave, and the asm memory clobbers keep
  // the LDS reads on their side of it.  A buffer is loaded again only after
  // the barrier that ends the slice that read it.
  // the two images are 32 chunks of 64 units (chunk c < 16: K image chunk
  // c, else V^T image chunk c - 16); wave w loads chunks w, w + NW, ...
  // (with 12 waves, waves 0..7 three chunks and waves 8..11 two)
  static_assert(NW == 8 || NW == 12, "8 or 12 waves");
  constexpr int kMaxPer = (32 + NW - 1) / NW;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto dma = [&](char* lb, int sl) {
    const uint16_t* ks = kimg + src(sl);
    const uint16_t* vs = vimg + src(sl);
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t lb_addr = (uint32_t)(uintptr_t)((lds_char*)lb);
#pragma unroll
    for (int x = 0; x < kMaxPer; ++x) {
      const int c = wv + NW * x;
      if (c < 32) {
        const int chunk = c & 15;
        const int u = chunk * 64 + lane;
        const uint32_t wb = __builtin_amdgcn_readfirstlane(lb_addr + (uint32_t)((c >> 4) * IMG_BYTES + chunk * 64 * 16));
        lds_dma16(wb, (c < 16 ? ks : vs) + u * 8);
      }
    }
  };
  auto slice = [&](const char* buf) {
    f32x16 sc[2];
    uint32_t pk[2][8];
    qk_img(buf + kofs, R.qb, sc);
    softmax_p<false>(sc, R, c, lane, NoMask{}, pk);
    pv_img(buf + IMG_BYTES + vofs, pk, R);
  };

  // wait until at most one slice's loads (this wave's 4, 3 or 2) are in
  // flight, then the barrier; no fence, so the younger slice's loads stay
  // in flight (a fence would wait for every load into LDS); the memory
  // clobber keeps the compiler from moving LDS accesses across
  auto publish = [&] {
    if (NW == 8)
      asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    else if (wv < 8)
      asm volatile("s_waitcnt vmcnt(3)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
  };
  drain_vmem();  // the query rows in before any slice load goes out
  dma(lb0, 0);
  dma(lb1, 1);
  publish();
  auto step = [&](int sl, char* cur, char* nx2) {
    dma(nx2, sl + 2);  // past the end: the last slice again
    slice(cur);
    publish();  // slice sl + 1 in, in every wave
  };
  for (int sl = 0; sl < nsl; sl += 3) {
    step(sl, lb0, lb2);
    if (sl + 1 >= nsl) break;
    step(sl + 1, lb1, lb0);
    if (sl + 2 >= nsl) break;
    step(sl + 2, lb2, lb1);
  }
  drain_vmem();

  const float ltot = pair_sum(R.l);
  if (valid) {
    const int64_t local_row = entry / a.kp, slot = entry - local_row * a.kp;
    const int64_t orow = partial_row(local_row / a.hq, (int)(local_row % a.hq), a.block, a.hkv, a.g);
    store_partial(a.part_o, a.part_rows, orow, slot, R.o, 1.f / ltot, lg);
    if (lg == 0) a.part_lse[slot * a.part_rows + orow] = R.m + fast_log2(ltot);
  }
}

// ---------------------------------------------------------------------------
// Row path (block a whole number of 64-key slices, K and V as they are).
//
// A slice goes from HBM straight into LDS (global_load_lds) in row form:
// 64 K rows and 64 V rows of 256 bytes, the sixteen 16-byte units of row r
// rotated by rot(r) = 4 (r & 3) + ((r >> 2) & 3) (unit u at position
// (u + rot(r)) & 15).  The rotation keeps two read shapes free of bank
// conflicts: 16 consecutive rows at one unit (the K operand of S^T = K Q^T,
// read as it is), and 4 consecutive rows across two adjacent units, 8 bytes
// each (the V^T operand of P V: eight consecutive keys of one d per lane,
// which the transposing load ds_read_b64_tr_b16 gathers from the V rows).
// So no slice images are needed, and nothing passes through registers.
constexpr int ROW_BYTES = HD * 2;           // one K or V row in LDS
constexpr int ROWS_BYTES = KT * ROW_BYTES;  // one slice of K (or V) rows, 16 KiB
__device__ __forceinline__ int row_rot(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// This lane's LDS byte offsets inside a slice of rows.  k[s]: the K operand
// of contraction step s (key lane & 31, d 16 s + 8 (lane / 32) .. + 7); the
// second 32-key block adds 32 rows.  va[b] / vb[b]: the two transposing V
// reads of d block b (keys 4 (lane / 32) + ((lane & 15) >> 2) and 8 more,
// d 32 b + 16 ((lane >> 4) & 1) + 4 (lane & 3) .. + 3); the 16-key step
// (kb, hs) adds 32 kb + 16 hs rows.
struct RowOffsets {
  int k[8];
  int va[4], vb[4];
  __device__ __forceinline__ void init(int lane) {
    const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int s = 0; s < 8; ++s) k[s] = lr * ROW_BYTES + (((2 * s + lg + row_rot(lr)) & 15) << 4);
    const int tr = 4 * lg + ((lane & 15) >> 2);
    const int tc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int u = 4 * b + (tc >> 3), half = ((tc >> 2) & 1) * 8;
      va[b] = tr * ROW_BYTES + (((u + row_rot(tr)) & 15) << 4) + half;
      vb[b] = (tr + 8) * ROW_BYTES + (((u + row_rot(tr + 8)) & 15) << 4) + half;
    }
  }
};

template <int NKB>
__device__ __forceinline__ void qk_rows(const char* kbuf, const bf16x8* qb, f32x16* s, const RowOffsets& ro) {
  bf16x8 ka[NKB][8];
#pragma unroll
  for (int st = 0; st < 8; ++st)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) ka[kb][st] = *reinterpret_cast<const bf16x8*>(kbuf + ro.k[st] + kb * 32 * ROW_BYTES);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
  for (int st = 0; st < 8; ++st)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][st], qb[st], s[kb], 0, 0, 0);
  // operand reads two MFMAs ahead
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int x = 0; x < 8 * NKB - 2; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// O^T += V^T P^T for one slice of V rows.  The transposing load gives lane l
// the values of column d = 32 b + (l & 31) on four consecutive rows; the two
// loads cover keys 4 lg .. 4 lg + 3 and 8 + 4 lg .. 8 + 4 lg + 3 of the
// 16-key step, the order in which P^T holds them (the score accumulator's
// row order).
template <int NKB>
__device__ __forceinline__ void pv_rows(const char* vbuf, const uint32_t (*pk)[8], WaveRows& R, const RowOffsets& ro) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  bf16x8 va[8 * NKB];
#pragma unroll
  for (int x = 0; x < 8 * NKB; ++x) {
    const int kb = x >> 3, hs = (x >> 2) & 1, b = x & 3;
    const char* base = vbuf + (32 * kb + 16 * hs) * ROW_BYTES;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + ro.va[b]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + ro.vb[b]));
    va[x] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const u32x4 pw = {pk[kb][4 * hs], pk[kb][4 * hs + 1], pk[kb][4 * hs + 2], pk[kb][4 * hs + 3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        R.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[8 * kb + 4 * hs + b], pb, R.o[b], 0, 0, 0);
    }
  // operand reads (two transposing loads per operand) two MFMAs ahead
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int x = 0; x < 8 * NKB - 2; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// Past-block tiles of NW * 32 rows over a block that is a whole number of
// slices, K and V read as rows (no images).  A slice is NKB blocks of 32
// keys (64 or 32 keys: the shorter slice halves the LDS a work-group needs,
// so more work-groups share a CU).  NBUF LDS slice buffers: with two, the
// loads of slice s+1 go out at the start of slice s; with three, those of
// slice s+2.  K (or V) rows of a slice are 8 NKB loads of 1 KiB (four whole
// rows each); wave w issues loads w, w + NW, ...
template <int NW, int NBUF, int NKB>
struct RowsCfg {
  static constexpr int SK = 32 * NKB;                  // keys per slice
  static constexpr int TBYTES = SK * ROW_BYTES;        // K (or V) rows of one slice
  static constexpr int BUF = 2 * TBYTES;               // one slice buffer
  static constexpr int PER = 8 * NKB / NW;             // loads per tensor, wave and slice
  static constexpr int WGS = (160 * 1024) / (NBUF * BUF);  // work-groups per CU by LDS
  static constexpr int WPS0 = WGS * NW / 4;            // waves per SIMD by LDS
  static constexpr int WPS = WPS0 < 1 ? 1 : (WPS0 > 3 ? 3 : WPS0);  // at most three (168 registers)
};

// The loads of one slice of K and V rows straight into an LDS buffer.  Load
// j of a tensor covers rows 4 j .. 4 j + 3 (lane / 16 picks the row, and the
// lane fetches the unit that the row's rotation puts at LDS position
// lane & 15); wave w issues loads w, w + NW, ...  kbase / vbase: row 0 of
// the block in K / V, rs: the row stride in elements.
template <int NW, int NBUF, int NKB>
struct RowSliceLoader {
  using C = RowsCfg<NW, NBUF, NKB>;
  const bf16raw* kbase;
  const bf16raw* vbase;
  int64_t rs;
  int nsl, wave;
  int goff[C::PER];
  __device__ __forceinline__ RowSliceLoader(const bf16raw* k, const bf16raw* v, int64_t rs_, int nsl_, int wave_,
                                            int lane)
      : kbase(k), vbase(v), rs(rs_), nsl(nsl_), wave(wave_) {
#pragma unroll
    for (int i = 0; i < C::PER; ++i) {
      const int row = 4 * (wave + NW * i) + (lane >> 4);
      goff[i] = row * (int)rs + (((lane & 15) - row_rot(row)) & 15) * 8;
    }
  }
  // slice sl into buf; past the last slice the loads repeat it, so every
  // pipeline step issues the same number of loads
  __device__ __forceinline__ void operator()(char* buf, int sl) const {
    const int64_t so = (int64_t)(sl < nsl ? sl : nsl - 1) * C::SK * rs;
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t lb_addr = (uint32_t)(uintptr_t)((lds_char*)buf);
#pragma unroll
    for (int i = 0; i < C::PER; ++i) {
      const uint32_t wb = __builtin_amdgcn_readfirstlane(lb_addr + (uint32_t)((wave + NW * i) * 1024));
      lds_dma16(wb, kbase + so + goff[i]);
      lds_dma16(wb + C::TBYTES, vbase + so + goff[i]);
    }
  }
};

// Slices 0 .. nsl - 1 through the NBUF buffers lb: load(buf, sl) issues a
// slice's loads into LDS, body(sl, buf) computes it.  The loads are inline
// asm, so the compiler neither tracks them nor waits for them: each barrier
// that publishes a slice first waits (vmcnt) until only the younger slices'
// loads (2 PER per wave and slice) are in flight, and the asm memory clobber
// keeps the LDS reads on their side of it.  A buffer is loaded again only
// after the barrier that ends the slice that read it.  With two buffers the
// loads of slice s+1 go out at the start of slice s; with three, those of
// slice s+2.  The caller's own loads must have landed (drain_vmem) before.
template <int NBUF, int PER, int BUF, typename Load, typename Body>
__device__ __forceinline__ void run_row_slices(char (*lb)[BUF], int nsl, const Load& load, Body&& body) {
  static_assert(NBUF == 2 || (NBUF == 3 && (2 * PER == 4 || 2 * PER == 8)), "two buffers, or three (vmcnt 4 or 8)");
  if constexpr (NBUF == 2) {
    auto publish = [] { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); };
    load(lb[0], 0);
    publish();
    for (int sl = 0; sl < nsl; ++sl) {
      if (sl + 1 < nsl) load(lb[(sl + 1) & 1], sl + 1);
      body(sl, lb[sl & 1]);
      publish();
    }
  } else {
    auto publish = [] {
      if constexpr (2 * PER == 8)
        asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    };
    load(lb[0], 0);
    load(lb[1], 1);
    publish();
    auto step = [&](int sl, char* cur, char* nx2) {
      load(nx2, sl + 2);  // past the end: the last slice again
      body(sl, cur);
      publish();  // slice sl + 1 in, in every wave
    };
    for (int sl = 0; sl < nsl; sl += 3) {
      step(sl, lb[0], lb[2]);
      if (sl + 1 >= nsl) break;
      step(sl + 1, lb[1], lb[0]);
      if (sl + 2 >= nsl) break;
      step(sl + 2, lb[2], lb[1]);
    }
    drain_vmem();
  }
}

template <int NW, int NBUF, int NKB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RowsCfg<NW, NBUF, NKB>::WPS,
                                                                         RowsCfg<NW, NBUF, NKB>::WPS))) void
attn_past_rows_kernel(PastArgs a) {
  using C = RowsCfg<NW, NBUF, NKB>;
  static_assert((8 * NKB) % NW == 0 && (NBUF == 2 || NBUF == 3), "whole loads per wave; two or three buffers");
  __shared__ __attribute__((aligned(16))) char lb[NBUF][C::BUF];
  constexpr int ROWS = NW * 32;
  constexpr int PER = C::PER;
  const int32_t total = a.tiles[0];
  const int32_t per_xcd = (total + 7) >> 3;
  const int32_t loc = blockIdx.x >> 3;
  if (loc >= per_xcd) return;
  const int32_t tile = (int32_t)(blockIdx.x & 7) * per_xcd + loc;
  if (tile >= total) return;
  const int32_t L = a.tiles[8 + 2 * tile];
  const int32_t start = a.tiles[9 + 2 * tile];
  const int32_t end = a.listoff[L] + a.count[L];
  const int32_t cnt = (end - start) < ROWS ? (end - start) : ROWS;
  const int hk = (int)(L / a.n);
  const int64_t blk = L % a.n;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  WaveRows R;
  const int r = wave * 32 + (lane & 31);
  const bool valid = r < cnt;
  const int32_t entry = a.entries[start + (valid ? r : 0)];
  {
    const int64_t local_row = entry / a.kp;
    const int64_t pic = local_row / a.hq;
    const int h = (int)(local_row % a.hq);
    const int64_t t = a.t0 + pic;
    load_q(reinterpret_cast<const bf16raw*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * HD, lane, R.qb);
  }
  rows_init(R);
  RowOffsets ro;
  ro.init(lane);

  const int nsl = a.block / C::SK;
  const int64_t rs = (int64_t)a.hkv * HD;
  const int64_t base = ((int64_t)a.bb * a.seqlen + blk * a.block) * rs + hk * HD;
  const RowSliceLoader<NW, NBUF, NKB> load(reinterpret_cast<const bf16raw*>(a.k) + base,
                                           reinterpret_cast<const bf16raw*>(a.v) + base, rs, nsl, wave, lane);
  const float c = a.scale_log2;
  drain_vmem();  // the query rows in before any slice load goes out
  run_row_slices<NBUF, PER>(lb, nsl, load, [&](int, const char* buf) {
    f32x16 sc[NKB];
    uint32_t pk[NKB][8];
    qk_rows<NKB>(buf, R.qb, sc, ro);
    softmax_p<false, NoMask, NKB>(sc, R, c, lane, NoMask{}, pk);
    pv_rows<NKB>(buf + C::TBYTES, pk, R, ro);
  });

  const int lg = lane >> 5;
  const float ltot = pair_sum(R.l);
  if (valid) {
    const int64_t local_row = entry / a.kp, slot = entry - local_row * a.kp;
    const int64_t orow = partial_row(local_row / a.hq, (int)(local_row % a.hq), a.block, a.hkv, a.g);
    store_partial(a.part_o, a.part_rows, orow, slot, R.o, 1.f / ltot, lg);
    if (lg == 0) a.part_lse[slot * a.part_rows + orow] = R.m + fast_log2(ltot);
  }
}

constexpr int OWN_NW = 8;  // own-block tiles: 8 waves x 32 rows

// Own block of each query (causal up to the query itself) plus the merge
// of the row's partials.  kImg: K and V come from the slice images (block a
// whole number of slices); otherwise from K and V directly.
template <bool kImg>
__global__ __launch_bounds__(OWN_NW * 64) void attn_own_kernel(OwnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kImg ? 2 * SLICE_BYTES : 2 * BUF_ELEMS * 2];
  // Tiles in (block, KV head, tile) order.  XCD-aware: work-group i runs on
  // XCD i % 8, and with at least 64 (block, KV head) units each XCD takes a
  // contiguous run of tiles, so the tiles that read one block's K/V slices
  // share that XCD's L2.  With fewer units a run would hold a few units'
  // longest tiles (causal tiles differ in length), so they are dealt round
  // robin instead.
  const int64_t tiles_per_block = (a.block + a.own_t - 1) / a.own_t;
  const int64_t units = (a.cnt / a.block) * a.hkv;
  const int64_t total = units * tiles_per_block;
  const int64_t lt = units >= 64 ? (int64_t)(blockIdx.x & 7) * ((total + 7) >> 3) + (blockIdx.x >> 3) : (int64_t)blockIdx.x;
  if (lt >= total) return;
  const int64_t jl = lt / tiles_per_block / a.hkv;  // block inside the chunk
  const int hk = (int)(lt / tiles_per_block % a.hkv);
  // the tiles of a block launch last position first: the longest causal
  // ranges start earliest, so the grid does not end on them
  const int64_t p0 = (tiles_per_block - 1 - lt % tiles_per_block) * a.own_t;  // first position
  const int64_t j = a.t0 / a.block + jl;
  const int G = a.g;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lg = lane >> 5;
  WaveRows R;
  const int rr = wave * 32 + (lane & 31);
  const int64_t pp = p0 + rr / G;
  const bool valid = rr < a.own_t * G && pp < a.block;
  const int64_t pos = valid ? pp : p0;  // position inside the block (clamped for invalid rows)
  const int h = valid ? hk * G + rr % G : hk * G;
  {
    const int64_t t = j * a.block + pos;
    load_q(reinterpret_cast<const bf16raw*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * HD, lane, R.qb);
  }
  rows_init(R);

  // this row's partials from the past-block kernel (slot s: past block s of
  // its selection), folded into the softmax state like further keys
  const int64_t nslot = a.causal ? (j < a.kp ? j : a.kp) : a.kp;
  const int64_t orow = partial_row(j * a.block + pos - a.t0, h, a.block, a.hkv, G);
  const bf16raw* po = reinterpret_cast<const bf16raw*>(a.part_o);
  const int64_t rows = a.part_rows;
  int64_t nfolded = 0;

  if (a.causal) {
    const int64_t last = (p0 + a.own_t < a.block ? p0 + a.own_t : a.block);  // keys [0, last) of the block
    const int nsl = (int)((last + KT - 1) / KT);
    // last position any row of this wave holds: later slices are invisible to it
    int64_t wmax = p0 + (wave * 32 + 31) / G;
    if (wmax > a.block - 1) wmax = a.block - 1;
    // slices wholly before the tile's first query need no mask
    const int nfree = (int)(p0 / KT);
    const float c = a.scale_log2;
    if constexpr (kImg) {
      // keys past `last` in the last slice exist (the block is whole
      // slices) and are masked like every key after the query
      const int64_t img0 = (((int64_t)a.bb * a.hkv + hk) * (a.seqlen / KT) + j * (a.block / KT)) * (KT * HD);
      const uint16_t* kimg = a.kimg + img0;
      const uint16_t* vimg = a.vimg + img0;
      const int kofs = lg * 1024 + (lane & 31) * 16;
      const int vofs = lg * 2048 + (lane & 31) * 16;
      // the loads of slice s+2 go out at the start of slice s (two register
      // sets, LDS double-buffered), as in the past-block kernel; past the
      // last slice they repeat it
      ImgStager<OWN_NW> st, st2;
      auto src = [&](int sl) { return (int64_t)(sl < nsl ? sl : nsl - 1) * (KT * HD); };
      // one instance of the slice code: the causal mask is a separate step
      // on the scores of the slices that reach the tile's first query.  The
      // partial of slot sl is loaded before the slice's K/V prefetch and
      // folded after its P V, so its loads overlap the slice's MFMAs.
      auto slice = [&](int sl, const char* buf, bool fold, const u32x4* pv, float pl) {
        const int64_t k0 = (int64_t)sl * KT;
        if (k0 <= wmax) {
          f32x16 sc[2];
          uint32_t pk[2][8];
          qk_img(buf + kofs, R.qb, sc);
          if (sl >= nfree) mask_scores(sc, CausalMask((int)(pos - k0), lane));
          softmax_p<false>(sc, R, c, lane, NoMask{}, pk);
          pv_img(buf + IMG_BYTES + vofs, pk, R);
        }
        if (fold) fold_partial(R, pv, pl, lg);
      };
      const int64_t nloop = nslot < nsl ? nslot : nsl;  // slots folded inside the slice loop
      auto slice_with_partial = [&](int sl, const char* buf, auto&& prefetch) {
        u32x4 pv[8];
        float pl = 0.f;
        const bool fold = sl < nloop;
        if (fold) {
          load_partial(po, rows, orow, sl, lg, pv);
          pl = a.part_lse[sl * rows + orow];
        }
        prefetch();
        slice(sl, buf, fold, pv, pl);
      };
      st.load(kimg, vimg);
      st.store(smem);
      // the query rows and slice 0 must be in before the prefetch loads go out
      drain_vmem();
      st2.load(kimg + src(1), vimg + src(1));
      __syncthreads();
      for (int sl = 0; sl < nsl; sl += 2) {
        slice_with_partial(sl, smem, [&] { st.load(kimg + src(sl + 2), vimg + src(sl + 2)); });
        if (sl + 1 < nsl) st2.store(smem + SLICE_BYTES);
        __syncthreads();
        if (sl + 1 >= nsl) break;
        slice_with_partial(sl + 1, smem + SLICE_BYTES, [&] { st2.load(kimg + src(sl + 3), vimg + src(sl + 3)); });
        if (sl + 2 < nsl) st.store(smem);
        __syncthreads();
      }
      drain_vmem();
      nfolded = nloop;
    } else {
      bf16raw* sb = reinterpret_cast<bf16raw*>(smem);
      VtOffsets vo;
      vo.init(lane);
      const int64_t rs = (int64_t)a.hkv * HD;
      const int rsi = (int)rs;
      const bf16raw* kblk = reinterpret_cast<const bf16raw*>(a.k) + (a.bb * a.seqlen + j * a.block) * rs + hk * HD;
      const bf16raw* vblk = reinterpret_cast<const bf16raw*>(a.v) + (a.bb * a.seqlen + j * a.block) * rs + hk * HD;
      KVStager<OWN_NW> st;
      auto fetch = [&](int sl) {
        const int64_t off = (int64_t)sl * KT * rs;
        if ((sl + 1) * KT <= last)
          st.template load<false>(kblk + off, vblk + off, rsi, KT);
        else
          st.template load<true>(kblk + off, vblk + off, rsi, (int)(last - sl * KT));
      };
      fetch(0);
      st.store(sb);
      __syncthreads();
      for (int sl = 0; sl < nfree; ++sl) {
        if (sl + 1 < nsl) fetch(sl + 1);
        attend_slice<false>(sb + (sl & 1) * BUF_ELEMS, R, vo, c, lane, NoMask{});
        if (sl + 1 < nsl) st.store(sb + ((sl + 1) & 1) * BUF_ELEMS);
        __syncthreads();
      }
      for (int sl = nfree; sl < nsl; ++sl) {
        const int64_t k0 = (int64_t)sl * KT;
        if (sl + 1 < nsl) fetch(sl + 1);
        if (k0 <= wmax) attend_slice<true>(sb + (sl & 1) * BUF_ELEMS, R, vo, c, lane, CausalMask((int)(pos - k0), lane));
        if (sl + 1 < nsl) st.store(sb + ((sl + 1) & 1) * BUF_ELEMS);
        __syncthreads();
      }
    }
  }

  // the partials not folded in the slice loop (all of them in non-causal
  // mode, where the own block has no visible key and starts with weight 0),
  // then normalise and store bf16
  for (int64_t s = nfolded; s < nslot; ++s) {
    u32x4 pv[8];
    load_partial(po, rows, orow, s, lg, pv);
    fold_partial(R, pv, a.part_lse[s * rows + orow], lg);
  }
  const float Lsum = pair_sum(R.l);
  if (valid) {
    const float inv = 1.f / Lsum;
    const int64_t t = j * a.block + pos;
    // the row's log-sum-exp of the scaled logits, natural log (for the backward)
    if (a.lse && lg == 0) a.lse[((int64_t)a.bb * a.hq + h) * a.seqlen + t] = (R.m + fast_log2(Lsum)) * 0.6931471805599453f;
    bf16raw* dst = reinterpret_cast<bf16raw*>(a.out) + ((a.bb * a.seqlen + t) * a.hq + h) * HD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 w2 = {pack_bf16x2(R.o[b][4 * q4] * inv, R.o[b][4 * q4 + 1] * inv),
                          pack_bf16x2(R.o[b][4 * q4 + 2] * inv, R.o[b][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(dst + b * 32 + 8 * q4 + lg * 4) = w2;
      }
  }
}

// The own block from K and V rows (block a whole number of NKB * 32-key
// slices), loaded straight into LDS as in attn_past_rows_kernel, in tiles of
// NW * 32 rows; the row's partials are folded after the slice loop.
template <int NW, int NBUF, int NKB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RowsCfg<NW, NBUF, NKB>::WPS,
                                                                         RowsCfg<NW, NBUF, NKB>::WPS))) void
attn_own_rows_kernel(OwnArgs a) {
  using C = RowsCfg<NW, NBUF, NKB>;
  static_assert((8 * NKB) % NW == 0 && (NBUF == 2 || NBUF == 3), "whole loads per wave; two or three buffers");
  __shared__ __attribute__((aligned(16))) char lb[NBUF][C::BUF];
  constexpr int PER = C::PER;
  // tile order as in attn_own_kernel
  const int64_t tiles_per_block = (a.block + a.own_t - 1) / a.own_t;
  const int64_t units = (a.cnt / a.block) * a.hkv;
  const int64_t total = units * tiles_per_block;
  const int64_t lt = units >= 64 ? (int64_t)(blockIdx.x & 7) * ((total + 7) >> 3) + (blockIdx.x >> 3) : (int64_t)blockIdx.x;
  if (lt >= total) return;
  const int64_t jl = lt / tiles_per_block / a.hkv;
  const int hk = (int)(lt / tiles_per_block % a.hkv);
  const int64_t p0 = (tiles_per_block - 1 - lt % tiles_per_block) * a.own_t;
  const int64_t j = a.t0 / a.block + jl;
  const int G = a.g;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lg = lane >> 5;
  WaveRows R;
  const int rr = wave * 32 + (lane & 31);
  const int64_t pp = p0 + rr / G;
  const bool valid = rr < a.own_t * G && pp < a.block;
  const int64_t pos = valid ? pp : p0;
  const int h = valid ? hk * G + rr % G : hk * G;
  {
    const int64_t t = j * a.block + pos;
    load_q(reinterpret_cast<const bf16raw*>(a.q) + ((a.bb * a.seqlen + t) * a.hq + h) * HD, lane, R.qb);
  }
  rows_init(R);

  const int64_t nslot = a.causal ? (j < a.kp ? j : a.kp) : a.kp;
  const int64_t orow = partial_row(j * a.block + pos - a.t0, h, a.block, a.hkv, G);
  const bf16raw* po = reinterpret_cast<const bf16raw*>(a.part_o);
  const int64_t rows = a.part_rows;

  if (a.causal) {
    const int64_t last = (p0 + a.own_t < a.block ? p0 + a.own_t : a.block);  // keys [0, last) of the block
    const int nsl = (int)((last + C::SK - 1) / C::SK);
    int64_t wmax = p0 + (wave * 32 + 31) / G;
    if (wmax > a.block - 1) wmax = a.block - 1;
    const int nfree = (int)(p0 / C::SK);
    const float c = a.scale_log2;
    RowOffsets ro;
    ro.init(lane);
    const int64_t rs = (int64_t)a.hkv * HD;
    const int64_t base = ((int64_t)a.bb * a.seqlen + j * a.block) * rs + hk * HD;
    // keys past `last` in the last slice exist (the block is whole slices)
    // and are masked like every key after the query
    const RowSliceLoader<NW, NBUF, NKB> load(reinterpret_cast<const bf16raw*>(a.k) + base,
                                             reinterpret_cast<const bf16raw*>(a.v) + base, rs, nsl, wave, lane);
    drain_vmem();  // the query rows in before any slice load goes out
    run_row_slices<NBUF, PER>(lb, nsl, load, [&](int sl, const char* buf) {
      const int64_t k0 = (int64_t)sl * C::SK;
      if (k0 <= wmax) {
        f32x16 sc[NKB];
        uint32_t pk[NKB][8];
        qk_rows<NKB>(buf, R.qb, sc, ro);
        if (sl >= nfree) mask_scores<CausalMask, NKB>(sc, CausalMask((int)(pos - k0), lane));
        softmax_p<false, NoMask, NKB>(sc, R, c, lane, NoMask{}, pk);
        pv_rows<NKB>(buf + C::TBYTES, pk, R, ro);
      }
    });
  }

  for (int64_t s = 0; s < nslot; ++s) {
    u32x4 pv[8];
    load_partial(po, rows, orow, s, lg, pv);
    fold_partial(R, pv, a.part_lse[s * rows + orow], lg);
  }
  const float Lsum = pair_sum(R.l);
  if (valid) {
    const float inv = 1.f / Lsum;
    const int64_t t = j * a.block + pos;
    if (a.lse && lg == 0) a.lse[((int64_t)a.bb * a.hq + h) * a.seqlen + t] = (R.m + fast_log2(Lsum)) * 0.6931471805599453f;
    bf16raw* dst = reinterpret_cast<bf16raw*>(a.out) + ((a.bb * a.seqlen + t) * a.hq + h) * HD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 w2 = {pack_bf16x2(R.o[b][4 * q4] * inv, R.o[b][4 * q4 + 1] * inv),
                          pack_bf16x2(R.o[b][4 * q4 + 2] * inv, R.o[b][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(dst + b * 32 + 8 * q4 + lg * 4) = w2;
      }
  }
}

int launch_attn_past(const PastArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.max_tiles);
  // the 384-row tiles read K and V only from the slice images
  if (a.tile_rows == 384 && (!a.kimg || !a.vimg || a.block % KT != 0)) return -1;
  if (a.tile_rows == 256) {
    // 8 waves, one work-group per CU; from the slice images the loads run two
    // slices ahead, otherwise one (any block size)
    hipLaunchKernelGGL((attn_past_kernel<8>), grid, dim3(512), 0, st, a);
  } else if (a.tile_rows == 384) {
    // 12 waves (three per SIMD) over the slice images
    hipLaunchKernelGGL((attn_past_img_kernel<12>), grid, dim3(768), 0, st, a);
  } else {
    // 4 waves: from K and V rows in 32-key slices (block a multiple of 32),
    // three work-groups per CU; otherwise two, with register staging
    if (a.block % 32 == 0)
      hipLaunchKernelGGL((attn_past_rows_kernel<4, 3, 1>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_past_kernel<4>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_kv_image(const void* k, const void* v, int64_t batch, int64_t seqlen, int hkv, uint16_t* kimg,
                    uint16_t* vimg, hipStream_t st) {
  hipLaunchKernelGGL(kv_image_kernel, dim3((unsigned)(seqlen / KT), (unsigned)hkv, (unsigned)batch), dim3(256), 0, st,
                     reinterpret_cast<const bf16raw*>(k), reinterpret_cast<const bf16raw*>(v), seqlen, hkv, kimg, vimg);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_attn_own(const OwnArgs& a, hipStream_t st) {
  const int64_t tiles_per_block = (a.block + a.own_t - 1) / a.own_t;
  const int64_t nblk = a.cnt / a.block;
  const int64_t per_xcd = (nblk * tiles_per_block * a.hkv + 7) / 8;  // see attn_own_kernel
  const dim3 grid((unsigned)(8 * per_xcd));
  if (a.rows) {
    // 128-row tiles from K and V rows, 32-key slices: three work-groups per CU
    if (a.own_t * a.g > 128) return -1;
    if (a.block % 32 != 0) return -1;
    hipLaunchKernelGGL((attn_own_rows_kernel<4, 3, 1>), grid, dim3(256), 0, st, a);
  } else if (a.kimg && a.block % KT == 0) {
    if (a.own_t * a.g > OWN_NW * 32) return -1;
    hipLaunchKernelGGL(attn_own_kernel<true>, grid, dim3(OWN_NW * 64), 0, st, a);
  } else {
    if (a.own_t * a.g > OWN_NW * 32) return -1;
    hipLaunchKernelGGL(attn_own_kernel<false>, grid, dim3(OWN_NW * 64), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
