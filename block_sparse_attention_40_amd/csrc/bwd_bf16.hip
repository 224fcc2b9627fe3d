// Backward of the MoBA attention on bf16 MFMA (gfx950), head dim 128.
//
// The gate is a hard top-k with no parameters (deep-dive report on MoBA,
// §2.2): it only decides which keys a row attends, and no gradient flows
// through that decision.  With each row's chosen keys fixed, the row is plain
// softmax attention, so with the forward's row log-sum-exp (lse) and
// delta = dout . out:
//   p = exp(scale q.k - lse),  dp = dout . v,  ds = p (dp - delta),
//   dq = scale sum_keys ds k,  dk += scale ds q,  dv += p dout.
// The report trains with this attention (§3.3) but prints no backward; this
// is the gradient of the forward as computed.
//
// Work split, reusing the forward's block-major dispatch (report §3.2):
//   bwd_dq_kernel    query-stationary, like the forward's past-block kernel:
//                    one work-group per tile of up to 256 (row, slot) entries
//                    of one list (KV head, block), the block's keys streamed
//                    through LDS from three slice images (K and V in the K
//                    layout, K in the V^T layout); per 32-key half:
//                    S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
//                    Own-block tiles (causal) mask keys after the row.  Each
//                    (row, slot) writes its dq contribution (fp32); a merge
//                    adds a row's contributions.
//   bwd_dkdv_kernel  key-stationary: one work-group per 128 keys of one block,
//                    two waves per 32-key group: one computes S = Q K^T, P
//                    and dV, the other dP = dO V^T, dS (with P handed over
//                    through LDS) and dK, so each wave holds one operand and
//                    one accumulator set (two waves per SIMD); it walks every
//                    row that attends the block
//                    (the block's whole-sequence list, then, causal, the
//                    block's own rows at or after the slice) in steps of 32
//                    rows staged in LDS, and accumulates
//                    dV += P^T dO and dK += dS^T Q on the MFMAs.  The row
//                    operands of those two products run along the
//                    contraction, so they are read with the transposing LDS
//                    load (ds_read_b64_tr_b16) from the row-major staging.
#include "moba_device.h"
#include "moba_kernels.h"
#include "moba_plan.h"

namespace moba {

namespace {

constexpr int BD = 128;              // head dim
constexpr int BKT = 64;              // keys per image slice
constexpr int BIMG = BKT * BD * 2;   // bytes of one slice image (16 KiB)
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wsum64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Slice-relative key held in accumulator element e of 32-key half kb (the
// C layout of v_mfma_f32_32x32x16: element e of lane l is row 8(e/4) +
// 4(l/32) + e%4 of the 32-row block).
__device__ __forceinline__ int acc_row(int e, int lg) { return 8 * (e >> 2) + 4 * lg + (e & 3); }

}  // namespace

// ---------------------------------------------------------------------------
// delta and base-2 lse per row.  One wave per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(const bf16raw* __restrict__ out, const bf16raw* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ lse2,
                                                       float* __restrict__ delta, int64_t rows, int64_t seqlen,
                                                       int hq) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint32_t o = *reinterpret_cast<const uint32_t*>(out + row * BD + 2 * lane);
  const uint32_t d = *reinterpret_cast<const uint32_t*>(dout + row * BD + 2 * lane);
  const float x = wsum64(bf16lo(o) * bf16lo(d) + bf16hi(o) * bf16hi(d));
  if (lane == 0) {
    const int64_t per_b = seqlen * hq;
    const int64_t bb = row / per_b, rem = row % per_b;
    const int64_t t = rem / hq;
    const int h = (int)(rem % hq);
    delta[row] = x;
    lse2[row] = lse[(bb * hq + h) * seqlen + t] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dq.  256 rows per work-group (8 waves x 32 rows); kOwn: the rows are
// 256 / g positions x g heads of one own block (grid (tiles, hkv)).
// ---------------------------------------------------------------------------
template <bool kOwn>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdArgs a) {
  // three slice buffers of the three images each (144 KiB), loaded straight
  // from HBM two slices ahead
  __shared__ __attribute__((aligned(16))) char lbs[3][3 * BIMG];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 5;
  int hk, cnt;
  int64_t blk, own_p0 = 0;
  int32_t start = 0;
  if constexpr (!kOwn) {
    // XCD-aware order: work-group i runs on XCD i % 8, and each XCD takes a
    // contiguous run of tiles, so the tiles of one list share an L2
    const int32_t total = a.tiles[0];
    const int32_t per_xcd = (total + 7) >> 3;
    const int32_t loc = (int32_t)(blockIdx.x >> 3);
    if (loc >= per_xcd) return;
    const int32_t tile = (int32_t)(blockIdx.x & 7) * per_xcd + loc;
    if (tile >= total) return;
    const int32_t L = a.tiles[8 + 2 * tile];
    start = a.tiles[9 + 2 * tile];
    const int32_t end = a.listoff[L] + a.count[L];
    cnt = (end - start) < 256 ? (end - start) : 256;
    hk = (int)(L / a.n);
    blk = L % a.n;
  } else {
    const int ppt = 256 / a.g;  // positions per tile
    const int64_t tpb = (a.block + ppt - 1) / ppt;
    // (block, KV head, tile) order; with at least 64 (block, KV head) units
    // each XCD takes a contiguous run of tiles, else they are dealt round
    // robin (a run would hold a few units' longest tiles)
    const int64_t units = (a.cnt / a.block) * a.hkv;
    const int64_t total = tpb * units;
    const int64_t lt = units >= 64 ? (int64_t)(blockIdx.x & 7) * ((total + 7) >> 3) + (blockIdx.x >> 3) : (int64_t)blockIdx.x;
    if (lt >= total) return;
    hk = (int)(lt / tpb % a.hkv);
    blk = a.t0 / a.block + lt / tpb / a.hkv;
    own_p0 = (lt % tpb) * ppt;
    const int64_t np = (a.block - own_p0) < ppt ? (a.block - own_p0) : ppt;
    cnt = (int)np * a.g;
  }
  const int r = wave * 32 + (lane & 31);
  const bool valid = r < cnt;
  const int rr = valid ? r : 0;
  int64_t t;
  int h;
  int32_t entry = 0;
  if constexpr (!kOwn) {
    entry = a.entries[start + rr];
    const int64_t local_row = entry / a.kp;
    t = a.t0 + local_row / a.hq;
    h = (int)(local_row % a.hq);
  } else {
    h = hk * a.g + rr % a.g;
    t = blk * a.block + own_p0 + rr / a.g;
  }
  const int64_t grow = ((int64_t)a.bb * a.seqlen + t) * a.hq + h;
  bf16x8 qb[8], db[8];
  {
    const bf16raw* qr = reinterpret_cast<const bf16raw*>(a.q) + grow * BD + lg * 8;
    const bf16raw* dr = reinterpret_cast<const bf16raw*>(a.dout) + grow * BD + lg * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qb[s] = *reinterpret_cast<const bf16x8*>(qr + 16 * s);
      db[s] = *reinterpret_cast<const bf16x8*>(dr + 16 * s);
    }
  }
  const float lse2 = valid ? a.lse2[grow] : __builtin_inff();  // invalid rows: p = 0
  const float dl = a.delta[grow];
  f32x16 o[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[b][e] = 0.f;

  const int nsl_blk = a.block / BKT;
  int nsl = nsl_blk;
  if constexpr (kOwn) {
    // slices up to the tile's last position
    const int64_t last = own_p0 + (cnt + a.g - 1) / a.g - 1;
    nsl = (int)(last / BKT) + 1;
  }
  const int64_t img0 = (((int64_t)a.bb * a.hkv + hk) * (a.seqlen / BKT) + blk * nsl_blk) * (BKT * BD);
  const uint16_t* im[3] = {a.kimg + img0, a.vkimg + img0, a.kvimg + img0};
  const int kofs = lg * 1024 + (lane & 31) * 16;  // K-layout operand base (unit-major images)
  const int vofs = lg * 2048 + (lane & 31) * 16;  // V^T-layout operand base
  const float c = a.scale_log2;

  // The slices go from HBM straight into LDS (global_load_lds, written as
  // inline asm so the compiler neither tracks nor waits for them): the three
  // images, 3 x 1024 units of 16 bytes, are 6 units per thread; the 64 lanes
  // of a wave load 64 consecutive units of one image, so their LDS
  // destinations are one contiguous kilobyte at a wave-uniform base (m0).
  // The loads of slice s + 2 go out at the start of slice s; the wait before
  // each barrier leaves only the youngest slice's 6 loads in flight.  Past the
  // last slice the loads repeat it, so every iteration issues the same loads.
  auto dma = [&](char* lb, int sl) {
    const int64_t so = (int64_t)(sl < nsl ? sl : nsl - 1) * (BKT * BD);
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t lb_addr = (uint32_t)(uintptr_t)((lds_char*)lb);
#pragma unroll
    for (int x = 0; x < 6; ++x) {
      const int u0 = wave * 64 + 512 * x;  // this wave's first unit (0 .. 3071, one image)
      const int img = u0 >> 10, unit = (u0 & 1023) + lane;
      const uint32_t wb = __builtin_amdgcn_readfirstlane(lb_addr + (uint32_t)(img * BIMG + (u0 & 1023) * 16));
      lds_dma16(wb, im[img] + so + unit * 8);
    }
  };
  auto publish = [] { asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory"); };
  auto slice = [&](const char* buf, int sl) {
    // own block: key kc of the slice (slice-relative, accumulator row
    // kc + 4 lg) is visible iff kc <= lim, one int32 limit per slice
    int lim = 0;
    if constexpr (kOwn) lim = (int)own_p0 + rr / a.g - sl * BKT - 4 * lg;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(buf + kofs + st * 2048 + kb * 512);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(buf + BIMG + kofs + st * 2048 + kb * 512);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[st], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, db[st], dp, 0, 0, 0);
        // own block: operands read four steps at a time (the mask's registers
        // would otherwise push the kernel past 256)
        if constexpr (kOwn)
          if (st == 3) __builtin_amdgcn_sched_barrier(0);
      }
      // dS^T, packed as the B operand of dQ^T (same order as the forward's P^T)
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float p0 = fast_exp2(__builtin_fmaf(s[e], c, -lse2));
        float p1 = fast_exp2(__builtin_fmaf(s[e + 1], c, -lse2));
        if constexpr (kOwn) {
          const int kc = kb * 32 + 8 * (e >> 2) + (e & 3);
          if (kc > lim) p0 = 0.f;
          if (kc + 1 > lim) p1 = 0.f;
        }
        pk[e >> 1] = pack_bf16x2(p0 * (dp[e] - dl), p1 * (dp[e + 1] - dl));
      }
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * hs], pk[4 * hs + 1], pk[4 * hs + 2], pk[4 * hs + 3]});
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(buf + 2 * BIMG + vofs + (4 * kb + 2 * hs) * 2048 + b * 512);
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, pb, o[b], 0, 0, 0);
        }
      }
    }
  };

  drain_vmem();  // the rows' q and dout in before any slice load goes out
  dma(lbs[0], 0);
  dma(lbs[1], 1);
  publish();  // slice 0 in
  for (int sl = 0, cur = 0; sl < nsl; ++sl, cur = cur == 2 ? 0 : cur + 1) {
    dma(lbs[cur == 0 ? 2 : cur - 1], sl + 2);  // buffer (sl + 2) % 3; past the end: the last slice again
    slice(lbs[cur], sl);
    publish();  // slice sl + 1 in, in every wave
  }
  drain_vmem();  // every slice load landed before the work-group ends

  if (valid) {
    // the row's contribution slot: its past slot, or the own slot kp
    int64_t pidx;
    if constexpr (!kOwn) {
      const int64_t local_row = entry / a.kp;
      pidx = local_row * a.kps + entry % a.kp;
    } else {
      pidx = ((blk * a.block + own_p0 + rr / a.g - a.t0) * a.hq + h) * a.kps + a.kp;
    }
    // lane holds d = 32 b + 8 q + 4 lg + i (i = 0..3) of its row
    float* dst = a.dq_part + pidx * BD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(dst + 32 * b + 8 * q4 + 4 * lg) =
            f32x4{o[b][4 * q4] * a.scale, o[b][4 * q4 + 1] * a.scale, o[b][4 * q4 + 2] * a.scale,
                  o[b][4 * q4 + 3] * a.scale};
  }
}

// dq of the chunk's rows: the sum of the row's slot contributions, bf16.  One
// wave per row (two dims per lane).
__global__ __launch_bounds__(256) void bwd_dq_merge_kernel(BwdArgs a) {
  const int64_t lr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // chunk-local row
  const int lane = threadIdx.x & 63;
  if (lr >= a.cnt * a.hq) return;
  const int64_t t = a.t0 + lr / a.hq;
  const int h = (int)(lr % a.hq);
  const int64_t j = t / a.block;
  const int npast = a.causal ? (int)(j < a.kp ? j : a.kp) : a.kp;
  const float* src = a.dq_part + lr * a.kps * BD + 2 * lane;
  float x0 = 0.f, x1 = 0.f;
  for (int s = 0; s < npast; ++s) {
    const float2 v = *reinterpret_cast<const float2*>(src + s * BD);
    x0 += v.x;
    x1 += v.y;
  }
  if (a.causal) {
    const float2 v = *reinterpret_cast<const float2*>(src + a.kp * BD);
    x0 += v.x;
    x1 += v.y;
  }
  bf16raw* dst = reinterpret_cast<bf16raw*>(a.dq) + (((int64_t)a.bb * a.seqlen + t) * a.hq + h) * BD + 2 * lane;
  *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(x0, x1);
}

// ---------------------------------------------------------------------------
// dk, dv.  grid (n * ceil(block / 128), hkv): 128 keys of one block per
// work-group, 4 waves x 32 keys.
// ---------------------------------------------------------------------------
namespace {
constexpr int RSTEP = 32;        // rows per step
constexpr int RROW = BD * 2;     // bytes per staged row (16 units of 16 bytes)
constexpr int RTILE = RSTEP * RROW;  // one staged tensor (8 KiB)
constexpr int kKvGroups = 4;         // key groups (32 keys each) per work-group
constexpr int kKvKeys = 32 * kKvGroups;
constexpr int kKvThreads = 2 * 64 * kKvGroups;  // two waves per key group

// Position of 16-byte unit u of staged row r: a rotation per row that keeps
// both the row-wise 16-byte operand reads (16 rows, one unit) and the
// transposing 8-byte reads (4 rows x 4 units per 16 lanes) free of bank
// conflicts.
__device__ __forceinline__ int unit_pos(int r, int u) { return (u + 4 * (r & 3) + ((r >> 2) & 3)) & 15; }
__device__ __forceinline__ int row_off(int r, int u) { return r * RROW + unit_pos(r, u) * 16; }

// Division of a 32-bit x by a divisor d fixed for the whole kernel, as the
// high half of x * ceil(2^64 / d): with ceil(2^64 / d) = 2^64 / d + e,
// 0 <= e < 1, the product is x / d + x e / 2^64 and x e / 2^64 < 2^-32 < 1 / d,
// so the floor is exact for every x < 2^32 and d < 2^32 (d = 1 is x itself).
// It replaces the VALU division sequence in each step's row decoding.
__device__ __forceinline__ uint64_t div_magic(uint32_t d) { return d <= 1 ? 0ull : (~0ull / d + 1ull); }
__device__ __forceinline__ uint32_t div_by(uint32_t x, uint32_t d, uint64_t m) {
  return d <= 1 ? x : (uint32_t)__umul64hi((uint64_t)x, m);
}
}  // namespace

__global__ __launch_bounds__(kKvThreads) void bwd_dkdv_kernel(BwdArgs a) {
  // three row stages and two P hand-over buffers: one barrier per step (see
  // the loop below)
  __shared__ __attribute__((aligned(16))) char rs[3][2 * RTILE];  // [stage][Q rows | dO rows]
  __shared__ __attribute__((aligned(16))) float rl[3][RSTEP];
  __shared__ __attribute__((aligned(16))) float rd[3][RSTEP];
  __shared__ __attribute__((aligned(16))) int32_t rt[3][RSTEP];
  __shared__ __attribute__((aligned(16))) uint32_t pex[2][kKvGroups][64 * 8];  // P handed from P-wave to dS-wave
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 5;
  const int kg = wave % kKvGroups;   // key group (32 keys)
  const bool pw = wave < kKvGroups;  // P-wave (S, P, dV) or dS-wave (dP, dS, dK)
  const int hk = (int)blockIdx.y;
  const uint64_t m_kp = div_magic((uint32_t)a.kp), m_hq = div_magic((uint32_t)a.hq), m_g = div_magic((uint32_t)a.g);
  const int spb = (a.block + kKvKeys - 1) / kKvKeys;  // work-groups per block
  const int64_t i = blockIdx.x / spb;
  // (consecutive work-groups, one block's slices, go to different XCDs and
  // read the block's rows at about the same time; measured slower: an order
  // keeping a block on one XCD (2.4x: the early blocks' long lists then load
  // a few XCDs) and one with the KV head fastest (4 %))
  const int64_t key0 = i * a.block + (int64_t)(blockIdx.x % spb) * kKvKeys;  // first key of the work-group
  const int64_t wkey = key0 + kg * 32;                                    // first key of this wave's group
  // a block of 64 keys leaves key groups without keys (wave-uniform)
  const bool wact = wkey < (i + 1) * a.block;
  const int64_t rowstride = (int64_t)a.hkv * BD;
  const int64_t bS = (int64_t)a.bb * a.seqlen;

  // the group's keys (P-wave) or values (dS-wave) as the B operand of
  // S = Q K^T or dP = dO V^T: lane = key (l % 32), 8 dims at 8 lg + 16 s
  bf16x8 kv[8];
  if (wact) {
    const int64_t key = wkey + (lane & 31);
    const bf16raw* src = reinterpret_cast<const bf16raw*>(pw ? a.k : a.v) + (bS + key) * rowstride + hk * BD + lg * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) kv[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
  }
  f32x16 acc[4];  // dV (P-wave) or dK (dS-wave): M = key, N = dim
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

  // rows: the block's list, then (causal) its own rows at or after key0
  const int64_t L = (int64_t)hk * a.n + i;
  // (no past slots, kp = 0: the lists were not built)
  const int32_t lbeg = a.kp > 0 ? a.listoff_f[L] : 0;
  const int64_t npast = a.kp > 0 ? a.count_f[L] : 0;
  const int64_t own_pos0 = key0;                    // positions before key0 see none of these keys
  const int64_t nown = a.causal ? ((i + 1) * a.block - own_pos0) * a.g : 0;
  const int64_t nrows = npast + nown;
  const int64_t nsteps = (nrows + RSTEP - 1) / RSTEP;

  // Staging: 32 rows x 16 units x 2 tensors = 1024 units per step.  The
  // loads of step s + 2 are issued during step s (two steps to arrive), the
  // list entries that locate them during step s - 1.
  constexpr int SU = 512 / kKvThreads;  // units per thread and tensor
  struct Desc {
    int32_t raw[SU];   // list entry (past rows) or own-row index
    bool past[SU];
    bool val[SU];
  };
  struct Stage {
    u32x4 q[SU], d[SU];
    float l[SU], dl[SU];
    int32_t pos[SU];
  };
  // only loads here: the entries are decoded a step later, when they have
  // arrived (a decode right after the load would wait for it)
  auto desc_of = [&](int64_t step, Desc& D) {
#pragma unroll
    for (int x = 0; x < SU; ++x) {
      const int row = (tid + kKvThreads * x) >> 4;
      int64_t rix = step * RSTEP + row;
      D.val[x] = rix < nrows;
      if (!D.val[x]) rix = nrows - 1;  // padding rows repeat the last row (weight 0)
      D.past[x] = rix < npast;
      D.raw[x] = D.past[x] ? a.entries_f[lbeg + rix] : (int32_t)(rix - npast);
    }
  };
  auto load_stage = [&](const Desc& D, Stage& St) {
#pragma unroll
    for (int x = 0; x < SU; ++x) {
      int64_t grow;
      int32_t pos;
      if (D.past[x]) {
        // whole-sequence list: entry = row * kp + slot, row = position * hq + head
        const int32_t lr = (int32_t)div_by((uint32_t)D.raw[x], (uint32_t)a.kp, m_kp);
        pos = (int32_t)div_by((uint32_t)lr, (uint32_t)a.hq, m_hq);
        grow = bS * a.hq + lr;
      } else {
        const int32_t qg = (int32_t)div_by((uint32_t)D.raw[x], (uint32_t)a.g, m_g);
        const int32_t p = (int32_t)own_pos0 + qg;
        pos = p;
        grow = (bS + p) * a.hq + hk * a.g + (D.raw[x] - qg * a.g);
      }
      const int u = tid & 15;
      St.q[x] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16raw*>(a.q) + grow * BD + u * 8);
      St.d[x] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16raw*>(a.dout) + grow * BD + u * 8);
      St.l[x] = D.val[x] ? a.lse2[grow] : __builtin_inff();  // padding rows: p = 0
      St.dl[x] = a.delta[grow];
      St.pos[x] = pos;
    }
  };
  auto store_stage = [&](const Stage& St, int buf) {
#pragma unroll
    for (int x = 0; x < SU; ++x) {
      const int row = (tid + kKvThreads * x) >> 4, u = tid & 15;
      *reinterpret_cast<u32x4*>(rs[buf] + row_off(row, u)) = St.q[x];
      *reinterpret_cast<u32x4*>(rs[buf] + RTILE + row_off(row, u)) = St.d[x];
      if (u == 0) {
        rl[buf][row] = St.l[x];
        rd[buf][row] = St.dl[x];
        rt[buf][row] = St.pos[x];
      }
    }
  };

  const float c = a.scale_log2;
  // transposing reads: lane l supplies row 4 (l / 32) + (l % 16) / 4 (+ 8) of
  // a 16-row step and dims 32 dt + 16 ((l / 16) & 1) + 4 (l % 4) .. + 3
  const int tr_r = 4 * lg + ((lane & 15) >> 2);
  const int tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // element offset inside a 32-dim tile
  const int32_t mykey = (int32_t)(wkey + (lane & 31));       // position of this lane's key

  // phase 1: S (P-wave) or dP (dS-wave) = rows x this group's keys; the
  // P-wave turns S into P and hands it over through LDS
  auto phase1 = [&](int buf, int pb, f32x16& x) {
    uint32_t* myex = pex[pb][kg] + lane * 8;
    const char* rowsrc = rs[buf] + (pw ? 0 : RTILE);  // Q rows or dO rows
    // the row-operand reads four MFMAs ahead of their MFMAs (left alone the
    // compiler read each operand just before its MFMA); the fence keeps
    // phase 2's reads out of this pattern
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = 0.f;
    const int ar = lane & 31;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 ra = *reinterpret_cast<const bf16x8*>(rowsrc + row_off(ar, lg + 2 * st));
      x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra, kv[st], x, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (pw) {
      uint32_t pk[8];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // rows 8 q4 + 4 lg + 0..3 are consecutive: one 16-byte read per array
        const int r0 = 8 * q4 + 4 * lg;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&rl[buf][r0]);
        const u32x4 t4 = *reinterpret_cast<const u32x4*>(&rt[buf][r0]);
        float p[4];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          p[y] = fast_exp2(__builtin_fmaf(x[4 * q4 + y], c, -l4[y]));
          if (a.causal && mykey > (int32_t)t4[y]) p[y] = 0.f;
        }
        pk[2 * q4] = pack_bf16x2(p[0], p[1]);
        pk[2 * q4 + 1] = pack_bf16x2(p[2], p[3]);
      }
      *reinterpret_cast<u32x4*>(myex) = u32x4{pk[0], pk[1], pk[2], pk[3]};
      *reinterpret_cast<u32x4*>(myex + 4) = u32x4{pk[4], pk[5], pk[6], pk[7]};
    }
  };
  // phase 2: dV += P^T dO (P-wave) or dK += dS^T Q with dS = P (dP - delta)
  // (dS-wave); M = key, N = dim, K = row, the row operand read transposed
  auto phase2 = [&](int buf, int pb, const f32x16& x) {
    const uint32_t* myex = pex[pb][kg] + lane * 8;
    uint32_t av[8];
    {
      const u32x4 p0 = *reinterpret_cast<const u32x4*>(myex);
      const u32x4 p1 = *reinterpret_cast<const u32x4*>(myex + 4);
      const uint32_t pk[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      if (pw) {
#pragma unroll
        for (int y = 0; y < 8; ++y) av[y] = pk[y];
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int r0 = 8 * q4 + 4 * lg;
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&rd[buf][r0]);
          av[2 * q4] = pack_bf16x2(bf16lo(pk[2 * q4]) * (x[4 * q4] - d4[0]), bf16hi(pk[2 * q4]) * (x[4 * q4 + 1] - d4[1]));
          av[2 * q4 + 1] = pack_bf16x2(bf16lo(pk[2 * q4 + 1]) * (x[4 * q4 + 2] - d4[2]),
                                       bf16hi(pk[2 * q4 + 1]) * (x[4 * q4 + 3] - d4[3]));
        }
      }
    }
    const char* tsrc = rs[buf] + (pw ? RTILE : 0);  // dO rows (for dV) or Q rows (for dK)
    // the transposed row operands two MFMAs ahead (fenced from the reads above)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bf16x8 A = __builtin_bit_cast(bf16x8, u32x4{av[4 * st], av[4 * st + 1], av[4 * st + 2], av[4 * st + 3]});
      const int ra = 16 * st + tr_r, rb = ra + 8;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int col = 32 * dt + tr_c;  // element; unit col / 8, half (col / 4) & 1
        const int oa = row_off(ra, col >> 3) + ((col >> 2) & 1) * 8;
        const int ob = row_off(rb, col >> 3) + ((col >> 2) & 1) * 8;
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tsrc + oa));
        const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tsrc + ob));
        const bf16x8 B = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int x = 0; x < 6; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  Desc D;
  Stage SA, SB, SC;
  if (nsteps > 0) {
    desc_of(0, D);
    load_stage(D, SA);
    store_stage(SA, 0);
    if (nsteps > 1) {
      desc_of(1, D);
      load_stage(D, SA);  // step 1, stored at the end of step 0
    }
    if (nsteps > 2) {
      desc_of(2, D);
      load_stage(D, SB);  // step 2, stored at the end of step 1
    }
    if (nsteps > 3) desc_of(3, D);
  }
  __syncthreads();
  // Iteration s runs phase 2 of step s - 1 and then phase 1 of step s, and
  // ends with the one barrier of the step.  Step s's rows sit in stage s % 3
  // and its P in hand-over buffer s % 2; X holds step s + 1's rows (stored
  // before the barrier, read from iteration s + 1 on), Y step s + 2's, Z is
  // free and D locates step s + 3: a step's rows are loaded three iterations
  // before they are read.  A stage or P buffer is rewritten only after a
  // barrier that follows every read of its previous contents: stage
  // (s + 1) % 3 was last read by phase 2 of step s - 2 (iteration s - 1), P
  // buffer s % 2 by phase 2 of step s - 2 (iteration s - 1).
  f32x16 x;  // phase 1's S (P-wave) or dP (dS-wave) of the previous step
  auto iter = [&](int64_t s, Stage& X, Stage& Z) {
    if (s + 3 < nsteps) load_stage(D, Z);
    if (s + 4 < nsteps) desc_of(s + 4, D);
    if (s > 0 && wact) phase2((int)((s - 1) % 3), (int)((s - 1) & 1), x);
    if (wact) phase1((int)(s % 3), (int)(s & 1), x);
    if (s + 1 < nsteps) store_stage(X, (int)((s + 1) % 3));
    __syncthreads();
  };
  for (int64_t s = 0; s < nsteps; s += 3) {
    iter(s, SA, SC);
    if (s + 1 >= nsteps) break;
    iter(s + 1, SB, SA);
    if (s + 2 >= nsteps) break;
    iter(s + 2, SC, SB);
  }
  if (nsteps > 0 && wact) phase2((int)((nsteps - 1) % 3), (int)((nsteps - 1) & 1), x);

  if (!wact) return;
  // C layout of the accumulator: lane = dim 32 dt + lane % 32, element e = key acc_row(e, lg)
  bf16raw* dst = reinterpret_cast<bf16raw*>(pw ? a.dv : a.dk) + (bS + wkey) * rowstride + hk * BD + (lane & 31);
  const float f = pw ? 1.f : a.scale;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      dst[(int64_t)acc_row(e, lg) * rowstride + 32 * dt] = (bf16raw)(pack_bf16x2(acc[dt][e] * f, 0.f) & 0xffffu);
}

int launch_bwd_prep(const void* out, const void* dout, const float* lse, float* lse2, float* delta, int64_t batch,
                    int64_t seqlen, int hq, hipStream_t st) {
  const int64_t rows = batch * seqlen * hq;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                     reinterpret_cast<const bf16raw*>(out), reinterpret_cast<const bf16raw*>(dout), lse, lse2, delta,
                     rows, seqlen, hq);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bwd_dq(const BwdArgs& a, int64_t max_tiles, hipStream_t st) {
  if (max_tiles > 0) hipLaunchKernelGGL((bwd_dq_kernel<false>), dim3((unsigned)max_tiles), dim3(512), 0, st, a);
  if (a.causal) {
    const int ppt = 256 / a.g;
    const int64_t tpb = (a.block + ppt - 1) / ppt;
    const int64_t nblk = a.cnt / a.block;
    const int64_t per_xcd = (tpb * nblk * a.hkv + 7) / 8;  // see bwd_dq_kernel
    hipLaunchKernelGGL((bwd_dq_kernel<true>), dim3((unsigned)(8 * per_xcd)), dim3(512), 0, st, a);
  }
  const int64_t rows = a.cnt * a.hq;
  hipLaunchKernelGGL(bwd_dq_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bwd_dkdv(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)(a.n * ((a.block + kKvKeys - 1) / kKvKeys)), (unsigned)a.hkv),
                     dim3(kKvThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
