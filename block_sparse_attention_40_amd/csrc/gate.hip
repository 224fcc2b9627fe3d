// MoBA gate (deep-dive report on MoBA, sections 2.2 and 2.3): fp32 scores
// s_i = <q, mu_i>, exclusion of future blocks, the forced own block, and a
// hard top-k with ties broken towards the lower block index.
//
// One work-group handles `gate_t` consecutive query positions of one KV head
// and all query heads of its group (one row per thread), so the block means
// of that KV head are staged once in LDS (in slices of kMuSlice blocks) and
// read by every row with broadcast loads.  Each thread keeps its running
// top-m list in registers as 64-bit keys (orderable score << 32 | ~index):
// a larger key is a larger score, and between equal scores the lower block
// index, which is exactly the tie rule.
//
// Besides sel_idx the kernel writes, per work-group, how many of its rows
// chose each block (used to build the per-block row lists).
#include "moba_device.h"
#include "moba_kernels.h"

namespace moba {

constexpr int kMuSlice = 32;  // block means staged in LDS at a time

template <typename T, int D, int KCAP>
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
  extern __shared__ float smem[];
  float* mu_s = smem;                                      // [kMuSlice][D]
  int* lhist = reinterpret_cast<int*>(smem + kMuSlice * D);  // [n]
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
    const float* mu_h = a.mu + ((int64_t)a.bb * a.hkv + hk) * n * D;
    for (int64_t c0 = 0; c0 < wg_cand; c0 += kMuSlice) {
      const int64_t c1 = (c0 + kMuSlice < wg_cand) ? c0 + kMuSlice : wg_cand;
      __syncthreads();
      const int nel = (int)(c1 - c0) * D;
      for (int e = tid * 4; e < nel; e += 256 * 4)
        *reinterpret_cast<f32x4*>(mu_s + e) = *reinterpret_cast<const f32x4*>(mu_h + c0 * D + e);
      __syncthreads();
      if (rank) {
        const int64_t cend = ncand < c1 ? ncand : c1;
        for (int64_t i = c0; i < cend; ++i) {
          const float* mrow = mu_s + (i - c0) * D;
          float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
          for (int d0 = 0; d0 < D; d0 += 4) {
            f32x4 mv = *reinterpret_cast<const f32x4*>(mrow + d0);
            s0 = __builtin_fmaf(qr[d0 + 0], mv[0], s0);
            s1 = __builtin_fmaf(qr[d0 + 1], mv[1], s1);
            s2 = __builtin_fmaf(qr[d0 + 2], mv[2], s2);
            s3 = __builtin_fmaf(qr[d0 + 3], mv[3], s3);
          }
          float s = (s0 + s1) + (s2 + s3);
          if (s != s) s = -__builtin_inff();  // NaN ranks lowest
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
    int32_t* dst = a.hist + ((int64_t)hk * a.gate_wg + w) * n;
    for (int64_t i = tid; i < n; i += 256) dst[i] = lhist[i];
  }
}

template <typename T, int D>
static void launch_gate_kcap(const GateArgs& a, int kcap, size_t shmem, hipStream_t st, dim3 grid) {
  if (kcap <= 4)
    hipLaunchKernelGGL((gate_kernel<T, D, 4>), grid, dim3(256), shmem, st, a);
  else if (kcap <= 16)
    hipLaunchKernelGGL((gate_kernel<T, D, 16>), grid, dim3(256), shmem, st, a);
  else
    hipLaunchKernelGGL((gate_kernel<T, D, 32>), grid, dim3(256), shmem, st, a);
}

int launch_gate(const GateArgs& a, int dtype, int d, hipStream_t st) {
  dim3 grid((unsigned)a.gate_wg, (unsigned)a.hkv);
  const size_t shmem = (size_t)kMuSlice * d * sizeof(float) + (a.hist ? (size_t)a.n * sizeof(int) : 0);
  const int kcap = a.kp < 1 ? 1 : a.kp;
  if (dtype == 1) {
    launch_gate_kcap<bf16raw, 128>(a, kcap, shmem, st, grid);
  } else if (d == 64) {
    launch_gate_kcap<float, 64>(a, kcap, shmem, st, grid);
  } else {
    launch_gate_kcap<float, 128>(a, kcap, shmem, st, grid);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
