// fp32 attention of the MoBA forward (deep-dive report on MoBA, section 2.2:
// softmax attention over the union of the chosen blocks; section 2.3: causal
// mask inside the own block).  This is the full-precision path for fp32
// inputs (head_dim 64 or 128); it is not the throughput path.
//
// One wave per query row.  The row's chosen blocks are read from sel_idx and
// walked in ascending order, 64 keys at a time: lane l scores key k0 + l with
// a full fp32 dot product, the wave agrees on the slice max and sum with
// butterfly reductions, and then every lane accumulates its own output
// coordinates (d = lane, and lane + 64 when D = 128) over the 64 keys.
#include "moba_device.h"
#include "moba_kernels.h"

namespace moba {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(F32Args a) {
  constexpr int NPL = D / 64;  // output coordinates per lane
  const int lane = threadIdx.x & 63;
  const int64_t rid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rid >= a.cnt * a.hq) return;
  const int64_t pic = rid / a.hq;
  const int h = (int)(rid % a.hq);
  const int64_t t = a.t0 + pic;
  const int64_t j = t / a.block;
  const int hk = h / a.g;
  const float* qrow = a.q + ((a.bb * a.seqlen + t) * a.hq + h) * D;
  const int64_t rs = (int64_t)a.hkv * D;
  const float* kb = a.k + (a.bb * a.seqlen) * rs + hk * D;
  const float* vb = a.v + (a.bb * a.seqlen) * rs + hk * D;
  float qv[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(qrow + d);
    qv[d] = x[0]; qv[d + 1] = x[1]; qv[d + 2] = x[2]; qv[d + 3] = x[3];
  }
  float m = -__builtin_inff(), l = 0.f, o[NPL];
#pragma unroll
  for (int x = 0; x < NPL; ++x) o[x] = 0.f;
  const int32_t* sel = a.sel + (int64_t)h * a.sel_stride_h + (t - a.sel_pos_base) * a.topk;
  for (int c = 0; c < a.topk; ++c) {
    const int32_t i = sel[c];
    if (i < 0) break;
    const int64_t kbeg = (int64_t)i * a.block;
    const int64_t kend = (a.causal && i == j) ? t + 1 : kbeg + a.block;
    for (int64_t k0 = kbeg; k0 < kend; k0 += 64) {
      const int64_t key = k0 + lane;
      float x = -__builtin_inff();
      if (key < kend) {
        const float* kr = kb + key * rs;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + d);
          s0 = __builtin_fmaf(qv[d], kv[0], s0);
          s1 = __builtin_fmaf(qv[d + 1], kv[1], s1);
          s2 = __builtin_fmaf(qv[d + 2], kv[2], s2);
          s3 = __builtin_fmaf(qv[d + 3], kv[3], s3);
        }
        x = ((s0 + s1) + (s2 + s3)) * a.scale_log2;
      }
      const float m_new = __builtin_fmaxf(m, wave_max(x));
      const float alpha = fast_exp2(m - m_new);
      const float p = fast_exp2(x - m_new);
      l = l * alpha + wave_sum(p);
      m = m_new;
#pragma unroll
      for (int xo = 0; xo < NPL; ++xo) o[xo] *= alpha;
      const int nk = (kend - k0) < 64 ? (int)(kend - k0) : 64;
      for (int u = 0; u < nk; ++u) {
        const float pu = __shfl(p, u);
        const float* vr = vb + (k0 + u) * rs;
#pragma unroll
        for (int xo = 0; xo < NPL; ++xo) o[xo] = __builtin_fmaf(pu, vr[lane + 64 * xo], o[xo]);
      }
    }
  }
  float* orow = a.out + ((a.bb * a.seqlen + t) * a.hq + h) * D;
  const float inv = 1.f / l;
  // the row's log-sum-exp of the scaled logits, natural log (for the backward)
  if (a.lse && lane == 0) a.lse[((int64_t)a.bb * a.hq + h) * a.seqlen + t] = (m + fast_log2(l)) * 0.6931471805599453f;
#pragma unroll
  for (int xo = 0; xo < NPL; ++xo) orow[lane + 64 * xo] = o[xo] * inv;
}

int launch_attn_f32(const F32Args& a, hipStream_t st) {
  const int64_t rows = a.cnt * a.hq;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (a.d == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
