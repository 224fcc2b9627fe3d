// Block mean of the keys (deep-dive report on MoBA, section 2.2: each block
// is summarised by the mean-pooled key).  HBM-bound: every key is read once.
//
// One work-group owns one block i of one batch entry and a slice of the
// row width W = num_kv_heads * head_dim.  Its 256 threads are split into
// R row groups x C column threads; a column thread owns 8 consecutive
// elements (one 16-byte load for bf16) and sums every R-th key row of the
// block in fp32 registers.  The R partial sums are then added in LDS in a
// fixed order, so the result does not depend on scheduling.
#include "moba_device.h"
#include "moba_kernels.h"

namespace moba {

template <typename T>
__global__ __launch_bounds__(256) void meanpool_kernel(const T* __restrict__ k, float* __restrict__ mu,
                                                       int64_t seqlen, int hkv, int d, int block,
                                                       int cols, int wv) {
  // cols: column threads per WG (C), wv: row width in 8-element units
  __shared__ float red[256 * 8];
  const int tid = threadIdx.x;
  const int R = 256 / cols;
  const int rg = tid / cols;
  const int c = tid % cols;
  const int v = blockIdx.y * cols + c;      // 8-element column unit
  const int64_t i = blockIdx.x;             // block index
  const int64_t bb = blockIdx.z;            // batch entry
  const int64_t W = (int64_t)hkv * d;
  const int64_t n = seqlen / block;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (v < wv && rg < R) {
    const T* base = k + ((bb * seqlen) + i * block) * W + (int64_t)v * 8;
    int s = rg;
    // four rows in flight per step
    for (; s + 3 * R < block; s += 4 * R) {
      float x0[8], x1[8], x2[8], x3[8];
      load8(base + (int64_t)s * W, x0);
      load8(base + (int64_t)(s + R) * W, x1);
      load8(base + (int64_t)(s + 2 * R) * W, x2);
      load8(base + (int64_t)(s + 3 * R) * W, x3);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x0[e];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x1[e];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x2[e];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x3[e];
    }
    for (; s < block; s += R) {
      float x0[8];
      load8(base + (int64_t)s * W, x0);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x0[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[(rg * cols + c) * 8 + e] = acc[e];
  __syncthreads();
  if (rg == 0 && v < wv) {
    float sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = red[c * 8 + e];
    for (int r = 1; r < R; ++r) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += red[(r * cols + c) * 8 + e];
    }
    const float den = (float)block;
    const int64_t col = (int64_t)v * 8;    // first element of this unit
    const int64_t hk = col / d;
    const int64_t dd = col % d;            // 8 | d, so the unit stays in one head
    float* dst = mu + ((bb * hkv + hk) * n + i) * d + dd;
    f32x4 o0, o1;
#pragma unroll
    for (int e = 0; e < 4; ++e) { o0[e] = sum[e] / den; o1[e] = sum[4 + e] / den; }
    *reinterpret_cast<f32x4*>(dst) = o0;
    *reinterpret_cast<f32x4*>(dst + 4) = o1;
  }
}

// Element-wise minimum and maximum of each block's keys (the Quest-style
// gate's pooling, report §1.3), same work split as the mean.  Exact: the
// results are input values.  lohi: [batch, hkv, n, 2, d] (min, then max).
template <typename T>
__global__ __launch_bounds__(256) void minmaxpool_kernel(const T* __restrict__ k, float* __restrict__ lohi,
                                                         int64_t seqlen, int hkv, int d, int block, int cols,
                                                         int wv) {
  __shared__ float rlo[256 * 8];
  __shared__ float rhi[256 * 8];
  const int tid = threadIdx.x;
  const int R = 256 / cols;
  const int rg = tid / cols;
  const int c = tid % cols;
  const int v = blockIdx.y * cols + c;
  const int64_t i = blockIdx.x;
  const int64_t bb = blockIdx.z;
  const int64_t W = (int64_t)hkv * d;
  const int64_t n = seqlen / block;
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { lo[e] = __builtin_inff(); hi[e] = -__builtin_inff(); }
  if (v < wv && rg < R) {
    const T* base = k + ((bb * seqlen) + i * block) * W + (int64_t)v * 8;
    int s = rg;
    for (; s + R < block; s += 2 * R) {
      float x0[8], x1[8];
      load8(base + (int64_t)s * W, x0);
      load8(base + (int64_t)(s + R) * W, x1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = __builtin_fminf(lo[e], __builtin_fminf(x0[e], x1[e]));
        hi[e] = __builtin_fmaxf(hi[e], __builtin_fmaxf(x0[e], x1[e]));
      }
    }
    for (; s < block; s += R) {
      float x0[8];
      load8(base + (int64_t)s * W, x0);
#pragma unroll
      for (int e = 0; e < 8; ++e) { lo[e] = __builtin_fminf(lo[e], x0[e]); hi[e] = __builtin_fmaxf(hi[e], x0[e]); }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) { rlo[(rg * cols + c) * 8 + e] = lo[e]; rhi[(rg * cols + c) * 8 + e] = hi[e]; }
  __syncthreads();
  if (rg == 0 && v < wv) {
    for (int r = 1; r < R; ++r) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = __builtin_fminf(lo[e], rlo[(r * cols + c) * 8 + e]);
        hi[e] = __builtin_fmaxf(hi[e], rhi[(r * cols + c) * 8 + e]);
      }
    }
    const int64_t col = (int64_t)v * 8;
    const int64_t hk = col / d;
    const int64_t dd = col % d;
    float* dst = lohi + (((bb * hkv + hk) * n + i) * 2) * d + dd;
    *reinterpret_cast<f32x4*>(dst) = f32x4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{lo[4], lo[5], lo[6], lo[7]};
    *reinterpret_cast<f32x4*>(dst + d) = f32x4{hi[0], hi[1], hi[2], hi[3]};
    *reinterpret_cast<f32x4*>(dst + d + 4) = f32x4{hi[4], hi[5], hi[6], hi[7]};
  }
}

int launch_minmaxpool(const void* k, int dtype, int64_t batch, int64_t seqlen, int hkv, int d, int block,
                      float* lohi, hipStream_t stream) {
  const int wv = hkv * d / 8;
  const int cols = wv < 64 ? wv : 64;
  dim3 grid((unsigned)(seqlen / block), (wv + cols - 1) / cols, (unsigned)batch);
  if (dtype == 1)
    hipLaunchKernelGGL(minmaxpool_kernel<bf16raw>, grid, dim3(256), 0, stream, (const bf16raw*)k, lohi, seqlen,
                       hkv, d, block, cols, wv);
  else
    hipLaunchKernelGGL(minmaxpool_kernel<float>, grid, dim3(256), 0, stream, (const float*)k, lohi, seqlen, hkv,
                       d, block, cols, wv);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_meanpool(const void* k, int dtype, int64_t batch, int64_t seqlen, int hkv, int d, int block,
                    float* mu, hipStream_t stream) {
  const int wv = hkv * d / 8;
  const int cols = wv < 64 ? wv : 64;
  dim3 grid((unsigned)(seqlen / block), (wv + cols - 1) / cols, (unsigned)batch);
  if (dtype == 1)
    hipLaunchKernelGGL(meanpool_kernel<bf16raw>, grid, dim3(256), 0, stream, (const bf16raw*)k, mu, seqlen,
                       hkv, d, block, cols, wv);
  else
    hipLaunchKernelGGL(meanpool_kernel<float>, grid, dim3(256), 0, stream, (const float*)k, mu, seqlen, hkv,
                       d, block, cols, wv);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
