// MoE-style dispatch of query rows to key blocks (deep-dive report on MoBA,
// section 3.2: the implementation groups work per selected block the way an
// MoE layer dispatches tokens to experts).
//
// For one query chunk, list (hk, i) collects every (row, slot) whose row is
// served by KV head hk and chose block i as a non-own block.  Three steps,
// all on the device (no host round trip):
//   1. list_scan:  per list (one work-group each), exclusive prefix over the
//                  gate work-groups of their counts for that list (written
//                  contiguous per list by the gate, or by hist_kernel from
//                  the selection: for the backward, and beyond 8192 blocks);
//   2. tile_plan:  one work-group scans the list sizes into list offsets and
//                  cuts every list into tiles of tile_rows rows;
//   3. scatter:    every row writes its (row, slot) entries into its lists at
//                  (list offset + work-group start + local rank).
// The order inside a work-group's stretch of a list may vary between runs;
// each entry is computed independently, so results do not.
#include "moba_device.h"
#include "moba_kernels.h"
#include "moba_plan.h"

namespace moba {

// Exclusive block scan of 1024 values in LDS (Hillis-Steele).
__device__ __forceinline__ int32_t block_excl_scan_1024(int32_t x, int32_t* buf, int32_t* total) {
  const int tid = threadIdx.x;
  buf[tid] = x;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t y = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += y;
    __syncthreads();
  }
  const int32_t incl = buf[tid];
  *total = buf[1023];
  __syncthreads();
  return incl - x;
}

// One work-group per list: exclusive prefix over the gate work-groups of
// their counts for this list (contiguous), in place; the total goes to count.
__global__ __launch_bounds__(1024) void list_scan_kernel(int32_t* __restrict__ hist, int32_t* __restrict__ count,
                                                         int64_t gate_wg) {
  __shared__ int32_t buf[1024];
  const int64_t L = blockIdx.x;
  int32_t* col = hist + L * gate_wg;
  int32_t carry = 0;
  for (int64_t base = 0; base < gate_wg; base += 1024) {
    const int64_t w = base + threadIdx.x;
    const int32_t c = w < gate_wg ? col[w] : 0;
    int32_t tot;
    const int32_t ex = block_excl_scan_1024(c, buf, &tot);
    if (w < gate_wg) col[w] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) count[L] = carry;
}

__global__ __launch_bounds__(1024) void tile_plan_kernel(const int32_t* __restrict__ count,
                                                         int32_t* __restrict__ listoff,
                                                         int32_t* __restrict__ tiles, int64_t lists,
                                                         int32_t tile_rows) {
  __shared__ int32_t buf[1024];
  int32_t carry_e = 0, carry_t = 0;
  for (int64_t base = 0; base < lists; base += 1024) {
    const int64_t L = base + threadIdx.x;
    const int32_t c = L < lists ? count[L] : 0;
    const int32_t nt = (c + tile_rows - 1) / tile_rows;
    int32_t tot_e, tot_t;
    const int32_t ex_e = block_excl_scan_1024(c, buf, &tot_e);
    const int32_t ex_t = block_excl_scan_1024(nt, buf, &tot_t);
    if (L < lists) {
      const int32_t off = carry_e + ex_e;
      listoff[L] = off;
      for (int32_t t = 0; t < nt; ++t) {
        tiles[8 + 2 * (carry_t + ex_t + t)] = (int32_t)L;
        tiles[9 + 2 * (carry_t + ex_t + t)] = off + t * tile_rows;
      }
    }
    carry_e += tot_e;
    carry_t += tot_t;
  }
  if (threadIdx.x == 0) {
    listoff[lists] = carry_e;
    tiles[0] = carry_t;
  }
}

// The (row, slot) entries of one gate work-group's rows: each row's s-th
// valid past block (ascending in its selection) is slot s.  Entries that can
// never be a valid choice (a block beyond the sequence, or after the own
// block) are skipped, so a malformed selection given to the backward stays
// inside the lists; the own block is handled by the own-block kernel.
// body(i, slot) is called for each remaining entry of a valid row.
template <typename Body>
__device__ __forceinline__ void for_each_past_entry(const DispatchArgs& a, const int32_t* row, int64_t j,
                                                    Body&& body) {
  int slot = 0;
  for (int c = 0; c < a.topk && slot < a.kp; ++c) {
    const int32_t i = row[c];
    if (i < 0) break;
    if (i >= a.n || (a.causal && i > j)) continue;
    if (a.causal && i == j) continue;
    body(i, slot);
    ++slot;
  }
}

// Blocks are counted in ranges of kDispatchRange (the LDS counters), one pass
// over the rows' selection per range; below that many blocks, one pass.
__global__ __launch_bounds__(256) void scatter_kernel(DispatchArgs a) {
  extern __shared__ int32_t lcnt[];  // [min(n, kDispatchRange)]
  const int tid = threadIdx.x;
  const int64_t w = blockIdx.x;
  const int hk = blockIdx.y;
  const int64_t n = a.n;
  const int g = a.g;
  const int64_t pic = w * a.gate_t + tid / g;
  const int h = hk * g + tid % g;
  const bool valid = tid < a.gate_t * g && pic < a.cnt;
  const int64_t t = a.t0 + (valid ? pic : 0);
  const int64_t j = t / a.block;
  const int32_t* row = a.sel + (int64_t)h * a.sel_stride_h + (t - a.sel_pos_base) * a.topk;
  const int32_t* wstart = a.hist + (int64_t)hk * n * a.gate_wg + w;  // list i: wstart[i * gate_wg]
  const int64_t local_row = pic * a.hq + h;
  for (int64_t r0 = 0; r0 < n; r0 += kDispatchRange) {
    const int64_t len = n - r0 < kDispatchRange ? n - r0 : kDispatchRange;
    for (int64_t i = tid; i < len; i += 256) lcnt[i] = 0;
    __syncthreads();
    if (valid)
      for_each_past_entry(a, row, j, [&](int32_t i, int slot) {
        if (i < r0 || i >= r0 + len) return;
        const int32_t r = atomicAdd(&lcnt[i - r0], 1);
        const int64_t L = (int64_t)hk * n + i;
        a.entries[a.listoff[L] + wstart[(int64_t)i * a.gate_wg] + r] = (int32_t)(local_row * a.kp + slot);
      });
    __syncthreads();  // the next range clears the counters
  }
}

// Counts per (list, gate work-group) from the selection alone: the same rows
// per work-group as the gate and the scatter, written contiguous per list.
__global__ __launch_bounds__(256) void hist_kernel(DispatchArgs a) {
  extern __shared__ int32_t lcnt[];  // [min(n, kDispatchRange)]
  const int tid = threadIdx.x;
  const int64_t w = blockIdx.x;
  const int hk = blockIdx.y;
  const int64_t n = a.n;
  const int g = a.g;
  const int64_t pic = w * a.gate_t + tid / g;
  const int h = hk * g + tid % g;
  const bool valid = tid < a.gate_t * g && pic < a.cnt;
  const int64_t t = a.t0 + (valid ? pic : 0);
  const int64_t j = t / a.block;
  const int32_t* row = a.sel + (int64_t)h * a.sel_stride_h + (t - a.sel_pos_base) * a.topk;
  int32_t* dst = a.hist + (int64_t)hk * n * a.gate_wg + w;
  for (int64_t r0 = 0; r0 < n; r0 += kDispatchRange) {
    const int64_t len = n - r0 < kDispatchRange ? n - r0 : kDispatchRange;
    for (int64_t i = tid; i < len; i += 256) lcnt[i] = 0;
    __syncthreads();
    if (valid)
      for_each_past_entry(a, row, j, [&](int32_t i, int) {
        if (i >= r0 && i < r0 + len) atomicAdd(&lcnt[i - r0], 1);
      });
    __syncthreads();
    for (int64_t i = tid; i < len; i += 256) dst[(r0 + i) * a.gate_wg] = lcnt[i];
    __syncthreads();  // the next range clears the counters
  }
}

static size_t range_lds(const DispatchArgs& a) {
  return (size_t)(a.n < kDispatchRange ? a.n : kDispatchRange) * sizeof(int32_t);
}

int launch_dispatch_from_sel(const DispatchArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(hist_kernel, dim3((unsigned)a.gate_wg, (unsigned)a.hkv), dim3(256), range_lds(a), st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  return launch_dispatch(a, st);
}

int launch_dispatch(const DispatchArgs& a, hipStream_t st) {
  const int64_t lists = (int64_t)a.hkv * a.n;
  hipLaunchKernelGGL(list_scan_kernel, dim3((unsigned)lists), dim3(1024), 0, st, a.hist, a.count, a.gate_wg);
  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(1024), 0, st, a.count, a.listoff, a.tiles, lists,
                     a.tile_rows);
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)a.gate_wg, (unsigned)a.hkv), dim3(256), range_lds(a), st,
                     a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moba
