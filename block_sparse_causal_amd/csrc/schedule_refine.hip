// Refinement of a CSR block schedule over blocks of B = 64 m rows to the CSR over
// 64-row blocks that allows exactly the same keys.
//
// The pages validate the block size of a schedule ("Add topology-derived sparse
// attention kernel", triton-lang/kernels PR 22, Summary, fifth bullet) and
// benchmark at 64.  The attention kernels here work on 64 x 64 tiles, so a
// schedule over coarser blocks is handed to them refined: with I = i / m, fine
// row i lists m J + b (b = 0 .. m-1, m J + b <= i) for every block J that coarse
// row I lists.  Query t then sees key u <= t exactly when u / B is listed in row
// t / B, as under the coarse schedule.  An entry of a coarse row counts when the
// attention kernels would accept it (within 0..I and above every earlier entry of
// the row that lies in 0..I).
//
// Three launches, no atomics: per fine row (one wave) the entry count, written to
// row_ptr64[i + 1]; one workgroup turns the counts into offsets in place; per
// fine row the entries, each accepted coarse entry writing its run of sub-blocks
// at its rank.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tsa {
namespace {

constexpr int kScanThreads = 1024;

__device__ __forceinline__ int wave_max_scan(int x, int l) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (l >= d) x = max(x, y);
  }
  return x;
}
__device__ __forceinline__ int wave_sum_scan(int x, int l) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (l >= d) x += y;
  }
  return x;
}

// Walks the accepted entries of coarse row I, 64 at a time; calls f(J, valid)
// with every lane taking part (valid: the lane holds an accepted entry J).
template <typename F>
__device__ __forceinline__ void for_accepted(const int32_t* __restrict__ row_ptr,
                                             const int32_t* __restrict__ col_idx, int64_t nnz,
                                             int I, int l, F&& f) {
  const int p0 = (int)min((int64_t)max(row_ptr[I], 0), nnz);
  const int end = (int)max(min((int64_t)row_ptr[I + 1], nnz), (int64_t)p0);
  int carry = -1;
  for (int p = p0; p < end; p += 64) {
    const int idx = p + l;
    const int c = idx < end ? col_idx[idx] : -1;
    const bool valid = idx < end && c >= 0 && c <= I;
    const int incl = wave_max_scan(valid ? c : -1, l);
    int excl = __shfl_up(incl, 1, 64);
    if (l == 0) excl = -1;
    f(c, valid && c > max(carry, excl));
    carry = max(carry, __shfl(incl, 63, 64));
  }
}

__global__ __launch_bounds__(64) void refine_count_kernel(const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx,
                                                          int64_t nnz, int m,
                                                          int32_t* __restrict__ row_ptr64) {
  const int i = blockIdx.x, l = threadIdx.x, I = i / m;
  int cnt = 0;
  for_accepted(row_ptr, col_idx, nnz, I, l, [&](int J, bool ok) {
    if (ok) cnt += J < I ? m : i - m * I + 1;
  });
  const int total = __shfl(wave_sum_scan(cnt, l), 63, 64);
  if (l == 0) {
    row_ptr64[i + 1] = total;
    if (i == 0) row_ptr64[0] = 0;
  }
}

// In-place inclusive scan of row_ptr64[1 .. n] by one workgroup, in chunks of
// kScanThreads entries.  Each fine row holds at most i + 1 entries, so a chunk's
// sum fits int32; the running total is kept in int64 and stored saturated at
// INT32_MAX (reachable only when coarse rows share entries), which the host
// reports as an overflow of the output's capacity.
__global__ __launch_bounds__(kScanThreads) void refine_scan_kernel(int n, int32_t* __restrict__ row_ptr64) {
  __shared__ int wsum[kScanThreads / 64];
  __shared__ int64_t carry_s;
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kScanThreads) {
    const int k = base + t;
    const int x = k < n ? row_ptr64[k + 1] : 0;
    const int incl = wave_sum_scan(x, l);
    if (l == 63) wsum[w] = incl;
    __syncthreads();
    int64_t before = carry_s;
    for (int v = 0; v < w; ++v) before += wsum[v];
    if (k < n) row_ptr64[k + 1] = (int32_t)min(before + incl, (int64_t)INT32_MAX);
    __syncthreads();
    if (t == kScanThreads - 1) carry_s = before + incl;
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void refine_emit_kernel(const int32_t* __restrict__ row_ptr,
                                                         const int32_t* __restrict__ col_idx,
                                                         int64_t nnz, int m,
                                                         const int32_t* __restrict__ row_ptr64,
                                                         int32_t* __restrict__ col_idx64,
                                                         int64_t capacity) {
  const int i = blockIdx.x, l = threadIdx.x, I = i / m;
  int64_t pos = row_ptr64[i];
  for_accepted(row_ptr, col_idx, nnz, I, l, [&](int J, bool ok) {
    const int k = ok ? (J < I ? m : i - m * I + 1) : 0;
    const int incl = wave_sum_scan(k, l);
    const int64_t at = pos + incl - k;
    // rows that share input entries (a row_ptr that is not non-decreasing) can
    // push the total past the host's bound: such entries are counted, not written
    for (int b = 0; b < k; ++b)
      if (at + b < capacity) col_idx64[at + b] = m * J + b;
    pos += __shfl(incl, 63, 64);
  });
}

}  // namespace

hipError_t launch_refine_schedule(int64_t S, int block, const int32_t* row_ptr,
                                  const int32_t* col_idx, int64_t nnz, int32_t* row_ptr64,
                                  int32_t* col_idx64, int64_t capacity, hipStream_t stream) {
  const int64_t nb64 = (S + 63) / 64;
  const int m = block / 64;
  if (nb64 == 0) return launch_dense_schedule(0, row_ptr64, col_idx64, stream);  // row_ptr64 = {0}
  hipLaunchKernelGGL(refine_count_kernel, dim3((unsigned)nb64), dim3(64), 0, stream, row_ptr, col_idx,
                     nnz, m, row_ptr64);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(refine_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, (int)nb64, row_ptr64);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(refine_emit_kernel, dim3((unsigned)nb64), dim3(64), 0, stream, row_ptr, col_idx, nnz,
                     m, row_ptr64, col_idx64, capacity);
  return hipGetLastError();
}

}  // namespace tsa
