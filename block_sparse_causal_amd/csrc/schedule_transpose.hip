// Column view (CSC) of a causal CSR block schedule, on the GPU.
//
// The key/value gradients of key block j gather over the query blocks whose
// rows list j (the backward of the forward over the CSR schedule of "Add
// topology-derived sparse attention kernel", triton-lang/kernels PR 22, Summary,
// first bullet).  Column j lists those query blocks i in ascending order.  An
// entry of row i counts when the attention kernels accept it: it lies in 0..i
// and exceeds every earlier entry of the row that lies in 0..i (for a row that
// is strictly ascending within 0..i, as the schedule contract asks, that is
// every entry).
//
// Three launches, no atomics on global memory, deterministic:
//   row_bits    one wave per row i: accepted entries -> bit j of a 32-bit word
//               (i, j / 32); words are stored word-group-major, bits[w * nb + i],
//               and only the groups w <= i / 32 a row can touch are written.
//   col_count   one wave per word group w (columns 32w .. 32w+31): for 64 rows at
//               a time, one ballot per column bit gives the rows that list it.
//   col_emit    one wave per word group: the exclusive prefix of all earlier
//               columns' counts (column pointers), then the same ballots again,
//               each set bit writing its row at its rank.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tsa {
namespace {

constexpr int kMaxWords = 4096 / 32;  // word groups of the largest schedule (4096 blocks)

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

__global__ __launch_bounds__(64) void row_bits_kernel(const int32_t* __restrict__ row_ptr,
                                                      const int32_t* __restrict__ col_idx,
                                                      int64_t nnz, int nb,
                                                      uint32_t* __restrict__ bits) {
  __shared__ uint32_t words[kMaxWords];
  const int i = blockIdx.x;
  const int l = threadIdx.x;
  const int nw = (i >> 5) + 1;
  for (int w = l; w < nw; w += 64) words[w] = 0u;
  __syncthreads();
  const int p0 = (int)min((int64_t)max(row_ptr[i], 0), nnz);
  const int end = (int)max(min((int64_t)row_ptr[i + 1], nnz), (int64_t)p0);
  int carry = -1;  // largest entry in 0..i seen so far
  for (int p = p0; p < end; p += 64) {
    const int idx = p + l;
    const int c = idx < end ? col_idx[idx] : -1;
    const bool valid = idx < end && c >= 0 && c <= i;
    const int incl = wave_max_scan(valid ? c : -1, l);
    int excl = __shfl_up(incl, 1, 64);
    if (l == 0) excl = -1;
    if (valid && c > max(carry, excl)) atomicOr(&words[c >> 5], 1u << (c & 31));
    carry = max(carry, __shfl(incl, 63, 64));
  }
  __syncthreads();
  for (int w = l; w < nw; w += 64) bits[(int64_t)w * nb + i] = words[w];
}

// Counts of columns 32w .. 32w+31 (lane b holds column 32w + b).  Rows below 32w
// cannot list these columns and are not read.
__device__ __forceinline__ int column_counts(const uint32_t* __restrict__ bits, int nb, int w, int l) {
  int mine = 0;
  for (int i0 = 32 * w; i0 < nb; i0 += 64) {
    const int i = i0 + l;
    const uint32_t word = i < nb ? bits[(int64_t)w * nb + i] : 0u;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      const int c = __popcll(__ballot((word >> b) & 1u));
      if (l == b) mine += c;
    }
  }
  return mine;
}

__global__ __launch_bounds__(64) void col_count_kernel(const uint32_t* __restrict__ bits, int nb,
                                                       int32_t* __restrict__ counts) {
  const int w = blockIdx.x, l = threadIdx.x;
  const int mine = column_counts(bits, nb, w, l);
  if (l < 32 && 32 * w + l < nb) counts[32 * w + l] = mine;
}

// Entries at or past `capacity` are counted in col_ptr but not written: a
// row_ptr that is not non-decreasing lets rows share entries, and then the
// column view can hold more entries than the CSR has.
__global__ __launch_bounds__(64) void col_emit_kernel(const uint32_t* __restrict__ bits,
                                                      const int32_t* __restrict__ counts, int nb,
                                                      int32_t* __restrict__ col_ptr,
                                                      int32_t* __restrict__ row_idx, int64_t capacity) {
  const int w = blockIdx.x, l = threadIdx.x;
  int part = 0;
  for (int c = l; c < 32 * w; c += 64) part += counts[c];
  const int before = __shfl(wave_sum_scan(part, l), 63, 64);
  const int col = 32 * w + l;
  const int cnt = (l < 32 && col < nb) ? counts[col] : 0;
  const int incl = wave_sum_scan(cnt, l);
  const int start = before + incl - cnt;
  const int total = before + __shfl(incl, 63, 64);  // every lane takes part in the shuffle
  if (l < 32 && col < nb) col_ptr[col] = start;
  if (w == (int)gridDim.x - 1 && l == 0) col_ptr[nb] = total;
  int run[32];
#pragma unroll
  for (int b = 0; b < 32; ++b) run[b] = __builtin_amdgcn_readlane(start, b);
  for (int i0 = 32 * w; i0 < nb; i0 += 64) {
    const int i = i0 + l;
    const uint32_t word = i < nb ? bits[(int64_t)w * nb + i] : 0u;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      const bool set = (word >> b) & 1u;
      const uint64_t m = __ballot(set);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (set && run[b] + below < capacity) row_idx[run[b] + below] = i;
      run[b] += __popcll(m);
    }
  }
}

}  // namespace

size_t transpose_workspace_bytes(int64_t nb) {
  const int64_t nw = (nb + 31) / 32;
  return (size_t)((nw * nb + nb) * 4);
}

hipError_t launch_schedule_transpose(int64_t nb, const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t nnz, int32_t* col_ptr, int32_t* row_idx,
                                     int64_t row_capacity, void* workspace, hipStream_t stream) {
  const int64_t nw = (nb + 31) / 32;
  uint32_t* bits = (uint32_t*)workspace;
  int32_t* counts = (int32_t*)(bits + nw * nb);
  if (nb > 0) {
    hipLaunchKernelGGL(row_bits_kernel, dim3((unsigned)nb), dim3(64), 0, stream, row_ptr, col_idx, nnz,
                       (int)nb, bits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(col_count_kernel, dim3((unsigned)nw), dim3(64), 0, stream, bits, (int)nb, counts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(col_emit_kernel, dim3((unsigned)(nw > 0 ? nw : 1)), dim3(64), 0, stream, bits, counts,
                     (int)nb, col_ptr, row_idx, row_capacity);
  return hipGetLastError();
}

}  // namespace tsa
