// GPU builder of the topology-derived CSR block schedule (gfx950).
//
// Follows "Add topology-derived sparse attention kernel" (triton-lang/kernels
// PR 22), Summary, second bullet: sink blocks + local-window blocks + the
// top-k key blocks ranked by a 0D-persistence salience of the key-block
// centroids.  Salience is the elder rule of the mirror page's Rust-port commit
// note, computed from minimum-spanning-tree edges as in its schedule.py commit
// note (same result as single linkage over all pairs).
//
// Three kernels on the caller's stream:
//   centroid_kernel  one workgroup per key block: fp64 mean of the block's keys.
//   distance_kernel  all pairwise Euclidean distances between centroids (fp64),
//                    from the coordinate differences.
//   topology_kernel  one wavefront: Prim's MST, then the MST edges in ascending
//                    (length, lower index, higher index) order through the
//                    elder-rule union-find, then top-k, then CSR emission.
// Per-block state of the single wavefront lives in registers: block v belongs
// to lane v % 64, slot v / 64.  Cross-lane minima use DPP / swizzle / permlane
// exchanges, so each sequential step costs a few dozen instructions.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tsa {
namespace {

constexpr int kBlock = 64;
constexpr int kTieShift = 16;  // edge tie key = lower * 2^16 + higher (blocks < 2^16)

__device__ __forceinline__ double key_to_double(uint16_t bits, bool bf16) {
  if (bf16) return (double)__uint_as_float((uint32_t)bits << 16);
  return (double)__builtin_bit_cast(_Float16, bits);
}

// ------------------------------------------------------------------ centroids

__global__ __launch_bounds__(64) void centroid_kernel(const uint16_t* __restrict__ keys, bool bf16,
                                                      int64_t S, int64_t D,
                                                      double* __restrict__ cent) {
  const int64_t j = blockIdx.x;
  const int64_t r0 = j * kBlock;
  const int64_t r1 = (r0 + kBlock < S) ? r0 + kBlock : S;
  for (int64_t d = threadIdx.x; d < D; d += blockDim.x) {
    double acc = 0.0;
    for (int64_t r = r0; r < r1; ++r) acc += key_to_double(keys[r * D + d], bf16);
    cent[j * D + d] = acc / (double)(r1 - r0);
  }
}

// ------------------------------------------------------------------ distances

__global__ __launch_bounds__(256) void distance_kernel(const double* __restrict__ cent, int nb,
                                                       int64_t D, double* __restrict__ dist) {
  const int i = blockIdx.y * 16 + threadIdx.y;
  const int j = blockIdx.x * 16 + threadIdx.x;
  if (i >= nb || j >= nb) return;
  const double* ci = cent + (int64_t)i * D;
  const double* cj = cent + (int64_t)j * D;
  double acc = 0.0;
  for (int64_t d = 0; d < D; ++d) {
    const double df = ci[d] - cj[d];
    acc = __builtin_fma(df, df, acc);
  }
  const double d = __builtin_sqrt(acc);
  dist[(int64_t)i * nb + j] = (d == d) ? d : __builtin_inf();  // NaN (from NaN keys) -> +inf
}

// ------------------------------------------------------------------ wave helpers

// 32-bit exchanges with a partner lane.  After the first four, every lane of a
// 16-lane row holds the row's result; the last two combine rows.
__device__ __forceinline__ int xchg_quad1(int x) { return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int xchg_quad2(int x) { return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int xchg_half_mirror(int x) { return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ int xchg_mirror(int x) { return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); }
__device__ __forceinline__ int xchg_xor16(int x) { return __builtin_amdgcn_ds_swizzle(x, 0x401F); }
__device__ __forceinline__ int xchg_xor32(int x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const int lane = __lane_id();
  return lane < 32 ? (int)r[1] : (int)r[0];
}

template <int (*X)(int)>
__device__ __forceinline__ double xchg_double(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = X((int)(uint32_t)u), hi = X((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ double wave_min(double v) {
  v = fmin(v, xchg_double<xchg_quad1>(v));
  v = fmin(v, xchg_double<xchg_quad2>(v));
  v = fmin(v, xchg_double<xchg_half_mirror>(v));
  v = fmin(v, xchg_double<xchg_mirror>(v));
  v = fmin(v, xchg_double<xchg_xor16>(v));
  v = fmin(v, xchg_double<xchg_xor32>(v));
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
  v = min(v, xchg_quad1(v));
  v = min(v, xchg_quad2(v));
  v = min(v, xchg_half_mirror(v));
  v = min(v, xchg_mirror(v));
  v = min(v, xchg_xor16(v));
  v = min(v, xchg_xor32(v));
  return v;
}

__device__ __forceinline__ int read_lane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Value of per-block register array `a` for block x (x uniform across the wave).
template <int SLOTS, typename T>
__device__ __forceinline__ T block_value(const T (&a)[SLOTS], int x) {
  const int s = x >> 6;
  T val = a[0];
#pragma unroll
  for (int k = 1; k < SLOTS; ++k)
    if (s == k) val = a[k];
  return read_lane(val, x & 63);
}

// Lexicographic (key, tie) minimum over the wave.  Every lane passes its own
// best candidate (key = +inf for none); all lanes receive the winner.
__device__ __forceinline__ void wave_argmin(double key, int tie, double& best_key, int& best_tie) {
  best_key = wave_min(key);
  const uint64_t hold = __ballot(key == best_key);
  if (__popcll(hold) == 1) {
    best_tie = read_lane(tie, __ffsll((unsigned long long)hold) - 1);
  } else {
    best_tie = wave_min(key == best_key ? tie : INT32_MAX);
  }
}

// ------------------------------------------------------------------ topology

template <int SLOTS>
__global__ __launch_bounds__(64) void topology_kernel(const double* __restrict__ dist_g, int nb,
                                                      int sink, int local_radius, int topk,
                                                      int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ col_idx,
                                                      int64_t col_capacity,
                                                      double* __restrict__ salience,
                                                      bool dist_in_lds) {
  extern __shared__ __attribute__((aligned(16))) double dist_lds[];
  const int lane = threadIdx.x;
  const double kInf = __builtin_inf();

  if (dist_in_lds) {
    const int64_t n2 = (int64_t)nb * nb;
    for (int64_t e = lane; e < n2; e += 64) dist_lds[e] = dist_g[e];
    __syncthreads();
  }
  const double* dist = dist_in_lds ? dist_lds : dist_g;

  // ---- Prim's MST from block 0.  Block v: lane v % 64, slot v / 64.
  double key[SLOTS];
  int src[SLOTS];
  bool in_tree[SLOTS];
  double edge_w[SLOTS];  // MST edge e sits at lane e % 64, slot e / 64
  int edge_t[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int v = lane + 64 * s;
    in_tree[s] = (v == 0) || (v >= nb);
    key[s] = (v < nb) ? dist[v] : kInf;  // row 0
    src[s] = 0;
    edge_w[s] = kInf;
    edge_t[s] = INT32_MAX;
  }
  for (int step = 0; step < nb - 1; ++step) {
    double bk = kInf;
    int bv = INT32_MAX;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int v = lane + 64 * s;
      // slots ascend in v, so ties keep the lower v; the first candidate is taken
      // even at +inf so that a vertex is always found while any remains
      if (!in_tree[s] && (key[s] < bk || bv == INT32_MAX)) {
        bk = key[s];
        bv = v;
      }
    }
    double w;
    int u;
    wave_argmin(bk, bv, w, u);
    if (u >= nb) break;  // unreachable: one vertex joins per step
    const int su = block_value<SLOTS>(src, u);
    const int a = su < u ? su : u, b = su < u ? u : su;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int v = lane + 64 * s;
      if (v == step) {
        edge_w[s] = w;
        edge_t[s] = (a << kTieShift) | b;
      }
      if (v == u) in_tree[s] = true;
    }
    const double* du = dist + (int64_t)u * nb;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int v = lane + 64 * s;
      if (!in_tree[s]) {
        const double d = du[v];
        if (d < key[s]) {
          key[s] = d;
          src[s] = u;
        }
      }
    }
  }

  // ---- Elder rule over MST edges in ascending (length, lower, higher) order.
  int root[SLOTS], size[SLOTS];
  double sal[SLOTS];
  bool done[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    root[s] = lane + 64 * s;
    size[s] = 1;
    sal[s] = 0.0;
    done[s] = false;
  }
  for (int e = 0; e < nb - 1; ++e) {
    double bw = kInf;
    int bt = INT32_MAX;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      if (!done[s] && (edge_w[s] < bw || (edge_w[s] == bw && edge_t[s] < bt))) {
        bw = edge_w[s];
        bt = edge_t[s];
      }
    }
    double w;
    int t;
    wave_argmin(bw, bt, w, t);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s)
      if (!done[s] && edge_w[s] == w && edge_t[s] == t) done[s] = true;
    const int a = t >> kTieShift, b = t & ((1 << kTieShift) - 1);
    const int ra = block_value<SLOTS>(root, a), rb = block_value<SLOTS>(root, b);
    const int sa = block_value<SLOTS>(size, ra), sb = block_value<SLOTS>(size, rb);
    // The larger component survives; on equal size the lower root index does.
    const bool a_survives = sa > sb || (sa == sb && ra < rb);
    const int surv = a_survives ? ra : rb, absorbed = a_survives ? rb : ra;
    const int grown = sa + sb;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int v = lane + 64 * s;
      if (root[s] == absorbed) root[s] = surv;
      if (v == surv) size[s] = grown;
      if (v == absorbed) sal[s] = w;
    }
  }

  // ---- Global top-k: the first min(topk, nb) blocks under (-salience, index).
  bool in_top[SLOTS];
  const int kk = topk < nb ? topk : nb;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) in_top[s] = (kk == nb) && (lane + 64 * s < nb);
  if (kk < nb) {
    for (int e = 0; e < kk; ++e) {
      double bk = kInf;
      int bv = INT32_MAX;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int v = lane + 64 * s;
        if (v < nb && !in_top[s] && (-sal[s] < bk || bv == INT32_MAX)) {
          bk = -sal[s];
          bv = v;
        }
      }
      double nk;
      int pick;
      wave_argmin(bk, bv, nk, pick);
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
        if (lane + 64 * s == pick) in_top[s] = true;
    }
  }
  uint64_t top_bits[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) top_bits[s] = __ballot(in_top[s]);

  // Number of top-k blocks with index <= x (x >= -1), per lane.
  auto top_upto = [&](int x) -> int {
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int lo = 64 * s;
      if (x >= lo + 63) {
        cnt += __popcll(top_bits[s]);
      } else if (x >= lo) {
        const int sh = x - lo + 1;  // 1 .. 63
        cnt += __popcll(top_bits[s] & ((1ull << sh) - 1ull));
      }
    }
    return cnt;
  };

  // ---- Row sizes: sink [0, min(sink, i+1)), top-k in [sink, i - r), local [max(sink, i - r), i].
  int cnt[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int i = lane + 64 * s;
    int c = 0;
    if (i < nb) {
      const int sink_hi = sink < i + 1 ? sink : i + 1;  // sink part: [0, sink_hi)
      const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
      c = sink_hi + (loc_lo <= i ? i - loc_lo + 1 : 0);
      const int t_hi = i - local_radius - 1;  // top-k part: [sink, t_hi]
      if (t_hi >= sink) c += top_upto(t_hi) - top_upto(sink - 1);
    }
    cnt[s] = c;
  }
  // Exclusive prefix over rows (row order: slot-major, lanes within a slot).
  int start[SLOTS];
  int carry = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    int incl = cnt[s];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int other = __shfl_up(incl, off);
      if (lane >= off) incl += other;
    }
    start[s] = carry + incl - cnt[s];
    carry += read_lane(incl, 63);
  }

  // ---- Emission.
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int i = lane + 64 * s;
    if (i >= nb) continue;
    row_ptr[i] = start[s];
    int64_t pos = start[s];
    auto put = [&](int j) {
      if (pos < col_capacity) col_idx[pos] = j;
      ++pos;
    };
    const int sink_hi = sink < i + 1 ? sink : i + 1;
    for (int j = 0; j < sink_hi; ++j) put(j);
    const int t_hi = i - local_radius - 1;
#pragma unroll
    for (int w = 0; w < SLOTS; ++w) {
      uint64_t bits = top_bits[w];
      while (bits) {
        const int j = 64 * w + __ffsll((unsigned long long)bits) - 1;
        bits &= bits - 1;
        if (j >= sink && j <= t_hi) put(j);
      }
    }
    const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
    for (int j = loc_lo; j <= i; ++j) put(j);
    if (salience) salience[i] = sal[s];
  }
  if (lane == 0) row_ptr[nb] = carry;
}

template <int SLOTS>
hipError_t launch_topology(const double* dist, int nb, int sink, int local_radius, int topk,
                           int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                           double* salience, hipStream_t stream) {
  const bool in_lds = nb <= kLdsDistBlocks;
  const size_t lds = in_lds ? (size_t)nb * nb * sizeof(double) : 0;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)topology_kernel<SLOTS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topology_kernel<SLOTS>, dim3(1), dim3(64), lds, stream, dist, nb, sink,
                     local_radius, topk, row_ptr, col_idx, col_capacity, salience, in_lds);
  return hipGetLastError();
}

__global__ void dense_schedule_kernel(int64_t nb, int32_t* __restrict__ row_ptr,
                                      int32_t* __restrict__ col_idx) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i > nb) return;
  const int64_t base = i * (i + 1) / 2;
  row_ptr[i] = (int32_t)base;
  if (i < nb)
    for (int64_t j = 0; j <= i; ++j) col_idx[base + j] = (int32_t)j;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t schedule_workspace_bytes(int64_t nb, int64_t D) {
  return align256((size_t)nb * D * sizeof(double)) + align256((size_t)nb * nb * sizeof(double));
}

hipError_t launch_build_schedule(const void* keys, bool bf16, int64_t S, int64_t D, int sink,
                                 int local_radius, int topk, int32_t* row_ptr, int32_t* col_idx,
                                 int64_t col_capacity, double* salience, void* workspace,
                                 hipStream_t stream) {
  const int64_t nb = (S + kBlock - 1) / kBlock;
  if (nb == 0) return launch_dense_schedule(0, row_ptr, col_idx, stream);
  double* cent = (double*)workspace;
  double* dist = (double*)((char*)workspace + align256((size_t)nb * D * sizeof(double)));
  hipLaunchKernelGGL(centroid_kernel, dim3((unsigned)nb), dim3(64), 0, stream,
                     (const uint16_t*)keys, bf16, S, D, cent);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned tiles = (unsigned)((nb + 15) / 16);
  hipLaunchKernelGGL(distance_kernel, dim3(tiles, tiles), dim3(16, 16), 0, stream, cent, (int)nb, D,
                     dist);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n = (int)nb;
  if (n <= 64) return launch_topology<1>(dist, n, sink, local_radius, topk, row_ptr, col_idx, col_capacity, salience, stream);
  if (n <= 128) return launch_topology<2>(dist, n, sink, local_radius, topk, row_ptr, col_idx, col_capacity, salience, stream);
  if (n <= 256) return launch_topology<4>(dist, n, sink, local_radius, topk, row_ptr, col_idx, col_capacity, salience, stream);
  if (n <= 512) return launch_topology<8>(dist, n, sink, local_radius, topk, row_ptr, col_idx, col_capacity, salience, stream);
  return launch_topology<16>(dist, n, sink, local_radius, topk, row_ptr, col_idx, col_capacity, salience, stream);
}

hipError_t launch_dense_schedule(int64_t nb, int32_t* row_ptr, int32_t* col_idx,
                                 hipStream_t stream) {
  const int64_t rows = nb + 1;
  const unsigned grid = (unsigned)((rows + 255) / 256);
  hipLaunchKernelGGL(dense_schedule_kernel, dim3(grid), dim3(256), 0, stream, nb, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace tsa
