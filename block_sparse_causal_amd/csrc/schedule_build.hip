// GPU builder of the topology-derived CSR block schedule (gfx950).
//
// Follows "Add topology-derived sparse attention kernel" (triton-lang/kernels
// PR 22), Summary, second bullet: sink blocks + local-window blocks + the
// top-k key blocks ranked by a 0D-persistence salience of the key-block
// centroids.  Salience is the elder rule of the mirror page's Rust-port commit
// note, computed from minimum-spanning-tree edges as in its schedule.py commit
// note (same result as single linkage over all pairs).
//
// Edges are ordered by (length, lower block index, higher block index).  That
// order is strict, so the MST is unique and is the tree that a scan of all
// pairs in that order builds; Boruvka's rounds find it with about log2(nb)
// parallel steps instead of the nb - 1 sequential steps of Prim or Kruskal.
//
// Kernels on the caller's stream:
//   centroid_kernel   one workgroup per key block: fp64 mean of its keys, stored
//                     dimension-major (dim d of centroid j at d * nbe + j, nbe =
//                     nb rounded up to even).
//   distance_kernel   the nb x nb distance matrix into the workspace, one entry
//                     per thread over many CUs.
//   nb <= 128, one workgroup (topology_small):
//     the matrix into LDS; Boruvka rounds; MST edges ranked; the elder rule
//     over them in rank order (one wavefront, per-block state in registers);
//     blocks ranked by salience; CSR rows emitted.
//   nb > 128:
//     boruvka_nearest   per block, the least edge to another component;
//     boruvka_merge     one workgroup: per-component least edge, hooking,
//                       pointer jumping, new labels, the new MST edges;
//                       (the pair is launched ceil(log2 nb) times: every round
//                       at least halves the number of components, and rounds
//                       after the last merge return at once)
//     finish_kernel     edge ranks, elder rule (union-find in LDS), top-k, CSR.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tsa {
namespace {

constexpr int kBlock = 64;
constexpr uint32_t kNoEdge = 0xffffffffu;          // "no candidate" edge tag
constexpr unsigned long long kNoLen = ~0ull;       // above the bits of +inf
constexpr int kStageBytes = 16384;                 // least LDS staging of centroid dims
constexpr int kSmallThreads = 512;
constexpr int kLargeThreads = 1024;
constexpr int kLargePerThread = 4;                 // blocks per thread in boruvka_merge
static_assert(kLargeThreads * kLargePerThread >= 4096, "boruvka_merge covers 4096 blocks");

__device__ __forceinline__ double key_to_double(uint16_t bits, bool bf16) {
  if (bf16) return (double)__uint_as_float((uint32_t)bits << 16);
  return (double)__builtin_bit_cast(_Float16, bits);
}

// Tag of the edge {x, y}: lower index in the high half, higher in the low half
// (block indices are below 2^16).  Comparing tags compares (lower, higher).
__device__ __forceinline__ uint32_t edge_tag(int x, int y) {
  return x < y ? ((uint32_t)x << 16) | (uint32_t)y : ((uint32_t)y << 16) | (uint32_t)x;
}
__device__ __forceinline__ bool edge_less(double d1, uint32_t t1, double d2, uint32_t t2) {
  return d1 < d2 || (d1 == d2 && t1 < t2);
}
// Lengths are >= 0 or +inf, so their bit patterns order like the values.
__device__ __forceinline__ unsigned long long len_bits(double d) {
  return __builtin_bit_cast(unsigned long long, d);
}
__device__ __forceinline__ double bits_len(unsigned long long b) { return __builtin_bit_cast(double, b); }
// NaN (from NaN keys) is treated as +inf so that the edge order stays total.
__device__ __forceinline__ double finite_or_inf(double d) { return d == d ? d : __builtin_inf(); }

// ------------------------------------------------------------------ wave helpers

// 32-bit exchanges with a partner lane.  After the first four, every lane of a
// 16-lane row has seen the whole row; the last two combine rows.
__device__ __forceinline__ int xchg_quad1(int x) { return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int xchg_quad2(int x) { return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int xchg_half_mirror(int x) { return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ int xchg_mirror(int x) { return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); }
__device__ __forceinline__ int xchg_xor16(int x) {
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return ((__lane_id() >> 4) & 1) ? (int)r[0] : (int)r[1];
}
__device__ __forceinline__ int xchg_xor32(int x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return __lane_id() < 32 ? (int)r[1] : (int)r[0];
}

template <int (*X)(int)>
__device__ __forceinline__ void edge_min_step(double& d, uint32_t& t) {
  const uint64_t u = __builtin_bit_cast(uint64_t, d);
  const int lo = X((int)(uint32_t)u), hi = X((int)(uint32_t)(u >> 32));
  const double od = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  const uint32_t ot = (uint32_t)X((int)t);
  if (edge_less(od, ot, d, t)) {
    d = od;
    t = ot;
  }
}

// Least (length, tag) over the wavefront, returned in every lane.
__device__ __forceinline__ void wave_edge_min(double& d, uint32_t& t) {
  edge_min_step<xchg_quad1>(d, t);
  edge_min_step<xchg_quad2>(d, t);
  edge_min_step<xchg_half_mirror>(d, t);
  edge_min_step<xchg_mirror>(d, t);
  edge_min_step<xchg_xor16>(d, t);
  edge_min_step<xchg_xor32>(d, t);
}

__device__ __forceinline__ int read_lane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ double read_lane(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Value of per-block register array `a` for block x (x uniform; block x lives
// in lane x % 64, slot x / 64).
template <int SLOTS>
__device__ __forceinline__ int block_value(const int (&a)[SLOTS], int x) {
  const int s = x >> 6;
  int val = a[0];
#pragma unroll
  for (int k = 1; k < SLOTS; ++k)
    if (s == k) val = a[k];
  return read_lane(val, x & 63);
}

// ------------------------------------------------------------------ workgroup helpers

// Exclusive prefix sum of a[0, n) in LDS, in place; returns the total.  Every
// thread of the workgroup calls it with the same n.  tmp: kThreads / 64 ints.
template <int kThreads>
__device__ int block_exclusive_scan(int* a, int n, int* tmp) {
  constexpr int kWaves = kThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    const int x = i < n ? a[i] : 0;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) tmp[w] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const int s = tmp[k];
      before += k < w ? s : 0;
      total += s;
    }
    if (i < n) a[i] = carry + before + incl - x;
    carry += total;
    __syncthreads();  // tmp is rewritten by the next chunk
  }
  return carry;
}

// rank[e] += number of items f in [0, n) with before(f, e), for a strict total
// order `before`; the n^2 comparisons are spread over the workgroup (item e
// and one part of the f range per thread).  rank must be zero on entry; the
// caller synchronises afterwards.
template <int kThreads, typename Before>
__device__ __forceinline__ void count_ranks(int n, int* rank, Before before) {
  if (n <= 0) return;
  const int np = (n + 63) & ~63;
  const int parts = np >= kThreads ? 1 : kThreads / np;
  const int len = (n + parts - 1) / parts;
  for (int x = threadIdx.x; x < np * parts; x += kThreads) {
    const int e = x % np, q = x / np;
    if (e >= n) continue;
    const int f0 = q * len, f1 = (f0 + len < n) ? f0 + len : n;
    int c = 0;
    for (int f = f0; f < f1; ++f) c += before(f, e) ? 1 : 0;
    if (c) atomicAdd(&rank[e], c);
  }
}

// Top-k selection and CSR emission from the per-block salience (LDS).
//   Blocks are ranked by (-salience, index); the first min(topk, nb) form the
//   global top-k set.  Row i lists, ascending: sink blocks [0, min(sink, i+1)),
//   top-k blocks in [sink, i - r - 1], local blocks [max(sink, i - r), i].
// Scratch (LDS): brank[nb], top[nb + 1], topidx[nb], cnt[nb + 1], tmp.
template <int kThreads>
__device__ void select_and_emit(const double* sal, int nb, int sink, int local_radius, int topk,
                                int* brank, int* top, int* topidx, int* cnt, int* tmp,
                                int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                int64_t col_capacity, double* __restrict__ salience) {
  const int tid = threadIdx.x;
  const int kk = topk < nb ? topk : nb;
  for (int v = tid; v < nb; v += kThreads) brank[v] = 0;
  __syncthreads();
  if (kk > 0 && kk < nb)
    count_ranks<kThreads>(nb, brank, [&](int u, int v) {
      const double su = sal[u], sv = sal[v];
      return su > sv || (su == sv && u < v);
    });
  __syncthreads();
  for (int v = tid; v <= nb; v += kThreads) top[v] = (v < nb && brank[v] < kk) ? 1 : 0;
  if (salience != nullptr)
    for (int v = tid; v < nb; v += kThreads) salience[v] = sal[v];
  __syncthreads();
  block_exclusive_scan<kThreads>(top, nb + 1, tmp);  // top[x] = selected blocks below x
  for (int v = tid; v < nb; v += kThreads)
    if (top[v + 1] > top[v]) topidx[top[v]] = v;

  // Row sizes, then starts.
  for (int i = tid; i <= nb; i += kThreads) {
    int c = 0;
    if (i < nb) {
      const int a_n = sink < i + 1 ? sink : i + 1;
      const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
      const int b_n = loc_lo <= i ? i - loc_lo + 1 : 0;
      const int t_hi = i - local_radius - 1;
      const int c_n = t_hi >= sink ? top[t_hi + 1] - top[sink] : 0;
      c = a_n + c_n + b_n;
    }
    cnt[i] = c;
  }
  __syncthreads();
  block_exclusive_scan<kThreads>(cnt, nb + 1, tmp);  // also leaves cnt[nb] = nnz
  for (int i = tid; i <= nb; i += kThreads) row_ptr[i] = cnt[i];

  // Entries: one wavefront per row, one entry per lane.
  const int lane = tid & 63;
  for (int i = tid >> 6; i < nb; i += kThreads / 64) {
    const int a_n = sink < i + 1 ? sink : i + 1;
    const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
    const int b_n = loc_lo <= i ? i - loc_lo + 1 : 0;
    const int t_hi = i - local_radius - 1;
    const int c_n = t_hi >= sink ? top[t_hi + 1] - top[sink] : 0;
    const int c0 = t_hi >= sink ? top[sink] : 0;
    const int n = a_n + c_n + b_n;
    const int64_t start = cnt[i];
    for (int k = lane; k < n; k += 64) {
      int j;
      if (k < a_n)
        j = k;
      else if (k < a_n + c_n)
        j = topidx[c0 + k - a_n];
      else
        j = loc_lo + (k - a_n - c_n);
      if (start + k < col_capacity) col_idx[start + k] = j;
    }
  }
}

// ------------------------------------------------------------------ centroids

// One workgroup per key block.  256 threads = 32 row groups x 8 column chunks;
// each thread sums its rows over 8 consecutive dims (one 16-byte load per row
// when D is a multiple of 8), then the 32 partial sums per dim are added in LDS.
// Sums of fp16/bf16 values in fp64 are exact for keys of ordinary magnitude, so
// the order of the additions does not change the centroid.  Output is
// dimension-major with an even row stride nbe = nb rounded up to even:
// cent_t[d * nbe + j].  When `comp` is given, the larger-schedule
// state is reset too: comp[j] = j, and counters {edges, done} = 0.
__global__ __launch_bounds__(256) void centroid_kernel(const uint16_t* __restrict__ keys, bool bf16,
                                                       int64_t S, int64_t D, int nb,
                                                       double* __restrict__ cent_t,
                                                       int* __restrict__ comp,
                                                       int* __restrict__ counters) {
  __shared__ double part[32][65];
  const int64_t j = blockIdx.x;
  const int64_t r0 = j * kBlock;
  const int rows = (int)((r0 + kBlock < S) ? kBlock : S - r0);
  const int tid = threadIdx.x, rg = tid >> 3, ch = tid & 7;
  const bool vec = (D % 8) == 0 && ((uintptr_t)keys % 16) == 0;  // 16-byte aligned rows
  for (int64_t d0 = 0; d0 < D; d0 += 64) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int64_t dc = d0 + 8 * ch;
    for (int r = rg; r < rows; r += 32) {
      const uint16_t* row = keys + (r0 + r) * D;
      if (vec && dc + 8 <= D) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 x = *(const u32x4*)(row + dc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += key_to_double((uint16_t)(x[e] & 0xffffu), bf16);
          acc[2 * e + 1] += key_to_double((uint16_t)(x[e] >> 16), bf16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (dc + e < D) acc[e] += key_to_double(row[dc + e], bf16);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg][8 * ch + e] = acc[e];
    __syncthreads();
    if (tid < 64 && d0 + tid < D) {
      double sum = 0.0;
      for (int g = 0; g < 32; ++g) sum += part[g][tid];
      cent_t[(d0 + tid) * ((nb + 1) & ~1) + j] = sum / (double)rows;
    }
    __syncthreads();
  }
  if (comp != nullptr && tid == 0) {
    comp[j] = (int)j;
    if (j == 0) counters[0] = counters[1] = 0;
  }
}

// ------------------------------------------------------------------ small schedules

// LDS after the distance matrix.  The first kStageBytes also stage centroid
// dims while the distances are formed; the rest of the state takes that space
// once the matrix is done.
struct SmallState {
  double part_d[kSmallThreads];
  uint32_t part_t[kSmallThreads];
  unsigned long long cmin_d[kLdsDistBlocks];  // per component: least outgoing length (bits)
  uint32_t cmin_t[kLdsDistBlocks];            //   and the least tag at that length
  int comp[kLdsDistBlocks];                   // component label = a block index
  int hook[kLdsDistBlocks];
  int par[kLdsDistBlocks];
  double edge_d[kLdsDistBlocks];              // MST edges, in discovery order
  uint32_t edge_t[kLdsDistBlocks];
  double sort_d[kLdsDistBlocks];              // MST edges, ascending
  uint32_t sort_t[kLdsDistBlocks];
  int rank[kLdsDistBlocks];
  double sal[kLdsDistBlocks];
  int topidx[kLdsDistBlocks];
  int nedges;
  int changed;
};
static_assert(sizeof(SmallState) <= kStageBytes, "small-schedule state fits the staging area");

// Elder rule over the MST edges in ascending order, one wavefront, nb <= 64 *
// SLOTS.  Per block (lane v % 64, slot v / 64): its component's root and size,
// and its salience.  The smaller component is absorbed (equal sizes: the
// larger root index); the absorbed root's salience is the edge length; the
// last survivor keeps 0.
template <int SLOTS>
__device__ __forceinline__ void elder_registers(const double* sd, const uint32_t* st, int ne,
                                                double (&sal)[SLOTS]) {
  const int lane = threadIdx.x & 63;
  int root[SLOTS], csz[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    root[s] = lane + 64 * s;
    csz[s] = 1;
    sal[s] = 0.0;
  }
  for (int base = 0; base < ne; base += 64) {
    const int r = base + lane;
    const int tw = r < ne ? (int)st[r] : 0;
    const double dw = r < ne ? sd[r] : 0.0;
    const int n = ne - base < 64 ? ne - base : 64;
    for (int k = 0; k < n; ++k) {
      const int t = read_lane(tw, k);
      const int a = (int)((uint32_t)t >> 16), b = t & 0xffff;
      const int ra = block_value<SLOTS>(root, a), rb = block_value<SLOTS>(root, b);
      const int sa = block_value<SLOTS>(csz, a), sb = block_value<SLOTS>(csz, b);
      const bool a_survives = sa > sb || (sa == sb && ra < rb);
      const int surv = a_survives ? ra : rb, absorbed = a_survives ? rb : ra;
      const int grown = sa + sb;
      const double w = read_lane(dw, k);
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const bool in = root[s] == ra || root[s] == rb;
        root[s] = in ? surv : root[s];
        csz[s] = in ? grown : csz[s];
        sal[s] = (lane + 64 * s == absorbed) ? w : sal[s];
      }
    }
  }
}

// The same rule for nb <= 64 with each block's component held as a 64-bit
// mask: component sizes are popcounts, and a merge rewrites the lanes of the
// merged mask.
__device__ __forceinline__ void elder_masks(const double* sd, const uint32_t* st, int ne,
                                            double (&sal)[1]) {
  const int lane = threadIdx.x & 63;
  uint32_t cm_lo = lane < 32 ? 1u << lane : 0u, cm_hi = lane < 32 ? 0u : 1u << (lane - 32);
  int root = lane;
  double s0 = 0.0;
  for (int base = 0; base < ne; base += 64) {
    const int r = base + lane;
    const uint32_t tw = r < ne ? st[r] : 0u;
    const int aw = (int)(tw >> 16), bw = (int)(tw & 0xffffu);
    const double dw = r < ne ? sd[r] : 0.0;
    const int n = ne - base < 64 ? ne - base : 64;
    for (int k = 0; k < n; ++k) {
      const int a = read_lane(aw, k), b = read_lane(bw, k);
      const uint64_t ma = ((uint64_t)(uint32_t)read_lane((int)cm_hi, a) << 32) | (uint32_t)read_lane((int)cm_lo, a);
      const uint64_t mb = ((uint64_t)(uint32_t)read_lane((int)cm_hi, b) << 32) | (uint32_t)read_lane((int)cm_lo, b);
      const int ra = read_lane(root, a), rb = read_lane(root, b);
      const int sa = __popcll(ma), sb = __popcll(mb);
      const bool a_survives = sa > sb || (sa == sb && ra < rb);
      const int surv = a_survives ? ra : rb, absorbed = a_survives ? rb : ra;
      const uint64_t m = ma | mb;
      const double w = read_lane(dw, k);
      if ((m >> lane) & 1ull) {
        cm_lo = (uint32_t)m;
        cm_hi = (uint32_t)(m >> 32);
        root = surv;
      }
      if (lane == absorbed) s0 = w;
    }
  }
  sal[0] = s0;
}

// Inclusive prefix sum over the wavefront: shifts within each 16-lane row,
// then the row totals carried across rows.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = read_lane(x, 15), r1 = read_lane(x, 31), r2 = read_lane(x, 47);
  const int row = __lane_id() >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Orders this wavefront's earlier LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Top-k selection and CSR emission by one wavefront (nb <= 64 * SLOTS), rows
// as in select_and_emit.  Row i = lane + 64 * slot writes its own entries.
// LDS scratch: sal_lds[nb], topidx[nb].
template <int SLOTS>
__device__ __forceinline__ void select_and_emit_wave(const double (&sal)[SLOTS], int nb, int sink,
                                                     int local_radius, int topk, double* sal_lds,
                                                     int* topidx, int32_t* __restrict__ row_ptr,
                                                     int32_t* __restrict__ col_idx,
                                                     int64_t col_capacity,
                                                     double* __restrict__ salience) {
  const int lane = threadIdx.x & 63;
  const int kk = topk < nb ? topk : nb;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int v = lane + 64 * s;
    if (v < nb) {
      sal_lds[v] = sal[s];
      if (salience != nullptr) salience[v] = sal[s];
    }
  }
  wave_lds_sync();
  // Top-k set as one bit mask per slot.
  uint64_t topm[SLOTS];
  if (kk >= nb || kk == 0) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) topm[s] = kk == 0 ? 0ull : (uint64_t)__ballot(lane + 64 * s < nb);
  } else {
    int brank[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) brank[s] = 0;
#pragma unroll 8
    for (int u = 0; u < nb; ++u) {
      const double su = sal_lds[u];
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
        brank[s] += (su > sal[s] || (su == sal[s] && u < lane + 64 * s)) ? 1 : 0;
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) topm[s] = __ballot(lane + 64 * s < nb && brank[s] < kk);
  }
  // Selected blocks below x, for a per-lane x in [0, nb].
  auto top_below = [&](int x) -> int {
    int c = 0;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int rel = x - 64 * s;
      if (rel >= 64)
        c += __popcll(topm[s]);
      else if (rel > 0)
        c += __popcll(topm[s] & ((1ull << rel) - 1ull));
    }
    return c;
  };
  // Selected blocks in ascending order.
  int below = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const uint32_t lo = (uint32_t)topm[s], hi = (uint32_t)(topm[s] >> 32);
    const int rank = below + (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
    if ((topm[s] >> lane) & 1ull) topidx[rank] = lane + 64 * s;
    below += __popcll(topm[s]);
  }
  wave_lds_sync();
  // Row sizes, starts, entries.
  int carry = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int i = lane + 64 * s;
    const int a_n = sink < i + 1 ? sink : i + 1;
    const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
    const int b_n = loc_lo <= i ? i - loc_lo + 1 : 0;
    const int t_hi = i - local_radius - 1;
    const int c0 = t_hi >= sink ? top_below(sink) : 0;
    const int c_n = t_hi >= sink ? top_below(t_hi + 1) - c0 : 0;
    const int n = i < nb ? a_n + c_n + b_n : 0;
    const int incl = wave_inclusive_scan(n);
    const int64_t start = carry + incl - n;
    carry += read_lane(incl, 63);
    if (i < nb) {
      row_ptr[i] = (int32_t)start;
      int64_t pos = start;
      for (int j = 0; j < a_n; ++j, ++pos)
        if (pos < col_capacity) col_idx[pos] = j;
      for (int k = 0; k < c_n; ++k, ++pos)
        if (pos < col_capacity) col_idx[pos] = topidx[c0 + k];
      for (int j = loc_lo; j <= i; ++j, ++pos)
        if (pos < col_capacity) col_idx[pos] = j;
    }
  }
  if (lane == 0) row_ptr[nb] = carry;
}

// Doubles of LDS before the staging area: the distance matrix, rounded up to
// an even count so that the staging area is 16-byte aligned.
__host__ __device__ constexpr int small_stage_offset(int nb) { return (nb * nb + 1) & ~1; }

// Everything after the distances for nb <= kLdsDistBlocks, in one workgroup of
// 512 threads.  Dynamic LDS: small_stage_offset(nb) doubles (the distance
// matrix) + kStageBytes (SmallState).
template <int SLOTS>
__global__ __launch_bounds__(kSmallThreads) void topology_small(
    const double* __restrict__ dist_g, int nb, int sink, int local_radius, int topk,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx, int64_t col_capacity,
    double* __restrict__ salience) {
  extern __shared__ __attribute__((aligned(16))) double smem[];
  double* dist = smem;
  SmallState& A = *reinterpret_cast<SmallState*>(smem + small_stage_offset(nb));  // 16-byte aligned
  const int tid = threadIdx.x;
  const double kInf = __builtin_inf();

  // ---- Distance matrix (formed by distance_kernel) into LDS, 16 bytes a load.
  {
    typedef double f64x2 __attribute__((ext_vector_type(2)));
    const int n16 = nb * nb / 2;
    const f64x2* src = (const f64x2*)dist_g;
    f64x2* dst = (f64x2*)dist;
    for (int e0 = 0; e0 < n16; e0 += 4 * kSmallThreads) {
      f64x2 r[4];  // unconditional (clamped) loads, so that all four are in flight
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kSmallThreads + tid;
        r[u] = src[e < n16 ? e : n16 - 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kSmallThreads + tid;
        if (e < n16) dst[e] = r[u];
      }
    }
    if ((nb & 1) && tid == 0) dist[nb * nb - 1] = dist_g[nb * nb - 1];  // odd element count
  }
  __syncthreads();

  // ---- Boruvka rounds.
  if (tid < nb) {
    A.comp[tid] = tid;
    A.cmin_d[tid] = kNoLen;
    A.cmin_t[tid] = kNoEdge;
    A.rank[tid] = 0;
  }
  if (tid == 0) A.nedges = 0;
  __syncthreads();
  const int nbp = (nb + 63) & ~63;           // 64 or 128: divides kSmallThreads
  const int parts = kSmallThreads / nbp;
  const int plen = (nb + parts - 1) / parts;
  for (int round = 0; round < 16; ++round) {  // ceil(log2 128) = 7 rounds suffice
    if (A.nedges >= nb - 1) break;
    // Least edge from each block to another component, over one part of the
    // candidates per thread; column reads of the symmetric matrix keep the
    // lanes on distinct banks.
    {
      const int v = tid % nbp, q = tid / nbp;
      double bd = kInf;
      uint32_t bt = kNoEdge;
      if (v < nb) {
        const int cv = A.comp[v];
        const int j1 = (q + 1) * plen < nb ? (q + 1) * plen : nb;
        for (int j = q * plen; j < j1; ++j) {
          if (A.comp[j] == cv) continue;
          const double d = dist[j * nb + v];
          const uint32_t t = edge_tag(v, j);
          if (edge_less(d, t, bd, bt)) {
            bd = d;
            bt = t;
          }
        }
      }
      A.part_d[tid] = bd;
      A.part_t[tid] = bt;
    }
    __syncthreads();
    double bd = kInf;
    uint32_t bt = kNoEdge;
    int cv = 0;
    if (tid < nb) {
      for (int q = 0; q < parts; ++q) {
        const double d = A.part_d[q * nbp + tid];
        const uint32_t t = A.part_t[q * nbp + tid];
        if (edge_less(d, t, bd, bt)) {
          bd = d;
          bt = t;
        }
      }
      cv = A.comp[tid];
      if (bt != kNoEdge) atomicMin(&A.cmin_d[cv], len_bits(bd));
    }
    __syncthreads();
    if (tid < nb && bt != kNoEdge && len_bits(bd) == A.cmin_d[cv]) atomicMin(&A.cmin_t[cv], bt);
    __syncthreads();
    // Each component hooks onto the component across its least edge.
    const bool is_root = tid < nb && A.comp[tid] == tid;
    if (is_root) {
      const uint32_t t = A.cmin_t[tid];  // always an edge while two components remain
      const int lo = (int)(t >> 16), hi = (int)(t & 0xffffu);
      A.hook[tid] = t == kNoEdge ? tid : A.comp[A.comp[lo] == tid ? hi : lo];
    }
    __syncthreads();
    // Two components that chose each other chose the same edge: the lower label
    // stays a root and records it; every other component records its own edge.
    if (is_root) {
      const int c2 = A.hook[tid];
      const bool mutual = A.hook[c2] == tid;  // includes c2 == tid (no edge): nothing recorded
      if (!mutual || tid < c2) {
        const int pos = atomicAdd(&A.nedges, 1);  // < nb - 1: each edge joins two components
        if (pos < kLdsDistBlocks) {
          A.edge_d[pos] = bits_len(A.cmin_d[tid]);
          A.edge_t[pos] = A.cmin_t[tid];
        }
      }
      A.par[tid] = (mutual && tid < c2) ? tid : c2;
      A.cmin_d[tid] = kNoLen;
      A.cmin_t[tid] = kNoEdge;
    }
    // Pointer jumping over the hook forest (depth halves per pass).
    for (int it = 0; it < 16; ++it) {
      __syncthreads();
      const int np = is_root ? A.par[A.par[tid]] : 0;
      if (tid == 0) A.changed = 0;
      __syncthreads();
      if (is_root && np != A.par[tid]) {
        A.par[tid] = np;
        A.changed = 1;
      }
      __syncthreads();
      if (!A.changed) break;
    }
    const int nc = tid < nb ? A.par[A.comp[tid]] : 0;
    __syncthreads();
    if (tid < nb) A.comp[tid] = nc;
    __syncthreads();
  }
  const int ne = A.nedges < nb - 1 ? A.nedges : nb - 1;

  // ---- MST edges in ascending (length, tag) order.
  count_ranks<kSmallThreads>(ne, A.rank, [&](int f, int e) {
    return edge_less(A.edge_d[f], A.edge_t[f], A.edge_d[e], A.edge_t[e]);
  });
  __syncthreads();
  if (tid < ne) {
    const int r = A.rank[tid];
    A.sort_d[r] = A.edge_d[tid];
    A.sort_t[r] = A.edge_t[tid];
  }
  __syncthreads();

  if (tid >= 64) return;  // one wavefront from here on

  // ---- Elder rule, top-k and CSR rows.
  double sal[SLOTS];
  if constexpr (SLOTS == 1)
    elder_masks(A.sort_d, A.sort_t, ne, sal);
  else
    elder_registers<SLOTS>(A.sort_d, A.sort_t, ne, sal);
  select_and_emit_wave<SLOTS>(sal, nb, sink, local_radius, topk, A.sal, A.topidx, row_ptr, col_idx,
                              col_capacity, salience);
}

// ------------------------------------------------------------------ larger schedules

// One 16 x 16 tile of the distance matrix per workgroup, one entry per thread.
// The tile's 16 + 16 centroids are staged into LDS 64 dims at a time (all loads
// of a chunk issued before any store), then each entry sums (c_i - c_j)^2 over
// d in ascending order, so entries (i, j) and (j, i) are bitwise equal.
constexpr int kDistTile = 16;
constexpr int kDistDims = 64;
__global__ __launch_bounds__(256) void distance_kernel(const double* __restrict__ cent_t, int nb,
                                                       int64_t D, double* __restrict__ dist) {
  __shared__ double ct[2][kDistDims][kDistTile];  // [i rows | j rows][dim][row]
  const int i0 = blockIdx.y * kDistTile, j0 = blockIdx.x * kDistTile;
  const int tid = threadIdx.x;
  const int ti = tid / kDistTile, tj = tid % kDistTile;
  const int nbe = (nb + 1) & ~1;
  double acc = 0.0;
  for (int64_t d0 = 0; d0 < D; d0 += kDistDims) {
    const int w = (int)((D - d0) < kDistDims ? (D - d0) : kDistDims);
    __syncthreads();  // previous chunk consumed
    // 2 x w x 16 values over 256 threads: up to 8 per thread, loaded first
    constexpr int kPer = 2 * kDistDims * kDistTile / 256;
    double r[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = u * 256 + tid;  // (side, d, row)
      const int side = e / (kDistDims * kDistTile), rem = e % (kDistDims * kDistTile);
      const int d = rem / kDistTile, row = rem % kDistTile;
      const int blk = (side ? j0 : i0) + row;
      const int dd = d < w ? d : w - 1;
      r[u] = cent_t[(d0 + dd) * nbe + (blk < nb ? blk : nb - 1)];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = u * 256 + tid;
      (&ct[0][0][0])[e] = r[u];
    }
    __syncthreads();
#pragma unroll 8
    for (int d = 0; d < w; ++d) {
      const double df = ct[0][d][ti] - ct[1][d][tj];
      acc = __builtin_fma(df, df, acc);
    }
  }
  const int i = i0 + ti, j = j0 + tj;
  if (i < nb && j < nb) dist[(int64_t)i * nb + j] = finite_or_inf(__builtin_sqrt(acc));
}

// One wavefront per block v: the least edge from v to a block of another
// component.  state = {MST edges so far, done}.
__global__ __launch_bounds__(256) void boruvka_nearest(const double* __restrict__ dist, int nb,
                                                       const int* __restrict__ comp,
                                                       const int* __restrict__ state,
                                                       double* __restrict__ best_d,
                                                       uint32_t* __restrict__ best_t) {
  if (state[1]) return;
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (v >= nb) return;  // whole wavefront
  const int cv = comp[v];
  const double* row = dist + (int64_t)v * nb;
  double bd = __builtin_inf();
  uint32_t bt = kNoEdge;
  for (int j = lane; j < nb; j += 64) {
    if (comp[j] == cv) continue;
    const double d = row[j];
    const uint32_t t = edge_tag(v, j);
    if (edge_less(d, t, bd, bt)) {
      bd = d;
      bt = t;
    }
  }
  wave_edge_min(bd, bt);
  if (lane == 0) {
    best_d[v] = bd;
    best_t[v] = bt;
  }
}

// One workgroup: per-component least edge, hooking, pointer jumping, new
// labels; the round's MST edges are appended to edge_d / edge_t.
// Dynamic LDS: comp, hook, par (int), cmin_t (u32), cmin_d (u64), nb each.
__global__ __launch_bounds__(kLargeThreads) void boruvka_merge(int nb, int* __restrict__ comp,
                                                               int* __restrict__ state,
                                                               const double* __restrict__ best_d,
                                                               const uint32_t* __restrict__ best_t,
                                                               double* __restrict__ edge_d,
                                                               uint32_t* __restrict__ edge_t) {
  if (state[1]) return;
  extern __shared__ __attribute__((aligned(16))) unsigned long long lds_u64[];
  unsigned long long* cmin_d = lds_u64;
  uint32_t* cmin_t = (uint32_t*)(cmin_d + nb);
  int* lcomp = (int*)(cmin_t + nb);
  int* hook = lcomp + nb;
  int* par = hook + nb;
  __shared__ int nedges, changed;
  const int tid = threadIdx.x;
  if (tid == 0) nedges = state[0];
  for (int v = tid; v < nb; v += kLargeThreads) {
    lcomp[v] = comp[v];
    cmin_d[v] = kNoLen;
    cmin_t[v] = kNoEdge;
  }
  __syncthreads();
  for (int v = tid; v < nb; v += kLargeThreads)
    if (best_t[v] != kNoEdge) atomicMin(&cmin_d[lcomp[v]], len_bits(best_d[v]));
  __syncthreads();
  for (int v = tid; v < nb; v += kLargeThreads) {
    const uint32_t t = best_t[v];
    if (t != kNoEdge && len_bits(best_d[v]) == cmin_d[lcomp[v]]) atomicMin(&cmin_t[lcomp[v]], t);
  }
  __syncthreads();
  for (int c = tid; c < nb; c += kLargeThreads)
    if (lcomp[c] == c) {
      const uint32_t t = cmin_t[c];  // always an edge while two components remain
      const int lo = (int)(t >> 16), hi = (int)(t & 0xffffu);
      hook[c] = t == kNoEdge ? c : lcomp[lcomp[lo] == c ? hi : lo];
    }
  __syncthreads();
  for (int c = tid; c < nb; c += kLargeThreads)
    if (lcomp[c] == c) {
      const int c2 = hook[c];
      const bool mutual = hook[c2] == c;
      if (!mutual || c < c2) {
        const int pos = atomicAdd(&nedges, 1);  // < nb - 1: each edge joins two components
        if (pos < nb) {
          edge_d[pos] = bits_len(cmin_d[c]);
          edge_t[pos] = cmin_t[c];
        }
      }
      par[c] = (mutual && c < c2) ? c : c2;
    }
  for (int it = 0; it < 32; ++it) {
    __syncthreads();
    int np[kLargePerThread];
#pragma unroll
    for (int k = 0; k < kLargePerThread; ++k) {
      const int c = tid + k * kLargeThreads;
      np[k] = (c < nb && lcomp[c] == c) ? par[par[c]] : -1;
    }
    if (tid == 0) changed = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kLargePerThread; ++k) {
      const int c = tid + k * kLargeThreads;
      if (np[k] >= 0 && np[k] != par[c]) {
        par[c] = np[k];
        changed = 1;
      }
    }
    __syncthreads();
    if (!changed) break;
  }
  for (int v = tid; v < nb; v += kLargeThreads) comp[v] = par[lcomp[v]];
  __syncthreads();
  if (tid == 0) {
    state[0] = nedges;
    state[1] = nedges >= nb - 1 ? 1 : 0;
  }
}

// Edge ranks, elder rule, top-k and CSR emission for nb > kLdsDistBlocks.
// Dynamic LDS regions (reused across phases):
//   R0 double[nb]  edge lengths   -> salience
//   R1 int[nb+1]   edge tags      -> union-find parent -> top prefix
//   R2 double[nb]  sorted lengths -> row sizes / starts (int[nb+1])
//   R3 int[nb]     sorted tags    -> top-k list
//   R4 int[nb+1]   edge ranks     -> component sizes -> block ranks
__global__ __launch_bounds__(kLargeThreads) void finish_kernel(
    int nb, const int* __restrict__ state, const double* __restrict__ edge_d_g,
    const uint32_t* __restrict__ edge_t_g, int sink, int local_radius, int topk,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx, int64_t col_capacity,
    double* __restrict__ salience) {
  extern __shared__ __attribute__((aligned(16))) double lds_f64[];
  const int n1 = (nb + 2) & ~1;  // nb + 1 rounded up to even (keeps doubles aligned)
  double* R0 = lds_f64;
  double* R2 = R0 + nb;
  int* R1 = (int*)(R2 + nb);
  int* R3 = R1 + n1;
  int* R4 = R3 + n1;
  __shared__ int tmp[kLargeThreads / 64];
  const int tid = threadIdx.x;
  const int ne = state[0] < nb - 1 ? state[0] : nb - 1;

  double* ed = R0;
  uint32_t* et = (uint32_t*)R1;
  double* sd = R2;
  uint32_t* st = (uint32_t*)R3;
  int* rank = R4;
  for (int e = tid; e < ne; e += kLargeThreads) {
    ed[e] = edge_d_g[e];
    et[e] = edge_t_g[e];
    rank[e] = 0;
  }
  __syncthreads();
  count_ranks<kLargeThreads>(ne, rank, [&](int f, int e) {
    return edge_less(ed[f], et[f], ed[e], et[e]);
  });
  __syncthreads();
  for (int e = tid; e < ne; e += kLargeThreads) {
    sd[rank[e]] = ed[e];
    st[rank[e]] = et[e];
  }
  __syncthreads();

  // Elder rule: union-find in LDS, union by size with the elder tie rule; lanes
  // 0 and 1 follow the parent chains of the two endpoints.
  double* sal = R0;
  int* parent = R1;
  int* csize = R4;
  for (int v = tid; v < nb; v += kLargeThreads) {
    sal[v] = 0.0;
    parent[v] = v;
    csize[v] = 1;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    for (int base = 0; base < ne; base += 64) {
      const int r = base + lane;
      const int tw = r < ne ? (int)st[r] : 0;
      const double dw = r < ne ? sd[r] : 0.0;
      const int n = ne - base < 64 ? ne - base : 64;
      for (int k = 0; k < n; ++k) {
        const int t = read_lane(tw, k);
        const int a = (int)((uint32_t)t >> 16), b = t & 0xffff;
        int x = lane == 0 ? a : b;
        if (lane < 2) {
          // parents only ever point at a root of the moment, so chains are
          // acyclic and at most log2(nb) long
          for (int h = 0; h < nb; ++h) {
            const int p = parent[x];
            if (p == x) break;
            x = p;
          }
        }
        const int ra = read_lane(x, 0), rb = read_lane(x, 1);
        const int sa = csize[ra], sb = csize[rb];
        const bool a_survives = sa > sb || (sa == sb && ra < rb);
        const int surv = a_survives ? ra : rb, absorbed = a_survives ? rb : ra;
        const double w = read_lane(dw, k);
        if (lane == 0) {
          parent[absorbed] = surv;
          parent[a] = surv;
          parent[b] = surv;
          csize[surv] = sa + sb;
          sal[absorbed] = w;
        }
      }
    }
  }
  __syncthreads();

  select_and_emit<kLargeThreads>(sal, nb, sink, local_radius, topk, R4, R1, R3, (int*)R2, tmp,
                                 row_ptr, col_idx, col_capacity, salience);
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

struct WorkspaceLayout {
  size_t cent, dist, comp, state, best_d, best_t, edge_d, edge_t, total;
};

WorkspaceLayout workspace_layout(int64_t nb, int64_t D) {
  WorkspaceLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t n = (size_t)nb;
  L.cent = take((size_t)((nb + 1) & ~1) * (size_t)D * sizeof(double));
  L.dist = take(n * n * sizeof(double));
  L.comp = take(n * sizeof(int));
  L.state = take(2 * sizeof(int));
  L.best_d = take(n * sizeof(double));
  L.best_t = take(n * sizeof(uint32_t));
  L.edge_d = take(n * sizeof(double));
  L.edge_t = take(n * sizeof(uint32_t));
  L.total = off;
  return L;
}

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

}  // namespace

size_t schedule_workspace_bytes(int64_t nb, int64_t D) { return workspace_layout(nb, D).total; }

hipError_t launch_build_schedule(const void* keys, bool bf16, int64_t S, int64_t D, int sink,
                                 int local_radius, int topk, int32_t* row_ptr, int32_t* col_idx,
                                 int64_t col_capacity, double* salience, void* workspace,
                                 hipStream_t stream) {
  const int64_t nb64 = (S + kBlock - 1) / kBlock;
  if (nb64 == 0) return launch_dense_schedule(0, row_ptr, col_idx, stream);
  const int nb = (int)nb64;
  const WorkspaceLayout L = workspace_layout(nb, D);
  char* ws = (char*)workspace;
  double* cent_t = (double*)(ws + L.cent);
  const bool small = nb <= kLdsDistBlocks;
  int* comp = (int*)(ws + L.comp);
  int* state = (int*)(ws + L.state);
  hipLaunchKernelGGL(centroid_kernel, dim3((unsigned)nb), dim3(256), 0, stream,
                     (const uint16_t*)keys, bf16, S, D, nb, cent_t, small ? nullptr : comp,
                     small ? nullptr : state);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  double* dist = (double*)(ws + L.dist);
  const unsigned tiles = (unsigned)((nb + kDistTile - 1) / kDistTile);
  hipLaunchKernelGGL(distance_kernel, dim3(tiles, tiles), dim3(256), 0, stream, cent_t, nb, D,
                     dist);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  if (small) {
    const size_t lds = (size_t)small_stage_offset(nb) * sizeof(double) + kStageBytes;
    if (nb <= 64) {
      if ((err = allow_lds(topology_small<1>, lds)) != hipSuccess) return err;
      hipLaunchKernelGGL(topology_small<1>, dim3(1), dim3(kSmallThreads), lds, stream, dist, nb,
                         sink, local_radius, topk, row_ptr, col_idx, col_capacity, salience);
    } else {
      if ((err = allow_lds(topology_small<2>, lds)) != hipSuccess) return err;
      hipLaunchKernelGGL(topology_small<2>, dim3(1), dim3(kSmallThreads), lds, stream, dist, nb,
                         sink, local_radius, topk, row_ptr, col_idx, col_capacity, salience);
    }
    return hipGetLastError();
  }

  double* best_d = (double*)(ws + L.best_d);
  uint32_t* best_t = (uint32_t*)(ws + L.best_t);
  double* edge_d = (double*)(ws + L.edge_d);
  uint32_t* edge_t = (uint32_t*)(ws + L.edge_t);
  const size_t merge_lds = (size_t)nb * (sizeof(unsigned long long) + sizeof(uint32_t) + 3 * sizeof(int));
  if ((err = allow_lds(boruvka_merge, merge_lds)) != hipSuccess) return err;
  int rounds = 0;
  while ((1 << rounds) < nb) ++rounds;  // components at least halve per round
  for (int r = 0; r < rounds; ++r) {
    hipLaunchKernelGGL(boruvka_nearest, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, stream, dist,
                       nb, comp, state, best_d, best_t);
    hipLaunchKernelGGL(boruvka_merge, dim3(1), dim3(kLargeThreads), merge_lds, stream, nb, comp,
                       state, best_d, best_t, edge_d, edge_t);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const size_t n1 = (size_t)((nb + 2) & ~1);
  const size_t finish_lds = 2 * (size_t)nb * sizeof(double) + 3 * n1 * sizeof(int);
  if ((err = allow_lds(finish_kernel, finish_lds)) != hipSuccess) return err;
  hipLaunchKernelGGL(finish_kernel, dim3(1), dim3(kLargeThreads), finish_lds, stream, nb, state,
                     edge_d, edge_t, sink, local_radius, topk, row_ptr, col_idx, col_capacity,
                     salience);
  return hipGetLastError();
}

hipError_t launch_dense_schedule(int64_t nb, int32_t* row_ptr, int32_t* col_idx,
                                 hipStream_t stream) {
  const int64_t rows = nb + 1;
  const unsigned grid = (unsigned)((rows + 255) / 256);
  hipLaunchKernelGGL(dense_schedule_kernel, dim3(grid), dim3(256), 0, stream, nb, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace tsa
