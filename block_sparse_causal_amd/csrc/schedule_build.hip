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
//   nb <= 128: one launch of schedule_small.  Each workgroup forms the
//     centroids of one tile of block pairs from the keys and their distances;
//     the workgroups then elect one (device-coherent flags and a claim word,
//     no waiting) that finishes alone: the matrix into LDS; Boruvka rounds;
//     MST edges ranked; the elder rule over them in rank order (one wavefront,
//     per-block component keys in registers); blocks ranked by salience with
//     an exact integer key; CSR rows emitted.
//   nb > 128:
//     centroid_kernel   one workgroup per key block: fp64 mean of its keys,
//                       stored dimension-major (dim d of centroid j at
//                       d * nbe + j, nbe = nb rounded up to even);
//     distance_kernel   the nb x nb distance matrix, one entry per thread over
//                       many CUs;
//     boruvka_round     ceil(log2 nb) launches (every round at least halves
//                       the number of components): per block, the least edge
//                       to another component, one wavefront each; then the
//                       workgroups elect one (as above) that merges the
//                       components (hooking, pointer jumping, new labels, the
//                       new MST edges).  In the last launch the elected
//                       workgroup goes on: MST edges sorted (bitonic network
//                       in registers), elder rule 32 edges at a time (one
//                       wavefront), blocks ranked from runs of equal edge
//                       lengths, top-k, CSR rows emitted.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <type_traits>

#include "kernels.h"
#include "tsa.h"

namespace tsa {
namespace {

constexpr int kBlock = 64;
constexpr uint32_t kNoEdge = 0xffffffffu;          // "no candidate" edge tag
constexpr unsigned long long kNoLen = ~0ull;       // above the bits of +inf
constexpr int kStageBytes = 16384;                 // least LDS staging of centroid dims
constexpr int kSmallThreads = 512;
constexpr int kLargeThreads = 1024;
constexpr int kLargePerThread = 4;                 // blocks per thread in merge_components
static_assert(kLargeThreads * kLargePerThread >= 4096, "merge_components covers 4096 blocks");

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
// The edge order on length bits, with bitwise operators so that no condition
// short-circuits into control flow (for loops that take the lesser edge).
__device__ __forceinline__ bool edge_less_bits(unsigned long long d1, uint32_t t1,
                                               unsigned long long d2, uint32_t t2) {
  return (d1 < d2) | ((d1 == d2) & (t1 < t2));
}
// NaN (from NaN keys) is treated as +inf so that the edge order stays total.
__device__ __forceinline__ double finite_or_inf(double d) { return d == d ? d : __builtin_inf(); }

// Device-coherent 64-bit store and load (agent scope, relaxed): they bypass
// the non-coherent caches, so a value stored by one workgroup is seen by a
// load in another once the store has completed.
__device__ __forceinline__ void store_coherent(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(double* p, unsigned long long v) {
  store_coherent(reinterpret_cast<unsigned long long*>(p), v);
}
__device__ __forceinline__ unsigned long long load_coherent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this thread's vector memory operations have completed, and keeps
// the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));  // vmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

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
// v with lane LANE replaced by the uniform value x: one v_writelane_b32 (no
// builtin for it in this compiler; the lane is an inline constant, so the
// instruction reads one scalar register).
template <int LANE>
__device__ __forceinline__ int write_lane(int v, int x) {
  static_assert(LANE >= 0 && LANE < 64, "lane");
  asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(x), "n"(LANE));
  return v;
}
// f(integral_constant<int, I>) for I = FIRST .. LAST - 1, unrolled at compile time.
template <int FIRST, int LAST, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (FIRST < LAST) {
    f(std::integral_constant<int, FIRST>{});
    static_for<FIRST + 1, LAST>(f);
  }
}

// Value of per-block register array `a` for block x (x uniform; block x lives
// in lane x % 64, slot x / 64).
// Every slot is read with readlane and the slot is chosen among the scalar
// results: selecting among the VGPRs first lets the compiler turn the choice
// into a dynamically indexed array, which it keeps in scratch memory.
template <int SLOTS>
__device__ __forceinline__ int block_value(const int (&a)[SLOTS], int x) {
  const int s = x >> 6, l = x & 63;
  int val = read_lane(a[0], l);
#pragma unroll
  for (int k = 1; k < SLOTS; ++k) {
    const int t = read_lane(a[k], l);
    val = s == k ? t : val;
  }
  return val;
}

// Value of `v` in lane (lane ^ M), for the partner patterns of a bitonic
// network: M = 1, 2, 4, ..., 32 and the mirrors 3, 7, 15, 31, 63.  Each is a
// DPP move or a lane swap, or two of them (lane ^ A ^ B).
template <int M>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (M == 1) return xchg_quad1(v);
  else if constexpr (M == 2) return xchg_quad2(v);
  else if constexpr (M == 3) return __builtin_amdgcn_mov_dpp(v, 0x1B, 0xF, 0xF, false);  // quad reversed
  else if constexpr (M == 7) return xchg_half_mirror(v);
  else if constexpr (M == 15) return xchg_mirror(v);
  else if constexpr (M == 16) return xchg_xor16(v);
  else if constexpr (M == 32) return xchg_xor32(v);
  else if constexpr (M == 4) return lane_xor<7>(lane_xor<3>(v));
  else if constexpr (M == 8) return lane_xor<15>(lane_xor<7>(v));
  else if constexpr (M == 31) return lane_xor<15>(lane_xor<16>(v));
  else {
    static_assert(M == 63, "bitonic partner pattern");
    return lane_xor<31>(lane_xor<32>(v));
  }
}

// Compare-exchange of one bitonic step: the lower position of the pair keeps
// the smaller of (d, t) and (od, ot), the upper one the larger (keys are
// distinct but for the padding, whose copies are equal).
__device__ __forceinline__ void cx_take(unsigned long long& d, uint32_t& t, unsigned long long od,
                                        uint32_t ot, bool lower) {
  const bool take = (od < d || (od == d && ot < t)) == lower;
  d = take ? od : d;
  t = take ? ot : t;
}
template <int M>
__device__ __forceinline__ void cx_lanes(unsigned long long& d, uint32_t& t, bool lower) {
  const uint32_t lo = (uint32_t)lane_xor<M>((int)(uint32_t)d);
  const uint32_t hi = (uint32_t)lane_xor<M>((int)(uint32_t)(d >> 32));
  const uint32_t ot = (uint32_t)lane_xor<M>((int)t);
  cx_take(d, t, ((unsigned long long)hi << 32) | lo, ot, lower);
}

// The steps of the bitonic network of sort_edges for P keys, from merge width
// K and step J on, unrolled: the first step of a merge pairs position x with
// x ^ (K - 1), the later ones with x ^ J.  Partners in the same wavefront
// exchange values across lanes; the others meet in LDS (buf: 2 * kThreads
// entries, the halves taken in turn so that each such step needs one barrier).
// Wavefronts past the P keys only join the barriers.
template <int kThreads, int P, int K, int J, int HALF>
__device__ __forceinline__ void bitonic_steps(unsigned long long& d, uint32_t& t, uint4* buf) {
  if constexpr (K <= P) {
    constexpr int M = J == K / 2 ? K - 1 : J;
    const int x = threadIdx.x;
    const bool lower = (x & J) == 0;
    constexpr int kNextHalf = M < 64 ? HALF : HALF ^ 1;
    if constexpr (M < 64) {
      if ((x & ~63) < P) cx_lanes<M>(d, t, lower);
    } else {
      uint4* b = buf + HALF * kThreads;
      if (x < P) b[x] = make_uint4((uint32_t)d, (uint32_t)(d >> 32), t, 0u);
      __syncthreads();
      if (x < P) {
        const uint4 o = b[x ^ M];
        cx_take(d, t, ((unsigned long long)o.y << 32) | o.x, o.z, lower);
      }
    }
    if constexpr (J > 1)
      bitonic_steps<kThreads, P, K, J / 2, kNextHalf>(d, t, buf);
    else
      bitonic_steps<kThreads, P, K * 2, K, kNextHalf>(d, t, buf);
  }
}

// Ascending sort of n <= kThreads keys (length bits, tag), one per thread in
// position order (threads at and past n hold kNoLen, kNoEdge, which sort last),
// by the bitonic network of sort_edges in registers.  Every thread of the
// workgroup calls it.
template <int kThreads>
__device__ void sort_keys_in_registers(unsigned long long& d, uint32_t& t, int n, uint4* buf) {
  static_assert(kThreads <= 1024, "unrolled networks up to 1024 keys");
  if (n <= 2) {
    bitonic_steps<kThreads, 2, 2, 1, 0>(d, t, buf);
  } else if (n <= 4) {
    bitonic_steps<kThreads, 4, 2, 1, 0>(d, t, buf);
  } else if (n <= 8) {
    bitonic_steps<kThreads, 8, 2, 1, 0>(d, t, buf);
  } else if (n <= 16) {
    bitonic_steps<kThreads, 16, 2, 1, 0>(d, t, buf);
  } else if (n <= 32) {
    bitonic_steps<kThreads, 32, 2, 1, 0>(d, t, buf);
  } else if (n <= 64) {
    bitonic_steps<kThreads, 64, 2, 1, 0>(d, t, buf);
  } else if (n <= 128) {
    bitonic_steps<kThreads, 128, 2, 1, 0>(d, t, buf);
  } else if (n <= 256) {
    bitonic_steps<kThreads, 256, 2, 1, 0>(d, t, buf);
  } else if (n <= 512) {
    bitonic_steps<kThreads, 512, 2, 1, 0>(d, t, buf);
  } else {
    bitonic_steps<kThreads, 1024, 2, 1, 0>(d, t, buf);
  }
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

// Orders this wavefront's earlier LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Ascending in-place sort of the n edges (d[i], t[i]) (lengths, then tags; the
// tags are distinct, so the order is total) by the whole workgroup: a bitonic
// network over the next power of two P >= n in which every merge starts by
// comparing each element with its mirror in the merge block, so that every
// compare-exchange puts the smaller key at the lower index.  Positions n..P-1
// stand for keys above every edge and are never touched: a pair whose upper
// position is past n keeps its lower element.  Pair x is handled by thread
// x % kThreads; while the pair distance is at most 32, the 64 pairs of a
// wavefront stay inside one 128-element window of that wavefront, so such a
// step needs only a wavefront-level sync before the next step of the same kind.
// Ends with a workgroup barrier when n > 1 (no step runs otherwise).
template <int kThreads>
__device__ void sort_edges(double* d, uint32_t* t, int n) {
  int P = 1;
  while (P < n) P <<= 1;
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int x = threadIdx.x; x < P / 2; x += kThreads) {
        int lo, hi;
        if (j == (k >> 1)) {  // mirror step of the merge
          const int blk = x / j, off = x % j;
          lo = blk * k + off;
          hi = blk * k + k - 1 - off;
        } else {
          const int blk = x / j, off = x % j;
          lo = blk * 2 * j + off;
          hi = lo + j;
        }
        if (hi < n) {
          const double dl = d[lo], dh = d[hi];
          const uint32_t tl = t[lo], th = t[hi];
          if (edge_less(dh, th, dl, tl)) {
            d[lo] = dh;
            t[lo] = th;
            d[hi] = dl;
            t[hi] = tl;
          }
        }
      }
      // distance of the next step: j / 2 within this merge, else the next merge's k
      const int next = j > 1 ? (j >> 1) : k;
      if (next > 32 || (j == 1 && 2 * k > P))
        __syncthreads();
      else
        wave_lds_sync();
    }
  }
}

// Per-row top-k rows for the workgroup (brank: rank of each block under
// (-salience, index), valid when 0 < topk < nb).  Block j enters the top-k set
// of every row i with j <= i < e_j, where e_j is the topk-th smallest index
// among the blocks ranked above j (nb when fewer are, 0 when topk is 0): row i
// has exactly topk blocks ranked above j among its blocks 0..i from row e_j on.
// Row i lists, ascending: sink blocks [0, min(sink, i+1)), blocks j in
// [sink, i - r - 1] with i < e_j, local blocks [max(sink, i - r), i].
// Scratch (LDS): e[nb + 1], cnt[nb + 1], tmp.
template <int kThreads>
__device__ void emit_rows_per_row(int nb, int sink, int local_radius, int topk, const int* brank,
                                  int* e, int* cnt, int* tmp, int32_t* __restrict__ row_ptr,
                                  int32_t* __restrict__ col_idx, int64_t col_capacity) {
  const int tid = threadIdx.x;
  for (int v = tid; v < nb; v += kThreads) {
    int ev = topk == 0 ? 0 : nb;
    if (topk > 0 && topk < nb) {
      const int rv = brank[v];
      int c = 0;
      for (int u = 0; u < nb; ++u)
        if (brank[u] < rv && ++c == topk) {
          ev = u;
          break;
        }
    }
    e[v] = ev;
  }
  __syncthreads();
  for (int i = tid; i <= nb; i += kThreads) {
    int c = 0;
    if (i < nb) {
      const int a_n = sink < i + 1 ? sink : i + 1;
      const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
      const int b_n = loc_lo <= i ? i - loc_lo + 1 : 0;
      for (int j = sink; j <= i - local_radius - 1; ++j) c += e[j] > i ? 1 : 0;
      c += a_n + b_n;
    }
    cnt[i] = c;
  }
  __syncthreads();
  block_exclusive_scan<kThreads>(cnt, nb + 1, tmp);  // also leaves cnt[nb] = nnz
  for (int i = tid; i <= nb; i += kThreads) row_ptr[i] = cnt[i];
  // Entries: one wavefront per row; the middle part is compacted with a ballot.
  const int lane = tid & 63;
  for (int i = tid >> 6; i < nb; i += kThreads / 64) {
    const int a_n = sink < i + 1 ? sink : i + 1;
    const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
    const int t_hi = i - local_radius - 1;
    int64_t pos = cnt[i];
    for (int k = lane; k < a_n; k += 64)
      if (pos + k < col_capacity) col_idx[pos + k] = k;
    pos += a_n;
    for (int j0 = sink; j0 <= t_hi; j0 += 64) {
      const int j = j0 + lane;
      const bool take = j <= t_hi && e[j] > i;
      const uint64_t m = (uint64_t)__ballot(take);
      const int at = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (take && pos + at < col_capacity) col_idx[pos + at] = j;
      pos += __popcll(m);
    }
    for (int k = lane; loc_lo + k <= i; k += 64)
      if (pos + k < col_capacity) col_idx[pos + k] = loc_lo + k;
  }
}

// Rank of every block under (salience descending, index ascending), for the
// large path.  sd: MST edge lengths, ascending; dead[v]: rank of the edge that
// absorbs block v, or -1 for a root (which has salience 0); absorbed[r]: the
// block absorbed at edge r.  Equal saliences are runs of equal lengths in sd,
// so the rank of v is the number of blocks absorbed by longer edges, plus the
// blocks of its own run with a lower index, plus the roots below v when its
// salience is 0.  One root when the tree spans all nb blocks (root_blk).
template <int kThreads>
__device__ void rank_blocks(const double* sd, int ne, int nb, const int* dead, const int* absorbed,
                            int root_blk, int* brank) {
  for (int v = threadIdx.x; v < nb; v += kThreads) {
    const int r = dead[v];
    const double len = r >= 0 ? sd[r] : 0.0;
    int lo = 0, hi = 0;
    if (r >= 0) {
      lo = r;
      while (lo > 0 && sd[lo - 1] == len) --lo;
      hi = r + 1;
    }
    while (hi < ne && sd[hi] == len) ++hi;
    int rank = ne - hi;
    for (int q = lo; q < hi; ++q) rank += absorbed[q] < v ? 1 : 0;
    if (len == 0.0) {
      if (ne == nb - 1) {
        rank += root_blk < v ? 1 : 0;
      } else {
        for (int u = 0; u < v; ++u) rank += dead[u] < 0 ? 1 : 0;
      }
    }
    brank[v] = rank;
  }
}

// Top-k selection and CSR emission from the block ranks (brank, valid when
// 0 < topk < nb) for the large path.  The first min(topk, nb) blocks form the
// global top-k set.  Row i lists, ascending: sink blocks [0, min(sink, i+1)),
// top-k blocks in [sink, i - r - 1], local blocks [max(sink, i - r), i].
// Scratch (LDS): top[nb + 1], topidx[nb], cnt[nb + 1], tmp.  salience (if
// given) gets the per-block saliences.
template <int kThreads>
__device__ void select_and_emit(const double* sd, const int* dead, int nb, int sink,
                                int local_radius, int topk, bool per_row, int* brank, int* top,
                                int* topidx, int* cnt, int* tmp, int32_t* __restrict__ row_ptr,
                                int32_t* __restrict__ col_idx, int64_t col_capacity,
                                double* __restrict__ salience) {
  const int tid = threadIdx.x;
  const int kk = topk < nb ? topk : nb;
  if (!(kk > 0 && kk < nb))
    for (int v = tid; v < nb; v += kThreads) brank[v] = 0;  // all blocks or none pass rank < kk
  __syncthreads();
  if (salience != nullptr)
    for (int v = tid; v < nb; v += kThreads) salience[v] = dead[v] >= 0 ? sd[dead[v]] : 0.0;
  if (per_row) {
    emit_rows_per_row<kThreads>(nb, sink, local_radius, topk, brank, top, cnt, tmp, row_ptr,
                                col_idx, col_capacity);
    return;
  }
  for (int v = tid; v <= nb; v += kThreads) top[v] = (v < nb && brank[v] < kk) ? 1 : 0;
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

  // Entries: one thread per row.
  for (int i = tid; i < nb; i += kThreads) {
    const int a_n = sink < i + 1 ? sink : i + 1;
    const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
    const int t_hi = i - local_radius - 1;
    const int c_n = t_hi >= sink ? top[t_hi + 1] - top[sink] : 0;
    const int c0 = t_hi >= sink ? top[sink] : 0;
    int64_t at = cnt[i];
    for (int j = 0; j < a_n; ++j, ++at)
      if (at < col_capacity) col_idx[at] = j;
    for (int q = 0; q < c_n; ++q, ++at)
      if (at < col_capacity) col_idx[at] = topidx[c0 + q];
    for (int j = loc_lo; j <= i; ++j, ++at)
      if (at < col_capacity) col_idx[at] = j;
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
                                                       int64_t S, int64_t D, int nb, int block,
                                                       double* __restrict__ cent_t,
                                                       int* __restrict__ comp,
                                                       int* __restrict__ counters) {
  __shared__ double part[32][65];
  const int64_t j = blockIdx.x;
  const int64_t r0 = j * block;
  const int rows = (int)((r0 + block < S) ? block : S - r0);
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
  int dead_at[kLdsDistBlocks];                // per block: rank of the edge that absorbs it
  int nedges;
};
static_assert(sizeof(SmallState) <= kStageBytes, "small-schedule state fits the staging area");


// Elder rule over the MST edges in ascending order, one wavefront, nb <= 64 *
// SLOTS <= 128.  Every component is named by key (size << 8) | (255 - root),
// held by each of its blocks: of the two components an edge joins, the larger
// key belongs to the larger one, or on equal sizes to the lower root index,
// and its root survives.  The other root is absorbed at that edge.  Output per
// block v (lane v % 64, slot v / 64): the rank of the edge at which v was
// absorbed, or -1 for a root that never is.  The absorbed root's salience is
// that edge's length.
// The edges are taken 64 at a time with the loop over them unrolled, so that
// every lane index is a constant; lane k records the block absorbed at edge
// base + k, and after each group those ranks are scattered to the blocks
// through dead_at (LDS, nb entries).
template <int SLOTS>
__device__ __forceinline__ void elder_ranks(const uint32_t* st, int ne, int (&dead)[SLOTS], int* dead_at) {
  const int lane = threadIdx.x & 63;
  int ckey[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    ckey[s] = (1 << 8) | (255 - (lane + 64 * s));
    dead_at[lane + 64 * s] = -1;
  }
  for (int base = 0; base < ne; base += 64) {
    const int r = base + lane;
    const uint32_t tw = r < ne ? st[r] : 0u;
    const int aw = (int)(tw >> 16), bw = (int)(tw & 0xffffu);
    const int n = __builtin_amdgcn_readfirstlane(ne - base < 64 ? ne - base : 64);
    int absorbed = -1;  // lane k: the block absorbed at edge base + k
    static_for<0, 64>([&](auto KC) {
      constexpr int k = decltype(KC)::value;
      if (k < n) {
        const int a = read_lane(aw, k), b = read_lane(bw, k);
        const uint32_t ka = (uint32_t)block_value<SLOTS>(ckey, a);
        const uint32_t kb = (uint32_t)block_value<SLOTS>(ckey, b);
        const uint32_t hi = ka > kb ? ka : kb, lo = ka > kb ? kb : ka;
        const int grown = (int)(hi + (lo & ~255u));
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
          ckey[s] = ((uint32_t)ckey[s] == ka || (uint32_t)ckey[s] == kb) ? grown : ckey[s];
        absorbed = write_lane<k>(absorbed, 255 - (int)(lo & 255u));
      }
    });
    wave_lds_sync();
    if (absorbed >= 0) dead_at[absorbed] = r;  // each block is absorbed at most once
  }
  wave_lds_sync();
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) dead[s] = dead_at[lane + 64 * s];
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


// The elder rule of elder_ranks for the large path (any nb up to 4096), by one
// wavefront over the MST edges in ascending order (tags st[0, ne)), 32 edges
// at a time.  Between chunks the components are a union-find over the blocks:
// parent[] leads every block to its component's surviving root, and csize[]
// holds the size at each root.  The edges of one chunk touch at most 64
// components.  Each of those gets a local id (the lane of one of its
// occurrences, agreed through lid[]) and, in that lane, the key
// (size << 12) | (4095 - root), and the chunk's edges are applied to the keys
// in order as in elder_ranks.  Outputs: dead[v] = rank of the edge at which
// root v is absorbed (dead[] must hold -1 on entry), absorbed[r] = the root
// absorbed at edge r.
__device__ void elder_chunked(const uint32_t* st, int ne, int* parent, int* csize, int* lid,
                              int* dead, int* absorbed) {
  const int lane = threadIdx.x & 63;
  const int k = lane >> 1;  // the chunk edge of this lane; lane & 1 picks its endpoint
  for (int c0 = 0; c0 < ne; c0 += 32) {
    const int m = ne - c0 < 32 ? ne - c0 : 32;
    int root = 0;
    if (k < m) {
      const uint32_t tw = st[c0 + k];
      int x = (lane & 1) ? (int)(tw & 0xffffu) : (int)(tw >> 16);
      // Root of x, halving the path on the way (every write points a block at
      // one of its ancestors, so lanes that walk the same path concurrently
      // still end at the root).
      for (;;) {
        const int px = parent[x];
        if (px == x) break;
        const int gx = parent[px];
        parent[x] = gx;
        x = gx;
      }
      root = x;
      lid[root] = lane;  // among the lanes of one root, one write stays
    }
    wave_lds_sync();
    int id = 0, key = 0;
    if (k < m) {
      id = lid[root];
      if (id == lane) key = (csize[root] << 12) | (4095 - root);
    }
    int lost = -1;  // lane e: the root absorbed at edge c0 + e
    static_for<0, 32>([&](auto EC) {
      constexpr int e = decltype(EC)::value;
      if (e < m) {
        const int ia = read_lane(id, 2 * e), ib = read_lane(id, 2 * e + 1);
        const uint32_t ka = (uint32_t)read_lane(key, ia), kb = (uint32_t)read_lane(key, ib);
        const uint32_t hi = ka > kb ? ka : kb, lo = ka > kb ? kb : ka;
        const int grown = (int)(hi + (lo & ~4095u));
        key = ((uint32_t)key == ka || (uint32_t)key == kb) ? grown : key;
        lost = write_lane<e>(lost, 4095 - (int)(lo & 4095u));
      }
    });
    if (lane < m) {
      dead[lost] = c0 + lane;
      absorbed[c0 + lane] = lost;
    }
    if (k < m && id == lane) {
      const int survivor = 4095 - (key & 4095);
      parent[root] = survivor;
      csize[survivor] = key >> 12;  // every local id merged into it writes the same size
    }
    wave_lds_sync();
  }
}

// Per-row top-k rows by one wavefront (nb <= 64 * SLOTS <= 128), from the exact
// ranking keys of select_and_emit_wave (larger key = ranked higher).  Block j
// enters the top-k set of every row i with j <= i < e_j, where e_j is the
// topk-th smallest index among the blocks ranked above j (nb when fewer are, 0
// when topk is 0).  Row i lists, ascending: sink blocks [0, min(sink, i+1)),
// blocks j in [sink, i - r - 1] with i < e_j, local blocks [max(sink, i - r), i].
template <int SLOTS>
__device__ __forceinline__ void emit_rows_per_row_wave(const int (&key)[SLOTS], int nb, int sink,
                                                       int local_radius, int topk,
                                                       int32_t* __restrict__ row_ptr,
                                                       int32_t* __restrict__ col_idx,
                                                       int64_t col_capacity) {
  const int lane = threadIdx.x & 63;
  int e[SLOTS], seen[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    e[s] = topk == 0 ? 0 : nb;
    seen[s] = 0;
  }
  if (topk > 0 && topk < nb) {
    for (int u = 0; u < nb; ++u) {
      const int ku = block_value<SLOTS>(key, u);
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const bool above = ku > key[s];
        seen[s] += above ? 1 : 0;
        e[s] = (above && seen[s] == topk) ? u : e[s];
      }
    }
  }
  // Middle-part sizes: blocks j in [sink, i - r - 1] with i < e_j.
  int mid[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) mid[s] = 0;
  for (int j = sink; j < nb; ++j) {
    const int ej = block_value<SLOTS>(e, j);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int i = lane + 64 * s;
      mid[s] += (j <= i - local_radius - 1 && i < ej) ? 1 : 0;
    }
  }
  int carry = 0;
  int64_t start[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int i = lane + 64 * s;
    const int a_n = sink < i + 1 ? sink : i + 1;
    const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
    const int b_n = loc_lo <= i ? i - loc_lo + 1 : 0;
    const int n = i < nb ? a_n + mid[s] + b_n : 0;
    const int incl = wave_inclusive_scan(n);
    start[s] = carry + incl - n;
    carry += read_lane(incl, 63);
    if (i < nb) {
      row_ptr[i] = (int32_t)start[s];
      for (int j = 0; j < a_n; ++j)
        if (start[s] + j < col_capacity) col_idx[start[s] + j] = j;
      int64_t pos = start[s] + a_n + mid[s];
      for (int j = loc_lo; j <= i; ++j, ++pos)
        if (pos < col_capacity) col_idx[pos] = j;
      start[s] += a_n;  // next free entry of the middle part
    }
  }
  for (int j = sink; j < nb; ++j) {
    const int ej = block_value<SLOTS>(e, j);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int i = lane + 64 * s;
      if (i < nb && j <= i - local_radius - 1 && i < ej) {
        if (start[s] < col_capacity) col_idx[start[s]] = j;
        ++start[s];
      }
    }
  }
  if (lane == 0) row_ptr[nb] = carry;
}

// Top-k selection and CSR emission by one wavefront (nb <= 64 * SLOTS <= 128),
// rows as in select_and_emit.  Row i = lane + 64 * slot writes its own entries.
// dead: per block, the rank of the edge (in sd, ascending lengths) at which it
// was absorbed, or -1.  LDS scratch: grp[ne].
//
// Ranking is by (salience descending, index ascending).  Every salience is an
// edge length or 0, and sd is sorted, so the salience order is the order of
// grp = the first rank holding the same length (0 for a zero length); blocks
// never absorbed have salience 0, which ties with zero-length edges and is
// below every other length.  key = ((grp + 1) << 8) | (255 - v) is therefore
// an exact integer form of the ranking, distinct per block, and the top-k set
// is the blocks whose key is at least the k-th largest key.
template <int SLOTS>
__device__ __forceinline__ void select_and_emit_wave(const int (&dead)[SLOTS], const double* sd,
                                                     int ne, int nb, int sink, int local_radius,
                                                     int topk, bool per_row, int* grp,
                                                     int32_t* __restrict__ row_ptr,
                                                     int32_t* __restrict__ col_idx,
                                                     int64_t col_capacity,
                                                     double* __restrict__ salience) {
  const int lane = threadIdx.x & 63;
  const int kk = topk < nb ? topk : nb;
  // grp per edge rank: the last rank <= j that starts a run of equal lengths.
  int run = 0;
  for (int base = 0; base < ne; base += 64) {
    const int j = base + lane;
    const bool starts = j < ne && (j == 0 || sd[j - 1] != sd[j]);
    const uint64_t sm = (uint64_t)__ballot(starts);
    const uint64_t upto = sm & (lane == 63 ? ~0ull : ((2ull << lane) - 1ull));
    if (j < ne) grp[j] = upto != 0ull ? base + 63 - __clzll((long long)upto) : run;
    if (sm != 0ull) run = base + 63 - __clzll((long long)sm);
  }
  wave_lds_sync();
  const int zero_grp = ne > 0 && sd[0] == 0.0 ? 0 : -1;
  int key[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int v = lane + 64 * s;
    const int g = dead[s] >= 0 ? grp[dead[s]] : zero_grp;
    key[s] = v < nb ? ((g + 1) << 8) | (255 - v) : 0;
    if (salience != nullptr && v < nb) salience[v] = dead[s] >= 0 ? sd[dead[s]] : 0.0;
  }
  if (per_row) {
    emit_rows_per_row_wave<SLOTS>(key, nb, sink, local_radius, topk, row_ptr, col_idx,
                                  col_capacity);
    return;
  }
  // Top-k set as one bit mask per slot: the k-th largest key, bit by bit.
  uint64_t topm[SLOTS];
  if (kk >= nb || kk == 0) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) topm[s] = kk == 0 ? 0ull : (uint64_t)__ballot(lane + 64 * s < nb);
  } else if (const int cut = ne - kk; cut >= 0 && grp[cut] == cut && !(cut == 0 && zero_grp == 0)) {
    // No run of equal lengths crosses edge rank cut (and the root, salience 0,
    // does not tie with a selected block): every block absorbed at an edge of
    // rank >= cut has a larger key than every other block, so those kk blocks
    // are the set.
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) topm[s] = (uint64_t)__ballot(lane + 64 * s < nb && dead[s] >= cut);
  } else {
    int thr = 0;
#pragma unroll
    for (int bit = 15; bit >= 0; --bit) {
      const int cand = thr | (1 << bit);
      int cnt = 0;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) cnt += __popcll((uint64_t)__ballot(key[s] >= cand));
      thr = cnt >= kk ? cand : thr;
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) topm[s] = (uint64_t)__ballot(key[s] >= thr);
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
  // Selected blocks at or above the sinks, one mask per slot (uniform).  Row
  // i takes the first c_n of them in ascending order, so every row walks the
  // same list with scalar bit scans and keeps the entries it needs.
  uint64_t upper[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int rel = sink - 64 * s;
    upper[s] = rel <= 0 ? topm[s] : rel >= 64 ? 0ull : topm[s] & ~((1ull << rel) - 1ull);
  }
  // Row sizes, starts, entries.
  int carry = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int i = lane + 64 * s;
    const int a_n = sink < i + 1 ? sink : i + 1;
    const int loc_lo = (i - local_radius > sink) ? i - local_radius : sink;
    const int b_n = loc_lo <= i ? i - loc_lo + 1 : 0;
    const int t_hi = i - local_radius - 1;
    const int c_n = t_hi >= sink ? top_below(t_hi + 1) - top_below(sink) : 0;
    const bool row = i < nb;
    const int n = row ? a_n + c_n + b_n : 0;
    const int incl = wave_inclusive_scan(n);
    const int64_t start = carry + incl - n;
    carry += read_lane(incl, 63);
    if (row) row_ptr[i] = (int32_t)start;
    int64_t pos = start;
    for (int j = 0; j < a_n; ++j, ++pos)
      if (row && pos < col_capacity) col_idx[pos] = j;
    int k = 0;
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      for (uint64_t m = upper[u]; m != 0ull; m &= m - 1ull, ++k) {
        const int64_t at = pos + k;
        if (row && k < c_n && at < col_capacity) col_idx[at] = 64 * u + __builtin_ctzll(m);
      }
    }
    pos += c_n;
    for (int j = loc_lo; j <= i; ++j, ++pos)
      if (row && pos < col_capacity) col_idx[pos] = j;
  }
  if (lane == 0) row_ptr[nb] = carry;
}

// Doubles of LDS before the staging area: the distance matrix, rounded up to
// an even count so that the staging area is 16-byte aligned.
__host__ __device__ constexpr int small_stage_offset(int nb) { return (nb * nb + 1) & ~1; }

// Everything after the distances for nb <= kLdsDistBlocks, by one workgroup of
// 512 threads.  LDS at smem: small_stage_offset(nb) doubles (the distance
// matrix) + kStageBytes (SmallState).
template <int SLOTS>
__device__ __forceinline__ void small_topology(
    double* smem, const double* dist_g, int nb, int sink, int local_radius, int topk, bool per_row,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx, int64_t col_capacity,
    double* __restrict__ salience) {
  double* dist = smem;
  SmallState& A = *reinterpret_cast<SmallState*>(smem + small_stage_offset(nb));  // 16-byte aligned
  const int tid = threadIdx.x;
  const double kInf = __builtin_inf();

  // ---- Distance matrix (stored by the tile workgroups) into LDS, by
  // device-coherent loads.
  {
    const unsigned long long* src = reinterpret_cast<const unsigned long long*>(dist_g);
    const int n = nb * nb;
    for (int e0 = 0; e0 < n; e0 += 8 * kSmallThreads) {
      unsigned long long r[8];  // unconditional (clamped) loads, so that all eight are in flight
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kSmallThreads + tid;
        r[u] = load_coherent(src + (e < n ? e : n - 1));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kSmallThreads + tid;
        if (e < n) dist[e] = bits_len(r[u]);
      }
    }
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
  int nedges = 0;                             // MST edges so far (wavefront 0)
  for (int round = 0; round < 16; ++round) {  // ceil(log2 128) = 7 rounds suffice
    if (A.nedges >= nb - 1) break;
    // Least edge from each block to another component, over one part of the
    // candidates per thread; column reads of the symmetric matrix keep the
    // lanes on distinct banks.
    {
      const int v = tid % nbp, q = tid / nbp;
      unsigned long long bd = len_bits(kInf);
      uint32_t bt = kNoEdge;
      if (v < nb) {
        const int cv = A.comp[v];
        const int j1 = (q + 1) * plen < nb ? (q + 1) * plen : nb;
        // Eight candidates a pass: every load is issued before any is used.
        for (int j0 = q * plen; j0 < j1; j0 += 8) {
          int cj[8];
          double dj[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int j = j0 + u < nb ? j0 + u : nb - 1;
            cj[u] = A.comp[j];
            dj[u] = dist[j * nb + v];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint32_t t = edge_tag(v, j0 + u);
            const unsigned long long db = len_bits(dj[u]);
            const bool take = (j0 + u < j1) & (cj[u] != cv) & edge_less_bits(db, t, bd, bt);
            bd = take ? db : bd;
            bt = take ? t : bt;
          }
        }
      }
      A.part_d[tid] = bits_len(bd);
      A.part_t[tid] = bt;
    }
    __syncthreads();
    // The rest of the round on one wavefront: block v = lane + 64 * slot.
    if (tid < 64) {
      const int lane = tid;
      double bd[SLOTS];
      uint32_t bt[SLOTS];
      int cv[SLOTS];
#pragma unroll
      for (int sl = 0; sl < SLOTS; ++sl) {
        const int v = lane + 64 * sl;
        bd[sl] = kInf;
        bt[sl] = kNoEdge;
        cv[sl] = v;
        if (v < nb) {
          double pd[kSmallThreads / 64];
          uint32_t pt[kSmallThreads / 64];
#pragma unroll
          for (int q = 0; q < kSmallThreads / 64; ++q) {
            pd[q] = q < parts ? A.part_d[q * nbp + v] : kInf;
            pt[q] = q < parts ? A.part_t[q * nbp + v] : kNoEdge;
          }
#pragma unroll
          for (int q = 0; q < kSmallThreads / 64; ++q) {
            const bool take = edge_less(pd[q], pt[q], bd[sl], bt[sl]);
            bd[sl] = take ? pd[q] : bd[sl];
            bt[sl] = take ? pt[q] : bt[sl];
          }
          cv[sl] = A.comp[v];
          if (bt[sl] != kNoEdge) atomicMin(&A.cmin_d[cv[sl]], len_bits(bd[sl]));
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int sl = 0; sl < SLOTS; ++sl)
        if (lane + 64 * sl < nb && bt[sl] != kNoEdge && len_bits(bd[sl]) == A.cmin_d[cv[sl]])
          atomicMin(&A.cmin_t[cv[sl]], bt[sl]);
      wave_lds_sync();
      // Each component hooks onto the component across its least edge.  Edges
      // are strictly ordered, so the only cycles are pairs that chose each
      // other, and such a pair chose the same edge: the lower label stays a
      // root and records it; every other component records its own edge.
      bool root[SLOTS];
#pragma unroll
      for (int sl = 0; sl < SLOTS; ++sl) {
        const int v = lane + 64 * sl;
        root[sl] = v < nb && cv[sl] == v;
        bool rec = false;
        uint32_t t = kNoEdge;
        if (root[sl]) {
          t = A.cmin_t[v];  // always an edge while two components remain
          const int lo = (int)(t >> 16), hi = (int)(t & 0xffffu);
          const int c2 = t == kNoEdge ? v : A.comp[A.comp[lo] == v ? hi : lo];
          const bool mutual = c2 == v || A.cmin_t[c2] == t;  // c2 == v (no edge): nothing recorded
          rec = !mutual || v < c2;
          A.par[v] = (mutual && v <= c2) ? v : c2;
        }
        const uint64_t m = (uint64_t)__ballot(rec);
        const int pos = nedges + (int)__builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (rec) {  // pos < nb - 1: each edge joins two components
          A.edge_d[pos] = bits_len(A.cmin_d[v]);
          A.edge_t[pos] = t;
        }
        nedges += __popcll(m);
      }
      wave_lds_sync();
      // New label of each component: the root of its hook tree, found by
      // walking the parent chain, which ends because the hooks hold no other
      // cycle.
#pragma unroll
      for (int sl = 0; sl < SLOTS; ++sl) {
        const int v = lane + 64 * sl;
        if (root[sl]) {
          int x = A.par[v];
          for (int y = A.par[x]; y != x; y = A.par[x]) x = y;
          A.hook[v] = x;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int sl = 0; sl < SLOTS; ++sl) {
        const int v = lane + 64 * sl;
        if (v < nb) A.comp[v] = A.hook[cv[sl]];
        if (root[sl]) {
          A.cmin_d[v] = kNoLen;
          A.cmin_t[v] = kNoEdge;
        }
      }
      if (lane == 0) A.nedges = nedges;
    }
    __syncthreads();
  }
  const int ne = A.nedges < nb - 1 ? A.nedges : nb - 1;

  // ---- MST edges in ascending (length, tag) order: one key per thread in
  // registers (the distance matrix is no longer needed; its LDS, at least
  // 66 x 66 doubles when there are more than 64 edges, holds the exchanges
  // between wavefronts).
  {
    unsigned long long d = kNoLen;
    uint32_t t = kNoEdge;
    if (tid < ne) {
      d = len_bits(A.edge_d[tid]);
      t = A.edge_t[tid];
    }
    sort_keys_in_registers<kSmallThreads>(d, t, ne, reinterpret_cast<uint4*>(smem));
    if (tid < ne) {
      A.sort_d[tid] = bits_len(d);
      A.sort_t[tid] = t;
    }
  }
  __syncthreads();
  if (tid >= 64) return;  // one wavefront from here on

  // ---- Elder rule, top-k and CSR rows.
  int dead[SLOTS];
  elder_ranks<SLOTS>(A.sort_t, ne, dead, A.dead_at);
  select_and_emit_wave<SLOTS>(dead, A.sort_d, ne, nb, sink, local_radius, topk, per_row, A.rank,
                              row_ptr,
                              col_idx, col_capacity, salience);
}

// Election of the one workgroup of a launch of nwg workgroups that goes on
// alone (the scheme is described at schedule_small).  Every value that
// crosses workgroups (results, flags, the claim, the counter) moves by
// device-coherent accesses that bypass the non-coherent caches, so ordering
// needs only waits for completion, not cache write-back or invalidation.
// Every thread calls it once its cross-workgroup stores are issued; epoch is
// flags[nwg + 1] as loaded by threads 0..63 at the start of the launch.  The
// answer is the same in every thread of a workgroup.  flags: nwg + 3 words
// (flags, claim, epoch, counter), nwg <= kMaxElectFlags.
//
// The usual path is one atomic add per workgroup on the counter word, whose
// upper 48 bits hold a tag derived from epoch and whose low 16 bits count the
// workgroups that are done: the one that takes the count to nwg is the last.
// The elected workgroup advances epoch and leaves the counter at the next
// epoch's tag with a zero count, so the next launch on this workspace finds
// it ready.  A counter whose tag does not match (the workspace's first build,
// or one last used with another block count) is seen by every workgroup of
// the launch, which then elects by the token flags instead.
constexpr int kMaxElectFlags = 256;
__device__ __forceinline__ unsigned long long counter_tag(unsigned long long epoch) {
  return (epoch * 0x9E3779B97F4A7C15ull) >> 16;
}
__device__ bool elect_last_workgroup(unsigned long long* flags, int nwg,
                                     unsigned long long host_token, unsigned long long epoch) {
  __shared__ int elected;
  const int tid = threadIdx.x;
  wait_vmem();  // this thread's cross-workgroup stores have completed
  __syncthreads();
  if (tid < 64) {
    unsigned long long old = 0;
    if (tid == 0)
      old = __hip_atomic_fetch_add(&flags[nwg + 2], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(old >> 32), 0) << 32) |
          (uint32_t)__builtin_amdgcn_readlane((int)old, 0);
    bool win;
    if ((old >> 16) == counter_tag(epoch)) {
      win = (int)(old & 0xffffu) == nwg - 1;
    } else {
      const unsigned long long token = host_token + epoch * 0x9E3779B97F4A7C15ull;
      if (tid == 0) store_coherent(&flags[blockIdx.x], token);
      wait_vmem();  // the flag store completes before any flag is read
      unsigned long long f[kMaxElectFlags / 64];  // all loads in flight before any is compared
#pragma unroll
      for (int u = 0; u < kMaxElectFlags / 64; ++u) {
        const int t = tid + 64 * u;
        f[u] = (t < nwg && t != (int)blockIdx.x) ? load_coherent(&flags[t]) : token;
      }
      bool mine = true;
#pragma unroll
      for (int u = 0; u < kMaxElectFlags / 64; ++u) mine &= f[u] == token;
      const bool all = __ballot(!mine) == 0ull;
      int claim = 0;
      if (tid == 0)
        claim = all && __hip_atomic_exchange(&flags[nwg], token, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) != token;
      win = __builtin_amdgcn_readlane(claim, 0) != 0;
    }
    if (tid == 0) {
      elected = win;
      // Every workgroup has read epoch and added to the counter (before its
      // flag store, on the flag path).  Nothing in this launch reads either
      // word again, so the stores are not waited for (the next launch sees
      // them).
      if (win) {
        store_coherent(&flags[nwg + 1], epoch + 1ull);
        store_coherent(&flags[nwg + 2], counter_tag(epoch + 1ull) << 16);
      }
    }
  }
  __syncthreads();
  return elected != 0;
}

// schedule_small splits the upper triangle of the distance matrix into tiles
// of TILE x TILE blocks, one per workgroup; TILE is the smallest of 2, 4, 8
// that keeps the tile count within one workgroup per CU, since a smaller tile
// means fewer centroids formed per workgroup.
constexpr int kTileDims = 64;  // centroid dims per pass
constexpr int kMaxTiles = 256;
static_assert(kMaxTiles <= kMaxElectFlags, "one election flag per tile");
static_assert(4096 / (kLargeThreads / 64) <= kMaxElectFlags, "one election flag per round workgroup");
__host__ __device__ constexpr int small_tile_count(int nb, int tile) {
  return ((nb + tile - 1) / tile) * ((nb + tile - 1) / tile + 1) / 2;
}
__host__ __device__ constexpr int small_tile_edge(int nb) {
  return small_tile_count(nb, 2) <= kMaxTiles ? 2 : small_tile_count(nb, 4) <= kMaxTiles ? 4 : 8;
}
// LDS of schedule_small: the topology's, or the tile pass's partial sums
// [row group][slot][kTileDims] and centroids [kTileDims][16] if that is more.
__host__ __device__ constexpr size_t small_lds_bytes(int nb) {
  const size_t topo = (size_t)small_stage_offset(nb) * sizeof(double) + kStageBytes;
  const size_t tile = (size_t)(kSmallThreads / 8 + 16) * kTileDims * sizeof(double);
  return topo > tile ? topo : tile;
}

// The whole schedule for nb <= kLdsDistBlocks in one launch of
// small_tile_count(nb, TILE) workgroups.  Workgroup w takes tile (ti, tj),
// ti <= tj, of the block grid: it forms the centroids of its TILE row and TILE
// column blocks from the keys (fp64 sums, then a division by the row count,
// as centroid_kernel), and the distances between them: (c_i - c_j)^2 summed
// with fma over each quarter of every 64 dims, the quarters then added in
// order.  Each distance is formed once and stored at (i, j) and (j, i).
//
// Then the workgroups elect the one that continues with small_topology, without
// any waiting.  Usually each workgroup adds one to a counter once its
// distances are stored, and the one that takes the count to the number of
// workgroups wins (elect_last_workgroup).  When the counter is not set up for
// the launch (a workspace's first build), a workgroup instead publishes the
// call's token in its flag; one that then finds every flag equal to the token
// tries to swap the token into the claim word, and the one that finds the
// claim not yet holding it wins.  A workgroup reads the flags only after its
// own flag store has completed, so the one whose store completes last sees
// every flag: at least one workgroup reaches the swap, and the swap admits one.
// No flag needs clearing: stale flags hold older tokens.  The token is
// host_token + epoch * K, with epoch a word of the workspace that every
// workgroup reads first and the elected one advances: consecutive calls
// differ by 1 + K, and so do replays of a captured launch (its host_token
// frozen) by K.  flags: small_tile_count + 3 words of workspace (flags, claim,
// epoch, counter).
template <int SLOTS, int TILE, bool BF16>
__global__ __launch_bounds__(kSmallThreads) void schedule_small(
    const uint16_t* __restrict__ keys, int64_t S, int64_t D, int nb, int block,
    double* dist_g, unsigned long long* flags, unsigned long long host_token, int sink,
    int local_radius, int topk, int per_row, int32_t* __restrict__ row_ptr,
    int32_t* __restrict__ col_idx, int64_t col_capacity,
    double* __restrict__ salience) {
  static_assert(TILE == 2 || TILE == 4 || TILE == 8, "tile edge");
  constexpr int kSlots = 2 * TILE;                           // TILE row + TILE column blocks
  constexpr int kGroups = kSmallThreads / (8 * kSlots);      // row groups per block
  constexpr int kRowsPer = kBlock / kGroups;                 // rows per group (= 2 * TILE)
  extern __shared__ __attribute__((aligned(16))) double smem[];
  const int tid = threadIdx.x;
  const int T = (nb + TILE - 1) / TILE;
  const int ntiles = T * (T + 1) / 2;
  int ti = 0, w = (int)blockIdx.x;
  while (w >= T - ti) {
    w -= T - ti;
    ++ti;
  }
  const int tj = ti + w;
  const bool diag = ti == tj;
  // Issued first; needed only at the election.
  const unsigned long long epoch = tid < 64 ? load_coherent(&flags[ntiles + 1]) : 0ull;
  // Slot q (below TILE: row blocks, from TILE: column blocks) -> block index;
  // a diagonal tile's columns are its rows.
  auto slot_block = [&](int q) { return q < TILE ? ti * TILE + q : tj * TILE + (q - TILE); };
  auto block_rows = [&](int blk) -> int {
    const int64_t r0 = (int64_t)blk * block;
    return blk < nb ? (int)(r0 + block < S ? block : S - r0) : 0;
  };
  {
    double* part = smem;                                     // [row group][slot][dim]
    double* ct = smem + kGroups * kSlots * kTileDims;        // [dim][16]
    const int c = tid & 7, g = (tid >> 3) % kGroups, q = tid / (8 * kGroups);  // 8 dims, group, slot
    const int blk = slot_block(q);
    const int rows_blk = (diag && q >= TILE) ? 0 : block_rows(blk);
    const int rlo = kRowsPer * g;
    const uint16_t* kb_blk = keys + (int64_t)blk * block * D;
    const bool vec = (D % 8) == 0 && ((uintptr_t)keys % 16) == 0;  // 16-byte aligned rows
    double acc = 0.0;  // distance (ti*TILE + tid/TILE, tj*TILE + tid%TILE) for tid < TILE^2
    for (int64_t d0 = 0; d0 < D; d0 += kTileDims) {
      double sum8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const int64_t dc = d0 + 8 * c;
      // A block of `block` rows is walked in runs of kBlock rows; group g takes
      // rows rlo .. rlo + kRowsPer - 1 of every run.
      for (int run0 = 0; run0 < rows_blk; run0 += kBlock) {
        const int rows = rows_blk - run0 < kBlock ? rows_blk - run0 : kBlock;
        const uint16_t* kb = kb_blk + (int64_t)run0 * D;
        if (rows > rlo && vec && dc + 8 <= D) {
          // All rows of the group in flight at once (rows past the block's end
          // re-read its last row and are not added).
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          u32x4 x[kRowsPer];
#pragma unroll
          for (int u = 0; u < kRowsPer; ++u) {
            const int r = rlo + u < rows ? rlo + u : rows - 1;
            x[u] = *(const u32x4*)(kb + (int64_t)r * D + dc);
          }
#pragma unroll
          for (int u = 0; u < kRowsPer; ++u) {
            if (rlo + u < rows) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                sum8[2 * e] += key_to_double((uint16_t)(x[u][e] & 0xffffu), BF16);
                sum8[2 * e + 1] += key_to_double((uint16_t)(x[u][e] >> 16), BF16);
              }
            }
          }
        } else if (rows > rlo) {
          const int r1 = rows < rlo + kRowsPer ? rows : rlo + kRowsPer;
          for (int r = rlo; r < r1; ++r) {
            const uint16_t* row = kb + (int64_t)r * D;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (dc + e < D) sum8[e] += key_to_double(row[dc + e], BF16);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[(g * kSlots + q) * kTileDims + 8 * c + e] = sum8[e];
      __syncthreads();
      for (int e = tid; e < kSlots * kTileDims; e += kSmallThreads) {
        const int qq = e / kTileDims, d = e % kTileDims;
        const int src = (diag && qq >= TILE) ? qq - TILE : qq;
        const int n = block_rows(slot_block(src));
        double sm = part[src * kTileDims + d];
#pragma unroll
        for (int gg = 1; gg < kGroups; ++gg) sm += part[(gg * kSlots + src) * kTileDims + d];
        ct[d * 16 + qq] = n > 0 ? sm / (double)n : 0.0;
      }
      __syncthreads();
      // Four threads per entry, a quarter of the pass's dims each; the four
      // partial sums are added to the running sum in dim order.
      if (tid < 4 * TILE * TILE) {
        const int ent = tid >> 2, qd = tid & 3;
        const int i = ent / TILE, j = ent % TILE;
        const int wd = (int)(D - d0 < kTileDims ? D - d0 : kTileDims);
        const int da = qd * (kTileDims / 4), db = da + kTileDims / 4 < wd ? da + kTileDims / 4 : wd;
        double p = 0.0;
#pragma unroll 16
        for (int d = da; d < db; ++d) {
          const double df = ct[d * 16 + i] - ct[d * 16 + TILE + j];
          p = __builtin_fma(df, df, p);
        }
        part[tid] = p;  // the partial sums are consumed above this pass
      }
      __syncthreads();
      if (tid < TILE * TILE) acc += ((part[4 * tid] + part[4 * tid + 1]) + part[4 * tid + 2]) + part[4 * tid + 3];
      __syncthreads();  // part and ct are rewritten by the next pass
    }
    if (tid < TILE * TILE) {
      const int gi = ti * TILE + tid / TILE, gj = tj * TILE + tid % TILE;
      if (gi < nb && gj < nb) {
        const unsigned long long v = len_bits(finite_or_inf(__builtin_sqrt(acc)));
        store_coherent(dist_g + (int64_t)gi * nb + gj, v);
        store_coherent(dist_g + (int64_t)gj * nb + gi, v);
      }
    }
  }
  if (!elect_last_workgroup(flags, ntiles, host_token, epoch)) return;
  small_topology<SLOTS>(smem, dist_g, nb, sink, local_radius, topk, per_row != 0, row_ptr, col_idx,
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

// Per block v (one wavefront each): the least edge from v to a block of
// another component, stored by device-coherent stores for the merge of the
// same launch.  COHERENT: comp was stored in this launch (device-coherent
// loads skip stale cache lines).
__device__ __forceinline__ int load_comp(const int* comp, int v, bool coherent) {
  return coherent ? __hip_atomic_load(comp + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : comp[v];
}
template <bool COHERENT>
__device__ void nearest_edge(const double* __restrict__ dist, int nb, const int* comp, int v,
                             double* best_d, uint32_t* best_t) {
  const int lane = threadIdx.x & 63;
  const int cv = load_comp(comp, v, COHERENT);
  const double* row = dist + (int64_t)v * nb;
  unsigned long long bd = len_bits(__builtin_inf());
  uint32_t bt = kNoEdge;
  for (int j = lane; j < nb; j += 64) {
    const int cj = load_comp(comp, j, COHERENT);
    const unsigned long long d = len_bits(row[j]);
    const uint32_t t = edge_tag(v, j);
    const bool take = (cj != cv) & edge_less_bits(d, t, bd, bt);
    bd = take ? d : bd;
    bt = take ? t : bt;
  }
  double bdd = bits_len(bd);
  wave_edge_min(bdd, bt);
  if (lane == 0) {
    store_coherent(best_d + v, len_bits(bdd));
    __hip_atomic_store(best_t + v, bt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Per-component least edge, hooking, pointer jumping, new labels, by one
// workgroup of kLargeThreads; the round's MST edges are appended to edge_d /
// edge_t, and the new edge count is returned (in every thread).  best_d /
// best_t come from the other workgroups of the launch (device-coherent loads).
// LDS at lds: cmin_d (u64), cmin_t (u32), lcomp, hook, par (int), nb each.
__device__ int merge_components(int nb, int* __restrict__ comp, int* __restrict__ state, int nedges0,
                                const double* best_d, const uint32_t* best_t,
                                double* __restrict__ edge_d, uint32_t* __restrict__ edge_t,
                                unsigned long long* lds) {
  unsigned long long* cmin_d = lds;
  uint32_t* cmin_t = (uint32_t*)(cmin_d + nb);
  int* lcomp = (int*)(cmin_t + nb);
  int* hook = lcomp + nb;
  int* par = hook + nb;
  __shared__ int nedges, changed;
  const int tid = threadIdx.x;
  if (tid == 0) nedges = nedges0;
  unsigned long long bd[kLargePerThread];
  uint32_t bt[kLargePerThread];
#pragma unroll
  for (int k = 0; k < kLargePerThread; ++k) {
    const int v = tid + k * kLargeThreads;
    bd[k] = kNoLen;
    bt[k] = kNoEdge;
    if (v < nb) {
      bd[k] = load_coherent(reinterpret_cast<const unsigned long long*>(best_d) + v);
      bt[k] = __hip_atomic_load(best_t + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lcomp[v] = load_comp(comp, v, true);
      cmin_d[v] = kNoLen;
      cmin_t[v] = kNoEdge;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kLargePerThread; ++k) {
    const int v = tid + k * kLargeThreads;
    if (v < nb && bt[k] != kNoEdge) atomicMin(&cmin_d[lcomp[v]], bd[k]);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kLargePerThread; ++k) {
    const int v = tid + k * kLargeThreads;
    if (v < nb && bt[k] != kNoEdge && bd[k] == cmin_d[lcomp[v]]) atomicMin(&cmin_t[lcomp[v]], bt[k]);
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
        if (pos < nb) {  // device-coherent: the last round reads them back in this workgroup
          store_coherent(edge_d + pos, cmin_d[c]);
          __hip_atomic_store(edge_t + pos, cmin_t[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  for (int v = tid; v < nb; v += kLargeThreads)
    __hip_atomic_store(comp + v, par[lcomp[v]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int n = nedges;
  if (tid == 0) {
    state[0] = n;
    state[1] = n >= nb - 1 ? 1 : 0;
  }
  return n;
}

// Edge sort, elder rule, top-k and CSR emission for nb > kLdsDistBlocks.
// Dynamic LDS (finish_lds_bytes): sd double[nb], the MST edge lengths in
// ascending order; then int regions of n1 = nb + 1 rounded up to even: st
// (their tags), dead (per block, the rank of the edge that absorbs it, or -1),
// absorbed (per edge, the block it absorbs), W0, W1, W2 (the elder rule's
// parent, size and local ids; then ranks, top-k prefix and top-k list); then,
// when the edges fit one per thread, the sort's exchange buffer.
__host__ __device__ constexpr size_t finish_lds_base(int nb) {
  return ((size_t)nb * sizeof(double) + 6 * (size_t)((nb + 2) & ~1) * sizeof(int) + 15) & ~(size_t)15;
}
__host__ __device__ constexpr size_t finish_lds_bytes(int nb) {
  return finish_lds_base(nb) + (nb - 1 <= kLargeThreads ? 2 * kLargeThreads * 16 : 0);
}

__device__ void finish_schedule(int nb, int nedges, const double* edge_d_g, const uint32_t* edge_t_g,
                                int sink, int local_radius, int topk, bool per_row,
                                int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                int64_t col_capacity, double* __restrict__ salience,
                                double* lds_f64) {
  const int n1 = (nb + 2) & ~1;
  double* sd = lds_f64;
  uint32_t* st = reinterpret_cast<uint32_t*>(sd + nb);
  int* dead = reinterpret_cast<int*>(st + n1);
  int* absorbed = dead + n1;
  int* W0 = absorbed + n1;
  int* W1 = W0 + n1;
  int* W2 = W1 + n1;
  __shared__ int tmp[kLargeThreads / 64];
  __shared__ int root_blk;
  const int tid = threadIdx.x;
  const int ne = nedges < nb - 1 ? nedges : nb - 1;

  // ---- MST edges in ascending (length, tag) order.
  if (ne <= kLargeThreads) {
    uint4* sbuf = reinterpret_cast<uint4*>(reinterpret_cast<char*>(lds_f64) + finish_lds_base(nb));
    unsigned long long d = kNoLen;
    uint32_t t = kNoEdge;
    if (tid < ne) {  // stored by this workgroup: coherent loads skip stale cache lines
      d = load_coherent(reinterpret_cast<const unsigned long long*>(edge_d_g) + tid);
      t = __hip_atomic_load(edge_t_g + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sort_keys_in_registers<kLargeThreads>(d, t, ne, sbuf);
    if (tid < ne) {
      sd[tid] = bits_len(d);
      st[tid] = t;
    }
  } else {
    for (int e = tid; e < ne; e += kLargeThreads) {
      sd[e] = bits_len(load_coherent(reinterpret_cast<const unsigned long long*>(edge_d_g) + e));
      st[e] = __hip_atomic_load(edge_t_g + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    sort_edges<kLargeThreads>(sd, st, ne);
  }
  for (int v = tid; v < nb; v += kLargeThreads) {
    W0[v] = v;  // union-find parent
    W1[v] = 1;  // component size, at roots
    dead[v] = -1;
  }
  __syncthreads();

  // ---- Elder rule (one wavefront).
  if (tid < 64) elder_chunked(st, ne, W0, W1, W2, dead, absorbed);
  __syncthreads();

  // ---- Block ranks, top-k and CSR rows.
  const int kk = topk < nb ? topk : nb;
  if (kk > 0 && kk < nb) {
    for (int v = tid; v < nb; v += kLargeThreads)
      if (dead[v] < 0) root_blk = v;  // one root when ne == nb - 1
    __syncthreads();
    rank_blocks<kLargeThreads>(sd, ne, nb, dead, absorbed, root_blk, W0);
  }
  select_and_emit<kLargeThreads>(sd, dead, nb, sink, local_radius, topk, per_row, W0, W1, W2,
                                 absorbed, tmp, row_ptr, col_idx, col_capacity, salience);
}

// One Boruvka round of the schedule build for nb > kLdsDistBlocks, in one
// launch of ceil(nb / 16) workgroups: every wavefront finds the least edge out
// of one block's component (nearest_edge); the workgroups then elect the one
// that ends last (elect_last_workgroup), which merges the components
// (merge_components).  In the build's last launch (FINISH) that workgroup runs
// any rounds still needed by itself, then sorts the MST edges, applies the
// elder rule and emits the CSR rows (finish_schedule).  A launch that starts
// with the tree complete has nothing to hand between workgroups: it returns
// at once, except workgroup 0 of the last one, which finishes.  flags:
// ceil(nb / 16) + 3 words of workspace.
template <bool FINISH>
__global__ __launch_bounds__(kLargeThreads) void boruvka_round(
    const double* __restrict__ dist, int nb, int* __restrict__ comp, int* __restrict__ state,
    double* best_d, uint32_t* best_t, double* edge_d, uint32_t* edge_t,
    unsigned long long* flags, unsigned long long host_token, int sink, int local_radius, int topk,
    int per_row, int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    int64_t col_capacity, double* __restrict__ salience) {
  extern __shared__ __attribute__((aligned(16))) unsigned long long lds_u64[];
  const int tid = threadIdx.x;
  int nedges = state[0];
  if (state[1] != 0) {  // tree complete before this launch
    if (!FINISH || blockIdx.x != 0) return;
  } else {
    const unsigned long long epoch = tid < 64 ? load_coherent(&flags[gridDim.x + 1]) : 0ull;
    const int v = (int)blockIdx.x * (kLargeThreads / 64) + (tid >> 6);
    if (v < nb) nearest_edge<false>(dist, nb, comp, v, best_d, best_t);
    if (!elect_last_workgroup(flags, (int)gridDim.x, host_token, epoch)) return;
    nedges = merge_components(nb, comp, state, nedges, best_d, best_t, edge_d, edge_t, lds_u64);
    if (!FINISH) return;
    // Rounds past the launched ones: every round adds at least one edge while
    // two components remain (and at least halves their number), so the loop
    // ends well within its bound.
    for (int extra = 0; nedges < nb - 1 && extra < 16; ++extra) {
      wait_vmem();  // this workgroup's comp stores have completed
      __syncthreads();
      for (int u = tid >> 6; u < nb; u += kLargeThreads / 64)
        nearest_edge<true>(dist, nb, comp, u, best_d, best_t);
      wait_vmem();
      __syncthreads();
      nedges = merge_components(nb, comp, state, nedges, best_d, best_t, edge_d, edge_t, lds_u64);
    }
    wait_vmem();  // the merge's edge stores have completed before they are read back
    __syncthreads();  // and its LDS is reused
  }
  if (FINISH)
    finish_schedule(nb, nedges, edge_d, edge_t, sink, local_radius, topk, per_row != 0, row_ptr,
                    col_idx, col_capacity, salience, reinterpret_cast<double*>(lds_u64));
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

// Fixed segments of L blocks: row i lists blocks L*(i/L) .. i.  Row i starts
// after i/L full segments of L(L+1)/2 entries and the first i%L rows of its
// own segment, so every row and its entries have a closed form; one thread
// per row, the last thread writes row_ptr[nb].
__global__ void segment_schedule_kernel(int64_t nb, int64_t L, int32_t* __restrict__ row_ptr,
                                        int32_t* __restrict__ col_idx) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i > nb) return;
  const int64_t q = i / L, r = i % L;
  const int64_t base = q * (L * (L + 1) / 2) + r * (r + 1) / 2;
  row_ptr[i] = (int32_t)base;
  if (i < nb)
    for (int64_t j = 0; j <= r; ++j) col_idx[base + j] = (int32_t)(q * L + j);
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WorkspaceLayout {
  size_t cent, dist, comp, state, best_d, best_t, edge_d, edge_t, flags, total;
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
  L.flags = take((nb <= kLdsDistBlocks ? (size_t)small_tile_count((int)nb, small_tile_edge((int)nb))
                                       : (size_t)((nb + kLargeThreads / 64 - 1) / (kLargeThreads / 64))) *
                     sizeof(unsigned long long) +
                 3 * sizeof(unsigned long long));
  L.total = off;
  return L;
}

// A value unique to each schedule_small launch of this process: a nonzero
// 64-bit start drawn from the clock and the process id, then consecutive.
unsigned long long next_call_token() {
  static std::atomic<unsigned long long> next{[] {
    unsigned long long x = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    x ^= (unsigned long long)getpid() << 40;
    x *= 0x9E3779B97F4A7C15ull;  // spread the bits (Fibonacci hashing constant)
    return (x ^ (x >> 29)) | 1ull;
  }()};
  unsigned long long t = next.fetch_add(1, std::memory_order_relaxed);
  if (t == 0) t = next.fetch_add(1, std::memory_order_relaxed);
  return t;
}

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

}  // namespace

size_t schedule_workspace_bytes(int64_t nb, int64_t D) { return workspace_layout(nb, D).total; }

// The builder's workspace for callers that cannot allocate
// (tsa_build_schedule_noalloc): a fixed array in device memory, one copy per
// GPU, held until the process ends.  Every no-allocation build on a GPU uses
// that GPU's copy, so two such builds that overlap on one GPU race.  The
// builder needs no part of its workspace cleared.  In host code `scratch` only
// names the symbol; its device address comes from noalloc_scratch().
static __device__ __align__(256) unsigned char scratch[TSA_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up (with that
// device current) on the first call per device and kept.
hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex lookup;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> hold(lookup);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_build_schedule(const void* keys, bool bf16, int64_t S, int64_t D, int block,
                                 int sink, int local_radius, int topk, bool per_row,
                                 int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                 double* salience, void* workspace, hipStream_t stream) {
  const int64_t nbl = (S + block - 1) / block;
  if (nbl == 0) return launch_dense_schedule(0, row_ptr, col_idx, stream);
  const int nb = (int)nbl;
  const WorkspaceLayout L = workspace_layout(nb, D);
  char* ws = (char*)workspace;
  double* dist = (double*)(ws + L.dist);
  hipError_t err;
  if (nb <= kLdsDistBlocks) {
    unsigned long long* flags = (unsigned long long*)(ws + L.flags);
    const unsigned long long token = next_call_token();  // host part of the call's token
    const size_t lds = small_lds_bytes(nb);
    const int tile = small_tile_edge(nb);
    const dim3 grid((unsigned)small_tile_count(nb, tile));
    auto launch = [&](auto kernel) -> hipError_t {
      hipError_t e = allow_lds(kernel, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kernel, grid, dim3(kSmallThreads), lds, stream, (const uint16_t*)keys, S,
                         D, nb, block, dist, flags, token, sink, local_radius, topk, (int)per_row,
                         row_ptr, col_idx, col_capacity, salience);
      return hipGetLastError();
    };
    if (bf16) {
      if (nb <= 64)
        return tile == 2 ? launch(schedule_small<1, 2, true>) : launch(schedule_small<1, 4, true>);
      return tile == 4 ? launch(schedule_small<2, 4, true>) : launch(schedule_small<2, 8, true>);
    }
    if (nb <= 64)
      return tile == 2 ? launch(schedule_small<1, 2, false>) : launch(schedule_small<1, 4, false>);
    return tile == 4 ? launch(schedule_small<2, 4, false>) : launch(schedule_small<2, 8, false>);
  }

  double* cent_t = (double*)(ws + L.cent);
  int* comp = (int*)(ws + L.comp);
  int* state = (int*)(ws + L.state);
  hipLaunchKernelGGL(centroid_kernel, dim3((unsigned)nb), dim3(256), 0, stream,
                     (const uint16_t*)keys, bf16, S, D, nb, block, cent_t, comp, state);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const unsigned tiles = (unsigned)((nb + kDistTile - 1) / kDistTile);
  hipLaunchKernelGGL(distance_kernel, dim3(tiles, tiles), dim3(256), 0, stream, cent_t, nb, D,
                     dist);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  double* best_d = (double*)(ws + L.best_d);
  uint32_t* best_t = (uint32_t*)(ws + L.best_t);
  double* edge_d = (double*)(ws + L.edge_d);
  uint32_t* edge_t = (uint32_t*)(ws + L.edge_t);
  unsigned long long* flags = (unsigned long long*)(ws + L.flags);
  const size_t merge_lds = (size_t)nb * (sizeof(unsigned long long) + sizeof(uint32_t) + 3 * sizeof(int));
  const size_t last_lds = merge_lds > finish_lds_bytes(nb) ? merge_lds : finish_lds_bytes(nb);
  if ((err = allow_lds(boruvka_round<false>, merge_lds)) != hipSuccess) return err;
  if ((err = allow_lds(boruvka_round<true>, last_lds)) != hipSuccess) return err;
  const dim3 grid((unsigned)((nb + kLargeThreads / 64 - 1) / (kLargeThreads / 64)));
  // Launched rounds: half the worst case (components at least halve per round)
  // plus two; typical inputs need fewer, and the last launch runs any others.
  int log2nb = 0;
  while ((1 << log2nb) < nb) ++log2nb;
  const int rounds = log2nb / 2 + 2;
  for (int r = 0; r < rounds; ++r) {
    const unsigned long long token = next_call_token();
    if (r + 1 < rounds)
      hipLaunchKernelGGL(boruvka_round<false>, grid, dim3(kLargeThreads), merge_lds, stream, dist, nb,
                         comp, state, best_d, best_t, edge_d, edge_t, flags, token, sink,
                         local_radius, topk, (int)per_row, row_ptr, col_idx, col_capacity, salience);
    else
      hipLaunchKernelGGL(boruvka_round<true>, grid, dim3(kLargeThreads), last_lds, stream, dist, nb,
                         comp, state, best_d, best_t, edge_d, edge_t, flags, token, sink,
                         local_radius, topk, (int)per_row, row_ptr, col_idx, col_capacity, salience);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_segment_schedule(int64_t nb, int64_t segment_blocks, int32_t* row_ptr,
                                   int32_t* col_idx, hipStream_t stream) {
  const int64_t rows = nb + 1;
  const unsigned grid = (unsigned)((rows + 255) / 256);
  hipLaunchKernelGGL(segment_schedule_kernel, dim3(grid), dim3(256), 0, stream, nb, segment_blocks,
                     row_ptr, col_idx);
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
