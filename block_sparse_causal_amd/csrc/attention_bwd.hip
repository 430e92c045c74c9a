// Scheduled block-sparse causal attention backward for gfx950 (CDNA4).
//
// The pages' kernel is forward-only ("Add topology-derived sparse attention
// kernel", triton-lang/kernels PR 22, Summary, first bullet; the mirror page's
// note on learned segment boundaries records that without a backward, training
// would run dense).  These kernels differentiate that forward over the same CSR
// schedule.  With P_tu = exp(z_tu - lse_t) on the allowed keys of query row t:
//   dV = P^T dO,  dP = dO V^T,  Delta_t = dO_t . O_t,  dS = P * (dP - Delta),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Two kernels, no atomics, every output element written once:
//   dq kernel   - one workgroup per (lane, query block i), walking CSR row i:
//                 recomputes S^T and P^T, forms dP^T = V . dO^T and dS^T, and
//                 accumulates dQ^T += K^T . dS^T.  It also writes the per-row
//                 statistics (lse in log2 units, Delta) the second kernel reads.
//   dkdv kernel - one workgroup per (lane, key block j), walking column j of the
//                 transposed schedule (the query blocks whose rows list j):
//                 recomputes S = Q . K^T and P, dP = dO . V^T and dS, and
//                 accumulates dV^T += dO^T . P and dK^T += Q^T . dS.
//
// Both kernels mirror the forward's layout (4 waves = 2 row halves x 2 column
// halves, v_mfma_f32_32x32x16, a two-stage ring of direct global->LDS copies).
// The streamed operand is always read twice from LDS: row-wise as the A operand
// of the score-shaped product (its rows permuted by swapping bits 2 and 3, so
// that the result registers are already the B operand of the next product) and
// with transposing reads (ds_read_b64_tr_b16) as the A operand of the gradient
// product.  The stationary operand (Q and dO rows in the dq kernel, K and V
// rows in the dkdv kernel) stays in registers as B operands.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "mfma_tile.h"

namespace tsa {
namespace {

using namespace tile;

constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Geo {
  static constexpr int kStepsD = D / 16;          // 16-deep steps over the head dims
  static constexpr int kTilesD = D / 32;          // 32-row tiles of a [D x 32] accumulator
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kBlock * kRowBytes;
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kTileOps = 2 * kTileBytes / 1024 / kWaves;  // 1 KB copy ops per wave, two tiles
};

// LDS row r of every tile holds block row (r & 32) | swap_bits23(r & 31) and the
// 16-byte chunk c of that row sits at chunk c ^ k_swizzle(r).  fill_offsets gives,
// for each 1 KB copy op of wave w, the byte offset in the block's rows of the
// 16 bytes lane l moves (op o fills LDS piece o * kWaves + w of [tile A | tile B]).
template <int D>
__device__ __forceinline__ void fill_offsets(uint32_t (&off)[Geo<D>::kTileOps], int w, int l) {
  using G = Geo<D>;
#pragma unroll
  for (int op = 0; op < G::kTileOps; ++op) {
    const int chunk = (op * kWaves + w) * 64 + l;
    const int cc = chunk % (kBlock * G::kChunksPerRow);
    const int r = cc / G::kChunksPerRow, pc = cc % G::kChunksPerRow;
    const int row = (r & 32) | swap_bits23(r & 31);
    off[op] = (uint32_t)(row * G::kRowBytes + 16 * (pc ^ k_swizzle<D>(r)));
  }
}

// LDS address (tile base + offsets) of this lane's row-wise A-operand read for
// step c: MFMA row n of half `half` (block row half*32 + pi(n)), dims 16c+8h..+7.
template <int D>
__device__ __forceinline__ uint32_t row_read_addr(uint32_t base, int half, int n, int h, int c) {
  return base + (uint32_t)k_chunk_offset<D>(32 * half + n, 2 * c + h);
}

// LDS addresses of this lane's transposing reads for head-dim tile dt: within
// each 16-lane group, lane gi supplies the 8-byte piece (dims 4 (gi & 3) .. +3 of
// the group's 16 dims) of row r0 = 32 half + 4 h + gi / 4, which holds block row
// 32 half + 8 h + gi / 4 (a[0]), and of row r0 + 8, block row +4 (a[1]).  Adding
// 16 rows (block rows +16) leaves k_swizzle unchanged, so that one is an offset.
template <int D>
__device__ __forceinline__ void tr_read_addrs(uint32_t (&a)[2], uint32_t base, int half, int g, int gi,
                                              int dt) {
  const int r0 = 32 * half + 4 * (g >> 1) + (gi >> 2);
  const int dchunk = 4 * dt + 2 * (g & 1) + ((gi & 3) >> 1);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = r0 + 8 * e;
    a[e] = base + (uint32_t)(r * Geo<D>::kRowBytes + 16 * (dchunk ^ k_swizzle<D>(r)) + 8 * (gi & 1));
  }
}

// Issue the four transposing reads of one head-dim tile: block rows 16 gg + 8 h +
// 4 e + 0..3 of the lane's half for (gg, e) = (0,0), (0,1), (1,0), (1,1).
template <int kOff, int kRowBytes>
__device__ __forceinline__ void tr_reads(u32x2* dst, const uint32_t (&a)[2]) {
  dst[0] = lds_read_tr16<kOff>(a[0]);
  dst[1] = lds_read_tr16<kOff>(a[1]);
  dst[2] = lds_read_tr16<kOff + 16 * kRowBytes>(a[0]);
  dst[3] = lds_read_tr16<kOff + 16 * kRowBytes>(a[1]);
}
// A operand of k-step gg from the reads of one tile.
__device__ __forceinline__ u32x4 tr_operand(const u32x2* t, int gg) {
  const u32x2 lo = t[2 * gg], hi = t[2 * gg + 1];
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Maps workgroup b to (lane, position): workgroup b runs on XCD b % 8, which takes
// a contiguous group of lanes (its L2 then holds their operands) and runs their
// positions 0, 1, ... in turn.
__device__ __forceinline__ void grid_position(int nb, int64_t lane_base, int64_t& lane, int& pos) {
  const uint32_t G = gridDim.x, bid = blockIdx.x;
  const int lanes = (int)(G / (uint32_t)nb);
  if (G % 8u == 0u && lanes % 8 == 0) {
    const uint32_t lx = (uint32_t)lanes / 8u, u = bid / 8u;
    lane = lane_base + (int64_t)((bid % 8u) * lx + u % lx);
    pos = (int)(u / lx);
  } else {
    lane = lane_base + (int64_t)(bid % (uint32_t)lanes);
    pos = (int)(bid / (uint32_t)lanes);
  }
}

// Walker over one CSR row (or CSC column) whose accepted entries are strictly
// ascending and within [lo, hi]: entries are read 64 at a time into one register
// per lane and handed out with readlane; a reload waits for the memory counter
// right away so no other read ever waits on it.
struct ListWalker {
  int p, end, win, cols, lo, hi;
  __device__ __forceinline__ void init(const int32_t* ptr, const int32_t* idx, int64_t nnz, int r,
                                       int lo_, int hi_, int l) {
    p = (int)min((int64_t)max(ptr[r], 0), nnz);
    end = (int)max(min((int64_t)ptr[r + 1], nnz), (int64_t)p);
    lo = lo_;
    hi = hi_;
    win = p;
    cols = (p + l < end) ? idx[p + l] : -1;
    idx_ = idx;
    l_ = l;
  }
  __device__ __forceinline__ int next(int last) {
    while (p < end) {
      if (p - win >= 64) {
        win = p;
        cols = (p + l_ < end) ? idx_[p + l_] : -1;
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      }
      const int c = __builtin_amdgcn_readlane(cols, p - win);
      ++p;
      if (c > last && c >= lo && c <= hi) return c;
    }
    return -1;
  }
  // A walker with no entries.
  __device__ __forceinline__ void clear(const int32_t* idx, int l) {
    p = end = win = 0;
    cols = -1;
    lo = 0;
    hi = -1;
    idx_ = idx;
    l_ = l;
  }
  const int32_t* idx_;
  int l_;
};

// ----------------------------------------------------------------------------
// dq kernel
// ----------------------------------------------------------------------------
template <int D, bool BF16, int DO>
__global__ __launch_bounds__(kThreads) void attention_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t nnz, int S,
    int nb, int64_t lane_base, float scale_log2, float scale, float2* __restrict__ stats,
    uint16_t* __restrict__ dq) {
  using E = Elem<BF16>;
  using G = Geo<D>;
  constexpr int kStepsD = G::kStepsD, kTilesD = G::kTilesD, kTileBytes = G::kTileBytes;
  constexpr int kStageBytes = 2 * kTileBytes;  // [K tile | V tile]
  // Head dims of dQ written here: all D, or the half of D = 256 that blockIdx.y
  // selects (S and dP always contract over all D).
  static_assert(DO == D || 2 * DO == D, "a workgroup writes all the head dims or one of two halves");
  constexpr int kTilesO = DO / 32;
  const int d0 = DO < D ? (int)blockIdx.y * DO : 0;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = w & 1;   // query half
  const int kh = w >> 1;  // key half of every visited block
  const int l = tid & 63, h = l >> 5, n = l & 31, g = l >> 4, gi = l & 15;

  int64_t lane;
  int pos;
  grid_position(nb, lane_base, lane, pos);
  const int i = nb - 1 - pos;  // longest rows first
  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* kg = k + lane_off;
  const uint16_t* vg = v + lane_off;

  // Stationary operands of query row qrow: Q^T and dO^T as B operands (dims
  // 16c + 8h .. +7), the row's lse (log2 units) and Delta = dO . O, whose two
  // halves of the dims live in the two half-waves.
  const int qrow = i * kBlock + 32 * qh + n;
  const int qrow_c = qrow < S ? qrow : S - 1;
  const int64_t row_off = lane_off + (int64_t)qrow_c * D + 8 * h;
  u32x4 qop[kStepsD], dop[kStepsD];
  float delta = 0.0f;
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    qop[c] = *(const u32x4*)(q + row_off + 16 * c);
    dop[c] = *(const u32x4*)(dout + row_off + 16 * c);
    const u32x4 oc = *(const u32x4*)(o + row_off + 16 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) delta = E::dot_pair(dop[c][e], oc[e], delta);
  }
  delta = sum_with_other_half(delta);
  float lse2 = lse[lane * (int64_t)S + qrow_c] * kLog2e;
  if (kh == 0 && qrow < S && d0 == 0) stats[lane * (int64_t)S + qrow] = float2{lse2, delta};
  // Every load above has landed before any copy is queued, so the ring's waits
  // below count copies only.
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    asm volatile("" : "+v"(qop[c]));
    asm volatile("" : "+v"(dop[c]));
  }
  asm volatile("" : "+v"(lse2), "+v"(delta));

  uint32_t fill_off[G::kTileOps];
  fill_offsets<D>(fill_off, w, l);
  auto fill = [&](int j, uint8_t* stage) {
    const int rows = S - j * kBlock < kBlock ? S - j * kBlock : kBlock;
    copy_block_to_lds<G::kTileOps, G::kTileOps / 2, kWaves>(kg + (int64_t)j * kBlock * D,
                                                           vg + (int64_t)j * kBlock * D,
                                                           rows * G::kRowBytes, fill_off, stage, w);
  };

  ListWalker walk;
  walk.init(row_ptr, col_idx, nnz, i, 0, i, l);

  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)&ring[0];
  uint32_t a_addr[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) a_addr[c] = row_read_addr<D>(base, kh, n, h, c);
  uint32_t t_addr[kTilesO][2];
#pragma unroll
  for (int dt = 0; dt < kTilesO; ++dt) tr_read_addrs<D>(t_addr[dt], base, kh, g, gi, d0 / 32 + dt);

  f32x16 acc[kTilesO];
#pragma unroll
  for (int dt = 0; dt < kTilesO; ++dt) acc[dt] = f32x16{};

  auto compute = [&](int j, auto T_c) {
    // Stage offset: in the reads' 16-bit offset field when it fits, else (D = 256,
    // second stage at 64 KB) added to the lane addresses.
    constexpr int kStageAll = decltype(T_c)::value * kStageBytes;
    constexpr int kOff = kStageAll + kTileBytes + 16 * G::kRowBytes < 65536 ? kStageAll : 0;
    constexpr uint32_t kReg = (uint32_t)(kStageAll - kOff);
    // Operand reads in flight at once: all of them, or four steps at D = 256.
    constexpr int kChunk = kStepsD > 8 ? 4 : kStepsD;
    if (j == i && kh > qh) return;  // keys of this half all after the queries
    // S^T = K . Q^T and dP^T = V . dO^T: MFMA row m holds key 32kh + pi(m).
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c0 = 0; c0 < kStepsD; c0 += kChunk) {
      u32x4 ka[kChunk], va[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        ka[c] = lds_read_b128<kOff>(a_addr[c0 + c] + kReg);
        va[c] = lds_read_b128<kOff + kTileBytes>(a_addr[c0 + c] + kReg);
      }
      lds_wait_all(ka);
      lds_wait_all(va);
#pragma unroll
      for (int c = 0; c < kChunk; ++c) s = E::mfma(ka[c], qop[c0 + c], s);
#pragma unroll
      for (int c = 0; c < kChunk; ++c) dp = E::mfma(va[c], dop[c0 + c], dp);
    }
    // K^T operands of dQ^T += K^T . dS^T, landing while dS is formed.
    u32x2 kt[kTilesO * 4];
#pragma unroll
    for (int dt = 0; dt < kTilesO; ++dt) {
      const uint32_t ta[2] = {t_addr[dt][0] + kReg, t_addr[dt][1] + kReg};
      tr_reads<kOff, G::kRowBytes>(&kt[dt * 4], ta);
    }
    if (j == i && kh == qh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kpos = 16 * (r >> 3) + 8 * h + (r & 7);
        if (kpos > n) s[r] = -__builtin_inff();
      }
    }
    u32x4 pb[2];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 8 * gg + 2 * x;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -lse2));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], scale_log2, -lse2));
        pb[gg][x] = E::pack(p0 * (dp[r] - delta), p1 * (dp[r + 1] - delta));
      }
    lds_wait_all(kt);
#pragma unroll
    for (int dt = 0; dt < kTilesO; ++dt)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) acc[dt] = E::mfma(tr_operand(&kt[dt * 4], gg), pb[gg], acc[dt]);
  };

  // Ring over the row's blocks, as in the forward: wait for the stage's copy,
  // barrier, queue the next block into the stage computed one step ago, compute.
  int blk[2];
  blk[0] = walk.next(-1);
  blk[1] = blk[0] >= 0 ? walk.next(blk[0]) : -1;
  if (blk[0] >= 0) {
    fill(blk[0], ring);
    if (blk[1] >= 0) fill(blk[1], ring + kStageBytes);
    bool pre = blk[1] >= 0;
    int last = pre ? blk[1] : blk[0];
    bool done = false;
    auto step = [&](auto T_c) {
      constexpr int t = decltype(T_c)::value;
      constexpr int refill = t ^ 1;
      if (pre)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(G::kTileOps));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      ring_barrier();
      if (!pre) {
        const int jn = last >= 0 ? walk.next(last) : -1;
        blk[refill] = jn;
        last = jn;
        if (jn >= 0) fill(jn, ring + refill * kStageBytes);
      }
      pre = false;
      compute(blk[t], T_c);
      done = blk[refill] < 0;
    };
    while (!done) {
      step(std::integral_constant<int, 0>{});
      if (!done) step(std::integral_constant<int, 1>{});
    }
    __syncthreads();
  }

  // Sum the two key halves: wave kh keeps tiles [kh, kh + 1) * kTilesO / 2 and
  // hands the others to its partner through LDS, then stores scale * sum.
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  // Register groups of 4 (4 consecutive head dims each): kTilesO * 4 per lane.
  // Wave kh keeps groups [kh, kh + 1) * kGroups / 2 and sends the others.
  constexpr int kGroups = kTilesO * 4;
  constexpr int kHalfGroups = kGroups / 2;
  constexpr int kSendStride = kHalfGroups * 4 + 4;
  static_assert(4 * 64 * kSendStride * 4 <= 2 * kStageBytes, "merge area exceeds the ring");
  float* const xbase = (float*)&ring[0];
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  auto merge = [&](auto KHc) {
    constexpr int KH = decltype(KHc)::value;
    float* send = xbase + ((qh * 2 + KH) * 64 + l) * kSendStride;
#pragma unroll
    for (int u = 0; u < kHalfGroups; ++u) {
      constexpr int kSendBase = (1 - KH) * kHalfGroups;
      const int gq = kSendBase + u;  // compile-time after unrolling
      *(f32x4*)(send + 4 * u) = f32x4{acc[gq / 4][4 * (gq % 4)], acc[gq / 4][4 * (gq % 4) + 1],
                                      acc[gq / 4][4 * (gq % 4) + 2], acc[gq / 4][4 * (gq % 4) + 3]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    ring_barrier();
    const float* recv = xbase + ((qh * 2 + (1 - KH)) * 64 + l) * kSendStride;
    if (qrow < S) {
      uint16_t* drow = dq + lane_off + (int64_t)qrow * D;
#pragma unroll
      for (int u = 0; u < kHalfGroups; ++u) {
        constexpr int kKeepBase = KH * kHalfGroups;
        const int gq = kKeepBase + u;
        const f32x4 y = *(const f32x4*)(recv + 4 * u);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (acc[gq / 4][4 * (gq % 4) + e] + y[e]) * scale;
        u32x2 val;
        val[0] = E::pack(x[0], x[1]);
        val[1] = E::pack(x[2], x[3]);
        // group gq: tile gq / 4, register group gq % 4 -> dims d0 + 32 (gq / 4) + 8 (gq % 4) + 4h
        *(u32x2*)(drow + d0 + 32 * (gq / 4) + 8 * (gq % 4) + 4 * h) = val;
      }
    }
  };
  if (kh == 0)
    merge(std::integral_constant<int, 0>{});
  else
    merge(std::integral_constant<int, 1>{});
}

// ----------------------------------------------------------------------------
// dq kernel, two query blocks per workgroup
// ----------------------------------------------------------------------------
// The dq kernel's work for the query-block pair (2g, 2g+1) of one lane in one
// workgroup of 4 waves: wave w owns query half w & 1 of block 2g + (w >> 1) and
// takes both key halves of every block its row lists, one after the other, into
// one dQ^T accumulator, so no merge of key halves is needed.  The workgroup
// walks the union of the two CSR rows (as the forward's two-block kernel);
// each union block's K and V tiles are copied once and serve both rows, which
// share most of their blocks.  Used for launches with enough (lane, query
// block) pairs that the halved grid still fills the CUs.
template <int D, bool BF16, bool SUB>
__global__ __launch_bounds__(kThreads) void attention_bwd_dq_duo_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t nnz, int S,
    int nb, int nrows, int npairs, int64_t lane_base, float scale_log2, float scale,
    float2* __restrict__ stats, uint16_t* __restrict__ dq) {
  using E = Elem<BF16>;
  using G = Geo<D>;
  constexpr int kStepsD = G::kStepsD, kTilesD = G::kTilesD, kTileBytes = G::kTileBytes;
  constexpr int kStageBytes = 2 * kTileBytes;  // [K tile | V tile]
  constexpr int kHalfKeyBytes = 32 * G::kRowBytes;  // key half 1: 32 rows further, same swizzle
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rsel = w >> 1;  // which query block of the pair
  const int qh = w & 1;     // query half of that block
  const int l = tid & 63, h = l >> 5, n = l & 31, g = l >> 4, gi = l & 15;

  int64_t lane;
  int pos;
  grid_position(npairs, lane_base, lane, pos);
  const int pair = npairs - 1 - pos;  // longest rows first
  const int my_i = 2 * pair + rsel;   // >= nb: this wave's block is past the end
  const int my_q32 = 4 * pair + w;    // and its 32-row query block (2 my_i + qh)
  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* kg = k + lane_off;
  const uint16_t* vg = v + lane_off;

  // Stationary operands of query row qrow (as in the one-block dq kernel).
  const int qrow = my_i * kBlock + 32 * qh + n;
  const int qrow_c = qrow < S ? qrow : S - 1;
  const int64_t row_off = lane_off + (int64_t)qrow_c * D + 8 * h;
  u32x4 qop[kStepsD], dop[kStepsD];
  float delta = 0.0f;
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    qop[c] = *(const u32x4*)(q + row_off + 16 * c);
    dop[c] = *(const u32x4*)(dout + row_off + 16 * c);
    const u32x4 oc = *(const u32x4*)(o + row_off + 16 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) delta = E::dot_pair(dop[c][e], oc[e], delta);
  }
  delta = sum_with_other_half(delta);
  float lse2 = lse[lane * (int64_t)S + qrow_c] * kLog2e;
  if (qrow < S) stats[lane * (int64_t)S + qrow] = float2{lse2, delta};

  // The rows' walkers (the two 64-row blocks, or with SUB the four 32-row
  // ones, wave w's being walker w): the union of the rows in ascending order.
  constexpr int kWalk = SUB ? 4 : 2;
  ListWalker walk[kWalk];
  int head[kWalk];
#pragma unroll
  for (int r = 0; r < kWalk; ++r) {
    const int row = kWalk * pair + r;
    if (row < nrows)
      walk[r].init(row_ptr, col_idx, nnz, row, 0, row, l);
    else
      walk[r].clear(col_idx, l);
  }
  // Every load above has landed before any copy is queued, so the ring's waits
  // below count copies only.
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    asm volatile("" : "+v"(qop[c]));
    asm volatile("" : "+v"(dop[c]));
  }
  asm volatile("" : "+v"(lse2), "+v"(delta));
#pragma unroll
  for (int r = 0; r < kWalk; ++r) head[r] = walk[r].next(-1);
  // Next 64-key block of the union (-1: none); `mine` gets bit h set when this
  // wave computes key half h of it: both when its 64-row block's row lists the
  // block, or (SUB) the halves its 32-row row lists.
  auto next_block = [&](int& mine) -> int {
    int hmin = INT_MAX;
#pragma unroll
    for (int r = 0; r < kWalk; ++r)
      if (head[r] >= 0) hmin = min(hmin, head[r]);
    mine = 0;
    if (hmin == INT_MAX) return -1;
    const int j = SUB ? hmin >> 1 : hmin;
#pragma unroll
    for (int r = 0; r < kWalk; ++r) {
      if constexpr (SUB) {
#pragma unroll
        for (int e = 0; e < 2; ++e)  // at most the two 32-key blocks of j, ascending
          if (head[r] >= 0 && (head[r] >> 1) == j) {
            if (r == w) mine |= 1 << (head[r] & 1);
            head[r] = walk[r].next(head[r]);
          }
      } else if (head[r] == j) {
        if (r == rsel) mine = 3;
        head[r] = walk[r].next(j);
      }
    }
    return j;
  };

  uint32_t fill_off[G::kTileOps];
  fill_offsets<D>(fill_off, w, l);
  auto fill = [&](int j, uint8_t* stage) {
    const int rows = S - j * kBlock < kBlock ? S - j * kBlock : kBlock;
    copy_block_to_lds<G::kTileOps, G::kTileOps / 2, kWaves>(kg + (int64_t)j * kBlock * D,
                                                           vg + (int64_t)j * kBlock * D,
                                                           rows * G::kRowBytes, fill_off, stage, w);
  };

  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)&ring[0];
  uint32_t a_addr[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) a_addr[c] = row_read_addr<D>(base, 0, n, h, c);
  uint32_t t_addr[kTilesD][2];
#pragma unroll
  for (int dt = 0; dt < kTilesD; ++dt) tr_read_addrs<D>(t_addr[dt], base, 0, g, gi, dt);

  f32x16 acc[kTilesD];
#pragma unroll
  for (int dt = 0; dt < kTilesD; ++dt) acc[dt] = f32x16{};

  // Key half KH of block j, held by ring stage T (both compile-time).
  auto compute_half = [&](int j, auto T_c, auto KH_c) {
    constexpr int KH = decltype(KH_c)::value;
    constexpr int kOff = decltype(T_c)::value * kStageBytes + KH * kHalfKeyBytes;
    // 32-row key block 2j + KH against this wave's 32-row query block: later
    // ones are fully masked (the acceptance rule never lists them under SUB).
    if (2 * j + KH > my_q32) return;
    u32x4 ka[kStepsD], va[kStepsD];
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) {
      ka[c] = lds_read_b128<kOff>(a_addr[c]);
      va[c] = lds_read_b128<kOff + kTileBytes>(a_addr[c]);
    }
    lds_wait_all(ka);
    lds_wait_all(va);
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) s = E::mfma(ka[c], qop[c], s);
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) dp = E::mfma(va[c], dop[c], dp);
    u32x2 kt[kTilesD * 4];
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) tr_reads<kOff, G::kRowBytes>(&kt[dt * 4], t_addr[dt]);
    if (2 * j + KH == my_q32) {  // key position must not exceed query position
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kpos = 16 * (r >> 3) + 8 * h + (r & 7);
        if (kpos > n) s[r] = -__builtin_inff();
      }
    }
    u32x4 pb[2];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 8 * gg + 2 * x;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -lse2));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], scale_log2, -lse2));
        pb[gg][x] = E::pack(p0 * (dp[r] - delta), p1 * (dp[r + 1] - delta));
      }
    lds_wait_all(kt);
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) acc[dt] = E::mfma(tr_operand(&kt[dt * 4], gg), pb[gg], acc[dt]);
  };

  // Ring over the union: the first two blocks are queued here, one per stage;
  // at step t the wave waits for stage t's copies (the other stage's may stay in
  // flight), passes the barrier, queues the next union block into the stage
  // computed one step earlier, and computes both key halves when its row lists
  // the block.
  int blk[2];
  int mine[2] = {0, 0};
  blk[0] = next_block(mine[0]);
  blk[1] = blk[0] >= 0 ? next_block(mine[1]) : -1;
  if (blk[0] >= 0) {
    fill(blk[0], ring);
    if (blk[1] >= 0) fill(blk[1], ring + kStageBytes);
    bool pre = blk[1] >= 0;
    bool done = false;
    auto step = [&](auto T_c) {
      constexpr int t = decltype(T_c)::value;
      constexpr int refill = t ^ 1;
      if (pre)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(G::kTileOps));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      ring_barrier();
      if (!pre) {
        blk[refill] = next_block(mine[refill]);
        if (blk[refill] >= 0) fill(blk[refill], ring + refill * kStageBytes);
      }
      pre = false;
      if (mine[t] & 1) compute_half(blk[t], T_c, std::integral_constant<int, 0>{});
      if (mine[t] & 2) compute_half(blk[t], T_c, std::integral_constant<int, 1>{});
      done = blk[refill] < 0;
    };
    while (!done) {
      step(std::integral_constant<int, 0>{});
      if (!done) step(std::integral_constant<int, 1>{});
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));

  // The wave holds the whole dQ^T of its 32 query rows: scale, pack, store.
  if (qrow < S && my_i < nb) {
    uint16_t* drow = dq + lane_off + (int64_t)qrow * D;
#pragma unroll
    for (int gq = 0; gq < kTilesD * 4; ++gq) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[gq / 4][4 * (gq % 4) + e] * scale;
      u32x2 val;
      val[0] = E::pack(x[0], x[1]);
      val[1] = E::pack(x[2], x[3]);
      // group gq: tile gq / 4, register group gq % 4 -> dims 32 (gq / 4) + 8 (gq % 4) + 4h
      *(u32x2*)(drow + 32 * (gq / 4) + 8 * (gq % 4) + 4 * h) = val;
    }
  }
}

// ----------------------------------------------------------------------------
// dkdv kernel
// ----------------------------------------------------------------------------
template <int D, bool BF16, int DO>
__global__ __launch_bounds__(kThreads) void attention_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float2* __restrict__ stats,
    const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx, int64_t nnz_t, int S,
    int nb, int64_t lane_base, float scale_log2, float scale, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv) {
  using E = Elem<BF16>;
  using G = Geo<D>;
  constexpr int kStepsD = G::kStepsD, kTilesD = G::kTilesD, kTileBytes = G::kTileBytes;
  constexpr int kStatBytes = 1024;  // 4 slots of 256 B; slots 0, 1 hold the block's 64 (lse2, Delta)
  constexpr int kStageBytes = 2 * kTileBytes + kStatBytes;  // [Q tile | dO tile | stats]
  constexpr int kFillOps = G::kTileOps + 1;
  // Head dims of dK and dV written here: all D, or the half of D = 256 that
  // blockIdx.y selects (S and dP always contract over all D).
  static_assert(DO == D || 2 * DO == D, "a workgroup writes all the head dims or one of two halves");
  constexpr int kTilesO = DO / 32;
  const int d0 = DO < D ? (int)blockIdx.y * DO : 0;
  // The ring, reused after the loop for the merge of the two query halves.
  constexpr int kMergeBytes = 4 * 64 * (kTilesO * 16 + 4) * 4;  // 2 accumulators x half the groups
  constexpr int kRingBytes = 2 * kStageBytes > kMergeBytes ? 2 * kStageBytes : kMergeBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = w & 1;   // key half owned
  const int qh = w >> 1;  // query half of every visited block
  const int l = tid & 63, h = l >> 5, n = l & 31, g = l >> 4, gi = l & 15;

  int64_t lane;
  int j;
  grid_position(nb, lane_base, lane, j);  // lowest key blocks (longest columns) first
  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* qg = q + lane_off;
  const uint16_t* dog = dout + lane_off;
  [[maybe_unused]] const float2* sg = stats + lane * (int64_t)S;

  // Stationary operands of key row krow: K^T and V^T as B operands.
  const int krow = j * kBlock + 32 * kh + n;
  const int krow_c = krow < S ? krow : S - 1;
  const int64_t row_off = lane_off + (int64_t)krow_c * D + 8 * h;
  u32x4 kop[kStepsD], vop[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    kop[c] = *(const u32x4*)(k + row_off + 16 * c);
    vop[c] = *(const u32x4*)(v + row_off + 16 * c);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    asm volatile("" : "+v"(kop[c]));
    asm volatile("" : "+v"(vop[c]));
  }

  uint32_t fill_off[G::kTileOps];
  fill_offsets<D>(fill_off, w, l);
  // Queue query block i: Q and dO tiles, and its rows' statistics (wave w copies
  // the 256 bytes (w & 1) into slot w; rows past S read as zero).
  auto fill = [&](int i, uint8_t* stage) {
    const int rows = S - i * kBlock < kBlock ? S - i * kBlock : kBlock;
    copy_block_to_lds<G::kTileOps, G::kTileOps / 2, kWaves>(qg + (int64_t)i * kBlock * D,
                                                           dog + (int64_t)i * kBlock * D,
                                                           rows * G::kRowBytes, fill_off, stage, w);
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(sg + (int64_t)i * kBlock), 0, rows * 8, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(stage + 2 * kTileBytes + 256 * w), 4,
        (uint32_t)(256 * (w & 1) + 4 * l), 0, 0, 0);
#endif
  };

  ListWalker walk;
  walk.init(col_ptr, row_idx, nnz_t, j, j, nb - 1, l);

  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)&ring[0];
  uint32_t a_addr[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) a_addr[c] = row_read_addr<D>(base, qh, n, h, c);
  uint32_t t_addr[kTilesO][2];
#pragma unroll
  for (int dt = 0; dt < kTilesO; ++dt) tr_read_addrs<D>(t_addr[dt], base, qh, g, gi, d0 / 32 + dt);
  // Statistics of the query rows of this lane's result registers: register r
  // holds query row 32qh + 16 (r >> 3) + 8h + (r & 7).
  const uint32_t st_addr = base + 2 * kTileBytes + 8 * (32 * qh + 8 * h);

  f32x16 adk[kTilesO], adv[kTilesO];
#pragma unroll
  for (int dt = 0; dt < kTilesO; ++dt) {
    adk[dt] = f32x16{};
    adv[dt] = f32x16{};
  }

  auto compute = [&](int i, auto T_c) {
    // Stage offset: in the reads' 16-bit offset field when it fits, else (D = 256,
    // second stage past 64 KB) added to the lane addresses.
    constexpr int kStageAll = decltype(T_c)::value * kStageBytes;
    constexpr int kOff = kStageAll + kTileBytes + 16 * G::kRowBytes < 65536 ? kStageAll : 0;
    constexpr uint32_t kReg = (uint32_t)(kStageAll - kOff);
    // Operand reads in flight at once: all of them, or four steps at D = 256.
    constexpr int kChunk = kStepsD > 8 ? 4 : kStepsD;
    if (i == j && qh < kh) return;  // queries of this half all before the keys
    u32x4 st[8];
    // S = Q . K^T and dP = dO . V^T: MFMA row m holds query 32qh + pi(m), column n key 32kh + n.
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c0 = 0; c0 < kStepsD; c0 += kChunk) {
      u32x4 qa[kChunk], da[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        qa[c] = lds_read_b128<kOff>(a_addr[c0 + c] + kReg);
        da[c] = lds_read_b128<kOff + kTileBytes>(a_addr[c0 + c] + kReg);
      }
      if (c0 == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st[e] = lds_read_b128<kOff>(st_addr + kReg + 16 * e);
          st[4 + e] = lds_read_b128<kOff + 128>(st_addr + kReg + 16 * e);
        }
      }
      lds_wait_all(qa);
      lds_wait_all(da);
      if (c0 == 0) lds_wait_all(st);
#pragma unroll
      for (int c = 0; c < kChunk; ++c) s = E::mfma(qa[c], kop[c0 + c], s);
#pragma unroll
      for (int c = 0; c < kChunk; ++c) dp = E::mfma(da[c], vop[c0 + c], dp);
    }
    u32x2 qt[kTilesO * 4], dt_[kTilesO * 4];
#pragma unroll
    for (int dt = 0; dt < kTilesO; ++dt) {
      const uint32_t ta[2] = {t_addr[dt][0] + kReg, t_addr[dt][1] + kReg};
      tr_reads<kOff, G::kRowBytes>(&qt[dt * 4], ta);
      tr_reads<kOff + kTileBytes, G::kRowBytes>(&dt_[dt * 4], ta);
    }
    if (i == j && qh == kh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qpos = 16 * (r >> 3) + 8 * h + (r & 7);
        if (qpos < n) s[r] = -__builtin_inff();
      }
    }
    u32x4 pp[2], pd[2];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 8 * gg + 2 * x;
        const u32x4 sv = st[4 * gg + x];  // rows r, r + 1: (lse2, Delta) pairs
        const float l0 = __uint_as_float(sv[0]), d0 = __uint_as_float(sv[1]);
        const float l1 = __uint_as_float(sv[2]), d1 = __uint_as_float(sv[3]);
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -l0));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], scale_log2, -l1));
        pp[gg][x] = E::pack(p0, p1);
        pd[gg][x] = E::pack(p0 * (dp[r] - d0), p1 * (dp[r + 1] - d1));
      }
    lds_wait_all(qt);
    lds_wait_all(dt_);
#pragma unroll
    for (int dt = 0; dt < kTilesO; ++dt)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        adv[dt] = E::mfma(tr_operand(&dt_[dt * 4], gg), pp[gg], adv[dt]);
        adk[dt] = E::mfma(tr_operand(&qt[dt * 4], gg), pd[gg], adk[dt]);
      }
  };

  int blk[2];
  blk[0] = walk.next(-1);
  blk[1] = blk[0] >= 0 ? walk.next(blk[0]) : -1;
  if (blk[0] >= 0) {
    fill(blk[0], ring);
    if (blk[1] >= 0) fill(blk[1], ring + kStageBytes);
    bool pre = blk[1] >= 0;
    int last = pre ? blk[1] : blk[0];
    bool done = false;
    auto step = [&](auto T_c) {
      constexpr int t = decltype(T_c)::value;
      constexpr int refill = t ^ 1;
      if (pre)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(kFillOps));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      ring_barrier();
      if (!pre) {
        const int in = last >= 0 ? walk.next(last) : -1;
        blk[refill] = in;
        last = in;
        if (in >= 0) fill(in, ring + refill * kStageBytes);
      }
      pre = false;
      compute(blk[t], T_c);
      done = blk[refill] < 0;
    };
    while (!done) {
      step(std::integral_constant<int, 0>{});
      if (!done) step(std::integral_constant<int, 1>{});
    }
    __syncthreads();
  }

  // Sum the two query halves: wave qh keeps head-dim tiles [qh, qh + 1) *
  // kTilesO / 2 of dK and dV and hands the others to its partner.
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  // Register groups of 4 head dims, kTilesO * 4 per accumulator; wave qh keeps
  // groups [qh, qh + 1) * kGroups / 2 of dK and dV and sends the others.
  constexpr int kGroups = kTilesO * 4;
  constexpr int kHalfGroups = kGroups / 2;
  constexpr int kSendStride = 2 * kHalfGroups * 4 + 4;
  static_assert(4 * 64 * kSendStride * 4 <= kRingBytes, "merge area exceeds the ring");
  float* const xbase = (float*)&ring[0];
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  auto merge = [&](auto QHc) {
    constexpr int QH = decltype(QHc)::value;
    constexpr int kSendBase = (1 - QH) * kHalfGroups;
    constexpr int kKeepBase = QH * kHalfGroups;
    float* send = xbase + ((kh * 2 + QH) * 64 + l) * kSendStride;
#pragma unroll
    for (int u = 0; u < kHalfGroups; ++u) {
      const int gq = kSendBase + u;
      *(f32x4*)(send + 4 * u) = f32x4{adk[gq / 4][4 * (gq % 4)], adk[gq / 4][4 * (gq % 4) + 1],
                                      adk[gq / 4][4 * (gq % 4) + 2], adk[gq / 4][4 * (gq % 4) + 3]};
      *(f32x4*)(send + 4 * (kHalfGroups + u)) =
          f32x4{adv[gq / 4][4 * (gq % 4)], adv[gq / 4][4 * (gq % 4) + 1], adv[gq / 4][4 * (gq % 4) + 2],
                adv[gq / 4][4 * (gq % 4) + 3]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    ring_barrier();
    const float* recv = xbase + ((kh * 2 + (1 - QH)) * 64 + l) * kSendStride;
    if (krow < S) {
      uint16_t* krow_dk = dk + lane_off + (int64_t)krow * D;
      uint16_t* krow_dv = dv + lane_off + (int64_t)krow * D;
#pragma unroll
      for (int u = 0; u < kHalfGroups; ++u) {
        const int gq = kKeepBase + u;
        const f32x4 yk = *(const f32x4*)(recv + 4 * u);
        const f32x4 yv = *(const f32x4*)(recv + 4 * (kHalfGroups + u));
        float xk[4], xv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xk[e] = (adk[gq / 4][4 * (gq % 4) + e] + yk[e]) * scale;
          xv[e] = adv[gq / 4][4 * (gq % 4) + e] + yv[e];
        }
        const int col = d0 + 32 * (gq / 4) + 8 * (gq % 4) + 4 * h;
        *(u32x2*)(krow_dk + col) = u32x2{E::pack(xk[0], xk[1]), E::pack(xk[2], xk[3])};
        *(u32x2*)(krow_dv + col) = u32x2{E::pack(xv[0], xv[1]), E::pack(xv[2], xv[3])};
      }
    }
  };
  if (qh == 0)
    merge(std::integral_constant<int, 0>{});
  else
    merge(std::integral_constant<int, 1>{});
}

// ----------------------------------------------------------------------------
// dkdv kernel, two key blocks per workgroup
// ----------------------------------------------------------------------------
// Columns of a causal schedule are unlike their neighbours (a column lists
// either most later rows, when its block is one every row picks, or only the
// rows of its local window), but columns of similar length list mostly the
// same rows.  col_order_kernel ranks the columns by their number of entries,
// longest first (ties by index), and the dkdv kernel's two-block form pairs
// ranks 2p and 2p+1: wave w owns key half w & 1 of column order[2p + (w >> 1)]
// and takes both query halves of every block its column lists, one after the
// other, into one dK^T and one dV^T, so no merge of query halves is needed.
// The workgroup walks the union of the two columns; each union block's Q, dO
// and statistics are copied once.
//
// order: nb int32, a permutation of 0..nb-1.  One thread per column: its rank is
// the number of columns with more entries, plus those with as many and a lower
// index.  Entry counts are taken from col_ptr clamped to [0, nnz_t], as the
// walkers read it.
constexpr int kOrderChunk = 2048;  // column counts staged in LDS at a time
__global__ __launch_bounds__(256) void col_order_kernel(const int32_t* __restrict__ col_ptr, int nb,
                                                        int64_t nnz_t, int32_t* __restrict__ order) {
  __shared__ int cnt[kOrderChunk];
  const int j = blockIdx.x * 256 + threadIdx.x;
  auto count = [&](int c) -> int {
    const int64_t p = min((int64_t)max(col_ptr[c], 0), nnz_t);
    const int64_t e = max(min((int64_t)col_ptr[c + 1], nnz_t), p);
    return (int)(e - p);
  };
  const int mine = j < nb ? count(j) : 0;
  int rank = 0;
  for (int c0 = 0; c0 < nb; c0 += kOrderChunk) {
    const int n = nb - c0 < kOrderChunk ? nb - c0 : kOrderChunk;
    __syncthreads();
    for (int c = threadIdx.x; c < n; c += 256) cnt[c] = count(c0 + c);
    __syncthreads();
    if (j < nb)
      for (int c = 0; c < n; ++c) {
        const int o = cnt[c];
        rank += (o > mine) | ((o == mine) & (c0 + c < j));
      }
  }
  if (j < nb) order[rank] = j;
}

// ncols: the column view's columns (nb, or ceil(S / 32) with SUB).  With SUB
// the workgroup at position pos takes 32-key columns 4 pos .. 4 pos + 3 (the
// 64-key blocks 2 pos and 2 pos + 1, no ranking), wave w column 4 pos + w, and
// walks the union of the 64-row query blocks they touch; a wave takes query
// half 2I + h of 64-row block I only when its column lists that 32-row block.
template <int D, bool BF16, bool SUB>
__global__ __launch_bounds__(kThreads) void attention_bwd_dkdv_duo_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float2* __restrict__ stats,
    const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx, int64_t nnz_t,
    const int32_t* __restrict__ order, int S, int nb, int ncols, int npairs, int64_t lane_base,
    float scale_log2, float scale, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  using E = Elem<BF16>;
  using G = Geo<D>;
  constexpr int kStepsD = G::kStepsD, kTilesD = G::kTilesD, kTileBytes = G::kTileBytes;
  constexpr int kStatBytes = 1024;  // 4 slots of 256 B; slots 0, 1 hold the block's 64 (lse2, Delta)
  constexpr int kStageBytes = 2 * kTileBytes + kStatBytes;  // [Q tile | dO tile | stats]
  constexpr int kFillOps = G::kTileOps + 1;
  constexpr int kHalfRowBytes = 32 * G::kRowBytes;  // query half 1: 32 rows further, same swizzle
  // Head dim 128 runs each half-step phase by phase (below): at one wave per
  // SIMD either way, that measured 4360 -> 4139 us for the backward at
  // [2,32,8192,128]; at head dim 64 the interleaved order is faster (203 against
  // 213 us at [4,16,4096,64]), even though the phased one fits three waves.
  constexpr bool kFewLive = D >= 128;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int csel = w >> 1;  // which column of the pair
  const int kh = w & 1;     // key half owned
  const int l = tid & 63, h = l >> 5, n = l & 31, g = l >> 4, gi = l & 15;

  int64_t lane;
  int pos;
  grid_position(npairs, lane_base, lane, pos);  // longest columns first
  const int slot = 2 * pos + csel;
  // -1: the pair's second column is past the end
  const int my_j = slot < nb ? (SUB ? slot : order[slot]) : -1;
  const int my_k32 = 2 * my_j + kh;  // this wave's 32-key block
  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* qg = q + lane_off;
  const uint16_t* dog = dout + lane_off;
  [[maybe_unused]] const float2* sg = stats + lane * (int64_t)S;

  // Stationary operands of key row krow: K^T and V^T as B operands.
  const int krow = (my_j >= 0 ? my_j : 0) * kBlock + 32 * kh + n;
  const int krow_c = krow < S ? krow : S - 1;
  const int64_t row_off = lane_off + (int64_t)krow_c * D + 8 * h;
  u32x4 kop[kStepsD], vop[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    kop[c] = *(const u32x4*)(k + row_off + 16 * c);
    vop[c] = *(const u32x4*)(v + row_off + 16 * c);
  }
  // The columns' walkers (the pair's two columns, or with SUB the four 32-key
  // ones, wave w's being walker w): the union of their rows in ascending order.
  constexpr int kWalk = SUB ? 4 : 2;
  ListWalker walk[kWalk];
  int head[kWalk];
#pragma unroll
  for (int r = 0; r < kWalk; ++r) {
    int jr;
    if constexpr (SUB) {
      jr = 4 * pos + r < ncols ? 4 * pos + r : -1;
    } else {
      const int sr = 2 * pos + r;
      jr = sr < nb ? order[sr] : -1;
    }
    if (jr >= 0)
      walk[r].init(col_ptr, row_idx, nnz_t, jr, jr, ncols - 1, l);
    else
      walk[r].clear(row_idx, l);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    asm volatile("" : "+v"(kop[c]));
    asm volatile("" : "+v"(vop[c]));
  }
#pragma unroll
  for (int r = 0; r < kWalk; ++r) head[r] = walk[r].next(-1);
  // Next 64-row query block of the union (-1: none); `mine` gets bit h set when
  // this wave computes query half h of it.
  auto next_block = [&](int& mine) -> int {
    int hmin = INT_MAX;
#pragma unroll
    for (int r = 0; r < kWalk; ++r)
      if (head[r] >= 0) hmin = min(hmin, head[r]);
    mine = 0;
    if (hmin == INT_MAX) return -1;
    const int i = SUB ? hmin >> 1 : hmin;
#pragma unroll
    for (int r = 0; r < kWalk; ++r) {
      if constexpr (SUB) {
#pragma unroll
        for (int e = 0; e < 2; ++e)  // at most the two 32-row blocks of i, ascending
          if (head[r] >= 0 && (head[r] >> 1) == i) {
            if (r == w) mine |= 1 << (head[r] & 1);
            head[r] = walk[r].next(head[r]);
          }
      } else if (head[r] == i) {
        if (r == csel) mine = 3;
        head[r] = walk[r].next(i);
      }
    }
    return i;
  };

  uint32_t fill_off[G::kTileOps];
  fill_offsets<D>(fill_off, w, l);
  // Queue query block i: Q and dO tiles, and its rows' statistics (wave w copies
  // the 256 bytes (w & 1) into slot w; rows past S read as zero).
  auto fill = [&](int i, uint8_t* stage) {
    const int rows = S - i * kBlock < kBlock ? S - i * kBlock : kBlock;
    copy_block_to_lds<G::kTileOps, G::kTileOps / 2, kWaves>(qg + (int64_t)i * kBlock * D,
                                                           dog + (int64_t)i * kBlock * D,
                                                           rows * G::kRowBytes, fill_off, stage, w);
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(sg + (int64_t)i * kBlock), 0, rows * 8, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(stage + 2 * kTileBytes + 256 * w), 4,
        (uint32_t)(256 * (w & 1) + 4 * l), 0, 0, 0);
#endif
  };

  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)&ring[0];
  uint32_t a_addr[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) a_addr[c] = row_read_addr<D>(base, 0, n, h, c);
  uint32_t t_addr[kTilesD][2];
#pragma unroll
  for (int dt = 0; dt < kTilesD; ++dt) tr_read_addrs<D>(t_addr[dt], base, 0, g, gi, dt);
  // Statistics of the query rows of this lane's result registers: register r
  // holds query row 32qh + 16 (r >> 3) + 8h + (r & 7).
  const uint32_t st_addr = base + 2 * kTileBytes + 8 * (8 * h);

  f32x16 adk[kTilesD], adv[kTilesD];
#pragma unroll
  for (int dt = 0; dt < kTilesD; ++dt) {
    adk[dt] = f32x16{};
    adv[dt] = f32x16{};
  }

  // Query half QH of block i, held by ring stage T (both compile-time).
  auto compute_half = [&](int i, auto T_c, auto QH_c) {
    constexpr int QH = decltype(QH_c)::value;
    constexpr int kOff = decltype(T_c)::value * kStageBytes + QH * kHalfRowBytes;
    constexpr int kStOff = decltype(T_c)::value * kStageBytes + QH * 256;
    // 32-row query block 2i + QH against this wave's 32-key block: earlier ones
    // are fully masked (the acceptance rule never lists them under SUB).
    if (2 * i + QH < my_k32) return;
    if constexpr (kFewLive) {
      // Head dim 128: phase by phase, so that fewer values are live at once
      // (398 -> 308 registers): the Q and dO operands only until the S and dP
      // products are issued, the row statistics one register group at a time,
      // the transposed tiles one 32-dim tile at a time after the softmax.
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        u32x4 qa[kStepsD], da[kStepsD];
#pragma unroll
        for (int c = 0; c < kStepsD; ++c) {
          qa[c] = lds_read_b128<kOff>(a_addr[c]);
          da[c] = lds_read_b128<kOff + kTileBytes>(a_addr[c]);
        }
        lds_wait_all(qa);
        lds_wait_all(da);
#pragma unroll
        for (int c = 0; c < kStepsD; ++c) s = E::mfma(qa[c], kop[c], s);
#pragma unroll
        for (int c = 0; c < kStepsD; ++c) dp = E::mfma(da[c], vop[c], dp);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (2 * i + QH == my_k32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qpos = 16 * (r >> 3) + 8 * h + (r & 7);
          if (qpos < n) s[r] = -__builtin_inff();
        }
      }
      u32x4 pp[2], pd[2];
      auto softmax_group = [&](auto GG_c) {
        constexpr int gg = decltype(GG_c)::value;
        u32x4 st[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) st[e] = lds_read_b128<kStOff + 128 * gg>(st_addr + 16 * e);
        lds_wait_all(st);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 8 * gg + 2 * x;
          const u32x4 sv = st[x];  // rows r, r + 1: (lse2, Delta) pairs
          const float l0 = __uint_as_float(sv[0]), d0 = __uint_as_float(sv[1]);
          const float l1 = __uint_as_float(sv[2]), d1 = __uint_as_float(sv[3]);
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -l0));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], scale_log2, -l1));
          pp[gg][x] = E::pack(p0, p1);
          pd[gg][x] = E::pack(p0 * (dp[r] - d0), p1 * (dp[r + 1] - d1));
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      softmax_group(std::integral_constant<int, 0>{});
      softmax_group(std::integral_constant<int, 1>{});
#pragma unroll
      for (int dt = 0; dt < kTilesD; ++dt) {
        u32x2 qt[4], dt_[4];
        tr_reads<kOff, G::kRowBytes>(qt, t_addr[dt]);
        tr_reads<kOff + kTileBytes, G::kRowBytes>(dt_, t_addr[dt]);
        lds_wait_all(qt);
        lds_wait_all(dt_);
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          adv[dt] = E::mfma(tr_operand(dt_, gg), pp[gg], adv[dt]);
          adk[dt] = E::mfma(tr_operand(qt, gg), pd[gg], adk[dt]);
        }
      }
    } else {
      u32x4 qa[kStepsD], da[kStepsD], st[8];
#pragma unroll
      for (int c = 0; c < kStepsD; ++c) {
        qa[c] = lds_read_b128<kOff>(a_addr[c]);
        da[c] = lds_read_b128<kOff + kTileBytes>(a_addr[c]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st[e] = lds_read_b128<kStOff>(st_addr + 16 * e);
        st[4 + e] = lds_read_b128<kStOff + 128>(st_addr + 16 * e);
      }
      lds_wait_all(qa);
      lds_wait_all(da);
      lds_wait_all(st);
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < kStepsD; ++c) s = E::mfma(qa[c], kop[c], s);
#pragma unroll
      for (int c = 0; c < kStepsD; ++c) dp = E::mfma(da[c], vop[c], dp);
      u32x2 qt[kTilesD * 4], dt_[kTilesD * 4];
#pragma unroll
      for (int dt = 0; dt < kTilesD; ++dt) {
        tr_reads<kOff, G::kRowBytes>(&qt[dt * 4], t_addr[dt]);
        tr_reads<kOff + kTileBytes, G::kRowBytes>(&dt_[dt * 4], t_addr[dt]);
      }
      if (2 * i + QH == my_k32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qpos = 16 * (r >> 3) + 8 * h + (r & 7);
          if (qpos < n) s[r] = -__builtin_inff();
        }
      }
      u32x4 pp[2], pd[2];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 8 * gg + 2 * x;
          const u32x4 sv = st[4 * gg + x];  // rows r, r + 1: (lse2, Delta) pairs
          const float l0 = __uint_as_float(sv[0]), d0 = __uint_as_float(sv[1]);
          const float l1 = __uint_as_float(sv[2]), d1 = __uint_as_float(sv[3]);
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -l0));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], scale_log2, -l1));
          pp[gg][x] = E::pack(p0, p1);
          pd[gg][x] = E::pack(p0 * (dp[r] - d0), p1 * (dp[r + 1] - d1));
        }
      lds_wait_all(qt);
      lds_wait_all(dt_);
#pragma unroll
      for (int dt = 0; dt < kTilesD; ++dt)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          adv[dt] = E::mfma(tr_operand(&dt_[dt * 4], gg), pp[gg], adv[dt]);
          adk[dt] = E::mfma(tr_operand(&qt[dt * 4], gg), pd[gg], adk[dt]);
        }
    }
  };

  // Ring over the union, as in the one-column kernel.
  int blk[2];
  int mine[2] = {0, 0};
  blk[0] = next_block(mine[0]);
  blk[1] = blk[0] >= 0 ? next_block(mine[1]) : -1;
  if (blk[0] >= 0) {
    fill(blk[0], ring);
    if (blk[1] >= 0) fill(blk[1], ring + kStageBytes);
    bool pre = blk[1] >= 0;
    bool done = false;
    auto step = [&](auto T_c) {
      constexpr int t = decltype(T_c)::value;
      constexpr int refill = t ^ 1;
      if (pre)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(kFillOps));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      ring_barrier();
      if (!pre) {
        blk[refill] = next_block(mine[refill]);
        if (blk[refill] >= 0) fill(blk[refill], ring + refill * kStageBytes);
      }
      pre = false;
      if (mine[t] & 1) compute_half(blk[t], T_c, std::integral_constant<int, 0>{});
      if (mine[t] & 2) compute_half(blk[t], T_c, std::integral_constant<int, 1>{});
      done = blk[refill] < 0;
    };
    while (!done) {
      step(std::integral_constant<int, 0>{});
      if (!done) step(std::integral_constant<int, 1>{});
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));

  // The wave holds the whole dK^T and dV^T of its 32 key rows: scale dK, pack, store.
  if (my_j >= 0 && krow < S) {
    uint16_t* krow_dk = dk + lane_off + (int64_t)krow * D;
    uint16_t* krow_dv = dv + lane_off + (int64_t)krow * D;
#pragma unroll
    for (int gq = 0; gq < kTilesD * 4; ++gq) {
      float xk[4], xv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xk[e] = adk[gq / 4][4 * (gq % 4) + e] * scale;
        xv[e] = adv[gq / 4][4 * (gq % 4) + e];
      }
      const int col = 32 * (gq / 4) + 8 * (gq % 4) + 4 * h;
      *(u32x2*)(krow_dk + col) = u32x2{E::pack(xk[0], xk[1]), E::pack(xk[2], xk[3])};
      *(u32x2*)(krow_dv + col) = u32x2{E::pack(xv[0], xv[1]), E::pack(xv[2], xv[3])};
    }
  }
}

constexpr int64_t kDqDuoMinPairs = 2048;

template <int D, bool BF16>
hipError_t launch_bwd_typed(const BwdArgs& a, hipStream_t stream) {
  const int64_t nb = (a.S + kBlock - 1) / kBlock;
  const int64_t max_wg = (int64_t(1) << 31) / kThreads;
  const int64_t lanes_per_launch = max_wg / nb > 0 ? max_wg / nb : 1;
  const int64_t npairs = (nb + 1) / 2;
  // Schedules over 32-row blocks always take the two-block kernels, whose four
  // waves are the four 32-row blocks of a pair of 64-row blocks.
  const bool sub = a.block == 32;
  const int64_t nrows = sub ? (a.S + 31) / 32 : nb;
  // At D = 256 the dQ, dK and dV accumulators of all the head dims do not fit a
  // wave's registers: the one-block kernels run twice as wide a grid, blockIdx.y
  // selecting the half of the head dims each workgroup writes, and recompute S
  // and dP (over all D) in both halves.
  constexpr bool kSplit = D > 128;
  constexpr int kDO = kSplit ? D / 2 : D;
  const unsigned halves = kSplit ? 2u : 1u;
  for (int64_t l0 = 0; l0 < a.lanes; l0 += lanes_per_launch) {
    const int64_t nl = a.lanes - l0 < lanes_per_launch ? a.lanes - l0 : lanes_per_launch;
    // Two query blocks per workgroup once the halved grid still fills every CU
    // (the forward's rule: 2048 (lane, query block) pairs).
    bool duo = false;
    if constexpr (!kSplit) {
      if (sub || nl * nb >= kDqDuoMinPairs) {
        duo = true;
        auto kern = sub ? attention_bwd_dq_duo_kernel<D, BF16, true> : attention_bwd_dq_duo_kernel<D, BF16, false>;
        hipLaunchKernelGGL(kern, dim3((unsigned)(nl * npairs)), dim3(kThreads), 0, stream, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.out,
                           (const uint16_t*)a.dout, a.lse, a.row_ptr, a.col_idx, a.nnz, (int)a.S, (int)nb,
                           (int)nrows, (int)npairs, l0, a.scale_log2, a.scale, (float2*)a.stats,
                           (uint16_t*)a.dq);
      }
    }
    if (!duo) {
      hipLaunchKernelGGL((attention_bwd_dq_kernel<D, BF16, kDO>), dim3((unsigned)(nl * nb), halves), dim3(kThreads), 0,
                         stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                         (const uint16_t*)a.out, (const uint16_t*)a.dout, a.lse, a.row_ptr, a.col_idx,
                         a.nnz, (int)a.S, (int)nb, l0, a.scale_log2, a.scale, (float2*)a.stats,
                         (uint16_t*)a.dq);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // Two key blocks per workgroup under the same rule, paired by entry count, up
  // to 4096 key blocks (the ranking compares every pair of columns: at most 16.8 M
  // comparisons; longer sequences keep one column per workgroup).  With 32-row
  // blocks the workgroup takes the four 32-key columns of two adjacent 64-key
  // blocks, unranked.
  constexpr int64_t kDkdvDuoMaxBlocks = 4096;
  const bool dkdv_duo = !kSplit && (sub || (a.lanes * nb >= kDqDuoMinPairs && nb <= kDkdvDuoMaxBlocks));
  if (dkdv_duo && !sub) {
    hipLaunchKernelGGL(col_order_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream, a.col_ptr,
                       (int)nb, a.nnz_t, a.col_order);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  for (int64_t l0 = 0; l0 < a.lanes; l0 += lanes_per_launch) {
    const int64_t nl = a.lanes - l0 < lanes_per_launch ? a.lanes - l0 : lanes_per_launch;
    bool duo = false;
    if constexpr (!kSplit) {
      if (dkdv_duo) {
        duo = true;
        auto kern = sub ? attention_bwd_dkdv_duo_kernel<D, BF16, true> : attention_bwd_dkdv_duo_kernel<D, BF16, false>;
        hipLaunchKernelGGL(kern, dim3((unsigned)(nl * npairs)), dim3(kThreads), 0, stream, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                           (const float2*)a.stats, a.col_ptr, a.row_idx, a.nnz_t, (const int32_t*)a.col_order,
                           (int)a.S, (int)nb, (int)nrows, (int)npairs, l0, a.scale_log2, a.scale,
                           (uint16_t*)a.dk, (uint16_t*)a.dv);
      }
    }
    if (!duo) {
      hipLaunchKernelGGL((attention_bwd_dkdv_kernel<D, BF16, kDO>), dim3((unsigned)(nl * nb), halves), dim3(kThreads), 0,
                         stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                         (const uint16_t*)a.dout, (const float2*)a.stats, a.col_ptr, a.row_idx, a.nnz_t,
                         (int)a.S, (int)nb, l0, a.scale_log2, a.scale, (uint16_t*)a.dk, (uint16_t*)a.dv);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attention_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.D == 64) return a.bf16 ? launch_bwd_typed<64, true>(a, stream) : launch_bwd_typed<64, false>(a, stream);
  if (a.D == 128) return a.bf16 ? launch_bwd_typed<128, true>(a, stream) : launch_bwd_typed<128, false>(a, stream);
  if (a.D == 32) return a.bf16 ? launch_bwd_typed<32, true>(a, stream) : launch_bwd_typed<32, false>(a, stream);
  if (a.D == 256 && a.block == 64)
    return a.bf16 ? launch_bwd_typed<256, true>(a, stream) : launch_bwd_typed<256, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace tsa
