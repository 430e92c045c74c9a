// Scheduled block-sparse causal attention forward for gfx950 (CDNA4), with two
// adjacent query blocks per workgroup sharing every K/V tile.
//
// Same operation as attention_fwd.hip ("Add topology-derived sparse attention
// kernel", triton-lang/kernels PR 22, Summary: each 64-row query block visits
// only the key blocks its CSR row lists; one schedule is shared by every
// batch/head lane; the output keeps the input dtype; running max and
// denominator per query row, rescaled by exp(m_prev - m_new) as in the mirror
// page's Rust-port commit note).
//
// Work decomposition
//   One workgroup = one lane and the query-block pair (2g, 2g+1): 512 threads,
//   8 waves.  Waves 4r .. 4r+3 own query block 2g+r exactly as the one-block
//   kernel's four waves own theirs (query half x key half, merged at the end).
//   The workgroup walks the union of the two CSR rows in ascending order: each
//   block of the union is copied into LDS once, and the waves of a row compute
//   it only when their row lists it.  Adjacent rows of a causal schedule share
//   most of their blocks (the sink, the top-k set, all but one of the local
//   window), so each copied tile serves about twice the queries, the per-
//   workgroup start-up is paid once per 128 queries, and the grid is half as
//   large.  Every wave sees exactly its own row's blocks in the same order as in
//   the one-block kernel, so the results are bit-identical to it.
//
//   Grid: x = lane (remapped so that each of the 8 XCDs holds a contiguous range
//   of lanes when the lane count is a multiple of 8; workgroup x + y * lanes
//   runs on XCD x % 8), y = pair position, last pairs (longest rows) first.
//
// Data movement: a ring of kStages [K tile | V tile] stages filled by
// global->LDS buffer loads (no registers in between); the copy of block t +
// kStages - 1 of the union is in flight while block t is computed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <type_traits>

#include "kernels.h"
#include "mfma_tile.h"

namespace tsa {
namespace {

using namespace tile;

constexpr int kRows = 2;                 // query blocks per workgroup
constexpr int kPairWaves = 4 * kRows;    // 4 waves per query block
constexpr int kPairThreads = 64 * kPairWaves;

// Cursor over the accepted entries of one CSR row (wave-uniform state, plus one
// per-lane register holding a window of 64 column indices).  An entry is
// accepted when it lies in 0..i and exceeds the previous accepted entry: the
// rule of the one-block kernel.
struct RowCursor {
  int i;      // query block, or -1 when the pair's second block is past the end
  int p, end; // next entry, end of the row (clamped to the readable entries)
  int win;    // first entry held in `cols`
  int cols;   // lane l: entry win + l (or -1)
  int last;   // last accepted block
  int head;   // next accepted block (INT_MAX: none left)

  __device__ __forceinline__ void start(const int32_t* __restrict__ row_ptr,
                                        const int32_t* __restrict__ col_idx, int64_t nnz, int row,
                                        int nb, int l) {
    i = row < nb ? row : -1;
    if (i >= 0) {
      p = (int)min((int64_t)max(row_ptr[i], 0), nnz);
      end = (int)max(min((int64_t)row_ptr[i + 1], nnz), (int64_t)p);
    } else {
      p = end = 0;
    }
    win = p;
    cols = (p + l < end) ? col_idx[p + l] : -1;
    last = -1;
    head = INT_MAX;
  }
  // Moves `head` to the next accepted entry.  A window reload waits for every
  // outstanding vector load of the wave (only rows of more than 64 entries).
  __device__ __forceinline__ void advance(const int32_t* __restrict__ col_idx, int l) {
    while (p < end) {
      if (p - win >= 64) {
        win = p;
        cols = (p + l < end) ? col_idx[p + l] : -1;
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      }
      const int c = __builtin_amdgcn_readlane(cols, p - win);
      ++p;
      if (c > last && c <= i) {
        head = c;
        return;
      }
    }
    head = INT_MAX;
  }
};

template <int D>
struct PairStages {
  // 16 KB stages at head dim 64 (two workgroups of 48 KB per CU), 32 KB at 128.
  static constexpr int value = D <= 64 ? 3 : 2;
};

template <int D, bool BF16>
__global__ __launch_bounds__(kPairThreads) void attention_fwd_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t nnz,
    int S, int nb, int64_t lane_base, float scale_log2, float inv_scale_log2) {
  using E = Elem<BF16>;
  constexpr int kStepsD = D / 16;
  constexpr int kTilesD = D / 32;
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlock * kRowBytes;
  constexpr int kStageBytes = 2 * kTileBytes;
  constexpr int kChunksPerRow = D / 8;
  constexpr int kWaves = kPairWaves;
  constexpr int kFillOps = kStageBytes / 1024 / kWaves;  // 1 KB fill ops per wave per stage
  constexpr float kRescaleSlack = 8.0f;
  constexpr int kStages = PairStages<D>::value;
  static_assert(kTilesD >= 2, "the merge below splits whole O tiles between the key halves");
  static_assert((kTileBytes / 1024) % kWaves == 0 && kFillOps % 2 == 0, "fill ops split K | V");
  // Merge area of one query block: 4 waves x 64 lanes x kSendStride floats, then
  // [query half][key half][m, l][lane].
  constexpr int kHalfTiles = kTilesD / 2;
  constexpr int kSendFloats = kHalfTiles * 16;
  constexpr int kSendStride = kSendFloats + 4;
  constexpr int kMergeFloats = 4 * 64 * kSendStride + 2 * 2 * 2 * 64;
  constexpr int kRingBytes = kStages * kStageBytes;
  constexpr int kMergeBytes = kRows * kMergeFloats * 4;
  constexpr int kLdsBytes = kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave (uniform)
  const int rsel = w >> 2;      // which query block of the pair
  const int qh = w & 1;         // query half of that block
  const int kh = (w >> 1) & 1;  // key half of every visited block
  const int l = tid & 63;
  const int h = l >> 5;
  const int n = l & 31;
  const int g = l >> 4;
  const int gi = l & 15;

  // Lane and pair position (see the header comment): no division.
  const uint32_t X = gridDim.x, x = blockIdx.x;
  int64_t lane;
  if (X % 8u == 0u)
    lane = lane_base + (int64_t)((x % 8u) * (X / 8u) + x / 8u);
  else
    lane = lane_base + (int64_t)x;
  const int npairs = (int)gridDim.y;
  const int pair = npairs - 1 - (int)blockIdx.y;
  const int my_i = kRows * pair + rsel;  // >= nb: this wave's block is past the end

  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* kg = k + lane_off;
  const uint16_t* vg = v + lane_off;

  // Column windows of both rows first, then the Q^T operands (lane: query row
  // qrow, dims 16c + 8h .. +7 for step c); the first wait below covers the
  // windows and lets the Q loads stay in flight.
  RowCursor rows[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) rows[r].start(row_ptr, col_idx, nnz, kRows * pair + r, nb, l);
  const int qrow = my_i * kBlock + 32 * qh + n;
  const int qrow_c = qrow < S ? qrow : S - 1;
  u32x4 qop[kStepsD];
  {
    const uint16_t* qp = q + lane_off + (int64_t)qrow_c * D + 8 * h;
    load_row_operands<kStepsD>(qop, qp);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(kStepsD));  // the windows (older than the Q loads)
#pragma unroll
  for (int r = 0; r < kRows; ++r) rows[r].advance(col_idx, l);

  // Next block of the union of the two rows (-1: none); `mine` tells whether
  // this wave's row lists it.
  auto next_block = [&](bool& mine) -> int {
    int j = INT_MAX;
#pragma unroll
    for (int r = 0; r < kRows; ++r) j = min(j, rows[r].head);
    if (j == INT_MAX) {
      mine = false;
      return -1;
    }
    mine = false;
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      if (rows[r].head == j) {
        if (r == rsel) mine = true;
        rows[r].last = j;
        rows[r].advance(col_idx, l);
      }
    return j;
  };

  static_assert((kTileBytes / 1024) % kWaves == 0, "whole rounds of 1 KB pieces per tile");
  uint32_t fill_off[kFillOps];
#pragma unroll
  for (int op = 0; op < kFillOps; ++op) {
    constexpr int kHalfOps = kFillOps / 2;
    const bool is_v = op >= kHalfOps;
    const int cc = ((is_v ? op - kHalfOps : op) * kWaves + w) * 64 + l;
    const int r = cc / kChunksPerRow, pc = cc % kChunksPerRow;
    const int key = is_v ? r : ((r & 32) | swap_bits23(r & 31));
    const int c = is_v ? (pc ^ v_swizzle<D>(r)) : (pc ^ k_swizzle<D>(r));
    fill_off[op] = (uint32_t)(key * kRowBytes + 16 * c);
  }
  auto fill = [&](int j, int t) {
    const int rows_j = S - j * kBlock < kBlock ? S - j * kBlock : kBlock;
    copy_block_to_lds<kFillOps, kTileBytes / 1024 / kWaves, kWaves>(
        kg + (int64_t)j * kBlock * D, vg + (int64_t)j * kBlock * D, rows_j * kRowBytes, fill_off,
        lds + t * kStageBytes, w);
  };

  f32x16 o[kTilesD];
#pragma unroll
  for (int dt = 0; dt < kTilesD; ++dt) o[dt] = f32x16{};
  float m_use = -__builtin_inff();
  float thr_raw = -__builtin_inff();
  float l_run = 0.0f;
  bool started = false;

  const uint32_t ring_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)&lds[0];
  uint32_t k_addr[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c)
    k_addr[c] = ring_base + (uint32_t)k_chunk_offset<D>(32 * kh + n, 2 * c + h);
  uint32_t v_addr[kTilesD];
  {
    const int r0 = 32 * kh + 8 * (g >> 1) + (gi >> 2);
    const uint32_t lane_addr = ring_base + (uint32_t)(kTileBytes + r0 * kRowBytes + 8 * (gi & 1));
    const int sw = v_swizzle<D>(r0);
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) {
      const int dchunk = 4 * dt + 2 * (g & 1) + ((gi & 3) >> 1);
      v_addr[dt] = lane_addr + 16u * (uint32_t)(dchunk ^ sw);
    }
  }

  const int diag_lim = n - 8 * h;
  // One visited block of this wave's row, held by ring stage T (compile-time).
  auto compute = [&](int j, auto T_c) {
    constexpr int kStageOff = decltype(T_c)::value * kStageBytes;
    static_assert(kStageOff + kStageBytes <= 65536, "stage offsets fit the LDS offset field");
    if (j == my_i && kh > qh) return;  // diagonal block: this key half is fully masked
    u32x4 ka[kStepsD];
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) ka[c] = lds_read_b128<kStageOff>(k_addr[c]);
    lds_wait_all(ka);
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) s = E::mfma(ka[c], qop[c], s);
    if (j == my_i && kh == qh) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (16 * (r >> 3) + (r & 7) > diag_lim) s[r] = -__builtin_inff();
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    if (__ballot(mx > thr_raw)) {
      const float mp = max_with_other_half(mx) * scale_log2;
      const bool grow = mp > m_use + kRescaleSlack;
      const float m_new = grow ? mp : m_use;
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      m_use = m_new;
      const float thr = (m_new + kRescaleSlack) * inv_scale_log2;
      thr_raw = thr - __builtin_fabsf(thr) * 0x1p-20f;
      if (started) {
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kTilesD; ++dt) o[dt] *= alpha;
      }
      started = true;
    }
    u32x2 va[kTilesD * 4];
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) {
      va[dt * 4 + 0] = lds_read_tr16<kStageOff>(v_addr[dt]);
      va[dt * 4 + 1] = lds_read_tr16<kStageOff + 4 * kRowBytes>(v_addr[dt]);
      va[dt * 4 + 2] = lds_read_tr16<kStageOff + 16 * kRowBytes>(v_addr[dt]);
      va[dt * 4 + 3] = lds_read_tr16<kStageOff + 20 * kRowBytes>(v_addr[dt]);
    }
    u32x4 pb[2];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * gg + 2 * xx], scale_log2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * gg + 2 * xx + 1], scale_log2, -m_use));
        pb[gg][xx] = E::pack(p0, p1);
      }
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) l_run = E::add_pair(pb[gg][xx], l_run);
    lds_wait_all(va);
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const u32x2 lo = va[dt * 4 + 2 * gg], hi = va[dt * 4 + 2 * gg + 1];
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        o[dt] = E::mfma(a, pb[gg], o[dt]);
      }
  };

  // Ring over the union.  blk[t]: block held by stage t (-1: none), mine[t]:
  // whether this wave's row lists it.  The first kStages - 1 blocks are queued
  // here; at step t the wave waits for stage t's copies (the copies of the
  // stages queued after it may stay in flight), passes the barrier, queues the
  // next union block into the stage computed one step earlier, and computes.
  int blk[kStages];
  bool mine[kStages];
#pragma unroll
  for (int t = 0; t < kStages; ++t) {
    blk[t] = -1;
    mine[t] = false;
  }
#pragma unroll
  for (int t = 0; t + 1 < kStages; ++t) {
    blk[t] = next_block(mine[t]);
    if (blk[t] >= 0) fill(blk[t], t);
  }
  bool done = blk[0] < 0;
  auto step = [&](auto T_c) {
    constexpr int t = decltype(T_c)::value;
    constexpr int refill = (t + kStages - 1) % kStages;
    if (blk[t] < 0) {
      done = true;
      return;
    }
    // stages queued after stage t that hold a block (they form a prefix)
    int later = 0;
#pragma unroll
    for (int d = 1; d + 1 < kStages; ++d) later += blk[(t + d) % kStages] >= 0 ? 1 : 0;
    if constexpr (kStages >= 3) {
      if (later >= 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(kStages >= 4 && later >= 2 ? 2 * kFillOps : kFillOps));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    }
    ring_barrier();
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) asm volatile("" : "+v"(qop[c]));  // loaded (waited above)
    blk[refill] = next_block(mine[refill]);
    if (blk[refill] >= 0) fill(blk[refill], refill);
    if (mine[t]) compute(blk[t], T_c);
  };
  static_assert(kStages >= 2 && kStages <= 4, "the wait above covers up to two later stages");
  while (!done) {
    step(std::integral_constant<int, 0>{});
    if (!done) step(std::integral_constant<int, 1>{});
    if constexpr (kStages >= 3)
      if (!done) step(std::integral_constant<int, 2>{});
    if constexpr (kStages >= 4)
      if (!done) step(std::integral_constant<int, 3>{});
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  __syncthreads();  // every wave is done with the stages before they hold the merge

  // Merge of the two key halves of each query half (as in the one-block
  // kernel), in the merge area of this wave's query block.
  const float l_half = sum_with_other_half(l_run);
  float* const xbase = (float*)lds + rsel * kMergeFloats;
  float* const mlbuf = xbase + 4 * 64 * kSendStride;  // [qh][kh][m, l][lane]
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  auto merge = [&](auto KHc) {
    constexpr int KH = decltype(KHc)::value;
    float* send = xbase + ((qh * 2 + KH) * 64 + l) * kSendStride;
#pragma unroll
    for (int t = 0; t < kHalfTiles; ++t) {
      constexpr int kSendBase = (1 - KH) * kHalfTiles;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(f32x4*)(send + t * 16 + 4 * g4) =
            f32x4{o[kSendBase + t][4 * g4], o[kSendBase + t][4 * g4 + 1], o[kSendBase + t][4 * g4 + 2],
                  o[kSendBase + t][4 * g4 + 3]};
    }
    mlbuf[((qh * 2 + KH) * 2 + 0) * 64 + l] = m_use;
    mlbuf[((qh * 2 + KH) * 2 + 1) * 64 + l] = l_half;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    ring_barrier();
    constexpr int PK = 1 - KH;
    const float* recv = xbase + ((qh * 2 + PK) * 64 + l) * kSendStride;
    const float m_p = mlbuf[((qh * 2 + PK) * 2 + 0) * 64 + l];
    const float l_p = mlbuf[((qh * 2 + PK) * 2 + 1) * 64 + l];
    const float m = fmaxf(m_use, m_p);
    const float fs = (m_use == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_use - m);
    const float fp = (m_p == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_p - m);
    const float l_tot = l_half * fs + l_p * fp;
    const float inv = l_tot > 0.0f ? __builtin_amdgcn_rcpf(l_tot) : 0.0f;  // 1 ulp; l_tot >= 2^-8
    const float cs = fs * inv, cp = fp * inv;
    if (KH == 0 && lse != nullptr && qrow < S)
      lse[lane * (int64_t)S + qrow] =
          l_tot > 0.0f ? (m + __builtin_log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
    if (qrow < S) {
      uint16_t* orow = out + lane_off + (int64_t)qrow * D;
#pragma unroll
      for (int t = 0; t < kHalfTiles; ++t) {
        constexpr int kKeepBase = KH * kHalfTiles;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const f32x4 y = *(const f32x4*)(recv + t * 16 + 4 * gg);
          float xv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[e] = o[kKeepBase + t][4 * gg + e] * cs + y[e] * cp;
          u32x2 val;
          val[0] = E::pack(xv[0], xv[1]);
          val[1] = E::pack(xv[2], xv[3]);
          *(u32x2*)(orow + 32 * (kKeepBase + t) + 8 * gg + 4 * h) = val;
        }
      }
    }
  };
  if (kh == 0)
    merge(std::integral_constant<int, 0>{});
  else
    merge(std::integral_constant<int, 1>{});
}

template <int D, bool BF16>
hipError_t launch_pair_typed(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t lanes, int64_t S, const int32_t* row_ptr, const int32_t* col_idx,
                             int64_t nnz, float scale_log2, hipStream_t stream) {
  const int64_t nb = (S + kBlock - 1) / kBlock;
  const int64_t npairs = (nb + kRows - 1) / kRows;
  // grid.x holds lanes; keep grid.x * block below 2^31 work-items per launch, in
  // multiples of 8 lanes so that every launch keeps the per-XCD lane order.
  const int64_t max_lanes = ((int64_t(1) << 31) / kPairThreads) & ~int64_t(7);
  for (int64_t l0 = 0; l0 < lanes; l0 += max_lanes) {
    const int64_t nl = lanes - l0 < max_lanes ? lanes - l0 : max_lanes;
    hipLaunchKernelGGL((attention_fwd_pair_kernel<D, BF16>), dim3((unsigned)nl, (unsigned)npairs),
                       dim3(kPairThreads), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (uint16_t*)out, lse, row_ptr, col_idx, nnz, (int)S, (int)nb,
                       l0, scale_log2, 1.0f / scale_log2);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

// grid.y holds the pair positions: at most 65535 of them (S up to 8 M tokens).
bool attention_fwd_pair_supported(int D, int64_t S) {
  const int64_t npairs = ((S + kBlock - 1) / kBlock + kRows - 1) / kRows;
  return (D == 64 || D == 128) && npairs <= 65535;
}

hipError_t launch_attention_fwd_pair(const void* q, const void* k, const void* v, void* out, float* lse,
                                     bool bf16, int64_t lanes, int64_t S, int D, const int32_t* row_ptr,
                                     const int32_t* col_idx, int64_t nnz, float scale_log2,
                                     hipStream_t stream) {
  if (D == 64)
    return bf16 ? launch_pair_typed<64, true>(q, k, v, out, lse, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream)
                : launch_pair_typed<64, false>(q, k, v, out, lse, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream);
  if (D == 128)
    return bf16 ? launch_pair_typed<128, true>(q, k, v, out, lse, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream)
                : launch_pair_typed<128, false>(q, k, v, out, lse, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream);
  return hipErrorInvalidValue;
}

}  // namespace tsa
