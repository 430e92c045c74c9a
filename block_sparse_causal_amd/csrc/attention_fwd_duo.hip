// Scheduled block-sparse causal attention forward for gfx950 (CDNA4), head dims
// 64 and 128 (and 32 with 32-row blocks): two adjacent query blocks per
// workgroup of four waves, each wave taking every key of a visited block.
//
// Same operation as attention_fwd.hip ("Add topology-derived sparse attention
// kernel", triton-lang/kernels PR 22, Summary: each 64-row query block visits
// only the key blocks its CSR row lists; one schedule is shared by every
// batch/head lane; the output keeps the input dtype; running max and
// denominator per query row, rescaled by exp(m_prev - m_new) as in the mirror
// page's Rust-port commit note).
//
// Work decomposition
//   One workgroup = one lane and the query-block pair (2g, 2g+1): 256 threads,
//   4 waves.  Wave w owns query half qh = w & 1 of block 2g + (w >> 1) and takes
//   both 32-key halves of every block its row lists, one after the other, into
//   one running max, denominator and O.  The workgroup walks the union of the
//   two CSR rows in ascending order; each block of the union is copied into LDS
//   once, and the waves of a row compute it only when their row lists it.
//   Adjacent rows of a causal schedule share most of their blocks (the sink,
//   the top-k set, all but one of the local window), so each copied tile serves
//   about twice the queries of the one-block kernel, and since each wave holds
//   whole rows no merge of key halves is needed at the end.
//
//   Grid: x = lane (remapped so that each of the 8 XCDs holds a contiguous range
//   of lanes when the lane count is a multiple of 8; workgroup x + y * lanes
//   runs on XCD x % 8), y = pair position, last pairs (longest rows) first.  At
//   head dim 128 each XCD runs its lanes two at a time instead (all pair
//   positions of a lane pair, longest first), which keeps the K/V blocks its
//   workgroups share within its L2.
//
// Schedules over 32-row blocks (SUB): the same workgroup serves the four
//   32-row query blocks 4g .. 4g+3, which are its waves' query halves, and
//   each wave walks its own CSR row.  The tiles stay 64 keys: the workgroup
//   walks the union of the 64-key blocks its four rows touch, and a wave takes
//   the key half 2J + h of 64-key block J only when its row lists that 32-key
//   block.  Each wave's work is then exactly a 32 x 32 tile per listed block,
//   with the causal mask on the tile whose key block equals its query block.
//
// Contractions, tile layouts, staging and the softmax are the one-block
// kernel's (attention_fwd.hip): S^T = K . Q^T with Q^T in registers, O^T +=
// V^T . P^T with transposing V reads, key rows permuted so that the S^T
// registers are the P^T operand, a two-stage ring of [K | V] tiles filled by
// direct global->LDS copies, lazy rescale, row sums on the matrix core at head
// dim 64.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <type_traits>

#include "kernels.h"
#include "mfma_tile.h"

namespace tsa {
namespace {

using namespace tile;

constexpr int kDuoThreads = 256;  // 2 query blocks x 2 query halves
constexpr int kDuoRows = 2;

// Inclusive prefix maximum across the wave's 64 lanes (lane l: the maximum over
// lanes 0..l): shifts by 1, 2, 4 and 8 lanes within each row of 16, then the
// last lane of rows 0 and 2 into rows 1 and 3, and lane 31 into rows 2 and 3.
// Lanes a step does not write take INT_MIN, which leaves the maximum unchanged.
__device__ __forceinline__ int wave_prefix_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}

// Cursor over the accepted entries of one CSR row.  An entry is accepted when it
// lies in 0..i and exceeds the previous accepted entry (the rule of the
// one-block kernel); equivalently, when it lies in 0..i and exceeds every
// earlier entry of the row that does, which a wave evaluates for a window of
// 64 entries at once with one prefix maximum.  The accepted lanes of the
// window form a wave-uniform bit mask, and taking the next entry is a
// find-first-set and one lane read.
struct DuoCursor {
  int i;         // CSR row, or -1 when it lies past the last row
  int p, end;    // start of the next window, end of the row (clamped to the readable entries)
  int cols;      // lane l: entry l of the current window (or -1)
  uint64_t acc;  // accepted lanes of the current window not yet taken
  int last;      // largest accepted entry so far (-1: none)
  int head;      // next accepted entry (INT_MAX: none left)
  // Issues the load of the first window; scan() reads it once it has arrived.
  __device__ __forceinline__ void start(const int32_t* __restrict__ row_ptr,
                                        const int32_t* __restrict__ col_idx, int64_t nnz, int row,
                                        int nrows, int l) {
    i = row < nrows ? row : -1;
    if (i >= 0) {
      p = (int)min((int64_t)max(row_ptr[i], 0), nnz);
      end = (int)max(min((int64_t)row_ptr[i + 1], nnz), (int64_t)p);
    } else {
      p = end = 0;
    }
    cols = (p + l < end) ? col_idx[p + l] : -1;
    acc = 0;
    last = -1;
    head = INT_MAX;
  }
  // Accepted lanes of the window loaded at p.  Entries are ranked by (value,
  // earlier lane first), so that a repeated value is never a new maximum; the
  // key fits 32 bits since rows are below 2^18 (the grid's pair limit).
  __device__ __forceinline__ void scan(int l) {
    const int x = (cols >= 0 && cols <= i) ? cols : -1;
    const int key = x * 64 + (63 - l);
    const int run = wave_prefix_max(key);
    acc = __builtin_amdgcn_ballot_w64(x > last && key == run);
    last = max(last, __builtin_amdgcn_readlane(run, 63) >> 6);  // -1 when nothing is valid
    p += 64;
  }
  // Moves `head` to the next accepted entry.  A window reload waits for every
  // outstanding vector load of the wave (only rows of more than 64 entries).
  __device__ __forceinline__ void advance(const int32_t* __restrict__ col_idx, int l) {
    while (acc == 0) {
      if (p >= end) {
        head = INT_MAX;
        return;
      }
      cols = (p + l < end) ? col_idx[p + l] : -1;
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      scan(l);
    }
    head = __builtin_amdgcn_readlane(cols, (int)__builtin_ctzll(acc));
    acc &= acc - 1;
  }
};

// nrows: the CSR's rows (ceil(S / 64), or ceil(S / 32) when SUB).
template <int D, bool BF16, bool SUB>
__global__ __launch_bounds__(kDuoThreads) void attention_fwd_duo_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t nnz,
    int S, int nrows, int64_t lane_base, float scale_log2, float inv_scale_log2) {
  using E = Elem<BF16>;
  constexpr int kStepsD = D / 16;
  constexpr int kTilesD = D / 32;
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlock * kRowBytes;
  constexpr int kStageBytes = 2 * kTileBytes;
  constexpr int kChunksPerRow = D / 8;
  constexpr int kWaves = kDuoThreads / 64;
  constexpr int kFillOps = kStageBytes / 1024 / kWaves;  // 1 KB fill ops per wave per stage
  constexpr float kRescaleSlack = 8.0f;
  constexpr int kStages = 2;
  constexpr int kHalfKeyBytes = 32 * kRowBytes;  // second key half: 32 rows further
  // Row sums: at head dim 64 the softmax, not the matrix core, bounds the loop,
  // so the sums of the rounded P run on the MFMA (two 16x16x32 products against
  // a 0/1 selector; lane l then holds the sum of query l % 32); at 128 each
  // lane sums its half-wave's share with v_dot2.
  constexpr bool kMfmaSums = D <= 64;
  // CSR rows a workgroup walks: the two 64-row blocks, or the four 32-row ones.
  constexpr int kCursors = SUB ? 4 : kDuoRows;
  // Lanes an XCD works on at a time at head dim 128 (0: all of its range, the
  // pair positions running across them).  Measured at [2,32,8192,128] over the
  // dense causal CSR: 1081 -> 1046 us with 2, 1056 with 4, 1075 with 1; at head
  // dim 64 every grouping was slower (57.0 -> 62.4 us at [4,16,4096,64]).
  constexpr uint32_t kLaneGroup = D == 128 ? 2u : 0u;
  static_assert((kTileBytes / 1024) % kWaves == 0 && kFillOps % 2 == 0, "fill ops split K | V");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStageBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave (uniform)
  const int rsel = w >> 1;  // which query block of the pair
  const int qh = w & 1;     // query half of that block
  const int l = tid & 63;
  const int h = l >> 5;
  const int n = l & 31;
  const int g = l >> 4;
  const int gi = l & 15;

  // Lane and pair position (see the header comment).
  const uint32_t X = gridDim.x, x = blockIdx.x;
  const int npairs = (int)gridDim.y;
  int64_t lane;
  int pair;
  if (kLaneGroup > 0 && X % (8u * kLaneGroup) == 0u) {
    // Head dim 128: XCD k (= workgroup id % 8) takes its lanes kLaneGroup at a
    // time, each group's pair positions longest first, so that the K/V blocks
    // its workgroups share fit its L2 (4 MB of K/V per lane of 8192 keys).
    const uint32_t id = x + (uint32_t)blockIdx.y * X;
    const uint32_t xcd = id % 8u, seq = id / 8u;
    const uint32_t per_group = kLaneGroup * (uint32_t)npairs;
    const uint32_t grp = seq / per_group, rem = seq % per_group;
    lane = lane_base + (int64_t)(xcd * (X / 8u) + grp * kLaneGroup + rem % kLaneGroup);
    pair = npairs - 1 - (int)(rem / kLaneGroup);
  } else if (X % 8u == 0u) {
    lane = lane_base + (int64_t)((x % 8u) * (X / 8u) + x / 8u);
    pair = npairs - 1 - (int)blockIdx.y;
  } else {
    lane = lane_base + (int64_t)x;
    pair = npairs - 1 - (int)blockIdx.y;
  }
  const int my_i = kDuoRows * pair + rsel;  // this wave's 64-row block (past the end: no rows)
  const int my_q32 = 4 * pair + w;         // and its 32-row query block

  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* kg = k + lane_off;
  const uint16_t* vg = v + lane_off;

  // Column windows of both rows first, then the Q^T operands (lane: query row
  // qrow, dims 16c + 8h .. +7 for step c); the first wait below covers the
  // windows and lets the Q loads stay in flight.
  DuoCursor rows[kCursors];
#pragma unroll
  for (int r = 0; r < kCursors; ++r) rows[r].start(row_ptr, col_idx, nnz, kCursors * pair + r, nrows, l);
  const int qrow = my_i * kBlock + 32 * qh + n;
  const int qrow_c = qrow < S ? qrow : S - 1;
  u32x4 qop[kStepsD];
  {
    const uint16_t* qp = q + lane_off + (int64_t)qrow_c * D + 8 * h;
    load_row_operands<kStepsD>(qop, qp);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(kStepsD));  // the windows (older than the Q loads)
#pragma unroll
  for (int r = 0; r < kCursors; ++r) {
    rows[r].scan(l);
    rows[r].advance(col_idx, l);
  }

  // Next 64-key block of the union of the rows (-1: none); `mine` gets bit h
  // set when this wave computes key half h of it: both halves when its 64-row
  // block's row lists the block, or (SUB) the halves its 32-row row lists.
  auto next_block = [&](int& mine) -> int {
    int hmin = INT_MAX;
#pragma unroll
    for (int r = 0; r < kCursors; ++r) hmin = min(hmin, rows[r].head);
    mine = 0;
    if (hmin == INT_MAX) return -1;
    const int j = SUB ? hmin >> 1 : hmin;  // (INT_MAX >> 1 is no block index)
#pragma unroll
    for (int r = 0; r < kCursors; ++r) {
      if constexpr (SUB) {
        // at most the two 32-key blocks of j, in ascending order
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if ((rows[r].head >> 1) == j) {
            if (r == w) mine |= 1 << (rows[r].head & 1);
            rows[r].advance(col_idx, l);
          }
      } else {
        if (rows[r].head == j) {
          if (r == rsel) mine = 3;
          rows[r].advance(col_idx, l);
        }
      }
    }
    return j;
  };

  // Per-lane byte offsets of the 16 bytes each fill op moves (as in the
  // one-block kernel: later ops of a tile half only add the row offset).
  constexpr int kOpRows = kWaves * 64 / kChunksPerRow;
  static_assert(kOpRows % 16 == 0, "fill ops of a tile half share the row swizzle");
  uint32_t fill_off[kFillOps];
#pragma unroll
  for (int op = 0; op < kFillOps; ++op) {
    constexpr int kHalfOps = kFillOps / 2;
    const bool is_v = op >= kHalfOps;
    const int oh = is_v ? op - kHalfOps : op;
    if (oh > 0) {
      fill_off[op] = fill_off[op - oh] + (uint32_t)(oh * kOpRows * kRowBytes);
      continue;
    }
    const int cc = w * 64 + l;
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
  float m_use = -__builtin_inff();   // exponent offset in use (log2 units)
  float neg_m = __builtin_inff();     // -m_use (written only on a rescale)
  float thr_raw = -__builtin_inff();  // trigger threshold for the raw-score max
  f32x4 l_acc = f32x4{};              // row sums of the rounded P on the matrix core
  float l_run = 0.0f;                 // or this half-wave's share of them
  const u32x4 sum_sel = row_sum_selector<E>(l);
  bool started = false;

  // LDS byte addresses (stage 0, key half 0) of this lane's K and V operand
  // reads; the stage and the key half are added through the offset field.
  const uint32_t ring_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)&lds[0];
  uint32_t k_addr[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) k_addr[c] = ring_base + (uint32_t)k_chunk_offset<D>(n, 2 * c + h);
  uint32_t v_addr[kTilesD];
  {
    const int r0 = 8 * (g >> 1) + (gi >> 2);
    const uint32_t lane_addr = ring_base + (uint32_t)(kTileBytes + r0 * kRowBytes + 8 * (gi & 1));
    const int sw = v_swizzle<D>(r0);
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) {
      const int dchunk = 4 * dt + 2 * (g & 1) + ((gi & 3) >> 1);
      v_addr[dt] = lane_addr + 16u * (uint32_t)(dchunk ^ sw);
    }
  }

  const int diag_lim = n - 8 * h;
  // One key half KH of a visited block held by ring stage T (both compile-time).
  auto compute_half = [&](int j, auto T_c, auto KH_c) {
    constexpr int KH = decltype(KH_c)::value;
    constexpr int kOff = decltype(T_c)::value * kStageBytes + KH * kHalfKeyBytes;
    static_assert(kOff + kTileBytes + 20 * kRowBytes < 65536, "offsets fit the LDS offset field");
    // 32-row key block 2j + KH against this wave's 32-row query block: later
    // ones are fully masked (the acceptance rule never lists them under SUB;
    // on the 64-row diagonal key half 1 is later than query half 0).
    if (2 * j + KH > my_q32) return;
    u32x4 ka[kStepsD];
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) ka[c] = lds_read_b128<kOff>(k_addr[c]);
    lds_wait_all(ka);
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) s = E::mfma(ka[c], qop[c], s);
    if (2 * j + KH == my_q32) {  // key position must not exceed query position
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
      neg_m = -m_new;
      const float thr = (m_new + kRescaleSlack) * inv_scale_log2;
      thr_raw = thr - __builtin_fabsf(thr) * 0x1p-20f;
      if (started) {
        if constexpr (kMfmaSums)
          l_acc *= alpha;
        else
          l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kTilesD; ++dt) o[dt] *= alpha;
      }
      started = true;
    }
    u32x2 va[kTilesD * 4];
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) {
      va[dt * 4 + 0] = lds_read_tr16<kOff>(v_addr[dt]);
      va[dt * 4 + 1] = lds_read_tr16<kOff + 4 * kRowBytes>(v_addr[dt]);
      va[dt * 4 + 2] = lds_read_tr16<kOff + 16 * kRowBytes>(v_addr[dt]);
      va[dt * 4 + 3] = lds_read_tr16<kOff + 20 * kRowBytes>(v_addr[dt]);
    }
    u32x4 pb[2];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * gg + 2 * xx], scale_log2, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * gg + 2 * xx + 1], scale_log2, neg_m));
        pb[gg][xx] = E::pack(p0, p1);
      }
    if constexpr (kMfmaSums) {
      l_acc = E::mfma16(sum_sel, pb[0], l_acc);
      l_acc = E::mfma16(sum_sel, pb[1], l_acc);
    } else {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) l_run = E::add_pair(pb[gg][xx], l_run);
    }
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

  // Ring over the union: blk[t] is the block held by stage t (-1: none),
  // mine[t] whether this wave's row lists it.  The first block is queued here;
  // at step t the wave waits for stage t's copies, passes the barrier, queues
  // the next union block into the stage computed one step earlier, and
  // computes both key halves.
  int blk[kStages];
  int mine[kStages];
  blk[1] = -1;
  mine[1] = 0;
  blk[0] = next_block(mine[0]);
  if (blk[0] >= 0) fill(blk[0], 0);
  bool done = blk[0] < 0;
  auto step = [&](auto T_c) {
    constexpr int t = decltype(T_c)::value;
    constexpr int refill = (t + 1) % kStages;
    if (blk[t] < 0) {
      done = true;
      return;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    ring_barrier();
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) asm volatile("" : "+v"(qop[c]));  // loaded (waited above)
    blk[refill] = next_block(mine[refill]);
    if (blk[refill] >= 0) fill(blk[refill], refill);
    if (mine[t] & 1) compute_half(blk[t], T_c, std::integral_constant<int, 0>{});
    if (mine[t] & 2) compute_half(blk[t], T_c, std::integral_constant<int, 1>{});
  };
  while (!done) {
    step(std::integral_constant<int, 0>{});
    if (!done) step(std::integral_constant<int, 1>{});
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));  // no load of this wave outlives it (empty rows)

  // O / l rounded to the input type (rows with no visible key get 0).  Lane l
  // holds the row sum of query l % 32 in l_acc[0] and dims 32t + 8(r/4) + 4h +
  // r%4 of that query in register r of o[t].
  const float l_tot = kMfmaSums ? l_acc[0] : sum_with_other_half(l_run);
  // v_rcp_f32 (1 ulp): once a row has a visible key, l_tot >= 1 (the element
  // that set the offset contributes exactly 1), far from the denormal range
  const float inv = l_tot > 0.0f ? __builtin_amdgcn_rcpf(l_tot) : 0.0f;
  if (h == 0 && lse != nullptr && qrow < S)
    lse[lane * (int64_t)S + qrow] =
        l_tot > 0.0f ? (m_use + __builtin_log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
  if (qrow < S) {
    uint16_t* orow = out + lane_off + (int64_t)qrow * D;
#pragma unroll
    for (int t = 0; t < kTilesD; ++t)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        u32x2 val;
        val[0] = E::pack(o[t][4 * gg] * inv, o[t][4 * gg + 1] * inv);
        val[1] = E::pack(o[t][4 * gg + 2] * inv, o[t][4 * gg + 3] * inv);
        if (!(l_tot > 0.0f)) val = u32x2{0u, 0u};  // no visible key: +0, whatever o holds
        *(u32x2*)(orow + 32 * t + 8 * gg + 4 * h) = val;
      }
  }
}

template <int D, bool BF16, bool SUB>
hipError_t launch_duo_typed(const void* q, const void* k, const void* v, void* out, float* lse,
                            int64_t lanes, int64_t S, const int32_t* row_ptr, const int32_t* col_idx,
                            int64_t nnz, float scale_log2, hipStream_t stream) {
  const int64_t nb = (S + kBlock - 1) / kBlock;
  const int64_t nrows = SUB ? (S + 31) / 32 : nb;
  const int64_t npairs = (nb + kDuoRows - 1) / kDuoRows;
  // grid.x holds lanes; keep grid.x * block below 2^31 work-items per launch, in
  // multiples of 8 lanes so that every launch keeps the per-XCD lane order.
  const int64_t max_lanes = ((int64_t(1) << 31) / kDuoThreads) & ~int64_t(7);
  for (int64_t l0 = 0; l0 < lanes; l0 += max_lanes) {
    const int64_t nl = lanes - l0 < max_lanes ? lanes - l0 : max_lanes;
    hipLaunchKernelGGL((attention_fwd_duo_kernel<D, BF16, SUB>), dim3((unsigned)nl, (unsigned)npairs),
                       dim3(kDuoThreads), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (uint16_t*)out, lse, row_ptr, col_idx, nnz, (int)S,
                       (int)nrows, l0, scale_log2, 1.0f / scale_log2);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

// grid.y holds the pair positions: at most 65535 of them (S up to 8 M tokens).
bool attention_fwd_duo_supported(int D, int64_t S) {
  const int64_t npairs = ((S + kBlock - 1) / kBlock + kDuoRows - 1) / kDuoRows;
  return (D == 32 || D == 64 || D == 128) && npairs <= 65535;
}

hipError_t launch_attention_fwd_duo(const void* q, const void* k, const void* v, void* out, float* lse,
                                    bool bf16, int64_t lanes, int64_t S, int D, int block,
                                    const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                    float scale_log2, hipStream_t stream) {
#define TSA_DUO_CASE(DD, SUBB)                                                                          \
  if (D == DD && (block == 32) == SUBB)                                                               \
    return bf16 ? launch_duo_typed<DD, true, SUBB>(q, k, v, out, lse, lanes, S, row_ptr, col_idx, nnz, \
                                                   scale_log2, stream)                                 \
                : launch_duo_typed<DD, false, SUBB>(q, k, v, out, lse, lanes, S, row_ptr, col_idx, nnz, \
                                                    scale_log2, stream);
  TSA_DUO_CASE(64, false)
  TSA_DUO_CASE(128, false)
  TSA_DUO_CASE(32, true)
  TSA_DUO_CASE(64, true)
  TSA_DUO_CASE(128, true)
#undef TSA_DUO_CASE
  return hipErrorInvalidValue;
}

}  // namespace tsa
