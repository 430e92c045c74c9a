// Scheduled block-sparse causal attention forward for gfx950 (CDNA4).
//
// Follows "Add topology-derived sparse attention kernel" (triton-lang/kernels
// PR 22), Summary: each 64-row query block visits only the key blocks its CSR
// row lists; one schedule is shared by every batch/head lane; the output keeps
// the input dtype.  The block loop keeps a running row max and denominator and
// rescales by exp(m_prev - m_new) (mirror page, Rust-port commit note), so one
// score tile is live at a time.
//
// Work decomposition
//   One workgroup = one (lane, query block) pair, 256 threads = 4 waves.  Wave w
//   owns query half qh = w & 1 (rows 32qh .. 32qh+31) and key half kh = w >> 1
//   (keys 32kh .. 32kh+31 of every visited block); each wave keeps its own
//   running max, denominator and O, and the two key halves of a query half are
//   merged once at the end.  Workgroup ids are remapped so that each of the 8
//   XCDs receives a contiguous range of lanes (its L2 then holds those lanes'
//   K/V).  Within that range the query blocks run by position, longest rows
//   first: the last query block of every lane of the range, then the one
//   before it, and so on, so that the short rows form the tail of the launch.
//
// Contractions (v_mfma_f32_32x32x16_{f16,bf16}, fp32 accumulation)
//   S^T = K . Q^T : A = K rows (keys) from LDS, B = Q^T held in registers.  The
//     result puts one query per lane column, so row statistics need only in-lane
//     reductions plus one exchange between the two half-waves.
//   O^T += V^T . P^T : A = V^T (head dims x keys) read from row-major V in LDS
//     with transposing reads (ds_read_b64_tr_b16); B = P^T straight from the S^T
//     result registers.  For this to line up, key 32kh + pi(m) is placed in MFMA
//     row m of the score tile, where pi swaps bits 2 and 3 of m; registers
//     8g .. 8g+7 of half-wave h then hold keys 16g + 8h + 0..7 of the half in
//     order, exactly the B operand of P.V step g.
//
// Data movement: K and V tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no registers in between) through a ring of stages;
// the copy of the next block is in flight while the current one is computed.
// 16-byte chunks inside a row are XOR-swizzled by row so that the operand reads
// spread over the LDS banks.  Probabilities use a lazy rescale: the exponent
// offset moves only when a row max exceeds it by more than 2^8.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "mfma_tile.h"

namespace tsa {
namespace {

using namespace tile;

constexpr int kThreads = 256;  // 4 waves: 2 query halves x 2 key halves

// Stages of the K/V ring: two ([K tile | V tile] each, 16 KB at head dim 64,
// 32 KB at 128); the copy of the next block lands while one is computed.
template <int D>
struct Stages {
  static constexpr int value = 2;
};

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void attention_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t nnz,
    int S, int nb, int64_t lane_base, int pos_base, float scale_log2, float inv_scale_log2) {
  using E = Elem<BF16>;
  constexpr int kStepsD = D / 16;                  // 16-deep steps of Q.K^T
  constexpr int kTilesD = D / 32;                  // 32-row tiles of O^T
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlock * kRowBytes;   // one K or V tile
  constexpr int kChunksPerRow = D / 8;
  constexpr int kWaves = kThreads / 64;
  constexpr int kFillOps = 2 * kTileBytes / 1024 / kWaves;  // 1 KB fill ops per wave per stage
  // Lazy rescale: the exponent offset moves only when a row's max exceeds it by
  // more than this many powers of two (P then stays <= 2^8).
  constexpr float kRescaleSlack = 8.0f;

  // A ring of kStages stages, each [K tile | V tile].  The copy of block n+kStages-1
  // is in flight while block n is computed.  Stage indices are compile-time
  // constants everywhere (the loop is unrolled by kStages), so the compiler can
  // tell copies into one stage from reads of another.
  constexpr int kStages = Stages<D>::value;
  __shared__ __attribute__((aligned(1024))) uint8_t stages[kStages][2 * kTileBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave (uniform)
  const int qh = w & 1;     // query half: rows 32qh .. 32qh+31 of the block
  const int kh = w >> 1;    // key half: keys 32kh .. 32kh+31 of every visited block
  const int l = tid & 63;
  const int h = l >> 5;     // half-wave
  const int n = l & 31;     // query column
  const int g = l >> 4;     // 16-lane group
  const int gi = l & 15;

  // Grid: x = lane, y = position nb - 1 - i (from pos_base).  Workgroup x + y X
  // runs on XCD x % 8; with X a multiple of 8, XCD c takes lanes c X/8 ..
  // (c + 1) X/8 - 1, so its L2 holds those lanes' K/V.  No division.
  const uint32_t X = gridDim.x, x = blockIdx.x;
  int64_t lane;
  if (X % 8u == 0u)
    lane = lane_base + (int64_t)((x % 8u) * (X / 8u) + x / 8u);
  else
    lane = lane_base + (int64_t)x;
  const int i = nb - 1 - (pos_base + (int)blockIdx.y);

  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* kg = k + lane_off;
  const uint16_t* vg = v + lane_off;

  // Q^T operands: lane holds query row qrow, dims 16c + 8h .. +7 for step c.
  const int qrow = i * kBlock + 32 * qh + n;
  const int qrow_c = qrow < S ? qrow : S - 1;
  // Issued before any copy: the first ring step's wait (at most the second
  // stage's copies outstanding) covers them.
  u32x4 qop[kStepsD];
  {
    const uint16_t* qp = q + lane_off + (int64_t)qrow_c * D + 8 * h;
    load_row_operands<kStepsD>(qop, qp);
  }

  // Per-lane byte offset, inside a block's rows, of the 16 bytes each fill op
  // moves.  Op o of wave w fills the 1 KB piece (o * kWaves + w) of [K | V]; a
  // tile is a whole number of kWaves-piece rounds, so the first half of the ops
  // fill K and the second half V (known at compile time).
  static_assert((kTileBytes / 1024) % kWaves == 0 && kFillOps % 2 == 0, "fill ops split K | V");
  // Consecutive ops of a tile half are kOpRows rows apart.  When that is a
  // multiple of 16 (D <= 128), the key permutation (bits 2, 3 of the row) and
  // both swizzles (bits 0..3) agree between them, so later ops only add the row
  // offset.
  constexpr int kOpRows = kWaves * 64 / kChunksPerRow;
  constexpr bool kDerive = kOpRows % 16 == 0;
  uint32_t fill_off[kFillOps];
#pragma unroll
  for (int op = 0; op < kFillOps; ++op) {
    constexpr int kHalfOps = kFillOps / 2;
    const bool is_v = op >= kHalfOps;
    const int oh = is_v ? op - kHalfOps : op;  // op within its tile half
    if (kDerive && oh > 0) {
      fill_off[op] = fill_off[op - oh] + (uint32_t)(oh * kOpRows * kRowBytes);
      continue;
    }
    const int cc = (oh * kWaves + w) * 64 + l;
    const int r = cc / kChunksPerRow, pc = cc % kChunksPerRow;
    const int key = is_v ? r : ((r & 32) | swap_bits23(r & 31));
    const int c = is_v ? (pc ^ v_swizzle<D>(r)) : (pc ^ k_swizzle<D>(r));
    fill_off[op] = (uint32_t)(key * kRowBytes + 16 * c);
  }
  // Queue the copy of K and V block j into one stage (no registers in between).
  // Rows past S read as zeros: only the last block, on its own diagonal, has
  // such rows, and the causal mask hides them.
  auto fill = [&](int j, uint8_t* stage) {
    const int rows = S - j * kBlock < kBlock ? S - j * kBlock : kBlock;
    copy_block_to_lds<kFillOps, kTileBytes / 1024 / kWaves, kWaves>(
        kg + (int64_t)j * kBlock * D, vg + (int64_t)j * kBlock * D, rows * kRowBytes, fill_off,
        stage, w);
  };

  // CSR row bounds, clamped to the readable entries (the C ABI caps entries at
  // int32 range).  The row's column indices are read 64 at a time into one
  // register per lane and handed out with readlane; a reload drains the memory
  // counter right away, so no other read of the window ever waits on memory.
  int p = (int)min((int64_t)max(row_ptr[i], 0), nnz);
  const int end = (int)max(min((int64_t)row_ptr[i + 1], nnz), (int64_t)p);
  // The row's first two blocks come from scalar loads, so that both ring
  // stages' copies are queued before the per-lane window of column indices
  // arrives (the compiler waits for the window only where it is first read).
  static_assert(kStages == 2, "the prologue below fills exactly two stages");
  int b_first = -1, b_second = -1;
  if (p < end) {
    const int c = col_idx[p];
    if (c >= 0 && c <= i) {
      b_first = c;
      ++p;
      if (p < end) {
        const int c2 = col_idx[p];
        if (c2 > c && c2 <= i) {
          b_second = c2;
          ++p;
        }
      }
    }
  }
  int win = p;
  int cols = (p + l < end) ? col_idx[p + l] : -1;
  if (b_first >= 0) fill(b_first, stages[0]);
  if (b_second >= 0) fill(b_second, stages[1]);
  auto next_block = [&](int last) -> int {
    while (p < end) {
      if (p - win >= 64) {
        win = p;
        cols = (p + l < end) ? col_idx[p + l] : -1;
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      }
      const int c = __builtin_amdgcn_readlane(cols, p - win);
      ++p;
      if (c > last && c <= i) return c;
    }
    return -1;
  };

  f32x16 o[kTilesD];
#pragma unroll
  for (int dt = 0; dt < kTilesD; ++dt) o[dt] = f32x16{};
  float m_use = -__builtin_inff();  // exponent offset in use (log2 units)
  float neg_m = __builtin_inff();    // -m_use, the FMA addend of the exponents (written only on a rescale)
  float thr_raw = -__builtin_inff();  // trigger threshold for the raw-score max (below)
  // Denominator.  At head dim <= 64 the softmax, not the matrix core, bounds
  // the block loop, so the row sums of the rounded P run on the MFMA (two
  // 16x16x32 products against a 0/1 selector, see row_sum_selector): lane l
  // then holds the whole sum of query l % 32 over this key half in l_acc[0].
  // Otherwise each lane sums its own half-wave's share with v_dot2.
  constexpr bool kMfmaSums = D <= 64;
  float l_run = 0.0f;
  f32x4 l_acc = f32x4{};
  const u32x4 sum_sel = row_sum_selector<E>(l);
  // Until the first offset is set nothing has been accumulated (O and l are 0 in
  // every lane), so that first rescale has nothing to scale (wave-uniform flag).
  bool started = false;

  // LDS byte addresses (stage 0) of this lane's K and V operand reads; stage t
  // adds t * 2 * kTileBytes through the instructions' offset field.
  const uint32_t ring_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)&stages[0][0];
  uint32_t k_addr[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c)
    k_addr[c] = ring_base + (uint32_t)k_chunk_offset<D>(32 * kh + n, 2 * c + h);
  uint32_t v_addr[kTilesD];
  {
    const int r0 = 32 * kh + 8 * (g >> 1) + (gi >> 2);  // key row for chunk 2kh, first read
    const uint32_t lane_addr = ring_base + (uint32_t)(kTileBytes + r0 * kRowBytes + 8 * (gi & 1));
    const int sw = v_swizzle<D>(r0);  // rows r0 + 4t + 16gg share r0's swizzle (same r & 3)
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) {
      const int dchunk = 4 * dt + 2 * (g & 1) + ((gi & 3) >> 1);
      v_addr[dt] = lane_addr + 16u * (uint32_t)(dchunk ^ sw);
    }
  }

  const int diag_lim = n - 8 * h;
  auto compute = [&](int j, auto T_c) {
    // Stage offset: in the instructions' 16-bit offset field when it fits (D <= 128),
    // else (D = 256, second stage at 64 KB) added to the lane addresses.
    constexpr int kStageAll = decltype(T_c)::value * 2 * kTileBytes;
    constexpr int kStageOff = kStageAll + 24 * kRowBytes < 65536 ? kStageAll : 0;
    constexpr uint32_t kStageReg = (uint32_t)(kStageAll - kStageOff);
    // On the diagonal block the key half above the query half is fully masked.
    if (j == i && kh > qh) return;
    // S^T (32 keys of this half x 32 queries) = K . Q^T.
    // K operands through asm reads: a plain LDS load here would make the
    // compiler wait for the next block's in-flight copy into the other stage.
    u32x4 ka[kStepsD];
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) ka[c] = lds_read_b128<kStageOff>(k_addr[c] + kStageReg);
    lds_wait_all(ka);
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < kStepsD; ++c) s = E::mfma(ka[c], qop[c], s);
    if (j == i && kh == qh) {  // diagonal sub-tile: key position must not exceed query position
      // key position of s[r] is 16 (r >> 3) + 8 h + (r & 7); compare its constant
      // part with n - 8 h
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (16 * (r >> 3) + (r & 7) > diag_lim) s[r] = -__builtin_inff();
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    // The pair of half-waves holding one query must share its offset, but the
    // pair's max is only needed when a half's own max can grow the offset: the
    // trigger compares raw scores with a threshold a little below
    // (m_use + slack) / scale_log2, and the exact test runs inside.
    if (__ballot(mx > thr_raw)) {
      const float mp = max_with_other_half(mx) * scale_log2;
      const bool grow = mp > m_use + kRescaleSlack;
      const float m_new = grow ? mp : m_use;
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      m_use = m_new;
      neg_m = -m_new;
      // a relative margin below the exact threshold, of either sign, covers the
      // rounding of mx * scale_log2, of the reciprocal and of the product
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
    // V^T operands for O^T += V^T . P^T over this half's two 16-key chunks come
    // from row-major V through transposing reads: lane (group g, index gi) gets
    // keys kb .. kb+3 of head dim 32dt + 16(g&1) + gi.  They are issued now and
    // land while the softmax runs.
    u32x2 va[kTilesD * 4];
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) {
      const uint32_t va_addr = v_addr[dt] + kStageReg;
      va[dt * 4 + 0] = lds_read_tr16<kStageOff>(va_addr);
      va[dt * 4 + 1] = lds_read_tr16<kStageOff + 4 * kRowBytes>(va_addr);
      va[dt * 4 + 2] = lds_read_tr16<kStageOff + 16 * kRowBytes>(va_addr);
      va[dt * 4 + 3] = lds_read_tr16<kStageOff + 20 * kRowBytes>(va_addr);
    }
    u32x4 pb[2];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * gg + 2 * x], scale_log2, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * gg + 2 * x + 1], scale_log2, neg_m));
        pb[gg][x] = E::pack(p0, p1);
      }
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if constexpr (!kMfmaSums) l_run = E::add_pair(pb[gg][x], l_run);
    if constexpr (kMfmaSums) {
      l_acc = E::mfma16(sum_sel, pb[0], l_acc);
      l_acc = E::mfma16(sum_sel, pb[1], l_acc);
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

  // Ring schedule.  blk[t] is the block held by stage t (-1: none).  At stage t:
  // wait until stage t's copy has landed (the other stage's may stay in
  // flight), barrier, queue the next block into the stage computed one step ago,
  // compute.  When the prologue queued two blocks, the first step has nothing
  // to refill.
  int blk[kStages];
  blk[0] = b_first >= 0 ? b_first : next_block(-1);
  blk[1] = b_first >= 0 ? b_second : -1;
  if (blk[0] >= 0) {
    if (b_first < 0) fill(blk[0], stages[0]);
    bool pre = blk[1] >= 0;  // stage 1 already queued: first step waits for stage 0 only
    int last = pre ? blk[1] : blk[0];
    bool done = false;
    auto step = [&](auto T_c) {
      constexpr int t = decltype(T_c)::value;
      constexpr int refill = (t + 1) % kStages;
      if (pre)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(kFillOps));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      ring_barrier();
#pragma unroll
      for (int c = 0; c < kStepsD; ++c) asm volatile("" : "+v"(qop[c]));  // loaded (waited above)
      if (!pre) {
        const int jn = last >= 0 ? next_block(last) : -1;
        blk[refill] = jn;
        last = jn;
        if (jn >= 0) fill(jn, stages[refill]);
      }
      pre = false;
      compute(blk[t], T_c);
      done = blk[refill] < 0;
    };
    while (!done) {
      step(std::integral_constant<int, 0>{});
      if (!done) step(std::integral_constant<int, 1>{});
    }
    __syncthreads();  // every wave is done with the stages before they hold the merge
  }

  // Merge the two key halves of each query half, then O / l rounded to the
  // input type (rows with no visible key get 0).  The two waves of a query half
  // split the head dims: wave kh keeps O tiles [kh, kh + 1) * kTilesD / 2 and
  // hands the other half, unscaled, to its partner together with its (m, l);
  // after one barrier each wave combines and stores its half.  The stage
  // buffers are free here (every wave has passed the last barrier).
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));  // no load of this wave outlives it (empty rows)
  const float l_half = kMfmaSums ? l_acc[0] : sum_with_other_half(l_run);
  // Wave kh keeps half of the O registers: whole tiles when there are two or more
  // (kHalfTiles each), else (D = 32) register groups 2kh, 2kh + 1 of the one tile.
  constexpr int kHalfTiles = kTilesD / 2;
  constexpr int kSendFloats = kTilesD >= 2 ? kHalfTiles * 16 : 8;
  constexpr int kSendStride = kSendFloats + 4;  // floats per lane (16-byte aligned, padded)
  static_assert((4 * 64 * kSendStride + 2 * 2 * 2 * 64) * 4 <= kStages * 2 * kTileBytes,
                "merge area exceeds the ring");
  float* const xbase = (float*)&stages[0][0];
  float* const mlbuf = xbase + 4 * 64 * kSendStride;  // [qh][kh][m, l][lane]
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  // KH is the wave's key half as a compile-time constant, so that the O tiles
  // are named by constants (a runtime index would put o in scratch memory).
  auto merge = [&](auto KHc) {
    constexpr int KH = decltype(KHc)::value;
    float* send = xbase + ((qh * 2 + KH) * 64 + l) * kSendStride;
    if constexpr (kTilesD >= 2) {
#pragma unroll
      for (int t = 0; t < kHalfTiles; ++t) {
        constexpr int kSendBase = (1 - KH) * kHalfTiles;  // tiles the partner keeps
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(f32x4*)(send + t * 16 + 4 * g4) =
              f32x4{o[kSendBase + t][4 * g4], o[kSendBase + t][4 * g4 + 1],
                    o[kSendBase + t][4 * g4 + 2], o[kSendBase + t][4 * g4 + 3]};
      }
    } else {
#pragma unroll
      for (int gl = 0; gl < 2; ++gl) {
        constexpr int kSendGroup = 2 * (1 - KH);  // groups the partner keeps
        *(f32x4*)(send + 4 * gl) = f32x4{o[0][4 * (kSendGroup + gl)], o[0][4 * (kSendGroup + gl) + 1],
                                         o[0][4 * (kSendGroup + gl) + 2], o[0][4 * (kSendGroup + gl) + 3]};
      }
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
    // v_rcp_f32 (1 ulp): l_tot >= 2^-8 here, far from the denormal range
    const float inv = l_tot > 0.0f ? __builtin_amdgcn_rcpf(l_tot) : 0.0f;
    const float cs = fs * inv, cp = fp * inv;
    // A row with no visible key (l_tot = 0) is written as +0 by a select, so its
    // output does not depend on what the accumulators or the exchange area hold
    // (products with a zero factor would carry their sign).
    const bool live = l_tot > 0.0f;
    // log of the row's denominator in natural units: log2(sum 2^(z log2 e)) = m + log2(l_tot)
    if (KH == 0 && lse != nullptr && qrow < S)
      lse[lane * (int64_t)S + qrow] =
          l_tot > 0.0f ? (m + __builtin_log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
    if (qrow < S) {
      uint16_t* orow = out + lane_off + (int64_t)qrow * D;
      if constexpr (kTilesD >= 2) {
#pragma unroll
        for (int t = 0; t < kHalfTiles; ++t) {
          constexpr int kKeepBase = KH * kHalfTiles;  // tiles this wave keeps
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const f32x4 y = *(const f32x4*)(recv + t * 16 + 4 * gg);
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = live ? o[kKeepBase + t][4 * gg + e] * cs + y[e] * cp : 0.0f;
            u32x2 val;
            val[0] = E::pack(x[0], x[1]);
            val[1] = E::pack(x[2], x[3]);
            *(u32x2*)(orow + 32 * (kKeepBase + t) + 8 * gg + 4 * h) = val;
          }
        }
      } else {
#pragma unroll
        for (int gl = 0; gl < 2; ++gl) {
          constexpr int kKeepGroup = 2 * KH;  // register groups this wave keeps
          const f32x4 y = *(const f32x4*)(recv + 4 * gl);
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = live ? o[0][4 * (kKeepGroup + gl) + e] * cs + y[e] * cp : 0.0f;
          u32x2 val;
          val[0] = E::pack(x[0], x[1]);
          val[1] = E::pack(x[2], x[3]);
          *(u32x2*)(orow + 8 * (kKeepGroup + gl) + 4 * h) = val;
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
hipError_t launch_typed(const void* q, const void* k, const void* v, void* out, float* lse, int64_t lanes,
                        int64_t S, const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                        float scale_log2, hipStream_t stream) {
  const int64_t nb = (S + kBlock - 1) / kBlock;
  // grid.x = lanes (at most 2^31 work-items per launch, in multiples of 8 lanes
  // so that every launch keeps the per-XCD lane order), grid.y = positions (at
  // most 65535 per launch); the positions of one lane range go longest first.
  const int64_t max_lanes = ((int64_t(1) << 31) / kThreads) & ~int64_t(7);
  constexpr int64_t kMaxPositions = 65535;
  for (int64_t l0 = 0; l0 < lanes; l0 += max_lanes) {
    const int64_t nl = lanes - l0 < max_lanes ? lanes - l0 : max_lanes;
    for (int64_t p0 = 0; p0 < nb; p0 += kMaxPositions) {
      const int64_t np = nb - p0 < kMaxPositions ? nb - p0 : kMaxPositions;
      hipLaunchKernelGGL((attention_fwd_kernel<D, BF16>), dim3((unsigned)nl, (unsigned)np), dim3(kThreads),
                         0, stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                         (uint16_t*)out, lse, row_ptr, col_idx, nnz, (int)S, (int)nb, l0, (int)p0,
                         scale_log2, 1.0f / scale_log2);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attention_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                                bool bf16, int64_t lanes, int64_t S, int D, int block,
                                const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                float scale_log2, hipStream_t stream) {
  // 32-row blocks: only the two-block kernel walks them (one CSR row per wave).
  if (block == 32)
    return attention_fwd_duo_supported(D, S)
               ? launch_attention_fwd_duo(q, k, v, out, lse, bf16, lanes, S, D, 32, row_ptr,
                                          col_idx, nnz, scale_log2, stream)
               : hipErrorInvalidValue;
  if (block != kBlock) return hipErrorInvalidValue;
  // Head dim 128: two query blocks per workgroup of eight waves share each 32 KB
  // K/V stage.  Head dim 64: two query blocks per workgroup of four waves, once
  // the launch has enough (lane, query block) pairs that the halved grid still
  // fills every CU four workgroups deep (256 CUs x 4 x 2 pairs); below that the
  // one-block kernel's twice larger grid is faster.
  if (D == 128 && attention_fwd_duo_supported(D, S))
    return launch_attention_fwd_duo(q, k, v, out, lse, bf16, lanes, S, D, kBlock, row_ptr, col_idx,
                                    nnz, scale_log2, stream);
  constexpr int64_t kDuoMinPairs = 2048;
  const int64_t nb = (S + kBlock - 1) / kBlock;
  if (D == 64 && lanes * nb >= kDuoMinPairs && attention_fwd_duo_supported(D, S))
    return launch_attention_fwd_duo(q, k, v, out, lse, bf16, lanes, S, D, kBlock, row_ptr, col_idx,
                                    nnz, scale_log2, stream);
#define TSA_FWD_CASE(DD)                                                                              \
  if (D == DD)                                                                                      \
    return bf16 ? launch_typed<DD, true>(q, k, v, out, lse, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream) \
                : launch_typed<DD, false>(q, k, v, out, lse, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream);
  TSA_FWD_CASE(64)
  TSA_FWD_CASE(128)
  TSA_FWD_CASE(32)
  TSA_FWD_CASE(256)
#undef TSA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tsa
