// Scheduled block-sparse causal attention forward for gfx950 (CDNA4).
//
// Follows "Add topology-derived sparse attention kernel" (triton-lang/kernels
// PR 22), Summary: each 64-row query block visits only the key blocks its CSR
// row lists; one schedule is shared by every batch/head lane; the output keeps
// the input dtype.  The block loop keeps a running row max and denominator and
// rescales by exp(m_prev - m_new) (mirror page, Rust-port commit note), so one
// 64x64 score tile is live at a time.
//
// Work decomposition
//   One workgroup = one (lane, query block) pair, 128 threads = 2 waves; wave w
//   owns query rows 32w .. 32w+31 of the block.  Workgroup ids are remapped so
//   that each of the 8 XCDs receives a contiguous range of lanes (its L2 then
//   holds those lanes' K/V), and within a lane query blocks run longest-row
//   first (descending block index).
//
// Contractions (v_mfma_f32_32x32x16_{f16,bf16}, fp32 accumulation)
//   S^T = K . Q^T : A = K tile rows (keys) from LDS, B = Q^T held in registers.
//     The result puts one query per lane column, so row statistics need only
//     in-lane reductions plus one exchange between the two half-waves.
//   O^T += V^T . P^T : A = V^T rows (head dims) from LDS, B = P^T straight from
//     the S^T result registers.  For this to line up, key 32t + pi(m) is placed
//     in MFMA row m of score tile t, where pi swaps bits 2 and 3 of m; then the
//     registers 8g .. 8g+7 of tile t of half-wave h hold keys
//     16(2t+g) + 8h + 0..7 in order, exactly the B operand of P.V step 2t+g.
//
// LDS (per workgroup, one stage): K tile [64][D] in MFMA row order, V^T tile
// [D][64].  Each 16-byte chunk index within a row is XORed with (row & 7) so
// both the staging writes and the MFMA operand reads are free of bank
// conflicts.  The next tile's global loads are issued into registers before the
// current tile's math and written to LDS after it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;
constexpr int kThreads = 128;

// Element-type specific pieces: the MFMA, the fp32 -> 2 x 16-bit pack (round to
// nearest even) and a pairwise add of a packed pair into an fp32 sum.
template <bool BF16>
struct Elem;

template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float add_pair(uint32_t p, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
  }
};

template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float add_pair(uint32_t p, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
  }
};

// Value of the partner lane l ^ 32, combined with the own value.
__device__ __forceinline__ float max_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMA row m of a score tile holds key pi(m) of that 32-key half; pi swaps bits 2, 3.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Byte offset, inside one tile, of the 16-byte chunk `c` (8 elements) of row `r`.
// K rows use chunk ^ (r & 7); V rows use chunk ^ 2*t(r & 3), where t spreads the
// four key rows that one transposing read touches over distinct bank groups.
template <int D>
__device__ __forceinline__ int k_chunk_offset(int r, int c) {
  return r * (D * 2) + 16 * (c ^ (r & 7));
}
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  if (D == 64) return 2 * (r & 3);
  const int t = (0x6530 >> (4 * (r & 3))) & 0xF;  // 0, 3, 5, 6
  return 2 * t;
}
template <int D>
__device__ __forceinline__ int v_chunk_offset(int r, int c) {
  return r * (D * 2) + 16 * (c ^ v_swizzle<D>(r));
}

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void attention_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t nnz,
    int S, int nb, int64_t lane_base, float scale_log2) {
  using E = Elem<BF16>;
  constexpr int kStepsD = D / 16;                  // 16-deep steps of Q.K^T
  constexpr int kTilesD = D / 32;                  // 32-row tiles of O^T
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBlock * kRowBytes;   // one K or V tile
  constexpr int kChunksPerRow = D / 8;
  constexpr int kFillOps = 2 * kTileBytes / (16 * 64) / 2;  // 16-byte-per-lane fills per wave per stage
  // Lazy rescale: the running max used for the exponent moves only when a row's
  // max exceeds it by more than this many powers of two (P then stays <= 2^8).
  constexpr float kRescaleSlack = 8.0f;

  // Two stages, each [K tile | V tile]; distinct objects so that the compiler
  // can tell loads into one stage from reads of the other.
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[2 * kTileBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave (uniform)
  const int l = tid & 63;   // lane in wave
  const int h = l >> 5;     // half-wave
  const int n = l & 31;     // query column within the wave's 32 rows
  const int g = l >> 4;     // 16-lane group
  const int gi = l & 15;

  const uint32_t G = gridDim.x;
  const uint32_t bid = blockIdx.x;
  const uint32_t logical = (G % 8u == 0u) ? (bid % 8u) * (G / 8u) + bid / 8u : bid;
  const int64_t lane = lane_base + logical / (uint32_t)nb;
  const int i = nb - 1 - (int)(logical % (uint32_t)nb);

  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* kg = k + lane_off;
  const uint16_t* vg = v + lane_off;

  // Q^T operands: lane holds query row qrow, dims 16c + 8h .. +7 for step c.
  const int qrow = i * kBlock + 32 * w + n;
  const int qrow_c = qrow < S ? qrow : S - 1;
  u32x4 qop[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c)
    qop[c] = *(const u32x4*)(q + lane_off + (int64_t)qrow_c * D + 16 * c + 8 * h);

  // CSR row bounds, clamped to the readable entries.  The row's column indices
  // are read 64 at a time into one register per lane and handed out with
  // readlane, so walking the row costs no memory latency per block.
  int64_t p = row_ptr[i];
  int64_t end = row_ptr[i + 1];
  p = p < 0 ? 0 : (p > nnz ? nnz : p);
  end = end < p ? p : (end > nnz ? nnz : end);
  int64_t win = p;  // first entry held in `cols`
  int cols = (p + l < end) ? col_idx[p + l] : -1;
  auto next_block = [&](int last) -> int {
    while (p < end) {
      if (p - win >= 64) {
        win = p;
        cols = (p + l < end) ? col_idx[p + l] : -1;
      }
      const int c = __builtin_amdgcn_readlane(cols, (int)(p - win));
      ++p;
      if (c > last && c <= i) return c;
    }
    return -1;
  };

  // Queue the copy of K and V block j into one stage: every lane moves 16 bytes
  // per op straight from global memory into LDS (no registers in between).
  // Rows past S are clamped to row S-1 (finite values that the causal mask or
  // a zero probability removes).
  // Per-lane byte offset, inside a block's rows, of the 16 bytes each fill op
  // moves; the ops of a wave alternate between the K and the V tile.
  uint32_t fill_off[kFillOps];
#pragma unroll
  for (int op = 0; op < kFillOps; ++op) {
    const int chunk = (op * 2 + w) * 64 + l;  // 16-byte chunk index within [K | V]
    const bool is_v = chunk >= kBlock * kChunksPerRow;
    const int cc = is_v ? chunk - kBlock * kChunksPerRow : chunk;
    const int r = cc / kChunksPerRow, pc = cc % kChunksPerRow;
    const int key = is_v ? r : ((r & 32) | swap_bits23(r & 31));
    const int c = is_v ? (pc ^ v_swizzle<D>(r)) : (pc ^ (r & 7));
    fill_off[op] = (uint32_t)(key * kRowBytes + 16 * c);
  }
  // Queue the copy of K and V block j into one stage: every lane moves 16 bytes
  // per op straight from global memory into LDS (no registers in between).
  auto fill = [&](int j, uint8_t* stage) {
    const char* kb = (const char*)(kg + (int64_t)j * kBlock * D);
    const char* vb = (const char*)(vg + (int64_t)j * kBlock * D);
    const int lim = S - j * kBlock;  // rows of this block that exist
    if (lim >= kBlock) {
#pragma unroll
      for (int op = 0; op < kFillOps; ++op) {
        const bool is_v = (op * 2 + w) * 64 >= kBlock * kChunksPerRow;  // uniform per op
        __builtin_amdgcn_global_load_lds((const void*)((is_v ? vb : kb) + fill_off[op]),
                                         (__attribute__((address_space(3))) void*)(stage + (op * 2 + w) * 1024),
                                         16, 0, 0);
      }
    } else {  // partial last block: rows past S are clamped to row S-1
#pragma unroll
      for (int op = 0; op < kFillOps; ++op) {
        const bool is_v = (op * 2 + w) * 64 >= kBlock * kChunksPerRow;
        uint32_t off = fill_off[op];
        const int key = (int)(off / kRowBytes);
        if (key >= lim) off -= (uint32_t)((key - (lim - 1)) * kRowBytes);
        __builtin_amdgcn_global_load_lds((const void*)((is_v ? vb : kb) + off),
                                         (__attribute__((address_space(3))) void*)(stage + (op * 2 + w) * 1024),
                                         16, 0, 0);
      }
    }
  };

  f32x16 o[kTilesD];
#pragma unroll
  for (int dt = 0; dt < kTilesD; ++dt) o[dt] = f32x16{};
  float m_use = -__builtin_inff();  // exponent offset in use (log2 units)
  float l_run = 0.0f;               // this half-wave's share of the denominator

  auto compute = [&](int j, const uint8_t* stage, bool first) {
    const uint8_t* ks = stage;
    const uint8_t* vs = stage + kTileBytes;
    // S^T = K . Q^T for key halves t = 0, 1: all K operands are read first, then
    // the two independent accumulation chains are interleaved.
    u32x4 ka[2][kStepsD];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < kStepsD; ++c)
        ka[t][c] = *(const u32x4*)(ks + k_chunk_offset<D>(32 * t + n, 2 * c + h));
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < kStepsD; ++c)
#pragma unroll
      for (int t = 0; t < 2; ++t) s[t] = E::mfma(ka[t][c], qop[c], s[t]);
    if (j == i) {  // diagonal block: key position must not exceed query position
      const int qpos = 32 * w + n;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kpos = 32 * t + 16 * (r >> 3) + 8 * h + (r & 7);
          if (kpos > qpos) s[t][r] = -__builtin_inff();
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = max_with_other_half(mx) * scale_log2;
    const bool grow = mx > m_use + kRescaleSlack;
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m_use;
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      m_use = m_new;
      if (!first) {  // before the first block O and l are still zero
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kTilesD; ++dt) o[dt] *= alpha;
      }
    }
    u32x4 pb[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * gg + 2 * x], scale_log2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * gg + 2 * x + 1], scale_log2, -m_use));
          pb[2 * t + gg][x] = E::pack(p0, p1);
        }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int x = 0; x < 4; ++x) l_run = E::add_pair(pb[c][x], l_run);
    // O^T += V^T . P^T; V^T operands come from row-major V through transposing reads:
    // lane (group g, index gi) gets keys kb .. kb+3 of head dim 32dt + 16(g&1) + gi.
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) {
      const int dchunk = 4 * dt + 2 * (g & 1) + ((gi & 3) >> 1);
      const int dbyte = 8 * (gi & 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 a;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = 16 * c + 8 * (g >> 1) + 4 * t + (gi >> 2);
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vs + v_chunk_offset<D>(r, dchunk) + dbyte));
          const u32x2 xx = __builtin_bit_cast(u32x2, x);
          a[2 * t] = xx[0];
          a[2 * t + 1] = xx[1];
        }
        o[dt] = E::mfma(a, pb[c], o[dt]);
      }
    }
  };

  int j = next_block(-1);
  if (j >= 0) {
    fill(j, stage0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    bool first = true;
    while (true) {
      int jn = next_block(j);
      if (jn >= 0) fill(jn, stage1);
      compute(j, stage0, first);
      first = false;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (jn < 0) break;
      j = jn;
      jn = next_block(j);
      if (jn >= 0) fill(jn, stage0);
      compute(j, stage1, false);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (jn < 0) break;
      j = jn;
    }
  }

  // Epilogue: O / l, rounded to the input type.  Rows with no visible key get 0.
  const float l_tot = sum_with_other_half(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < S) {
    uint16_t* orow = out + lane_off + (int64_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        u32x2 val;
        val[0] = E::pack(o[dt][4 * gg + 0] * inv, o[dt][4 * gg + 1] * inv);
        val[1] = E::pack(o[dt][4 * gg + 2] * inv, o[dt][4 * gg + 3] * inv);
        *(u32x2*)(orow + 32 * dt + 8 * gg + 4 * h) = val;
      }
  }
}

template <int D, bool BF16>
hipError_t launch_typed(const void* q, const void* k, const void* v, void* out, int64_t lanes,
                        int64_t S, const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                        float scale_log2, hipStream_t stream) {
  const int64_t nb = (S + kBlock - 1) / kBlock;
  // Keep grid * block below 2^32 work-items per launch: split over lanes.
  const int64_t max_wg = (int64_t(1) << 31) / kThreads;
  const int64_t lanes_per_launch = max_wg / nb > 0 ? max_wg / nb : 1;
  for (int64_t l0 = 0; l0 < lanes; l0 += lanes_per_launch) {
    const int64_t nl = lanes - l0 < lanes_per_launch ? lanes - l0 : lanes_per_launch;
    hipLaunchKernelGGL((attention_fwd_kernel<D, BF16>), dim3((unsigned)(nl * nb)), dim3(kThreads), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (uint16_t*)out, row_ptr, col_idx, nnz, (int)S, (int)nb, l0, scale_log2);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attention_fwd(const void* q, const void* k, const void* v, void* out, bool bf16,
                                int64_t lanes, int64_t S, int D, const int32_t* row_ptr,
                                const int32_t* col_idx, int64_t nnz, float scale_log2,
                                hipStream_t stream) {
  if (D == 64) {
    return bf16 ? launch_typed<64, true>(q, k, v, out, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream)
                : launch_typed<64, false>(q, k, v, out, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream);
  }
  return bf16 ? launch_typed<128, true>(q, k, v, out, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream)
              : launch_typed<128, false>(q, k, v, out, lanes, S, row_ptr, col_idx, nnz, scale_log2, stream);
}

}  // namespace tsa
