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

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void attention_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t nnz,
    int S, int nb, int64_t lane_base, float scale_log2) {
  using E = Elem<BF16>;
  constexpr int kStepsD = D / 16;           // 16-deep steps of Q.K^T
  constexpr int kTilesD = D / 32;           // 32-row tiles of O^T
  constexpr int kRowBytes = D * 2;          // bytes per K row in LDS
  constexpr int kChunksPerRow = D / 8;      // 16-byte chunks per K row
  constexpr int kLoads = kBlock * D / 8 / kThreads;  // 16-byte loads per thread per tile
  constexpr int kVPairs = kLoads / 4;       // (4 keys x 8 dims) V pieces per thread

  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kBlock * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_vt[D * kBlock * 2];

  const int tid = threadIdx.x;
  const int w = tid >> 6;   // wave
  const int l = tid & 63;   // lane in wave
  const int h = l >> 5;     // half-wave
  const int n = l & 31;     // query column within the wave's 32 rows

  // Workgroup -> (lane, query block).  Hardware places workgroup b on XCD b % 8.
  const uint32_t G = gridDim.x;
  const uint32_t bid = blockIdx.x;
  const uint32_t logical = (G % 8u == 0u) ? (bid % 8u) * (G / 8u) + bid / 8u : bid;
  const int64_t lane = lane_base + logical / (uint32_t)nb;
  const int i = nb - 1 - (int)(logical % (uint32_t)nb);

  const int64_t lane_off = lane * (int64_t)S * D;
  const uint16_t* qg = q + lane_off;
  const uint16_t* kg = k + lane_off;
  const uint16_t* vg = v + lane_off;
  uint16_t* og = out + lane_off;

  // Q^T operands: lane holds query row qrow, dims 16c + 8h .. +7 for step c.
  const int qrow = i * kBlock + 32 * w + n;
  u32x4 qop[kStepsD];
#pragma unroll
  for (int c = 0; c < kStepsD; ++c) {
    qop[c] = (qrow < S) ? *(const u32x4*)(qg + (int64_t)qrow * D + 16 * c + 8 * h) : u32x4{0, 0, 0, 0};
  }

  // CSR row bounds, clamped to the readable entries.
  int64_t p = row_ptr[i];
  int64_t end = row_ptr[i + 1];
  p = p < 0 ? 0 : (p > nnz ? nnz : p);
  end = end < p ? p : (end > nnz ? nnz : end);
  // Next accepted key block after `last` (strictly ascending, within 0..i), or -1.
  auto next_block = [&](int last) -> int {
    while (p < end) {
      const int c = col_idx[p++];
      if (c > last && c <= i) return c;
    }
    return -1;
  };

  u32x4 kreg[kLoads];
  u32x4 vreg[kLoads];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int id = it * kThreads + tid;
      const int row = id / kChunksPerRow, cb = id % kChunksPerRow;
      const int grow = j * kBlock + row;
      kreg[it] = (grow < S) ? *(const u32x4*)(kg + (int64_t)grow * D + 8 * cb) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int pi = 0; pi < kVPairs; ++pi) {
      const int id = pi * kThreads + tid;
      const int a = id & 15, b = id >> 4;  // keys 4a .. 4a+3, dims 8b .. 8b+7
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int grow = j * kBlock + 4 * a + r;
        vreg[pi * 4 + r] = (grow < S) ? *(const u32x4*)(vg + (int64_t)grow * D + 8 * b) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int id = it * kThreads + tid;
      const int row = id / kChunksPerRow, cb = id % kChunksPerRow;
      const int rho = (row & 32) | swap_bits23(row & 31);
      *(u32x4*)(lds_k + rho * kRowBytes + 16 * (cb ^ (rho & 7))) = kreg[it];
    }
#pragma unroll
    for (int pi = 0; pi < kVPairs; ++pi) {
      const int id = pi * kThreads + tid;
      const int a = id & 15, b = id >> 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * b + e;
        const uint32_t r0 = vreg[pi * 4 + 0][e >> 1], r1 = vreg[pi * 4 + 1][e >> 1];
        const uint32_t r2 = vreg[pi * 4 + 2][e >> 1], r3 = vreg[pi * 4 + 3][e >> 1];
        u32x2 val;
        if (e & 1) {
          val[0] = (r0 >> 16) | (r1 & 0xffff0000u);
          val[1] = (r2 >> 16) | (r3 & 0xffff0000u);
        } else {
          val[0] = (r0 & 0xffffu) | (r1 << 16);
          val[1] = (r2 & 0xffffu) | (r3 << 16);
        }
        *(u32x2*)(lds_vt + d * (kBlock * 2) + 16 * ((a >> 1) ^ (d & 7)) + 8 * (a & 1)) = val;
      }
    }
  };

  f32x16 o[kTilesD];
#pragma unroll
  for (int dt = 0; dt < kTilesD; ++dt) o[dt] = f32x16{};
  float m_run = -__builtin_inff();  // running max, in log2 units
  float l_run = 0.0f;               // this half-wave's share of the denominator

  int j = next_block(-1);
  if (j >= 0) load_tile(j);
  while (j >= 0) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();  // tile j is in LDS
    const int j_next = next_block(j);
    if (j_next >= 0) load_tile(j_next);  // in flight during the math below

    // S^T = K . Q^T for key halves t = 0, 1.
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x16{};
      const uint8_t* krow = lds_k + (32 * t + n) * kRowBytes;
#pragma unroll
      for (int c = 0; c < kStepsD; ++c) {
        const u32x4 a = *(const u32x4*)(krow + 16 * ((2 * c + h) ^ (n & 7)));
        s[t] = E::mfma(a, qop[c], s[t]);
      }
    }

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
    mx = max_with_other_half(mx);
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    // P = exp2(s * scale_log2 - m), rounded to the input type; B operands of P.V.
    u32x4 pb[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * g + 2 * x], scale_log2, -m_new));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * g + 2 * x + 1], scale_log2, -m_new));
          pb[2 * t + g][x] = E::pack(p0, p1);
        }
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int x = 0; x < 4; ++x) l_run = E::add_pair(pb[c][x], l_run);

    if (__builtin_amdgcn_read_exec() & __ballot(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < kTilesD; ++dt) o[dt] *= alpha;
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt) {
      const uint8_t* vrow = lds_vt + (32 * dt + n) * (kBlock * 2);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 a = *(const u32x4*)(vrow + 16 * ((2 * c + h) ^ (n & 7)));
        o[dt] = E::mfma(a, pb[c], o[dt]);
      }
    }
    j = j_next;
  }

  // Epilogue: O / l, rounded to the input type.  Rows with no visible key get 0.
  const float l_tot = sum_with_other_half(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < S) {
    uint16_t* orow = og + (int64_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < kTilesD; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 val;
        val[0] = E::pack(o[dt][4 * g + 0] * inv, o[dt][4 * g + 1] * inv);
        val[1] = E::pack(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
        *(u32x2*)(orow + 32 * dt + 8 * g + 4 * h) = val;
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
