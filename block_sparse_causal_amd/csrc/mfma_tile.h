// Device building blocks shared by the attention kernels for gfx950 (CDNA4):
// the 32x32x16 MFMA per element type, the row swizzles of 64-row tiles in LDS,
// asm wrappers for loads whose waits are placed by hand, the direct
// global->LDS tile copy and the ring barrier.  Internal to libtsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {
namespace tile {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;
// Fourth word of a raw buffer resource on gfx9-family targets (32-bit data
// format, no swizzle, no index stride): loads past the size read as zero.
[[maybe_unused]] constexpr int kBufferWord3 = 0x00020000;

// Element-type specific pieces: the MFMA, the fp32 -> 2 x 16-bit pack (round to
// nearest even), a pairwise add of a packed pair into an fp32 sum and the dot
// product of two packed pairs.
template <bool BF16>
struct Elem;

template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // 16x16x32 MFMA (A 16 x 32, B 32 x 16, C 16 x 16)
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static constexpr uint32_t kOnePair = 0x3C003C00u;  // two 1.0 halves
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float add_pair(uint32_t p, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
  }
  // acc + a.lo * b.lo + a.hi * b.hi for two packed pairs
  static __device__ __forceinline__ float dot_pair(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
  }
};

template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static constexpr uint32_t kOnePair = 0x3F803F80u;  // two 1.0 bf16 values
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float add_pair(uint32_t p, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
  }
  static __device__ __forceinline__ float dot_pair(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc,
                                           false);
  }
};

// A operand of a 16x16x32 MFMA that sums, for the query of each lane, a P^T
// register group taken as its B operand.  A P^T group (8 values per lane: keys
// 8h .. 8h+7 of a 16-key chunk for query l % 32, h = l / 32) read as the B
// operand puts query 16 (kg % 2) + c in column c of k-group kg = l / 16.  With
// A[m][k] = 1 exactly when (k / 8) % 2 == (m / 4) % 2, row m of C sums the
// k-groups of parity (m / 4) % 2, and C's lane l (rows 4 (l / 16) .. +3, column
// l % 16) then holds the chunk's sum for query l % 32 over both h.
template <typename E>
__device__ __forceinline__ u32x4 row_sum_selector(int l) {
  const uint32_t v = ((l >> 4) & 1) == ((l >> 2) & 1) ? E::kOnePair : 0u;
  return u32x4{v, v, v, v};
}

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
// K rows use chunk ^ k_swizzle(r); V rows use chunk ^ 2*t(r & 3), where t spreads
// the four key rows that one transposing read touches over distinct bank groups.
// K-layout swizzle: 16-byte chunk c of data row r sits at chunk c ^ k_swizzle(r).
// gfx950's LDS has 64 four-byte banks.  A row-wise operand read has 16 lanes
// reading one 16-byte chunk each from 16 consecutive rows; a transposing read
// has 32 lanes reading four chunks (64 bytes) from each of 4 consecutive rows.
// Rows of 2D bytes start at bank 16 (r mod 128 / D) for D < 128 and at bank 0
// from D = 128 on, so the XOR value must differ between same-bank-offset rows:
//   D = 32:  the 4 rows of a bank offset among 16: bits 2-3 of r;
//   D = 64:  8 same-parity rows among 16 (bits 1-3 of r), with rows r and r + 2
//            of a 4-row group 4 chunks apart (bit 1 -> XOR bit 2);
//   D >= 128: 16 rows (bits 0-3), the 4 rows of a group 4 chunks apart.
// The value never exceeds the row's chunk count minus one.
template <int D>
__device__ __forceinline__ int k_swizzle(int r) {
  if constexpr (D == 32) return (r >> 2) & 3;
  else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int k_chunk_offset(int r, int c) {
  return r * (D * 2) + 16 * (c ^ k_swizzle<D>(r));
}
// At D = 32 the four rows one transposing read touches already sit 64 bytes
// apart, in distinct bank groups, so V rows are not swizzled.
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  if (D == 32) return 0;
  if (D == 64) return 2 * (r & 3);
  const int t = (0x6530 >> (4 * (r & 3))) & 0xF;  // 0, 3, 5, 6
  return 2 * t;
}
template <int D>
__device__ __forceinline__ int v_chunk_offset(int r, int c) {
  return r * (D * 2) + 16 * (c ^ v_swizzle<D>(r));
}

// s_waitcnt immediate that waits until at most `n` vector memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_wait(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

// Transposing LDS read (ds_read_b64_tr_b16), issued through asm so that the
// compiler does not order it behind the in-flight global->LDS copies of other
// stages; the values may only be used after lds_wait_all().  Within each
// 16-lane group, lane i receives element i % 4 of the 8-byte pieces addressed by
// lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4.
template <int kOffset>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOffset));
  return r;
}
// 16-byte global load issued through asm, so that the compiler does not wait
// for it (and with it for every later copy) at each use.  The value may only be
// used after an s_waitcnt that covers it.
template <int kOffset>
__device__ __forceinline__ u32x4 global_load_b128(const uint16_t* p) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(r) : "v"(p), "i"(kOffset) : "memory");
  return r;
}
// 16-byte LDS read, issued through asm for the same reason.
template <int kOffset>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOffset));
  return r;
}
// The B operands of one 32-query column: 16 bytes (dims 16c + 8h .. +7) for each
// c < C from one row, through global_load_b128 at compile-time offsets.
template <int C>
__device__ __forceinline__ void load_row_operands(u32x4* dst, const uint16_t* p) {
  if constexpr (C > 0) {
    load_row_operands<C - 1>(dst, p);
    dst[C - 1] = global_load_b128<32 * (C - 1)>(p);
  }
}
// Wait for every outstanding LDS read of this wave; the values pass through the
// asm statement so that no use of them can be scheduled above the wait.
template <typename T, int N>
__device__ __forceinline__ void lds_wait_all(T (&x)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int e = 0; e < N; ++e) asm volatile("" : "+v"(x[e]));
}

// Copy one K tile and one V tile (`bytes` each, the rows that exist) into a
// stage of [K tile | V tile] with buffer loads straight into LDS: op o of wave
// w moves 1 KB piece (o * kWaves + w), 16 bytes per lane from byte offset
// off[o] of its tile's rows; the piece lies in the V half exactly when o >=
// kOpsPerTile.  Loads past `bytes` read as zero.
// (The host pass of the kernel never runs this; the buffer builtins exist only
// in the device pass.)
template <int kOps, int kOpsPerTile, int kWaves>
__host__ __device__ __forceinline__ void copy_block_to_lds(const uint16_t* kb, const uint16_t* vb,
                                                           int bytes, const uint32_t (&off)[kOps],
                                                           uint8_t* stage, int w) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, bytes, kBufferWord3);
#pragma unroll
  for (int op = 0; op < kOps; ++op)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op >= kOpsPerTile ? rv : rk,
                                             (__attribute__((address_space(3))) void*)(stage + (op * kWaves + w) * 1024),
                                             16, off[op], 0, 0, 0);
#endif
}

// Workgroup barrier for the K/V ring.  Each wave has already waited (s_waitcnt)
// for exactly the copies the next step reads, so the barrier must not drain the
// copies still in flight, which a fenced __syncthreads() would.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace tile
}  // namespace tsa
