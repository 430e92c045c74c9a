// Internal launchers of libtsa (not part of the C ABI).  Each returns the
// hipError_t of its launch; argument checking is done by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {

// Scheduled attention forward over `lanes` lanes of [S, D] (D = 32, 64, 128 or
// 256) with a CSR over blocks of `block` rows (64, or 32 at D <= 128); lse
// [lanes, S] (natural log of each row's denominator) is written when not null.
hipError_t launch_attention_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                                bool bf16, int64_t lanes, int64_t S, int D, int block,
                                const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                float scale_log2, hipStream_t stream);

// The same forward at head dims 32, 64 and 128 with two adjacent 64-row query
// blocks per workgroup of four waves (attention_fwd_duo.hip); with block 32 the
// CSR is over 32-row blocks and each wave walks the row of its 32 queries.
// Supported when D is one of those and the grid's pair count fits (S <= 8 M).
bool attention_fwd_duo_supported(int D, int64_t S);
hipError_t launch_attention_fwd_duo(const void* q, const void* k, const void* v, void* out, float* lse,
                                    bool bf16, int64_t lanes, int64_t S, int D, int block,
                                    const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                    float scale_log2, hipStream_t stream);

// Scheduled attention backward: the dq kernel (CSR rows, also writes the per-row
// statistics) and then the dkdv kernel (columns of the transposed schedule).
struct BwdArgs {
  const void *q, *k, *v, *out, *dout;
  const float* lse;               // [lanes, S], natural log
  const int32_t *row_ptr, *col_idx;
  int64_t nnz;
  const int32_t *col_ptr, *row_idx;
  int64_t nnz_t;
  void *dq, *dk, *dv;
  void* stats;                    // [lanes, S] float2 workspace
  int32_t* col_order;             // [nb] workspace: columns ranked by entry count
  bool bf16;
  int64_t lanes, S;
  int D;
  int block;                      // 64, or 32 (schedules over 32-row blocks)
  float scale, scale_log2;
};
hipError_t launch_attention_bwd(const BwdArgs& args, hipStream_t stream);

// Column view of a CSR schedule (see schedule_transpose.hip).
size_t transpose_workspace_bytes(int64_t nb);
hipError_t launch_schedule_transpose(int64_t nb, const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t nnz, int32_t* col_ptr, int32_t* row_idx,
                                     int64_t row_capacity, void* workspace, hipStream_t stream);

// Schedule builder: centroids -> distances -> MST -> elder rule -> top-k -> CSR.
struct ScheduleWorkspace {
  double* centroids;  // [nb, D]
  double* dist;       // [nb, nb], only when nb > kLdsDistBlocks
};
constexpr int kLdsDistBlocks = 128;  // distance matrix kept in LDS up to this many blocks
size_t schedule_workspace_bytes(int64_t nb, int64_t D);
// Device address (current device) of the library's fixed builder workspace of
// TSA_NOALLOC_SCRATCH_BYTES bytes (see schedule_build.hip).
hipError_t noalloc_scratch(void** ptr);
// block: rows per key block, a positive multiple of 64; nb = ceil(S / block).
hipError_t launch_build_schedule(const void* keys, bool bf16, int64_t S, int64_t D, int block,
                                 int sink, int local_radius, int topk, bool per_row,
                                 int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                 double* salience, void* workspace, hipStream_t stream);

// Refinement of a CSR over blocks of `block` rows (a multiple of 64) to the CSR
// over 64-row blocks that allows exactly the same keys (see schedule_refine.hip).
hipError_t launch_refine_schedule(int64_t S, int block, const int32_t* row_ptr,
                                  const int32_t* col_idx, int64_t nnz, int32_t* row_ptr64,
                                  int32_t* col_idx64, int64_t capacity, hipStream_t stream);

hipError_t launch_dense_schedule(int64_t nb, int32_t* row_ptr, int32_t* col_idx,
                                 hipStream_t stream);
hipError_t launch_segment_schedule(int64_t nb, int64_t segment_blocks, int32_t* row_ptr,
                                   int32_t* col_idx, hipStream_t stream);

}  // namespace tsa
