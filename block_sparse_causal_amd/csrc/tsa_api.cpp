// C ABI of libtsa: argument checking, error reporting and dispatch to the HIP
// launchers.  Every check that needs no GPU runs before any HIP call, so the
// validation paths are usable (and tested) on hosts without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/tsa.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return TSA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TSA_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

// The pointer must be device (or managed) memory that lives on the current device.
int check_device_ptr(const void* p, const char* name) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipPointerAttribute_t attr;
  e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return fail(TSA_ERR_DEVICE, "%s is not a HIP allocation", name);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(TSA_ERR_DEVICE, "%s is not device memory", name);
  if (attr.device != dev)
    return fail(TSA_ERR_DEVICE, "%s lives on device %d, current device is %d", name, attr.device,
                dev);
  return TSA_OK;
}

// Block sizes the refinement accepts: multiples of the kernels' 64-row block.
bool block_ok(int32_t block) {
  return block >= TSA_BLOCK && block <= TSA_MAX_SCHEDULE_BLOCK && block % TSA_BLOCK == 0;
}

// Block sizes the schedule builder accepts: those, and 32-row blocks, which the
// forward takes directly.
bool build_block_ok(int32_t block) { return block == TSA_SUB_BLOCK || block_ok(block); }

int64_t row_cap(int32_t sink, int32_t local_radius, int32_t topk) {
  return (int64_t)sink + (int64_t)local_radius + 1 + (int64_t)topk;
}


// Checks shared by the attention entry points (no GPU call); sets *lanes.
// max_d: the largest head dim the entry point takes (256 for the forward and the
// backward); the others are 32, 64 and 128.  sub_block: the entry point also
// takes schedules over 32-row blocks (the forward and the backward, at head dims
// up to 128).
int check_attention_args(const char* fn, int32_t dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                         int64_t nnz, int32_t block, float sm_scale, int64_t max_d, bool sub_block,
                         int64_t* lanes) {
  if (dtype != TSA_F16 && dtype != TSA_BF16)
    return fail(TSA_ERR_INVALID_ARG, "%s: dtype must be TSA_F16 or TSA_BF16", fn);
  if (B < 0 || H < 0 || S < 0 || nnz < 0)
    return fail(TSA_ERR_INVALID_ARG, "%s: B, H, S and nnz must be >= 0", fn);
  if (block != TSA_BLOCK && !(sub_block && block == TSA_SUB_BLOCK))
    return fail(TSA_ERR_UNSUPPORTED, "%s: block must be %d%s, got %d", fn, TSA_BLOCK,
                sub_block ? " or 32" : "", block);
  if (!(D == 32 || D == 64 || D == 128 || D == 256) || D > max_d)
    return fail(TSA_ERR_UNSUPPORTED, "%s: head dim must be 32, 64, 128%s, got %lld", fn,
                max_d >= 256 ? " or 256" : "", (long long)D);
  if (block == TSA_SUB_BLOCK && !tsa::attention_fwd_duo_supported((int)D, S))
    return fail(TSA_ERR_UNSUPPORTED,
                "%s: 32-row blocks need head dim 32, 64 or 128 and S <= %lld, got D=%lld S=%lld",
                fn, (long long)65535 * 128, (long long)D, (long long)S);
  if (std::isnan(sm_scale) || std::isinf(sm_scale))
    return fail(TSA_ERR_INVALID_ARG, "%s: sm_scale must be finite", fn);
  if (S > INT32_MAX - TSA_BLOCK) return fail(TSA_ERR_SHAPE, "%s: S=%lld too large", fn, (long long)S);
  if (B > 0 && H > INT64_MAX / B) return fail(TSA_ERR_SHAPE, "%s: B*H overflows", fn);
  *lanes = B * H;
  if (*lanes > 0 && S > 0 && *lanes > INT64_MAX / (S * D))
    return fail(TSA_ERR_SHAPE, "%s: B*H*S*D overflows", fn);
  return TSA_OK;
}

// lse_required: the entry point returns lse (a NULL lse is then an error).
int attention_fwd(const char* fn, const void* q, const void* k, const void* v, void* out, float* lse,
                  bool lse_required, int32_t dtype, int64_t B, int64_t H, int64_t S, int64_t D, const int32_t* row_ptr,
                  const int32_t* col_idx, int64_t nnz, int32_t block, float sm_scale, void* stream) {
  int64_t lanes = 0;
  int rc = check_attention_args(fn, dtype, B, H, S, D, nnz, block, sm_scale, 256, true, &lanes);
  if (rc != TSA_OK) return rc;
  if (lanes == 0 || S == 0) return ok();  // empty problem: nothing to read or write
  if (!q || !k || !v || !out || !row_ptr || (nnz > 0 && !col_idx) || (lse_required && !lse))
    return fail(TSA_ERR_INVALID_ARG, "%s: NULL pointer argument", fn);
  for (const void* p : {q, k, v, (const void*)out})
    if (((uintptr_t)p) % 16 != 0)
      return fail(TSA_ERR_INVALID_ARG, "%s: q, k, v and out must be 16-byte aligned", fn);
  if (lse && ((uintptr_t)lse) % 4 != 0)
    return fail(TSA_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", fn);
  const size_t bytes = (size_t)(lanes * S * D) * 2;
  const size_t lse_bytes = (size_t)(lanes * S) * 4;
  const char* o0 = (const char*)out;
  const char* l0 = (const char*)lse;
  const char* ins[3] = {(const char*)q, (const char*)k, (const char*)v};
  for (const char* p : ins) {
    if (o0 < p + bytes && p < o0 + bytes)
      return fail(TSA_ERR_INVALID_ARG, "%s: out overlaps an input", fn);
    if (lse && l0 < p + bytes && p < l0 + lse_bytes)
      return fail(TSA_ERR_INVALID_ARG, "%s: lse overlaps an input", fn);
  }
  if (lse && l0 < o0 + bytes && o0 < l0 + lse_bytes)
    return fail(TSA_ERR_INVALID_ARG, "%s: lse overlaps out", fn);
  if ((rc = check_device_ptr(q, "q")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(k, "k")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(v, "v")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(out, "out")) != TSA_OK) return rc;
  if (lse && (rc = check_device_ptr(lse, "lse")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(row_ptr, "row_ptr")) != TSA_OK) return rc;
  if (nnz > 0 && (rc = check_device_ptr(col_idx, "col_idx")) != TSA_OK) return rc;
  const double scale = sm_scale > 0.0f ? (double)sm_scale : 1.0 / std::sqrt((double)D);
  const float scale_log2 = (float)(scale * 1.4426950408889634);  // log2(e)
  hipError_t e = tsa::launch_attention_fwd(q, k, v, out, lse, dtype == TSA_BF16, lanes, S, (int)D,
                                           block, row_ptr, col_idx, nnz, scale_log2,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

}  // namespace

extern "C" {

int tsa_version(void) { return 100; }

const char* tsa_last_error(void) { return g_last_error.c_str(); }

int64_t tsa_schedule_max_nnz(int64_t nb, int32_t sink, int32_t local_radius, int32_t topk) {
  if (nb < 0 || sink < 0 || local_radius < 0 || topk < 0) {
    fail(TSA_ERR_INVALID_ARG, "tsa_schedule_max_nnz: arguments must be >= 0");
    return -1;
  }
  const int64_t cap = row_cap(sink, local_radius, topk);
  // rows i < cap hold i + 1 entries; the remaining rows hold cap entries
  const int64_t full = nb < cap ? nb : cap;
  return full * (full + 1) / 2 + (nb - full) * cap;
}

size_t tsa_build_schedule_workspace_bytes(int64_t S, int64_t D, int32_t block) {
  if (S < 0 || D <= 0 || !build_block_ok(block)) return 0;
  const int64_t nb = (S + block - 1) / block;
  if (nb > TSA_MAX_SCHEDULE_BLOCKS) return 0;
  return tsa::schedule_workspace_bytes(nb, D) + 256;
}

int tsa_build_schedule(const void* keys, int32_t dtype, int64_t S, int64_t D, int32_t block,
                       int32_t sink, int32_t local_radius, int32_t topk, int32_t* row_ptr,
                       int32_t* col_idx, int64_t col_capacity, double* salience, void* workspace,
                       size_t workspace_bytes, int64_t* nnz_host, void* stream) {
  return tsa_build_schedule_ex(keys, dtype, S, D, block, sink, local_radius, topk, TSA_TOPK_GLOBAL,
                               row_ptr, col_idx, col_capacity, salience, workspace, workspace_bytes,
                               nnz_host, stream);
}

namespace {

// Checks of a schedule build that need no GPU call, except the workspace's.
int check_build_args(const void* keys, int32_t dtype, int64_t S, int64_t D, int32_t block,
                     int32_t sink, int32_t local_radius, int32_t topk, int32_t topk_scope,
                     int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity) {
  if (topk_scope != TSA_TOPK_GLOBAL && topk_scope != TSA_TOPK_PER_ROW)
    return fail(TSA_ERR_INVALID_ARG,
                "tsa_build_schedule: topk_scope must be TSA_TOPK_GLOBAL or TSA_TOPK_PER_ROW, got %d",
                topk_scope);
  if (dtype != TSA_F16 && dtype != TSA_BF16)
    return fail(TSA_ERR_INVALID_ARG, "tsa_build_schedule: dtype must be TSA_F16 or TSA_BF16");
  if (S < 0 || D <= 0)
    return fail(TSA_ERR_INVALID_ARG, "tsa_build_schedule: need S >= 0 and D > 0 (S=%lld D=%lld)",
                (long long)S, (long long)D);
  if (sink < 0 || local_radius < 0 || topk < 0)
    return fail(TSA_ERR_INVALID_ARG,
                "tsa_build_schedule: sink, local_radius and topk must be >= 0 (%d, %d, %d)", sink,
                local_radius, topk);
  if (!build_block_ok(block))
    return fail(TSA_ERR_UNSUPPORTED,
                "tsa_build_schedule: block must be 32 or a multiple of %d up to %d, got %d",
                TSA_BLOCK, TSA_MAX_SCHEDULE_BLOCK, block);
  const int64_t nb = (S + block - 1) / block;
  if (nb > TSA_MAX_SCHEDULE_BLOCKS)
    return fail(TSA_ERR_UNSUPPORTED, "tsa_build_schedule: %lld blocks exceed the limit of %d",
                (long long)nb, TSA_MAX_SCHEDULE_BLOCKS);
  if (D > (int64_t(1) << 20))
    return fail(TSA_ERR_SHAPE, "tsa_build_schedule: D=%lld too large", (long long)D);
  if (row_ptr == nullptr) return fail(TSA_ERR_INVALID_ARG, "tsa_build_schedule: row_ptr is NULL");
  const int64_t need = tsa_schedule_max_nnz(nb, sink, local_radius, topk);
  if (col_capacity < need)
    return fail(TSA_ERR_SCHEDULE, "tsa_build_schedule: col_capacity %lld < required %lld",
                (long long)col_capacity, (long long)need);
  if (need > INT32_MAX)
    return fail(TSA_ERR_SHAPE, "tsa_build_schedule: schedule would exceed int32 offsets");
  if (nb > 0) {
    if (keys == nullptr || col_idx == nullptr)
      return fail(TSA_ERR_INVALID_ARG, "tsa_build_schedule: keys and col_idx must be non-NULL");
    if (((uintptr_t)keys) % 2 != 0)
      return fail(TSA_ERR_INVALID_ARG, "tsa_build_schedule: keys must be 2-byte aligned");
  }
  return TSA_OK;
}

// Device checks of the build's pointers (the workspace's are the caller's).
int check_build_ptrs(const void* keys, int64_t nb, int32_t* row_ptr, int32_t* col_idx,
                     double* salience) {
  int rc;
  if ((rc = check_device_ptr(row_ptr, "row_ptr")) != TSA_OK) return rc;
  if (nb > 0) {
    if ((rc = check_device_ptr(keys, "keys")) != TSA_OK) return rc;
    if ((rc = check_device_ptr(col_idx, "col_idx")) != TSA_OK) return rc;
    if (salience && (rc = check_device_ptr(salience, "salience")) != TSA_OK) return rc;
  }
  return TSA_OK;
}

}  // namespace

int tsa_build_schedule_ex(const void* keys, int32_t dtype, int64_t S, int64_t D, int32_t block,
                          int32_t sink, int32_t local_radius, int32_t topk, int32_t topk_scope,
                          int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                          double* salience, void* workspace, size_t workspace_bytes,
                          int64_t* nnz_host, void* stream) {
  int rc = check_build_args(keys, dtype, S, D, block, sink, local_radius, topk, topk_scope, row_ptr,
                            col_idx, col_capacity);
  if (rc != TSA_OK) return rc;
  const int64_t nb = (S + block - 1) / block;
  if (nb > 0) {
    if (workspace == nullptr)
      return fail(TSA_ERR_INVALID_ARG, "tsa_build_schedule: workspace must be non-NULL");
    const size_t ws = tsa::schedule_workspace_bytes(nb, D);
    if (workspace_bytes < ws)
      return fail(TSA_ERR_INVALID_ARG, "tsa_build_schedule: workspace of %zu bytes < required %zu",
                  workspace_bytes, ws);
    if (((uintptr_t)workspace) % 256 != 0)
      return fail(TSA_ERR_INVALID_ARG, "tsa_build_schedule: workspace must be 256-byte aligned");
  }
  if ((rc = check_build_ptrs(keys, nb, row_ptr, col_idx, salience)) != TSA_OK) return rc;
  if (nb > 0 && (rc = check_device_ptr(workspace, "workspace")) != TSA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = tsa::launch_build_schedule(keys, dtype == TSA_BF16, S, D, block, sink, local_radius,
                                            topk, topk_scope == TSA_TOPK_PER_ROW, row_ptr, col_idx,
                                            col_capacity, salience, workspace, st);
  if (e != hipSuccess) return hip_fail(e, "schedule kernels");
  if (nnz_host) {
    int32_t n = 0;
    e = hipMemcpyAsync(&n, row_ptr + nb, sizeof n, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "reading nnz");
    *nnz_host = n;
  }
  return ok();
}

int tsa_build_schedule_noalloc(const void* keys, int32_t dtype, int64_t S, int64_t D, int32_t block,
                               int32_t sink, int32_t local_radius, int32_t topk, int32_t topk_scope,
                               int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                               double* salience, void* stream) {
  const char* fn = "tsa_build_schedule_noalloc";
  int rc = check_build_args(keys, dtype, S, D, block, sink, local_radius, topk, topk_scope, row_ptr,
                            col_idx, col_capacity);
  if (rc != TSA_OK) return rc;
  const int64_t nb = (S + block - 1) / block;
  const size_t ws = nb > 0 ? tsa::schedule_workspace_bytes(nb, D) : 0;
  if (ws > TSA_NOALLOC_SCRATCH_BYTES)
    return fail(TSA_ERR_UNSUPPORTED,
                "%s: the build needs %zu bytes of workspace, more than the library's fixed %zu "
                "(tsa_build_schedule takes a caller-owned workspace of any size)",
                fn, ws, (size_t)TSA_NOALLOC_SCRATCH_BYTES);
  if ((rc = check_build_ptrs(keys, nb, row_ptr, col_idx, salience)) != TSA_OK) return rc;
  void* scratch = nullptr;
  if (nb > 0) {
    hipError_t e = tsa::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "looking up the builder's device scratch");
  }
  hipError_t e = tsa::launch_build_schedule(keys, dtype == TSA_BF16, S, D, block, sink, local_radius,
                                            topk, topk_scope == TSA_TOPK_PER_ROW, row_ptr, col_idx,
                                            col_capacity, salience, scratch, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "schedule kernels");
  return ok();
}

int tsa_dense_causal_schedule(int64_t nb, int32_t* row_ptr, int32_t* col_idx,
                              int64_t col_capacity, void* stream) {
  if (nb < 0) return fail(TSA_ERR_INVALID_ARG, "tsa_dense_causal_schedule: nb must be >= 0");
  const int64_t need = nb * (nb + 1) / 2;
  if (need > INT32_MAX)
    return fail(TSA_ERR_SHAPE, "tsa_dense_causal_schedule: %lld entries exceed int32 offsets",
                (long long)need);
  if (col_capacity < need)
    return fail(TSA_ERR_SCHEDULE, "tsa_dense_causal_schedule: col_capacity %lld < %lld",
                (long long)col_capacity, (long long)need);
  if (row_ptr == nullptr || (nb > 0 && col_idx == nullptr))
    return fail(TSA_ERR_INVALID_ARG, "tsa_dense_causal_schedule: NULL output");
  int rc;
  if ((rc = check_device_ptr(row_ptr, "row_ptr")) != TSA_OK) return rc;
  if (nb > 0 && (rc = check_device_ptr(col_idx, "col_idx")) != TSA_OK) return rc;
  hipError_t e = tsa::launch_dense_schedule(nb, row_ptr, col_idx, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dense schedule kernel");
  return ok();
}

int64_t tsa_segment_schedule_nnz(int64_t nb, int32_t segment_blocks) {
  if (nb < 0 || segment_blocks < 1) return -1;
  const int64_t L = segment_blocks < nb ? segment_blocks : (nb > 0 ? nb : 1);
  const int64_t q = nb / L, r = nb % L;
  return q * (L * (L + 1) / 2) + r * (r + 1) / 2;
}

int tsa_segment_schedule(int64_t nb, int32_t segment_blocks, int32_t* row_ptr, int32_t* col_idx,
                         int64_t col_capacity, void* stream) {
  if (nb < 0) return fail(TSA_ERR_INVALID_ARG, "tsa_segment_schedule: nb must be >= 0");
  if (segment_blocks < 1)
    return fail(TSA_ERR_INVALID_ARG, "tsa_segment_schedule: segment_blocks must be >= 1, got %d",
                segment_blocks);
  const int64_t need = tsa_segment_schedule_nnz(nb, segment_blocks);
  if (need > INT32_MAX)
    return fail(TSA_ERR_SHAPE, "tsa_segment_schedule: %lld entries exceed int32 offsets",
                (long long)need);
  if (col_capacity < need)
    return fail(TSA_ERR_SCHEDULE, "tsa_segment_schedule: col_capacity %lld < %lld",
                (long long)col_capacity, (long long)need);
  if (row_ptr == nullptr || (nb > 0 && col_idx == nullptr))
    return fail(TSA_ERR_INVALID_ARG, "tsa_segment_schedule: NULL output");
  int rc;
  if ((rc = check_device_ptr(row_ptr, "row_ptr")) != TSA_OK) return rc;
  if (nb > 0 && (rc = check_device_ptr(col_idx, "col_idx")) != TSA_OK) return rc;
  const int64_t L = segment_blocks < nb ? segment_blocks : (nb > 0 ? nb : 1);
  hipError_t e = tsa::launch_segment_schedule(nb, L, row_ptr, col_idx, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "segment schedule kernel");
  return ok();
}

int tsa_scheduled_attention_fwd(const void* q, const void* k, const void* v, void* out,
                                int32_t dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                                const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                int32_t block, float sm_scale, void* stream) {
  return attention_fwd("tsa_scheduled_attention_fwd", q, k, v, out, nullptr, false, dtype, B, H, S, D,
                       row_ptr, col_idx, nnz, block, sm_scale, stream);
}

int tsa_scheduled_attention_fwd_lse(const void* q, const void* k, const void* v, void* out,
                                    float* lse, int32_t dtype, int64_t B, int64_t H, int64_t S,
                                    int64_t D, const int32_t* row_ptr, const int32_t* col_idx,
                                    int64_t nnz, int32_t block, float sm_scale, void* stream) {
  return attention_fwd("tsa_scheduled_attention_fwd_lse", q, k, v, out, lse, true, dtype, B, H, S, D,
                       row_ptr, col_idx, nnz, block, sm_scale, stream);
}

int64_t tsa_refine_schedule_max_nnz(int64_t S, int32_t block, int64_t nnz) {
  if (S < 0 || nnz < 0 || !block_ok(block)) {
    fail(TSA_ERR_INVALID_ARG, "tsa_refine_schedule_max_nnz: need S, nnz >= 0 and a valid block");
    return -1;
  }
  const int64_t m = block / TSA_BLOCK, nb64 = (S + TSA_BLOCK - 1) / TSA_BLOCK;
  const int64_t tri = nb64 * (nb64 + 1) / 2;
  return nnz > tri / (m * m) ? tri : nnz * m * m;
}

int tsa_refine_schedule(int64_t S, int32_t block, const int32_t* row_ptr, const int32_t* col_idx,
                        int64_t nnz, int32_t* row_ptr64, int32_t* col_idx64, int64_t capacity,
                        int64_t* nnz_host, void* stream) {
  const char* fn = "tsa_refine_schedule";
  if (S < 0 || nnz < 0 || capacity < 0)
    return fail(TSA_ERR_INVALID_ARG, "%s: S, nnz and capacity must be >= 0", fn);
  if (!block_ok(block))
    return fail(TSA_ERR_UNSUPPORTED, "%s: block must be a multiple of %d up to %d, got %d", fn,
                TSA_BLOCK, TSA_MAX_SCHEDULE_BLOCK, block);
  const int64_t nb64 = (S + TSA_BLOCK - 1) / TSA_BLOCK;
  if (nb64 > TSA_MAX_REFINED_BLOCKS)
    return fail(TSA_ERR_UNSUPPORTED, "%s: %lld 64-row blocks exceed the limit of %d", fn,
                (long long)nb64, TSA_MAX_REFINED_BLOCKS);
  const int64_t need = tsa_refine_schedule_max_nnz(S, block, nnz);
  if (need > INT32_MAX)
    return fail(TSA_ERR_SHAPE, "%s: the refined schedule may exceed int32 offsets", fn);
  if (capacity < need)
    return fail(TSA_ERR_SCHEDULE, "%s: capacity %lld < tsa_refine_schedule_max_nnz = %lld", fn,
                (long long)capacity, (long long)need);
  if (row_ptr == nullptr || row_ptr64 == nullptr || (nnz > 0 && col_idx == nullptr) ||
      (need > 0 && col_idx64 == nullptr))
    return fail(TSA_ERR_INVALID_ARG, "%s: NULL pointer argument", fn);
  int rc;
  if ((rc = check_device_ptr(row_ptr, "row_ptr")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(row_ptr64, "row_ptr64")) != TSA_OK) return rc;
  if (nnz > 0 && (rc = check_device_ptr(col_idx, "col_idx")) != TSA_OK) return rc;
  if (need > 0 && (rc = check_device_ptr(col_idx64, "col_idx64")) != TSA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = tsa::launch_refine_schedule(S, block, row_ptr, col_idx, nnz, row_ptr64, col_idx64,
                                             capacity, st);
  if (e != hipSuccess) return hip_fail(e, "refine kernels");
  if (nnz_host) {
    int32_t n = 0;
    e = hipMemcpyAsync(&n, row_ptr64 + nb64, sizeof n, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "reading nnz");
    *nnz_host = n;
    if (n > capacity)
      return fail(TSA_ERR_SCHEDULE,
                  "%s: the refined schedule needs %lld entries > capacity %lld (rows of the input share "
                  "entries: row_ptr is not non-decreasing); entries past the capacity were not written",
                  fn, (long long)n, (long long)capacity);
  }
  return ok();
}

size_t tsa_schedule_transpose_workspace_bytes(int64_t nb) {
  if (nb <= 0 || nb > TSA_MAX_SCHEDULE_BLOCKS) return 0;
  return tsa::transpose_workspace_bytes(nb);
}

int tsa_schedule_transpose(int64_t nb, const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                           int32_t* col_ptr, int32_t* row_idx, int64_t row_capacity,
                           void* workspace, size_t workspace_bytes, int64_t* nnz_host,
                           void* stream) {
  const char* fn = "tsa_schedule_transpose";
  if (nb < 0 || nnz < 0 || row_capacity < 0)
    return fail(TSA_ERR_INVALID_ARG, "%s: nb, nnz and row_capacity must be >= 0", fn);
  if (nb > TSA_MAX_SCHEDULE_BLOCKS)
    return fail(TSA_ERR_UNSUPPORTED, "%s: %lld blocks exceed the limit of %d", fn, (long long)nb,
                TSA_MAX_SCHEDULE_BLOCKS);
  const int64_t tri = nb * (nb + 1) / 2;
  const int64_t need = nnz < tri ? nnz : tri;
  if (row_capacity < need)
    return fail(TSA_ERR_SCHEDULE, "%s: row_capacity %lld < min(nnz, nb*(nb+1)/2) = %lld", fn,
                (long long)row_capacity, (long long)need);
  if (row_ptr == nullptr || col_ptr == nullptr || (nnz > 0 && col_idx == nullptr) ||
      (need > 0 && row_idx == nullptr))
    return fail(TSA_ERR_INVALID_ARG, "%s: NULL pointer argument", fn);
  if (nb > 0) {
    const size_t ws = tsa::transpose_workspace_bytes(nb);
    if (workspace == nullptr || workspace_bytes < ws)
      return fail(TSA_ERR_INVALID_ARG, "%s: workspace of %zu bytes < required %zu", fn,
                  workspace_bytes, ws);
    if (((uintptr_t)workspace) % 256 != 0)
      return fail(TSA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  }
  int rc;
  if ((rc = check_device_ptr(row_ptr, "row_ptr")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(col_ptr, "col_ptr")) != TSA_OK) return rc;
  if (nnz > 0 && (rc = check_device_ptr(col_idx, "col_idx")) != TSA_OK) return rc;
  if (need > 0 && (rc = check_device_ptr(row_idx, "row_idx")) != TSA_OK) return rc;
  if (nb > 0 && (rc = check_device_ptr(workspace, "workspace")) != TSA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = tsa::launch_schedule_transpose(nb, row_ptr, col_idx, nnz, col_ptr, row_idx,
                                                row_capacity, workspace, st);
  if (e != hipSuccess) return hip_fail(e, "transpose kernels");
  if (nnz_host) {
    int32_t n = 0;
    e = hipMemcpyAsync(&n, col_ptr + nb, sizeof n, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "reading nnz");
    *nnz_host = n;
    if (n > row_capacity)
      return fail(TSA_ERR_SCHEDULE,
                  "%s: the column view has %lld entries > row_capacity %lld (rows share entries: "
                  "row_ptr is not non-decreasing); entries past the capacity were not written",
                  fn, (long long)n, (long long)row_capacity);
  }
  return ok();
}

// Backward workspace: each row's (lse, Delta) as float2 [lanes, S], then, from
// the next 16-byte boundary, the column ranking [nb] int32.
static int64_t bwd_order_offset(int64_t lanes, int64_t S) { return (lanes * S * 8 + 15) / 16 * 16; }
static int64_t bwd_workspace(int64_t lanes, int64_t S) {
  return bwd_order_offset(lanes, S) + ((S + 63) / 64) * 4;
}

size_t tsa_scheduled_attention_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S) {
  if (B < 0 || H < 0 || S < 0) return 0;
  if (B > 0 && H > INT64_MAX / B) return 0;
  const int64_t lanes = B * H;
  if (lanes > 0 && S > (INT64_MAX / 2) / 8 / lanes) return 0;
  return (size_t)bwd_workspace(lanes, S);
}

int tsa_scheduled_attention_bwd(const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, int32_t dtype, int64_t B,
                                int64_t H, int64_t S, int64_t D, const int32_t* row_ptr,
                                const int32_t* col_idx, int64_t nnz, const int32_t* col_ptr,
                                const int32_t* row_idx, int64_t nnz_t, int32_t block,
                                float sm_scale, void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const char* fn = "tsa_scheduled_attention_bwd";
  int64_t lanes = 0;
  int rc = check_attention_args(fn, dtype, B, H, S, D, nnz, block, sm_scale, 256, true, &lanes);
  if (rc != TSA_OK) return rc;
  if (nnz_t < 0) return fail(TSA_ERR_INVALID_ARG, "%s: nnz_t must be >= 0", fn);
  if (lanes == 0 || S == 0) return ok();
  if (!q || !k || !v || !out || !dout || !lse || !row_ptr || (nnz > 0 && !col_idx) || !col_ptr ||
      (nnz_t > 0 && !row_idx) || !dq || !dk || !dv || !workspace)
    return fail(TSA_ERR_INVALID_ARG, "%s: NULL pointer argument", fn);
  for (const void* p : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (((uintptr_t)p) % 16 != 0)
      return fail(TSA_ERR_INVALID_ARG, "%s: q, k, v, out, dout, dq, dk and dv must be 16-byte aligned", fn);
  if (((uintptr_t)lse) % 4 != 0 || ((uintptr_t)workspace) % 16 != 0)
    return fail(TSA_ERR_INVALID_ARG, "%s: lse must be 4-byte and workspace 16-byte aligned", fn);
  const size_t ws = (size_t)bwd_workspace(lanes, S);
  if (workspace_bytes < ws)
    return fail(TSA_ERR_INVALID_ARG, "%s: workspace of %zu bytes < required %zu", fn,
                workspace_bytes, ws);
  const size_t bytes = (size_t)(lanes * S * D) * 2;
  const char* ins[6] = {(const char*)q, (const char*)k, (const char*)v, (const char*)out,
                        (const char*)dout, (const char*)lse};
  const size_t in_bytes[6] = {bytes, bytes, bytes, bytes, bytes, (size_t)(lanes * S * 4)};
  const char* outs[4] = {(const char*)dq, (const char*)dk, (const char*)dv, (const char*)workspace};
  const size_t out_bytes[4] = {bytes, bytes, bytes, ws};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (outs[a] < ins[b] + in_bytes[b] && ins[b] < outs[a] + out_bytes[a])
        return fail(TSA_ERR_INVALID_ARG, "%s: an output or the workspace overlaps an input", fn);
    for (int b = a + 1; b < 4; ++b)
      if (outs[a] < outs[b] + out_bytes[b] && outs[b] < outs[a] + out_bytes[a])
        return fail(TSA_ERR_INVALID_ARG, "%s: dq, dk, dv and the workspace must not overlap", fn);
  }
  const char* names[] = {"q", "k", "v", "out", "dout", "lse"};
  for (int b = 0; b < 6; ++b)
    if ((rc = check_device_ptr(ins[b], names[b])) != TSA_OK) return rc;
  if ((rc = check_device_ptr(dq, "dq")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(dk, "dk")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(dv, "dv")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(workspace, "workspace")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(row_ptr, "row_ptr")) != TSA_OK) return rc;
  if (nnz > 0 && (rc = check_device_ptr(col_idx, "col_idx")) != TSA_OK) return rc;
  if ((rc = check_device_ptr(col_ptr, "col_ptr")) != TSA_OK) return rc;
  if (nnz_t > 0 && (rc = check_device_ptr(row_idx, "row_idx")) != TSA_OK) return rc;
  tsa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
  a.row_ptr = row_ptr; a.col_idx = col_idx; a.nnz = nnz;
  a.col_ptr = col_ptr; a.row_idx = row_idx; a.nnz_t = nnz_t;
  a.dq = dq; a.dk = dk; a.dv = dv; a.stats = workspace;
  a.col_order = (int32_t*)((char*)workspace + bwd_order_offset(lanes, S));
  a.bf16 = dtype == TSA_BF16;
  a.lanes = lanes; a.S = S; a.D = (int)D; a.block = block;
  const double scale = sm_scale > 0.0f ? (double)sm_scale : 1.0 / std::sqrt((double)D);
  a.scale = (float)scale;
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  hipError_t e = tsa::launch_attention_bwd(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention backward kernels");
  return ok();
}

}  // extern "C"
