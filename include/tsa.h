/*
 * tsa.h -- C ABI of libtsa: topology-scheduled block-sparse causal attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the pages "Add topology-derived sparse attention
 * kernel" (triton-lang/kernels pull request 22) and its mirror page, plus the
 * backward pass of the attention, which the pages do not have:
 *   - a forward-only causal attention that consumes a CSR block schedule
 *     (Summary, first bullet), for [S, D] and [B, H, S, D] inputs with one
 *     schedule shared by every batch/head lane (third bullet), whose output has
 *     the input dtype (fourth bullet);
 *   - a schedule builder that takes sink blocks, local-window blocks and the
 *     top-k key blocks ranked by a 0D-persistence salience of the key-block
 *     centroids (second bullet), elder-rule salience as described in the
 *     mirror page's Rust-port commit note, computed from MST edges as in its
 *     schedule.py commit note;
 *   - the dense causal CSR used as the like-for-like baseline (Local benchmark);
 *   - the gradients of the attention with respect to q, k and v over the same
 *     schedule, and the column view of a schedule they gather over.
 *
 * Conventions shared by every entry point
 *   - All functions are callable from C; none throws.  Status: 0 = TSA_OK,
 *     negative = error.  On error nothing has been written to any output and
 *     tsa_last_error() returns a message (thread-local, valid until the next
 *     call on the same thread).
 *   - Arguments are checked before any GPU work (PR page, Summary, fifth bullet:
 *     inputs are validated ahead of the launch): sizes and parameters first (no GPU call),
 *     then every device pointer must be device memory on the current HIP device.
 *   - Device pointers are owned by the caller; libtsa allocates nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is queued on it asynchronously unless a *_host output asks for a value
 *     back, in which case the call waits for the stream.
 *   - Tensors are dense row-major: [S, D] or [B, H, S, D] with D contiguous.
 *     A lane is one (b, h) pair; lane l = b*H + h starts at element l*S*D.
 *   - CSR schedule: row_ptr int32 [nb+1], col_idx int32 [nnz], nb = ceil(S/64).
 *     Row i lists the key blocks query block i visits, strictly ascending,
 *     each in 0..i.
 */
#ifndef TSA_H
#define TSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define TSA_OK 0
#define TSA_ERR_INVALID_ARG (-1) /* null pointer, negative size or parameter, bad dtype */
#define TSA_ERR_UNSUPPORTED (-2) /* unsupported block or head dim, too many blocks */
#define TSA_ERR_SHAPE (-3)       /* sizes that overflow or do not fit together */
#define TSA_ERR_SCHEDULE (-4)    /* CSR arguments inconsistent (nnz, capacity) */
#define TSA_ERR_DEVICE (-5)      /* a pointer is not device memory of the current device */
#define TSA_ERR_HIP (-6)         /* a HIP runtime call or kernel launch failed */

/* Element types of q/k/v/out and of the builder's keys. */
#define TSA_F16 0
#define TSA_BF16 1

/* Block size of the attention kernels (rows per query block and per key block).
 * The schedule builder and tsa_refine_schedule also take schedules over blocks of
 * any multiple of it up to TSA_MAX_SCHEDULE_BLOCK rows; the builder and the
 * forward also take TSA_SUB_BLOCK. */
#define TSA_BLOCK 64
/* The smaller block the forward entry points and the schedule builder also take
 * (head dims 32, 64 and 128): rows per query block and per key block. */
#define TSA_SUB_BLOCK 32
#define TSA_MAX_SCHEDULE_BLOCK 4096
/* Largest number of key blocks the schedule builder accepts (S <= 262144 at block 64). */
#define TSA_MAX_SCHEDULE_BLOCKS 4096
/* Largest number of 64-row blocks tsa_refine_schedule emits (S <= 2^28). */
#define TSA_MAX_REFINED_BLOCKS (1 << 22)

/* Library version, e.g. 100 for 0.1.0. */
int tsa_version(void);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* tsa_last_error(void);

/*
 * Upper bound on the entries the builder can emit for nb query blocks:
 * sum over rows i of min(i + 1, sink + local_radius + 1 + topk).  Host-only.
 * Returns -1 (and sets the error) for negative arguments.
 */
int64_t tsa_schedule_max_nnz(int64_t nb, int32_t sink, int32_t local_radius, int32_t topk);

/*
 * Device workspace, in bytes, that tsa_build_schedule needs for keys [S, D]
 * and the given block size (256-byte aligned start required).  Host-only.
 * Returns 0 for invalid sizes.
 */
size_t tsa_build_schedule_workspace_bytes(int64_t S, int64_t D, int32_t block);

/*
 * Build the topology-derived CSR schedule from one lane of keys.
 * (PR page, Summary, second bullet; mirror page, Rust-port and schedule.py
 * commit notes.)
 *
 *   keys        device, [S, D] of `dtype` (TSA_F16 / TSA_BF16), row-major.
 *               For [B, H, S, D] inputs pass lane (0, 0).
 *   block       rows per block: TSA_SUB_BLOCK (32) or a multiple of 64 up to
 *               TSA_MAX_SCHEDULE_BLOCK.  nb = ceil(S / block); a partial last
 *               block's centroid is the mean of its valid rows.  A schedule over
 *               blocks larger than 64 is handed to the attention entry points
 *               through tsa_refine_schedule; one over 32-row blocks goes to the
 *               forward entry points as it is (block = 32 there).
 *   sink, local_radius, topk   >= 0.  Row i lists every block j <= i with
 *               j < sink, or j >= i - local_radius, or j among the topk blocks
 *               of highest salience (ties: lower index; topk >= nb: all).
 *   Salience: centroids c_j (fp64 mean of the block's keys); the minimum
 *               spanning tree of the complete graph with Euclidean distances;
 *               its edges taken in ascending (length, lower, higher index)
 *               order through a union-find where the smaller component is
 *               absorbed (equal sizes: the root with the larger index) and the
 *               absorbed root's salience is the edge length.  One block, the
 *               last survivor, scores 0.
 *   row_ptr     device int32 [nb + 1], written.
 *   col_idx     device int32 [col_capacity], entries [0, nnz) written.
 *               col_capacity must be >= tsa_schedule_max_nnz(nb, sink,
 *               local_radius, topk), so the build can never overflow it.
 *   salience    device double [nb] or NULL; written when not NULL.
 *   workspace   device, >= tsa_build_schedule_workspace_bytes(S, D, block) bytes,
 *               256-byte aligned.  Its contents on entry may be anything (it needs
 *               no clearing) and are unspecified on return.  Two builds that may
 *               run at the same time (on different streams) must not share one
 *               workspace.  A build captured in a HIP graph rebuilds the schedule
 *               on every replay (the call's state lives in the workspace).
 *   nnz_host    host int64 or NULL.  When not NULL the call waits for the
 *               stream and stores row_ptr[nb] (the number of entries) there.
 *   S == 0 builds an empty schedule (row_ptr = {0}).
 * Edges are taken in ascending (length, lower index, higher index) order, a
 * strict order: exactly tied distances are resolved by the block indices, as a
 * scan of all pairs in that order resolves them, so the schedule is a function
 * of the keys alone.
 */
int tsa_build_schedule(const void* keys, int32_t dtype, int64_t S, int64_t D, int32_t block,
                       int32_t sink, int32_t local_radius, int32_t topk, int32_t* row_ptr,
                       int32_t* col_idx, int64_t col_capacity, double* salience, void* workspace,
                       size_t workspace_bytes, int64_t* nnz_host, void* stream);

/* Scope of the top-k term of a schedule row. */
#define TSA_TOPK_GLOBAL 0  /* one set: the topk blocks of highest salience */
#define TSA_TOPK_PER_ROW 1 /* each row: the topk highest among its blocks j <= i */

/*
 * tsa_build_schedule with a choice of top-k scope.  (PR page, Summary, second
 * bullet: a top-k selection of salient key blocks; the pages do not settle
 * whether the selection is one set for all rows or one per row.)
 *   topk_scope  TSA_TOPK_GLOBAL: exactly tsa_build_schedule.
 *               TSA_TOPK_PER_ROW: row i takes the min(topk, i+1) blocks of
 *               highest salience among blocks 0..i (same ranking: salience
 *               descending, lower index first on ties), besides its sink and
 *               local blocks; the sets may overlap.  The same capacity bound,
 *               tsa_schedule_max_nnz, holds.
 * Every other argument, the workspace contract and the errors are those of
 * tsa_build_schedule; an unknown topk_scope is TSA_ERR_INVALID_ARG.
 */
int tsa_build_schedule_ex(const void* keys, int32_t dtype, int64_t S, int64_t D, int32_t block,
                          int32_t sink, int32_t local_radius, int32_t topk, int32_t topk_scope,
                          int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                          double* salience, void* workspace, size_t workspace_bytes,
                          int64_t* nnz_host, void* stream);

/*
 * Upper bound on the entries of tsa_refine_schedule's output: min(m^2 nnz,
 * n(n+1)/2) with m = block / 64 and n = ceil(S / 64).  Host-only; -1 for negative
 * sizes or an unsupported block.
 */
int64_t tsa_refine_schedule_max_nnz(int64_t S, int32_t block, int64_t nnz);

/*
 * The CSR over 64-row blocks that allows exactly the keys a CSR over blocks of
 * `block` rows allows, for the attention entry points, which work on 64-row
 * blocks.  (PR page, Summary, fifth bullet: a schedule's block size is validated;
 * the Local benchmark uses 64.)  With m = block / 64 and I = i / m, row i of the
 * output lists m*J + b (b = 0..m-1, m*J + b <= i) for every block J that row I
 * of the input lists, ascending; query t then sees key u <= t exactly when
 * u / block is listed in row t / block.  An input entry counts when the attention
 * kernels would accept it (within 0..I and above every earlier entry of its row
 * that lies in 0..I).
 *   S           sequence length; the input has ceil(S / block) rows, the output
 *               ceil(S / 64) <= TSA_MAX_REFINED_BLOCKS.
 *   row_ptr, col_idx   device int32 input CSR, `nnz` readable entries.
 *   row_ptr64   device int32 [ceil(S / 64) + 1], written.
 *   col_idx64   device int32 [capacity], entries [0, row_ptr64[n]) written;
 *               capacity >= tsa_refine_schedule_max_nnz(S, block, nnz).  That
 *               bound holds when row_ptr is non-decreasing.  Rows that share
 *               input entries (a row_ptr that is not) can need more; entries at
 *               or past `capacity` are then counted in row_ptr64 (saturated at
 *               INT32_MAX) but never written.
 *   nnz_host    host int64 or NULL: when not NULL the call waits for the stream
 *               and stores the output's entry count there; a count above
 *               `capacity` returns TSA_ERR_SCHEDULE (the one error found after
 *               the kernels ran: row_ptr64 and the first `capacity` entries are
 *               then written).
 * block = 64 returns the input's accepted entries unchanged.  Errors: negative
 * sizes (TSA_ERR_INVALID_ARG), an unsupported block or too many output rows
 * (TSA_ERR_UNSUPPORTED), more entries than int32 offsets hold (TSA_ERR_SHAPE), a
 * short capacity (TSA_ERR_SCHEDULE), NULL or non-device pointers.
 */
int tsa_refine_schedule(int64_t S, int32_t block, const int32_t* row_ptr, const int32_t* col_idx,
                        int64_t nnz, int32_t* row_ptr64, int32_t* col_idx64, int64_t capacity,
                        int64_t* nnz_host, void* stream);

/* Size of the library's fixed builder workspace on each GPU (tsa_build_schedule_noalloc). */
#define TSA_NOALLOC_SCRATCH_BYTES (4u << 20)

/*
 * tsa_build_schedule_ex without a workspace argument and without allocating,
 * for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The build runs in a
 * fixed array of TSA_NOALLOC_SCRATCH_BYTES bytes that the library holds in each
 * GPU's memory until the process ends; the call allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine) and does not wait for the stream.
 *   Every argument is that of tsa_build_schedule_ex; the count of entries is
 *   row_ptr[nb] (read it back after the stream is done).
 *   Limit: builds whose tsa_build_schedule_workspace_bytes(S, D, block) exceeds
 *   TSA_NOALLOC_SCRATCH_BYTES are rejected with TSA_ERR_UNSUPPORTED before any GPU
 *   work (nb <= 512 blocks fits at D <= 256, e.g. 32768 tokens at block 64).
 *   Concurrency: all no-allocation builds on one GPU share its array, so two of
 *   them that may overlap in time (different streams, or different host threads
 *   on one stream without ordering) race; calls ordered on one stream do not.
 *   The array needs no clearing between calls (the builder's state carries a
 *   per-call token), and a build captured in a HIP graph rebuilds on replay.
 * Errors: those of tsa_build_schedule_ex, plus TSA_ERR_UNSUPPORTED for the limit
 * and TSA_ERR_HIP if the array's device address cannot be looked up.
 */
int tsa_build_schedule_noalloc(const void* keys, int32_t dtype, int64_t S, int64_t D, int32_t block,
                               int32_t sink, int32_t local_radius, int32_t topk, int32_t topk_scope,
                               int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                               double* salience, void* stream);

/*
 * The dense causal (lower-triangular) CSR for nb blocks: row i lists 0..i.
 * (PR page, Summary: the tests cover the dense causal CSR; Local benchmark: the dense CSR
 * path visits every causal block.)  row_ptr int32 [nb + 1] and col_idx int32
 * [col_capacity >= nb*(nb+1)/2], both device memory.
 */
int tsa_dense_causal_schedule(int64_t nb, int32_t* row_ptr, int32_t* col_idx,
                              int64_t col_capacity, void* stream);

/*
 * Entries of the fixed-segment CSR for nb blocks and segments of segment_blocks
 * blocks (below).  Host-only; returns -1 if nb < 0 or segment_blocks < 1.
 */
int64_t tsa_segment_schedule_nnz(int64_t nb, int32_t segment_blocks);

/*
 * The fixed-segment (block-diagonal causal) CSR: with L = segment_blocks, row i
 * lists blocks L*floor(i/L) .. i, so attention never crosses a segment
 * boundary.  (Mirror page, commit note on learned segment boundaries: a merged
 * causal CSR kernel consumes segment boundaries exactly; fixed 512- and 256-token
 * segments at S 4096 visit 288 and 160 blocks.)
 *   row_ptr   device int32 [nb + 1], written.
 *   col_idx   device int32 [col_capacity], entries [0, nnz) written;
 *             col_capacity >= tsa_segment_schedule_nnz(nb, segment_blocks).
 * Errors: nb < 0 or segment_blocks < 1 (TSA_ERR_INVALID_ARG), more entries than
 * int32 offsets hold (TSA_ERR_SHAPE), a short col_idx (TSA_ERR_SCHEDULE), NULL
 * or non-device pointers.  Nothing is written on error.
 */
int tsa_segment_schedule(int64_t nb, int32_t segment_blocks, int32_t* row_ptr, int32_t* col_idx,
                         int64_t col_capacity, void* stream);

/*
 * Forward scheduled attention.  (PR page, Summary, first, third and fourth
 * bullets; mirror page, Rust-port commit note: running row max and denominator
 * rescaled by exp(m_prev - m_new), one score tile live at a time.)
 *
 *   q, k, v, out  device, [B, H, S, D] row-major of `dtype` (out has q's dtype).
 *                 [S, D] inputs are B = H = 1.  out must not overlap q, k, v; all four
 *                 must be 16-byte aligned.
 *   D             32, 64, 128 or 256.
 *   row_ptr, col_idx  device int32 CSR with nb = ceil(S/block) rows; `nnz` is
 *                 the number of readable col_idx entries.  Row i must list key
 *                 blocks strictly ascending within 0..i.  For memory safety the
 *                 kernel clamps row bounds to [0, nnz] and skips entries that
 *                 are negative, greater than i, or not greater than the
 *                 previous accepted entry.
 *   block         rows per query block and per key block: TSA_BLOCK (64), or
 *                 TSA_SUB_BLOCK (32) at D 32, 64 or 128 with S <= 65535 * 128
 *                 (TSA_ERR_UNSUPPORTED otherwise).  The row_ptr array must hold
 *                 nb + 1 entries for this block size; the library cannot check it.
 *   sm_scale      softmax scale; <= 0 selects 1/sqrt(D).
 * For query row t in block i the output is the softmax-weighted mean of v over
 * keys u <= t whose block is listed in row i; a row with no such key is 0.
 * Scores and running statistics are fp32; the probabilities are rounded to the
 * input dtype for the P*V product (the denominator is summed from the same
 * rounded values); the output is rounded to nearest even.
 * B, H or S equal to 0 is a valid empty call.
 */
int tsa_scheduled_attention_fwd(const void* q, const void* k, const void* v, void* out,
                                int32_t dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                                const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                int32_t block, float sm_scale, void* stream);

/*
 * Forward scheduled attention that also returns each row's log-sum-exp, the
 * statistic the backward pass reads.  (Same passages as
 * tsa_scheduled_attention_fwd; the mirror page's Rust-port commit note: the
 * running maximum and denominator of each row.)
 *   lse   device float [B, H, S], written: lse[t] = log of the row's softmax
 *         denominator in natural units, log sum_{u in A(t)} exp(scale q_t.k_u),
 *         from the same fp32 running max and denominator the output is
 *         normalised by; -inf for a row with no allowed key.  4-byte aligned,
 *         must not overlap q, k, v or out.
 * Every other argument, the output and the errors are those of
 * tsa_scheduled_attention_fwd; a NULL lse is TSA_ERR_INVALID_ARG.
 */
int tsa_scheduled_attention_fwd_lse(const void* q, const void* k, const void* v, void* out,
                                    float* lse, int32_t dtype, int64_t B, int64_t H, int64_t S,
                                    int64_t D, const int32_t* row_ptr, const int32_t* col_idx,
                                    int64_t nnz, int32_t block, float sm_scale, void* stream);

/*
 * Device workspace, in bytes, of tsa_schedule_transpose for nb blocks (256-byte
 * aligned start required).  Host-only.  0 when nb <= 0 (none is needed for nb = 0)
 * or nb > TSA_MAX_SCHEDULE_BLOCKS.
 */
size_t tsa_schedule_transpose_workspace_bytes(int64_t nb);

/*
 * Column view (CSC) of a causal CSR schedule: column j lists, ascending, the
 * query blocks i whose row lists key block j.  The key and value gradients of
 * block j gather over exactly these rows (backward of the forward of PR page,
 * Summary, first bullet; the pages' kernel has none, see
 * tsa_scheduled_attention_bwd).  Build it once per schedule.
 *   row_ptr, col_idx  device int32 CSR, nb rows, `nnz` readable entries.  An
 *               entry of row i counts exactly when the attention kernels accept
 *               it: it lies in 0..i and exceeds every earlier entry of the row
 *               that lies in 0..i (all entries, for a row that is strictly
 *               ascending within 0..i as the schedule contract asks).
 *   col_ptr     device int32 [nb + 1], written.
 *   row_idx     device int32 [row_capacity], entries [0, col_ptr[nb]) written;
 *               row_capacity >= min(nnz, nb*(nb+1)/2), which holds every entry
 *               when row_ptr is non-decreasing.  Rows that share entries (a
 *               row_ptr that is not) can need more; entries at or past
 *               row_capacity are then counted in col_ptr but never written.
 *   workspace   device, >= tsa_schedule_transpose_workspace_bytes(nb) bytes,
 *               256-byte aligned, any contents on entry (NULL allowed when nb = 0).
 *   nnz_host    host int64 or NULL: when not NULL the call waits for the stream
 *               and stores col_ptr[nb] there; a count above row_capacity returns
 *               TSA_ERR_SCHEDULE (found after the kernels ran: col_ptr and the
 *               first row_capacity entries are then written).
 * Errors: negative sizes (TSA_ERR_INVALID_ARG), nb > TSA_MAX_SCHEDULE_BLOCKS
 * (TSA_ERR_UNSUPPORTED), a short row_idx (TSA_ERR_SCHEDULE), a short or misaligned
 * workspace, NULL or non-device pointers.  Nothing is written on these errors.
 */
int tsa_schedule_transpose(int64_t nb, const int32_t* row_ptr, const int32_t* col_idx,
                           int64_t nnz, int32_t* col_ptr, int32_t* row_idx, int64_t row_capacity,
                           void* workspace, size_t workspace_bytes, int64_t* nnz_host,
                           void* stream);

/*
 * Device workspace, in bytes, of tsa_scheduled_attention_bwd: 8 bytes per query
 * row of every lane (B * H * S * 8), rounded up to 16, plus 4 bytes per key
 * block (ceil(S / 64) * 4).  Host-only; 0 for negative or overflowing sizes.
 */
size_t tsa_scheduled_attention_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S);

/*
 * Backward of tsa_scheduled_attention_fwd: the gradients of q, k and v for an
 * upstream gradient dout of the output.  The pages' kernel is forward-only (PR
 * page, Summary, first bullet; the mirror page's note on learned segment
 * boundaries says training would otherwise run dense).  With P_tu = exp(scale
 * q_t.k_u - lse_t) on the allowed keys A(t) of row t (0 elsewhere):
 *   dV = P^T dout,  dS = P * (dout V^T - Delta),  Delta_t = dout_t . out_t,
 *   dQ = scale dS K,  dK = scale dS^T Q.
 *   q, k, v, out, dout   device, [B, H, S, D] of `dtype` ([S, D]: B = H = 1);
 *               out is the forward's output for these q, k, v and schedule.
 *   lse         device float [B, H, S] from tsa_scheduled_attention_fwd_lse.
 *   row_ptr, col_idx, nnz   the CSR the forward used (same contract).
 *   col_ptr, row_idx, nnz_t its column view from tsa_schedule_transpose
 *               (nnz_t readable row_idx entries).  The kernels skip entries of a
 *               column that are outside j..nb-1 or not above the previous accepted
 *               one; a column view that is not the CSR's transpose gives
 *               unspecified gradients (never an out-of-bounds access).
 *   block       64, or TSA_SUB_BLOCK (32) for a schedule over 32-row blocks,
 *               whose column view is then over 32-key blocks (nb = ceil(S / 32)
 *               in both; D up to 128 there);  D 32, 64, 128 or 256 at block
 *               64 (at 256 each workgroup writes half the head dims and forms S
 *               and dP over all of them, so those two products run twice);
 *               sm_scale as in the forward.
 *   dq, dk, dv  device, q's shape and dtype, written (rounded to nearest even).
 *   workspace   device, >= tsa_scheduled_attention_bwd_workspace_bytes(B, H, S)
 *               bytes, 16-byte aligned, any contents on entry; it holds each
 *               row's (lse, Delta) between the two kernels and an order of the
 *               key blocks by column length.
 * All 16-bit tensors 16-byte aligned; dq, dk, dv and the workspace must not
 * overlap each other or any input.  Scores, statistics and accumulators are
 * fp32; P and dS are rounded to the input dtype as MFMA operands.  B, H or S
 * equal to 0 is a valid empty call.  Errors as tsa_scheduled_attention_fwd, plus
 * a short or misaligned workspace (TSA_ERR_INVALID_ARG).
 */
int tsa_scheduled_attention_bwd(const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, int32_t dtype, int64_t B,
                                int64_t H, int64_t S, int64_t D, const int32_t* row_ptr,
                                const int32_t* col_idx, int64_t nnz, const int32_t* col_ptr,
                                const int32_t* row_idx, int64_t nnz_t, int32_t block,
                                float sm_scale, void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSA_H */
