/*
 * pred.h -- C ABI of the low-rank block predictor for a paged KV cache (MI355X / gfx950).
 *
 * What it computes (predictor.rs page, module doc): a seeded projection
 * P [head_dim, r] maps every query (Q @ P) and every key of a KV block (K @ P)
 * to rank r; the projected keys live in A_g [layers, max_blocks, num_kv_heads,
 * block_size, r] (bf16, layout comment on a_g_bytes and on the Predictor
 * fields); a block's score is the max, over query heads, query rows and the
 * block's tokens, of the projected dot product, and an ascending sort of the
 * scores ranks eviction victims (lowest score first).
 *
 * Conventions for every call below
 *   - Return value: 0 on success, a negative PRED_ERR_* code on failure; the
 *     thread-local pred_last_error() string then says what was wrong.  A call
 *     that fails argument checks enqueues nothing.
 *   - Pointers marked "device" are HIP device pointers the caller owns and
 *     keeps alive until the enqueued work has finished; "host" pointers are
 *     read or written before the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call except
 *     pred_create, pred_copy_projection, pred_read_slot and pred_device_error
 *     only enqueues work on `stream` and returns without synchronising
 *     (the pages' *_on_stream variants).
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16_t), row-major.
 *   - The library allocates device memory only in pred_create (P, A_g and a
 *     4-byte error word) and frees it in pred_destroy.
 */
#ifndef PRED_H
#define PRED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pred_bf16;
typedef struct pred_handle pred_t;

/* PredictorDims (predictor.rs page).  All fields must be > 0 and
 * num_q_heads must be a multiple of num_kv_heads (PredictorDims::validate). */
typedef struct {
    int32_t num_layers;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t r;
    int32_t block_size;
    int64_t max_blocks;
} pred_dims;

enum {
    PRED_OK = 0,
    PRED_ERR_INVALID_DIMS = -1, /* a dim <= 0, nq % nkv != 0, or a size overflows int64 */
    PRED_ERR_OUT_OF_RANGE = -2, /* layer / block / count outside the dims */
    PRED_ERR_OOM = -3,          /* A_g does not fit in 95% of free HBM */
    PRED_ERR_UNSUPPORTED = -4,  /* a shape this library's kernels do not handle */
    PRED_ERR_NULL_ARG = -5,     /* a required pointer is NULL */
    PRED_ERR_HIP = -6,          /* a HIP runtime call or kernel launch failed */
    PRED_ERR_WORKSPACE = -7,    /* workspace missing or too small */
    PRED_ERR_DEVICE = -8        /* a kernel met an invalid block-table entry */
};

/* pred_create flags */
#define PRED_FLAG_ZERO_AG 1u /* zero A_g after allocation (it is left unzeroed by default) */

/* ------------------------------------------------------------------ sizing (pure) */

/* Bytes of A_g: num_layers * max_blocks * num_kv_heads * block_size * r * 2
 * (predictor.rs page, a_g_bytes).  Returns a negative code if the dims are
 * invalid or the product overflows. */
int64_t pred_a_g_bytes(const pred_dims* d);

/* The fit check made by pred_create before it allocates A_g (predictor.rs
 * page, new_on_stream): A_g must not exceed 95% of `free_bytes`, the rest being
 * kept for scratch and attention.  Returns 0 if it fits, PRED_ERR_OOM with a
 * message naming r, max_blocks and the sizing formula otherwise, or
 * PRED_ERR_INVALID_DIMS.  No device access. */
int pred_check_fit(const pred_dims* d, uint64_t free_bytes);

/* Largest r and max_blocks this library's kernels accept, and other shape
 * limits, as a human-readable message (host string, static storage). */
const char* pred_limits(void);

/* ------------------------------------------------------------------ lifetime */

/* Validate the dims, build P on the host from `seed` (N(0, 1/r) rounded to
 * bf16 by the SplitMix64 / Box-Muller rule the library documents), check the
 * fit against hipMemGetInfo, allocate P and A_g on the current device, upload
 * P on `stream` and synchronise it (predictor.rs page, new_on_stream).
 * A_g is not zeroed unless PRED_FLAG_ZERO_AG is set: score_blocks may read
 * slots that project_kv_block never wrote.  On any failure everything
 * allocated is freed and *out is left NULL. */
int pred_create(const pred_dims* d, uint64_t seed, uint32_t flags, void* stream, pred_t** out);

/* As pred_create, but P is taken from `p_host` [head_dim, r] bf16 (host) instead
 * of being generated.  For tests that need a chosen P (identity, hand-worked
 * examples). */
int pred_create_with_projection(const pred_dims* d, const pred_bf16* p_host, uint32_t flags,
                                void* stream, pred_t** out);

/* Free P, A_g and the handle.  Waits for the device first.  NULL is a no-op. */
void pred_destroy(pred_t* p);

/* ------------------------------------------------------------------ hot path */

/* q_proj = bf16(q @ P) (predictor.rs page, project_q).
 *   q       device, [n_vec, num_q_heads, head_dim] bf16 (n_vec stacked query rows,
 *           e.g. layers x sequences x rows)
 *   q_proj  device, [n_vec, num_q_heads, r] bf16 output
 * Every output element is the float64 sum of its head_dim exact bf16 products,
 * rounded once to bf16 (nearest, ties to even).  n_vec == 0 is a no-op. */
int pred_project_q(pred_t* p, const pred_bf16* q, int64_t n_vec, pred_bf16* q_proj, void* stream);

/* Project whole KV blocks of `n_layers` layers and write their low-rank keys
 * into A_g through block tables (predictor.rs page, project_kv_block, batched
 * over blocks and layers).
 *   k            device, [n_layers, n_blocks, block_size, num_kv_heads, head_dim]
 *                bf16 (one block per [block_size, num_kv_heads, head_dim] slice,
 *                the page's k_block layout)
 *   block_table  device, [n_layers, n_blocks] int32 physical slot ids, or NULL
 *                for slots 0..n_blocks-1 in every layer
 * Block i of layer layer0 + l lands in A_g[layer0 + l, block_table[l, i]] as
 * [num_kv_heads, block_size, r], each element bf16(float64 sum).  Host-side
 * errors: layers outside [0, num_layers) or (NULL table) n_blocks > max_blocks
 * -> PRED_ERR_OUT_OF_RANGE.  A table entry outside [0, max_blocks) is skipped on
 * the device and raises the device error word (see pred_device_error).  Two
 * entries naming one slot of one layer race.  Any count of zero is a no-op. */
int pred_project_kv_block(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* k,
                          const int32_t* block_table, int64_t n_blocks, void* stream);

/* The two projections of one decode step in one call: exactly
 * pred_project_kv_block(p, layer0, n_layers, k_new, new_table, n_new, stream)
 * followed by pred_project_q(p, q, n_vec, q_proj, stream), with the same
 * arguments, checks and results (predictor.rs page: project_kv_block and
 * project_q, both run once per step).  Both parts are checked before either is
 * enqueued.  When both are small (a decode step's one new block per layer and
 * its query rows) they share one kernel launch, which saves a launch's fixed
 * cost on the step's critical path; larger calls take the two usual launches.
 *   k_new      device, [n_layers, n_new, block_size, num_kv_heads, head_dim] bf16
 *   new_table  device, [n_layers, n_new] int32 or NULL (slots 0..n_new-1)
 *   q          device, [n_vec, num_q_heads, head_dim] bf16
 *   q_proj     device, [n_vec, num_q_heads, r] bf16 output
 * A zero count skips its part. */
int pred_project_step(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* k_new,
                      const int32_t* new_table, int64_t n_new, const pred_bf16* q, int64_t n_vec,
                      pred_bf16* q_proj, void* stream);

/* Block scores (predictor.rs page, score_blocks, extended to several layers,
 * sequences and query rows).
 *   q_proj        device, [n_layers, n_seqs, n_rows, num_q_heads, r] bf16
 *   block_tables  device, [n_seqs, n_blocks] int32 physical ids, or NULL for the
 *                 identity (every sequence reads slots 0..n_blocks-1)
 *   scores        device, [n_layers, n_seqs, n_blocks] float32 output
 * scores[l, s, b] = max over rows i, query heads h, tokens t of
 *   sum_j q_proj[l, s, i, h, j] * A_g[layer0 + l, table[s, b], h / g, t, j]
 * with g = num_q_heads / num_kv_heads, accumulated in float32, no scale.
 * Scores are indexed by logical block position b.  Slots never written hold
 * whatever A_g held.  Errors: layer0 + n_layers > num_layers, n_blocks >
 * max_blocks with a NULL table -> PRED_ERR_OUT_OF_RANGE.  A table entry outside
 * [0, max_blocks) gives that block a NaN score and raises the device error word.
 * Any count of zero is a no-op. */
int pred_score_blocks(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* q_proj,
                      int32_t n_rows, const int32_t* block_tables, int64_t n_blocks, int32_t n_seqs,
                      float* scores, void* stream);

/* As pred_score_blocks, but the last block of each sequence (logical block
 * n_blocks - 1) is partly filled: only its first last_fill[s] tokens are scored
 * (a decode step appends one token at a time; the predictor.rs page scores all
 * block_size tokens of every block, which equals last_fill[s] = block_size).
 *   last_fill  device, [n_seqs] int32 in [0, block_size], or NULL for full blocks.
 * A last block with fill 0 scores -inf.  A value outside [0, block_size] is
 * clamped to it and raises the device error word (see pred_device_error). */
int pred_score_blocks_masked(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* q_proj,
                             int32_t n_rows, const int32_t* block_tables, int64_t n_blocks, int32_t n_seqs,
                             const int32_t* last_fill, float* scores, void* stream);

/* Eviction order (predictor.rs page, module doc: scores rank eviction victims;
 * qsa_select.rs page, host top-k: lower index on ties).
 *   scores     device, [n_segments, n_blocks] float32
 *   victims    device, [n_segments, n_blocks] int32 output: each row is the
 *              permutation of 0..n_blocks-1 that sorts the row's scores
 *              ascending, equal scores in ascending index order, -0 equal to
 *              +0, NaN before everything
 *   workspace  device scratch of at least pred_rank_workspace_bytes() bytes
 *              (may be NULL when that is 0)
 * n_blocks and n_segments must be <= 2^31 - 1.  A call too large for one
 * launch (over 2^31 - 1 workgroups) fails with PRED_ERR_OUT_OF_RANGE before
 * anything is enqueued; the same holds for the other entry points. */
int pred_rank_victims(pred_t* p, const float* scores, int64_t n_blocks, int64_t n_segments,
                      int32_t* victims, void* workspace, size_t ws_bytes, void* stream);

/* pred_rank_victims for callers that cannot allocate or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments (without the workspace), checks and result as
 * pred_rank_victims; the sorted runs live instead in a static device array of
 * PRED_NOALLOC_SCRATCH_BYTES bytes that each GPU holds from library load to
 * process end (its address is found once per device by pred_create).  The call
 * allocates nothing and makes no memset: every byte of scratch it reads it has
 * written first in the same call.
 *   scores   device, [n_segments, n_blocks] float32
 *   victims  device, [n_segments, n_blocks] int32 output
 * A shape needing more than PRED_NOALLOC_SCRATCH_BYTES
 * (pred_rank_workspace_bytes(n_blocks, n_segments) above it, e.g. more than
 * 1048576 keys in rows of 2049..8192) fails with PRED_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU shares that GPU's array, across
 * handles and streams: two calls that can run at the same time on one GPU
 * (different streams or threads without ordering between them) race and give
 * wrong rankings; order them on one stream. */
#define PRED_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int pred_rank_victims_noalloc(pred_t* p, const float* scores, int64_t n_blocks, int64_t n_segments,
                              int32_t* victims, void* stream);

/* The k lowest-scored blocks of every segment, in eviction order: row s of
 * victims is exactly the first k entries of pred_rank_victims's row s (scores
 * ascending, equal scores in ascending index order, -0 equal to +0, NaN
 * first).  This is the step after the ranking (predictor.rs page, module doc:
 * scores rank eviction victims; a cache evicts k blocks at a time).
 *   scores     device, [n_segments, n_blocks] float32
 *   k          0 <= k <= n_blocks (k = n_blocks is the full ranking)
 *   victims    device, [n_segments, k] int32 output (row stride k)
 *   workspace  as for pred_rank_victims (pred_rank_workspace_bytes(n_blocks,
 *              n_segments) bytes; NULL when that is 0)
 * Only each sorted run's first k places are merged, so small k costs less
 * than the full ranking. */
int pred_select_victims(pred_t* p, const float* scores, int64_t n_blocks, int64_t n_segments, int64_t k,
                        int32_t* victims, void* workspace, size_t ws_bytes, void* stream);

/* Name of the kernel pred_score_blocks (and pred_score_blocks_masked) runs for
 * this handle's dims and n_rows query rows per sequence (host only, static
 * string): "score_prefill_kernel" (more than 16 queries per kv head: bf16
 * MFMA), "score_decode_mfma_kernel" (5 to 16), "score_decode_kernel" (up to 4,
 * or shapes the matrix-core variant does not take) or "score_generic_kernel"
 * (r or block_size outside the streaming layouts).  NULL for a NULL handle or
 * n_rows < 1. */
const char* pred_score_kernel_name(pred_t* p, int32_t n_rows);

/* As pred_score_kernel_name, with the kernel's template arguments for a call
 * of n_blocks blocks per sequence, e.g.
 * "score_decode_kernel<lanes_per_row=4,queries=4,slots=2,q_in_lds=1,offset=u32,uniform_slots=1>"
 * (q_in_lds: the q_proj slab of one (layer, sequence) is staged in LDS, which
 * it is up to 32 KiB; offset: u64 when one layer of A_g is 4 GiB or more).
 * Host only; the string is thread-local storage valid until the next call on
 * the same thread.  NULL for a NULL handle, n_rows < 1 or n_blocks < 1. */
const char* pred_score_kernel_variant(pred_t* p, int32_t n_rows, int64_t n_blocks);

/* Score kernel override, a debugging switch (qsa_select.rs page: the prefill
 * selection's environment switch that forces its scalar scorer in place of the
 * tensor-core one).  PRED_SCORE_PATH_AUTO is the library's own choice; _DECODE
 * routes every pred_score_blocks / pred_score_blocks_masked call through the
 * vector-ALU streaming decode kernel (or the plain kernel where its layout does
 * not fit); _GENERIC routes those and pred_score_rows through the plain
 * per-block / per-cell kernels.  Every path gives the same scores within
 * float32 rounding.  The initial value comes from the environment variable
 * PRED_SCORE_PATH (auto, decode or generic), read once per process; the
 * variable PRED_LOG=1 makes every score launch print one line on stderr naming
 * its kernel.  Process-wide, not tied to a handle; set it while no other
 * thread is enqueueing score calls. */
enum { PRED_SCORE_PATH_AUTO = 0, PRED_SCORE_PATH_DECODE = 1, PRED_SCORE_PATH_GENERIC = 2 };
/* Returns 0, or PRED_ERR_OUT_OF_RANGE for a value not in the enum above. */
int pred_set_score_path(int32_t path);
/* The current PRED_SCORE_PATH_* value (host only, no device needed). */
int pred_get_score_path(void);

/* Per-row causal block scores of a prefill chunk (qsa_select.rs page, prefill
 * selection: each query row is scored against the blocks complete at its
 * position; the score is the predictor's, predictor.rs page, score_blocks, kept
 * per row instead of maximised over rows).
 *   layer        A_g layer to read, 0 <= layer < num_layers
 *   q_proj       device, [rows, num_q_heads, r] bf16; row i sits at position
 *                first_pos + i of the sequence
 *   block_table  device, [n_blocks] int32 physical ids of the sequence's
 *                blocks, or NULL for slots 0..n_blocks-1
 *   scores       device, [rows, stride] float32 output
 * With complete(i) = min(n_blocks, (first_pos + i + 1) / block_size), the
 * blocks whose every token is at or before row i's position:
 *   scores[i, b] = max over query heads h, tokens t of
 *                  sum_j q_proj[i, h, j] * A_g[layer, table[b], h / g, t, j]
 * for b < complete(i) (float32 accumulation, no scale), and -inf for
 * complete(i) <= b < stride.  A table entry outside [0, max_blocks) gives a
 * complete block a NaN score and raises the device error word.  rows and
 * n_blocks <= 2^31-1; rows * stride == 0 is a no-op; q_proj must be 16-byte
 * aligned. */
int pred_score_rows(pred_t* p, int32_t layer, const pred_bf16* q_proj, int64_t rows, int64_t first_pos,
                    const int32_t* block_table, int64_t n_blocks, float* scores, int64_t stride,
                    void* stream);

/* Per-row keep sets (qsa_select.rs page, prefill selection's top-k per row,
 * here on the device): for row i the first c(i) = min(stride,
 * (first_pos + i + 1) / ratio) entries of scores row i, ordered by descending
 * score with equal scores in ascending index order (-0 equal to +0, NaN after
 * everything), and the first topk of them written to keep row i.  Slots past
 * c(i) hold -1.
 *   scores     device, [rows, stride] float32 (e.g. pred_score_rows's output,
 *              with ratio = block_size)
 *   keep       device, [rows, topk] int32 output
 *   ratio      >= 1; first_pos in [0, 2^62]; 0 <= topk <= stride
 *   workspace  pred_rank_workspace_bytes(stride, rows) bytes (NULL when 0)
 * rows and stride must be <= 2^31-1. */
int pred_select_keep(pred_t* p, const float* scores, int64_t rows, int64_t stride, int64_t first_pos,
                     int32_t ratio, int64_t topk, int32_t* keep, void* workspace, size_t ws_bytes,
                     void* stream);

/* One decode step in one call: the step's new blocks into A_g, q_proj of every
 * layer, block scores and each (layer, sequence) row's k lowest blocks in
 * eviction order -- pred_project_step (pred_project_kv_block and
 * pred_project_q), pred_score_blocks_masked and pred_select_victims (pred_rank_victims when
 * k = n_blocks) on one stream, in that order, with the same arguments and
 * results (predictor.rs page: project_q, project_kv_block and score_blocks of
 * one step; module doc: the scores rank eviction victims).
 *   k_new       device, [n_layers, n_new, block_size, num_kv_heads, head_dim] bf16
 *   new_table   device, [n_layers, n_new] int32 slots for them (NULL: 0..n_new-1)
 *   q           device, [n_layers, n_seqs, n_rows, num_q_heads, head_dim] bf16
 *   q_proj      device, [n_layers, n_seqs, n_rows, num_q_heads, r] bf16 output
 *   block_tables, n_blocks, n_seqs, last_fill: as for pred_score_blocks_masked
 *   scores      device, [n_layers, n_seqs, n_blocks] float32 output
 *   victims     device, [n_layers * n_seqs, k] int32 output, 0 <= k <= n_blocks
 *   workspace   pred_rank_workspace_bytes(n_blocks, n_layers * n_seqs) bytes
 * Every part's arguments are checked before anything is enqueued.  The step
 * allocates nothing, never synchronises and issues no memset, so a caller may
 * capture it into a HIP graph and replay it (the arguments are then fixed). */
int pred_decode_step(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* k_new,
                     const int32_t* new_table, int64_t n_new, const pred_bf16* q, int32_t n_rows,
                     pred_bf16* q_proj, const int32_t* block_tables, int64_t n_blocks, int32_t n_seqs,
                     const int32_t* last_fill, float* scores, int64_t k, int32_t* victims,
                     void* workspace, size_t ws_bytes, void* stream);

/* Workspace pred_rank_victims needs for this shape: 0 for n_blocks <= 2048
 * (each segment is sorted inside one workgroup), else 8 bytes per key for the
 * sorted runs, twice that for n_blocks > 8192 (pairwise merge buffers). */
size_t pred_rank_workspace_bytes(int64_t n_blocks, int64_t n_segments);

/* ------------------------------------------------------------------ inspection */

/* The P that pred_create builds for (head_dim, r, seed), computed on the host
 * only (no device needed): `out` is [head_dim, r] bf16.  Returns
 * PRED_ERR_INVALID_DIMS for non-positive sizes. */
int pred_projection_host(int32_t head_dim, int32_t r, uint64_t seed, pred_bf16* out);

/* Copy P [head_dim, r] bf16 to `host_out` (synchronous). */
int pred_copy_projection(pred_t* p, pred_bf16* host_out);

/* Device address of A_g [num_layers, max_blocks, num_kv_heads, block_size, r]
 * bf16 (predictor.rs page, a_g_dev_ptr).  The library owns it. */
void* pred_a_g_ptr(pred_t* p);

/* Copy the A_g slot (layer, block) [num_kv_heads, block_size, r] bf16 to
 * `host_out` and synchronise `stream` (predictor.rs page, read_k_lr_slot). */
int pred_read_slot(pred_t* p, int32_t layer, int64_t block, pred_bf16* host_out, void* stream);

/* The dims the handle was created with (predictor.rs page, dims). */
int pred_get_dims(pred_t* p, pred_dims* out);

/* Synchronise `stream`, read and clear the device error word.  Returns 0, or
 * PRED_ERR_DEVICE if a kernel since the last call met an invalid table entry
 * or a last-block fill count outside [0, block_size]. */
int pred_device_error(pred_t* p, void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* pred_last_error(void);

/* Library version string. */
const char* pred_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PRED_H */
