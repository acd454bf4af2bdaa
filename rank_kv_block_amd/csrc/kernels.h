// Launchers of the predictor's HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "common.h"

namespace pred {

// A launch takes at most 2^31 - 1 workgroups; a call that would need more is
// rejected with hipErrorInvalidConfiguration before anything is enqueued.
inline bool grid_fits(int64_t workgroups) { return workgroups >= 0 && workgroups <= 0x7FFFFFFF; }

// ---- projections (proj.hip) ----------------------------------------------
// out[v, :] = bf16(in[v, :] @ P) for n_vec rows of D bf16 (dense output [n_vec, R]).
hipError_t launch_project_dense(const uint16_t* in, const double* pf, uint16_t* out, int64_t n_vec,
                                int D, int R, hipStream_t stream);
// Whole blocks k [n_layers, n_blocks, B, Hk, D] -> A_g slabs starting at a_first
// ([n_layers][N, Hk, B, R]) through table [n_layers, n_blocks] (null = identity).
hipError_t launch_project_paged(const uint16_t* k, const double* pf, uint16_t* a_first,
                                const int32_t* table, int n_layers, int64_t n_blocks, int64_t N, int Hk,
                                int B, int D, int R, uint32_t* err, hipStream_t stream);
// Both of the above, in that order and with the same results; one launch when
// both are small (a decode step), otherwise the two launches.
hipError_t launch_project_pair(const uint16_t* k, uint16_t* a_first, const int32_t* table, int n_layers,
                               int64_t n_blocks, int64_t N, int Hk, int B, uint32_t* err, const uint16_t* q,
                               uint16_t* q_out, int64_t n_q, const double* pf, int D, int R, hipStream_t stream);

// ---- scores (score_decode.hip, score_prefill.hip) --------------------------
struct ScoreArgs {
    const uint16_t* qp;     // [n_layers, S, M, Hq, R]
    const uint16_t* ag;     // A_g base [L, N, Hk, B, R]
    const int32_t* tables;  // [S, n] or null
    const int32_t* fill;    // [S] tokens held by each sequence's last block (n - 1), or null (all B)
    float* scores;          // [n_layers, S, n]
    uint32_t* err;
    int64_t N;              // max_blocks
    int64_t n;              // blocks per sequence
    int layer0, n_layers, S, M, Hq, Hk, B, R;
};
// Tokens of block b of sequence s that are scored: B, except the last block
// with a fill array (clamped to [0, B]; a value outside raises DEVERR_FILL).
__device__ inline int fill_of(const ScoreArgs& a, int s) {
    if (!a.fill) return a.B;
    const int f = a.fill[s];
    return f < 0 ? 0 : (f > a.B ? a.B : f);
}
// Score kernel choices.  AUTO is the library's own choice; the others are a
// debugging override (PRED_SCORE_PATH, pred_set_score_path) that routes every
// score call through one kernel family.
enum : int {
    SCORE_PATH_AUTO = 0,
    SCORE_PATH_DECODE = 1,        // vector-ALU streaming decode kernel (plain kernel where its layout does not fit)
    SCORE_PATH_GENERIC = 2,       // plain per-block kernel
    SCORE_PATH_DECODE_MFMA = 3,   // (a kind only) matrix-core streaming decode kernel
    SCORE_PATH_PREFILL = 4        // (a kind only) many-row MFMA kernel
};
// Streaming decode scorer when the shape allows it, else a plain per-block
// kernel; force = SCORE_PATH_AUTO, _DECODE or _GENERIC.
hipError_t launch_score_decode_or_generic(const ScoreArgs& a, int force, hipStream_t stream);
const char* score_decode_path_name(const ScoreArgs& a, int force);
// The kernel and its template arguments, e.g. "score_decode_kernel<lanes_per_row=4,...>".
std::string score_decode_variant(const ScoreArgs& a, int force);

// ---- per-row causal scores (score_rows.hip) --------------------------------
struct RowScoreArgs {
    const uint16_t* qp;     // [rows, Hq, R]; row r sits at position first_pos + r
    const uint16_t* ag;     // A_g base [L, N, Hk, B, R]
    const int32_t* table;   // [n] physical ids, or null for slots 0..n-1
    float* scores;          // [rows, stride]
    uint32_t* err;
    int64_t N;              // max_blocks
    int64_t layer;
    int64_t n;              // blocks of the sequence (table entries)
    int64_t rows, first_pos, stride;
    int Hq, Hk, B, R;
    int n_cu;               // compute units of the device (the MFMA kernel launches one workgroup per CU)
};
// Blocks complete at the position of row r: min(n, (first_pos + r + 1) / B).
// force = SCORE_PATH_GENERIC takes the plain per-cell kernel for every shape.
hipError_t launch_score_rows(const RowScoreArgs& a, int force, hipStream_t stream);
const char* score_rows_path_name(const RowScoreArgs& a, int force);

// ---- ranking (rank.hip) --------------------------------------------------
size_t rank_workspace_bytes(int64_t n, int64_t n_seg);
// Per-device set-up of the ranking kernels (their LDS limits); called by pred_create.
hipError_t rank_prepare();
// Static device scratch for callers that cannot allocate: its size, the set-up
// that finds its address on `device` (that device current; once per device,
// repeat calls are no-ops) and that address (null before the set-up).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t rank_scratch_prepare(int device);
void* rank_scratch(int device);
// Sort order of a ranking row.  Ascending (eviction order): the order key of
// the score, NaN first.  Descending (a keep set, larger score first): keys
// flipped inside [0, 0xFF800001] so that they stay below the padding key and
// key + 1 never overflows; NaN last.  Ties always go to the lower index.
// With ratio > 0 only the first min(n, (first_pos + row + 1) / ratio) entries
// of row `row` take part (the blocks complete at that row's position).
struct RowOrder {
    int desc;
    int64_t first_pos;
    int32_t ratio;

    __device__ inline uint32_t key(float v) const {
        if (!desc) return order_key(v);
        return v != v ? 0xFF800001u : 0xFF800000u - order_key(v);
    }
    __host__ __device__ inline int64_t row_len(int64_t row, int64_t n) const {
        if (ratio <= 0) return n;
        const int64_t c = (first_pos + row + 1) / ratio;
        return c < n ? c : n;
    }
};

hipError_t launch_rank(const float* scores, int64_t n, int64_t n_seg, int64_t k, RowOrder ro, int32_t* victims,
                       void* ws, hipStream_t stream);

}  // namespace pred
