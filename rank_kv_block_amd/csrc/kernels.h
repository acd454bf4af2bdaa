// Launchers of the predictor's HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// ---- scores (score_decode.hip, score_prefill.hip) --------------------------
struct ScoreArgs {
    const uint16_t* qp;     // [n_layers, S, M, Hq, R]
    const uint16_t* ag;     // A_g base [L, N, Hk, B, R]
    const int32_t* tables;  // [S, n] or null
    float* scores;          // [n_layers, S, n]
    uint32_t* err;
    int64_t N;              // max_blocks
    int64_t n;              // blocks per sequence
    int layer0, n_layers, S, M, Hq, Hk, B, R;
};
// Streaming decode scorer when the shape allows it, else a plain per-block kernel.
hipError_t launch_score_decode_or_generic(const ScoreArgs& a, hipStream_t stream);
const char* score_decode_path_name(const ScoreArgs& a);

// ---- ranking (rank.hip) --------------------------------------------------
size_t rank_workspace_bytes(int64_t n, int64_t n_seg);
hipError_t launch_rank(const float* scores, int64_t n, int64_t n_seg, int64_t k, int32_t* victims, void* ws,
                       hipStream_t stream);

}  // namespace pred
