// Projection kernels: Q @ P and K @ P with float64 accumulation and one RNE
// rounding to bf16 (predictor.rs page: project_q, project_kv_block).
//
// Products of two bf16 values are exact in float64 and a float64 sum of
// head_dim of them loses nothing for realistic data, so every output is the
// correctly rounded bf16 of the exact dot product; a float32 accumulator would
// miss that by more than one bf16 ulp for outputs near zero.
//
// Main path: float64 MFMA (v_mfma_f64_16x16x4_f64).  A wave owns 16 output
// columns and keeps the matching slice of P as B operands in registers (lane
// group q = lane / 16 takes the head_dim range [q*D/4, (q+1)*D/4), one value
// per k-step), then streams tiles of 16 input vectors as A operands, converted
// bf16 -> float64 on the fly.  Each 16x16 float64 tile is rounded to bf16 in
// the epilogue and written either densely (project_q) or into the A_g slot the
// block table names, transposing [B, Hk] -> [Hk, B] (project_kv_block).
//
// Small calls (a decode step projects ~1000-4000 vectors, too few 16-vector
// tiles to give every SIMD a wave) split the head_dim sum instead: the four
// waves of a workgroup take a quarter of head_dim each for the same 16x16
// tile, so each runs a quarter of the MFMA chain, and wave 0 adds the three
// other float64 partials from LDS before the one rounding.
//
// Fallback (head_dim not in {32, 64, 128, 256} or r not a multiple of 16): one
// lane per vector with float64 FMAs, P read through the scalar cache.
#include "common.h"
#include "kernels.h"

// tile count below which a call splits head_dim across a workgroup's waves
// (at 1024 tiles both kernels take 9.3 us; below 4096 two small projections
// can then share one launch)
#ifndef PRED_PROJ_SPLITK_BELOW
#define PRED_PROJ_SPLITK_BELOW 4096
#endif

namespace pred {

namespace {

template <int RC>
__device__ inline void project_vector(const uint16_t* __restrict__ src, const double* __restrict__ pf,
                                      int D, int R, int j0, uint16_t* __restrict__ dst) {
    double acc[RC];
#pragma unroll
    for (int j = 0; j < RC; ++j) acc[j] = 0.0;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    for (int dc = 0; dc < (D >> 3); ++dc) {
        const uint4 w = s4[dc];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        double x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = (double)bf16_lo(ww[e]);
            x[2 * e + 1] = (double)bf16_hi(ww[e]);
        }
        const double* prow = pf + (int64_t)(dc << 3) * R + j0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
            for (int j = 0; j < RC; ++j) acc[j] = __builtin_fma(x[e], prow[e * R + j], acc[j]);
        }
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int c = 0; c < RC / 8; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = f64_to_bf16_rne(acc[8 * c + 2 * e]);
            const uint32_t hi = f64_to_bf16_rne(acc[8 * c + 2 * e + 1]);
            w[e] = lo | (hi << 16);
        }
        d4[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

template <int RC>
__global__ __launch_bounds__(256) void project_dense_kernel(const uint16_t* __restrict__ in,
                                                            const double* __restrict__ pf,
                                                            uint16_t* __restrict__ out, int64_t n_vec,
                                                            int D, int R) {
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= n_vec) return;
    const int j0 = blockIdx.y * RC;
    project_vector<RC>(in + v * D, pf, D, R, j0, out + v * R + j0);
}

// Vector v enumerates k [n_layers, n_blocks, B, Hk, D] in memory order:
// v = ((l*n_blocks + i)*B + t)*Hk + kv.  Its output row is
// A_g[layer0 + l, table[l, i], kv, t, :] (slot layout [Hk, B, R]).
template <int RC>
__global__ __launch_bounds__(256) void project_paged_kernel(
    const uint16_t* __restrict__ k, const double* __restrict__ pf, uint16_t* __restrict__ a_first,
    const int32_t* __restrict__ table, int64_t n_vec, int64_t n_blocks, int64_t N, int Hk, int B, int D, int R,
    uint32_t* __restrict__ err) {
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= n_vec) return;
    const int64_t per_block = (int64_t)B * Hk;
    const int64_t li = v / per_block;  // l * n_blocks + i
    const int rem = (int)(v - li * per_block);
    const int t = rem / Hk;
    const int kv = rem - t * Hk;
    const int64_t l = li / n_blocks;
    const int64_t phys = table ? (int64_t)table[li] : (li - l * n_blocks);
    if (phys < 0 || phys >= N) {
        if (rem == 0 && blockIdx.y == 0) atomicOr(err, DEVERR_TABLE);
        return;
    }
    const int j0 = blockIdx.y * RC;
    uint16_t* dst = a_first + (((l * N + phys) * Hk + kv) * B + t) * (int64_t)R + j0;
    project_vector<RC>(k + v * D, pf, D, R, j0, dst);
}

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// Where the projection of input vector `row` goes.
struct OutMap {
    uint16_t* out;          // dense: [n_vec, R]; paged: first layer's A_g slab
    const int32_t* table;   // paged: [n_layers, n_blocks] or null (identity)
    uint32_t* err;
    int64_t n_blocks, N;
    int Hk, B, R;
    bool paged;

    // Element offset of the row's output, or -1 when its table entry is invalid.
    __device__ inline int64_t row_offset(int64_t row) const {
        if (!paged) return row * R;
        const int64_t per_block = (int64_t)B * Hk;
        const int64_t li = row / per_block;
        const int rem = (int)(row - li * per_block);
        const int t = rem / Hk;
        const int kv = rem - t * Hk;
        const int64_t l = li / n_blocks;
        const int64_t phys = table ? (int64_t)table[li] : (li - l * n_blocks);
        if (phys < 0 || phys >= N) return -1;
        return (((l * N + phys) * Hk + kv) * B + t) * (int64_t)R;
    }
};

template <int DG>
__device__ inline void load_row_quarter(const uint16_t* in, int64_t row, int q, uint4 (&w)[DG / 8]) {
    const uint4* src = reinterpret_cast<const uint4*>(in + row * (4 * DG) + q * DG);
#pragma unroll
    for (int c = 0; c < DG / 8; ++c) w[c] = src[c];
}

// unit = (vector group, 16-column tile); a vector group is VT tiles of 16 vectors.
template <int DG>
__global__ __launch_bounds__(256) void project_mfma_kernel(const uint16_t* __restrict__ in,
                                                           const double* __restrict__ pf, OutMap om,
                                                           int64_t n_vec, int VT, int64_t units) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= units) return;
    const int R = om.R;
    const int jtiles = R >> 4;
    const int jt = (int)(unit % jtiles);
    const int64_t vgrp = unit / jtiles;
    const int col = lane & 15;
    const int q = lane >> 4;
    const int j = jt * 16 + col;

    const int64_t v_first = vgrp * VT * 16;
    if (v_first >= n_vec) return;
    const int64_t v_end = (v_first + (int64_t)VT * 16) < n_vec ? (v_first + (int64_t)VT * 16) : n_vec;
    auto clamp_row = [&](int64_t r) { return r < n_vec ? r : n_vec - 1; };  // tail rows are computed, not stored

    // the first input tile and this wave's slice of P are requested together
    uint4 w[DG / 8], wn[DG / 8];
    load_row_quarter<DG>(in, clamp_row(v_first + col), q, w);
    double pb[DG];   // B operands: P[q*DG + s][j]
#pragma unroll
    for (int s = 0; s < DG; ++s) pb[s] = pf[(int64_t)(q * DG + s) * R + j];

    for (int64_t v0 = v_first; v0 < v_end; v0 += 16) {
        if (v0 + 16 < v_end) load_row_quarter<DG>(in, clamp_row(v0 + 16 + col), q, wn);
        // two accumulators (even / odd k-steps) halve the dependent MFMA chain
        f64x4_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int c = 0; c < DG / 8; ++c) {
            const uint32_t ww[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_lo(ww[e]), pb[c * 8 + 2 * e], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_hi(ww[e]), pb[c * 8 + 2 * e + 1], acc1, 0, 0, 0);
            }
        }
        const f64x4_t acc = acc0 + acc1;
        // acc[v] of lane group q is output (row v0 + q + 4v, column j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t row = v0 + q + 4 * v;
            if (row < v_end) {
                const int64_t off = om.row_offset(row);
                if (off >= 0) om.out[off + j] = f64_to_bf16_rne(acc[v]);
                else if (col == 0 && jt == 0) atomicOr(om.err, DEVERR_TABLE);
            }
        }
        if (v0 + 16 < v_end) {
#pragma unroll
            for (int c = 0; c < DG / 8; ++c) w[c] = wn[c];
        }
    }
}

// DW consecutive bf16 input values as DW / 2 packed words (DW in {2, 4, 8, 16}).
template <int DW>
__device__ inline void load_words(const uint16_t* p, uint32_t (&wd)[DW / 2]) {
    if constexpr (DW >= 8) {
#pragma unroll
        for (int c = 0; c < DW / 8; ++c) {
            const uint4 v = reinterpret_cast<const uint4*>(p)[c];
            wd[4 * c] = v.x; wd[4 * c + 1] = v.y; wd[4 * c + 2] = v.z; wd[4 * c + 3] = v.w;
        }
    } else if constexpr (DW == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        wd[0] = v.x; wd[1] = v.y;
    } else {
        wd[0] = *reinterpret_cast<const uint32_t*>(p);
    }
}

// One workgroup per (16-vector tile, 16-column tile); wave w sums head_dim
// values [w*D/4, (w+1)*D/4), lane group q the DW of them starting at
// w*D/4 + q*DW (DW = D/16 k-steps per wave).  `unit` is the workgroup's tile.
template <int DW>
__device__ inline void splitk_unit(const uint16_t* __restrict__ in, const double* __restrict__ pf, const OutMap& om,
                                   int64_t n_vec, int64_t unit, f64x4_t (*part)[64]) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int D = 16 * DW;
    const int R = om.R;
    const int jtiles = R >> 4;
    const int jt = (int)(unit % jtiles);
    const int64_t v0 = (unit / jtiles) * 16;
    const int col = lane & 15;
    const int q = lane >> 4;
    const int j = jt * 16 + col;
    const int k0 = w * 4 * DW + q * DW;   // this lane's first head_dim index
    const int64_t row_in = (v0 + col) < n_vec ? (v0 + col) : n_vec - 1;   // tail rows computed, not stored

    uint32_t wd[DW / 2];
    load_words<DW>(in + row_in * D + k0, wd);
    double pb[DW];
#pragma unroll
    for (int s = 0; s < DW; ++s) pb[s] = pf[(int64_t)(k0 + s) * R + j];
    // output offsets of this lane's four rows, looked up (block table) before the
    // MFMA chain so the lookup's latency overlaps it
    int64_t off[4];
    if (w == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t row = v0 + q + 4 * v;
            off[v] = row < n_vec ? om.row_offset(row) : -2;
        }
    }

    f64x4_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int e = 0; e < DW / 2; ++e) {
        acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_lo(wd[e]), pb[2 * e], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_hi(wd[e]), pb[2 * e + 1], acc1, 0, 0, 0);
    }
    f64x4_t acc = acc0 + acc1;
    if (w > 0) part[w - 1][lane] = acc;
    __syncthreads();
    if (w > 0) return;
    acc += part[0][lane];
    acc += part[1][lane];
    acc += part[2][lane];
    // acc[v] of lane group q is output (row v0 + q + 4v, column j); off -1: invalid
    // table entry, -2: tail row past n_vec
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        if (off[v] >= 0) om.out[off[v] + j] = f64_to_bf16_rne(acc[v]);
        else if (off[v] == -1 && col == 0 && jt == 0) atomicOr(om.err, DEVERR_TABLE);
    }
}

template <int DW>
__global__ __launch_bounds__(256) void project_splitk_kernel(const uint16_t* __restrict__ in,
                                                             const double* __restrict__ pf, OutMap om,
                                                             int64_t n_vec, int64_t units) {
    __shared__ f64x4_t part[3][64];
    if ((int64_t)blockIdx.x >= units) return;   // whole workgroup
    splitk_unit<DW>(in, pf, om, n_vec, blockIdx.x, part);
}

// Two small projections in one launch (a decode step's new KV blocks and its
// queries): workgroups [0, units0) take the first job's tiles, the rest the
// second's.  Each tile is computed exactly as by project_splitk_kernel.
template <int DW>
__global__ __launch_bounds__(256) void project_splitk_pair_kernel(const uint16_t* __restrict__ in0, OutMap om0,
                                                                  int64_t n0, int64_t units0,
                                                                  const uint16_t* __restrict__ in1, OutMap om1,
                                                                  int64_t n1, int64_t units1,
                                                                  const double* __restrict__ pf) {
    __shared__ f64x4_t part[3][64];
    const int64_t u = blockIdx.x;
    if (u < units0) splitk_unit<DW>(in0, pf, om0, n0, u, part);
    else if (u - units0 < units1) splitk_unit<DW>(in1, pf, om1, n1, u - units0, part);
}

bool mfma_path(int D, int R) { return (D == 32 || D == 64 || D == 128 || D == 256) && R % 16 == 0; }

hipError_t launch_mfma(const uint16_t* in, const double* pf, const OutMap& om, int64_t n_vec, int D,
                       hipStream_t stream) {
    const int64_t vtiles = (n_vec + 15) / 16;
    const int jtiles = om.R / 16;
    if (!grid_fits(vtiles * jtiles)) return hipErrorInvalidConfiguration;
    if (vtiles * jtiles < PRED_PROJ_SPLITK_BELOW) {
        // too few tiles to occupy the SIMDs: split head_dim over a workgroup's waves
        const int64_t units = vtiles * jtiles;
        switch (D) {
            case 32: project_splitk_kernel<2><<<(unsigned)units, 256, 0, stream>>>(in, pf, om, n_vec, units); break;
            case 64: project_splitk_kernel<4><<<(unsigned)units, 256, 0, stream>>>(in, pf, om, n_vec, units); break;
            case 128: project_splitk_kernel<8><<<(unsigned)units, 256, 0, stream>>>(in, pf, om, n_vec, units); break;
            default: project_splitk_kernel<16><<<(unsigned)units, 256, 0, stream>>>(in, pf, om, n_vec, units); break;
        }
        return hipGetLastError();
    }
    // about two waves per SIMD when there is that much work, one vector tile per wave otherwise
    int64_t vt = (vtiles * jtiles) / 2048;
    if (vt < 1) vt = 1;
    const int64_t units = ((vtiles + vt - 1) / vt) * jtiles;
    const unsigned grid = (unsigned)((units + 3) / 4);
    switch (D) {
        case 32: project_mfma_kernel<8><<<grid, 256, 0, stream>>>(in, pf, om, n_vec, (int)vt, units); break;
        case 64: project_mfma_kernel<16><<<grid, 256, 0, stream>>>(in, pf, om, n_vec, (int)vt, units); break;
        case 128: project_mfma_kernel<32><<<grid, 256, 0, stream>>>(in, pf, om, n_vec, (int)vt, units); break;
        default: project_mfma_kernel<64><<<grid, 256, 0, stream>>>(in, pf, om, n_vec, (int)vt, units); break;
    }
    return hipGetLastError();
}

// Output chunk width: the widest of 64/32/16/8 that divides R, narrowed while
// the grid would leave the 1024 SIMDs with fewer than ~4 waves each.
int pick_rc(int R, int64_t n_vec) {
    const int opts[4] = {64, 32, 16, 8};
    int rc = 8;
    for (int o : opts)
        if (R % o == 0) { rc = o; break; }
    const int64_t waves = (n_vec + 63) / 64;
    while (rc > 8 && waves * (R / rc) < 4096 && R % (rc / 2) == 0) rc /= 2;
    return rc;
}

}  // namespace

hipError_t launch_project_dense(const uint16_t* in, const double* pf, uint16_t* out, int64_t n_vec,
                                int D, int R, hipStream_t stream) {
    if (n_vec <= 0) return hipSuccess;
    if (mfma_path(D, R)) {
        OutMap om{out, nullptr, nullptr, 0, 0, 0, 0, R, false};
        return launch_mfma(in, pf, om, n_vec, D, stream);
    }
    const int rc = pick_rc(R, n_vec);
    if (!grid_fits((n_vec + 255) / 256)) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((n_vec + 255) / 256), (unsigned)(R / rc));
    switch (rc) {
        case 64: project_dense_kernel<64><<<grid, 256, 0, stream>>>(in, pf, out, n_vec, D, R); break;
        case 32: project_dense_kernel<32><<<grid, 256, 0, stream>>>(in, pf, out, n_vec, D, R); break;
        case 16: project_dense_kernel<16><<<grid, 256, 0, stream>>>(in, pf, out, n_vec, D, R); break;
        default: project_dense_kernel<8><<<grid, 256, 0, stream>>>(in, pf, out, n_vec, D, R); break;
    }
    return hipGetLastError();
}

hipError_t launch_project_paged(const uint16_t* k, const double* pf, uint16_t* a_first,
                                const int32_t* table, int n_layers, int64_t n_blocks, int64_t N, int Hk,
                                int B, int D, int R, uint32_t* err, hipStream_t stream) {
    const int64_t n_vec = (int64_t)n_layers * n_blocks * B * Hk;
    if (n_vec <= 0) return hipSuccess;
    if (mfma_path(D, R)) {
        OutMap om{a_first, table, err, n_blocks, N, Hk, B, R, true};
        return launch_mfma(k, pf, om, n_vec, D, stream);
    }
    const int rc = pick_rc(R, n_vec);
    if (!grid_fits((n_vec + 255) / 256)) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((n_vec + 255) / 256), (unsigned)(R / rc));
#define PRED_PAGED(RCV)                                                                                      \
    project_paged_kernel<RCV><<<grid, 256, 0, stream>>>(k, pf, a_first, table, n_vec, n_blocks, N, Hk, B, D, R, err)
    switch (rc) {
        case 64: PRED_PAGED(64); break;
        case 32: PRED_PAGED(32); break;
        case 16: PRED_PAGED(16); break;
        default: PRED_PAGED(8); break;
    }
#undef PRED_PAGED
    return hipGetLastError();
}

hipError_t launch_project_pair(const uint16_t* k, uint16_t* a_first, const int32_t* table, int n_layers,
                               int64_t n_blocks, int64_t N, int Hk, int B, uint32_t* err, const uint16_t* q,
                               uint16_t* q_out, int64_t n_q, const double* pf, int D, int R, hipStream_t stream) {
    const int64_t n_k = (int64_t)n_layers * n_blocks * B * Hk;
    const int jtiles = R / 16;
    const int64_t units_k = (n_k + 15) / 16 * jtiles;
    const int64_t units_q = (n_q + 15) / 16 * jtiles;
    // one launch only where each job on its own would take the split-head_dim kernel
    if (n_k > 0 && n_q > 0 && mfma_path(D, R) && units_k < PRED_PROJ_SPLITK_BELOW &&
        units_q < PRED_PROJ_SPLITK_BELOW) {
        const OutMap om_k{a_first, table, err, n_blocks, N, Hk, B, R, true};
        const OutMap om_q{q_out, nullptr, nullptr, 0, 0, 0, 0, R, false};
        const unsigned grid = (unsigned)(units_k + units_q);
#define PRED_PAIR(DWV)                                                                                       \
    project_splitk_pair_kernel<DWV><<<grid, 256, 0, stream>>>(k, om_k, n_k, units_k, q, om_q, n_q, units_q, pf)
        switch (D) {
            case 32: PRED_PAIR(2); break;
            case 64: PRED_PAIR(4); break;
            case 128: PRED_PAIR(8); break;
            default: PRED_PAIR(16); break;
        }
#undef PRED_PAIR
        return hipGetLastError();
    }
    hipError_t e = launch_project_paged(k, pf, a_first, table, n_layers, n_blocks, N, Hk, B, D, R, err, stream);
    if (e != hipSuccess) return e;
    return launch_project_dense(q, pf, q_out, n_q, D, R, stream);
}

}  // namespace pred
