// Projection kernels: Q @ P and K @ P with float64 accumulation and one RNE
// rounding to bf16 (predictor.rs page: project_q, project_kv_block).
//
// One lane owns one input vector (D bf16) and RC of its R outputs.  Products
// of two bf16 values are exact in float64 and a float64 sum of head_dim of them
// loses nothing for realistic data, so the output is the correctly rounded
// bf16 of the exact dot product; a float32 accumulator would miss that by more
// than one bf16 ulp for outputs near zero.
//
// P is read as float64 [D, R] (converted once at create time) through the
// scalar data cache: every lane of a wave needs the same P element at the same
// time, so the compiler issues uniform scalar loads and the FMAs take P from
// SGPRs.  A copy in LDS would cost one 8-byte return per lane per FMA from
// the LDS, four times the fp64 FMA rate of the CU.
#include "common.h"
#include "kernels.h"

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
    const int rc = pick_rc(R, n_vec);
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
    const int rc = pick_rc(R, n_vec);
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

}  // namespace pred
