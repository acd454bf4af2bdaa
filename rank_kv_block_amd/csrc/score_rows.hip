// Per-row causal block scores for a prefill chunk.  The qsa_select.rs page
// (prefill selection) scores each query row of a chunk against the blocks that
// are complete at that row's position -- (position + 1) / ratio of them -- and
// keeps every row's top-k.  Here the score is the predictor's (predictor.rs
// page, score_blocks), kept per row instead of maximised over rows, with the
// block size as the ratio:
//   out[r, b] = max over heads h, tokens t of q_proj[r, h, :] . A[layer, T[b], h / g, t, :]
// for b < complete(r) = min(n, (first_pos + r + 1) / B), and -inf for
// complete(r) <= b < stride.  A complete block whose table entry is outside
// [0, max_blocks) scores NaN and raises the device error word.
//
// Per row tile the contraction is Q_h [32 rows, R] x A_kv(h)^T [R, 32 keys] for
// every query head h, on v_mfma_f32_32x32x16_bf16 with f32 accumulation.  A wave
// keeps NKT tiles of 32 keys (consecutive tokens of consecutive blocks) of every
// kv head in registers as B operands, so a row's max over heads is an
// elementwise max of the heads' accumulators: the same lane and element hold
// the same (row, key) for every head.  Query vectors stream through LDS in
// stages of 32 rows x 4 heads, double-buffered: all 256 threads load the next
// stage with coalesced 16-byte reads while the current one is multiplied, and
// the waves read their A operands from LDS in the MFMA layout (vectors padded by
// 16 bytes so the rows of one read fall in distinct banks).  After a row tile's
// last head each lane reduces its key column's 16 rows over the B lanes of its
// block, and one lane per block writes the 16 row scores.
//
// Causality: the key tiles of a wave that start at or past the last row's
// complete blocks skip their MFMAs (all their scores are -inf); tiles are in key
// order, so the ones still needed are a prefix.
//
// Workgroups are (key group of 4 waves x NKT tiles) x (row part) with the row
// part fastest: with 4 or 8 parts every XCD (each takes every 8th workgroup)
// serves one or two parts, and its L2 holds only those parts' queries.
#include "common.h"
#include "kernels.h"

namespace pred {

namespace {

constexpr int kWaves = 4;
constexpr int kStageHeads = 4;                    // query heads per LDS stage
constexpr int kStageVecs = 32 * kStageHeads;      // query vectors per stage
constexpr int64_t kTargetWaves = 2048;            // two per SIMD

struct RowGeom {
    int64_t groups;       // key groups (kWaves * NKT * 32 keys each)
    int row_tiles;        // ceil(rows / 32)
    int parts;            // row parts
    int tiles_per_part;
    int stages;           // ceil(Hq / 4) stages per row tile
};

__device__ inline int64_t complete_blocks(const RowScoreArgs& a, int64_t r) {
    const int64_t c = (a.first_pos + r + 1) / a.B;
    return c < a.n ? c : a.n;
}

// R: projected width; HK: kv heads (keys of all of them sit in registers);
// NKT: 32-key tiles per wave.
template <int R, int HK, int NKT>
__global__ __launch_bounds__(256) void score_rows_kernel(RowScoreArgs a, RowGeom gm) {
    constexpr int RS = R / 16;                        // MFMA k-steps of 16
    constexpr int CPR = R / 8;                        // 16-byte pieces per query vector
    constexpr int ROWB = R * 2 + 16;                  // LDS bytes per query vector
    constexpr int PIECES = kStageVecs * CPR;          // 16-byte pieces per stage
    constexpr int PPT = (PIECES + 255) / 256;         // pieces per thread
    __shared__ __attribute__((aligned(16))) unsigned char lds[2][kStageVecs * ROWB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int part = (int)(blockIdx.x % gm.parts);
    const int64_t grp = blockIdx.x / gm.parts;
    const int rt_begin = part * gm.tiles_per_part;
    const int rt_end = (rt_begin + gm.tiles_per_part) < gm.row_tiles ? (rt_begin + gm.tiles_per_part) : gm.row_tiles;
    if (rt_begin >= rt_end) return;   // whole workgroup
    const int g = a.Hq / HK;
    const int col = lane & 31;        // key column of a tile / query row of a tile
    const int half = lane >> 5;       // which 8 of the 16 k-values of one MFMA step
    const int64_t n_keys = a.n * a.B;
    const int64_t key0 = (grp * kWaves + wave) * (NKT * 32);
    const int64_t slot_elems = (int64_t)HK * a.B * R;

    // B operands: this lane's key column of every tile and kv head.
    bf16x8_t kb[NKT][HK][RS];
    uint32_t live = 0;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
        const int64_t key = key0 + t * 32 + col;
        const uint16_t* src = a.ag;   // in bounds for lanes without a key; never used then
        if (key < n_keys) {
            const int64_t b = key / a.B;
            const int tok = (int)(key - b * a.B);
            const int64_t phys = a.table ? (int64_t)a.table[b] : b;
            if (phys >= 0 && phys < a.N) {
                src = a.ag + (a.layer * a.N + phys) * slot_elems + (int64_t)tok * R;
                live |= 1u << t;
            }
        }
#pragma unroll
        for (int k = 0; k < HK; ++k)
#pragma unroll
            for (int st = 0; st < RS; ++st) kb[t][k][st] = load8(src + (int64_t)k * a.B * R + st * 16 + half * 8);
    }

    f32x16_t rm[NKT];
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) rm[t][i] = -__builtin_inff();

    // stage (row tile rt, heads 4s..4s+3): piece p -> row p / (4 * CPR), head
    // (p / CPR) % 4, piece p % CPR; global reads run along a row's four heads,
    // LDS holds the stage head-major ([head][row]) for the MFMA reads
    // (plain functions of the piece index, so the prefetch registers stay registers)
    u32x4_t gq[PPT];
    auto piece_src = [&](int rt, int s, int p) -> const u32x4_t* {
        const int hv = p / CPR;
        int64_t r = (int64_t)rt * 32 + hv / kStageHeads;
        if (r >= a.rows) r = a.rows - 1;   // padding rows repeat a real row
        int h = s * kStageHeads + hv % kStageHeads;
        if (h >= a.Hq) h = a.Hq - 1;       // padding heads are never multiplied
        return reinterpret_cast<const u32x4_t*>(a.qp + (r * a.Hq + h) * R + (p % CPR) * 8);
    };
    auto piece_dst = [&](int buf, int p) -> u32x4_t* {
        const int hv = p / CPR;
        const int vec = (hv % kStageHeads) * 32 + hv / kStageHeads;
        return reinterpret_cast<u32x4_t*>(&lds[buf][vec * ROWB + (p % CPR) * 16]);
    };
    // the stage's heads against this wave's first ntl key tiles; the keys of
    // kv head k are registers, so k is unrolled and its heads of the stage
    // (those with h / g == k) run as a loop
    auto stage_mfma = [&](int buf, int s, int ntl) {
        const int h0 = s * kStageHeads;
        const int h_end = (h0 + kStageHeads) < a.Hq ? (h0 + kStageHeads) : a.Hq;
#pragma unroll
        for (int k = 0; k < HK; ++k) {
            const int lo = h0 > k * g ? h0 : k * g;
            const int hi = h_end < (k + 1) * g ? h_end : (k + 1) * g;
            for (int h = lo; h < hi; ++h) {   // wave-uniform bounds
                bf16x8_t qa[RS];
#pragma unroll
                for (int st = 0; st < RS; ++st)
                    qa[st] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                            &lds[buf][((h - h0) * 32 + col) * ROWB + (st * 2 + half) * 16]));
                f32x16_t acc[NKT];
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    if (t < ntl) {
                        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0], kb[t][k][0], f32x16_t{}, 0, 0, 0);
#pragma unroll
                        for (int st = 1; st < RS; ++st)
                            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[st], kb[t][k][st], acc[t], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int t = 0; t < NKT; ++t)
                    if (t < ntl)
#pragma unroll
                        for (int i = 0; i < 16; ++i) rm[t][i] = fmaxf(rm[t][i], acc[t][i]);
            }
        }
    };
    // row tile rt done: block maxima of every row, written out; rm reset
    auto epilogue = [&](int rt) {
        const int64_t r0 = (int64_t)rt * 32;
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            // element i of the accumulator is row (i / 4) * 8 + half * 4 + i % 4 of the tile
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float v = fmaxf(rm[t][i], lane_xor<1>(rm[t][i]));
                rm[t][i] = fmaxf(v, lane_xor<2>(v));
            }
            if (a.B >= 8)
#pragma unroll
                for (int i = 0; i < 16; ++i) rm[t][i] = fmaxf(rm[t][i], lane_xor<7>(rm[t][i]));
            if (a.B >= 16)
#pragma unroll
                for (int i = 0; i < 16; ++i) rm[t][i] = fmaxf(rm[t][i], lane_xor<15>(rm[t][i]));
            if (a.B >= 32)
#pragma unroll
                for (int i = 0; i < 16; ++i) rm[t][i] = fmaxf(rm[t][i], lane_xor<16>(rm[t][i]));
            const int64_t key = key0 + t * 32 + col;
            if ((col % a.B) == 0 && key < n_keys) {
                const int64_t b = key / a.B;
                const bool ok = (live >> t) & 1u;
                bool bad = false;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int64_t r = r0 + (i / 4) * 8 + half * 4 + (i % 4);
                    if (r < a.rows) {
                        const bool inside = b < complete_blocks(a, r);
                        bad |= inside && !ok;
                        a.scores[r * a.stride + b] =
                            inside ? (ok ? rm[t][i] : __uint_as_float(0x7FC00000u)) : -__builtin_inff();
                    }
                }
                if (bad) atomicOr(a.err, DEVERR_TABLE);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) rm[t][i] = -__builtin_inff();
        }
    };

    static_assert(PIECES % 256 == 0, "whole pieces per thread");
    int buf = 0;
#pragma unroll
    for (int i = 0; i < PPT; ++i) gq[i] = *piece_src(rt_begin, 0, tid + 256 * i);
#pragma unroll
    for (int i = 0; i < PPT; ++i) *piece_dst(0, tid + 256 * i) = gq[i];
    __syncthreads();
    for (int rt = rt_begin; rt < rt_end; ++rt) {
        // key tiles of this wave that hold a block complete for the tile's last row
        const int64_t last = ((int64_t)rt * 32 + 31) < a.rows ? ((int64_t)rt * 32 + 31) : a.rows - 1;
        const int64_t climit = complete_blocks(a, last);
        int ntl = 0;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            if ((key0 + t * 32) / a.B < climit) ntl = t + 1;
        for (int s = 0; s < gm.stages; ++s) {
            const bool last_stage = s + 1 == gm.stages;
            const int nrt = last_stage ? rt + 1 : rt;   // the next stage
            const int ns = last_stage ? 0 : s + 1;
            const bool more = nrt < rt_end;
            if (more)   // in flight while this stage is multiplied
#pragma unroll
                for (int i = 0; i < PPT; ++i) gq[i] = *piece_src(nrt, ns, tid + 256 * i);
            if (ntl > 0) stage_mfma(buf, s, ntl);
            if (more)   // that buffer was last read before the previous barrier
#pragma unroll
                for (int i = 0; i < PPT; ++i) *piece_dst(buf ^ 1, tid + 256 * i) = gq[i];
            __syncthreads();
            buf ^= 1;
        }
        epilogue(rt);
    }
}

// Any shape: one thread per (row, column of the stride), f32 dot products.
__global__ __launch_bounds__(256) void score_rows_generic_kernel(RowScoreArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.rows * a.stride) return;
    const int64_t r = i / a.stride;
    const int64_t b = i - r * a.stride;
    float* out = a.scores + i;
    if (b >= complete_blocks(a, r)) {
        *out = -__builtin_inff();
        return;
    }
    const int64_t phys = a.table ? (int64_t)a.table[b] : b;
    if (phys < 0 || phys >= a.N) {
        *out = __uint_as_float(0x7FC00000u);
        atomicOr(a.err, DEVERR_TABLE);
        return;
    }
    const int g = a.Hq / a.Hk;
    const uint16_t* slot = a.ag + (a.layer * a.N + phys) * ((int64_t)a.Hk * a.B * a.R);
    float best = -__builtin_inff();
    for (int h = 0; h < a.Hq; ++h) {
        const uint16_t* q = a.qp + (r * a.Hq + h) * a.R;
        for (int t = 0; t < a.B; ++t) {
            const uint16_t* k = slot + ((int64_t)(h / g) * a.B + t) * a.R;
            float d = 0.f;
            for (int j = 0; j < a.R; ++j)
                d = fmaf(__uint_as_float((uint32_t)q[j] << 16), __uint_as_float((uint32_t)k[j] << 16), d);
            best = fmaxf(best, d);
        }
    }
    *out = best;
}

// Columns [n, stride) of every row: no block there, -inf.
__global__ __launch_bounds__(256) void fill_tail_cols_kernel(float* scores, int64_t rows, int64_t stride,
                                                             int64_t n) {
    const int64_t w = stride - n;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * w) return;
    const int64_t r = i / w;
    scores[r * stride + n + (i - r * w)] = -__builtin_inff();
}

// 32-key tiles per wave: the keys take NKT * HK * R / 4 registers, kept at 128
constexpr int nkt_rows(int r, int hk) {
    const int t = 32 / (hk * (r / 16));
    return t < 1 ? 1 : (t > 4 ? 4 : t);
}

template <int R, int HK>
hipError_t launch_rk(const RowScoreArgs& a, hipStream_t st) {
    constexpr int NKT = nkt_rows(R, HK);
    RowGeom gm;
    const int64_t n_keys = a.n * a.B;
    const int64_t keys_per_group = (int64_t)kWaves * NKT * 32;
    gm.groups = (n_keys + keys_per_group - 1) / keys_per_group;
    gm.row_tiles = (int)((a.rows + 31) / 32);
    gm.stages = (a.Hq + kStageHeads - 1) / kStageHeads;
    int64_t parts = (kTargetWaves + gm.groups * kWaves - 1) / (gm.groups * kWaves);
    if (parts > gm.row_tiles) parts = gm.row_tiles;
    if (parts < 1) parts = 1;
    gm.tiles_per_part = (int)((gm.row_tiles + parts - 1) / parts);
    gm.parts = (gm.row_tiles + gm.tiles_per_part - 1) / gm.tiles_per_part;   // no empty parts
    const int64_t wgs = gm.groups * gm.parts;
    if (!grid_fits(wgs)) return hipErrorInvalidConfiguration;
    score_rows_kernel<R, HK, NKT><<<(unsigned)wgs, 256, 0, st>>>(a, gm);
    return hipGetLastError();
}

template <int HK>
hipError_t launch_hk(const RowScoreArgs& a, hipStream_t st) {
    switch (a.R) {
        case 16: return launch_rk<16, HK>(a, st);
        case 32: return launch_rk<32, HK>(a, st);
        case 64: return launch_rk<64, HK>(a, st);
        default:
            if constexpr (HK <= 4) return launch_rk<128, HK>(a, st);
            return hipErrorInvalidValue;   // excluded by rows_mfma_supported
    }
}

bool rows_mfma_supported(const RowScoreArgs& a) {
    const bool r_ok = a.R == 16 || a.R == 32 || a.R == 64 || a.R == 128;
    const bool hk_ok = a.Hk == 1 || a.Hk == 2 || a.Hk == 4 || a.Hk == 8;
    const bool b_ok = a.B == 8 || a.B == 16 || a.B == 32;
    return r_ok && hk_ok && b_ok && a.Hk * a.R <= 512;
}

}  // namespace

const char* score_rows_path_name(const RowScoreArgs& a) { return rows_mfma_supported(a) ? "mfma" : "generic"; }

hipError_t launch_score_rows(const RowScoreArgs& a, hipStream_t st) {
    if (a.rows <= 0 || a.stride <= 0) return hipSuccess;
    if (!rows_mfma_supported(a) || a.n == 0) {
        if (!grid_fits((a.rows * a.stride + 255) / 256)) return hipErrorInvalidConfiguration;
        score_rows_generic_kernel<<<(unsigned)((a.rows * a.stride + 255) / 256), 256, 0, st>>>(a);
        return hipGetLastError();
    }
    const int64_t n_cols = a.n < a.stride ? a.n : a.stride;   // columns that hold a block
    RowScoreArgs m = a;
    m.n = n_cols;
    const int64_t tail = a.rows * (a.stride - n_cols);
    if (!grid_fits((tail + 255) / 256)) return hipErrorInvalidConfiguration;
    hipError_t e;
    switch (a.Hk) {
        case 1: e = launch_hk<1>(m, st); break;
        case 2: e = launch_hk<2>(m, st); break;
        case 4: e = launch_hk<4>(m, st); break;
        default: e = launch_hk<8>(m, st); break;
    }
    if (e != hipSuccess || tail == 0) return e;
    fill_tail_cols_kernel<<<(unsigned)((tail + 255) / 256), 256, 0, st>>>(a.scores, a.rows, a.stride, n_cols);
    return hipGetLastError();
}

}  // namespace pred
