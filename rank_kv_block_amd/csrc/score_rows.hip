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
// Per row tile of 32 rows the contraction is A_kv(h) [32 keys, R] x Q_h^T [R,
// 32 rows] for every query head h, on v_mfma_f32_32x32x16_bf16 with f32
// accumulation (keys as the A operand, so a lane holds one query row and 16
// keys of the tile: element i is key (i / 4) * 8 + 4 * (lane / 32) + i % 4).
// The four waves of a workgroup share one range of NKT tiles of 32 keys
// (consecutive tokens of consecutive blocks) and split the query heads: wave w
// takes heads [w * Hq / 4, (w + 1) * Hq / 4), whose one or two kv heads' keys
// it keeps in registers.  Each query operand read from LDS then serves NKT
// tiles.  After every head a lane folds its 16 products into the running
// maxima of the tile's blocks (B / 2 elements per block, max3 chains); after a
// row tile the two lane halves are combined, the four waves' partial maxima
// meet in LDS and the workgroup writes each row's blocks with stores that run
// along the row.
//
// Query vectors stream through LDS in stages of 32 rows x (4 waves x SH heads),
// double-buffered: all 256 threads load the next stage with 16-byte reads while
// the current one is multiplied, and each wave reads its own heads' vectors in
// the MFMA layout (vectors padded by 16 bytes so the rows of one read fall in
// distinct banks).
//
// Causality: key tiles that start at or past the last row's complete blocks
// skip their MFMAs (their scores are all -inf); tiles are in key order, so the
// ones still needed are a prefix, the same for every wave.
//
// A workgroup holds PRED_ROWS_KG key groups of four waves that share each query
// stage.  Workgroups are (key range) x (row part) with the row part fastest:
// with 4 or 8 parts every XCD (each takes every 8th workgroup) serves one or
// two parts, and its L2 holds only those parts' queries.
#include "common.h"
#include "kernels.h"

// Tuning knobs (compile-time), each measured on the 2048-row prefill chunk
// (r = 64, 8 kv heads): 96 key registers (3 tiles) keep two waves per SIMD
// (128 registers: 4 tiles, one wave, 580 us; 96: 455 us); 8192 target waves
// give 8 row parts there, so an XCD's L2 holds one part's 1 MiB of queries
// (444 us); two key groups per workgroup share each query stage, halving the
// query reads (427-440 us).  Two-head stages at r = 64 measured no better.
#ifndef PRED_ROWS_TARGET_WAVES
#define PRED_ROWS_TARGET_WAVES 8192
#endif
// key groups per workgroup: KG groups of four waves share each query stage
#ifndef PRED_ROWS_KG
#define PRED_ROWS_KG 2
#endif
// stages of two heads per wave for r up to this (one head above)
#ifndef PRED_ROWS_SH2_MAX_R
#define PRED_ROWS_SH2_MAX_R 32
#endif

namespace pred {

namespace {

constexpr int kWaves = 4;                         // waves of one key group (they split the heads)
constexpr int kKG = PRED_ROWS_KG;
constexpr int kThreads = 256 * kKG;
constexpr int64_t kTargetWaves = PRED_ROWS_TARGET_WAVES;

struct RowGeom {
    int64_t groups;       // workgroups along the keys (kKG * NKT * 32 keys each)
    int row_tiles;        // ceil(rows / 32)
    int parts;            // row parts
    int tiles_per_part;
    int stages;           // stages per row tile: (Hq / 4) / SH
};

__device__ inline int64_t complete_blocks(const RowScoreArgs& a, int64_t r) {
    const int64_t c = (a.first_pos + r + 1) / a.B;
    return c < a.n ? c : a.n;
}

// R: projected width; KPW: kv heads per wave (2 when Hk = 8, else 1); NKT:
// 32-key tiles per wave; SH: heads per wave per stage; BS: block size.
template <int R, int KPW, int NKT, int SH, int BS>
__global__ __launch_bounds__(kThreads) void score_rows_kernel(RowScoreArgs a, RowGeom gm) {
    constexpr int RS = R / 16;                        // MFMA k-steps of 16
    constexpr int CPR = R / 8;                        // 16-byte pieces per query vector
    constexpr int ROWB = R * 2 + 16;                  // LDS bytes per query vector
    constexpr int VEC = 32 * kWaves * SH;             // query vectors per stage
    constexpr int PIECES = VEC * CPR;                 // 16-byte pieces per stage
    constexpr int PPT = (PIECES + kThreads - 1) / kThreads;   // pieces per thread
    constexpr bool kFull = PIECES % kThreads == 0;            // every thread has PPT pieces
    constexpr int BPT = 32 / BS;                      // blocks per key tile
    constexpr int EPB = BS / 2;                       // accumulator elements per block in a lane
    constexpr int NB = NKT * BPT;                     // blocks of a key group
    __shared__ __attribute__((aligned(16))) unsigned char lds[2][VEC * ROWB];
    __shared__ float red[kKG][kWaves][NB * 32];       // partial maxima [key group][wave][block][row]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = (tid >> 6) % kWaves;             // head quarter
    const int kg = (tid >> 6) / kWaves;               // key group of this wave
    const int part = (int)(blockIdx.x % gm.parts);
    const int64_t grp = blockIdx.x / gm.parts;
    const int rt_begin = part * gm.tiles_per_part;
    const int rt_end = (rt_begin + gm.tiles_per_part) < gm.row_tiles ? (rt_begin + gm.tiles_per_part) : gm.row_tiles;
    if (rt_begin >= rt_end) return;   // whole workgroup
    const int qh = a.Hq / kWaves;     // heads per wave
    const int g = a.Hq / a.Hk;
    const int kv_first = (wave * qh) / g;
    const int col = lane & 31;        // key of a tile (A operand) / query row (B operand)
    const int half = lane >> 5;       // which 8 of the 16 k-values of one MFMA step
    const int64_t n_keys = a.n * BS;
    const int64_t key0 = (grp * kKG + kg) * (NKT * 32);
    const int64_t slot_elems = (int64_t)a.Hk * BS * R;

    // A operands: this lane's key of every tile, for the wave's kv heads.
    bf16x8_t kb[NKT][KPW][RS];
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
        const int64_t key = key0 + t * 32 + col;
        const uint16_t* src = a.ag;   // in bounds for lanes without a valid key; their blocks are never stored
        if (key < n_keys) {
            const int64_t b = key / BS;
            const int tok = (int)(key - b * BS);
            const int64_t phys = a.table ? (int64_t)a.table[b] : b;
            if (phys >= 0 && phys < a.N) src = a.ag + (a.layer * a.N + phys) * slot_elems + (int64_t)tok * R;
        }
#pragma unroll
        for (int k = 0; k < KPW; ++k) {
            const int kv = (kv_first + k) < a.Hk ? kv_first + k : a.Hk - 1;
#pragma unroll
            for (int st = 0; st < RS; ++st) kb[t][k][st] = load8(src + (int64_t)kv * BS * R + st * 16 + half * 8);
        }
    }

    float rm[NKT][BPT];
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int bi = 0; bi < BPT; ++bi) rm[t][bi] = -__builtin_inff();

    // stage (row tile rt, stage s): vector v = row * (4 SH) + slot, slot = wave * SH + j,
    // holding head wave * qh + s * SH + j of that row; LDS keeps it at slot * 32 + row
    u32x4_t gq[PPT];
    auto piece_src = [&](int rt, int s, int p) -> const u32x4_t* {
        const int v = p / CPR;
        const int slot = v % (kWaves * SH);
        int64_t r = (int64_t)rt * 32 + v / (kWaves * SH);
        if (r >= a.rows) r = a.rows - 1;   // padding rows repeat a real row
        const int h = (slot / SH) * qh + s * SH + slot % SH;
        return reinterpret_cast<const u32x4_t*>(a.qp + (r * a.Hq + h) * R + (p % CPR) * 8);
    };
    auto piece_dst = [&](int buf, int p) -> u32x4_t* {
        const int v = p / CPR;
        const int vec = (v % (kWaves * SH)) * 32 + v / (kWaves * SH);
        return reinterpret_cast<u32x4_t*>(&lds[buf][vec * ROWB + (p % CPR) * 16]);
    };
    // this wave's heads of stage s against its first ntl key tiles
    auto stage_mfma = [&](int buf, int s, int ntl) {
#pragma unroll
        for (int j = 0; j < SH; ++j) {
            const int h = wave * qh + s * SH + j;
            const int lk = h / g - kv_first;   // which of the wave's kv heads (wave-uniform)
            bf16x8_t qb[RS];
#pragma unroll
            for (int st = 0; st < RS; ++st)
                qb[st] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                        &lds[buf][((wave * SH + j) * 32 + col) * ROWB + (st * 2 + half) * 16]));
#pragma unroll
            for (int k = 0; k < KPW; ++k) {
                if (KPW > 1 && k != lk) continue;
                // each tile's chain, then its fold: the fold of tile t overlaps the
                // chain of tile t + 1, and only two accumulators are live
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    if (t < ntl) {
                        f32x16_t acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t][k][0], qb[0], f32x16_t{}, 0, 0, 0);
#pragma unroll
                        for (int st = 1; st < RS; ++st)
                            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t][k][st], qb[st], acc, 0, 0, 0);
#pragma unroll
                        for (int bi = 0; bi < BPT; ++bi) {
                            float m = rm[t][bi];
#pragma unroll
                            for (int e = 0; e < EPB; e += 2) m = fmaxf(m, fmaxf(acc[bi * EPB + e], acc[bi * EPB + e + 1]));
                            rm[t][bi] = m;
                        }
                    }
                }
            }
        }
    };
    // row tile rt done: combine the lane halves and the waves, store, reset
    auto epilogue = [&](int rt) {
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int bi = 0; bi < BPT; ++bi) {
                const float v = fmaxf(rm[t][bi], lane_xor<32>(rm[t][bi]));
                if (half == 0) red[kg][wave][(t * BPT + bi) * 32 + col] = v;
                rm[t][bi] = -__builtin_inff();
            }
        __syncthreads();
        const int64_t r0 = (int64_t)rt * 32;
        const int64_t blk0 = grp * kKG * NB;          // first block of the workgroup
        for (int i = tid; i < kKG * NB * 32; i += kThreads) {
            const int row = i / (kKG * NB);           // consecutive threads: consecutive blocks of a row
            const int bw = i - row * (kKG * NB);
            const int g2 = bw / NB;
            const int blk = bw - g2 * NB;
            const int64_t r = r0 + row;
            const int64_t b = blk0 + bw;
            if (r < a.rows && b < a.n) {
                float v = fmaxf(fmaxf(red[g2][0][blk * 32 + row], red[g2][1][blk * 32 + row]),
                                fmaxf(red[g2][2][blk * 32 + row], red[g2][3][blk * 32 + row]));
                if (b >= complete_blocks(a, r)) {
                    v = -__builtin_inff();
                } else if (a.table) {
                    const int64_t phys = a.table[b];
                    if (phys < 0 || phys >= a.N) {
                        v = __uint_as_float(0x7FC00000u);
                        atomicOr(a.err, DEVERR_TABLE);
                    }
                }
                a.scores[r * a.stride + b] = v;
            }
        }
        // red is written again only after the next row tile's stage barriers
    };

    int buf = 0;
#pragma unroll
    for (int i = 0; i < PPT; ++i)
        if (kFull || tid + kThreads * i < PIECES) gq[i] = *piece_src(rt_begin, 0, tid + kThreads * i);
#pragma unroll
    for (int i = 0; i < PPT; ++i)
        if (kFull || tid + kThreads * i < PIECES) *piece_dst(0, tid + kThreads * i) = gq[i];
    __syncthreads();
    for (int rt = rt_begin; rt < rt_end; ++rt) {
        // key tiles that hold a block complete for the tile's last row
        const int64_t last = ((int64_t)rt * 32 + 31) < a.rows ? ((int64_t)rt * 32 + 31) : a.rows - 1;
        const int64_t climit = complete_blocks(a, last);
        int ntl = 0;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            if ((key0 + t * 32) / BS < climit) ntl = t + 1;
        for (int s = 0; s < gm.stages; ++s) {
            const bool last_stage = s + 1 == gm.stages;
            const int nrt = last_stage ? rt + 1 : rt;   // the next stage
            const int ns = last_stage ? 0 : s + 1;
            const bool more = nrt < rt_end;
            if (more)   // in flight while this stage is multiplied
#pragma unroll
                for (int i = 0; i < PPT; ++i)
                    if (kFull || tid + kThreads * i < PIECES) gq[i] = *piece_src(nrt, ns, tid + kThreads * i);
            if (ntl > 0) stage_mfma(buf, s, ntl);
            if (more)   // that buffer was last read before the previous barrier
#pragma unroll
                for (int i = 0; i < PPT; ++i)
                    if (kFull || tid + kThreads * i < PIECES) *piece_dst(buf ^ 1, tid + kThreads * i) = gq[i];
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

// 32-key tiles per wave: the keys take NKT * KPW * R / 4 registers, kept at
// PRED_ROWS_KEY_REGS
#ifndef PRED_ROWS_KEY_REGS
#define PRED_ROWS_KEY_REGS 96
#endif
constexpr int nkt_rows(int r, int kpw) {
    const int t = (PRED_ROWS_KEY_REGS / 4) / (kpw * (r / 16));
    return t < 1 ? 1 : (t > 4 ? 4 : t);
}

template <int R, int KPW, int BS>
hipError_t launch_rk(const RowScoreArgs& a, hipStream_t st) {
    constexpr int NKT = nkt_rows(R, KPW);
    const int qh = a.Hq / kWaves;
    const int sh = (R <= PRED_ROWS_SH2_MAX_R && qh % 2 == 0) ? 2 : 1;
    RowGeom gm;
    const int64_t n_keys = a.n * BS;
    gm.groups = (n_keys + kKG * NKT * 32 - 1) / (kKG * NKT * 32);
    gm.row_tiles = (int)((a.rows + 31) / 32);
    gm.stages = qh / sh;
    int64_t parts = (kTargetWaves + gm.groups * kWaves * kKG - 1) / (gm.groups * kWaves * kKG);
    if (parts > gm.row_tiles) parts = gm.row_tiles;
    if (parts < 1) parts = 1;
    gm.tiles_per_part = (int)((gm.row_tiles + parts - 1) / parts);
    gm.parts = (gm.row_tiles + gm.tiles_per_part - 1) / gm.tiles_per_part;   // no empty parts
    const int64_t wgs = gm.groups * gm.parts;
    if (!grid_fits(wgs)) return hipErrorInvalidConfiguration;
    if constexpr (R <= PRED_ROWS_SH2_MAX_R) {
        if (sh == 2) {
            score_rows_kernel<R, KPW, NKT, 2, BS><<<(unsigned)wgs, kThreads, 0, st>>>(a, gm);
            return hipGetLastError();
        }
    }
    score_rows_kernel<R, KPW, NKT, 1, BS><<<(unsigned)wgs, kThreads, 0, st>>>(a, gm);
    return hipGetLastError();
}

template <int R, int KPW>
hipError_t launch_rb(const RowScoreArgs& a, hipStream_t st) {
    switch (a.B) {
        case 8: return launch_rk<R, KPW, 8>(a, st);
        case 16: return launch_rk<R, KPW, 16>(a, st);
        default: return launch_rk<R, KPW, 32>(a, st);
    }
}

template <int KPW>
hipError_t launch_kpw(const RowScoreArgs& a, hipStream_t st) {
    switch (a.R) {
        case 16: return launch_rb<16, KPW>(a, st);
        case 32: return launch_rb<32, KPW>(a, st);
        case 64: return launch_rb<64, KPW>(a, st);
        default: return launch_rb<128, KPW>(a, st);
    }
}

bool rows_mfma_supported(const RowScoreArgs& a) {
    const bool r_ok = a.R == 16 || a.R == 32 || a.R == 64 || a.R == 128;
    const bool hk_ok = a.Hk == 1 || a.Hk == 2 || a.Hk == 4 || a.Hk == 8;
    const bool b_ok = a.B == 8 || a.B == 16 || a.B == 32;
    return r_ok && hk_ok && b_ok && a.Hq % kWaves == 0;
}

}  // namespace

const char* score_rows_path_name(const RowScoreArgs& a, int force) {
    return force != SCORE_PATH_GENERIC && rows_mfma_supported(a) ? "score_rows_kernel" : "score_rows_generic_kernel";
}

hipError_t launch_score_rows(const RowScoreArgs& a, int force, hipStream_t st) {
    if (a.rows <= 0 || a.stride <= 0) return hipSuccess;
    if (force == SCORE_PATH_GENERIC || !rows_mfma_supported(a) || a.n == 0) {
        if (!grid_fits((a.rows * a.stride + 255) / 256)) return hipErrorInvalidConfiguration;
        score_rows_generic_kernel<<<(unsigned)((a.rows * a.stride + 255) / 256), 256, 0, st>>>(a);
        return hipGetLastError();
    }
    const int64_t n_cols = a.n < a.stride ? a.n : a.stride;   // columns that hold a block
    RowScoreArgs m = a;
    m.n = n_cols;
    const int64_t tail = a.rows * (a.stride - n_cols);
    if (!grid_fits((tail + 255) / 256)) return hipErrorInvalidConfiguration;
    const hipError_t e = a.Hk == 8 ? launch_kpw<2>(m, st) : launch_kpw<1>(m, st);
    if (e != hipSuccess || tail == 0) return e;
    fill_tail_cols_kernel<<<(unsigned)((tail + 255) / 256), 256, 0, st>>>(a.scores, a.rows, a.stride, n_cols);
    return hipGetLastError();
}

}  // namespace pred
