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
// Work split.  A workgroup has 8 waves; wave w serves kv head w % Hk and, when
// there are fewer than 8 kv heads, the (w / Hk)-th of 8 / Hk key sub-ranges.
// A key group is the workgroup's keys: 8 / Hk sub-ranges of KT tiles of 32
// keys (consecutive tokens of consecutive blocks).  A wave keeps its keys of
// its kv head as MFMA A operands in registers and, per row tile of 32 rows,
// multiplies them by the queries of that kv head's g query heads, one head per
// step: A_kv [32 keys, R] x Q_h^T [R, 32 rows] on v_mfma_f32_32x32x16_bf16 (f32
// accumulation; a lane holds one query row and 16 keys of a tile: element i is
// key (i / 4) * 8 + 4 * (lane / 32) + i % 4), and folds each product into the
// running maxima of the tile's blocks.
//
// Each wave streams its own queries: per step it loads the next step's 32
// query vectors with 16-byte coalesced reads into registers, multiplies the
// current step's vectors from its private LDS buffer (padded rows, so the MFMA
// operand reads are free of bank conflicts), then writes the next step's
// vectors to its other private buffer.  No query stage is shared, so the waves
// never wait for each other inside a row tile.  They meet once per row tile:
// each wave's block maxima (lane halves combined) go to LDS, one barrier, and
// the workgroup takes the max over kv heads and stores the row tile's scores
// along rows.  The reduction buffer is double-buffered where LDS allows, so
// that barrier is the only one.
//
// Scheduling.  One workgroup per CU (two waves per SIMD), as many as the GPU
// has CUs.  The rows are cut into up to 8 parts; workgroup i serves part
// i % parts, so with 8 parts each XCD (which takes every 8th workgroup) serves
// one part and its L2 holds that part's queries.  A part's work items --
// (key group, row tile), key group major -- are split into equal contiguous
// ranges over its workgroups; a wave reloads its keys only when the group
// changes, and issues that load before the previous item's reduction so the
// reduction hides part of its latency.  Key tiles past the row tile's last
// complete block skip their MFMAs (their scores are -inf).
#include "common.h"
#include "kernels.h"

// Tuning knobs (compile-time).
// key registers per wave: KT = PRED_ROWS_KEY_REGS / (4 * R / 16) tiles, at most 8
#ifndef PRED_ROWS_KEY_REGS
#define PRED_ROWS_KEY_REGS 96
#endif
// row parts (an XCD's L2 holds one part's queries when there are 8)
#ifndef PRED_ROWS_MAX_PARTS
#define PRED_ROWS_MAX_PARTS 8
#endif

namespace pred {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsBytes = 160 * 1024;

struct RowGeom {
    int wpk;              // waves per kv head: 8 / Hk key sub-ranges
    int64_t groups;       // key groups (wpk * KT * 32 keys each)
    int row_tiles;        // ceil(rows / 32)
    int parts;            // row parts
    int tiles_per_part;
    int wg_per_part;      // workgroups serving each part
};

__device__ inline int64_t complete_blocks(const RowScoreArgs& a, int64_t r) {
    const int64_t c = (a.first_pos + r + 1) / a.B;
    return c < a.n ? c : a.n;
}

constexpr int kt_rows(int r) {
    const int t = (PRED_ROWS_KEY_REGS / 4) / (r / 16);
    return t < 1 ? 1 : (t > 8 ? 8 : t);
}

template <int R, int BS>
struct RowsLds {
    static constexpr int KT = kt_rows(R);
    static constexpr int ROWB = R * 2 + 16;                    // LDS bytes per query vector
    static constexpr int BPT = 32 / BS;                        // blocks per key tile
    static constexpr int NB = KT * BPT;                        // blocks of a wave's keys
    static constexpr int NBP = NB | 1;                         // reduction row stride (odd: no bank conflicts)
    static constexpr int STAGE = 32 * ROWB;                    // one head of one row tile
    static constexpr int RED = kWaves * 32 * NBP * 4;          // one reduction buffer
    static constexpr int NRED = (kWaves * 2 * STAGE + 2 * RED <= kLdsBytes) ? 2 : 1;
    static_assert(kWaves * 2 * STAGE + RED <= kLdsBytes, "query stages and reduction exceed LDS");
};

// R: projected width; BS: block size.
template <int R, int BS>
__global__ __launch_bounds__(kThreads) void score_rows_kernel(RowScoreArgs a, RowGeom gm) {
    using L = RowsLds<R, BS>;
    constexpr int KT = L::KT;
    constexpr int RS = R / 16;                        // MFMA k-steps of 16
    constexpr int CPR = R / 8;                        // 16-byte pieces per query vector
    constexpr int ROWB = L::ROWB;
    constexpr int PPL = (32 * CPR) / 64;              // pieces per lane per step (>= 1 for R >= 16)
    constexpr int BPT = L::BPT;
    constexpr int EPB = BS / 2;                       // accumulator elements per block in a lane
    constexpr int NB = L::NB;
    constexpr int NRED = L::NRED;
    __shared__ __attribute__((aligned(16))) unsigned char stage[kWaves][2][L::STAGE];
    constexpr int NBP = L::NBP;
    __shared__ float red[NRED][kWaves][32 * NBP];     // per wave: block maxima [row][block]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kv = w % a.Hk;
    const int sub = w / a.Hk;
    const int g = a.Hq / a.Hk;
    const int part = (int)(blockIdx.x % gm.parts);
    const int jw = (int)(blockIdx.x / gm.parts);
    const int t_first = part * gm.tiles_per_part;
    const int nt = (gm.row_tiles - t_first) < gm.tiles_per_part ? (gm.row_tiles - t_first) : gm.tiles_per_part;
    if (nt <= 0) return;   // whole workgroup
    const int64_t items = gm.groups * nt;
    const int64_t i_begin = items * jw / gm.wg_per_part;
    const int64_t i_end = items * (jw + 1) / gm.wg_per_part;
    if (i_begin >= i_end) return;   // whole workgroup
    const int col = lane & 31;      // key of a tile (A operand) / query row (B operand)
    const int half = lane >> 5;     // which 8 of the 16 k-values of one MFMA step
    const int64_t n_keys = a.n * BS;
    const int64_t slot_elems = (int64_t)a.Hk * BS * R;
    const uint32_t row_bytes = (uint32_t)a.Hq * R * 2;   // one query row, all heads
    const uint32_t my_lds = (uint32_t)(uintptr_t)&stage[w][0][0];

    // Per-lane constants of a step: piece i of the lane is query row p / CPR of
    // the tile, 16-byte piece p % CPR (p = lane + 64 i): its byte offset from the
    // tile's head-0 vector of row 0, and its LDS offset in a stage buffer.
    uint32_t q_off[PPL], l_off[PPL];
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
        const int p = lane + 64 * i;
        q_off[i] = (uint32_t)(p / CPR) * row_bytes + (uint32_t)(p % CPR) * 16;
        l_off[i] = (uint32_t)((p / CPR) * ROWB + (p % CPR) * 16);
    }
    const uint32_t rd_off = (uint32_t)(col * ROWB + half * 16);   // MFMA operand read, k-step 0

    // A operands: this lane's key of each of the wave's tiles in group grp
    bf16x8_t kb[KT][RS];
    auto load_keys = [&](int64_t grp) {
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int64_t key = (grp * gm.wpk + sub) * (KT * 32) + t * 32 + col;
            const uint16_t* src = a.ag;   // lanes without a valid key: in bounds; their blocks are never stored
            if (key < n_keys) {
                const int64_t b = key / BS;
                const int tok = (int)(key - b * BS);
                const int64_t phys = a.table ? (int64_t)a.table[b] : b;
                if (phys >= 0 && phys < a.N)
                    src = a.ag + (a.layer * a.N + phys) * slot_elems + ((int64_t)kv * BS + tok) * R;
            }
#pragma unroll
            for (int st = 0; st < RS; ++st) kb[t][st] = load8(src + st * 16 + half * 8);
        }
    };

    float rm[KT][BPT];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int bi = 0; bi < BPT; ++bi) rm[t][bi] = -__builtin_inff();

    // query vectors of one step (row tile rt, head h) -> registers: buffer loads
    // from the tile's first row, whose range ends at the last real row, so the
    // padding rows of a partial tile read zeros (never stored)
    u32x4_t gq[PPL];
    auto fetch = [&](int rt, int h) {
        const int64_t r0 = (int64_t)rt * 32;
        const int64_t left = a.rows - r0 < 32 ? a.rows - r0 : 32;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(a.qp + r0 * a.Hq * R), (short)0, (int)((uint32_t)left * row_bytes), 0x00020000);
        const int soff = h * R * 2;
#pragma unroll
        for (int i = 0; i < PPL; ++i)
            gq[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)q_off[i], soff, 0));
    };
    auto put = [&](int buf) {
        const uint32_t base = my_lds + (uint32_t)(buf * L::STAGE);
#pragma unroll
        for (int i = 0; i < PPL; ++i)
            *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(base + l_off[i]) = gq[i];
    };
    auto chain = [&](int t, const bf16x8_t (&qb)[RS]) {
        f32x16_t acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t][0], qb[0], f32x16_t{}, 0, 0, 0);
#pragma unroll
        for (int st = 1; st < RS; ++st) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t][st], qb[st], acc, 0, 0, 0);
        return acc;
    };
    auto fold = [&](int t, const f32x16_t& acc) {
#pragma unroll
        for (int bi = 0; bi < BPT; ++bi) {
            float m = rm[t][bi];
#pragma unroll
            for (int e = 0; e < EPB; e += 2) m = fmaxf(fmaxf(m, acc[bi * EPB + e]), acc[bi * EPB + e + 1]);
            rm[t][bi] = m;
        }
    };
    // The wave's first ntl key tiles against the vectors in buffer buf.  With
    // every tile live, tile t + 1's chain is issued before tile t's fold, so the
    // fold's VALU work runs while the matrix core multiplies.
    auto multiply = [&](int buf, int ntl) {
        const uint32_t base = my_lds + (uint32_t)(buf * L::STAGE) + rd_off;
        bf16x8_t qb[RS];
#pragma unroll
        for (int st = 0; st < RS; ++st)
            qb[st] = __builtin_bit_cast(bf16x8_t,
                                        *reinterpret_cast<__attribute__((address_space(3))) const u32x4_t*>(base + st * 32));
        if (ntl == KT) {
            f32x16_t acc[2];
            acc[0] = chain(0, qb);
#pragma unroll
            for (int t = 1; t < KT; ++t) {
                acc[t & 1] = chain(t, qb);
                fold(t - 1, acc[(t - 1) & 1]);
            }
            fold(KT - 1, acc[(KT - 1) & 1]);
            return;
        }
#pragma unroll
        for (int t = 0; t < KT; ++t)
            if (t < ntl) fold(t, chain(t, qb));
    };

    // Stores of one row tile: entry i = tid + 512 j of the 32 x nbg (row, block)
    // maxima, consecutive threads on consecutive blocks of a row; the max over
    // the kv heads' partial maxima, -inf for an incomplete block, NaN for an
    // invalid table entry.
    const int nbg = gm.wpk * NB;   // blocks of a group
    auto store_tile = [&](int rb, int64_t sgrp, int srt) {
        const int64_t r0 = (int64_t)srt * 32;
        const int64_t blk0 = sgrp * nbg;
        for (int i = tid; i < nbg * 32; i += kThreads) {
            const int row = i / nbg;
            const int bw = i - row * nbg;
            const int s2 = bw / NB;
            const int blk = bw - s2 * NB;
            const int64_t r = r0 + row;
            const int64_t b = blk0 + bw;
            if (r < a.rows && b < a.n) {
                const bool complete = b < (a.first_pos + r + 1) / BS;
                const int64_t phys = (complete && a.table) ? (int64_t)a.table[b] : 0;   // in flight during the reads
                // the kv heads' partial maxima: all reads issued before the first is needed
                const float* src = &red[rb][s2 * a.Hk][row * NBP + blk];
                float part[kWaves];
#pragma unroll
                for (int k = 0; k < kWaves; ++k) part[k] = k < a.Hk ? src[k * 32 * NBP] : -__builtin_inff();
                float v = part[0];
#pragma unroll
                for (int k = 1; k < kWaves; ++k) v = fmaxf(v, part[k]);
                uint32_t bits = __float_as_uint(v);
                if (!complete) {
                    bits = 0xFF800000u;   // -inf
                } else if (phys < 0 || phys >= a.N) {
                    bits = 0x7FC00000u;   // NaN (as bits: this file is compiled without NaN semantics)
                    atomicOr(a.err, DEVERR_TABLE);
                }
                reinterpret_cast<uint32_t*>(a.scores)[r * a.stride + b] = bits;
            }
        }
    };

    int64_t grp = i_begin / nt;
    int rt = t_first + (int)(i_begin - grp * nt);
    int buf = 0;
    int red_buf = 0;
    // the previous row tile, stored during this one's first step (two reduction buffers)
    bool pending = false;
    int64_t p_grp = 0;
    int p_rt = 0;
    load_keys(grp);
    fetch(rt, kv * g);
    put(0);
    for (int64_t item = i_begin; item < i_end; ++item) {
        const bool more = item + 1 < i_end;
        const int n_rt = (rt + 1 - t_first) < nt ? rt + 1 : t_first;
        const int64_t n_grp = n_rt == t_first ? grp + 1 : grp;
        // key tiles holding a block complete for the row tile's last row
        const int64_t last = ((int64_t)rt * 32 + 31) < a.rows ? ((int64_t)rt * 32 + 31) : a.rows - 1;
        int64_t climit = (a.first_pos + last + 1) / BS;
        if (climit > a.n) climit = a.n;
        const int64_t key_first = (grp * gm.wpk + sub) * (KT * 32);
        int ntl = 0;
#pragma unroll
        for (int t = 0; t < KT; ++t)
            if ((key_first + t * 32) / BS < climit) ntl = t + 1;
        for (int hs = 0; hs < g; ++hs) {
            // The next step's vectors are in flight during this step's MFMAs.  The
            // fetch is unconditional (the last step re-reads its own vectors) so
            // that on every path the newest loads are queries, and waiting for the
            // keys never waits for them.
            const bool last_step = hs + 1 == g;
            fetch(last_step ? (more ? n_rt : rt) : rt, kv * g + (last_step ? (more ? 0 : hs) : hs + 1));
            multiply(buf, ntl);
            if (NRED == 2 && hs == 0 && pending) {
                // the previous row tile's stores, while this step's MFMAs run
                store_tile(red_buf ^ 1, p_grp, p_rt);
                pending = false;
            }
            put(buf ^ 1);   // that buffer's vectors were read by the previous step
            buf ^= 1;
        }
        // row tile done: the next group's keys first (their latency overlaps the reduction)
        if (more && n_grp != grp) load_keys(n_grp);
        float* rw = &red[red_buf][w][0];
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int bi = 0; bi < BPT; ++bi) {
                // rows 0..15 and 16..31 of each key sit in the two lane halves
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rm[t][bi]),
                                                                 __float_as_uint(rm[t][bi]), false, false);
                if (half == 0) rw[col * NBP + t * BPT + bi] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                rm[t][bi] = -__builtin_inff();
            }
        // every wave's maxima of this row tile are in LDS; every wave has also
        // finished the previous row tile's stores, so its buffer is free again
        __syncthreads();
        if constexpr (NRED == 2) {
            pending = true;
            p_grp = grp;
            p_rt = rt;
            red_buf ^= 1;
        } else {
            store_tile(0, grp, rt);
            __syncthreads();   // the buffer is written again next row tile
        }
        grp = n_grp;
        rt = n_rt;
    }
    if (pending) store_tile(red_buf ^ 1, p_grp, p_rt);
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
        *reinterpret_cast<uint32_t*>(out) = 0x7FC00000u;   // NaN (as bits: no NaN semantics in this file)
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

template <int R, int BS>
hipError_t launch_rk(const RowScoreArgs& a, hipStream_t st) {
    constexpr int KT = RowsLds<R, BS>::KT;
    RowGeom gm;
    gm.wpk = kWaves / a.Hk;
    const int64_t n_keys = a.n * BS;
    const int64_t keys_per_group = (int64_t)gm.wpk * KT * 32;
    gm.groups = (n_keys + keys_per_group - 1) / keys_per_group;
    gm.row_tiles = (int)((a.rows + 31) / 32);
    int parts = PRED_ROWS_MAX_PARTS;
    while (parts > 1 && parts > gm.row_tiles) parts >>= 1;
    gm.tiles_per_part = (gm.row_tiles + parts - 1) / parts;
    gm.parts = (gm.row_tiles + gm.tiles_per_part - 1) / gm.tiles_per_part;   // no empty parts
    const int64_t items_per_part = gm.groups * gm.tiles_per_part;
    int64_t wpp = (a.n_cu > 0 ? a.n_cu : 256) / gm.parts;
    if (wpp < 1) wpp = 1;
    if (wpp > items_per_part) wpp = items_per_part;
    gm.wg_per_part = (int)wpp;
    const int64_t wgs = (int64_t)gm.parts * wpp;
    if (!grid_fits(wgs)) return hipErrorInvalidConfiguration;
    score_rows_kernel<R, BS><<<(unsigned)wgs, kThreads, 0, st>>>(a, gm);
    return hipGetLastError();
}

template <int R>
hipError_t launch_rb(const RowScoreArgs& a, hipStream_t st) {
    switch (a.B) {
        case 8: return launch_rk<R, 8>(a, st);
        case 16: return launch_rk<R, 16>(a, st);
        default: return launch_rk<R, 32>(a, st);
    }
}

bool rows_mfma_supported(const RowScoreArgs& a) {
    const bool r_ok = a.R == 16 || a.R == 32 || a.R == 64 || a.R == 128;
    const bool hk_ok = a.Hk == 1 || a.Hk == 2 || a.Hk == 4 || a.Hk == 8;
    const bool b_ok = a.B == 8 || a.B == 16 || a.B == 32;
    return r_ok && hk_ok && b_ok;
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
    hipError_t e;
    switch (a.R) {
        case 16: e = launch_rb<16>(m, st); break;
        case 32: e = launch_rb<32>(m, st); break;
        case 64: e = launch_rb<64>(m, st); break;
        default: e = launch_rb<128>(m, st); break;
    }
    if (e != hipSuccess || tail == 0) return e;
    fill_tail_cols_kernel<<<(unsigned)((tail + 255) / 256), 256, 0, st>>>(a.scores, a.rows, a.stride, n_cols);
    return hipGetLastError();
}

}  // namespace pred
