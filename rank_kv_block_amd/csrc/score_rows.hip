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
// Work split.  An item is (row range, key range): RR row tiles of 32 rows and
// 8 x KT tiles of 32 keys (consecutive tokens of consecutive blocks).  A
// workgroup of 8 waves takes a contiguous range of items; wave w owns the w-th
// KT key tiles of the item's key range for every kv head in turn, so the 8
// waves always work on the same kv head and the same query rows.  That makes
// the query operands shareable: per pass (one kv head and up to GS of its
// query heads) they are staged once in LDS for the whole workgroup, already in
// the MFMA B-operand layout (1 KiB per row tile, head and k-step of 16: lane
// (col, half) at byte 16 * lane holds row col's k-values st * 16 + half * 8 ..
// + 8), written by direct buffer-to-LDS loads.  A wave keeps its keys of the
// current kv head as MFMA A operands in registers and multiplies them by the
// staged queries on v_mfma_f32_32x32x16_bf16 (f32 accumulation): A [32 keys, R]
// x Q^T [R, 32 rows], where a lane holds one query row and 16 keys of a tile
// (element i is key (i / 4) * 8 + 4 * (lane / 32) + i % 4), folded into that
// row's running maxima of the tile's blocks.  The maxima run over every kv
// head and query head of the item in registers, so a wave ends the item with
// the final scores of its (row, block) cells: no reduction across waves.
//
// Pipelining.  Stages and key sets are double-buffered: while a pass
// multiplies, the next pass's queries load into the other LDS stage and, on a
// pass that starts a kv head, the next kv head's keys load into the other
// register set.  One barrier per pass.  Passes run back to back across items,
// so an item's first keys and queries load during the previous item.
//
// Scheduling.  One workgroup per CU (the stages take most of the LDS), at
// most as many as the GPU has CUs.  Items are numbered key range fastest and
// split into equal contiguous ranges, so the workgroups of one XCD (every 8th)
// share a few key ranges in their L2.  Key tiles past a row tile's last
// complete block skip their MFMAs (their scores are -inf).
#include "common.h"
#include "kernels.h"

namespace pred {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

struct RowGeom {
    int64_t n_kr;     // key ranges
    int64_t items;    // row ranges x key ranges
    int gs;           // query heads per pass
    int hp;           // passes per kv head
    int wgs;          // workgroups
};

__device__ inline int64_t complete_blocks(const RowScoreArgs& a, int64_t r) {
    const int64_t c = (a.first_pos + r + 1) / a.B;
    return c < a.n ? c : a.n;
}

// Shape constants.  KT * RS = 16 (128 registers for two key sets), at most 8
// tiles; RR row tiles keep the running maxima at 32 registers; GS query heads
// fill a 64 KiB stage.
template <int R, int BS>
struct RowsCfg {
    static constexpr int RS = R / 16;                              // MFMA k-steps of 16
    static constexpr int KT = (16 / RS) < 8 ? 16 / RS : 8;         // key tiles per wave
    static constexpr int BPT = 32 / BS;                            // blocks per key tile
    static constexpr int NB = KT * BPT;                            // blocks of a wave
    static constexpr int RR = (32 / NB) < 1 ? 1 : ((32 / NB) > 4 ? 4 : 32 / NB);   // row tiles per item
    static constexpr int GS = 16 / RS;                             // query heads per stage
    static constexpr int STAGE = RR * GS * RS * 1024;              // bytes of one stage
    static constexpr int KEYS = kWaves * KT * 32;                  // keys per item
    static_assert(2 * STAGE <= 160 * 1024, "stages exceed LDS");
};

template <int R, int BS>
__global__ __launch_bounds__(kThreads) void score_rows_kernel(RowScoreArgs a, RowGeom gm) {
    using C = RowsCfg<R, BS>;
    constexpr int RS = C::RS, KT = C::KT, BPT = C::BPT, NB = C::NB, RR = C::RR, GS = C::GS;
    constexpr int EPB = BS / 2;                       // accumulator elements per block in a lane
    __shared__ __attribute__((aligned(1024))) unsigned char stage[2][C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;      // key of a tile (A operand) / query row (B operand)
    const int half = lane >> 5;     // which 8 of the 16 k-values of one MFMA step
    const int g = a.Hq / a.Hk;
    const int64_t i_begin = gm.items * blockIdx.x / gm.wgs;
    const int64_t i_end = gm.items * (blockIdx.x + 1) / gm.wgs;
    if (i_begin >= i_end) return;   // whole workgroup
    const int64_t n_keys = a.n * BS;
    const int64_t slot_elems = (int64_t)a.Hk * BS * R;
    const uint32_t row_bytes = (uint32_t)a.Hq * R * 2;   // one query row, all heads
    const int epochs_per_item = a.Hk;                     // one epoch per kv head
    const int64_t e_begin = i_begin * epochs_per_item;
    const int64_t e_end = i_end * epochs_per_item;

    // A operands of one epoch (item, kv head): this lane's key of each of the
    // wave's tiles.  Returns the wave's blocks whose table entry is invalid,
    // bit t * BPT + bi for block bi of tile t.
    auto load_keys = [&](bf16x8_t (&kb)[KT][RS], int64_t e) -> uint32_t {
        const int64_t item = e / epochs_per_item;
        const int kv = (int)(e - item * epochs_per_item);
        const int64_t kr = item % gm.n_kr;
        const int64_t key0 = kr * C::KEYS + (int64_t)w * (KT * 32) + col;
        int64_t phys[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int64_t key = key0 + t * 32;
            phys[t] = (key < n_keys ? key : n_keys - 1) / BS;
        }
        if (a.table) {   // every table read in flight at once
#pragma unroll
            for (int t = 0; t < KT; ++t) phys[t] = a.table[phys[t]];
        }
        uint32_t bad = 0;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int64_t key = key0 + t * 32;
            const bool live = key < n_keys;
            const bool valid = phys[t] >= 0 && phys[t] < a.N;
            const int tok = (int)(key % BS);
            // lanes without a valid key read in bounds; their blocks are never stored as scores
            const uint16_t* src =
                live && valid ? a.ag + (a.layer * a.N + phys[t]) * slot_elems + ((int64_t)kv * BS + tok) * R : a.ag;
#pragma unroll
            for (int st = 0; st < RS; ++st) kb[t][st] = load8(src + st * 16 + half * 8);
            const uint64_t m = __ballot(live && !valid);
#pragma unroll
            for (int bi = 0; bi < BPT; ++bi)
                if ((m >> (bi * BS)) & ((1ull << BS) - 1)) bad |= 1u << (t * BPT + bi);
        }
        return bad;
    };

    // Queries of one pass (epoch e, head group hg) into stage buffer sb: chunk
    // (rt, j, st) of the stage is row tile rt, query head kv * g + hg * gs + j,
    // k-step st; each wave loads every 8th chunk.  The buffer range ends at the
    // item's last real row, so the padding rows of a partial tile read zeros.
    auto load_stage = [&](int64_t e, int hg, int sb) {
        const int64_t item = e / epochs_per_item;
        const int kv = (int)(e - item * epochs_per_item);
        const int64_t r0 = (item / gm.n_kr) * (RR * 32);
        const int64_t left = a.rows - r0 < RR * 32 ? a.rows - r0 : RR * 32;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(a.qp + r0 * a.Hq * R), (short)0, (int)((uint32_t)left * row_bytes), 0x00020000);
        const int h0 = kv * g + hg * gm.gs;
        const int ge = (g - hg * gm.gs) < gm.gs ? g - hg * gm.gs : gm.gs;
        const uint32_t lane_off = (uint32_t)col * row_bytes + (uint32_t)half * 16;
#pragma unroll
        for (int i = 0; i < (RR * GS * RS + kWaves - 1) / kWaves; ++i) {
            const int c = w + kWaves * i;
            const int st = c % RS;
            const int j = (c / RS) % GS;
            const int rt = c / (RS * GS);
            if (c < RR * GS * RS && j < ge)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (__attribute__((address_space(3))) void*)&stage[sb][c * 1024], 16,
                    (int)(lane_off + (uint32_t)rt * 32 * row_bytes + st * 32), (h0 + j) * R * 2, 0, 0);
        }
    };

    float rm[RR][KT][BPT];
#pragma unroll
    for (int rt = 0; rt < RR; ++rt)
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int bi = 0; bi < BPT; ++bi) rm[rt][t][bi] = -__builtin_inff();

    auto chain = [&](const bf16x8_t (&kb)[KT][RS], int t, const bf16x8_t (&qb)[RS]) {
        f32x16_t acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t][0], qb[0], f32x16_t{}, 0, 0, 0);
#pragma unroll
        for (int st = 1; st < RS; ++st) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t][st], qb[st], acc, 0, 0, 0);
        return acc;
    };
    auto fold = [&](float (&m)[KT][BPT], int t, const f32x16_t& acc) {
#pragma unroll
        for (int bi = 0; bi < BPT; ++bi) {
            float v = m[t][bi];
#pragma unroll
            for (int e = 0; e < EPB; e += 2) v = fmaxf(fmaxf(v, acc[bi * EPB + e]), acc[bi * EPB + e + 1]);
            m[t][bi] = v;
        }
    };
    // The wave's first ntl key tiles against one step's query operands.  With
    // every tile live, tile t + 1's chain is issued before tile t's fold, so the
    // fold's VALU work runs while the matrix core multiplies.
    auto multiply = [&](const bf16x8_t (&kb)[KT][RS], const bf16x8_t (&qb)[RS], float (&m)[KT][BPT], int ntl) {
        if (ntl == KT) {
            f32x16_t acc[2];
            acc[0] = chain(kb, 0, qb);
#pragma unroll
            for (int t = 1; t < KT; ++t) {
                acc[t & 1] = chain(kb, t, qb);
                fold(m, t - 1, acc[(t - 1) & 1]);
            }
            fold(m, KT - 1, acc[(KT - 1) & 1]);
            return;
        }
#pragma unroll
        for (int t = 0; t < KT; ++t)
            if (t < ntl) fold(m, t, chain(kb, t, qb));
    };

    // One pass over stage buffer sb: every row tile of the item against ge
    // query heads, B operands read from LDS per step.
    auto compute_pass = [&](const bf16x8_t (&kb)[KT][RS], int sb, int ge, const int (&ntl)[RR]) {
        const uint32_t base = (uint32_t)(uintptr_t)&stage[sb][0] + (uint32_t)lane * 16;
#pragma unroll
        for (int rt = 0; rt < RR; ++rt) {
            if (ntl[rt] == 0) continue;
            for (int j = 0; j < ge; ++j) {
                bf16x8_t qb[RS];
#pragma unroll
                for (int st = 0; st < RS; ++st)
                    qb[st] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<__attribute__((address_space(3))) const u32x4_t*>(
                                                              base + (uint32_t)(((rt * GS + j) * RS + st) * 1024)));
                // the wave's MFMA stream issues ahead of the other wave's VALU and LDS work
                __builtin_amdgcn_s_setprio(1);
                multiply(kb, qb, rm[rt], ntl[rt]);
                __builtin_amdgcn_s_setprio(0);
            }
        }
    };

    // Scores of the item ending with epoch e: the two lane halves hold
    // different keys of the same row; after combining them, half h stores the
    // wave's blocks h * NB / 2 .. of its row (consecutive floats along the
    // row), -inf for an incomplete block, NaN for an invalid table entry.
    auto store_item = [&](int64_t item, uint32_t bad) {
        const int64_t r0 = (item / gm.n_kr) * (RR * 32);
        const int64_t blk0 = ((item % gm.n_kr) * C::KEYS + (int64_t)w * (KT * 32)) / BS;
#pragma unroll
        for (int rt = 0; rt < RR; ++rt) {
            const int64_t r = r0 + rt * 32 + col;
            const int64_t cb = r < a.rows ? (a.first_pos + r + 1) / BS : 0;   // complete blocks of row r
            float v[NB];
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int bi = 0; bi < BPT; ++bi) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rm[rt][t][bi]),
                                                                     __float_as_uint(rm[rt][t][bi]), false, false);
                    v[t * BPT + bi] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                    rm[rt][t][bi] = -__builtin_inff();
                }
            if (r < a.rows) {
                uint32_t* out = reinterpret_cast<uint32_t*>(a.scores) + r * a.stride;
#pragma unroll
                for (int i = 0; i < (NB + 1) / 2; ++i) {
                    const int k = half * ((NB + 1) / 2) + i;   // the wave's block index
                    if (k < NB && blk0 + k < a.n) {
                        uint32_t bits = __float_as_uint(v[k]);
                        if (blk0 + k >= cb) {
                            bits = 0xFF800000u;   // incomplete: -inf
                        } else if ((bad >> k) & 1u) {
                            bits = 0x7FC00000u;   // NaN (as bits: this file is compiled without NaN semantics)
                            atomicOr(a.err, DEVERR_TABLE);
                        }
                        out[blk0 + k] = bits;
                    }
                }
            }
        }
    };

    // key tiles holding a block complete for each row tile's last row
    auto live_tiles = [&](int64_t item, int (&ntl)[RR]) {
        const int64_t r0 = (item / gm.n_kr) * (RR * 32);
        const int64_t key_first = (item % gm.n_kr) * C::KEYS + (int64_t)w * (KT * 32);
#pragma unroll
        for (int rt = 0; rt < RR; ++rt) {
            const int64_t last = (r0 + rt * 32 + 31) < a.rows ? r0 + rt * 32 + 31 : a.rows - 1;
            int64_t climit = (a.first_pos + last + 1) / BS;
            if (climit > a.n) climit = a.n;
            int n = 0;
#pragma unroll
            for (int t = 0; t < KT; ++t)
                if ((key_first + t * 32) / BS < climit) n = t + 1;
            ntl[rt] = r0 + rt * 32 < a.rows ? n : 0;
        }
    };

    // One epoch (item, kv head) with its keys in kc; the next epoch's keys go
    // to kn.  Passes alternate the stage buffers (pass parity sb).
    int sb = 0;
    uint32_t bad_cur = 0, bad_next = 0;
    int ntl[RR];
    auto epoch = [&](bf16x8_t (&kc)[KT][RS], bf16x8_t (&kn)[KT][RS], int64_t e) {
        const int64_t item = e / epochs_per_item;
        const int kv = (int)(e - item * epochs_per_item);
        if (kv == 0) live_tiles(item, ntl);
        for (int hg = 0; hg < gm.hp; ++hg) {
            // this pass's queries (and keys) have landed for every wave, and
            // every wave is done with the other stage buffer
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (hg == 0 && e + 1 < e_end) {
                const uint32_t b = load_keys(kn, e + 1);
                if ((e + 1) % epochs_per_item == 0) bad_next = b;
            }
            if (hg + 1 < gm.hp) load_stage(e, hg + 1, sb ^ 1);
            else if (e + 1 < e_end) load_stage(e + 1, 0, sb ^ 1);
            const int ge = (g - hg * gm.gs) < gm.gs ? g - hg * gm.gs : gm.gs;
            compute_pass(kc, sb, ge, ntl);
            sb ^= 1;
        }
        if (kv + 1 == epochs_per_item) {
            store_item(item, bad_cur);
            bad_cur = bad_next;
        }
    };

    bf16x8_t k0[KT][RS], k1[KT][RS];
    bad_cur = load_keys(k0, e_begin);
    load_stage(e_begin, 0, 0);
    for (int64_t e = e_begin; e < e_end; e += 2) {
        epoch(k0, k1, e);
        if (e + 1 < e_end) epoch(k1, k0, e + 1);
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
    using C = RowsCfg<R, BS>;
    RowGeom gm;
    const int64_t n_keys = a.n * BS;
    gm.n_kr = (n_keys + C::KEYS - 1) / C::KEYS;
    const int64_t n_rr = (a.rows + C::RR * 32 - 1) / (C::RR * 32);
    gm.items = n_rr * gm.n_kr;
    const int g = a.Hq / a.Hk;
    gm.gs = g < C::GS ? g : C::GS;
    gm.hp = (g + gm.gs - 1) / gm.gs;
    int64_t wgs = a.n_cu > 0 ? a.n_cu : 256;
    if (wgs > gm.items) wgs = gm.items;
    gm.wgs = (int)wgs;
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
