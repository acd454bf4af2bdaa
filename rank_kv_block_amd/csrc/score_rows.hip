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
// Work split.  A workgroup of 4 waves owns one (kv head, key group, row part),
// as the many-row block scorer does: wave w keeps NKT key tiles of the group
// (32 consecutive tokens each) as MFMA A operands in registers for the whole
// kernel, and the part's query rows stream through LDS, a stage of 32 rows and
// up to HC of the kv head's query heads at a time, already in the B-operand
// layout (1 KiB per head and k-step of 16: lane (col, half) at byte 16 * lane
// holds row col's k-values st * 16 + half * 8 .. + 8).  A lane of the
// v_mfma_f32_32x32x16_bf16 accumulator (f32) holds one query row and 16 keys
// of a tile (element i is key (i / 4) * 8 + 4 * (lane / 32) + i % 4), so the
// max over a block's tokens and the stage's heads runs in registers.
//
// Combining kv heads.  When a 32-row chunk has seen all g heads of the kv
// head, each wave writes its blocks' maxima into an LDS slot (the chunk's 32
// rows x every block of the group) and the 256 threads move the slot to the
// scores with integer atomic max (or min) on the float bit patterns, which
// orders floats: the kv heads of one cell meet there, and each row's blocks of
// the group sit on consecutive addresses (one 128-byte line for 32 blocks), so
// an atomic instruction covers two lines.  The scores start at -inf (a fill
// launched first); cells never updated -- incomplete blocks, columns past n --
// stay -inf.
//
// Pipelining.  Stages are double-buffered in LDS.  A stage's queries are read
// into registers by buffer loads right after its predecessor's barrier and
// written to LDS at the end of that stage: staged through registers, rather
// than by direct buffer-to-LDS loads, the prefetch is not a dependence of the
// LDS reads that feed the multiplies, so they never wait for it.  A chunk's
// atomics go out at the end of the next stage, after the prefetch is written,
// so the wait for a prefetch finds the atomics before it long done.
//
// Scheduling.  One straight-line block per full stage: per head, every key
// tile's MFMA chain into its own accumulator, then the folds, interleaved two
// MFMAs to eight max3 instructions; the wave's priority is raised while it
// multiplies.  Workgroups are numbered kv head fastest: with 8 kv heads each
// XCD (every 8th workgroup) serves one kv head and its L2 keeps that head's
// queries.  Key tiles past a chunk's last complete block skip their MFMAs.
#include "common.h"
#include "kernels.h"

namespace pred {

namespace {

__device__ inline int64_t complete_blocks(const RowScoreArgs& a, int64_t r) {
    const int64_t c = (a.first_pos + r + 1) / a.B;
    return c < a.n ? c : a.n;
}

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// s_waitcnt immediate (gfx9 encoding) for "every vector memory access done":
// vmcnt 0 (bits 3:0 and 15:14), expcnt 7 and lgkmcnt 15 (bits 6:4, 11:8: no wait)
constexpr int kWaitVmcnt0 = 0x0F70;

struct RowGeom {
    int64_t groups;        // key groups per kv head
    int chunks_per_part;   // 32-row chunks per row part
    int hc;                // query heads per stage
    int hp;                // stages per chunk
};

template <int R, int NKT, int BS>
struct RowsCfg {
    static constexpr int RS = R / 16;                // MFMA k-steps of 16
    static constexpr int BPT = 32 / BS;              // blocks per key tile
    static constexpr int NB = NKT * BPT;             // blocks of a wave
    static constexpr int KG = kWaves * NKT * 32;     // keys of a group
    static constexpr int NBG = KG / BS;              // blocks of a group
    static constexpr int HC = 16 / RS;               // query heads per stage (16 KiB)
    static constexpr int STAGE = HC * RS * 1024;
    static constexpr int SROW = NBG + 4;             // floats per slot row (16-byte aligned rows)
    static_assert(kThreads % NBG == 0 && 32 * NBG >= kThreads, "a thread's slot cells share one block");
    static_assert(NB % 2 == 0, "lane halves write half of the wave's blocks each");
};

template <int R, int NKT, int BS>
__global__ __launch_bounds__(kThreads) void score_rows_kernel(RowScoreArgs a, RowGeom gm) {
    using C = RowsCfg<R, NKT, BS>;
    constexpr int RS = C::RS, BPT = C::BPT, NB = C::NB, NBG = C::NBG, EPB = BS / 2;
    __shared__ __attribute__((aligned(1024))) unsigned char stage[2][C::STAGE];
    __shared__ __attribute__((aligned(16))) float slot[2][32 * C::SROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;      // key of a tile (A operand) / query row (B operand)
    const int half = lane >> 5;     // which 8 of the 16 k-values of one MFMA step
    const int g = a.Hq / a.Hk;
    int64_t id = blockIdx.x;
    const int kv = (int)(id % a.Hk);
    id /= a.Hk;
    const int64_t grp = id % gm.groups;
    const int64_t rc_begin = (id / gm.groups) * gm.chunks_per_part;
    const int64_t n_chunks = (a.rows + 31) / 32;
    const int64_t rc_end = rc_begin + gm.chunks_per_part < n_chunks ? rc_begin + gm.chunks_per_part : n_chunks;
    const int64_t n_keys = a.n * BS;
    const int64_t slot_elems = (int64_t)a.Hk * BS * R;
    const uint32_t row_bytes = (uint32_t)a.Hq * R * 2;   // one query row, all heads
    const int64_t key_first = grp * C::KG + (int64_t)w * (NKT * 32);   // the wave's first key

    // The wave's keys (A operands), read once.  Lanes without a valid key
    // read in bounds; their blocks are never stored.
    bf16x8_t kb[NKT][RS];
    {
        int64_t phys[NKT];
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            const int64_t key = key_first + t * 32 + col;
            phys[t] = (key < n_keys ? key : n_keys - 1) / BS;
        }
        if (a.table) {   // every table read in flight at once
#pragma unroll
            for (int t = 0; t < NKT; ++t) phys[t] = a.table[phys[t]];
        }
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            const int64_t key = key_first + t * 32 + col;
            const bool ok = key < n_keys && phys[t] >= 0 && phys[t] < a.N;
            const uint16_t* src =
                ok ? a.ag + (a.layer * a.N + phys[t]) * slot_elems + ((int64_t)kv * BS + key % BS) * R : a.ag;
#pragma unroll
            for (int st = 0; st < RS; ++st) kb[t][st] = load8(src + st * 16 + half * 8);
        }
    }
    // The block this thread moves to the scores (the same for all its slot
    // cells) and whether its table entry is invalid.
    const int fb = tid % NBG;
    const int64_t fblk = grp * NBG + fb;
    bool fbad = false;
    if (fblk < a.n) {
        const int64_t ph = a.table ? (int64_t)a.table[fblk] : fblk;
        fbad = ph < 0 || ph >= a.N;
    }

    // Stage loads, through registers: piece c = j * RS + st of a stage is
    // query head kv * g + hg * hc + j, k-step st, and lane (col, half) of a
    // piece holds row col's k-values st * 16 + half * 8 .. + 8 (the MFMA B
    // layout, 1 KiB per piece); wave w moves every 4th piece.  Buffer loads of
    // the rows past the chunk's last real row read zeros.  (Staging through
    // registers rather than direct buffer-to-LDS loads keeps the loads off the
    // LDS reads' dependences: a read of the current stage does not wait for the
    // next stage's loads.)
    constexpr int PPW = (C::HC * RS + kWaves - 1) / kWaves;   // pieces per wave
    u32x4_t gq[PPW];
    auto load_stage = [&](int64_t rc, int hg) {
        const int64_t r0 = rc * 32;
        const int64_t left = a.rows - r0 < 32 ? a.rows - r0 : 32;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(a.qp + r0 * a.Hq * R), (short)0, (int)((uint32_t)left * row_bytes), 0x00020000);
        const int h0 = kv * g + hg * gm.hc;
        const int ge = (g - hg * gm.hc) < gm.hc ? g - hg * gm.hc : gm.hc;
        const uint32_t lane_off = (uint32_t)col * row_bytes + (uint32_t)half * 16;
#pragma unroll
        for (int i = 0; i < PPW; ++i) {
            const int c = w + kWaves * i;
            const int st = c % RS;
            const int j = c / RS;
            if (c < C::HC * RS && j < ge)
                gq[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rsrc, (int)(lane_off + st * 32), (h0 + j) * R * 2, 0));
        }
    };
    auto store_stage = [&](int hg, int sb) {
        const int ge = (g - hg * gm.hc) < gm.hc ? g - hg * gm.hc : gm.hc;
#pragma unroll
        for (int i = 0; i < PPW; ++i) {
            const int c = w + kWaves * i;
            if (c < C::HC * RS && c / RS < ge)
                *reinterpret_cast<u32x4_t*>(&stage[sb][c * 1024 + lane * 16]) = gq[i];
        }
    };

    float rm[NKT][BPT];
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int bi = 0; bi < BPT; ++bi) rm[t][bi] = -__builtin_inff();

    auto chain = [&](int t, const bf16x8_t (&qb)[RS]) {
        f32x16_t acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t][0], qb[0], f32x16_t{}, 0, 0, 0);
#pragma unroll
        for (int st = 1; st < RS; ++st) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t][st], qb[st], acc, 0, 0, 0);
        return acc;
    };
    // element i of a tile's accumulator is key (i / 4) * 8 + 4 * half + i % 4,
    // so block bi's keys are elements bi * EPB .. + EPB
    auto fold = [&](int t, const f32x16_t& acc) {
#pragma unroll
        for (int bi = 0; bi < BPT; ++bi) {
            float v = rm[t][bi];
#pragma unroll
            for (int e = 0; e < EPB; e += 2) v = fmaxf(fmaxf(v, acc[bi * EPB + e]), acc[bi * EPB + e + 1]);
            rm[t][bi] = v;
        }
    };
    auto read_q = [&](int sb, int j, bf16x8_t (&qb)[RS]) {
#pragma unroll
        for (int st = 0; st < RS; ++st)
            qb[st] = __builtin_bit_cast(bf16x8_t,
                                        *reinterpret_cast<const u32x4_t*>(&stage[sb][(j * RS + st) * 1024 + lane * 16]));
    };
    // A stage: ge heads against the wave's first ntl key tiles.  The wave's
    // MFMA stream issues ahead of the other wave's VALU and LDS work (raised
    // priority).  A full stage with every tile live is one straight-line
    // block: per head all chains first, each into its own accumulator, then
    // the folds, scheduled as two MFMAs and the max instructions that match
    // them (8 max3 per key tile against RS MFMAs), repeated, so one tile's
    // folds issue between later tiles' MFMAs, across heads too.
    auto compute = [&](int sb, int ge, int ntl) {
        __builtin_amdgcn_s_setprio(1);
        if (ge == C::HC && ntl == NKT) {
#pragma unroll
            for (int j = 0; j < C::HC; ++j) {
                bf16x8_t qb[RS];
                read_q(sb, j, qb);
                f32x16_t acc[NKT];
#pragma unroll
                for (int t = 0; t < NKT; ++t) acc[t] = chain(t, qb);
#pragma unroll
                for (int t = 0; t < NKT; ++t) fold(t, acc[t]);
#pragma unroll
                for (int i = 0; i < NKT * RS / 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);          // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 16 / RS, 0);    // VALU
                }
            }
        } else {
            for (int j = 0; j < ge; ++j) {
                bf16x8_t qb[RS];
                read_q(sb, j, qb);
#pragma unroll
                for (int t = 0; t < NKT; ++t)
                    if (t < ntl) fold(t, chain(t, qb));
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // key tiles of the wave holding a block complete at the chunk's last row
    auto live_tiles = [&](int64_t rc) {
        const int64_t last = rc * 32 + 31 < a.rows ? rc * 32 + 31 : a.rows - 1;
        int64_t climit = (a.first_pos + last + 1) / BS;
        if (climit > a.n) climit = a.n;
        int n = 0;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            if ((key_first + t * 32) / BS < climit) n = t + 1;
        return n;
    };
    // The chunk's maxima into its slot: after the two lane halves are
    // combined, half h writes the wave's blocks h * NB / 2 .. of row col.
    auto write_slot = [&](int64_t rc) {
        float* sl = &slot[rc & 1][col * C::SROW + w * NB + half * (NB / 2)];
        float v[NB];
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int bi = 0; bi < BPT; ++bi) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rm[t][bi]), __float_as_uint(rm[t][bi]),
                                                                 false, false);
                v[t * BPT + bi] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                rm[t][bi] = -__builtin_inff();
            }
#pragma unroll
        for (int i = 0; i < NB / 2; ++i) sl[i] = half ? v[NB / 2 + i] : v[i];
    };
    // The slot of chunk rc to the scores: cell i = tid + kThreads * k is row
    // i / NBG, block fb of the group.  Per thread: its first row, its block's
    // first complete row (block fblk is complete at row r iff r >= r_cmp) and
    // its score address in row 0; a chunk and a k step add uniform offsets.
    constexpr int RPK = kThreads / NBG;   // rows between a thread's cells
    const int row0 = tid / NBG;
    const int64_t r_cmp = (fblk + 1) * BS - 1 - a.first_pos;
    uint32_t* const p_thread = reinterpret_cast<uint32_t*>(a.scores) + (int64_t)row0 * a.stride + fblk;
    auto flush = [&](int64_t rc) {
        if (fblk >= a.n) return;
        const float* sl = &slot[rc & 1][0];
        uint32_t* const p_chunk = p_thread + rc * 32 * a.stride;
#pragma unroll
        for (int k = 0; k < 32 * NBG / kThreads; ++k) {
            const int row = row0 + RPK * k;
            const int64_t r = rc * 32 + row;
            if (r < a.rows && r >= r_cmp) {
                uint32_t* p = p_chunk + (int64_t)(RPK * k) * a.stride;
                if (fbad) {
                    atomicMax(reinterpret_cast<int*>(p), 0x7FC00000);   // NaN (as bits: no NaN semantics here)
                    atomicOr(a.err, DEVERR_TABLE);
                } else {
                    atomic_max_bits(p, sl[row * C::SROW + fb]);
                }
            }
        }
    };

    // Stage order: chunk by chunk, head group by head group.  At a stage's
    // barrier its queries are in LDS for every wave, every wave is done with
    // the other buffer, and the previous chunk's slot is complete.
    int sb = 0, ntl = 0;
    load_stage(rc_begin, 0);
    store_stage(0, 0);
    // Every load so far (keys, table entries, the first stage) complete on
    // every path into the loop: otherwise the compiler keeps the key loads
    // pending at the loop header, and the waits it places before the
    // multiplies would also wait for each stage's own prefetch.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int64_t rc = rc_begin; rc < rc_end; ++rc) {
        for (int hg = 0; hg < gm.hp; ++hg) {
            __syncthreads();
            // the next stage's loads, in flight while this stage multiplies
            const bool more = hg + 1 < gm.hp || rc + 1 < rc_end;
            const int64_t rc_n = hg + 1 < gm.hp ? rc : rc + 1;
            const int hg_n = hg + 1 < gm.hp ? hg + 1 : 0;
            if (more) load_stage(rc_n, hg_n);
            if (hg == 0) ntl = live_tiles(rc);
            const int ge = (g - hg * gm.hc) < gm.hc ? g - hg * gm.hc : gm.hc;
            if (ntl > 0) compute(sb, ge, ntl);
            if (hg + 1 == gm.hp) write_slot(rc);
            if (more) store_stage(hg_n, sb ^ 1);   // that buffer was last read before this barrier
            // The previous chunk's slot (complete since this stage's barrier)
            // goes out last: the wait for the next prefetch, a stage from now,
            // then finds these atomics long done.
            if (hg == 0 && rc > rc_begin) flush(rc - 1);
            sb ^= 1;
        }
    }
    __syncthreads();
    flush(rc_end - 1);
}

// -inf into n floats: VEC threads write 4 floats each with one 16-byte store
// (p 16-byte aligned), the last thread the ragged end.
template <bool VEC>
__global__ __launch_bounds__(256) void fill_neg_inf_kernel(uint32_t* p, int64_t n) {
    constexpr uint32_t kNegInf = 0xFF800000u;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if constexpr (VEC) {
        const int64_t i = t * 4;
        if (i + 4 <= n) {
            *reinterpret_cast<u32x4_t*>(p + i) = u32x4_t{kNegInf, kNegInf, kNegInf, kNegInf};
        } else {
            for (int64_t k = i; k < n; ++k) p[k] = kNegInf;
        }
    } else {
        if (t < n) p[t] = kNegInf;
    }
}

hipError_t fill_neg_inf(float* scores, int64_t n, hipStream_t st) {
    uint32_t* p = reinterpret_cast<uint32_t*>(scores);
    if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
        const int64_t blocks = ((n + 3) / 4 + 255) / 256;
        if (!grid_fits(blocks)) return hipErrorInvalidConfiguration;
        fill_neg_inf_kernel<true><<<(unsigned)blocks, 256, 0, st>>>(p, n);
    } else {
        const int64_t blocks = (n + 255) / 256;
        if (!grid_fits(blocks)) return hipErrorInvalidConfiguration;
        fill_neg_inf_kernel<false><<<(unsigned)blocks, 256, 0, st>>>(p, n);
    }
    return hipSuccess;
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

// waves the launch aims for when it splits the rows (two per SIMD)
#ifndef PRED_ROWS_TARGET_WAVES
#define PRED_ROWS_TARGET_WAVES 2048
#endif
// key tiles per wave: the keys' A operands take NKT * R / 4 registers
constexpr int rows_nkt(int r) { return r == 128 ? 2 : 4; }

template <int R, int BS>
hipError_t launch_rk(const RowScoreArgs& a, hipStream_t st) {
    constexpr int NKT = rows_nkt(R);
    using C = RowsCfg<R, NKT, BS>;
    RowGeom gm;
    const int g = a.Hq / a.Hk;
    gm.hc = g < C::HC ? g : C::HC;
    gm.hp = (g + gm.hc - 1) / gm.hc;
    gm.groups = (a.n * BS + C::KG - 1) / C::KG;
    const int64_t n_chunks = (a.rows + 31) / 32;
    const int64_t base_waves = gm.groups * a.Hk * kWaves;
    int64_t split = (PRED_ROWS_TARGET_WAVES + base_waves - 1) / base_waves;
    if (split > n_chunks) split = n_chunks;
    if (split < 1) split = 1;
    const int64_t cpp = (n_chunks + split - 1) / split;
    gm.chunks_per_part = (int)cpp;
    const int64_t parts = (n_chunks + cpp - 1) / cpp;   // no empty parts
    const int64_t wgs = (int64_t)a.Hk * gm.groups * parts;
    if (!grid_fits(wgs)) return hipErrorInvalidConfiguration;
    const hipError_t e = fill_neg_inf(a.scores, a.rows * a.stride, st);
    if (e != hipSuccess) return e;
    score_rows_kernel<R, NKT, BS><<<(unsigned)wgs, kThreads, 0, st>>>(a, gm);
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
    const bool b_ok = a.B == 8 || a.B == 16 || a.B == 32;
    return r_ok && b_ok;
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
    switch (a.R) {
        case 16: return launch_rb<16>(m, st);
        case 32: return launch_rb<32>(m, st);
        case 64: return launch_rb<64>(m, st);
        default: return launch_rb<128>(m, st);
    }
}

}  // namespace pred
