// Many-row block scorer for a prefill chunk (predictor.rs page, score_blocks,
// with many query rows): the same score as the decode kernel,
//   score[l, s, b] = max over rows i, heads h, tokens t of q_proj[l, s, i, h, :] . A[l, T[s, b], h / g, t, :]
// but with M * g queries per kv head it is a real contraction: for kv head k,
// Q_k [M*g, R] times A_k^T [R, n*B] followed by a max over the query axis and
// over each block's B columns.  It runs on bf16 MFMA (v_mfma_f32_32x32x16_bf16,
// f32 accumulation) with the max fused into the epilogue, so the [M*g, n*B]
// product never leaves registers.
//
// Tiling: a workgroup owns one (layer, sequence, kv head, query part) and 4
// waves x NKT key tiles of 32 keys (consecutive tokens of consecutive blocks).
// A wave keeps its keys as MFMA B operands in registers for the whole kernel.
// The part's queries stream through LDS in chunks of kChunk: the 256 threads
// load a chunk with coalesced 16-byte reads while the previous chunk is being
// multiplied, and every wave reads its A operands from LDS in the MFMA layout
// (rows padded by 16 bytes so one read's rows fall in distinct banks).  Each
// lane of the 32x32 f32 accumulator holds one key column (16 of the tile's 32
// query rows); the lane keeps a running max of its column over all query
// tiles.  At the end the two lane halves are combined, then the 8, 16 or 32
// lanes of one block, and the block's max goes to the score array with an
// integer atomic max (or min) on the float's bit pattern, which orders floats
// (kv heads and query parts sit in different workgroups).  A fill kernel sets
// the scores to -inf first.
//
// Workgroups are numbered kv-head fastest, so with 8 kv heads each XCD (which
// takes every 8th workgroup) serves one kv head and its L2 holds one kv head's
// queries.
#include "common.h"
#include "kernels.h"

namespace pred {

namespace {

constexpr int kWaves = 4;
#ifndef PRED_PREFILL_CHUNK
#define PRED_PREFILL_CHUNK 128
#endif
// Queries per LDS stage (a multiple of 32).  128 measured 2-3% faster than 64
// on the 2048-row chunk (one barrier per 64 MFMAs of a wave instead of 32).  A
// part's last chunk computes all its tiles, padding included: skipping tiles
// wholly past the queries behind a branch cost more than it saved there.
constexpr int kChunk = PRED_PREFILL_CHUNK;

struct PrefillGeom {
    int n_eff;            // queries per kv head = M * g
    int chunks;           // ceil(n_eff / kChunk)
    int q_split;          // query parts (workgroups per key group and kv head)
    int chunks_per_part;
    int64_t n_keys;       // n * B keys per sequence
    int64_t groups;       // key groups per (layer, sequence, kv head)
};

// R: projected width; NKT: 32-key tiles per wave; BS: block size in tokens.
template <int R, int NKT, int BS>
__global__ __launch_bounds__(256) void score_prefill_kernel(ScoreArgs a, PrefillGeom gm, uint32_t* __restrict__ bits) {
    constexpr int RS = R / 16;                  // MFMA k-steps of 16
    constexpr int CPR = R / 8;                  // 16-byte pieces per query vector
    constexpr int ROWB = R * 2 + 16;            // LDS bytes per query row (16 bytes of padding)
    constexpr int PIECES = kChunk * CPR;        // 16-byte pieces per chunk
    constexpr int PPT = (PIECES + 255) / 256;   // pieces per thread
    __shared__ __attribute__((aligned(16))) unsigned char lds[2][kChunk * ROWB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kv = (int)(blockIdx.x % a.Hk);
    int64_t rest = blockIdx.x / a.Hk;
    const int part = (int)(rest % gm.q_split);
    rest /= gm.q_split;
    const int64_t grp = rest % gm.groups;
    rest /= gm.groups;
    const int s = (int)(rest % a.S);
    const int l = (int)(rest / a.S);
    const int c_begin = part * gm.chunks_per_part;
    const int c_end = (c_begin + gm.chunks_per_part) < gm.chunks ? (c_begin + gm.chunks_per_part) : gm.chunks;
    if (c_begin >= c_end) return;   // whole workgroup: no query in this part
    const int g = a.Hq / a.Hk;
    const int col = lane & 31;      // key column of a tile / query row of a tile
    const int half = lane >> 5;     // which 8 of the 16 k-values of one MFMA step
    const int64_t key0 = (grp * kWaves + wave) * (NKT * 32);
    const bool active = key0 < gm.n_keys;   // wave-uniform; idle waves still take part in the barriers
    const int64_t layer = a.layer0 + l;
    const int64_t slot_elems = (int64_t)a.Hk * BS * R;

    // B operands: this lane's key column of every key tile, k-values st*16 + half*8 .. +8.
    bf16x8_t kb[NKT][RS];
    uint32_t live = 0;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
        const int64_t key = key0 + t * 32 + col;
        const uint16_t* src = a.ag;
        if (key < gm.n_keys) {
            const int64_t b = key / BS;
            const int tok = (int)(key - b * BS);
            const int64_t phys = a.tables ? (int64_t)a.tables[(int64_t)s * a.n + b] : b;
            if (phys >= 0 && phys < a.N) {
                src = a.ag + (layer * a.N + phys) * slot_elems + ((int64_t)kv * BS + tok) * R;
                live |= 1u << t;
            }
        }
#pragma unroll
        for (int st = 0; st < RS; ++st) kb[t][st] = load8(src + st * 16 + half * 8);
    }

    float rm[NKT];
#pragma unroll
    for (int t = 0; t < NKT; ++t) rm[t] = -__builtin_inff();

    // query chunk c -> registers (16-byte piece p: query row p / CPR, piece p % CPR)
    const uint16_t* qrows = a.qp + ((int64_t)l * a.S + s) * (int64_t)a.M * a.Hq * R;
    u32x4_t gq[PPT];
    // When g divides the chunk, a piece's (row, head) advance by a fixed step
    // per chunk: its offset is computed once and a whole chunk adds a constant.
    const bool steady = kChunk % g == 0;
    const int64_t chunk_step = steady ? (int64_t)(kChunk / g) * a.Hq * R : 0;
    int64_t piece_off[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int e = (tid + 256 * i) / CPR;
        piece_off[i] = steady ? ((int64_t)(e / g) * a.Hq + kv * g + e % g) * R + ((tid + 256 * i) % CPR) * 8 : 0;
    }
    auto load_chunk = [&](int c) {
        if (steady && (c + 1) * kChunk <= gm.n_eff) {
#pragma unroll
            for (int i = 0; i < PPT; ++i)
                if (PIECES % 256 == 0 || tid + 256 * i < PIECES)
                    gq[i] = *reinterpret_cast<const u32x4_t*>(qrows + c * chunk_step + piece_off[i]);
            return;
        }
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + 256 * i;
            if (PIECES % 256 == 0 || p < PIECES) {
                int e = c * kChunk + p / CPR;
                if (e >= gm.n_eff) e = gm.n_eff - 1;   // padding rows repeat a real query
                const int row = e / g;
                const int h = e - row * g;
                gq[i] = *reinterpret_cast<const u32x4_t*>(qrows + ((int64_t)row * a.Hq + kv * g + h) * R + (p % CPR) * 8);
            }
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + 256 * i;
            if (PIECES % 256 == 0 || p < PIECES)
                *reinterpret_cast<u32x4_t*>(&lds[buf][(p / CPR) * ROWB + (p % CPR) * 16]) = gq[i];
        }
    };
    // one 32-query tile of the chunk in LDS buffer buf
    auto tile = [&](int buf, int qt) {
        bf16x8_t qa[RS];
#pragma unroll
        for (int st = 0; st < RS; ++st)
            qa[st] = __builtin_bit_cast(bf16x8_t,
                    *reinterpret_cast<const uint4*>(&lds[buf][(qt * 32 + col) * ROWB + (st * 2 + half) * 16]));
        // all key tiles' MFMAs first, each into its own accumulator, so the
        // max epilogue of one tile overlaps the matrix work of the next
        f32x16_t acc[NKT];
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0], kb[t][0], f32x16_t{}, 0, 0, 0);
#pragma unroll
            for (int st = 1; st < RS; ++st)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[st], kb[t][st], acc[t], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            float m = rm[t];
#pragma unroll
            for (int i = 0; i < 16; i += 2) m = fmaxf(fmaxf(m, acc[t][i]), acc[t][i + 1]);
            rm[t] = m;
        }
        // Schedule: two MFMAs, then the max instructions that match them (8
        // max3 per key tile against RS MFMAs), repeated, so the max of one key
        // tile issues between the next tiles' MFMAs instead of after all of
        // them (r = 64: 2.5% faster than the compiler's own order)
#pragma unroll
        for (int i = 0; i < NKT * RS / 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);          // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 16 / RS, 0);    // VALU
        }
    };

    load_chunk(c_begin);
    store_chunk(0);
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
        const int buf = (c - c_begin) & 1;
        // The next chunk's loads are in flight while this chunk is multiplied.
        // They are issued on every iteration (the last one reloads its own
        // chunk) so that the newest loads are always queries: waiting for the
        // key operands then never waits for them.
        load_chunk(c + 1 < c_end ? c + 1 : c);
        if (active) {
#pragma unroll
            for (int qt = 0; qt < kChunk / 32; ++qt) tile(buf, qt);
        }
        store_chunk(buf ^ 1);   // that buffer was last read before the previous barrier
        __syncthreads();
    }
    if (!active) return;

    uint32_t* out = bits + ((int64_t)l * a.S + s) * a.n;
    const int fill_s = fill_of(a, s);   // tokens of the last block that are scored
    if (a.fill && grp == 0 && kv == 0 && part == 0 && l == 0 && tid == 0 && (a.fill[s] < 0 || a.fill[s] > BS))
        atomicOr(a.err, DEVERR_FILL);
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
        {
            const int64_t key = key0 + t * 32 + col;
            if (key / BS == a.n - 1 && (int)(key % BS) >= fill_s) rm[t] = -__builtin_inff();
        }
        float v = fmaxf(rm[t], lane_xor<32>(rm[t]));   // rows split across the two lane halves
        v = fmaxf(v, lane_xor<1>(v));
        v = fmaxf(v, lane_xor<2>(v));
        if constexpr (BS >= 8) v = fmaxf(v, lane_xor<7>(v));
        if constexpr (BS >= 16) v = fmaxf(v, lane_xor<15>(v));
        if constexpr (BS >= 32) v = fmaxf(v, lane_xor<16>(v));
        const int64_t key = key0 + t * 32 + col;
        if (half == 0 && (col % BS) == 0 && key < gm.n_keys) {
            if ((live >> t) & 1u) {
                atomic_max_bits(out + key / BS, v);
            } else if (kv == 0 && part == 0) {
                atomicMax(reinterpret_cast<int*>(out + key / BS), 0x7FC00000);   // NaN: above every number's bits
                atomicOr(a.err, DEVERR_TABLE);
            }
        }
    }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

template <int R, int NKT, int BS>
void launch_t(const ScoreArgs& a, const PrefillGeom& gm, uint32_t* keys, hipStream_t st) {
    const int64_t wgs = gm.groups * gm.q_split * a.Hk * a.S * a.n_layers;
    score_prefill_kernel<R, NKT, BS><<<(unsigned)wgs, 256, 0, st>>>(a, gm, keys);
}

template <int R, int NKT>
void launch_bs(const ScoreArgs& a, const PrefillGeom& gm, uint32_t* keys, hipStream_t st) {
    switch (a.B) {
        case 8: launch_t<R, NKT, 8>(a, gm, keys, st); break;
        case 16: launch_t<R, NKT, 16>(a, gm, keys, st); break;
        default: launch_t<R, NKT, 32>(a, gm, keys, st); break;
    }
}

// 32-key tiles per wave: the keys' B operands take NKT * R / 4 registers
constexpr int nkt_for(int r) { return r == 128 ? 2 : 4; }

// waves the launch aims for when it splits the query axis (two per SIMD)
#ifndef PRED_PREFILL_TARGET_WAVES
#define PRED_PREFILL_TARGET_WAVES 2048
#endif
constexpr int64_t kTargetWaves = PRED_PREFILL_TARGET_WAVES;

}  // namespace

bool prefill_supported(const ScoreArgs& a) {
    return (a.R == 16 || a.R == 32 || a.R == 64 || a.R == 128) && (a.B == 8 || a.B == 16 || a.B == 32);
}

hipError_t launch_score_prefill(const ScoreArgs& a, hipStream_t st) {
    PrefillGeom gm;
    const int g = a.Hq / a.Hk;
    gm.n_eff = a.M * g;
    gm.chunks = (gm.n_eff + kChunk - 1) / kChunk;
    gm.n_keys = a.n * a.B;
    const int64_t keys_per_group = (int64_t)kWaves * nkt_for(a.R) * 32;
    gm.groups = (gm.n_keys + keys_per_group - 1) / keys_per_group;
    // split the query axis when the key groups alone give too few waves
    const int64_t base_waves = gm.groups * a.Hk * a.S * a.n_layers * kWaves;
    int64_t split = (kTargetWaves + base_waves - 1) / base_waves;
    if (split > gm.chunks) split = gm.chunks;
    if (split < 1) split = 1;
    gm.chunks_per_part = (int)((gm.chunks + split - 1) / split);
    gm.q_split = (gm.chunks + gm.chunks_per_part - 1) / gm.chunks_per_part;   // no empty parts
    uint32_t* keys = reinterpret_cast<uint32_t*>(a.scores);
    const int64_t total = (int64_t)a.n_layers * a.S * a.n;
    if (!grid_fits(gm.groups * gm.q_split * a.Hk * a.S * a.n_layers) || !grid_fits((total + 255) / 256))
        return hipErrorInvalidConfiguration;
    const unsigned fill_grid = (unsigned)((total + 255) / 256);
    fill_u32_kernel<<<fill_grid, 256, 0, st>>>(keys, total, 0xFF800000u);   // -inf
    switch (a.R) {
        case 16: launch_bs<16, nkt_for(16)>(a, gm, keys, st); break;
        case 32: launch_bs<32, nkt_for(32)>(a, gm, keys, st); break;
        case 64: launch_bs<64, nkt_for(64)>(a, gm, keys, st); break;
        default: launch_bs<128, nkt_for(128)>(a, gm, keys, st); break;
    }
    return hipGetLastError();
}

}  // namespace pred
