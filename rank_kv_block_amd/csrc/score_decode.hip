// Decode block scorer (predictor.rs page: score_blocks / predictor_score):
//   score[l, s, b] = max over rows i, heads h, tokens t of
//                    sum_j q_proj[l, s, i, h, j] * A_g[layer0 + l, table[s, b], h / g, t, j]
// for the case where a kv head's query set (rows x GQA group, padded to a power
// of two QH <= 16) fits in registers.  The kernel streams A_g once.
//
// Data layout per A_g slot: [Hk][B][R] bf16.  A kv head's region of one slot is
// B rows of R values, U = B * R / 8 chunks of 16 bytes.  A wave reads 64
// consecutive chunks with one 16-byte load per lane (1 KiB, fully coalesced);
// LPR = R / 8 consecutive lanes hold one row, lane p of a row holding values
// [8p, 8p + 8).  A lane takes the dot products of its 8 values with all QH
// queries of the kv head (4 v_dot2c_f32_bf16 each) and the LPR lanes of a row
// then add their partial sums with DPP.
//
// Reduction across a row without a full butterfly per head: lane p keeps its
// partial sums in a lane-specific order -- register i holds head label
// i ^ f(p).  At level m the partner lane is p ^ M_m (M = 1, 2, 7, 15, 16:
// quad_perm, quad_perm, row_half_mirror, row_mirror, swizzle), each lane keeps
// the lower half of its registers and adds the partner's upper half.  With
// f linear over GF(2) and f(M_m) = QH >> (m + 1) the labels the two lanes add
// are the same head, so level m costs QH >> (m + 1) DPP adds instead of QH,
// and after log2(LPR) levels each lane holds complete dot products of
// max(QH / LPR, 1) heads.  The block max then needs no sums at all.
#include "common.h"
#include "kernels.h"

// Tuning knobs (compile-time).  PRED_DECODE_AUX is the cache-policy field of
// the streamed A_g buffer loads: 2 = nontemporal (A_g is read once per call,
// so it should not displace q_proj, tables and other cached data), measured
// 5-8% faster than the default policy.  WAVES_PER_EU caps registers for that
// many waves per SIMD (0 = compiler's choice).
#ifndef PRED_DECODE_AUX
#define PRED_DECODE_AUX 2
#endif
#ifndef PRED_DECODE_ROTATE
#define PRED_DECODE_ROTATE 1
#endif
#ifndef PRED_DECODE_WAVES_PER_EU
#define PRED_DECODE_WAVES_PER_EU 0
#endif
// Queries per kv head (rows x GQA group) from which the matrix-core variant
// scores instead of the vector-ALU dot products (at 4 queries both stream at
// the same rate: 316 vs 315-318 us for 32 layers x 8192 blocks).
#ifndef PRED_DECODE_MFMA_MIN_QUERIES
#define PRED_DECODE_MFMA_MIN_QUERIES 5
#endif
// Matrix-core decode with 4 wave-loads per kv region: split each block over
// two waves of 2 load slots (1) or give each wave a whole block (0).  Split
// measured 157.5 vs 159.3 us for a 70B-shaped layer (32768 blocks of 32 KiB),
// in alternating runs on one MI355X (smaller work items shorten the drain).
#ifndef PRED_DECODE_MFMA_SPLIT
#define PRED_DECODE_MFMA_SPLIT 1
#endif

namespace pred {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                          false);
}

// Value of `v` held by this lane's partner at reduction level M.
template <int M>
__device__ inline float partner(float v) {
    if constexpr (M == 0) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));  // xor 1
    } else if constexpr (M == 1) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));  // xor 2
    } else if constexpr (M == 2) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));  // 7 - p
    } else if constexpr (M == 3) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));  // 15 - p
    } else {
        return __shfl_xor(v, 16);  // xor 16
    }
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

// Label offset f(p): decompose p over the level masks (1, 2, 7, 15, 16), whose
// top bits are bits 0..4, and xor together the QH >> (m + 1) of the masks used.
template <int LPR, int QH>
__device__ inline int label_xor(int p) {
    constexpr int msk[5] = {1, 2, 7, 15, 16};
    int f = 0;
#pragma unroll
    for (int m = ilog2(LPR) - 1; m >= 0; --m) {
        if ((p >> m) & 1) {
            p ^= msk[m];
            f ^= (QH >> (m + 1));
        }
    }
    return f;
}

template <int LPR, int QH, int M>
__device__ inline void reduce_levels(float* v) {
    if constexpr ((1 << M) < LPR) {
        constexpr int w = (QH >> M) > 0 ? (QH >> M) : 1;
        if constexpr (w >= 2) {
#pragma unroll
            for (int i = 0; i < w / 2; ++i) v[i] += partner<M>(v[i + w / 2]);
        } else {
            v[0] += partner<M>(v[0]);
        }
        reduce_levels<LPR, QH, M + 1>(v);
    }
}

__device__ inline float wave_max_xor(float v, int upto) {
    // max over aligned groups of `upto` lanes (power of two, <= 64)
    if (upto > 1) v = fmaxf(v, partner<0>(v));
    if (upto > 2) v = fmaxf(v, partner<1>(v));
    if (upto > 4) v = fmaxf(v, partner<2>(v));
    if (upto > 8) v = fmaxf(v, partner<3>(v));
    if (upto > 16) v = fmaxf(v, __shfl_xor(v, 16));
    if (upto > 32) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

struct DecodeGeom {
    int U, log2U;          // chunks per (block, kv head) region; U is a power of two
    int NBW;               // blocks per wave
    int SPB;               // load slots per block (U / 64 when U >= 64, else 1)
    int n_eff;             // effective heads per kv head = M * g
    int n_groups;          // ceil(n_eff / QH)
    int q_chunks;          // 16-byte chunks of one (layer, sequence) q_proj slab [M, Hq, R]
    int64_t wgs_per_seq;   // workgroups per (layer, sequence); a workgroup never spans two
    int WPB;               // waves per block (2: a block's kv regions split over two waves)
};

constexpr int kWaves = 4;

// QLDS: the (layer, sequence) q_proj slab is staged in LDS once per workgroup
// and every wave reads its query fragments from there, which keeps the vector
// memory pipeline for A_g alone.  UNI: a kv head's region of a block spans one
// or more whole wave-loads (U >= 64), so the block of every load slot is the
// same across the wave and its table entry and slab offset are scalar.
// Off: 32-bit byte offsets when a layer's slab is below 4 GiB, else 64-bit.
template <int LPR, int QH, int NS, bool QLDS, typename Off, bool UNI>
__global__ __launch_bounds__(256)
#if PRED_DECODE_WAVES_PER_EU
__attribute__((amdgpu_waves_per_eu(PRED_DECODE_WAVES_PER_EU)))
#endif
void score_decode_kernel(ScoreArgs a, DecodeGeom gm) {
    extern __shared__ uint4 q_lds[];
    const int lane = threadIdx.x & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wgb = blockIdx.x % gm.wgs_per_seq;
    const int64_t ls = blockIdx.x / gm.wgs_per_seq;
    const int s = (int)(ls % a.S);
    const int l = (int)(ls / a.S);
    const int64_t b_first = (wgb * kWaves + wave_id) * gm.NBW;
    const uint16_t* qrows = a.qp + ((int64_t)l * a.S + s) * (int64_t)a.M * a.Hq * a.R;
    const bool has_work = b_first < a.n;   // wave-uniform; idle waves still meet the barrier
    const int p = lane & (LPR - 1);
    const int g = a.Hq / a.Hk;
    const int64_t layer = a.layer0 + l;
    const int64_t slot_elems = (int64_t)a.Hk * a.B * a.R;

    // Per load slot: byte offset, within this layer's A_g slab, of the lane's
    // row of its block's region at kv head 0.  The wave's NBW table entries
    // (consecutive logical blocks) come in with one coalesced load, lane j
    // holding block j, and each slot takes its block's entry from that lane.
    // Slots past the end or with an invalid entry read the slab's first slot
    // and are masked out of the max.
    const char* slab = reinterpret_cast<const char*>(a.ag + layer * a.N * slot_elems);
    int32_t tab_lane = -1;
    {
        const int64_t b = b_first + lane;
        if (lane < gm.NBW && b < a.n) tab_lane = a.tables ? a.tables[(int64_t)s * a.n + b] : (int32_t)b;
    }
    // the sequence's last block holds fill_s tokens; its other rows are left out
    // of the max (only the live bit of their slots changes, nothing per step)
    const int fill_s = fill_of(a, s);
    if (a.fill && wgb == 0 && threadIdx.x == 0 && (a.fill[s] < 0 || a.fill[s] > a.B)) atomicOr(a.err, DEVERR_FILL);
    Off voff[NS];
    uint32_t soff_slot[NS];   // UNI: the whole slot offset is wave-uniform (SGPR)
    uint32_t live = 0;
    uint32_t okbits = 0;      // slot sl's block has a valid table entry (the stores reuse it)
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
        const int f = sl * 64 + lane;
        const int bi = UNI ? ((sl * 64) >> gm.log2U) : (f >> gm.log2U);
        const int t = (f & (gm.U - 1)) / LPR;
        int32_t phys;
        if constexpr (UNI) phys = __builtin_amdgcn_readlane(tab_lane, bi);
        else phys = __shfl(tab_lane, bi);
        const bool ok = bi < gm.NBW && b_first + bi < a.n && phys >= 0 && (int64_t)phys < a.N;
        voff[sl] = (Off)(((ok ? (int64_t)phys : 0) * slot_elems + (int64_t)t * a.R + p * 8) * 2);
        // UNI: row t, lane part p of slot sl is byte 1024 * (sl % SPB) + 16 * lane of the block's region
        soff_slot[sl] = (uint32_t)((ok ? (int64_t)phys : 0) * slot_elems * 2 + 1024 * (sl % gm.SPB));
        const bool cut = b_first + bi == a.n - 1 && t >= fill_s;
        live |= ((ok && !cut) ? 1u : 0u) << sl;
        okbits |= (ok ? 1u : 0u) << sl;
    }

    float rm[NS];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) rm[sl] = -__builtin_inff();

    const int fx = label_xor<LPR, QH>(p);
    const int64_t kv_bytes = (int64_t)a.B * a.R * 2;
    // 32-bit offsets: raw buffer loads with the slab as the resource base, the
    // lane offset in a VGPR and the kv-head offset in an SGPR.
    __amdgpu_buffer_rsrc_t rsrc;
    if constexpr (sizeof(Off) == 4)
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(slab), (short)0, (int)0xFFFFFFFF, 0x00020000);
    auto load_a = [&](uint4 (&dst)[NS], int kv) {
        if constexpr (sizeof(Off) == 4 && UNI) {
            const uint32_t kvoff = (uint32_t)(kv * kv_bytes);
#pragma unroll
            for (int sl = 0; sl < NS; ++sl)
                dst[sl] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rsrc, lane * 16, (int)(soff_slot[sl] + kvoff), PRED_DECODE_AUX));
        } else if constexpr (sizeof(Off) == 4) {
            const int soff = (int)(kv * kv_bytes);
#pragma unroll
            for (int sl = 0; sl < NS; ++sl)
                dst[sl] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)voff[sl], soff, PRED_DECODE_AUX));
        } else {
            const char* kbase = slab + kv * kv_bytes;
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) dst[sl] = *reinterpret_cast<const uint4*>(kbase + voff[sl]);
        }
    };
    // Query fragment i of this lane at kv head 0, in 16-byte units: computed
    // once per head group, the kv head only adds g*R/8 per step.
    int qoff[QH];
    auto set_qoff = [&](int hg) {
#pragma unroll
        for (int i = 0; i < QH; ++i) {
            int e = hg * QH + (i ^ fx);
            if (e >= gm.n_eff) e = gm.n_eff - 1;  // padding: repeat a real head (max unchanged)
            const int row = e / g;
            const int h = e - row * g;
            qoff[i] = (int)((((int64_t)row * a.Hq + h) * a.R + p * 8) >> 3);
        }
    };
    const int q_kv_step = g * a.R / 8;
    auto score_kv = [&](const uint4 (&av)[NS], int kv, int hg) {
        (void)hg;
        uint32_t q[QH][4];
#pragma unroll
        for (int i = 0; i < QH; ++i) {
            const int o = qoff[i] + kv * q_kv_step;
            uint4 w;
            if constexpr (QLDS) w = q_lds[o];
            else w = reinterpret_cast<const uint4*>(qrows)[o];
            q[i][0] = w.x; q[i][1] = w.y; q[i][2] = w.z; q[i][3] = w.w;
        }
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            float v[QH];
#pragma unroll
            for (int i = 0; i < QH; ++i) {
                float acc = dot2(av[sl].x, q[i][0], 0.0f);
                acc = dot2(av[sl].y, q[i][1], acc);
                acc = dot2(av[sl].z, q[i][2], acc);
                v[i] = dot2(av[sl].w, q[i][3], acc);
            }
            reduce_levels<LPR, QH, 0>(v);
            constexpr int rem = (QH / LPR) > 0 ? (QH / LPR) : 1;
            float mx = v[0];
#pragma unroll
            for (int i = 1; i < rem; ++i) mx = fmaxf(mx, v[i]);
            rm[sl] = ((live >> sl) & 1u) ? fmaxf(rm[sl], mx) : rm[sl];
        }
    };

    // Two buffers in ping-pong: the loads of kv head k+1 are in flight while
    // kv head k is scored.  The steady-state loop has no conditional loads, so
    // each score step waits only for its own buffer.  The first buffer is
    // requested before q_proj is staged in LDS, so both round trips overlap.
    // Each wave starts at a different kv head (and wraps around), so the waves
    // in flight spread their reads over every kv region's offset instead of
    // all hitting offset k * B * R * 2 of their slots at the same time.
    const int kv0 = PRED_DECODE_ROTATE ? (int)((b_first / gm.NBW) % a.Hk) : 0;
    auto kvr = [&](int k) { const int r = kv0 + k; return r < a.Hk ? r : r - a.Hk; };
    uint4 A0[NS], A1[NS];
    if (has_work) load_a(A0, kvr(0));
    if constexpr (QLDS) {
        const uint4* src = reinterpret_cast<const uint4*>(qrows);
        for (int i = threadIdx.x; i < gm.q_chunks; i += 256) q_lds[i] = src[i];
        __syncthreads();
    }
    if (!has_work) return;   // after the only barrier
    for (int hg = 0; hg < gm.n_groups; ++hg) {
        set_qoff(hg);
        if (hg > 0) load_a(A0, kvr(0));
        int kv = 0;
        for (; kv + 2 < a.Hk; kv += 2) {
            load_a(A1, kvr(kv + 1));
            score_kv(A0, kvr(kv), hg);
            load_a(A0, kvr(kv + 2));
            score_kv(A1, kvr(kv + 1), hg);
        }
        if (kv + 1 < a.Hk) {
            load_a(A1, kvr(kv + 1));
            score_kv(A0, kvr(kv), hg);
            score_kv(A1, kvr(kv + 1), hg);
        } else {
            score_kv(A0, kvr(kv), hg);
        }
    }

    // Block maxima and stores.
    float* out = a.scores + ((int64_t)l * a.S + s) * a.n;
    // slot sl holds block bi for the storing lane; its table check was made at set-up
    auto store = [&](int bi, int sl, float v) {
        const int64_t b = b_first + bi;
        if (bi < gm.NBW && b < a.n) {
            if ((okbits >> sl) & 1u) {
                out[b] = v;
            } else {
                out[b] = __uint_as_float(0x7FC00000u);
                atomicOr(a.err, DEVERR_TABLE);
            }
        }
    };
    if (gm.U >= 64) {
        // a kv region spans SPB whole load slots (slot sl holds block sl / SPB,
        // also without UNI): the block's max runs over its SPB slots
        float acc = -__builtin_inff();
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            acc = fmaxf(acc, rm[sl]);
            if ((sl + 1) % gm.SPB == 0) {
                const float v = wave_max_xor(acc, 64);
                if (lane == 0) store(sl / gm.SPB, sl, v);
                acc = -__builtin_inff();
            }
        }
    } else {
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            const float v = wave_max_xor(rm[sl], gm.U);
            const int f = sl * 64 + lane;
            if ((lane & (gm.U - 1)) == 0) store(f >> gm.log2U, sl, v);
        }
    }
}

// Matrix-core variant for kv heads with 5..16 queries (rows x GQA group), where
// the dot products above would cost ~8-16 VALU instructions per loaded word.
// It streams A_g exactly as the kernel above (one contiguous 1 KiB wave-load per
// load slot, slot offsets in SGPRs) and multiplies each wave-load on
// v_mfma_f32_16x16x32_bf16 against the kv head's queries (B operand [32, 16]:
// column n is query n, columns past the query count repeat a real query).
//
// A wave-load holds 16 / H token rows of R values, H = R / 32.  The MFMA's 16
// A rows are (token, part) pairs: row m is part m % H (values [32p, 32p + 32))
// of token m / H, and lane (m, c) = (lane % 16, lane / 16) takes 16-byte piece
// 4p + c of that row -- a permutation of the 1 KiB, so the load stays one
// contiguous access.  MFMA j multiplies the whole tile by values
// [32j, 32j + 32) of the queries; row m is meaningful in MFMA j = m % H only,
// and the full dot product of a token is the sum over its H rows, each from its
// own MFMA.  Accumulator lane (n, c) holds rows 4c .. 4c + 3 of column n, i.e.
// tokens 4c/H .. of the wave-load, so the sums stay inside a lane: token
// 4c/H + v gets sum over p of C_p[v*H + p].
template <int R, int NS, int WPB>
__global__ __launch_bounds__(256) void score_decode_mfma_kernel(ScoreArgs a, DecodeGeom gm) {
    constexpr int H = R / 32;             // parts per token row = MFMAs per wave-load
    constexpr int ROWB = R * 2;           // bytes per token row
    constexpr int TPL = 4 / H;            // tokens per accumulator lane per wave-load
    static_assert(NS <= 16, "4 live bits per load slot in 64 bits");
    extern __shared__ uint4 q_lds[];
    const int lane = threadIdx.x & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wgb = blockIdx.x % gm.wgs_per_seq;
    const int64_t ls = blockIdx.x / gm.wgs_per_seq;
    const int s = (int)(ls % a.S);
    const int l = (int)(ls / a.S);
    const int64_t b_first = ((wgb * kWaves + wave_id) / WPB) * gm.NBW;
    const int pbase = (wave_id % WPB) * NS;   // first wave-load of the block's regions this wave streams
    const uint16_t* qrows = a.qp + ((int64_t)l * a.S + s) * (int64_t)a.M * a.Hq * R;
    const bool has_work = b_first < a.n;
    const int m = lane & 15;
    const int c = lane >> 4;
    const int g = a.Hq / a.Hk;
    const int64_t layer = a.layer0 + l;
    const int64_t slot_bytes = (int64_t)a.Hk * a.B * ROWB;
    const char* slab = reinterpret_cast<const char*>(a.ag + layer * a.N * (slot_bytes >> 1));
    int32_t tab_lane = -1;
    {
        const int64_t b = b_first + lane;
        if (lane < gm.NBW && b < a.n) tab_lane = a.tables ? a.tables[(int64_t)s * a.n + b] : (int32_t)b;
    }
    const int fill_s = fill_of(a, s);
    if (a.fill && wgb == 0 && threadIdx.x == 0 && (a.fill[s] < 0 || a.fill[s] > a.B)) atomicOr(a.err, DEVERR_FILL);
    // Slot sl: block bi = sl / SPB, wave-load sl % SPB of its kv region (tokens
    // (sl % SPB) * 16 / H ..).  live: TPL bits per slot, token 4c/H + v scored.
    uint32_t soff_slot[NS];
    uint64_t live = 0;
    uint32_t okbits = 0;   // slot sl's block has a valid table entry (the stores reuse it)
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
        const int bi = (sl * 64) >> gm.log2U;
        const int piece = pbase + sl - bi * gm.SPB;
        const int32_t phys = __builtin_amdgcn_readlane(tab_lane, bi);
        const bool ok = bi < gm.NBW && b_first + bi < a.n && phys >= 0 && (int64_t)phys < a.N;
        soff_slot[sl] = (uint32_t)((ok ? (int64_t)phys : 0) * slot_bytes + 1024 * piece);
        const bool last = b_first + bi == a.n - 1;
        uint32_t bits = 0;
#pragma unroll
        for (int v = 0; v < TPL; ++v) {
            const int tok = piece * (16 / H) + (4 * c) / H + v;
            bits |= ((ok && !(last && tok >= fill_s)) ? 1u : 0u) << v;
        }
        live |= (uint64_t)bits << (4 * sl);
        okbits |= (ok ? 1u : 0u) << sl;
    }
    float rm[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) rm[t] = -__builtin_inff();

    // query column m of kv head 0, 16-byte units; the kv head adds g*R/8, MFMA j adds 4j
    const int e = m < gm.n_eff ? m : gm.n_eff - 1;
    const int qrow = e / g;
    const int qoff = (int)((((int64_t)qrow * a.Hq + (e - qrow * g)) * R + c * 8) >> 3);
    const int q_kv_step = g * R / 8;
    const int64_t kv_bytes = (int64_t)a.B * ROWB;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(slab), (short)0, (int)0xFFFFFFFF, 0x00020000);
    const int voff = (m / H) * ROWB + ((m % H) * 4 + c) * 16;
    auto load_a = [&](u32x4_t (&dst)[NS], int kv) {
        const uint32_t kvoff = (uint32_t)(kv * kv_bytes);
#pragma unroll
        for (int sl = 0; sl < NS; ++sl)
            dst[sl] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rsrc, voff, (int)(soff_slot[sl] + kvoff), PRED_DECODE_AUX));
    };
    auto score_kv = [&](const u32x4_t (&av)[NS], int kv) {
        bf16x8_t qb[H];
#pragma unroll
        for (int j = 0; j < H; ++j) qb[j] = __builtin_bit_cast(bf16x8_t, q_lds[qoff + kv * q_kv_step + j * 4]);
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            f32x4_t cp[H];
#pragma unroll
            for (int j = 0; j < H; ++j)
                cp[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[sl]), qb[j],
                                                                f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            const uint32_t bits = (uint32_t)(live >> (4 * sl)) & 0xFu;
            float mx = rm[sl];
#pragma unroll
            for (int v = 0; v < TPL; ++v) {
                float d = cp[0][v * H];
#pragma unroll
                for (int j = 1; j < H; ++j) d += cp[j][v * H + j];
                mx = ((bits >> v) & 1u) ? fmaxf(mx, d) : mx;
            }
            rm[sl] = mx;
        }
    };

    const int kv0 = PRED_DECODE_ROTATE ? (int)((b_first / gm.NBW) % a.Hk) : 0;
    auto kvr = [&](int k) { const int r = kv0 + k; return r < a.Hk ? r : r - a.Hk; };
    u32x4_t A0[NS], A1[NS];
    if (has_work) load_a(A0, kvr(0));
    {
        const uint4* src = reinterpret_cast<const uint4*>(qrows);
        for (int i = threadIdx.x; i < gm.q_chunks; i += 256) q_lds[i] = src[i];
        __syncthreads();
    }
    if (WPB == 1 && !has_work) return;   // after the only barrier (a split block meets one more)
    if (has_work) {
        int kv = 0;
        for (; kv + 2 < a.Hk; kv += 2) {
            load_a(A1, kvr(kv + 1));
            score_kv(A0, kvr(kv));
            load_a(A0, kvr(kv + 2));
            score_kv(A1, kvr(kv + 1));
        }
        if (kv + 1 < a.Hk) {
            load_a(A1, kvr(kv + 1));
            score_kv(A0, kvr(kv));
            score_kv(A1, kvr(kv + 1));
        } else {
            score_kv(A0, kvr(kv));
        }
    }

    float* out = a.scores + ((int64_t)l * a.S + s) * a.n;
    // slot sl holds block b; its table check was made at set-up
    auto store = [&](int64_t b, int sl, float v) {
        if ((okbits >> sl) & 1u) {
            out[b] = v;
        } else {
            out[b] = __uint_as_float(0x7FC00000u);
            atomicOr(a.err, DEVERR_TABLE);
        }
    };
    if constexpr (WPB > 1) {
        // one block per wave pair: each wave's max of its half, combined in LDS
        __shared__ float half_max[kWaves];
        float acc = -__builtin_inff();
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) acc = fmaxf(acc, rm[sl]);
        acc = wave_max_xor(acc, 64);
        if (lane == 0) half_max[wave_id] = acc;
        __syncthreads();
        if (has_work && lane == 0 && wave_id % WPB == 0) {
            float v = half_max[wave_id];
#pragma unroll
            for (int w = 1; w < WPB; ++w) v = fmaxf(v, half_max[wave_id + w]);
            store(b_first, 0, v);
        }
        return;
    } else {
        float acc = -__builtin_inff();
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            acc = fmaxf(acc, rm[sl]);
            if ((sl + 1) % gm.SPB == 0) {
                const float v = wave_max_xor(acc, 64);
                const int bi = sl / gm.SPB;
                const int64_t b = b_first + bi;
                if (lane == 0 && bi < gm.NBW && b < a.n) store(b, sl, v);
                acc = -__builtin_inff();
            }
        }
    }
}

// Any shape: one thread per (layer, sequence, block), plain loops.  Used when
// R or block_size is not one the streaming kernel is laid out for.
__global__ __launch_bounds__(256) void score_generic_kernel(ScoreArgs a) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.n_layers * a.S * a.n;
    if (id >= total) return;
    const int64_t b = id % a.n;
    const int64_t ls = id / a.n;
    const int s = (int)(ls % a.S);
    const int l = (int)(ls / a.S);
    const int g = a.Hq / a.Hk;
    const int64_t phys = a.tables ? (int64_t)a.tables[(int64_t)s * a.n + b] : b;
    if (phys < 0 || phys >= a.N) {
        a.scores[id] = __uint_as_float(0x7FC00000u);
        atomicOr(a.err, DEVERR_TABLE);
        return;
    }
    const uint16_t* slot = a.ag + ((a.layer0 + l) * a.N + phys) * (int64_t)a.Hk * a.B * a.R;
    const uint16_t* qrows = a.qp + ((int64_t)l * a.S + s) * (int64_t)a.M * a.Hq * a.R;
    const int n_tok = b == a.n - 1 ? fill_of(a, s) : a.B;
    if (a.fill && b == a.n - 1 && l == 0 && (a.fill[s] < 0 || a.fill[s] > a.B)) atomicOr(a.err, DEVERR_FILL);
    float best = -__builtin_inff();
    for (int i = 0; i < a.M; ++i)
        for (int h = 0; h < a.Hq; ++h) {
            const uint16_t* qv = qrows + ((int64_t)i * a.Hq + h) * a.R;
            const uint16_t* kbase = slot + (int64_t)(h / g) * a.B * a.R;
            for (int t = 0; t < n_tok; ++t) {
                float acc = 0.0f;
                for (int j = 0; j < a.R; ++j)
                    acc = __builtin_fmaf(__uint_as_float((uint32_t)qv[j] << 16),
                                         __uint_as_float((uint32_t)kbase[(int64_t)t * a.R + j] << 16), acc);
                best = fmaxf(best, acc);
            }
        }
    a.scores[id] = best;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int pick_qh(int n_eff) {
    int qh = 1;
    while (qh < n_eff && qh < 16) qh <<= 1;
    return qh;
}

constexpr int kQLdsMaxBytes = 32768;

// Everything the launcher decides for one call: which kernel, its template
// arguments and its geometry.  The launch and the reported variant name both
// come from this one decision.
struct DecodePlan {
    int kind;        // SCORE_PATH_* of the kernel that runs: generic, decode (vector ALU) or decode_mfma
    DecodeGeom gm;
    int ns, lpr, qh; // load slots per wave, lanes per row, queries per register group
    bool q_lds;      // q_proj slab staged in LDS (it fits in 32 KiB)
    bool wide;       // a layer's slab is 4 GiB or more (64-bit slab offsets, as without q_lds)
    bool uni;        // a kv region spans whole wave-loads (wave-uniform slot offsets)
};

template <int LPR, int QH, int NS>
void launch_decode_t(const ScoreArgs& a, const DecodePlan& pl, hipStream_t st) {
    const DecodeGeom& gm = pl.gm;
    const unsigned grid = (unsigned)(gm.wgs_per_seq * a.S * a.n_layers);
    const int q_bytes = gm.q_chunks * 16;
    if (pl.q_lds && !pl.wide) {
        if (pl.uni) score_decode_kernel<LPR, QH, NS, true, uint32_t, true><<<grid, 256, q_bytes, st>>>(a, gm);
        else score_decode_kernel<LPR, QH, NS, true, uint32_t, false><<<grid, 256, q_bytes, st>>>(a, gm);
    } else if (pl.q_lds) {
        score_decode_kernel<LPR, QH, NS, true, uint64_t, false><<<grid, 256, q_bytes, st>>>(a, gm);
    } else {
        score_decode_kernel<LPR, QH, NS, false, uint64_t, false><<<grid, 256, 0, st>>>(a, gm);
    }
}

template <int LPR, int NS>
void launch_decode_qh(const ScoreArgs& a, const DecodePlan& pl, hipStream_t st) {
    switch (pl.qh) {
        case 1: launch_decode_t<LPR, 1, NS>(a, pl, st); break;
        case 2: launch_decode_t<LPR, 2, NS>(a, pl, st); break;
        case 4: launch_decode_t<LPR, 4, NS>(a, pl, st); break;
        case 8: launch_decode_t<LPR, 8, NS>(a, pl, st); break;
        default: launch_decode_t<LPR, 16, NS>(a, pl, st); break;
    }
}

template <int NS>
void launch_decode_ns(const ScoreArgs& a, const DecodePlan& pl, hipStream_t st) {
    switch (pl.lpr) {
        case 2: launch_decode_qh<2, NS>(a, pl, st); break;
        case 4: launch_decode_qh<4, NS>(a, pl, st); break;
        case 8: launch_decode_qh<8, NS>(a, pl, st); break;
        default: launch_decode_qh<16, NS>(a, pl, st); break;
    }
}

// Geometry of the streaming kernels; mfma: the slot count for
// score_decode_mfma_kernel (2 with a split block, 4 or 16).
bool decode_geometry(const ScoreArgs& a, DecodeGeom& gm, int& ns, int& lpr, int& qh, bool mfma = false) {
    if (!(a.R == 16 || a.R == 32 || a.R == 64 || a.R == 128)) return false;
    lpr = a.R / 8;
    const int64_t U = (int64_t)a.B * lpr;
    if (!is_pow2(U) || U > 1024 || U < 8) return false;
    gm.U = (int)U;
    gm.log2U = 0;
    while ((1 << gm.log2U) < gm.U) ++gm.log2U;
    // 4 load slots per wave (two 4 KiB buffers in flight): measured faster
    // than 8 on every decode shape (2.6% on 32 layers x 8192 blocks, more on
    // shapes with few workgroups, where small work items also shorten the
    // drain at the end of the launch).  A region of 512+ chunks takes 16, so
    // that one load slot never covers less than a whole wave-load.  At r = 32
    // with one wave-load per kv region (block_size 16) the vector-ALU kernel
    // takes 2: 312 vs 315 us for 32 layers x 8192 blocks, the same on 64
    // sequences x 2048 blocks.
    ns = U >= 512 ? 16 : ((U == 64 && lpr == 4 && !mfma) ? 2 : 4);
    gm.WPB = 1;
    if (mfma && U == 256 && PRED_DECODE_MFMA_SPLIT) {
        ns = 2;
        gm.WPB = 2;
    }
    const int chunks = ns * 64 * gm.WPB;
    gm.NBW = (int)(chunks / U);
    gm.SPB = U >= 64 ? (int)(U / 64) : 1;
    const int g = a.Hq / a.Hk;
    gm.n_eff = a.M * g;
    qh = pick_qh(gm.n_eff);
    gm.n_groups = (gm.n_eff + qh - 1) / qh;
    gm.q_chunks = (int)((int64_t)a.M * a.Hq * a.R / 8);
    const int64_t waves_per_seq = (a.n + gm.NBW - 1) / gm.NBW * gm.WPB;
    gm.wgs_per_seq = (waves_per_seq + kWaves - 1) / kWaves;
    return true;
}

bool slab_is_narrow(const ScoreArgs& a) { return a.N * (int64_t)a.Hk * a.B * a.R * 2 < (int64_t(1) << 32); }

// The matrix-core scorer takes kv heads with more than 4 queries (at 4 or fewer
// the dot products cost ~1% of the stream), r a multiple of 32 up to 128, kv
// regions of whole wave-loads, 32-bit slab offsets and the query slab in LDS.
bool decode_mfma_ok(const ScoreArgs& a, const DecodeGeom& gm) {
    return (a.R == 32 || a.R == 64 || a.R == 128) && gm.U >= 64 && slab_is_narrow(a) &&
           gm.q_chunks * 16 <= kQLdsMaxBytes && gm.n_eff >= PRED_DECODE_MFMA_MIN_QUERIES && gm.n_eff <= 16;
}

DecodePlan make_plan(const ScoreArgs& a, int force) {
    DecodePlan pl{};
    pl.kind = SCORE_PATH_GENERIC;
    if (force == SCORE_PATH_GENERIC || !decode_geometry(a, pl.gm, pl.ns, pl.lpr, pl.qh)) return pl;
    pl.kind = SCORE_PATH_DECODE;
    if (force == SCORE_PATH_AUTO && decode_mfma_ok(a, pl.gm)) {
        decode_geometry(a, pl.gm, pl.ns, pl.lpr, pl.qh, true);
        pl.kind = SCORE_PATH_DECODE_MFMA;
    }
    pl.q_lds = pl.gm.q_chunks * 16 <= kQLdsMaxBytes;
    pl.wide = !slab_is_narrow(a);
    pl.uni = pl.gm.U >= 64 && pl.q_lds && !pl.wide;
    return pl;
}

}  // namespace

hipError_t launch_score_decode_or_generic(const ScoreArgs& a, int force, hipStream_t stream) {
    const DecodePlan pl = make_plan(a, force);
    if (pl.kind == SCORE_PATH_GENERIC) {
        const int64_t total = (int64_t)a.n_layers * a.S * a.n;
        if (!grid_fits((total + 255) / 256)) return hipErrorInvalidConfiguration;
        score_generic_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(a);
        return hipGetLastError();
    }
    const DecodeGeom& gm = pl.gm;
    if (!grid_fits(gm.wgs_per_seq * a.S * a.n_layers)) return hipErrorInvalidConfiguration;
    if (pl.kind == SCORE_PATH_DECODE_MFMA) {
        const unsigned grid = (unsigned)(gm.wgs_per_seq * a.S * a.n_layers);
        const int q_bytes = gm.q_chunks * 16;
#define PRED_DMFMA(RV, NSV) score_decode_mfma_kernel<RV, NSV, 1><<<grid, 256, q_bytes, stream>>>(a, gm)
        if (gm.WPB == 2) {
            if (a.R == 64) score_decode_mfma_kernel<64, 2, 2><<<grid, 256, q_bytes, stream>>>(a, gm);
            else if (a.R == 128) score_decode_mfma_kernel<128, 2, 2><<<grid, 256, q_bytes, stream>>>(a, gm);
            else score_decode_mfma_kernel<32, 2, 2><<<grid, 256, q_bytes, stream>>>(a, gm);
        } else if (pl.ns == 16) {
            if (a.R == 32) PRED_DMFMA(32, 16);
            else if (a.R == 64) PRED_DMFMA(64, 16);
            else PRED_DMFMA(128, 16);
        } else {
            if (a.R == 32) PRED_DMFMA(32, 4);
            else if (a.R == 64) PRED_DMFMA(64, 4);
            else PRED_DMFMA(128, 4);
        }
#undef PRED_DMFMA
        return hipGetLastError();
    }
    if (pl.ns == 16) launch_decode_ns<16>(a, pl, stream);
    else if (pl.ns == 4) launch_decode_ns<4>(a, pl, stream);
    else launch_decode_qh<4, 2>(a, pl, stream);   // ns == 2: r = 32 only
    return hipGetLastError();
}

const char* score_decode_path_name(const ScoreArgs& a, int force) {
    switch (make_plan(a, force).kind) {
        case SCORE_PATH_DECODE_MFMA: return "score_decode_mfma_kernel";
        case SCORE_PATH_DECODE: return "score_decode_kernel";
        default: return "score_generic_kernel";
    }
}

std::string score_decode_variant(const ScoreArgs& a, int force) {
    const DecodePlan pl = make_plan(a, force);
    char buf[160];
    if (pl.kind == SCORE_PATH_GENERIC) return "score_generic_kernel";
    if (pl.kind == SCORE_PATH_DECODE_MFMA)
        snprintf(buf, sizeof(buf), "score_decode_mfma_kernel<r=%d,slots=%d,waves_per_block=%d>", a.R, pl.ns,
                 pl.gm.WPB);
    else
        snprintf(buf, sizeof(buf), "score_decode_kernel<lanes_per_row=%d,queries=%d,slots=%d,q_in_lds=%d,offset=%s,"
                 "uniform_slots=%d>", pl.lpr, pl.qh, pl.ns, pl.q_lds ? 1 : 0, (pl.wide || !pl.q_lds) ? "u64" : "u32",
                 pl.uni ? 1 : 0);
    return buf;
}

}  // namespace pred
