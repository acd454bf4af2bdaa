// Eviction ranking: per segment, the stable ascending argsort of float32 scores
// (predictor.rs page, module doc: scores only rank eviction victims; the
// qsa_select.rs page's host top-k breaks ties toward the lower index).
//
// Scores map to order-preserving uint32 keys (-0 == +0, NaN first).  A segment
// of up to 8192 keys is sorted inside one workgroup by an LSD radix sort over
// eight 4-bit digits.  Items sit in blocked order (thread t owns positions
// t*IPT .. t*IPT+IPT-1), so a pass is stable if each thread ranks its own items
// in order and (digit, thread) counts are scanned digit-major:
//   * a thread counts its items per digit in one packed register (sixteen
//     4-bit counters in 64 bits, IPT <= 15) -- no cross-lane work;
//   * the counts, as eight words of two 16-bit halves, are prefix-summed across
//     the wave with DPP row shifts and row broadcasts, across the waves through
//     one small LDS table, and across digits from the grand totals;
//   * items are scattered as (key, index) pairs into one of two LDS buffers and
//     read back in blocked order.
// That is two barriers and about sixteen LDS instructions per thread and pass.
// A pass whose digit is the same for every item (common for the high digits of
// scores in a narrow range) is the identity and is skipped.  The first pass
// starts in index order, so equal keys end in index order.
//
// Longer segments: sorted 8192-key runs of (key << 32 | index) go to the
// workspace and are merged pairwise; each element finds its place in the
// merged run by binary search in the other run (the 64-bit composites are
// distinct, so positions never collide).
#include "common.h"
#include "kernels.h"

namespace pred {

namespace {

constexpr int kMaxLdsItems = 8192;

template <int CTRL, int ROW_MASK>
__device__ inline uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes (packed 16-bit halves add independently).
__device__ inline uint32_t wave_incl_scan(uint32_t v) {
    v += dpp<0x111, 0xF>(v);   // row_shr:1
    v += dpp<0x112, 0xF>(v);   // row_shr:2
    v += dpp<0x114, 0xF>(v);   // row_shr:4
    v += dpp<0x118, 0xF>(v);   // row_shr:8
    v += dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// Inclusive prefix sum over lanes 0..15 (row 0); other rows get their own.
__device__ inline uint32_t row_incl_scan(uint32_t v) {
    v += dpp<0x111, 0xF>(v);
    v += dpp<0x112, 0xF>(v);
    v += dpp<0x114, 0xF>(v);
    v += dpp<0x118, 0xF>(v);
    return v;
}

__device__ inline uint32_t select8(const uint32_t (&o)[8], uint32_t i) {
    const uint32_t a0 = (i & 1u) ? o[1] : o[0];
    const uint32_t a1 = (i & 1u) ? o[3] : o[2];
    const uint32_t a2 = (i & 1u) ? o[5] : o[4];
    const uint32_t a3 = (i & 1u) ? o[7] : o[6];
    const uint32_t b0 = (i & 2u) ? a1 : a0;
    const uint32_t b1 = (i & 2u) ? a3 : a2;
    return (i & 4u) ? b1 : b0;
}

// One workgroup per (segment, chunk) of up to CAP = 64*NW*IPT keys, NW <= 16.
template <int NW, int IPT>
__global__ __launch_bounds__(NW * 64) void rank_lds_kernel(const float* __restrict__ scores, int64_t n,
                                                           int64_t chunk_len, int nchunks,
                                                           int32_t* __restrict__ victims,
                                                           uint64_t* __restrict__ runs) {
    static_assert(IPT <= 15 && IPT % 2 == 0, "packed 4-bit counters hold at most 15 items per thread");
    static_assert(NW <= 16, "the cross-wave scan runs in one DPP row");
    constexpr int T = NW * 64;
    constexpr int CAP = T * IPT;
    __shared__ __align__(16) uint2 kvb[2][CAP];       // (key, index) pairs, double-buffered
    __shared__ __align__(16) uint4 wsum[2][NW][2];    // per-wave digit totals, double-buffered

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t seg = blockIdx.x / nchunks;
    const int64_t off = (int64_t)(blockIdx.x % nchunks) * chunk_len;
    const int len = (int)((n - off) < chunk_len ? (n - off) : chunk_len);
    const float* src = scores + seg * n + off;

    uint32_t key[IPT], idx[IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int pos = t * IPT + j;
        if (pos < len) {
            key[j] = order_key(src[pos]);
            idx[j] = (uint32_t)(off + pos);
        } else {
            key[j] = 0xFFFFFFFFu;  // above every real key: padding sorts last
            idx[j] = 0xFFFFFFFFu;
        }
    }

    int buf = 0;
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 4 * pass;
        const int wb = pass & 1;
        // rank each item among this thread's earlier items with the same digit
        uint64_t packed = 0;
        uint32_t dig[IPT], rnk[IPT];
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const uint32_t d = (key[j] >> shift) & 15u;
            dig[j] = d;
            rnk[j] = (uint32_t)(packed >> (4 * d)) & 15u;
            packed += 1ull << (4 * d);
        }
        // counts as eight words: word i = count(2i) | count(2i+1) << 16
        uint32_t cnt[8], inc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t pair = (uint32_t)(packed >> (8 * i)) & 0xFFu;
            cnt[i] = (pair & 15u) | ((pair >> 4) << 16);
            inc[i] = wave_incl_scan(cnt[i]);
        }
        if (lane == 63) {
            wsum[wb][w][0] = make_uint4(inc[0], inc[1], inc[2], inc[3]);
            wsum[wb][w][1] = make_uint4(inc[4], inc[5], inc[6], inc[7]);
        }
        __syncthreads();
        // lanes 0..NW-1 scan the wave totals; every wave reads its prefix and the grand totals
        uint4 t0 = make_uint4(0u, 0u, 0u, 0u), t1 = t0;
        if (lane < NW) {
            t0 = wsum[wb][lane][0];
            t1 = wsum[wb][lane][1];
        }
        const uint32_t tw[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
        uint32_t base[8];
        uint32_t grand[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t sc = row_incl_scan(tw[i]);
            grand[i] = (uint32_t)__builtin_amdgcn_readlane((int)sc, NW - 1);
            base[i] = w > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)sc, w - 1) : 0u;
        }
        // digit bases: exclusive prefix of the grand totals over digits 0..15
        uint32_t run = 0;
        bool identity = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = grand[i] & 0xFFFFu, hi = grand[i] >> 16;
            identity |= (lo == (uint32_t)CAP) | (hi == (uint32_t)CAP);
            const uint32_t dlo = run;
            const uint32_t dhi = run + lo;
            run = dhi + hi;
            base[i] += dlo | (dhi << 16);
        }
        if (identity) continue;   // uniform: one digit holds every item
        // first destination of (digit, this thread)
        uint32_t first[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) first[i] = base[i] + inc[i] - cnt[i];
        uint2* dstb = kvb[buf];
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const uint32_t word = select8(first, dig[j] >> 1);
            const uint32_t o = (dig[j] & 1u) ? (word >> 16) : (word & 0xFFFFu);
            dstb[o + rnk[j]] = make_uint2(key[j], idx[j]);
        }
        __syncthreads();
        const uint4* mine = reinterpret_cast<const uint4*>(dstb + t * IPT);
#pragma unroll
        for (int c = 0; c < IPT / 2; ++c) {
            const uint4 v = mine[c];
            key[2 * c] = v.x; idx[2 * c] = v.y;
            key[2 * c + 1] = v.z; idx[2 * c + 1] = v.w;
        }
        buf ^= 1;
    }

#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int pos = t * IPT + j;
        if (pos < len) {
            if (runs) runs[seg * n + off + pos] = ((uint64_t)key[j] << 32) | idx[j];
            else victims[seg * n + off + pos] = (int32_t)idx[j];
        }
    }
}

// Merge sorted runs [base, base+run) and [base+run, base+2run) of every segment.
__global__ __launch_bounds__(256) void rank_merge_kernel(const uint64_t* __restrict__ in,
                                                         uint64_t* __restrict__ out,
                                                         int32_t* __restrict__ victims, int64_t n,
                                                         int64_t n_seg, int64_t run) {
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gi >= n * n_seg) return;
    const int64_t seg = gi / n;
    const int64_t pos = gi - seg * n;
    const uint64_t* row = in + seg * n;
    const int64_t base = (pos / (2 * run)) * (2 * run);
    const int64_t a_end = (base + run) < n ? (base + run) : n;
    const int64_t b_end = (base + 2 * run) < n ? (base + 2 * run) : n;
    const uint64_t x = row[pos];
    int64_t lo, hi, mine;
    if (pos < a_end) {  // count elements of B below x
        lo = a_end; hi = b_end; mine = pos - base;
    } else {            // count elements of A below x
        lo = base; hi = a_end; mine = pos - a_end;
    }
    const int64_t first = lo;
    while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) >> 1);
        if (row[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    const int64_t dst = base + mine + (lo - first);
    if (victims) victims[seg * n + dst] = (int32_t)(uint32_t)x;
    else out[seg * n + dst] = x;
}

template <int NW, int IPT>
void launch_lds(const float* scores, int64_t n, int64_t chunk_len, int nchunks, int64_t n_seg,
                int32_t* victims, uint64_t* runs, hipStream_t st) {
    rank_lds_kernel<NW, IPT><<<(unsigned)(n_seg * nchunks), NW * 64, 0, st>>>(scores, n, chunk_len, nchunks,
                                                                              victims, runs);
}

}  // namespace

size_t rank_workspace_bytes(int64_t n, int64_t n_seg) {
    if (n <= kMaxLdsItems || n_seg <= 0) return 0;
    return (size_t)(2 * n * n_seg) * sizeof(uint64_t);
}

hipError_t launch_rank(const float* scores, int64_t n, int64_t n_seg, int32_t* victims, void* ws,
                       hipStream_t st) {
    if (n <= 0 || n_seg <= 0) return hipSuccess;
    if (n <= 512) {
        launch_lds<1, 8>(scores, n, n, 1, n_seg, victims, nullptr, st);
    } else if (n <= 2048) {
        launch_lds<4, 8>(scores, n, n, 1, n_seg, victims, nullptr, st);
    } else if (n <= kMaxLdsItems) {
        launch_lds<16, 8>(scores, n, n, 1, n_seg, victims, nullptr, st);
    } else {
        uint64_t* r0 = static_cast<uint64_t*>(ws);
        uint64_t* r1 = r0 + n * n_seg;
        const int nchunks = (int)((n + kMaxLdsItems - 1) / kMaxLdsItems);
        launch_lds<16, 8>(scores, n, kMaxLdsItems, nchunks, n_seg, nullptr, r0, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const unsigned grid = (unsigned)((n * n_seg + 255) / 256);
        for (int64_t run = kMaxLdsItems; run < n; run *= 2) {
            const bool last = 2 * run >= n;
            rank_merge_kernel<<<grid, 256, 0, st>>>(r0, r1, last ? victims : nullptr, n, n_seg, run);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            uint64_t* tmp = r0; r0 = r1; r1 = tmp;
        }
    }
    return hipGetLastError();
}

}  // namespace pred
