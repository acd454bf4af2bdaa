// Eviction ranking: per segment, the stable ascending argsort of float32 scores
// (predictor.rs page, module doc: scores only rank eviction victims; the
// qsa_select.rs page's host top-k breaks ties toward the lower index).
//
// Scores map to order-preserving uint32 keys (-0 == +0, NaN first).  A segment
// of up to 16384 keys is sorted inside one workgroup by an LSD radix sort over
// four 8-bit digits, keys and indices kept in LDS between passes.  Each pass is
// stable, and the first starts in index order, so ties end in index order.
// Ranking a digit within a wave uses a match over 8 ballots (lanes with equal
// digits) and a per-wave digit counter in LDS; an exclusive scan of the
// [digit][wave] counters then gives every item its destination.  A pass whose
// digit is the same for every item (common for the top byte of scores in a
// narrow range) is the identity and is skipped.
//
// Longer segments: sorted 16384-key runs of (key << 32 | index) go to the
// workspace and are merged pairwise; each element finds its place in the
// merged run by binary search in the other run (the 64-bit composites are
// distinct, so positions never collide).
#include "common.h"
#include "kernels.h"

namespace pred {

namespace {

constexpr int kMaxLdsItems = 16384;

__device__ inline uint64_t match_digit(uint32_t d) {
    uint64_t m = ~0ull;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

__device__ inline uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ inline uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

// One workgroup per (segment, chunk).  Items of wave w, round j, lane l sit at
// position w*IPT*64 + j*64 + l, so (wave, round, lane) order is index order.
template <int NW, int IPT>
__global__ __launch_bounds__(NW * 64) void rank_lds_kernel(const float* __restrict__ scores, int64_t n,
                                                           int64_t chunk_len, int nchunks,
                                                           int32_t* __restrict__ victims,
                                                           uint64_t* __restrict__ runs) {
    constexpr int T = NW * 64;
    constexpr int CAP = T * IPT;
    __shared__ uint32_t kbuf[CAP];
    __shared__ uint32_t ibuf[CAP];
    __shared__ uint32_t cnt[256 * NW];
    __shared__ uint32_t wsum[NW];
    __shared__ int same_digit[4];  // one flag per pass: no reset races

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t seg = blockIdx.x / nchunks;
    const int64_t off = (int64_t)(blockIdx.x % nchunks) * chunk_len;
    const int len = (int)((n - off) < chunk_len ? (n - off) : chunk_len);
    const float* src = scores + seg * n + off;

    if (threadIdx.x < 4) same_digit[threadIdx.x] = 0;
    uint32_t key[IPT], idx[IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int pos = w * IPT * 64 + j * 64 + lane;
        if (pos < len) {
            key[j] = order_key(src[pos]);
            idx[j] = (uint32_t)(off + pos);
        } else {
            key[j] = 0xFFFFFFFFu;  // above every real key: padding sorts last
            idx[j] = 0xFFFFFFFFu;
        }
    }

    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 8 * pass;
        for (int i = threadIdx.x; i < 256 * NW; i += T) cnt[i] = 0u;
        __syncthreads();
        uint32_t rnk[IPT], dig[IPT];
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const uint32_t d = (key[j] >> shift) & 255u;
            dig[j] = d;
            const uint64_t peers = match_digit(d);
            const uint32_t below = lanes_below(peers);
            const uint32_t old = cnt[d * NW + w];
            rnk[j] = old + below;
            if (below == 0) cnt[d * NW + w] = old + (uint32_t)__popcll(peers);
        }
        __syncthreads();
        // Does one digit hold every item?  Then the pass is the identity.
        for (int d = threadIdx.x; d < 256; d += T) {
            uint32_t tot = 0;
            for (int ww = 0; ww < NW; ++ww) tot += cnt[d * NW + ww];
            if (tot == (uint32_t)CAP) same_digit[pass] = 1;
        }
        // Exclusive scan of cnt in [digit][wave] order; 4 counters per thread.
        const uint32_t c0 = cnt[4 * threadIdx.x], c1 = cnt[4 * threadIdx.x + 1];
        const uint32_t c2 = cnt[4 * threadIdx.x + 2], c3 = cnt[4 * threadIdx.x + 3];
        const uint32_t sum = c0 + c1 + c2 + c3;
        const uint32_t incl = wave_incl_scan(sum, lane);
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        if (same_digit[pass]) continue;  // uniform across the workgroup
        uint32_t base = incl - sum;
        for (int ww = 0; ww < w; ++ww) base += wsum[ww];
        cnt[4 * threadIdx.x] = base;
        cnt[4 * threadIdx.x + 1] = base + c0;
        cnt[4 * threadIdx.x + 2] = base + c0 + c1;
        cnt[4 * threadIdx.x + 3] = base + c0 + c1 + c2;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const uint32_t dst = cnt[dig[j] * NW + w] + rnk[j];
            kbuf[dst] = key[j];
            ibuf[dst] = idx[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const int pos = w * IPT * 64 + j * 64 + lane;
            key[j] = kbuf[pos];
            idx[j] = ibuf[pos];
        }
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int pos = w * IPT * 64 + j * 64 + lane;
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
    } else if (n <= 8192) {
        launch_lds<16, 8>(scores, n, n, 1, n_seg, victims, nullptr, st);
    } else if (n <= kMaxLdsItems) {
        launch_lds<16, 16>(scores, n, n, 1, n_seg, victims, nullptr, st);
    } else {
        uint64_t* r0 = static_cast<uint64_t*>(ws);
        uint64_t* r1 = r0 + n * n_seg;
        const int nchunks = (int)((n + kMaxLdsItems - 1) / kMaxLdsItems);
        launch_lds<16, 16>(scores, n, kMaxLdsItems, nchunks, n_seg, nullptr, r0, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const unsigned grid = (unsigned)((n * n_seg + 255) / 256);
        for (int64_t run = kMaxLdsItems; run < n; run *= 2) {
            const bool last = 2 * run >= n;
            rank_merge_kernel<<<grid, 256, 0, st>>>(r0, r1, last ? victims : nullptr, n, n_seg, run);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            uint64_t* t = r0; r0 = r1; r1 = t;
        }
    }
    return hipGetLastError();
}

}  // namespace pred
