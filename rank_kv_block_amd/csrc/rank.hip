// Eviction ranking: per segment, the stable ascending argsort of float32 scores
// (predictor.rs page, module doc: scores only rank eviction victims; the
// qsa_select.rs page's host top-k breaks ties toward the lower index).
//
// Scores map to order-preserving uint32 keys (-0 == +0, NaN first).  A segment
// of up to 8192 keys is sorted inside one workgroup by an LSD radix sort over
// eight 4-bit digits, keys and indices kept in LDS between passes.  Items sit
// in blocked order (thread t owns positions t*IPT .. t*IPT+IPT-1), so a pass
// is stable if each thread ranks its own items in order and the (digit,
// thread) counts are scanned digit-major: the thread counts its items per
// digit in a packed register (16 four-bit counters in 64 bits, IPT <= 15), with
// no cross-lane work at all; one exclusive scan over the 16 x T counts in LDS
// gives every (digit, thread) its first destination.  A pass whose digit is the
// same for every item (common for the high digits of scores in a narrow range)
// is the identity and is skipped.  The first pass starts in index order, so
// equal keys end in index order.
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

__device__ inline uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

// One workgroup per (segment, chunk) of up to CAP = 64*NW*IPT keys.
template <int NW, int IPT>
__global__ __launch_bounds__(NW * 64) void rank_lds_kernel(const float* __restrict__ scores, int64_t n,
                                                           int64_t chunk_len, int nchunks,
                                                           int32_t* __restrict__ victims,
                                                           uint64_t* __restrict__ runs) {
    static_assert(IPT <= 15 && IPT % 4 == 0, "packed 4-bit counters hold at most 15 items per thread");
    constexpr int T = NW * 64;
    constexpr int CAP = T * IPT;
    __shared__ __align__(16) uint32_t kbuf[CAP];
    __shared__ __align__(16) uint32_t ibuf[CAP];
    __shared__ __align__(16) uint16_t cnt[16 * T];   // [digit][thread]
    __shared__ uint32_t wsum[NW];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
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

    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 4 * pass;
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
#pragma unroll
        for (int d = 0; d < 16; ++d) cnt[d * T + t] = (uint16_t)((packed >> (4 * d)) & 15u);
        __syncthreads();
        // exclusive scan of the 16*T counts in [digit][thread] order, 16 per thread
        uint4* c4 = reinterpret_cast<uint4*>(cnt) + 2 * t;
        const uint4 lo = c4[0], hi = c4[1];
        const uint32_t wd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        uint32_t vals[16];
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            vals[2 * i] = wd[i] & 0xFFFFu;
            vals[2 * i + 1] = wd[i] >> 16;
            sum += vals[2 * i] + vals[2 * i + 1];
        }
        const uint32_t incl = wave_incl_scan(sum, lane);
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        uint32_t run = incl - sum;
        for (int ww = 0; ww < w; ++ww) run += wsum[ww];
        uint32_t out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t a = run;
            run += vals[2 * i];
            const uint32_t b = run;
            run += vals[2 * i + 1];
            out[i] = a | (b << 16);
        }
        c4[0] = make_uint4(out[0], out[1], out[2], out[3]);
        c4[1] = make_uint4(out[4], out[5], out[6], out[7]);
        __syncthreads();
        // a digit holding every item makes the pass the identity
        uint32_t first = 0, next = CAP;
        if (lane < 16) {
            first = cnt[lane * T];
            next = lane < 15 ? cnt[(lane + 1) * T] : (uint32_t)CAP;
        }
        const bool identity = __ballot(lane < 16 && first == 0 && next == (uint32_t)CAP) != 0;
        if (!identity) {   // uniform across the workgroup
#pragma unroll
            for (int j = 0; j < IPT; ++j) {
                const uint32_t dst = cnt[dig[j] * T + t] + rnk[j];
                kbuf[dst] = key[j];
                ibuf[dst] = idx[j];
            }
            __syncthreads();
            const uint4* k4 = reinterpret_cast<const uint4*>(kbuf) + t * (IPT / 4);
            const uint4* i4 = reinterpret_cast<const uint4*>(ibuf) + t * (IPT / 4);
#pragma unroll
            for (int c = 0; c < IPT / 4; ++c) {
                const uint4 kk = k4[c], ii = i4[c];
                key[4 * c] = kk.x; key[4 * c + 1] = kk.y; key[4 * c + 2] = kk.z; key[4 * c + 3] = kk.w;
                idx[4 * c] = ii.x; idx[4 * c + 1] = ii.y; idx[4 * c + 2] = ii.z; idx[4 * c + 3] = ii.w;
            }
        }
        __syncthreads();
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
