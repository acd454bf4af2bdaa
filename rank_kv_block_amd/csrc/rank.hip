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
// Segments over 2048 keys use every CU instead of one per segment:
//   1. chunks of 1024 keys are sorted as above, one workgroup each, and written
//      as sorted runs of keys and of their indexes;
//   2. runs are merged in groups of up to 8192 keys by counting: one workgroup
//      per run loads its group's keys into LDS, and each element's place in the
//      group is its index in its own run plus, for every other run, how many of
//      that run's keys come before it -- keys below it, and for a run of lower
//      indexes (an earlier chunk) also keys equal to it.  A branch-free binary
//      search over the run (padded to 1024 with keys above every real one)
//      counts them;
//   3. groups (segments over 8192 keys) are merged pairwise as 64-bit
//      (key << 32 | index) composites, which are distinct and order exactly as
//      the stable sort must; each element finds its place in the merged run by
//      binary search in the other run.
#include "common.h"
#include "kernels.h"

namespace pred {

namespace {

constexpr int kMaxLdsItems = 8192;   // keys one workgroup sorts or merges in LDS
#ifndef PRED_RANK_CHUNK
#define PRED_RANK_CHUNK 1024
#endif
constexpr int kChunk = PRED_RANK_CHUNK;   // keys per sorted run of step 1
constexpr int kSingle = 2048;        // up to this many keys a segment is sorted by one workgroup

// step 1 workgroup shape for a chunk (waves x keys per thread = kChunk / 64) and
// step 2 threads per workgroup
#ifndef PRED_RANK_NW
#define PRED_RANK_NW 4
#define PRED_RANK_IPT 4
#endif
#ifndef PRED_RANK_MERGE_TPB
#define PRED_RANK_MERGE_TPB 1024
#endif
static_assert(PRED_RANK_NW * 64 * PRED_RANK_IPT == kChunk, "a step-1 workgroup sorts one chunk");
static_assert(PRED_RANK_MERGE_TPB <= kChunk, "a step-2 thread places at least one key of its run");

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

// o[i] for a per-lane i in 0..7, as a tree of selects on registers.  The
// words are made opaque first: otherwise the compiler turns the selects back
// into an indexed array and places it in LDS (or scratch), costing a round trip
// per item.
__device__ inline uint32_t select8(const uint32_t (&o)[8], uint32_t i) {
    uint32_t r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        r[k] = o[k];
        asm volatile("" : "+v"(r[k]));
    }
    const uint32_t a0 = (i & 1u) ? r[1] : r[0];
    const uint32_t a1 = (i & 1u) ? r[3] : r[2];
    const uint32_t a2 = (i & 1u) ? r[5] : r[4];
    const uint32_t a3 = (i & 1u) ? r[7] : r[6];
    const uint32_t b0 = (i & 2u) ? a1 : a0;
    const uint32_t b1 = (i & 2u) ? a3 : a2;
    return (i & 4u) ? b1 : b0;
}

// One workgroup per (segment, chunk) of up to CAP = 64*NW*IPT keys, NW <= 16.
template <int NW, int IPT>
__global__ __launch_bounds__(NW * 64) void rank_lds_kernel(const float* __restrict__ scores, int64_t n,
                                                           int64_t chunk_len, int nchunks,
                                                           int32_t* __restrict__ victims,
                                                           uint32_t* __restrict__ run_keys,
                                                           uint32_t* __restrict__ run_idx) {
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
            if (run_keys) {
                run_keys[seg * n + off + pos] = key[j];
                run_idx[seg * n + off + pos] = idx[j];
            } else {
                victims[seg * n + off + pos] = (int32_t)idx[j];
            }
        }
    }
}

// Step 2: one workgroup per (segment, run).  Runs of kChunk keys, grouped by
// group_len (a multiple of kChunk, at most kMaxLdsItems); the output is the group
// sorted, as victims when one group spans the segment, else as composites.
template <int TPB>
__global__ __launch_bounds__(TPB) void rank_count_merge_kernel(const uint32_t* __restrict__ run_keys,
                                                               const uint32_t* __restrict__ run_idx, int64_t n,
                                                               int64_t group_len, int nruns,
                                                               int32_t* __restrict__ victims,
                                                               uint64_t* __restrict__ out) {
    constexpr int G = kMaxLdsItems / kChunk;   // runs per group, at most
    constexpr int E = kChunk / TPB;            // elements of the run per thread
    constexpr int L = kMaxLdsItems / TPB;      // group keys loaded per thread
    __shared__ uint32_t gk[kMaxLdsItems];
    const int t = threadIdx.x;
    const int64_t seg = blockIdx.x / nruns;
    const int run = (int)(blockIdx.x % nruns);
    const int64_t run0 = (int64_t)run * kChunk;                       // run start in the segment
    const int64_t g0 = (run0 / group_len) * group_len;                // group start
    const int glen = (int)((n - g0) < group_len ? (n - g0) : group_len);
    const int own = (int)((run0 - g0) / kChunk);
    const uint32_t* src = run_keys + seg * n + g0;
    {
        // the group's keys, padded to G full runs with a key above every real one
        // (order keys never exceed that of +inf); clamped indexes keep every load
        // in bounds and let all of them issue back to back
        uint32_t v[L];
#pragma unroll
        for (int k = 0; k < L; ++k) {
            const int i = t + TPB * k;
            v[k] = src[i < glen ? i : glen - 1];
        }
#pragma unroll
        for (int k = 0; k < L; ++k) {
            const int i = t + TPB * k;
            gk[i] = i < glen ? v[k] : 0xFFFFFFFFu;
        }
    }
    __syncthreads();

    const int rlen = (glen - own * kChunk) < kChunk ? (glen - own * kChunk) : kChunk;
    uint32_t x[E];
    int pos[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = t + TPB * e;
        x[e] = gk[own * kChunk + (i < rlen ? i : 0)];
        pos[e] = i;   // the elements of its own run before it
    }
    // every run is searched (the own run too, its count discarded): no branch, so
    // the G * E searches are independent chains of LDS reads that interleave
#pragma unroll
    for (int r = 0; r < G; ++r) {
        const uint32_t bias = r < own ? 1u : 0u;   // earlier run: equal keys count as well
        const uint32_t* a = gk + r * kChunk;
        uint32_t xr[E];
        int lo[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            xr[e] = x[e] + bias;                   // no overflow: x <= order key of +inf
            lo[e] = 0;
        }
#pragma unroll
        for (int step = kChunk / 2; step >= 1; step >>= 1) {
#pragma unroll
            for (int e = 0; e < E; ++e) lo[e] += a[lo[e] + step - 1] < xr[e] ? step : 0;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            lo[e] += a[lo[e]] < xr[e] ? 1 : 0;     // lo <= kChunk - 1 before this
            pos[e] += r == own ? 0 : lo[e];
        }
    }
    const bool whole = g0 == 0 && glen == n;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = t + TPB * e;
        if (i < rlen && pos[e] < glen) {   // pos < glen always holds; never write outside the group
            const int64_t dst = seg * n + g0 + pos[e];
            const uint32_t id = run_idx[seg * n + run0 + i];
            if (whole) victims[dst] = (int32_t)id;
            else out[dst] = ((uint64_t)x[e] << 32) | id;
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
                int32_t* victims, uint32_t* run_keys, uint32_t* run_idx, hipStream_t st) {
    rank_lds_kernel<NW, IPT><<<(unsigned)(n_seg * nchunks), NW * 64, 0, st>>>(scores, n, chunk_len, nchunks,
                                                                              victims, run_keys, run_idx);
}

}  // namespace

size_t rank_workspace_bytes(int64_t n, int64_t n_seg) {
    if (n <= kSingle || n_seg <= 0) return 0;
    // sorted runs; segments over kMaxLdsItems keys also need a second buffer for the pairwise merges
    return (size_t)((n <= kMaxLdsItems ? 1 : 2) * n * n_seg) * sizeof(uint64_t);
}

hipError_t launch_rank(const float* scores, int64_t n, int64_t n_seg, int32_t* victims, void* ws,
                       hipStream_t st) {
    if (n <= 0 || n_seg <= 0) return hipSuccess;
    if (n <= 512) {
        launch_lds<1, 8>(scores, n, n, 1, n_seg, victims, nullptr, nullptr, st);
        return hipGetLastError();
    }
    if (n <= kSingle) {
        launch_lds<4, 8>(scores, n, n, 1, n_seg, victims, nullptr, nullptr, st);
        return hipGetLastError();
    }
    // workspace: run keys and run indexes (4 + 4 bytes per key), then for long
    // segments one more 8 bytes per key for the pairwise merges
    uint32_t* rk = static_cast<uint32_t*>(ws);
    uint32_t* ri = rk + n * n_seg;
    uint64_t* r0 = static_cast<uint64_t*>(ws);
    uint64_t* r1 = r0 + n * n_seg;
    const int nruns = (int)((n + kChunk - 1) / kChunk);
    launch_lds<PRED_RANK_NW, PRED_RANK_IPT>(scores, n, kChunk, nruns, n_seg, nullptr, rk, ri, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t group = n < kMaxLdsItems ? n : kMaxLdsItems;
    rank_count_merge_kernel<PRED_RANK_MERGE_TPB><<<(unsigned)(n_seg * nruns), PRED_RANK_MERGE_TPB, 0, st>>>(
        rk, ri, n, group, nruns, victims, n <= kMaxLdsItems ? nullptr : r1);
    e = hipGetLastError();
    if (e != hipSuccess || n <= kMaxLdsItems) return e;
    // sorted groups of kMaxLdsItems are in r1; merge them pairwise
    uint64_t* in = r1;
    uint64_t* outb = r0;
    const unsigned grid = (unsigned)((n * n_seg + 255) / 256);
    for (int64_t run = kMaxLdsItems; run < n; run *= 2) {
        const bool last = 2 * run >= n;
        rank_merge_kernel<<<grid, 256, 0, st>>>(in, outb, last ? victims : nullptr, n, n_seg, run);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        uint64_t* tmp = in; in = outb; outb = tmp;
    }
    return hipSuccess;
}

}  // namespace pred
