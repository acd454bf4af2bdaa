// Eviction ranking: per segment, the stable ascending argsort of float32 scores
// (predictor.rs page, module doc: scores only rank eviction victims; the
// qsa_select.rs page's host top-k breaks ties toward the lower index).
//
// Scores map to order-preserving uint32 keys (-0 == +0, NaN first) and are
// sorted as 64-bit (key << 32 | index) composites.  The composites are all
// distinct and order exactly as the stable sort must, so any correct sort of
// them -- stable or not -- gives the stable order.
//
// A segment of up to 2048 keys is sorted inside one workgroup by a bitonic
// network (rank_bitonic_kernel: registers, in-wave lane exchanges and, for the
// largest strides only, LDS; above 1024 keys rank_bitonic2_kernel, the same
// network with two keys per thread and twice the waves).  Longer segments use every CU instead of one per
// segment:
//   1. chunks of 1024 keys are sorted by the same network with two keys per
//      thread (rank_bitonic2_kernel, 512 threads), one workgroup each, and
//      written as sorted runs of keys and of their indexes;
//   2. runs are merged in groups of up to 8192 keys by counting: one workgroup
//      per run loads its group's keys into LDS, and each element's place in the
//      group is its index in its own run plus, for every other run, how many of
//      that run's keys come before it -- keys below it, and for a run of lower
//      indexes (an earlier chunk) also keys equal to it.  A branch-free binary
//      search over the run (padded to 1024 with keys above every real one)
//      counts them;
//   3. rows over 8192 keys repeat step 2 on the sorted groups: up to four runs
//      of 8192 (128 KiB of keys in LDS); rows over 32768 then merge runs
//      pairwise, each element finding its place by binary search in the other
//      run.
//
// The k lowest of each row only, for k <= 256 and many rows of 513..2048
// keys (a prefill chunk's keep sets), take a radix select instead of a sort
// (select_radix_kernel): the row is never sorted, only its k lowest.
//
// The same machinery gives a per-row keep set (qsa_select.rs page, host top-k
// of a prefill chunk): descending order keys (larger score first, ties still to
// the lower index) and, per row, only the blocks complete at that row's
// position.  A row's other entries enter as padding keys above every real key;
// the merges place padding like equal keys and carry index -1 for it, so the
// slots of a row with fewer eligible blocks than asked for come out as -1.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace pred {

// Device-resident scratch of the no-allocation ranking entry point
// (pred_rank_victims_noalloc): the sorted runs of a call live here instead of
// in a caller workspace.  Each GPU holds its own copy from module load to
// process end.  In host code `scratch` names only a host-side stand-in, so the
// kernels get the device address found by hipGetSymbolAddress at set-up.
static __device__ __align__(256) uint64_t scratch[kNoAllocScratchBytes / sizeof(uint64_t)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices] = {};
}  // namespace

hipError_t rank_scratch_prepare(int device) {
    if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[device]) return hipSuccess;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_dev[device] = ptr;
    return hipSuccess;
}

void* rank_scratch(int device) {
    if (device < 0 || device >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_dev[device];
}

namespace {

constexpr int kMaxLdsItems = 8192;   // keys of one step-2 group, merged in LDS
constexpr int kChunk = 1024;         // keys per sorted run of step 1 (measured best of 512 / 1024 / 2048)
constexpr int kSingle = 2048;        // up to this many keys a segment is sorted by one workgroup
constexpr int kMergeTPB = 1024;      // step-2 threads per workgroup (one key of its run each)
constexpr uint32_t kPadKey = 0xFFFFFFFFu;   // padding: above every sort key
constexpr int kMaxGroup2 = 32768;    // keys of one second-level group (128 KiB of LDS)
// chunk sort of the chunked path with two keys per thread (1) or four (0):
// two waves per SIMD instead of one; 32 rows of 8192 keys ranked in 17.5-17.9
// vs 19.2-19.3 us, one row of 32768 in 21.6-22.0 vs 22.4-22.9 us (alternating
// runs on one MI355X)
#ifndef PRED_RANK_CHUNK_2KEYS
#define PRED_RANK_CHUNK_2KEYS 1
#endif
// one-workgroup sort of rows of 1025..2048 keys with two keys per thread (1)
// or four (0): 64 rows of 2048 keys 11.8-12.1 vs 13.2-13.5 us, one row 10.9 vs
// 11.7 us (alternating runs on one MI355X)
#ifndef PRED_RANK_SINGLE_2KEYS
#define PRED_RANK_SINGLE_2KEYS 1
#endif
#ifndef PRED_SELECT_MAX_K
#define PRED_SELECT_MAX_K 256
#endif
constexpr int kSelectMaxK = PRED_SELECT_MAX_K;   // radix select for k up to this (the selected keys fill one wave)
constexpr int kSelectMinN = 512;     // rows up to this length keep the bitonic sort
// Radix select only pays when the GPU is full of rows (sorting is then
// throughput-bound): 2048 rows of 2048, top 64: 30.8 vs 40.6 us; with 64 rows
// the per-row latency of its four histogram passes loses (14.6 vs 11.5 us).
constexpr int64_t kSelectMinRows = 512;

// Sorting network for one chunk of CH keys (power of two, 256..2048), 4 per
// thread in blocked order (thread t holds positions 4t .. 4t+3).  Values are
// (key << 32 | index) composites, all distinct, so the unstable network yields
// exactly the stable order.  Bitonic stage (k, j) pairs positions p and p ^ j
// inside runs of k; the lower position keeps the min when its run ascends
// ((p & k) == 0).  j = 1, 2 pair registers of one thread; j = 4 .. 128 pair
// lanes of one wave (lane distance j / 4: DPP for 1 and 2, swizzles for 4 to
// 16, a permute for 32); j >= 256 pairs waves, through LDS (two buffers, so one
// barrier per such stage).
template <int M>
__device__ inline uint32_t lane_xor_u32(uint32_t v) {
    if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);
    else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);
    else if constexpr (M <= 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (M << 10) | 0x1F);   // xor within 32 lanes
    else return (uint32_t)__shfl_xor((int)v, M);
}

template <int M>
__device__ inline uint64_t lane_xor_u64(uint64_t v) {
    const uint32_t lo = lane_xor_u32<M>((uint32_t)v);
    const uint32_t hi = lane_xor_u32<M>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int CH, int K, int J>
__device__ inline void bitonic_stage(uint64_t (&x)[4], uint64_t (*xb)[CH], int& lb, int t) {
    const int lane = t & 63;
    const int w = t >> 6;
    if constexpr (J <= 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if ((e & J) == 0) {
                const bool asc = ((4 * t + e) & K) == 0;
                const uint64_t a = x[e], b = x[e | J];
                const uint64_t lo = a < b ? a : b, hi = a < b ? b : a;
                x[e] = asc ? lo : hi;
                x[e | J] = asc ? hi : lo;
            }
        }
    } else {
        const bool asc = ((4 * t) & K) == 0;   // K >= 8: the same for the thread's four positions
        uint64_t y[4];
        bool lower;
        if constexpr (J < 256) {
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = lane_xor_u64<J / 4>(x[e]);
            lower = (lane & (J / 4)) == 0;
        } else {
            uint64_t* buf = xb[lb];
            *reinterpret_cast<uint4*>(&buf[4 * t]) = make_uint4((uint32_t)x[0], (uint32_t)(x[0] >> 32),
                                                                (uint32_t)x[1], (uint32_t)(x[1] >> 32));
            *reinterpret_cast<uint4*>(&buf[4 * t + 2]) = make_uint4((uint32_t)x[2], (uint32_t)(x[2] >> 32),
                                                                    (uint32_t)x[3], (uint32_t)(x[3] >> 32));
            __syncthreads();
            const int pt = t ^ (J / 4);   // partner thread, the same four offsets
            const uint4 u0 = *reinterpret_cast<const uint4*>(&buf[4 * pt]);
            const uint4 u1 = *reinterpret_cast<const uint4*>(&buf[4 * pt + 2]);
            y[0] = ((uint64_t)u0.y << 32) | u0.x;
            y[1] = ((uint64_t)u0.w << 32) | u0.z;
            y[2] = ((uint64_t)u1.y << 32) | u1.x;
            y[3] = ((uint64_t)u1.w << 32) | u1.z;
            lb ^= 1;
            lower = (w & (J / 256)) == 0;
        }
        const bool keep_min = lower == asc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint64_t a = x[e], b = y[e];
            x[e] = (keep_min == (a < b)) ? a : b;
        }
    }
}

template <int CH, int K, int J>
__device__ inline void bitonic_js(uint64_t (&x)[4], uint64_t (*xb)[CH], int& lb, int t) {
    bitonic_stage<CH, K, J>(x, xb, lb, t);
    if constexpr (J > 1) bitonic_js<CH, K, J / 2>(x, xb, lb, t);
}

template <int CH, int K>
__device__ inline void bitonic_ks(uint64_t (&x)[4], uint64_t (*xb)[CH], int& lb, int t) {
    bitonic_js<CH, K, K / 2>(x, xb, lb, t);
    if constexpr (K < CH) bitonic_ks<CH, K * 2>(x, xb, lb, t);
}

// The same network with two keys per thread (thread t holds positions 2t and
// 2t + 1), so a chunk of CH keys takes CH / 2 threads: twice the waves of the
// four-key version for the same chunk, for chunks whose workgroups would
// otherwise leave one wave per SIMD.  J = 1 pairs the two registers; J = 2 ..
// 64 pair lanes (distance J / 2); J >= 128 pairs waves through LDS.
template <int CH, int K, int J>
__device__ inline void bitonic2_stage(uint64_t (&x)[2], uint64_t (*xb)[CH], int& lb, int t) {
    const int lane = t & 63;
    const int w = t >> 6;
    const bool asc = ((2 * t) & K) == 0;   // K >= 2: the same for the thread's two positions
    if constexpr (J == 1) {
        const uint64_t a = x[0], b = x[1];
        const uint64_t lo = a < b ? a : b, hi = a < b ? b : a;
        x[0] = asc ? lo : hi;
        x[1] = asc ? hi : lo;
    } else {
        uint64_t y[2];
        bool lower;
        if constexpr (J < 128) {
#pragma unroll
            for (int e = 0; e < 2; ++e) y[e] = lane_xor_u64<J / 2>(x[e]);
            lower = (lane & (J / 2)) == 0;
        } else {
            uint64_t* buf = xb[lb];
            *reinterpret_cast<uint4*>(&buf[2 * t]) = make_uint4((uint32_t)x[0], (uint32_t)(x[0] >> 32),
                                                                (uint32_t)x[1], (uint32_t)(x[1] >> 32));
            __syncthreads();
            const int pt = t ^ (J / 2);   // partner thread, the same two offsets
            const uint4 u = *reinterpret_cast<const uint4*>(&buf[2 * pt]);
            y[0] = ((uint64_t)u.y << 32) | u.x;
            y[1] = ((uint64_t)u.w << 32) | u.z;
            lb ^= 1;
            lower = (w & (J / 128)) == 0;
        }
        const bool keep_min = lower == asc;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint64_t a = x[e], b = y[e];
            x[e] = (keep_min == (a < b)) ? a : b;
        }
    }
}

template <int CH, int K, int J>
__device__ inline void bitonic2_js(uint64_t (&x)[2], uint64_t (*xb)[CH], int& lb, int t) {
    bitonic2_stage<CH, K, J>(x, xb, lb, t);
    if constexpr (J > 1) bitonic2_js<CH, K, J / 2>(x, xb, lb, t);
}

template <int CH, int K>
__device__ inline void bitonic2_ks(uint64_t (&x)[2], uint64_t (*xb)[CH], int& lb, int t) {
    bitonic2_js<CH, K, K / 2>(x, xb, lb, t);
    if constexpr (K < CH) bitonic2_ks<CH, K * 2>(x, xb, lb, t);
}

// rank_bitonic_kernel with two keys per thread: sorted runs of CH keys (step
// 1 of the chunked path), or with run_keys null a whole segment of up to CH
// keys straight to victims (row stride vstride); only the first klim places
// are written.
template <int CH>
__global__ __launch_bounds__(CH / 2) void rank_bitonic2_kernel(const float* __restrict__ scores, int64_t n,
                                                               int nchunks, int64_t klim, int64_t vstride,
                                                               RowOrder ro, int32_t* __restrict__ victims,
                                                               uint32_t* __restrict__ run_keys,
                                                               uint32_t* __restrict__ run_idx) {
    __shared__ __align__(16) uint64_t xb[2][CH];
    const int t = threadIdx.x;
    const int64_t seg = blockIdx.x / nchunks;
    const int64_t off = (int64_t)(blockIdx.x % nchunks) * CH;
    const int len = (int)((n - off) < CH ? (n - off) : CH);
    const float* src = scores + seg * n + off;
    const int64_t valid = ro.row_len(seg, n);
    uint64_t x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int pos = 2 * t + e;
        x[e] = (pos < len && off + pos < valid) ? (((uint64_t)ro.key(src[pos]) << 32) | (uint32_t)(off + pos))
                                                : ~0ull;
    }
    int lb = 0;
    bitonic2_ks<CH, 2>(x, xb, lb, t);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int pos = 2 * t + e;
        if (pos < len && pos < klim) {
            if (run_keys) {
                const int64_t o = seg * n + off + pos;
                run_keys[o] = (uint32_t)(x[e] >> 32);
                run_idx[o] = (uint32_t)x[e];
            } else {
                victims[seg * vstride + off + pos] = (int32_t)(uint32_t)x[e];
            }
        }
    }
}

// One workgroup per (segment, chunk) of up to CH keys.  Only the first klim
// places of each sorted chunk are written (klim = n for a full ranking); victims
// rows are vstride apart.
template <int CH>
__global__ __launch_bounds__(CH / 4) void rank_bitonic_kernel(const float* __restrict__ scores, int64_t n,
                                                              int64_t chunk_len, int nchunks, int64_t klim,
                                                              int64_t vstride, RowOrder ro,
                                                              int32_t* __restrict__ victims,
                                                              uint32_t* __restrict__ run_keys,
                                                              uint32_t* __restrict__ run_idx) {
    static_assert(CH >= 256 && CH <= 2048 && (CH & (CH - 1)) == 0, "one to eight waves of four keys per lane");
    __shared__ __align__(16) uint64_t xb[2][CH];
    const int t = threadIdx.x;
    const int64_t seg = blockIdx.x / nchunks;
    const int64_t off = (int64_t)(blockIdx.x % nchunks) * chunk_len;
    const int len = (int)((n - off) < chunk_len ? (n - off) : chunk_len);
    const float* src = scores + seg * n + off;
    const int64_t valid = ro.row_len(seg, n);   // entries of this row that take part
    uint64_t x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int pos = 4 * t + e;
        // padding sorts after every real key (sort keys stay below kPadKey)
        x[e] = (pos < len && off + pos < valid) ? (((uint64_t)ro.key(src[pos]) << 32) | (uint32_t)(off + pos))
                                                : ~0ull;
    }
    int lb = 0;
    bitonic_ks<CH, 2>(x, xb, lb, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int pos = 4 * t + e;
        if (pos < len && pos < klim) {
            if (run_keys) {
                const int64_t o = seg * n + off + pos;
                run_keys[o] = (uint32_t)(x[e] >> 32);
                run_idx[o] = (uint32_t)x[e];
            } else {
                victims[seg * vstride + off + pos] = (int32_t)(uint32_t)x[e];
            }
        }
    }
}

// The k lowest places of a row of up to 256 * KPT keys, for k <= 256, without
// sorting the row (the k lowest of each row of a keep-set or victim
// selection).  One workgroup per row; thread t holds positions t*KPT ..
// t*KPT + KPT - 1.  Four 8-bit radix-select passes (most significant digit
// first, LDS histograms of the keys that still match the digits found) find
// T, the k-th smallest order key, and how many of the keys equal to T the k
// lowest places hold (want).  Every key below T is taken, and of the keys equal
// to T the want ones with the lowest positions (a block prefix count over
// positions), which is exactly the first k places of the (key, position)
// order.  The k taken (key << 32 | position) composites are then sorted by
// one wave with the bitonic network above.  Padding keys (a row's entries past
// its eligible count) are keys like any other and come out as -1.
template <int KPT>
__global__ __launch_bounds__(256) void select_radix_kernel(const float* __restrict__ scores, int64_t n, int64_t k,
                                                           int64_t vstride, RowOrder ro,
                                                           int32_t* __restrict__ out) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t found[2];              // digit, rank wanted inside it
    __shared__ uint32_t wave_tot[4];
    __shared__ uint32_t n_sel;
    __shared__ __align__(16) uint64_t sel[2][256];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int64_t seg = blockIdx.x;
    const float* src = scores + seg * n;
    const int64_t valid = ro.row_len(seg, n);
    uint32_t key[KPT];
    uint32_t present = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int64_t p = (int64_t)t * KPT + j;
        key[j] = p < valid ? ro.key(src[p]) : kPadKey;
        present |= (p < n ? 1u : 0u) << j;
    }
    if (t == 0) n_sel = 0;
    uint32_t prefix = 0;
    uint32_t want = (uint32_t)k;              // rank (1-based) of T among the keys matching prefix
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int sh = 24 - 8 * pass;
        hist[t] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool match = ((present >> j) & 1u) && (pass == 0 || (key[j] >> (sh + 8)) == (prefix >> (sh + 8)));
            if (match) atomicAdd(&hist[(key[j] >> sh) & 255u], 1u);
        }
        __syncthreads();
        if (w == 0) {
            // lane l owns digits 4l .. 4l+3; exclusive scan of the lane sums
            const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
            const uint32_t mine = h0 + h1 + h2 + h3;
            uint32_t incl = mine;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t o = (uint32_t)__shfl_up((int)incl, d);
                if (lane >= d) incl += o;
            }
            uint32_t before = incl - mine;
            const uint32_t hs[4] = {h0, h1, h2, h3};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (before < want && want <= before + hs[e]) {
                    found[0] = 4u * lane + e;
                    found[1] = want - before;
                }
                before += hs[e];
            }
        }
        __syncthreads();
        prefix |= found[0] << sh;
        want = found[1];
    }
    // prefix is T; take every key below it and the first `want` keys equal to it
    uint32_t eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) eq += (((present >> j) & 1u) && key[j] == prefix) ? 1u : 0u;
    uint32_t incl = eq;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    uint32_t eq_before = incl - eq;
    for (int v = 0; v < w; ++v) eq_before += wave_tot[v];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (!((present >> j) & 1u)) continue;
        bool take = key[j] < prefix;
        if (key[j] == prefix) {
            take = eq_before < want;
            ++eq_before;
        }
        if (take) {
            const uint32_t slot = atomicAdd(&n_sel, 1u);
            sel[0][slot] = ((uint64_t)key[j] << 32) | (uint32_t)(t * KPT + j);
        }
    }
    __syncthreads();
    if (w == 0) {
        uint64_t x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int pos = 4 * lane + e;
            x[e] = pos < (int)k ? sel[0][pos] : ~0ull;
        }
        int lb = 0;
        bitonic_ks<256, 2>(x, sel, lb, lane);   // strides below 256: registers and lane exchanges only
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int pos = 4 * lane + e;
            if (pos < (int)k) out[seg * vstride + pos] = (uint32_t)(x[e] >> 32) == kPadKey ? -1 : (int32_t)(uint32_t)x[e];
        }
    }
}

// Steps 2 and 3: merges by counting.  Sorted runs of RL keys (with their
// indexes) are merged G at a time; a group's keys sit in LDS (G*RL*4 bytes: 32
// KiB for 8 runs of 1024, 128 KiB for 4 runs of 8192).  One workgroup places TPB
// consecutive elements of one run; the output is the group sorted, as victims
// when one group spans the segment, else as keys and indexes again.
//
// With klim < n (the k lowest only) a run's places from klim on are neither
// placed nor counted: they are read as keys above every real one.  An element
// among the k lowest has fewer than klim keys below it in any run, so its count
// is unchanged; any other element still counts klim or more.  So the first
// klim places come out exactly as in the full merge, and only they are written.
template <int RL, int G, int TPB>
__global__ __launch_bounds__(TPB) void rank_count_merge_kernel(const uint32_t* __restrict__ in_keys,
                                                               const uint32_t* __restrict__ in_idx, int64_t n,
                                                               int nruns, int64_t klim, int64_t vstride,
                                                               int32_t* __restrict__ victims,
                                                               uint32_t* __restrict__ out_keys,
                                                               uint32_t* __restrict__ out_idx) {
    constexpr int GL = G * RL;       // keys of a full group
    constexpr int PPR = RL / TPB;    // workgroups per run
    constexpr int L = GL / TPB;      // group keys each thread loads
    static_assert(RL % TPB == 0 && GL % TPB == 0, "whole workgroups per run and per group");
    extern __shared__ uint32_t gk[];
    const int t = threadIdx.x;
    const int64_t per_seg = (int64_t)nruns * PPR;
    const int64_t seg = blockIdx.x / per_seg;
    const int64_t rem = blockIdx.x - seg * per_seg;
    const int run = (int)(rem / PPR);
    const int piece = (int)(rem - (int64_t)run * PPR);
    const int64_t run0 = (int64_t)run * RL;                 // run start in the segment
    const int64_t g0 = (run0 / GL) * GL;                    // group start
    const int glen = (int)((n - g0) < GL ? (n - g0) : GL);
    const int own = (int)((run0 - g0) / RL);
    const int kl = klim < RL ? (int)klim : RL;              // places of a run that can matter
    const int rlen0 = (glen - own * RL) < RL ? (glen - own * RL) : RL;
    const int rlen = rlen0 < kl ? rlen0 : kl;               // elements of its own run placed here
    if (piece * TPB >= rlen) return;                         // whole workgroup: nothing to place
    const uint32_t* src = in_keys + seg * n + g0;
    const int i = piece * TPB + t;                           // this thread's element of its run
    // its index, requested now so the load overlaps the group load and the searches
    const uint32_t id = in_idx[seg * n + run0 + (i < rlen ? i : 0)];
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
            gk[i] = (i < glen && (i & (RL - 1)) < kl) ? v[k] : 0xFFFFFFFFu;
        }
    }
    __syncthreads();

    const uint32_t x = gk[own * RL + (i < rlen ? i : 0)];
    const bool pad = x == kPadKey;                           // a row's entries past its eligible count
    int pos = i;                                             // the elements of its own run before it
    // every run is searched (the own run too, its count discarded): no branch, so
    // the G searches are independent chains of LDS reads that interleave
#pragma unroll
    for (int r = 0; r < G; ++r) {
        const uint32_t xr = x + (r < own ? 1u : 0u);         // earlier run: equal keys count as well
        const uint32_t* a = gk + r * RL;                     // (x + 1 wraps only for padding, not used then)
        int lo = 0;
#pragma unroll
        for (int step = RL / 2; step >= 1; step >>= 1) lo += a[lo + step - 1] < xr ? step : 0;
        lo += a[lo] < xr ? 1 : 0;                            // lo <= RL - 1 before this
        // padding is placed as a key equal to the other padding: all of an
        // earlier run (a whole run of RL) comes before it, and a later run's
        // real keys; it carries index -1 to the output
        pos += r == own ? 0 : ((pad && r < own) ? RL : lo);
    }
    if (i < rlen && pos < glen && pos < klim) {             // pos < glen always holds
        if (g0 == 0 && glen == n) {
            victims[seg * vstride + pos] = (int32_t)id;
        } else {
            out_keys[seg * n + g0 + pos] = x;
            out_idx[seg * n + g0 + pos] = id;
        }
    }
}

// Rows over 32768 keys: merge sorted runs [base, base+run) and [base+run,
// base+2run) of every segment.  An element counts the other run's keys before
// it by binary search: keys below it, and for the first run (lower indexes)
// also keys equal to it (padding of the second run counts the whole first run).  With klim < n only each run's first klim places take
// part (the same argument as for the counting merge).
__global__ __launch_bounds__(256) void rank_merge_kernel(const uint32_t* __restrict__ in_keys,
                                                         const uint32_t* __restrict__ in_idx,
                                                         uint32_t* __restrict__ out_keys,
                                                         uint32_t* __restrict__ out_idx,
                                                         int32_t* __restrict__ victims, int64_t n,
                                                         int64_t n_seg, int64_t run, int64_t klim,
                                                         int64_t vstride) {
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gi >= n * n_seg) return;
    const int64_t seg = gi / n;
    const int64_t pos = gi - seg * n;
    const uint32_t* row = in_keys + seg * n;
    const int64_t base = (pos / (2 * run)) * (2 * run);
    const int64_t a_end = (base + run) < n ? (base + run) : n;
    const int64_t b_end = (base + 2 * run) < n ? (base + 2 * run) : n;
    const uint32_t x = row[pos];
    int64_t lo, hi, mine;
    uint32_t xr;
    if (pos < a_end) {  // keys of the second run below x
        lo = a_end; hi = b_end; mine = pos - base; xr = x;
    } else {            // keys of the first run at most x
        lo = base; hi = a_end; mine = pos - a_end; xr = x + 1u;
    }
    if (mine >= klim) return;
    if (hi - lo > klim) hi = lo + klim;
    const int64_t first = lo;
    if (x == kPadKey && pos >= a_end) lo = hi;   // padding of the second run: all of the first comes before
    while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) >> 1);
        if (row[mid] < xr) lo = mid + 1;
        else hi = mid;
    }
    const int64_t place = mine + (lo - first);               // in the merged run starting at base
    if (place >= klim) return;
    const uint32_t id = in_idx[seg * n + pos];
    if (victims) {
        victims[seg * vstride + base + place] = (int32_t)id;   // base is 0 in the last merge
    } else {
        out_keys[seg * n + base + place] = x;
        out_idx[seg * n + base + place] = id;
    }
}

template <int RL, int G, int TPB>
hipError_t launch_count_merge(const uint32_t* ik, const uint32_t* ii, int64_t n, int64_t n_seg, int64_t klim,
                              int64_t vstride, int32_t* victims, uint32_t* ok, uint32_t* oi, hipStream_t st) {
    const int nruns = (int)((n + RL - 1) / RL);
    const size_t lds = (size_t)G * RL * sizeof(uint32_t);   // above 64 KiB: allowed by rank_prepare
    rank_count_merge_kernel<RL, G, TPB><<<(unsigned)(n_seg * nruns * (RL / TPB)), TPB, lds, st>>>(
        ik, ii, n, nruns, klim, vstride, victims, ok, oi);
    return hipGetLastError();
}

}  // namespace

hipError_t rank_prepare() {
    // the second merge level keeps 128 KiB of keys in LDS; set once per device
    // at handle creation, so a ranking call makes no attribute call (it can be
    // captured into a graph)
    return hipFuncSetAttribute(
        reinterpret_cast<const void*>(&rank_count_merge_kernel<kMaxLdsItems, kMaxGroup2 / kMaxLdsItems, kMergeTPB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kMaxGroup2 * sizeof(uint32_t)));
}

size_t rank_workspace_bytes(int64_t n, int64_t n_seg) {
    if (n <= kSingle || n_seg <= 0) return 0;
    // sorted runs as keys + indexes; longer rows ping-pong between two such buffers
    return (size_t)((n <= kMaxLdsItems ? 1 : 2) * n * n_seg) * sizeof(uint64_t);
}

hipError_t launch_rank(const float* scores, int64_t n, int64_t n_seg, int64_t k, RowOrder ro, int32_t* victims,
                       void* ws, hipStream_t st) {
    if (n <= 0 || n_seg <= 0) return hipSuccess;
    // largest grids of the path this row length takes: the step-1 sort, the
    // second merge level (8 workgroups per run of 8192) and the pairwise merges
    const int64_t chunks = n <= kSingle ? 1 : (n + kChunk - 1) / kChunk;
    if (!grid_fits(n_seg * chunks) || !grid_fits(n_seg * ((n + kMaxLdsItems - 1) / kMaxLdsItems) * 8) ||
        !grid_fits((n * n_seg + 255) / 256))
        return hipErrorInvalidConfiguration;
    if (k <= kSelectMaxK && n > kSelectMinN && n <= kSingle && k < n && n_seg >= kSelectMinRows) {
        // the k lowest only, many rows: select, then sort k keys
        if (n <= 1024) select_radix_kernel<4><<<(unsigned)n_seg, 256, 0, st>>>(scores, n, k, k, ro, victims);
        else select_radix_kernel<8><<<(unsigned)n_seg, 256, 0, st>>>(scores, n, k, k, ro, victims);
        return hipGetLastError();
    }
    if (n <= 256) {
        rank_bitonic_kernel<256><<<(unsigned)n_seg, 64, 0, st>>>(scores, n, n, 1, k, k, ro, victims, nullptr, nullptr);
        return hipGetLastError();
    }
    if (n <= 1024) {
        rank_bitonic_kernel<1024><<<(unsigned)n_seg, 256, 0, st>>>(scores, n, n, 1, k, k, ro, victims, nullptr, nullptr);
        return hipGetLastError();
    }
    if (n <= kSingle) {
#if PRED_RANK_SINGLE_2KEYS
        rank_bitonic2_kernel<2048><<<(unsigned)n_seg, 1024, 0, st>>>(scores, n, 1, k, k, ro, victims, nullptr, nullptr);
#else
        rank_bitonic_kernel<2048><<<(unsigned)n_seg, 512, 0, st>>>(scores, n, n, 1, k, k, ro, victims, nullptr, nullptr);
#endif
        return hipGetLastError();
    }
    // workspace: buffer A = run keys then run indexes (4 + 4 bytes per key), and
    // for rows over 8192 keys buffer B of the same shape
    const int64_t total = n * n_seg;
    uint32_t* ak = static_cast<uint32_t*>(ws);
    uint32_t* ai = ak + total;
    uint32_t* bk = ai + total;
    uint32_t* bi = bk + total;
    const int nruns = (int)((n + kChunk - 1) / kChunk);
#if PRED_RANK_CHUNK_2KEYS
    rank_bitonic2_kernel<kChunk><<<(unsigned)(n_seg * nruns), kChunk / 2, 0, st>>>(scores, n, nruns, k, k, ro,
                                                                                 nullptr, ak, ai);
#else
    rank_bitonic_kernel<kChunk><<<(unsigned)(n_seg * nruns), kChunk / 4, 0, st>>>(scores, n, kChunk, nruns, k, k,
                                                                                ro, nullptr, ak, ai);
#endif
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // runs of 1024 -> groups of 8192 (the whole row when it is no longer)
    e = launch_count_merge<kChunk, kMaxLdsItems / kChunk, kMergeTPB>(ak, ai, n, n_seg, k, k, victims, bk, bi, st);
    if (e != hipSuccess || n <= kMaxLdsItems) return e;
    // runs of 8192 -> groups of 32768 (128 KiB of keys in LDS)
    e = launch_count_merge<kMaxLdsItems, kMaxGroup2 / kMaxLdsItems, kMergeTPB>(bk, bi, n, n_seg, k, k, victims, ak,
                                                                               ai, st);
    if (e != hipSuccess || n <= kMaxGroup2) return e;
    // longer rows: pairwise merges of runs of 32768, 65536, ...
    uint32_t *ik = ak, *ii = ai, *ok = bk, *oi = bi;
    const unsigned grid = (unsigned)((total + 255) / 256);
    for (int64_t run = kMaxGroup2; run < n; run *= 2) {
        const bool last = 2 * run >= n;
        rank_merge_kernel<<<grid, 256, 0, st>>>(ik, ii, ok, oi, last ? victims : nullptr, n, n_seg, run, k, k);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        uint32_t* tk = ik; ik = ok; ok = tk;
        uint32_t* ti = ii; ii = oi; oi = ti;
    }
    return hipSuccess;
}

}  // namespace pred
