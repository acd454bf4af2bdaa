// C ABI of the block predictor: argument checks, ownership of P and A_g, and
// dispatch to the HIP kernels.  The call shapes follow the predictor.rs page
// (Predictor::new_on_stream, project_q, project_kv_block, score_blocks,
// a_g_dev_ptr, dims, read_k_lr_slot), batched over blocks, layers, sequences
// and query rows, plus the victim ranking the page's module doc describes.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "pred.h"

namespace pred {
void build_projection(int head_dim, int r, uint64_t seed, uint16_t* out);
hipError_t launch_score_prefill(const ScoreArgs& a, hipStream_t stream);
bool prefill_supported(const ScoreArgs& a);
}  // namespace pred

struct pred_handle {
    pred_dims d;
    int device;
    int n_cu;          // compute units of that device
    uint16_t* p_dev;   // [D, R] bf16
    double* pf_dev;    // [D, R] float64 copy read by the projection kernels
    uint16_t* ag_dev;  // [L, N, Hk, B, R] bf16
    uint32_t* err_dev; // device error word
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[2048];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return PRED_OK;
}

int hip_fail(hipError_t e, const char* what) {
    if (e == hipErrorInvalidConfiguration)   // raised by the launchers themselves, before enqueueing
        return fail(PRED_ERR_OUT_OF_RANGE, "%s: the call needs more than 2^31-1 workgroups; split it", what);
    return fail(PRED_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Dims check of PredictorDims::validate (nq a multiple of nkv) plus positivity
// and overflow of A_g's size.  Returns the A_g byte count or a negative code.
int64_t checked_a_g_bytes(const pred_dims* d) {
    if (!d) return fail(PRED_ERR_NULL_ARG, "dims is NULL");
    if (d->num_layers <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 || d->r <= 0 ||
        d->block_size <= 0 || d->max_blocks <= 0)
        return fail(PRED_ERR_INVALID_DIMS,
                    "every dim must be > 0 (layers %d, q heads %d, kv heads %d, head_dim %d, r %d, block_size %d, "
                    "max_blocks %lld)",
                    d->num_layers, d->num_q_heads, d->num_kv_heads, d->head_dim, d->r, d->block_size,
                    (long long)d->max_blocks);
    if (d->num_q_heads % d->num_kv_heads != 0)
        return fail(PRED_ERR_INVALID_DIMS, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                    d->num_q_heads, d->num_kv_heads);
    int64_t v = d->num_layers;
    if (!mul_ok(v, d->max_blocks, &v) || !mul_ok(v, d->num_kv_heads, &v) || !mul_ok(v, d->block_size, &v) ||
        !mul_ok(v, d->r, &v) || !mul_ok(v, 2, &v))
        return fail(PRED_ERR_INVALID_DIMS, "A_g size overflows 64 bits");
    return v;
}

int check_supported(const pred_dims* d) {
    if (d->head_dim % 8 != 0 || d->r % 8 != 0)
        return fail(PRED_ERR_UNSUPPORTED, "head_dim (%d) and r (%d) must be multiples of 8 (16-byte vectors)",
                    d->head_dim, d->r);
    if (d->r > 256) return fail(PRED_ERR_UNSUPPORTED, "r (%d) above 256", d->r);
    if (d->head_dim > 65536) return fail(PRED_ERR_UNSUPPORTED, "head_dim (%d) above 65536", d->head_dim);
    return PRED_OK;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Run-time options, read from the environment once per process:
//   PRED_SCORE_PATH = auto | decode | generic   which score kernel family every
//       score call takes (auto: the library's choice; decode: the vector-ALU
//       streaming decode kernel, or the plain kernel where its layout does not
//       fit; generic: the plain per-block and per-cell kernels).  A debugging
//       switch: every path computes the same scores within float32 rounding.
//   PRED_LOG = 1   one line on stderr per score launch naming the kernel.
// pred_set_score_path changes the first at run time.
struct Options {
    std::atomic<int> score_path{PRED_SCORE_PATH_AUTO};
    bool log = false;
};

int parse_score_path(const char* v) {
    if (!v || !*v || !strcmp(v, "auto") || !strcmp(v, "0")) return PRED_SCORE_PATH_AUTO;
    if (!strcmp(v, "decode") || !strcmp(v, "valu") || !strcmp(v, "1")) return PRED_SCORE_PATH_DECODE;
    if (!strcmp(v, "generic") || !strcmp(v, "2")) return PRED_SCORE_PATH_GENERIC;
    fprintf(stderr, "libpred: PRED_SCORE_PATH=%s is not one of auto, decode, generic; using auto\n", v);
    return PRED_SCORE_PATH_AUTO;
}

Options& options() {
    static Options* o = [] {
        Options* x = new Options();
        x->score_path.store(parse_score_path(getenv("PRED_SCORE_PATH")));
        const char* lg = getenv("PRED_LOG");
        x->log = lg && *lg && strcmp(lg, "0") != 0;
        return x;
    }();
    return *o;
}

int score_path() { return options().score_path.load(std::memory_order_relaxed); }

// The kernel family a score_blocks call takes: the many-row MFMA scorer when a
// kv head has more than 16 queries and the shape is one it handles, else the
// decode or plain kernel (score_decode.hip decides between those).
bool takes_prefill(const pred::ScoreArgs& a, int path) {
    return path == PRED_SCORE_PATH_AUTO && (int64_t)a.M * (a.Hq / a.Hk) > 16 && pred::prefill_supported(a);
}

int create_impl(const pred_dims* d, const uint16_t* p_host_in, uint64_t seed, uint32_t flags, void* stream,
                pred_t** out) {
    if (!out) return fail(PRED_ERR_NULL_ARG, "out is NULL");
    *out = nullptr;
    const int64_t need = checked_a_g_bytes(d);
    if (need < 0) return (int)need;
    int rc = check_supported(d);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;

    const int64_t pn = (int64_t)d->head_dim * d->r;
    std::vector<uint16_t> p_host((size_t)pn);
    if (p_host_in) memcpy(p_host.data(), p_host_in, (size_t)pn * 2);
    else pred::build_projection(d->head_dim, d->r, seed, p_host.data());
    std::vector<double> pf_host((size_t)pn);
    for (int64_t i = 0; i < pn; ++i) {
        uint32_t w = (uint32_t)p_host[i] << 16;
        float f;
        memcpy(&f, &w, 4);
        pf_host[i] = (double)f;
    }

    size_t free_b = 0, total_b = 0;
    hipError_t e = hipMemGetInfo(&free_b, &total_b);
    if (e != hipSuccess) return hip_fail(e, "hipMemGetInfo");
    rc = pred_check_fit(d, (uint64_t)free_b);
    if (rc) return rc;

    pred_t* p = new pred_t();
    p->d = *d;
    // frees on a failure path: their own errors cannot change the outcome
    auto cleanup = [&](int code) {
        if (p->p_dev) (void)hipFree(p->p_dev);
        if (p->pf_dev) (void)hipFree(p->pf_dev);
        if (p->ag_dev) (void)hipFree(p->ag_dev);
        if (p->err_dev) (void)hipFree(p->err_dev);
        delete p;
        return code;
    };
    if ((e = hipGetDevice(&p->device)) != hipSuccess) return cleanup(hip_fail(e, "hipGetDevice"));
    if ((e = hipDeviceGetAttribute(&p->n_cu, hipDeviceAttributeMultiprocessorCount, p->device)) != hipSuccess)
        return cleanup(hip_fail(e, "compute unit count"));
    if ((e = pred::rank_prepare()) != hipSuccess) return cleanup(hip_fail(e, "ranking kernel set-up"));
    if ((e = pred::rank_scratch_prepare(p->device)) != hipSuccess)
        return cleanup(hip_fail(e, "address of the static ranking scratch"));
    if ((e = hipMalloc(&p->p_dev, (size_t)pn * 2)) != hipSuccess) return cleanup(hip_fail(e, "hipMalloc(P)"));
    if ((e = hipMalloc(&p->pf_dev, (size_t)pn * 8)) != hipSuccess) return cleanup(hip_fail(e, "hipMalloc(P f64)"));
    if ((e = hipMalloc(&p->err_dev, 4)) != hipSuccess) return cleanup(hip_fail(e, "hipMalloc(error word)"));
    if ((e = hipMalloc(&p->ag_dev, (size_t)need)) != hipSuccess)
        return cleanup(fail(PRED_ERR_OOM, "hipMalloc of A_g (%lld bytes) failed: %s", (long long)need,
                            hipGetErrorString(e)));
    if ((e = hipMemcpyAsync(p->p_dev, p_host.data(), (size_t)pn * 2, hipMemcpyHostToDevice, st)) != hipSuccess)
        return cleanup(hip_fail(e, "upload P"));
    if ((e = hipMemcpyAsync(p->pf_dev, pf_host.data(), (size_t)pn * 8, hipMemcpyHostToDevice, st)) != hipSuccess)
        return cleanup(hip_fail(e, "upload P f64"));
    if ((e = hipMemsetAsync(p->err_dev, 0, 4, st)) != hipSuccess) return cleanup(hip_fail(e, "clear error word"));
    if (flags & PRED_FLAG_ZERO_AG) {
        if ((e = hipMemsetAsync(p->ag_dev, 0, (size_t)need, st)) != hipSuccess)
            return cleanup(hip_fail(e, "zero A_g"));
    }
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return cleanup(hip_fail(e, "hipStreamSynchronize"));
    *out = p;
    return ok();
}

}  // namespace

extern "C" {

int64_t pred_a_g_bytes(const pred_dims* d) {
    const int64_t v = checked_a_g_bytes(d);
    if (v >= 0) ok();
    return v;
}

int pred_check_fit(const pred_dims* d, uint64_t free_bytes) {
    const int64_t need = checked_a_g_bytes(d);
    if (need < 0) return (int)need;
    // 5% of free memory stays for scratch and attention buffers.
    const uint64_t budget = (free_bytes / 100u) * 95u + (free_bytes % 100u) * 95u / 100u;
    if ((uint64_t)need > budget) {
        return fail(PRED_ERR_OOM,
                    "predictor A_g would need %.2f GiB but only %.2f GiB fits in 95%% of the %.2f GiB of free HBM "
                    "(5%% is kept for scratch and attention). Shrink one of: r = %d (r = %d halves A_g); "
                    "max_blocks = %lld (halving the maximum sequence length halves A_g); the KV-cache footprint or "
                    "other allocations, to free HBM. A_g bytes = num_layers (%d) x max_blocks (%lld) x "
                    "num_kv_heads (%d) x block_size (%d) x r (%d) x 2.",
                    need / 1073741824.0, budget / 1073741824.0, free_bytes / 1073741824.0, d->r, d->r / 2,
                    (long long)d->max_blocks, d->num_layers, (long long)d->max_blocks, d->num_kv_heads,
                    d->block_size, d->r);
    }
    return ok();
}

const char* pred_limits(void) {
    return "head_dim and r multiples of 8; r <= 256; head_dim <= 65536; 16-byte aligned q, q_proj and k "
           "buffers. Streaming decode scorer: r in {16,32,64,128} and block_size*r/8 a power of two <= 1024 "
           "(5 to 16 queries per kv head with r in {32,64,128} and block_size*r >= 512: its matrix-core "
           "variant); other shapes use a plain per-block kernel; more than 16 queries per kv head with r in "
           "{16,32,64,128} and block_size in {8,16,32}: the many-row MFMA scorer. Rank: n_blocks <= 2^31-1; above 2048 per segment a "
           "workspace of 8*n_blocks*n_segments bytes is needed (16*n_blocks*n_segments above 8192); select_keep "
           "the same with n_blocks = stride, n_segments = rows. Row scorer: MFMA for r in {16,32,64,128}, "
           "block_size in {8,16,32}, num_kv_heads in {1,2,4,8}, num_q_heads a multiple of 4; a plain kernel "
           "otherwise.";
}

const char* pred_version(void) { return "rank_kv_block_amd 0.1 (gfx950)"; }

int pred_create(const pred_dims* d, uint64_t seed, uint32_t flags, void* stream, pred_t** out) {
    return create_impl(d, nullptr, seed, flags, stream, out);
}

int pred_create_with_projection(const pred_dims* d, const pred_bf16* p_host, uint32_t flags, void* stream,
                                pred_t** out) {
    if (!p_host) return fail(PRED_ERR_NULL_ARG, "p_host is NULL");
    return create_impl(d, p_host, 0, flags, stream, out);
}

void pred_destroy(pred_t* p) {
    if (!p) return;
    // best effort: pred_destroy has no way to report a failure, and every
    // allocation is released whatever the earlier calls return
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    (void)hipSetDevice(p->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(p->p_dev);
    (void)hipFree(p->pf_dev);
    (void)hipFree(p->ag_dev);
    (void)hipFree(p->err_dev);
    if (have_cur) (void)hipSetDevice(cur);
    delete p;
}

// Every entry point's work is an impl(..., go): all host checks first, and with
// go == false it returns after them, so a composite call (pred_decode_step)
// can check every part before it enqueues anything.
namespace {

int project_q_impl(pred_t* p, const pred_bf16* q, int64_t n_vec, pred_bf16* q_proj, void* stream, bool go) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    if (n_vec < 0) return fail(PRED_ERR_OUT_OF_RANGE, "n_vec (%lld) < 0", (long long)n_vec);
    if (n_vec == 0) return ok();
    if (!q || !q_proj) return fail(PRED_ERR_NULL_ARG, "q or q_proj is NULL");
    if (!aligned16(q) || !aligned16(q_proj)) return fail(PRED_ERR_UNSUPPORTED, "q and q_proj must be 16-byte aligned");
    int64_t rows;
    if (!mul_ok(n_vec, p->d.num_q_heads, &rows)) return fail(PRED_ERR_OUT_OF_RANGE, "n_vec too large");
    if (!go) return ok();
    hipError_t e = pred::launch_project_dense(q, p->pf_dev, q_proj, rows, p->d.head_dim, p->d.r, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "project_q launch");
    return ok();
}

int project_kv_impl(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* k, const int32_t* block_table,
                    int64_t n_blocks, void* stream, bool go) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    if (layer0 < 0 || n_layers < 0 || (int64_t)layer0 + n_layers > p->d.num_layers)
        return fail(PRED_ERR_OUT_OF_RANGE, "project_kv_block out of range: layers [%d, %d) of %d", layer0,
                    layer0 + n_layers, p->d.num_layers);
    if (n_blocks < 0) return fail(PRED_ERR_OUT_OF_RANGE, "n_blocks (%lld) < 0", (long long)n_blocks);
    if (!block_table && n_blocks > p->d.max_blocks)
        return fail(PRED_ERR_OUT_OF_RANGE, "project_kv_block out of range: %lld blocks without a table, max_blocks %lld",
                    (long long)n_blocks, (long long)p->d.max_blocks);
    if (n_blocks == 0 || n_layers == 0) return ok();
    if (!k) return fail(PRED_ERR_NULL_ARG, "k is NULL");
    if (!aligned16(k)) return fail(PRED_ERR_UNSUPPORTED, "k must be 16-byte aligned");
    if (!go) return ok();
    const pred_dims& d = p->d;
    uint16_t* a_first = p->ag_dev + (int64_t)layer0 * d.max_blocks * d.num_kv_heads * d.block_size * d.r;
    hipError_t e = pred::launch_project_paged(k, p->pf_dev, a_first, block_table, n_layers, n_blocks, d.max_blocks,
                                              d.num_kv_heads, d.block_size, d.head_dim, d.r, p->err_dev,
                                              (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "project_kv_block launch");
    return ok();
}

// project_kv_block then project_q, both checked before either is enqueued; the
// two small projections of a decode step share one launch.
int project_step_impl(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* k, const int32_t* new_table,
                      int64_t n_new, const pred_bf16* q, int64_t n_vec, pred_bf16* q_proj, void* stream, bool go) {
    int rc = project_kv_impl(p, layer0, n_layers, k, new_table, n_new, stream, false);
    if (rc == 0) rc = project_q_impl(p, q, n_vec, q_proj, stream, false);
    if (rc || !go) return rc;
    const pred_dims& d = p->d;
    const bool kv_work = n_new > 0 && n_layers > 0;
    const int64_t rows = n_vec > 0 ? n_vec * d.num_q_heads : 0;   // product checked by project_q_impl
    uint16_t* a_first = p->ag_dev + (int64_t)layer0 * d.max_blocks * d.num_kv_heads * d.block_size * d.r;
    hipError_t e = pred::launch_project_pair(kv_work ? k : nullptr, a_first, new_table, kv_work ? n_layers : 0,
                                             kv_work ? n_new : 0, d.max_blocks, d.num_kv_heads, d.block_size,
                                             p->err_dev, q, q_proj, rows, p->pf_dev, d.head_dim, d.r,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "project_step launch");
    return ok();
}

int score_impl(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* q_proj, int32_t n_rows,
               const int32_t* block_tables, int64_t n_blocks, int32_t n_seqs, const int32_t* last_fill,
               float* scores, void* stream, bool go) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    if (layer0 < 0 || n_layers < 0 || (int64_t)layer0 + n_layers > p->d.num_layers)
        return fail(PRED_ERR_OUT_OF_RANGE, "score_blocks layers [%d, %d) outside [0, %d)", layer0, layer0 + n_layers,
                    p->d.num_layers);
    if (n_blocks < 0 || n_seqs < 0 || n_rows < 0)
        return fail(PRED_ERR_OUT_OF_RANGE, "negative count (n_blocks %lld, n_seqs %d, n_rows %d)",
                    (long long)n_blocks, n_seqs, n_rows);
    if (!block_tables && n_blocks > p->d.max_blocks)
        return fail(PRED_ERR_OUT_OF_RANGE, "score_blocks: %lld blocks without a table, max_blocks %lld",
                    (long long)n_blocks, (long long)p->d.max_blocks);
    if (n_layers == 0 || n_blocks == 0 || n_seqs == 0) return ok();
    if (n_rows == 0) return fail(PRED_ERR_OUT_OF_RANGE, "n_rows must be >= 1");
    if (!q_proj || !scores) return fail(PRED_ERR_NULL_ARG, "q_proj or scores is NULL");
    if (!aligned16(q_proj)) return fail(PRED_ERR_UNSUPPORTED, "q_proj must be 16-byte aligned");
    if (!go) return ok();
    pred::ScoreArgs a;
    a.qp = q_proj;
    a.ag = p->ag_dev;
    a.tables = block_tables;
    a.fill = last_fill;
    a.scores = scores;
    a.err = p->err_dev;
    a.N = p->d.max_blocks;
    a.n = n_blocks;
    a.layer0 = layer0;
    a.n_layers = n_layers;
    a.S = n_seqs;
    a.M = n_rows;
    a.Hq = p->d.num_q_heads;
    a.Hk = p->d.num_kv_heads;
    a.B = p->d.block_size;
    a.R = p->d.r;
    hipError_t e;
    const int path = score_path();
    const bool prefill = takes_prefill(a, path);
    if (options().log)
        fprintf(stderr, "libpred: score_blocks layers [%d, %d) seqs %d blocks %lld rows %d -> %s\n", layer0,
                layer0 + n_layers, n_seqs, (long long)n_blocks, n_rows,
                prefill ? "score_prefill_kernel" : pred::score_decode_variant(a, path).c_str());
    if (prefill) e = pred::launch_score_prefill(a, (hipStream_t)stream);
    else e = pred::launch_score_decode_or_generic(a, path, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "score_blocks launch");
    return ok();
}

}  // namespace

int pred_project_q(pred_t* p, const pred_bf16* q, int64_t n_vec, pred_bf16* q_proj, void* stream) {
    return project_q_impl(p, q, n_vec, q_proj, stream, true);
}

int pred_project_kv_block(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* k,
                          const int32_t* block_table, int64_t n_blocks, void* stream) {
    return project_kv_impl(p, layer0, n_layers, k, block_table, n_blocks, stream, true);
}

int pred_project_step(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* k_new, const int32_t* new_table,
                      int64_t n_new, const pred_bf16* q, int64_t n_vec, pred_bf16* q_proj, void* stream) {
    return project_step_impl(p, layer0, n_layers, k_new, new_table, n_new, q, n_vec, q_proj, stream, true);
}

int pred_score_blocks(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* q_proj, int32_t n_rows,
                      const int32_t* block_tables, int64_t n_blocks, int32_t n_seqs, float* scores, void* stream) {
    return score_impl(p, layer0, n_layers, q_proj, n_rows, block_tables, n_blocks, n_seqs, nullptr, scores, stream,
                      true);
}

int pred_score_blocks_masked(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* q_proj, int32_t n_rows,
                             const int32_t* block_tables, int64_t n_blocks, int32_t n_seqs, const int32_t* last_fill,
                             float* scores, void* stream) {
    return score_impl(p, layer0, n_layers, q_proj, n_rows, block_tables, n_blocks, n_seqs, last_fill, scores,
                      stream, true);
}

namespace {

// ScoreArgs carrying the handle's dims and n_rows rows (enough for the kernel choice)
bool choice_args(pred_t* p, int32_t n_rows, pred::ScoreArgs& a, const char* what) {
    if (!p || n_rows < 1) {
        fail(p ? PRED_ERR_OUT_OF_RANGE : PRED_ERR_NULL_ARG, "%s: %s", what, p ? "n_rows < 1" : "NULL handle");
        return false;
    }
    a = pred::ScoreArgs{};
    a.N = p->d.max_blocks;
    a.n = 1;
    a.n_layers = 1;
    a.S = 1;
    a.M = n_rows;
    a.Hq = p->d.num_q_heads;
    a.Hk = p->d.num_kv_heads;
    a.B = p->d.block_size;
    a.R = p->d.r;
    return true;
}

thread_local std::string g_variant;

}  // namespace

const char* pred_score_kernel_name(pred_t* p, int32_t n_rows) {
    pred::ScoreArgs a;
    if (!choice_args(p, n_rows, a, "score_kernel_name")) return nullptr;
    const int path = score_path();
    ok();
    if (takes_prefill(a, path)) return "score_prefill_kernel";
    return pred::score_decode_path_name(a, path);
}

const char* pred_score_kernel_variant(pred_t* p, int32_t n_rows, int64_t n_blocks) {
    pred::ScoreArgs a;
    if (!choice_args(p, n_rows, a, "score_kernel_variant")) return nullptr;
    if (n_blocks < 1) {
        fail(PRED_ERR_OUT_OF_RANGE, "score_kernel_variant: n_blocks < 1");
        return nullptr;
    }
    a.n = n_blocks;
    const int path = score_path();
    ok();
    g_variant = takes_prefill(a, path) ? std::string("score_prefill_kernel") : pred::score_decode_variant(a, path);
    return g_variant.c_str();
}

int pred_set_score_path(int32_t path) {
    if (path != PRED_SCORE_PATH_AUTO && path != PRED_SCORE_PATH_DECODE && path != PRED_SCORE_PATH_GENERIC)
        return fail(PRED_ERR_OUT_OF_RANGE, "score path %d is not PRED_SCORE_PATH_AUTO, _DECODE or _GENERIC", path);
    options().score_path.store(path);
    return ok();
}

int pred_get_score_path(void) { return score_path(); }

int pred_score_rows(pred_t* p, int32_t layer, const pred_bf16* q_proj, int64_t rows, int64_t first_pos,
                    const int32_t* block_table, int64_t n_blocks, float* scores, int64_t stride, void* stream) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    if (layer < 0 || layer >= p->d.num_layers)
        return fail(PRED_ERR_OUT_OF_RANGE, "score_rows: layer %d outside [0, %d)", layer, p->d.num_layers);
    if (rows < 0 || first_pos < 0 || n_blocks < 0 || stride < 0)
        return fail(PRED_ERR_OUT_OF_RANGE, "negative count (rows %lld, first_pos %lld, n_blocks %lld, stride %lld)",
                    (long long)rows, (long long)first_pos, (long long)n_blocks, (long long)stride);
    if (rows > 2147483647LL || first_pos > (1LL << 62) || n_blocks > 2147483647LL)
        return fail(PRED_ERR_OUT_OF_RANGE, "score_rows: rows and n_blocks must be <= 2^31-1, first_pos <= 2^62");
    if (!block_table && n_blocks > p->d.max_blocks)
        return fail(PRED_ERR_OUT_OF_RANGE, "score_rows: %lld blocks without a table, max_blocks %lld",
                    (long long)n_blocks, (long long)p->d.max_blocks);
    int64_t cells;
    if (!mul_ok(rows, stride, &cells)) return fail(PRED_ERR_OUT_OF_RANGE, "rows * stride too large");
    if (cells == 0) return ok();
    if (!q_proj || !scores) return fail(PRED_ERR_NULL_ARG, "q_proj or scores is NULL");
    if (!aligned16(q_proj)) return fail(PRED_ERR_UNSUPPORTED, "q_proj must be 16-byte aligned");
    pred::RowScoreArgs a;
    a.qp = q_proj;
    a.ag = p->ag_dev;
    a.table = block_table;
    a.scores = scores;
    a.err = p->err_dev;
    a.N = p->d.max_blocks;
    a.layer = layer;
    a.n = n_blocks;
    a.rows = rows;
    a.first_pos = first_pos;
    a.stride = stride;
    a.Hq = p->d.num_q_heads;
    a.Hk = p->d.num_kv_heads;
    a.B = p->d.block_size;
    a.R = p->d.r;
    a.n_cu = p->n_cu;
    const int path = score_path();
    if (options().log)
        fprintf(stderr, "libpred: score_rows layer %d rows %lld blocks %lld -> %s\n", layer, (long long)rows,
                (long long)n_blocks, pred::score_rows_path_name(a, path));
    hipError_t e = pred::launch_score_rows(a, path, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "score_rows launch");
    return ok();
}

namespace {

// The k lowest of every segment, in eviction order; k = n_blocks is the full ranking.
int rank_or_select(pred_t* p, const float* scores, int64_t n_blocks, int64_t n_segments, int64_t k,
                   pred::RowOrder ro, int32_t* victims, void* workspace, size_t ws_bytes, void* stream,
                   const char* what, bool go = true) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    if (n_blocks < 0 || n_segments < 0)
        return fail(PRED_ERR_OUT_OF_RANGE, "negative count (n_blocks %lld, n_segments %lld)", (long long)n_blocks,
                    (long long)n_segments);
    if (n_blocks > 2147483647LL || n_segments > 2147483647LL)
        return fail(PRED_ERR_OUT_OF_RANGE, "n_blocks and n_segments must be <= 2^31-1");
    if (k < 0 || k > n_blocks)
        return fail(PRED_ERR_OUT_OF_RANGE, "k (%lld) outside [0, n_blocks = %lld]", (long long)k, (long long)n_blocks);
    if (n_blocks == 0 || n_segments == 0 || k == 0) return ok();
    if (!scores || !victims) return fail(PRED_ERR_NULL_ARG, "scores or victims is NULL");
    const size_t need = pred::rank_workspace_bytes(n_blocks, n_segments);
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(PRED_ERR_WORKSPACE, "%s needs a %zu-byte workspace (%zu given)", what, need,
                    workspace ? ws_bytes : (size_t)0);
    if (need > 0 && ((uintptr_t)workspace & 7u)) return fail(PRED_ERR_WORKSPACE, "workspace must be 8-byte aligned");
    if (!go) return ok();
    hipError_t e = pred::launch_rank(scores, n_blocks, n_segments, k, ro, victims, workspace, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, what);
    return ok();
}

}  // namespace

int pred_rank_victims(pred_t* p, const float* scores, int64_t n_blocks, int64_t n_segments, int32_t* victims,
                      void* workspace, size_t ws_bytes, void* stream) {
    return rank_or_select(p, scores, n_blocks, n_segments, n_blocks, pred::RowOrder{0, 0, 0}, victims, workspace,
                          ws_bytes, stream, "rank_victims");
}

static_assert(pred::kNoAllocScratchBytes == PRED_NOALLOC_SCRATCH_BYTES, "scratch size differs from pred.h");

int pred_rank_victims_noalloc(pred_t* p, const float* scores, int64_t n_blocks, int64_t n_segments, int32_t* victims,
                              void* stream) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    if (n_blocks > 0 && n_segments > 0 && n_blocks <= 2147483647LL && n_segments <= 2147483647LL) {
        const size_t need = pred::rank_workspace_bytes(n_blocks, n_segments);
        if (need > pred::kNoAllocScratchBytes)
            return fail(PRED_ERR_WORKSPACE,
                        "rank_victims_noalloc: %lld segments of %lld blocks need %zu bytes of scratch, above its "
                        "%zu-byte static maximum; use pred_rank_victims with a workspace",
                        (long long)n_segments, (long long)n_blocks, need, pred::kNoAllocScratchBytes);
    }
    void* ws = pred::rank_scratch(p->device);
    if (!ws) return fail(PRED_ERR_HIP, "rank_victims_noalloc: the static scratch of device %d was not set up", p->device);
    return rank_or_select(p, scores, n_blocks, n_segments, n_blocks, pred::RowOrder{0, 0, 0}, victims, ws,
                          pred::kNoAllocScratchBytes, stream, "rank_victims_noalloc");
}

int pred_select_victims(pred_t* p, const float* scores, int64_t n_blocks, int64_t n_segments, int64_t k,
                        int32_t* victims, void* workspace, size_t ws_bytes, void* stream) {
    return rank_or_select(p, scores, n_blocks, n_segments, k, pred::RowOrder{0, 0, 0}, victims, workspace, ws_bytes,
                          stream, "select_victims");
}

int pred_select_keep(pred_t* p, const float* scores, int64_t rows, int64_t stride, int64_t first_pos, int32_t ratio,
                     int64_t topk, int32_t* keep, void* workspace, size_t ws_bytes, void* stream) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    if (ratio < 1) return fail(PRED_ERR_OUT_OF_RANGE, "ratio (%d) must be >= 1", ratio);
    if (first_pos < 0 || first_pos > (1LL << 62))
        return fail(PRED_ERR_OUT_OF_RANGE, "first_pos (%lld) outside [0, 2^62]", (long long)first_pos);
    return rank_or_select(p, scores, stride, rows, topk, pred::RowOrder{1, first_pos, ratio}, keep, workspace,
                          ws_bytes, stream, "select_keep");
}

int pred_decode_step(pred_t* p, int32_t layer0, int32_t n_layers, const pred_bf16* k_new, const int32_t* new_table,
                     int64_t n_new, const pred_bf16* q, int32_t n_rows, pred_bf16* q_proj,
                     const int32_t* block_tables, int64_t n_blocks, int32_t n_seqs, const int32_t* last_fill,
                     float* scores, int64_t k, int32_t* victims, void* workspace, size_t ws_bytes, void* stream) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    if (n_layers < 0 || n_seqs < 0 || n_rows < 0)
        return fail(PRED_ERR_OUT_OF_RANGE, "negative count (n_layers %d, n_seqs %d, n_rows %d)", n_layers, n_seqs,
                    n_rows);
    int64_t n_vec, n_seg;
    if (!mul_ok((int64_t)n_layers * n_seqs, n_rows, &n_vec) || !mul_ok(n_layers, n_seqs, &n_seg))
        return fail(PRED_ERR_OUT_OF_RANGE, "decode_step: too many rows");
    // every part is checked before anything is enqueued
    for (int pass = 0; pass < 2; ++pass) {
        const bool go = pass == 1;
        int rc = project_step_impl(p, layer0, n_layers, k_new, new_table, n_new, q, n_vec, q_proj, stream, go);
        if (rc == 0)
            rc = score_impl(p, layer0, n_layers, q_proj, n_rows, block_tables, n_blocks, n_seqs, last_fill, scores,
                            stream, go);
        if (rc == 0)
            rc = rank_or_select(p, scores, n_blocks, n_seg, k, pred::RowOrder{0, 0, 0}, victims, workspace, ws_bytes,
                                stream, "decode_step ranking", go);
        if (rc) return rc;
    }
    return ok();
}

size_t pred_rank_workspace_bytes(int64_t n_blocks, int64_t n_segments) {
    return pred::rank_workspace_bytes(n_blocks, n_segments);
}

int pred_projection_host(int32_t head_dim, int32_t r, uint64_t seed, pred_bf16* out) {
    if (!out) return fail(PRED_ERR_NULL_ARG, "out is NULL");
    if (head_dim <= 0 || r <= 0) return fail(PRED_ERR_INVALID_DIMS, "head_dim and r must be > 0");
    pred::build_projection(head_dim, r, seed, out);
    return ok();
}

int pred_copy_projection(pred_t* p, pred_bf16* host_out) {
    if (!p || !host_out) return fail(PRED_ERR_NULL_ARG, "predictor or host_out is NULL");
    hipError_t e = hipMemcpy(host_out, p->p_dev, (size_t)p->d.head_dim * p->d.r * 2, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "copy P");
    return ok();
}

void* pred_a_g_ptr(pred_t* p) { return p ? p->ag_dev : nullptr; }

int pred_read_slot(pred_t* p, int32_t layer, int64_t block, pred_bf16* host_out, void* stream) {
    if (!p || !host_out) return fail(PRED_ERR_NULL_ARG, "predictor or host_out is NULL");
    if (layer < 0 || layer >= p->d.num_layers || block < 0 || block >= p->d.max_blocks)
        return fail(PRED_ERR_OUT_OF_RANGE, "read_slot out of range: layer %d, block %lld", layer, (long long)block);
    const pred_dims& d = p->d;
    const int64_t slot = (int64_t)d.num_kv_heads * d.block_size * d.r;
    const uint16_t* src = p->ag_dev + ((int64_t)layer * d.max_blocks + block) * slot;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(host_out, src, (size_t)slot * 2, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "read slot");
    return ok();
}

int pred_get_dims(pred_t* p, pred_dims* out) {
    if (!p || !out) return fail(PRED_ERR_NULL_ARG, "predictor or out is NULL");
    *out = p->d;
    return ok();
}

int pred_device_error(pred_t* p, void* stream) {
    if (!p) return fail(PRED_ERR_NULL_ARG, "predictor is NULL");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    uint32_t w = 0;
    e = hipMemcpy(&w, p->err_dev, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "read error word");
    if (w) {
        e = hipMemset(p->err_dev, 0, 4);
        if (e != hipSuccess) return hip_fail(e, "clear error word");
        return fail(PRED_ERR_DEVICE, "%s%s(flags 0x%x)",
                    (w & 1u) ? "a kernel met a block-table entry outside [0, max_blocks) " : "",
                    (w & 2u) ? "a last-block fill count was outside [0, block_size] " : "", w);
    }
    return ok();
}

const char* pred_last_error(void) { return g_err.c_str(); }

}  // extern "C"
