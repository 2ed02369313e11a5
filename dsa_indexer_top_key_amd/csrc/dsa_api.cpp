// Host side of the C ABI declared in include/dsa.h: argument validation (before any HIP
// call), workspace sizing, launch dispatch and error reporting.  No allocation and no host
// synchronisation; between calls only per-device lookups are kept (the scratch array's
// address here, the CU count in the top-k launcher).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <mutex>

#include "dsa.h"

namespace dsa {
hipError_t launch_ln_keys(const float* raw, const float* gamma, const float* beta, float eps,
                          uint16_t* keys, int64_t n_rows, hipStream_t stream);
hipError_t launch_indexer_scores(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                                 const int64_t* kv_off, const int32_t* q_req,
                                 const int32_t* q_pos, int32_t T, int32_t B, int64_t max_s,
                                 float* scores, int64_t ld, hipStream_t stream,
                                 const int32_t* page_table = nullptr, int lg_page = 0,
                                 int max_pages = 0);
hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid,
                       const int64_t* kv_off, const int32_t* q_req, const int32_t* q_pos,
                       int32_t B, int32_t T, int64_t max_n, int32_t* ids, hipStream_t stream,
                       int32_t* cand_ws);
size_t topk_workspace_bytes(int32_t T, int64_t max_n);
hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* latent, int64_t ld_lat,
                             const uint16_t* kpe, int64_t ld_kpe, const int64_t* kv_off,
                             const int32_t* q_req, const int32_t* ids, int32_t T, int32_t B,
                             float scale, void* out, bool out_f32, float* lse, void* workspace,
                             hipStream_t stream, const int32_t* page_table = nullptr,
                             int lg_page = 0, int max_pages = 0);
size_t sparse_mla_workspace_bytes(int32_t T);
hipError_t launch_value_gate(const uint16_t* o, const uint16_t* w_uv, const uint16_t* gate,
                             int32_t T, uint16_t* out, hipStream_t stream);
size_t proj_workspace_bytes(int32_t T);
hipError_t launch_quantize_keys_fp8(const uint16_t* keys, int64_t n_rows, uint8_t* codes,
                                    float* scales, hipStream_t stream);
hipError_t launch_indexer_scores_fp8(const uint16_t* q_idx, const uint16_t* w, const uint8_t* codes,
                                     const float* kscale, const int64_t* kv_off,
                                     const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                     int32_t B, int64_t max_s, float* scores, int64_t ld,
                                     hipStream_t stream);
hipError_t launch_indexer_proj(const uint16_t* c_q, const uint16_t* h, const uint16_t* w_qi,
                               const uint16_t* w_k, const uint16_t* w_w, const float* gamma,
                               const float* beta, float eps, int32_t T, uint16_t* q_idx,
                               uint16_t* w, uint16_t* keys, const int64_t* key_rows,
                               void* workspace, hipStream_t stream);
}  // namespace dsa

namespace {

thread_local char g_err[512] = "";

dsa_status_t fail(dsa_status_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

dsa_status_t ok() {
    g_err[0] = '\0';
    return DSA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

dsa_status_t from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

#define DSA_REQUIRE(cond, code, ...) \
    do {                             \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

constexpr size_t kAlign = DSA_WORKSPACE_ALIGN;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Common checks of the indexer arguments (stages 2 and 2+3).
dsa_status_t check_indexer(const char* fn, const uint16_t* q_idx, const uint16_t* w,
                           const uint16_t* keys, const int64_t* kv_off, const int32_t* q_req,
                           const int32_t* q_pos, int32_t T, int32_t B, int64_t max_S,
                           int32_t n_heads, int32_t head_dim) {
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    DSA_REQUIRE(B >= 1, DSA_ERR_INVALID_ARG, "%s: B=%d must be >= 1", fn, B);
    DSA_REQUIRE(max_S >= 1 && max_S <= INT32_MAX, DSA_ERR_INVALID_ARG,
                "%s: max_S=%lld must be in [1, 2^31-1]", fn, static_cast<long long>(max_S));
    DSA_REQUIRE(n_heads == DSA_INDEX_HEADS && head_dim == DSA_INDEX_DIM, DSA_ERR_UNSUPPORTED,
                "%s: indexer shape %d heads x %d is unsupported (only %d x %d)", fn, n_heads,
                head_dim, DSA_INDEX_HEADS, DSA_INDEX_DIM);
    DSA_REQUIRE(q_idx && w && keys && kv_off && q_req && q_pos, DSA_ERR_INVALID_ARG,
                "%s: null input pointer", fn);
    DSA_REQUIRE(aligned(q_idx, 16) && aligned(keys, 16), DSA_ERR_INVALID_ARG,
                "%s: q_idx and keys must be 16-byte aligned", fn);
    DSA_REQUIRE(aligned(w, 2) && aligned(kv_off, 8) && aligned(q_req, 4) && aligned(q_pos, 4),
                DSA_ERR_INVALID_ARG, "%s: misaligned w/kv_off/q_req/q_pos", fn);
    return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return 1; }

const char* dsa_status_string(int status) {
    switch (status) {
        case DSA_OK: return "DSA_OK";
        case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
        case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape or option not implemented";
        case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP runtime error";
        default: return "unknown dsa status";
    }
}

const char* dsa_last_error(void) { return g_err; }

dsa_status_t dsa_index_keys_layernorm(const float* raw, const float* gamma, const float* beta,
                                      float eps, uint16_t* keys, int64_t n_rows, void* stream) {
    const char* fn = "dsa_index_keys_layernorm";
    DSA_REQUIRE(n_rows >= 0, DSA_ERR_INVALID_ARG, "%s: n_rows=%lld is negative", fn,
                static_cast<long long>(n_rows));
    DSA_REQUIRE(std::isfinite(eps) && eps >= 0.f, DSA_ERR_INVALID_ARG,
                "%s: eps must be finite and >= 0", fn);
    if (n_rows == 0) return ok();
    DSA_REQUIRE(raw && gamma && beta && keys, DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
    DSA_REQUIRE(aligned(raw, 16) && aligned(gamma, 16) && aligned(beta, 16) && aligned(keys, 16),
                DSA_ERR_INVALID_ARG, "%s: raw, gamma, beta and keys must be 16-byte aligned", fn);
    return from_hip(dsa::launch_ln_keys(raw, gamma, beta, eps, keys, n_rows,
                                        static_cast<hipStream_t>(stream)), fn);
}

dsa_status_t dsa_indexer_scores(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                                const int64_t* kv_off, const int32_t* q_req,
                                const int32_t* q_pos, int32_t T, int32_t B, int64_t max_S,
                                int32_t n_heads, int32_t head_dim, float* scores,
                                int64_t ld_scores, void* stream) {
    const char* fn = "dsa_indexer_scores";
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    if (T == 0) return ok();
    dsa_status_t st = check_indexer(fn, q_idx, w, keys, kv_off, q_req, q_pos, T, B, max_S,
                                    n_heads, head_dim);
    if (st != DSA_OK) return st;
    DSA_REQUIRE(scores, DSA_ERR_INVALID_ARG, "%s: scores is null", fn);
    DSA_REQUIRE(aligned(scores, 4), DSA_ERR_INVALID_ARG, "%s: scores must be 4-byte aligned", fn);
    DSA_REQUIRE(ld_scores >= max_S, DSA_ERR_INVALID_ARG, "%s: ld_scores=%lld < max_S=%lld", fn,
                static_cast<long long>(ld_scores), static_cast<long long>(max_S));
    return from_hip(dsa::launch_indexer_scores(q_idx, w, keys, kv_off, q_req, q_pos, T, B,
                                               max_S, scores, ld_scores,
                                               static_cast<hipStream_t>(stream)), fn);
}

dsa_status_t dsa_topk(const float* scores, int64_t ld, const int32_t* n_valid, int32_t T,
                      int64_t max_n, int32_t topk, int32_t* ids, void* stream) {
    const char* fn = "dsa_topk";
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    DSA_REQUIRE(topk == DSA_TOPK, DSA_ERR_UNSUPPORTED, "%s: topk=%d unsupported (only %d)", fn,
                topk, DSA_TOPK);
    if (T == 0) return ok();
    DSA_REQUIRE(scores && n_valid && ids, DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
    DSA_REQUIRE(max_n >= 0 && max_n <= INT32_MAX, DSA_ERR_INVALID_ARG,
                "%s: max_n=%lld must be in [0, 2^31-1]", fn, static_cast<long long>(max_n));
    DSA_REQUIRE(ld >= max_n && ld >= 1, DSA_ERR_INVALID_ARG, "%s: ld=%lld < max_n=%lld", fn,
                static_cast<long long>(ld), static_cast<long long>(max_n));
    DSA_REQUIRE(aligned(scores, 4) && aligned(n_valid, 4) && aligned(ids, 4),
                DSA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    return from_hip(dsa::launch_topk(scores, ld, n_valid, nullptr, nullptr, nullptr, 0, T, max_n,
                                     ids, static_cast<hipStream_t>(stream), nullptr), fn);
}

// Score rows are padded to a multiple of four floats so every row starts 16-byte aligned.
static int64_t score_ld(int64_t max_S) { return (max_S + 3) & ~static_cast<int64_t>(3); }

// Workspace: fp32 scores [T, score_ld] then, when rows are split for the selection, the
// per-part candidate lists [T * parts, 2048] int32.
static size_t score_bytes(int32_t T, int64_t max_S) {
    return round_up(static_cast<size_t>(T) * static_cast<size_t>(score_ld(max_S)) * sizeof(float));
}

size_t dsa_indexer_topk_workspace_size(int32_t T, int64_t max_S) {
    if (T <= 0 || max_S <= 0) return 0;
    return score_bytes(T, max_S) + round_up(dsa::topk_workspace_bytes(T, max_S));
}

// Page-table arguments of the paged entry points: page_size a power of two in [64, 2^20],
// max_pages >= 1, the table non-null and 4-byte aligned.  lg_page gets log2(page_size).
static dsa_status_t check_pages(const char* fn, const int32_t* page_table, int32_t page_size,
                                int32_t max_pages, int* lg_page) {
    DSA_REQUIRE(page_size >= 64 && page_size <= (1 << 20) && (page_size & (page_size - 1)) == 0,
                DSA_ERR_UNSUPPORTED, "%s: page_size=%d must be a power of two in [64, 2^20]", fn,
                page_size);
    DSA_REQUIRE(max_pages >= 1, DSA_ERR_INVALID_ARG, "%s: max_pages=%d must be >= 1", fn, max_pages);
    DSA_REQUIRE(page_table && aligned(page_table, 4), DSA_ERR_INVALID_ARG,
                "%s: page_table null or misaligned", fn);
    *lg_page = __builtin_ctz(static_cast<unsigned>(page_size));
    return DSA_OK;
}

// Scratch of the allocation-free entry point (dsa_indexer_topk_noalloc): a file-scope device
// array that stands in for the caller's workspace.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code the array's name is only a host-side stand-in, so
// the device address is looked up once per device (with that device current) and only that
// address is handed to kernels.  The scores and candidate lists it holds are fully written
// before they are read within one call, so nothing needs clearing between calls; calls that
// overlap on one GPU share the array and race.
constexpr size_t kNoAllocScratch = DSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on a device's first call).
static dsa_status_t scratch_address(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    DSA_REQUIRE(dev >= 0 && dev < kMaxDevices, DSA_ERR_UNSUPPORTED,
                "%s: device %d beyond the %d devices the scratch table covers", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(DSA_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed: %s", fn,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

// Stages 2+3.  With use_scratch the caller's workspace is ignored and this file's scratch
// array of the current device is used instead (after every other argument has been checked).
static dsa_status_t indexer_topk_impl(const char* fn, const uint16_t* q_idx, const uint16_t* w,
                                      const uint16_t* keys, const int64_t* kv_off,
                                      const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                      int32_t B, int64_t max_S, int32_t n_heads, int32_t head_dim,
                                      int32_t topk, int32_t* ids, void* workspace,
                                      size_t workspace_bytes, void* stream,
                                      const int32_t* page_table, int lg_page, int max_pages,
                                      bool use_scratch = false) {
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    DSA_REQUIRE(topk == DSA_TOPK, DSA_ERR_UNSUPPORTED, "%s: topk=%d unsupported (only %d)", fn,
                topk, DSA_TOPK);
    if (T == 0) return ok();
    dsa_status_t st = check_indexer(fn, q_idx, w, keys, kv_off, q_req, q_pos, T, B, max_S,
                                    n_heads, head_dim);
    if (st != DSA_OK) return st;
    DSA_REQUIRE(ids && aligned(ids, 4), DSA_ERR_INVALID_ARG, "%s: ids null or misaligned", fn);
    const size_t need = dsa_indexer_topk_workspace_size(T, max_S);
    if (use_scratch) {
        DSA_REQUIRE(need <= kNoAllocScratch, DSA_ERR_UNSUPPORTED,
                    "%s: T=%d, max_S=%lld need %zu bytes of scratch, more than the %zu bytes this "
                    "entry point holds per GPU (use dsa_indexer_topk with a workspace)", fn, T,
                    static_cast<long long>(max_S), need, kNoAllocScratch);
        const dsa_status_t st2 = scratch_address(fn, &workspace);
        if (st2 != DSA_OK) return st2;
        workspace_bytes = kNoAllocScratch;
    }
    DSA_REQUIRE(workspace && aligned(workspace, kAlign), DSA_ERR_WORKSPACE,
                "%s: workspace null or not %zu-byte aligned", fn, kAlign);
    DSA_REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE,
                "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* scores = static_cast<float*>(workspace);
    const int64_t ld = score_ld(max_S);
    hipError_t e = dsa::launch_indexer_scores(q_idx, w, keys, kv_off, q_req, q_pos, T, B, max_S,
                                              scores, ld, s, page_table, lg_page, max_pages);
    if (e != hipSuccess) return from_hip(e, fn);
    int32_t* cand = dsa::topk_workspace_bytes(T, max_S) > 0
                        ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + score_bytes(T, max_S))
                        : nullptr;
    return from_hip(dsa::launch_topk(scores, ld, nullptr, kv_off, q_req, q_pos, B, T, max_S, ids,
                                     s, cand),
                    fn);
}

dsa_status_t dsa_indexer_topk(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                              const int64_t* kv_off, const int32_t* q_req,
                              const int32_t* q_pos, int32_t T, int32_t B, int64_t max_S,
                              int32_t n_heads, int32_t head_dim, int32_t topk, int32_t* ids,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return indexer_topk_impl("dsa_indexer_topk", q_idx, w, keys, kv_off, q_req, q_pos, T, B,
                             max_S, n_heads, head_dim, topk, ids, workspace, workspace_bytes,
                             stream, nullptr, 0, 0);
}

dsa_status_t dsa_indexer_topk_noalloc(const uint16_t* q_idx, const uint16_t* w,
                                      const uint16_t* keys, const int64_t* kv_off,
                                      const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                      int32_t B, int64_t max_S, int32_t n_heads,
                                      int32_t head_dim, int32_t topk, int32_t* ids,
                                      void* stream) {
    return indexer_topk_impl("dsa_indexer_topk_noalloc", q_idx, w, keys, kv_off, q_req, q_pos, T,
                             B, max_S, n_heads, head_dim, topk, ids, nullptr, 0, stream, nullptr,
                             0, 0, /*use_scratch=*/true);
}

dsa_status_t dsa_indexer_topk_paged(const uint16_t* q_idx, const uint16_t* w,
                                    const uint16_t* key_pool, const int32_t* page_table,
                                    int32_t page_size, int32_t max_pages, const int64_t* kv_off,
                                    const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                    int32_t B, int64_t max_S, int32_t n_heads, int32_t head_dim,
                                    int32_t topk, int32_t* ids, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    const char* fn = "dsa_indexer_topk_paged";
    int lg = 0;
    if (T > 0) {
        const dsa_status_t st = check_pages(fn, page_table, page_size, max_pages, &lg);
        if (st != DSA_OK) return st;
    }
    return indexer_topk_impl(fn, q_idx, w, key_pool, kv_off, q_req, q_pos, T, B, max_S, n_heads,
                             head_dim, topk, ids, workspace, workspace_bytes, stream, page_table,
                             lg, max_pages);
}

size_t dsa_sparse_mla_workspace_size(int32_t T, int32_t n_heads, int32_t topk) {
    if (T <= 0 || n_heads != DSA_MLA_HEADS || topk != DSA_TOPK) return 0;
    return round_up(dsa::sparse_mla_workspace_bytes(T));
}

static dsa_status_t sparse_mla_impl(const char* fn, const uint16_t* q, const uint16_t* latent,
                                    int64_t ld_latent, const uint16_t* kpe, int64_t ld_kpe,
                                    const int64_t* kv_off, const int32_t* q_req,
                                    const int32_t* ids, int32_t T, int32_t B, int32_t n_heads,
                                    int32_t topk, float scale, void* out, int32_t out_dtype,
                                    float* lse, void* workspace, size_t workspace_bytes,
                                    void* stream, const int32_t* page_table, int lg_page,
                                    int max_pages) {
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    DSA_REQUIRE(n_heads == DSA_MLA_HEADS, DSA_ERR_UNSUPPORTED,
                "%s: n_heads=%d unsupported (only %d)", fn, n_heads, DSA_MLA_HEADS);
    DSA_REQUIRE(topk == DSA_TOPK, DSA_ERR_UNSUPPORTED, "%s: topk=%d unsupported (only %d)", fn,
                topk, DSA_TOPK);
    if (T == 0) return ok();
    DSA_REQUIRE(B >= 1, DSA_ERR_INVALID_ARG, "%s: B=%d must be >= 1", fn, B);
    DSA_REQUIRE(std::isfinite(scale), DSA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    DSA_REQUIRE(out_dtype == DSA_OUT_BF16 || out_dtype == DSA_OUT_F32, DSA_ERR_UNSUPPORTED,
                "%s: out_dtype=%d unsupported (DSA_OUT_BF16 or DSA_OUT_F32)", fn, out_dtype);
    DSA_REQUIRE(q && latent && kpe && kv_off && q_req && ids && out, DSA_ERR_INVALID_ARG,
                "%s: null pointer", fn);
    DSA_REQUIRE(aligned(q, 16) && aligned(latent, 16) && aligned(kpe, 16) && aligned(out, 16),
                DSA_ERR_INVALID_ARG, "%s: q, latent, kpe and out must be 16-byte aligned", fn);
    DSA_REQUIRE(aligned(kv_off, 8) && aligned(q_req, 4) && aligned(ids, 4) &&
                    (lse == nullptr || aligned(lse, 4)),
                DSA_ERR_INVALID_ARG, "%s: misaligned kv_off/q_req/ids/lse", fn);
    DSA_REQUIRE(ld_latent >= DSA_LATENT_DIM && ld_latent % 8 == 0, DSA_ERR_INVALID_ARG,
                "%s: ld_latent=%lld must be >= 512 and a multiple of 8", fn,
                static_cast<long long>(ld_latent));
    DSA_REQUIRE(ld_kpe >= DSA_COMPANION_DIM && ld_kpe % 8 == 0, DSA_ERR_INVALID_ARG,
                "%s: ld_kpe=%lld must be >= 64 and a multiple of 8", fn,
                static_cast<long long>(ld_kpe));
    const size_t need = dsa_sparse_mla_workspace_size(T, n_heads, topk);
    if (need > 0) {
        DSA_REQUIRE(workspace && aligned(workspace, kAlign), DSA_ERR_WORKSPACE,
                    "%s: workspace null or not %zu-byte aligned", fn, kAlign);
        DSA_REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE,
                    "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
    }
    return from_hip(dsa::launch_sparse_mla(q, latent, ld_latent, kpe, ld_kpe, kv_off, q_req, ids,
                                           T, B, scale, out, out_dtype == DSA_OUT_F32, lse,
                                           workspace, static_cast<hipStream_t>(stream),
                                           page_table, lg_page, max_pages), fn);
}

dsa_status_t dsa_sparse_mla_attn(const uint16_t* q, const uint16_t* latent, int64_t ld_latent,
                                 const uint16_t* kpe, int64_t ld_kpe, const int64_t* kv_off,
                                 const int32_t* q_req, const int32_t* ids, int32_t T,
                                 int32_t B, int32_t n_heads, int32_t topk, float scale,
                                 void* out, int32_t out_dtype, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return sparse_mla_impl("dsa_sparse_mla_attn", q, latent, ld_latent, kpe, ld_kpe, kv_off, q_req,
                           ids, T, B, n_heads, topk, scale, out, out_dtype, lse, workspace,
                           workspace_bytes, stream, nullptr, 0, 0);
}

dsa_status_t dsa_sparse_mla_attn_paged(const uint16_t* q, const uint16_t* latent_pool,
                                       int64_t ld_latent, const uint16_t* kpe_pool,
                                       int64_t ld_kpe, const int32_t* page_table,
                                       int32_t page_size, int32_t max_pages,
                                       const int64_t* kv_off, const int32_t* q_req,
                                       const int32_t* ids, int32_t T, int32_t B, int32_t n_heads,
                                       int32_t topk, float scale, void* out, int32_t out_dtype,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
    const char* fn = "dsa_sparse_mla_attn_paged";
    int lg = 0;
    if (T > 0) {
        const dsa_status_t st = check_pages(fn, page_table, page_size, max_pages, &lg);
        if (st != DSA_OK) return st;
    }
    return sparse_mla_impl(fn, q, latent_pool, ld_latent, kpe_pool, ld_kpe, kv_off, q_req, ids, T,
                           B, n_heads, topk, scale, out, out_dtype, lse, workspace,
                           workspace_bytes, stream, page_table, lg, max_pages);
}


dsa_status_t dsa_value_gate(const uint16_t* o, const uint16_t* w_uv, const uint16_t* gate,
                            int32_t T, int32_t n_heads, uint16_t* out, void* stream) {
    const char* fn = "dsa_value_gate";
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    DSA_REQUIRE(n_heads == DSA_MLA_HEADS, DSA_ERR_UNSUPPORTED, "%s: n_heads=%d unsupported (only %d)",
                fn, n_heads, DSA_MLA_HEADS);
    if (T == 0) return ok();
    DSA_REQUIRE(o && w_uv && gate && out, DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
    DSA_REQUIRE(aligned(o, 16) && aligned(w_uv, 16) && aligned(gate, 2) && aligned(out, 4),
                DSA_ERR_INVALID_ARG, "%s: o and w_uv must be 16-byte, gate 2-byte, out 4-byte aligned", fn);
    return from_hip(dsa::launch_value_gate(o, w_uv, gate, T, out, static_cast<hipStream_t>(stream)), fn);
}

size_t dsa_indexer_project_workspace_size(int32_t T) {
    return T > 0 ? round_up(dsa::proj_workspace_bytes(T)) : 0;
}

dsa_status_t dsa_indexer_project(const uint16_t* c_q, const uint16_t* h, const uint16_t* w_qi,
                                 const uint16_t* w_k, const uint16_t* w_w, const float* gamma,
                                 const float* beta, float eps, int32_t T, uint16_t* q_idx,
                                 uint16_t* w, uint16_t* keys, const int64_t* key_rows,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "dsa_indexer_project";
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    DSA_REQUIRE(std::isfinite(eps) && eps >= 0.f, DSA_ERR_INVALID_ARG,
                "%s: eps must be finite and >= 0", fn);
    if (T == 0) return ok();
    DSA_REQUIRE(c_q && h && w_qi && w_k && w_w && gamma && beta && q_idx && w && keys && key_rows,
                DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
    DSA_REQUIRE(aligned(c_q, 16) && aligned(h, 16) && aligned(w_qi, 16) && aligned(w_k, 16) &&
                aligned(w_w, 16) && aligned(q_idx, 16) && aligned(keys, 16),
                DSA_ERR_INVALID_ARG, "%s: c_q, h, w_qi, w_k, w_w, q_idx and keys must be 16-byte aligned", fn);
    DSA_REQUIRE(aligned(gamma, 4) && aligned(beta, 4) && aligned(w, 2) && aligned(key_rows, 8),
                DSA_ERR_INVALID_ARG, "%s: misaligned gamma/beta/w/key_rows", fn);
    const size_t need = dsa_indexer_project_workspace_size(T);
    DSA_REQUIRE(workspace && aligned(workspace, kAlign) && workspace_bytes >= need,
                DSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) needed, got %zu",
                fn, need, workspace_bytes);
    return from_hip(dsa::launch_indexer_proj(c_q, h, w_qi, w_k, w_w, gamma, beta, eps, T, q_idx,
                                             w, keys, key_rows, workspace,
                                             static_cast<hipStream_t>(stream)), fn);
}

dsa_status_t dsa_quantize_index_keys_fp8(const uint16_t* keys, int64_t n_rows, uint8_t* codes,
                                         float* scales, void* stream) {
    const char* fn = "dsa_quantize_index_keys_fp8";
    DSA_REQUIRE(n_rows >= 0, DSA_ERR_INVALID_ARG, "%s: n_rows=%lld is negative", fn,
                static_cast<long long>(n_rows));
    if (n_rows == 0) return ok();
    DSA_REQUIRE(keys && codes && scales, DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
    DSA_REQUIRE(aligned(keys, 16) && aligned(codes, 16) && aligned(scales, 4), DSA_ERR_INVALID_ARG,
                "%s: keys and codes must be 16-byte, scales 4-byte aligned", fn);
    return from_hip(dsa::launch_quantize_keys_fp8(keys, n_rows, codes, scales,
                                                  static_cast<hipStream_t>(stream)), fn);
}

dsa_status_t dsa_indexer_scores_fp8(const uint16_t* q_idx, const uint16_t* w, const uint8_t* codes,
                                    const float* scales, const int64_t* kv_off,
                                    const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                    int32_t B, int64_t max_S, int32_t n_heads, int32_t head_dim,
                                    float* scores, int64_t ld_scores, void* stream) {
    const char* fn = "dsa_indexer_scores_fp8";
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    if (T == 0) return ok();
    dsa_status_t st = check_indexer(fn, q_idx, w, reinterpret_cast<const uint16_t*>(codes), kv_off,
                                    q_req, q_pos, T, B, max_S, n_heads, head_dim);
    if (st != DSA_OK) return st;
    DSA_REQUIRE(scales && aligned(scales, 4), DSA_ERR_INVALID_ARG, "%s: scales null or misaligned", fn);
    DSA_REQUIRE(scores && aligned(scores, 4), DSA_ERR_INVALID_ARG, "%s: scores null or misaligned", fn);
    DSA_REQUIRE(ld_scores >= max_S, DSA_ERR_INVALID_ARG, "%s: ld_scores=%lld < max_S=%lld", fn,
                static_cast<long long>(ld_scores), static_cast<long long>(max_S));
    return from_hip(dsa::launch_indexer_scores_fp8(q_idx, w, codes, scales, kv_off, q_req, q_pos, T,
                                                   B, max_S, scores, ld_scores,
                                                   static_cast<hipStream_t>(stream)), fn);
}

dsa_status_t dsa_indexer_topk_fp8(const uint16_t* q_idx, const uint16_t* w, const uint8_t* codes,
                                  const float* scales, const int64_t* kv_off,
                                  const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                  int32_t B, int64_t max_S, int32_t n_heads, int32_t head_dim,
                                  int32_t topk, int32_t* ids, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    const char* fn = "dsa_indexer_topk_fp8";
    DSA_REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "%s: T=%d is negative", fn, T);
    DSA_REQUIRE(topk == DSA_TOPK, DSA_ERR_UNSUPPORTED, "%s: topk=%d unsupported (only %d)", fn,
                topk, DSA_TOPK);
    if (T == 0) return ok();
    dsa_status_t st = check_indexer(fn, q_idx, w, reinterpret_cast<const uint16_t*>(codes), kv_off,
                                    q_req, q_pos, T, B, max_S, n_heads, head_dim);
    if (st != DSA_OK) return st;
    DSA_REQUIRE(scales && aligned(scales, 4), DSA_ERR_INVALID_ARG, "%s: scales null or misaligned", fn);
    DSA_REQUIRE(ids && aligned(ids, 4), DSA_ERR_INVALID_ARG, "%s: ids null or misaligned", fn);
    const size_t need = dsa_indexer_topk_workspace_size(T, max_S);
    DSA_REQUIRE(workspace && aligned(workspace, kAlign), DSA_ERR_WORKSPACE,
                "%s: workspace null or not %zu-byte aligned", fn, kAlign);
    DSA_REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE,
                "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* scores = static_cast<float*>(workspace);
    const int64_t ld = score_ld(max_S);
    hipError_t e = dsa::launch_indexer_scores_fp8(q_idx, w, codes, scales, kv_off, q_req, q_pos, T,
                                                  B, max_S, scores, ld, s);
    if (e != hipSuccess) return from_hip(e, fn);
    int32_t* cand = dsa::topk_workspace_bytes(T, max_S) > 0
                        ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + score_bytes(T, max_S))
                        : nullptr;
    return from_hip(dsa::launch_topk(scores, ld, nullptr, kv_off, q_req, q_pos, B, T, max_S, ids,
                                     s, cand),
                    fn);
}

}  // extern "C"
