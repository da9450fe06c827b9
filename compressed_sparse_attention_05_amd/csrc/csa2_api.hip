// C-ABI entry points of libcsa2 (declared in include/csa2.h): argument
// validation on the host, workspace sizing, and stream-ordered launches.
// Nothing here allocates, frees or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/csa2.h"
#include "csa2_internal.h"

// Device scratch of csa2_sparse_attn_decode_noalloc: each GPU the library
// runs on holds one copy, loaded with the code object, until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory;
// the device address comes from hipGetSymbolAddress, taken once per device
// (scratch_on_current_device) and used everywhere host code hands the array
// to a kernel.
static __device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return CSA2_OK;
}

int device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(CSA2_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(int dt) { return dt == CSA2_F32 || dt == CSA2_BF16; }
size_t dtype_size(int dt) { return dt == CSA2_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with that device current) and kept.
int scratch_on_current_device(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CSA2_E_DEVICE, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(CSA2_E_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(CSA2_E_DEVICE, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CSA2_OK;
}

}  // namespace

extern "C" {

const char* csa2_version(void) { return "csa2-mi355x 0.1 (gfx950)"; }

const char* csa2_last_error(void) { return g_last_error.c_str(); }

// --------------------------------------------------------------------------
int mxfp4_kv_write(const void* x, int x_dtype, int64_t n_rows, int32_t D, const int64_t* dst_row,
                   int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const void* idx_k_rows,
                   int idx_k_dtype, int32_t d_I, void* idx_k_cache, void* stream) {
    if (n_rows < 0) return fail(CSA2_E_INVALID, "mxfp4_kv_write: n_rows < 0");
    if (D <= 0 || D % 16 != 0) return fail(CSA2_E_INVALID, "mxfp4_kv_write: D=%d must be a positive multiple of 16", D);
    if (!valid_dtype(x_dtype)) return fail(CSA2_E_INVALID, "mxfp4_kv_write: bad x_dtype %d", x_dtype);
    if (n_cache_rows < 0) return fail(CSA2_E_INVALID, "mxfp4_kv_write: n_cache_rows < 0");
    if (n_rows == 0) return ok();
    if (!x || !dst_row || !codes || !scales) return fail(CSA2_E_INVALID, "mxfp4_kv_write: null pointer");
    if (!aligned(x, 16) || !aligned(codes, 8))
        return fail(CSA2_E_INVALID, "mxfp4_kv_write: x must be 16-byte and codes 8-byte aligned");
    if (idx_k_rows) {
        if (!idx_k_cache) return fail(CSA2_E_INVALID, "mxfp4_kv_write: idx_k_cache is null");
        if (!valid_dtype(idx_k_dtype)) return fail(CSA2_E_INVALID, "mxfp4_kv_write: bad idx_k_dtype");
        const int64_t rb = static_cast<int64_t>(d_I) * static_cast<int64_t>(dtype_size(idx_k_dtype));
        if (d_I <= 0 || rb % 16 != 0) return fail(CSA2_E_INVALID, "mxfp4_kv_write: indexer row bytes must be a positive multiple of 16");
        if (n_cache_rows % 64 != 0) return fail(CSA2_E_INVALID, "mxfp4_kv_write: the tiled indexer cache needs n_cache_rows %% 64 == 0");
        if (!aligned(idx_k_rows, 16) || !aligned(idx_k_cache, 16))
            return fail(CSA2_E_INVALID, "mxfp4_kv_write: indexer rows must be 16-byte aligned");
    }
    const int64_t rb = idx_k_rows ? static_cast<int64_t>(d_I) * static_cast<int64_t>(dtype_size(idx_k_dtype)) : 0;
    hipError_t e = csa2::launch_kv_write(x, x_dtype == CSA2_BF16, n_rows, D, dst_row, n_cache_rows, codes,
                                         scales, idx_k_rows, rb, idx_k_cache, as_stream(stream));
    return device_status(e, "mxfp4_kv_write");
}

// --------------------------------------------------------------------------
int csa2_kv_write_project(const void* x, int x_dtype, int64_t n_rows, int32_t D, const int64_t* dst_row,
                          int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const float* w_ik,
                          int32_t d_I, void* idx_k_cache, void* stream) {
    if (n_rows < 0) return fail(CSA2_E_INVALID, "csa2_kv_write_project: n_rows < 0");
    if (D <= 0 || D % 16 != 0)
        return fail(CSA2_E_INVALID, "csa2_kv_write_project: D=%d must be a positive multiple of 16", D);
    if (d_I <= 0 || d_I % 8 != 0)
        return fail(CSA2_E_INVALID, "csa2_kv_write_project: d_I=%d must be a positive multiple of 8", d_I);
    if (!valid_dtype(x_dtype)) return fail(CSA2_E_INVALID, "csa2_kv_write_project: bad x_dtype %d", x_dtype);
    if (n_cache_rows < 0 || n_cache_rows % 64 != 0)
        return fail(CSA2_E_INVALID, "csa2_kv_write_project: the tiled indexer cache needs n_cache_rows %% 64 == 0");
    if (!csa2::kv_project_shape_supported(D, d_I))
        return fail(CSA2_E_UNSUPPORTED, "csa2_kv_write_project: D=%d not supported (D <= 512)", D);
    if (n_rows == 0) return ok();
    if (!x || !dst_row || !codes || !scales || !w_ik || !idx_k_cache)
        return fail(CSA2_E_INVALID, "csa2_kv_write_project: null pointer");
    if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(idx_k_cache, 16) || !aligned(w_ik, 16))
        return fail(CSA2_E_INVALID,
                    "csa2_kv_write_project: x, w_ik and idx_k_cache must be 16-byte and codes 8-byte aligned");
    hipError_t e = csa2::launch_kv_write_project(x, x_dtype == CSA2_BF16, n_rows, D, dst_row, n_cache_rows, codes,
                                                 scales, w_ik, d_I, idx_k_cache, as_stream(stream));
    return device_status(e, "csa2_kv_write_project");
}

// --------------------------------------------------------------------------
static int check_score_args(const csa2_score_args* a) {
    if (!a) return fail(CSA2_E_INVALID, "csa2_index_score: args is null");
    if (a->B < 0 || a->Tq < 0 || a->cap < 0) return fail(CSA2_E_INVALID, "csa2_index_score: negative size");
    if (!valid_dtype(a->q_dtype) || !valid_dtype(a->k_dtype))
        return fail(CSA2_E_INVALID, "csa2_index_score: bad dtype");
    if (a->H_I <= 0 || a->d_I <= 0) return fail(CSA2_E_INVALID, "csa2_index_score: H_I and d_I must be positive");
    if (!csa2::score_shape_supported(a->H_I, a->d_I))
        return fail(CSA2_E_UNSUPPORTED, "csa2_index_score: (H_I=%d, d_I=%d) not instantiated (have 8x128, 4x64, 2x32)",
                    a->H_I, a->d_I);
    if (a->m < 1) return fail(CSA2_E_INVALID, "csa2_index_score: m must be >= 1");
    if (a->ld_scores < 0) return fail(CSA2_E_INVALID, "csa2_index_score: ld_scores < 0");
    if (a->pool_blocks) {
        if (a->P_b <= 0) return fail(CSA2_E_INVALID, "csa2_index_score: P_b must be positive");
        if (a->ld_scores < static_cast<int64_t>(a->P_b) * 8)
            return fail(CSA2_E_INVALID, "csa2_index_score: ld_scores must be >= 8*P_b in pool mode");
        if (a->block_max) return fail(CSA2_E_INVALID, "csa2_index_score: block_max is for Full mode only");
    }
    if (a->cap % 64 != 0) return fail(CSA2_E_INVALID, "csa2_index_score: cap must be a multiple of 64 (tiled indexer cache)");
    if (a->B * a->Tq == 0) return CSA2_OK;
    if (!a->q_idx || !a->w || !a->k_idx || !a->ctx_len || !a->scores)
        return fail(CSA2_E_INVALID, "csa2_index_score: null pointer");
    if (!aligned(a->k_idx, 16)) return fail(CSA2_E_INVALID, "csa2_index_score: k_idx must be 16-byte aligned");
    return CSA2_OK;
}

size_t csa2_index_score_workspace_size(const csa2_score_args* a) {
    (void)a;
    return 0;
}

int csa2_index_score(const csa2_score_args* a, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_score_args(a);
    if (rc != CSA2_OK) return rc;
    if (a->B * a->Tq == 0 || a->ld_scores == 0) return ok();
    (void)ws; (void)ws_bytes;
    csa2::ScoreLaunch p;
    p.q_idx = a->q_idx; p.q_bf16 = a->q_dtype == CSA2_BF16;
    p.w = a->w; p.k_idx = a->k_idx; p.k_bf16 = a->k_dtype == CSA2_BF16;
    p.B = a->B; p.Tq = a->Tq; p.cap = a->cap; p.H_I = a->H_I; p.d_I = a->d_I;
    p.ctx_len = a->ctx_len; p.q_pos = a->q_pos; p.m = a->m;
    p.pool = a->pool_blocks; p.P_b = a->pool_blocks ? a->P_b : 0;
    p.scores = a->scores; p.ld = a->ld_scores;
    p.block_max = a->block_max; p.ld_bm = (a->ld_scores + 7) / 8;
    return device_status(csa2::launch_score(p, as_stream(stream)), "csa2_index_score");
}

// --------------------------------------------------------------------------
int csa2_write_and_score(const void* x, int x_dtype, int32_t D, const int64_t* dst_row, uint8_t* codes,
                         uint8_t* scales, const void* idx_k_rows, const csa2_score_args* a, void* ws,
                         size_t ws_bytes, void* stream) {
    int rc = check_score_args(a);
    if (rc != CSA2_OK) return rc;
    if (a->Tq != 1) return fail(CSA2_E_INVALID, "csa2_write_and_score: decode only (Tq must be 1)");
    if (D <= 0 || D % 16 != 0)
        return fail(CSA2_E_INVALID, "csa2_write_and_score: D=%d must be a positive multiple of 16", D);
    if (!valid_dtype(x_dtype)) return fail(CSA2_E_INVALID, "csa2_write_and_score: bad x_dtype %d", x_dtype);
    const int64_t nch = static_cast<int64_t>(a->d_I) * dtype_size(a->k_dtype) / 16;
    if (D / 16 + nch > 256)
        return fail(CSA2_E_UNSUPPORTED, "csa2_write_and_score: D/16 + indexer chunks = %lld exceeds one workgroup",
                    static_cast<long long>(D / 16 + nch));
    if (a->B == 0) return ok();
    if (!x || !dst_row || !codes || !scales || !idx_k_rows)
        return fail(CSA2_E_INVALID, "csa2_write_and_score: null pointer");
    if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(idx_k_rows, 16))
        return fail(CSA2_E_INVALID, "csa2_write_and_score: x and idx_k_rows must be 16-byte and codes 8-byte aligned");
    (void)ws; (void)ws_bytes;
    csa2::ScoreLaunch p;
    p.q_idx = a->q_idx; p.q_bf16 = a->q_dtype == CSA2_BF16;
    p.w = a->w; p.k_idx = a->k_idx; p.k_bf16 = a->k_dtype == CSA2_BF16;
    p.B = a->B; p.Tq = 1; p.cap = a->cap; p.H_I = a->H_I; p.d_I = a->d_I;
    p.ctx_len = a->ctx_len; p.q_pos = a->q_pos; p.m = a->m;
    p.pool = a->pool_blocks; p.P_b = a->pool_blocks ? a->P_b : 0;
    p.scores = a->scores; p.ld = a->ld_scores;
    p.block_max = a->block_max; p.ld_bm = (a->ld_scores + 7) / 8;
    p.knew = idx_k_rows; p.wx = x; p.wx_bf16 = x_dtype == CSA2_BF16; p.wD = D; p.wdst = dst_row;
    p.wcodes = codes; p.wscales = scales;
    return device_status(csa2::launch_score(p, as_stream(stream)), "csa2_write_and_score");
}

// --------------------------------------------------------------------------
size_t csa2_topk_workspace_size(int64_t rows, int64_t n, int32_t k) {
    (void)k;
    if (rows <= 0 || n <= 0) return 0;
    return csa2::topk_workspace_bytes(rows, n);
}

int csa2_topk(const float* scores, int64_t rows, int64_t n, int64_t ld, int32_t k,
              const int32_t* pool_blocks, int32_t P_b, int32_t* out_idx, void* ws, size_t ws_bytes,
              void* stream) {
    if (rows < 0 || n < 0 || ld < n) return fail(CSA2_E_INVALID, "csa2_topk: need rows >= 0 and 0 <= n <= ld");
    if (k <= 0) return fail(CSA2_E_INVALID, "csa2_topk: k must be positive");
    if (n > (int64_t(1) << 31) - 1) return fail(CSA2_E_UNSUPPORTED, "csa2_topk: n above 2^31-1");
    if (pool_blocks && (P_b <= 0 || n != static_cast<int64_t>(P_b) * 8))
        return fail(CSA2_E_INVALID, "csa2_topk: with pool_blocks, n must equal 8*P_b");
    if (rows == 0) return ok();
    if (!scores || !out_idx) return fail(CSA2_E_INVALID, "csa2_topk: null pointer");
    const size_t need = csa2_topk_workspace_size(rows, n, k);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(CSA2_E_WORKSPACE, "csa2_topk: workspace %zu bytes < required %zu", ws_bytes, need);
    if (need > 0 && !aligned(ws, 256)) return fail(CSA2_E_INVALID, "csa2_topk: workspace must be 256-byte aligned");
    return device_status(csa2::launch_topk(scores, rows, n, ld, k, pool_blocks, P_b, out_idx, ws, as_stream(stream)),
                         "csa2_topk");
}

size_t csa2_build_candidate_pool_workspace_size(int64_t rows, int64_t n_blocks, int32_t P_b) {
    if (csa2::pool_in_lds(n_blocks, P_b)) return 0;
    return csa2_topk_workspace_size(rows, n_blocks, P_b);
}

int csa2_build_candidate_pool(const float* block_max, int64_t rows, int64_t n_blocks, int64_t ld,
                              int32_t P_b, int32_t* out_blocks, void* ws, size_t ws_bytes, void* stream) {
    if (P_b <= 0) return fail(CSA2_E_INVALID, "csa2_build_candidate_pool: P_b must be positive");
    if (rows < 0 || n_blocks < 0 || ld < n_blocks)
        return fail(CSA2_E_INVALID, "csa2_build_candidate_pool: need rows >= 0 and 0 <= n_blocks <= ld");
    if (rows == 0) return ok();
    if (!block_max || !out_blocks) return fail(CSA2_E_INVALID, "csa2_build_candidate_pool: null pointer");
    if (csa2::pool_in_lds(n_blocks, P_b))
        return device_status(csa2::launch_pool(block_max, rows, n_blocks, ld, P_b, out_blocks, as_stream(stream)),
                             "csa2_build_candidate_pool");
    int rc = csa2_topk(block_max, rows, n_blocks, ld, P_b, nullptr, 0, out_blocks, ws, ws_bytes, stream);
    if (rc != CSA2_OK) {
        std::string m = "csa2_build_candidate_pool: " + g_last_error;
        g_last_error = m;
    }
    return rc;
}

int csa2_topk_from_pool(const float* scores, int64_t rows, int64_t ld, const int32_t* pool_blocks, int32_t P_b,
                        int32_t k, int32_t* out_idx, void* stream) {
    if (rows < 0 || ld < 0) return fail(CSA2_E_INVALID, "csa2_topk_from_pool: negative size");
    if (k <= 0 || P_b <= 0 || k > P_b)
        return fail(CSA2_E_INVALID, "csa2_topk_from_pool: need 0 < k <= P_b (the pool holds the top-k only then)");
    if (static_cast<int64_t>(P_b) * 8 > 32768)
        return fail(CSA2_E_UNSUPPORTED, "csa2_topk_from_pool: 8*P_b above 32768");
    if (rows == 0) return ok();
    if (!scores || !pool_blocks || !out_idx) return fail(CSA2_E_INVALID, "csa2_topk_from_pool: null pointer");
    return device_status(csa2::launch_topk_from_pool(scores, rows, ld, pool_blocks, P_b, k, out_idx, as_stream(stream)),
                         "csa2_topk_from_pool");
}

int csa2_pool_topk(const float* block_max, int64_t rows, int64_t n_blocks, int64_t ld_bm, int32_t P_b,
                   int32_t* out_blocks, const float* scores, int64_t ld, int32_t k, int32_t* out_idx,
                   void* stream) {
    if (rows < 0 || rows > (int64_t{1} << 30) || n_blocks < 0 || ld_bm < n_blocks || ld < 0)
        return fail(CSA2_E_INVALID, "csa2_pool_topk: need 0 <= rows <= 2^30, 0 <= n_blocks <= ld_bm, ld >= 0");
    if (k <= 0 || P_b <= 0 || k > P_b)
        return fail(CSA2_E_INVALID, "csa2_pool_topk: need 0 < k <= P_b (the pool holds the top-k only then)");
    if (!csa2::pool_topk_supported(n_blocks, P_b, k))
        return fail(CSA2_E_UNSUPPORTED,
                    "csa2_pool_topk: P_b=%d, n_blocks=%lld outside the one-workgroup path (P_b <= 2048, "
                    "n_blocks <= 32,768): call csa2_build_candidate_pool and csa2_topk_from_pool",
                    P_b, static_cast<long long>(n_blocks));
    if (rows == 0) return ok();
    if (!block_max || !out_blocks || !scores || !out_idx) return fail(CSA2_E_INVALID, "csa2_pool_topk: null pointer");
    return device_status(csa2::launch_pool_topk(block_max, rows, n_blocks, ld_bm, P_b, out_blocks, scores, ld, k,
                                                out_idx, as_stream(stream)),
                         "csa2_pool_topk");
}

// --------------------------------------------------------------------------
static int check_attn_common(const char* fn, const void* q, int q_dtype, const uint8_t* codes,
                             const uint8_t* scales, int64_t cap, const int32_t* idx, int32_t k,
                             const void* swa, int swa_dtype, int32_t W, int64_t units, int32_t H,
                             int32_t D, const float* out) {
    if (units < 0 || cap < 0) return fail(CSA2_E_INVALID, "%s: negative size", fn);
    if (k < 0 || W < 0 || k + W <= 0) return fail(CSA2_E_INVALID, "%s: need k >= 0, W >= 0, k + W > 0", fn);
    if (!valid_dtype(q_dtype) || !valid_dtype(swa_dtype)) return fail(CSA2_E_INVALID, "%s: bad dtype", fn);
    if (q_dtype != swa_dtype) return fail(CSA2_E_UNSUPPORTED, "%s: q and swa must share a dtype", fn);
    if (H <= 0 || D <= 0 || D % 16 != 0) return fail(CSA2_E_INVALID, "%s: bad H=%d or D=%d", fn, H, D);
    if (!csa2::attn_shape_supported(H, D))
        return fail(CSA2_E_UNSUPPORTED, "%s: (H=%d, D=%d) not instantiated (D=512 with H %% 64 == 0, or D=64 with H <= 64)",
                    fn, H, D);
    if (k > 0 && cap <= 0) return fail(CSA2_E_INVALID, "%s: k > 0 needs a non-empty cache (cap >= 1)", fn);
    if (units == 0) return CSA2_OK;
    if (!q || !out || (k > 0 && (!codes || !scales || !idx)) || (W > 0 && !swa))
        return fail(CSA2_E_INVALID, "%s: null pointer", fn);
    if (!aligned(q, 16) || !aligned(out, 16) || (swa && !aligned(swa, 16)) || (codes && !aligned(codes, 4)))
        return fail(CSA2_E_INVALID, "%s: q/out/swa must be 16-byte and codes 4-byte aligned", fn);
    return CSA2_OK;
}

size_t csa2_sparse_attn_decode_workspace_size(const csa2_attn_args* a) {
    if (!a || a->B <= 0 || !csa2::attn_shape_supported(a->H, a->D)) return 0;
    return csa2::attn_workspace_bytes(a->B, a->H, a->D, a->k, a->W);
}

// Shared by csa2_sparse_attn_decode (caller's workspace) and
// csa2_sparse_attn_decode_noalloc (the library's device scratch).
static int attn_decode_checked(const char* fn, const csa2_attn_args* a, void* ws, size_t ws_bytes,
                               bool use_scratch, void* stream) {
    if (!a) return fail(CSA2_E_INVALID, "%s: args is null", fn);
    int rc = check_attn_common(fn, a->q, a->q_dtype, a->codes, a->scales, a->cap,
                               a->idx, a->k, a->swa, a->swa_dtype, a->W, a->B, a->H, a->D, a->out);
    if (rc != CSA2_OK) return rc;
    if (a->B == 0) return ok();
    if (a->W > 0 && !a->swa_len) return fail(CSA2_E_INVALID, "%s: swa_len is null", fn);
    const size_t need = csa2_sparse_attn_decode_workspace_size(a);
    if (use_scratch) {
        if (need > CSA2_NOALLOC_SCRATCH_BYTES)
            return fail(CSA2_E_WORKSPACE,
                        "%s: this call needs %zu bytes of scratch, more than the %zu the library holds per "
                        "device; use csa2_sparse_attn_decode with a workspace",
                        fn, need, static_cast<size_t>(CSA2_NOALLOC_SCRATCH_BYTES));
        ws = nullptr;
        ws_bytes = 0;
        if (need > 0) {
            rc = scratch_on_current_device(fn, &ws);
            if (rc != CSA2_OK) return rc;
            ws_bytes = CSA2_NOALLOC_SCRATCH_BYTES;
        }
    }
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(CSA2_E_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    if (ws && !aligned(ws, 16)) return fail(CSA2_E_INVALID, "%s: workspace must be 16-byte aligned", fn);
    csa2::AttnLaunch L;
    L.q = a->q; L.q_bf16 = a->q_dtype == CSA2_BF16;
    L.codes = a->codes; L.scales = a->scales; L.cap = a->cap; L.kv_unit_stride = a->cap;
    L.idx = a->idx; L.k = a->k;
    L.swa = a->swa; L.swa_bf16 = a->swa_dtype == CSA2_BF16; L.W = a->W; L.swa_len = a->swa_len;
    L.q_pos0 = 0; L.swa_start = 0; L.prefill = false;
    L.units = a->B; L.H = a->H; L.D = a->D; L.sm_scale = a->sm_scale; L.out = a->out;
    L.ws = need > 0 ? static_cast<float*>(ws) : nullptr; L.ws_bytes = ws_bytes;
    return device_status(csa2::launch_attn(L, as_stream(stream)), fn);
}

int csa2_sparse_attn_decode(const csa2_attn_args* a, void* ws, size_t ws_bytes, void* stream) {
    return attn_decode_checked("csa2_sparse_attn_decode", a, ws, ws_bytes, false, stream);
}

int csa2_sparse_attn_decode_noalloc(const csa2_attn_args* a, void* stream) {
    return attn_decode_checked("csa2_sparse_attn_decode_noalloc", a, nullptr, 0, true, stream);
}

size_t csa2_sparse_attn_prefill_workspace_size(const csa2_attn_prefill_args* a) {
    if (!a || a->T <= 0 || !csa2::attn_shape_supported(a->H, a->D)) return 0;
    return csa2::attn_workspace_bytes(a->T, a->H, a->D, a->k, a->W);
}

int csa2_sparse_attn_prefill(const csa2_attn_prefill_args* a, void* ws, size_t ws_bytes, void* stream) {
    if (!a) return fail(CSA2_E_INVALID, "csa2_sparse_attn_prefill: args is null");
    int rc = check_attn_common("csa2_sparse_attn_prefill", a->q, a->q_dtype, a->codes, a->scales, a->cap,
                               a->idx, a->k, a->swa, a->swa_dtype, a->W, a->T, a->H, a->D, a->out);
    if (rc != CSA2_OK) return rc;
    if (a->T == 0) return ok();
    if (a->q_pos0 < 0 || a->swa_start < 0) return fail(CSA2_E_INVALID, "csa2_sparse_attn_prefill: negative position");
    const size_t need = csa2_sparse_attn_prefill_workspace_size(a);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(CSA2_E_WORKSPACE, "csa2_sparse_attn_prefill: workspace %zu bytes < required %zu", ws_bytes, need);
    if (ws && !aligned(ws, 16)) return fail(CSA2_E_INVALID, "csa2_sparse_attn_prefill: workspace must be 16-byte aligned");
    csa2::AttnLaunch L;
    L.q = a->q; L.q_bf16 = a->q_dtype == CSA2_BF16;
    L.codes = a->codes; L.scales = a->scales; L.cap = a->cap; L.kv_unit_stride = 0;
    L.idx = a->idx; L.k = a->k;
    L.swa = a->swa; L.swa_bf16 = a->swa_dtype == CSA2_BF16; L.W = a->W; L.swa_len = nullptr;
    L.q_pos0 = a->q_pos0; L.swa_start = a->swa_start; L.prefill = true;
    L.units = a->T; L.H = a->H; L.D = a->D; L.sm_scale = a->sm_scale; L.out = a->out;
    L.ws = need > 0 ? static_cast<float*>(ws) : nullptr; L.ws_bytes = ws_bytes;
    return device_status(csa2::launch_attn(L, as_stream(stream)), "csa2_sparse_attn_prefill");
}

}  // extern "C"

// --------------------------------------------------------------------------
namespace {
int check_prefill_topk(const csa2_prefill_topk_args* a) {
    const char* fn = "csa2_prefill_topk";
    if (!a) return fail(CSA2_E_INVALID, "%s: args is null", fn);
    if (a->T < 0) return fail(CSA2_E_INVALID, "%s: T < 0", fn);
    if (a->cap < 0 || a->cap % 64 != 0) return fail(CSA2_E_INVALID, "%s: cap=%lld must be a multiple of 64", fn,
                                                    static_cast<long long>(a->cap));
    if (a->ctx_len < 0 || a->ctx_len > a->cap) return fail(CSA2_E_INVALID, "%s: ctx_len outside [0, cap]", fn);
    if (a->m < 1) return fail(CSA2_E_INVALID, "%s: m must be >= 1", fn);
    if (a->q_pos0 < 0) return fail(CSA2_E_INVALID, "%s: q_pos0 < 0", fn);
    if (a->k < 1) return fail(CSA2_E_INVALID, "%s: k must be >= 1", fn);
    if (!valid_dtype(a->q_dtype) || !valid_dtype(a->k_dtype)) return fail(CSA2_E_INVALID, "%s: bad dtype", fn);
    if (a->q_dtype != CSA2_BF16 || a->k_dtype != CSA2_BF16)
        return fail(CSA2_E_UNSUPPORTED, "%s: q and k must be bf16", fn);
    if (a->H_I != 8 || a->d_I != 128)
        return fail(CSA2_E_UNSUPPORTED, "%s: H_I=%d d_I=%d (8 x 128 only)", fn, a->H_I, a->d_I);
    if (a->k > csa2::prefill_topk_max_k())
        return fail(CSA2_E_UNSUPPORTED, "%s: k=%d above %d", fn, a->k, csa2::prefill_topk_max_k());
    if (a->T > 0 && (!a->q_idx || !a->w || !a->out_idx || (a->ctx_len > 0 && !a->k_idx)))
        return fail(CSA2_E_INVALID, "%s: null tensor", fn);
    if (!aligned(a->q_idx, 16) || !aligned(a->k_idx, 16))
        return fail(CSA2_E_INVALID, "%s: q_idx and k_idx must be 16-byte aligned", fn);
    if (csa2::prefill_cols(a->T, a->ctx_len, a->q_pos0, a->m) > csa2::prefill_topk_max_cols())
        return fail(CSA2_E_UNSUPPORTED, "%s: more than %lld visible entries", fn,
                    static_cast<long long>(csa2::prefill_topk_max_cols()));
    return CSA2_OK;
}

int check_decode_select(const csa2_decode_select_args* a) {
    const char* fn = "csa2_decode_select";
    if (!a) return fail(CSA2_E_INVALID, "%s: args is null", fn);
    if (a->B < 0) return fail(CSA2_E_INVALID, "%s: B < 0", fn);
    if (a->cap <= 0 || a->cap % 64 != 0)
        return fail(CSA2_E_INVALID, "%s: cap=%lld must be a positive multiple of 64", fn,
                    static_cast<long long>(a->cap));
    if (a->k < 1 || a->P_b < 1 || a->k > a->P_b)
        return fail(CSA2_E_INVALID, "%s: need 1 <= k <= P_b (the pool holds the top-k only then)", fn);
    if (!valid_dtype(a->q_dtype) || !valid_dtype(a->k_dtype)) return fail(CSA2_E_INVALID, "%s: bad dtype", fn);
    if (a->q_dtype != CSA2_BF16 || a->k_dtype != CSA2_BF16)
        return fail(CSA2_E_UNSUPPORTED, "%s: q and k must be bf16", fn);
    if (!csa2::decode_select_supported(a->cap, a->H_I, a->d_I, a->P_b, a->k))
        return fail(CSA2_E_UNSUPPORTED,
                    "%s: H_I=%d d_I=%d cap=%lld P_b=%d outside the one-workgroup path (8 x 128, cap <= 262,144, "
                    "P_b <= 2048): use csa2_index_score with the pool and top-k calls",
                    fn, a->H_I, a->d_I, static_cast<long long>(a->cap), a->P_b);
    if (a->B > 0 && (!a->q_idx || !a->w || !a->k_idx || !a->ctx_len || !a->out_pool || !a->out_idx))
        return fail(CSA2_E_INVALID, "%s: null tensor", fn);
    if (!aligned(a->q_idx, 16) || !aligned(a->k_idx, 16))
        return fail(CSA2_E_INVALID, "%s: q_idx and k_idx must be 16-byte aligned", fn);
    return CSA2_OK;
}
}  // namespace

extern "C" {

size_t csa2_decode_select_workspace_size(const csa2_decode_select_args* a) {
    if (check_decode_select(a) != CSA2_OK) return 0;
    return csa2::decode_select_workspace_bytes(a->B, a->cap);
}

static int decode_select_call(const csa2_decode_select_args* a, void* ws, size_t ws_bytes, void* stream, bool scan) {
    const char* fn = scan ? "csa2_decode_scan" : "csa2_decode_select";
    const int rc = check_decode_select(a);
    if (rc != CSA2_OK) return rc;
    if (a->B == 0) return ok();
    const size_t need = csa2::decode_select_workspace_bytes(a->B, a->cap);
    if (!ws || ws_bytes < need) return fail(CSA2_E_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    if (!aligned(ws, 256)) return fail(CSA2_E_INVALID, "%s: workspace must be 256-byte aligned", fn);
    csa2::DecodeSelectLaunch L;
    L.q_idx = a->q_idx; L.w = a->w; L.k_idx = a->k_idx; L.ctx_len = a->ctx_len; L.B = a->B; L.cap = a->cap;
    L.P_b = a->P_b; L.k = a->k; L.out_pool = a->out_pool; L.out_idx = a->out_idx;
    return device_status(scan ? csa2::launch_decode_scan(L, ws, as_stream(stream))
                              : csa2::launch_decode_select(L, ws, as_stream(stream)), fn);
}

int csa2_decode_scan(const csa2_decode_select_args* a, void* ws, size_t ws_bytes, void* stream) {
    return decode_select_call(a, ws, ws_bytes, stream, true);
}

int csa2_decode_select(const csa2_decode_select_args* a, void* ws, size_t ws_bytes, void* stream) {
    return decode_select_call(a, ws, ws_bytes, stream, false);
}

size_t csa2_prefill_topk_workspace_size(const csa2_prefill_topk_args* a) {
    if (check_prefill_topk(a) != CSA2_OK) return 0;
    return csa2::prefill_topk_workspace_bytes(a->T, a->ctx_len, a->q_pos0, a->m);
}

int csa2_prefill_topk(const csa2_prefill_topk_args* a, void* ws, size_t ws_bytes, void* stream) {
    const int rc = check_prefill_topk(a);
    if (rc != CSA2_OK) return rc;
    if (a->T == 0) return ok();
    const size_t need = csa2::prefill_topk_workspace_bytes(a->T, a->ctx_len, a->q_pos0, a->m);
    if (!ws || ws_bytes < need)
        return fail(CSA2_E_WORKSPACE, "csa2_prefill_topk: workspace %zu bytes < required %zu", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(CSA2_E_INVALID, "csa2_prefill_topk: workspace must be 256-byte aligned");
    csa2::PrefillLaunch L;
    L.q = a->q_idx; L.w = a->w; L.k_idx = a->k_idx; L.T = a->T; L.cap = a->cap; L.ctx_len = a->ctx_len;
    L.q_pos0 = a->q_pos0; L.m = a->m; L.k = a->k; L.out = a->out_idx;
    return device_status(csa2::launch_prefill_topk(L, ws, as_stream(stream)), "csa2_prefill_topk");
}

// --------------------------------------------------------------------------
int csa2_mhc_step(const csa2_mhc_args* m, void* stream) {
    if (!m) return fail(CSA2_E_INVALID, "csa2_mhc_step: args is null");
    if (m->T < 0) return fail(CSA2_E_INVALID, "csa2_mhc_step: T < 0");
    if (m->n <= 0 || m->d <= 0) return fail(CSA2_E_INVALID, "csa2_mhc_step: n and d must be positive");
    if (m->iters < 0) return fail(CSA2_E_INVALID, "csa2_mhc_step: iters < 0");
    if (!csa2::mhc_shape_supported(m->n, m->d))
        return fail(CSA2_E_UNSUPPORTED, "csa2_mhc_step: (n=%d, d=%d) not supported (n = 4, d a multiple of 128)",
                    m->n, m->d);
    if (m->T == 0) return ok();
    if (!m->X || !m->f || !m->A || !m->B || !m->C || !m->phiT || !m->bias || !m->X_next || !m->u_next ||
        !m->A_next || !m->B_next || !m->C_next)
        return fail(CSA2_E_INVALID, "csa2_mhc_step: null pointer");
    if (!aligned(m->X, 16) || !aligned(m->f, 16) || !aligned(m->phiT, 16) || !aligned(m->X_next, 16) ||
        !aligned(m->u_next, 16))
        return fail(CSA2_E_INVALID, "csa2_mhc_step: X, f, phiT, X_next and u_next must be 16-byte aligned");
    if (m->X_next == m->X || m->u_next == m->f)
        return fail(CSA2_E_INVALID, "csa2_mhc_step: X_next and u_next must not alias X and f");
    csa2::MhcLaunch p;
    p.X = static_cast<const uint16_t*>(m->X); p.f = static_cast<const uint16_t*>(m->f);
    p.A = m->A; p.B = m->B; p.C = m->C;
    p.phiT = static_cast<const uint16_t*>(m->phiT); p.bias = m->bias;
    p.alpha_pre = m->alpha_pre; p.alpha_post = m->alpha_post; p.alpha_res = m->alpha_res;
    p.T = m->T; p.d = m->d; p.iters = m->iters;
    p.Xn = static_cast<uint16_t*>(m->X_next); p.u = static_cast<uint16_t*>(m->u_next);
    p.An = m->A_next; p.Bn = m->B_next; p.Cn = m->C_next;
    return device_status(csa2::launch_mhc_step(p, as_stream(stream)), "csa2_mhc_step");
}

}  // extern "C"
