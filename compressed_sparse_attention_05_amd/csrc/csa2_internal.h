// Internal declarations shared by the libcsa2 translation units (host side).
// Not part of the public ABI (include/csa2.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Launchers: return hipSuccess or the launch error.  Arguments are already
// validated by the entry points in csa2_api.hip.
// MXFP4 quantisation of n_rows rows plus (krows != NULL) the copy of their
// indexer-K rows (krow_bytes each) into the tiled indexer cache.
hipError_t launch_kv_write(const void* x, bool x_bf16, int64_t n_rows, int D, const int64_t* dst_row,
                           int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const void* krows,
                           int64_t krow_bytes, void* kcache, hipStream_t st);
// MXFP4 quantisation plus the indexer-K projection k = bf16(x . W) of the same
// rows into the tiled bfloat16 indexer cache, in one launch.
bool kv_project_shape_supported(int D, int d_I);
hipError_t launch_kv_write_project(const void* x, bool x_bf16, int64_t n_rows, int D, const int64_t* dst_row,
                                   int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const float* W,
                                   int d_I, void* kcache, hipStream_t st);

// Monotone 32-bit key of a score for the selections: strictly increasing
// in the score with -0 == +0; 0 is reserved for -inf (an empty slot).
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0xff800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct ScoreLaunch {
    const void* q_idx; bool q_bf16;
    const float* w;
    const void* k_idx; bool k_bf16;
    int64_t B, Tq, cap;
    int H_I, d_I;
    const int32_t* ctx_len;
    const int64_t* q_pos;
    int m;
    const int32_t* pool; int P_b;
    float* scores; int64_t ld;
    float* block_max; int64_t ld_bm;
    // decode write in the same launch (knew == nullptr: none; Tq == 1):
    // sequence b's MXFP4 row from wx[b] (wD channels) to flat row wdst[b]
    // of wcodes/wscales and its indexer key knew[b] into k_idx, skipped
    // unless wdst[b] lies in sequence b; its scores read the key from knew.
    const void* knew = nullptr;
    const void* wx = nullptr; bool wx_bf16 = false; int wD = 0;
    const int64_t* wdst = nullptr;
    uint8_t* wcodes = nullptr; uint8_t* wscales = nullptr;
};
bool score_shape_supported(int H_I, int d_I);
hipError_t launch_score(const ScoreLaunch& p, hipStream_t st);

size_t topk_workspace_bytes(int64_t rows, int64_t n);
// Full-mode top-k gathered through a candidate pool (k <= P_b, 8*P_b <= 32768).
hipError_t launch_topk_from_pool(const float* scores, int64_t rows, int64_t ld, const int32_t* pool, int P_b,
                                 int k, int32_t* out, hipStream_t st);
// Pool selection staged in LDS (directly, or through super-blocks of 8 blocks).
bool pool_in_lds(int64_t n_blocks, int P_b);
hipError_t launch_pool(const float* bmax, int64_t rows, int64_t n_blocks, int64_t ld, int P_b, int32_t* out,
                       hipStream_t st);
bool pool_topk_supported(int64_t n_blocks, int P_b, int k);
hipError_t launch_pool_topk(const float* bmax, int64_t rows, int64_t n_blocks, int64_t ld_bm, int P_b,
                            int32_t* pool, const float* scores, int64_t ld, int k, int32_t* out, hipStream_t st);
hipError_t launch_topk(const float* scores, int64_t rows, int64_t n, int64_t ld, int k,
                       const int32_t* pool, int P_b, int32_t* out, void* ws, hipStream_t st);

struct AttnLaunch {
    const void* q; bool q_bf16;
    const uint8_t* codes; const uint8_t* scales; int64_t cap;
    int64_t kv_unit_stride;      // cache rows between consecutive units (cap or 0)
    const int32_t* idx; int k;
    const void* swa; bool swa_bf16; int W;
    const int32_t* swa_len;      // decode: [units]; prefill: NULL
    int64_t q_pos0, swa_start;   // prefill window geometry
    bool prefill;
    int64_t units; int H, D;
    float sm_scale;
    float* out;
    float* ws; size_t ws_bytes;
};
bool attn_shape_supported(int H, int D);
size_t attn_workspace_bytes(int64_t units, int H, int D, int k, int W);
hipError_t launch_attn(const AttnLaunch& p, hipStream_t st);


// ---- prefill Full-mode top-k (matrix-core scores, exact band)
struct PrefillLaunch {
    const void* q;          // [T][8][128] bf16
    const float* w;         // [T][8]
    const void* k_idx;      // tiled bf16 indexer cache, cap rows
    int64_t T, cap;
    int32_t ctx_len;
    int64_t q_pos0;
    int32_t m;
    int32_t k;
    int32_t* out;           // [T][k]
};
size_t prefill_topk_workspace_bytes(int64_t T, int32_t ctx_len, int64_t q_pos0, int32_t m);
int prefill_topk_max_k();
// most visible entries a prefill chunk may have (a wave's 8 candidate rows
// stay one buffer range below 2^31 bytes)
int64_t prefill_topk_max_cols();
int64_t prefill_cols(int64_t T, int32_t ctx_len, int64_t q_pos0, int32_t m);
hipError_t launch_prefill_topk(const PrefillLaunch& L, void* ws, hipStream_t st);

struct DecodeSelectLaunch {
    const void* q_idx;      // [B][8][128] bf16
    const float* w;         // [B][8]
    const void* k_idx;      // tiled bf16 indexer cache, [B][cap]
    const int32_t* ctx_len; // [B] (device)
    int64_t B, cap;
    int32_t P_b, k;
    int32_t* out_pool;      // [B][P_b]
    int32_t* out_idx;       // [B][k]
};
bool decode_select_supported(int64_t cap, int H_I, int d_I, int P_b, int k);
size_t decode_select_workspace_bytes(int64_t B, int64_t cap);
hipError_t launch_decode_scan(const DecodeSelectLaunch& L, void* ws, hipStream_t st);
hipError_t launch_decode_select(const DecodeSelectLaunch& L, void* ws, hipStream_t st);

// ---- single-pass mHC block step (n = 4 streams, bfloat16 storage)
struct MhcLaunch {
    const uint16_t* X; const uint16_t* f;        // [T][4][d], [T][d] bf16
    const float* A; const float* B; const float* C;  // [T][4], [T][4][4], [T][4]
    const uint16_t* phiT; const float* bias;     // [24][4d] bf16, [24]
    float alpha_pre, alpha_post, alpha_res;
    int64_t T; int d; int iters;
    uint16_t* Xn; uint16_t* u;                   // [T][4][d], [T][d] bf16
    float* An; float* Bn; float* Cn;             // [T][4], [T][4][4], [T][4]
};
bool mhc_shape_supported(int n, int d);
hipError_t launch_mhc_step(const MhcLaunch& p, hipStream_t st);

}  // namespace csa2
