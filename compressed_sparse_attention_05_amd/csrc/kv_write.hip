// MXFP4 main-KV writer for gfx950 (the block format and its rounding rules
// are in mxfp4_quant.h).
//
// One thread per (row, 16-channel block), plus one per 16-byte chunk of the
// indexer-K rows: the work is a few hundred bytes per decode token, so the
// kernel is launch-bound and does both jobs in one launch.  A decode step
// whose first scan can absorb the write does it there instead (score.hip).
#include "csa2_internal.h"

namespace csa2 {
namespace {

#include "mxfp4_quant.h"

// Threads [0, n_rows*D/16) quantise one 16-channel block each; the next
// n_rows*nch threads copy one 16-byte chunk of an indexer-K row each into the
// tiled indexer cache (chunk c of flat row r at ((r/64)*nch + c)*64 + r%64,
// in 16-byte units).  One launch per write.
template <bool BF16>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const void* __restrict__ x, int64_t n_rows, int D, const int64_t* __restrict__ dst_row,
    int64_t n_cache_rows, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const uint4* __restrict__ krows, int nch, uint4* __restrict__ kcache) {
    const int nblk = D / 16;
    int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= n_rows * nblk) {
        gid -= n_rows * nblk;
        if (gid >= n_rows * nch) return;
        const int64_t row = gid / nch;
        const int c = static_cast<int>(gid % nch);
        const uint4 val = krows[row * nch + c];
        const int64_t r = dst_row[row];
        if (r < 0 || r >= n_cache_rows) return;
        kcache[((r >> 6) * nch + c) * 64 + (r & 63)] = val;
        return;
    }
    const int64_t row = gid / nblk;
    const int blk = static_cast<int>(gid % nblk);
    float v[16];
    load_block<BF16>(x, row, blk, D, v);           // issued together with the dst_row load
    const int64_t dst = dst_row[row];
    if (dst < 0 || dst >= n_cache_rows) return;
    quantise_block(v, blk, D, dst, codes, scales);
}

// ---------------------------------------------------------------------------
// Indexer-K projection fused into the write.  A Full layer derives its
// indexer key directly from its main KV ("DeepSeek-V4.1-Flash KV Cache
// Compression" notes, section 2); the pages give neither the weights nor the
// precision.  Here the key is the pre-quantisation latent row times float32
// weights W[D][d_I], each output an fma chain over the channels in order,
// rounded to the nearest bfloat16 (ties to even, never to infinity):
//     acc = +0; for c in 0..D-1: acc = fma(x[c], W[c][j], acc)
// Each output is a chain of D dependent fmas, so the design keeps every
// chain's operands in LDS and gives every thread exactly one chain: a
// workgroup of 32 ROWS threads owns ROWS rows x a slice of 32 output columns
// (ROWS = 8 for a decode batch, so its few rows still spread over many
// workgroups; 32 for a prefill chunk's entries, so each staged weight slice
// serves more rows).  It stages the latent rows (float32) and the weight
// slice, transposed to
// [column][channel] (rows padded by 16 bytes against bank conflicts), with
// whole-workgroup coalesced loads, then thread (r, j) runs its chain with two
// 16-byte LDS reads per four fmas.  The bfloat16 keys are restaged in LDS so
// every store is a whole 16-byte chunk of the tiled indexer cache.
constexpr int PROJ_COLS = 32;
constexpr int PROJ_DMAX = 512;
constexpr int PROJ_QTHREADS = 256;     // quantising workgroups use their first 256 threads

// bfloat16 nearest to a finite float (ties to the even mantissa).  A float
// past the largest bfloat16 by at least half an ulp stays at the largest
// finite value: the key is the nearest representable number, never infinity.
__device__ __forceinline__ uint16_t bf16_nearest_finite(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return ((r & 0x7f80u) == 0x7f80u) ? static_cast<uint16_t>(u >> 16) : static_cast<uint16_t>(r);
}

template <int ROWS>
struct ProjLds {
    float xs[ROWS][PROJ_DMAX];                 // latent rows (reused for the bf16 keys)
    float wt[PROJ_COLS][PROJ_DMAX + 4];        // W slice, [column][channel]
};

template <bool BF16, int ROWS>
__device__ __forceinline__ void project_slice(const void* __restrict__ x, int64_t n_rows, int D,
                                              const int64_t* __restrict__ dst_row, int64_t n_cache_rows,
                                              const float* __restrict__ W, int d_I, uint4* __restrict__ kcache,
                                              int64_t row0, int j0, ProjLds<ROWS>& sh) {
    constexpr int NT = ROWS * PROJ_COLS;
    const int tid = threadIdx.x;
    const int nr = static_cast<int>(min<int64_t>(ROWS, n_rows - row0));
    // weight slice: thread -> (channel, column quad); quads past d_I are zero
    for (int i = tid; i < D * (PROJ_COLS / 4); i += NT) {
        const int c = i >> 3, g = i & 7;
        const int j = j0 + 4 * g;
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (j < d_I) v = *reinterpret_cast<const float4*>(W + static_cast<int64_t>(c) * d_I + j);
        sh.wt[4 * g][c] = v.x; sh.wt[4 * g + 1][c] = v.y; sh.wt[4 * g + 2][c] = v.z; sh.wt[4 * g + 3][c] = v.w;
    }
    // latent rows, widened to float32 (rows past the end read as zero)
    for (int i = tid; i < ROWS * (D / 8); i += NT) {
        const int r = i / (D / 8), c = (i - r * (D / 8)) * 8;
        float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (r < nr) {
            const int64_t g = (row0 + r) * D + c;
            if (BF16) {
                const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + g);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = __uint_as_float(ww[e] << 16);
                    v[2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
                }
            } else {
                const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + g);
                const float4 a = p[0], b = p[1];
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            }
        }
        *reinterpret_cast<float4*>(&sh.xs[r][c]) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(&sh.xs[r][c + 4]) = make_float4(v[4], v[5], v[6], v[7]);
    }
    __syncthreads();
    // one chain per thread: row r, column j0 + jj
    const int r = tid >> 5, jj = tid & 31;
    float acc = 0.0f;
#pragma unroll 4
    for (int c = 0; c < D; c += 4) {
        const float4 xv = *reinterpret_cast<const float4*>(&sh.xs[r][c]);
        const float4 wv = *reinterpret_cast<const float4*>(&sh.wt[jj][c]);
        acc = __builtin_fmaf(xv.x, wv.x, acc);
        acc = __builtin_fmaf(xv.y, wv.y, acc);
        acc = __builtin_fmaf(xv.z, wv.z, acc);
        acc = __builtin_fmaf(xv.w, wv.w, acc);
    }
    __syncthreads();                    // every chain is done reading xs: reuse it for the keys
    uint16_t* ks = reinterpret_cast<uint16_t*>(&sh.xs[0][0]);     // [ROWS][PROJ_COLS]
    ks[r * PROJ_COLS + jj] = bf16_nearest_finite(acc);
    __syncthreads();
    const int nch = d_I / 8;
    if (tid < ROWS * (PROJ_COLS / 8)) {
        const int rr = tid >> 2, q = tid & 3;
        const int ch = j0 / 8 + q;
        if (rr < nr && ch < nch) {
            const int64_t dst = dst_row[row0 + rr];
            if (dst >= 0 && dst < n_cache_rows)
                kcache[((dst >> 6) * nch + ch) * 64 + (dst & 63)] =
                    *reinterpret_cast<const uint4*>(ks + rr * PROJ_COLS + 8 * q);
        }
    }
}

// One launch: workgroups [0, nq) quantise 256 (row, block) units each (with
// their first 256 threads), the rest project one (ROWS-row, 32-column) tile
// each: tile pb covers rows ROWS (pb / ncs) and columns 32 (pb % ncs).
template <bool BF16, int ROWS>
__global__ __launch_bounds__(ROWS * PROJ_COLS) void kv_write_project_kernel(
    const void* __restrict__ x, int64_t n_rows, int D, const int64_t* __restrict__ dst_row,
    int64_t n_cache_rows, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const float* __restrict__ W, int d_I, uint4* __restrict__ kcache, int64_t nq, int ncs) {
    __shared__ __attribute__((aligned(16))) ProjLds<ROWS> sh;
    if (blockIdx.x < nq) {
        if (threadIdx.x >= PROJ_QTHREADS) return;
        const int nblk = D / 16;
        const int64_t gid = static_cast<int64_t>(blockIdx.x) * PROJ_QTHREADS + threadIdx.x;
        if (gid >= n_rows * nblk) return;
        const int64_t row = gid / nblk;
        const int blk = static_cast<int>(gid % nblk);
        float v[16];
        load_block<BF16>(x, row, blk, D, v);
        const int64_t dst = dst_row[row];
        if (dst < 0 || dst >= n_cache_rows) return;
        quantise_block(v, blk, D, dst, codes, scales);
        return;
    }
    const int64_t pb = static_cast<int64_t>(blockIdx.x) - nq;
    const int64_t row0 = (pb / ncs) * ROWS;
    const int j0 = static_cast<int>(pb % ncs) * PROJ_COLS;
    project_slice<BF16, ROWS>(x, n_rows, D, dst_row, n_cache_rows, W, d_I, kcache, row0, j0, sh);
}

}  // namespace

hipError_t launch_kv_write(const void* x, bool x_bf16, int64_t n_rows, int D, const int64_t* dst_row,
                           int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const void* krows,
                           int64_t krow_bytes, void* kcache, hipStream_t st) {
    const int nch = krows ? static_cast<int>(krow_bytes / 16) : 0;
    const int64_t n = n_rows * (D / 16) + n_rows * nch;
    if (n == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((n + 255) / 256));
    const uint4* kr = static_cast<const uint4*>(krows);
    uint4* kc = static_cast<uint4*>(kcache);
    if (x_bf16)
        kv_write_kernel<true><<<grid, 256, 0, st>>>(x, n_rows, D, dst_row, n_cache_rows, codes, scales, kr, nch, kc);
    else
        kv_write_kernel<false><<<grid, 256, 0, st>>>(x, n_rows, D, dst_row, n_cache_rows, codes, scales, kr, nch, kc);
    return hipGetLastError();
}

}  // namespace csa2

namespace csa2 {

bool kv_project_shape_supported(int D, int d_I) {
    return D % 16 == 0 && D > 0 && D <= PROJ_DMAX && d_I % 8 == 0 && d_I > 0;
}

template <int ROWS>
static hipError_t launch_project(const void* x, bool x_bf16, int64_t n_rows, int D, const int64_t* dst_row,
                                 int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const float* W, int d_I,
                                 void* kcache, hipStream_t st) {
    const int64_t nq = (n_rows * (D / 16) + PROJ_QTHREADS - 1) / PROJ_QTHREADS;
    const int ncs = (d_I + PROJ_COLS - 1) / PROJ_COLS;
    const int64_t np = (n_rows + ROWS - 1) / ROWS * ncs;
    const dim3 grid(static_cast<unsigned>(nq + np));
    uint4* kc = static_cast<uint4*>(kcache);
    if (x_bf16)
        kv_write_project_kernel<true, ROWS><<<grid, ROWS * PROJ_COLS, 0, st>>>(x, n_rows, D, dst_row, n_cache_rows,
                                                                               codes, scales, W, d_I, kc, nq, ncs);
    else
        kv_write_project_kernel<false, ROWS><<<grid, ROWS * PROJ_COLS, 0, st>>>(x, n_rows, D, dst_row, n_cache_rows,
                                                                                codes, scales, W, d_I, kc, nq, ncs);
    return hipGetLastError();
}

hipError_t launch_kv_write_project(const void* x, bool x_bf16, int64_t n_rows, int D, const int64_t* dst_row,
                                   int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const float* W,
                                   int d_I, void* kcache, hipStream_t st) {
    if (n_rows == 0) return hipSuccess;
    if (n_rows <= 512)
        return launch_project<8>(x, x_bf16, n_rows, D, dst_row, n_cache_rows, codes, scales, W, d_I, kcache, st);
    return launch_project<32>(x, x_bf16, n_rows, D, dst_row, n_cache_rows, codes, scales, W, d_I, kcache, st);
}

}  // namespace csa2
