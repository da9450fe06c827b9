// MXFP4 main-KV writer for gfx950.
//
// Format ("DeepSeek-V4.1-Flash KV Cache Compression" notes, section 4; summary
// page, Methodology item 5): per block of 16 channels one E4M3 (OCP FN) scale
// byte and 16 E2M1 nibbles, no second-level scale.  scale = E4M3 nearest to
// amax/6 (ties to even, saturating at 448); element = E2M1 nearest to
// |x|/scale (ties to even, saturating at 6).  Every decision below is an
// exact float32 comparison against a threshold that float32 holds exactly,
// so the bytes are reproducible on any device.
//
// One thread per (row, 16-channel block), plus one per 16-byte chunk of the
// indexer-K rows: the work is a few hundred bytes per decode token, so the
// kernel is launch-bound and does both jobs in one launch.
#include "csa2_internal.h"

namespace csa2 {
namespace {

// Value of a non-negative finite E4M3 code (0..126), exact in float32.
__device__ __forceinline__ float e4m3_nonneg(int c) {
    return (c < 8) ? static_cast<float>(c) * 0x1p-9f
                   : __uint_as_float((static_cast<uint32_t>(c) << 20) + (120u << 23));
}

// Nearest E4M3 code to amax/6, ties to even, saturating at 126 (448).
// Binary search for the largest code c with 6*v(c) <= amax (6*v(c) is exact),
// then the tie/round decision against 3*(v(c) + v(c+1)) (also exact).
__device__ __forceinline__ int scale_code(float amax) {
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (6.0f * e4m3_nonneg(mid) <= amax) lo = mid; else hi = mid - 1;
    }
    if (lo == 126) return 126;
    float t = 3.0f * (e4m3_nonneg(lo) + e4m3_nonneg(lo + 1));
    if (amax > t) return lo + 1;
    if (amax == t) return (lo & 1) ? lo + 1 : lo;
    return lo;
}

// E2M1 magnitude code (0..7) nearest to a/s: count the midpoints a exceeds,
// and at an exact midpoint pick the even code (midpoints 0.75, 1.75, 3.5
// round up to codes 2, 4, 6; 0.25, 1.25, 2.5, 5 round down to 0, 2, 4, 6).
__device__ __forceinline__ uint32_t mag_code(float a, float s) {
    const float t0 = s * 0.25f, t1 = s * 0.75f, t2 = s * 1.25f, t3 = s * 1.75f;
    const float t4 = s * 2.5f, t5 = s * 3.5f, t6 = s * 5.0f;
    uint32_t c = (a > t0) + (a > t1) + (a > t2) + (a > t3) + (a > t4) + (a > t5) + (a > t6);
    c += (a == t1) + (a == t3) + (a == t5);
    return c;
}

// Quantise block `blk` (16 channels) of input row `row` into flat cache row
// `dst`: scale byte, then eight code bytes (channel 2j in the low nibble).
template <bool BF16>
__device__ __forceinline__ void quantise_block(const void* __restrict__ x, int64_t row, int blk, int D,
                                               int64_t dst, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales) {
    const int nblk = D / 16;
    float v[16];
    if (BF16) {
        const uint4* p = reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(x) + row * D + blk * 16);
        uint4 a = p[0], b = p[1];
        uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(
            static_cast<const float*>(x) + row * D + blk * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 f = p[i];
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int sc = scale_code(amax);
    uint32_t lo = 0, hi = 0;
    if (sc != 0) {
        const float s = e4m3_nonneg(sc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t c = mag_code(fabsf(v[i]), s);
            if (v[i] < 0.0f && c != 0) c |= 8u;
            if (i < 8) lo |= c << (4 * i); else hi |= c << (4 * (i - 8));
        }
    }
    uint2* cp = reinterpret_cast<uint2*>(codes + dst * (D / 2) + blk * 8);
    *cp = make_uint2(lo, hi);
    scales[dst * nblk + blk] = static_cast<uint8_t>(sc);
}

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
        const int64_t r = dst_row[row];
        if (r < 0 || r >= n_cache_rows) return;
        kcache[((r >> 6) * nch + c) * 64 + (r & 63)] = krows[row * nch + c];
        return;
    }
    const int64_t row = gid / nblk;
    const int blk = static_cast<int>(gid % nblk);
    const int64_t dst = dst_row[row];
    if (dst < 0 || dst >= n_cache_rows) return;
    quantise_block<BF16>(x, row, blk, D, dst, codes, scales);
}

// ---------------------------------------------------------------------------
// Indexer-K projection fused into the write.  A Full layer derives its
// indexer key directly from its main KV ("DeepSeek-V4.1-Flash KV Cache
// Compression" notes, section 2); the pages give neither the weights nor the
// precision.  Here the key is the pre-quantisation latent row times float32
// weights W[D][d_I], each output an fma chain over the channels in order,
// rounded to the nearest bfloat16 (ties to even, never to infinity):
//     acc = +0; for c in 0..D-1: acc = fma(x[c], W[c][j], acc)
// A workgroup takes 2*RPT rows: their latent rows sit in LDS as float32, and
// each thread runs the chains of one column j for RPT rows (broadcast LDS
// reads of x; one coalesced read of W[c][j] per channel serves RPT fmas).  The
// weights stream through a ring of PF_BLOCKS register blocks of 16 channels,
// so 64 channels of loads are in flight while a block is consumed.  RPT = 1
// for a decode token's few rows (many workgroups, short critical path), 8 for
// a prefill chunk's thousands.  The bfloat16 results are restaged in LDS so
// every store is a whole 16-byte chunk of the tiled indexer cache.
constexpr int PROJ_THREADS = 256;
constexpr int PROJ_CB = 16;       // channels per register block
constexpr int PROJ_PF = 4;        // blocks in flight
constexpr int PROJ_MAX_RPT = 8;

// bfloat16 nearest to a finite float (ties to the even mantissa).  A float
// past the largest bfloat16 by at least half an ulp stays at the largest
// finite value: the key is the nearest representable number, never infinity.
__device__ __forceinline__ uint16_t bf16_nearest_finite(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return ((r & 0x7f80u) == 0x7f80u) ? static_cast<uint16_t>(u >> 16) : static_cast<uint16_t>(r);
}

__device__ __forceinline__ void load_wblock(float (&w)[PROJ_CB], const float* __restrict__ W, int c, int D,
                                            int d_I, int j) {
    if (c < D) {
#pragma unroll
        for (int i = 0; i < PROJ_CB; ++i) w[i] = W[static_cast<int64_t>(c + i) * d_I + j];
    }
}

template <bool BF16, int RPT>
__device__ __forceinline__ void project_rows(const void* __restrict__ x, int64_t n_rows, int D,
                                             const int64_t* __restrict__ dst_row, int64_t n_cache_rows,
                                             const float* __restrict__ W, int d_I, uint4* __restrict__ kcache,
                                             int64_t row0, float* xs) {
    constexpr int ROWS = 2 * RPT;
    const int tid = threadIdx.x;
    const int nr = static_cast<int>(min<int64_t>(ROWS, n_rows - row0));
    // Stage the rows as float32 (missing rows of a last group read as zero).
    for (int i = tid; i < ROWS * D; i += PROJ_THREADS) {
        const int r = i / D, c = i - r * D;
        float v = 0.0f;
        if (r < nr) {
            const int64_t g = (row0 + r) * D + c;
            v = BF16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(x)[g]) << 16)
                     : static_cast<const float*>(x)[g];
        }
        xs[i] = v;
    }
    __syncthreads();
    // Unit u: column j = u % d_I, rows (u / d_I)*RPT .. +RPT-1.  Results go to
    // the bfloat16 tile ks [ROWS][d_I] behind the staged rows.
    uint16_t* ks = reinterpret_cast<uint16_t*>(xs + ROWS * D);
    for (int u = tid; u < d_I * 2; u += PROJ_THREADS) {
        const int j = u % d_I, g = u / d_I;
        const float* xr = xs + g * RPT * D;
        float acc[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) acc[r] = 0.0f;
        float wr[PROJ_PF][PROJ_CB];
#pragma unroll
        for (int b = 0; b < PROJ_PF; ++b) load_wblock(wr[b], W, b * PROJ_CB, D, d_I, j);
        for (int c0 = 0; c0 < D; c0 += PROJ_PF * PROJ_CB) {
#pragma unroll
            for (int b = 0; b < PROJ_PF; ++b) {
                const int c = c0 + b * PROJ_CB;
                if (c < D) {
#pragma unroll
                    for (int r = 0; r < RPT; ++r) {
                        float a = acc[r];
#pragma unroll
                        for (int q = 0; q < PROJ_CB / 4; ++q) {
                            const float4 xv = *reinterpret_cast<const float4*>(xr + r * D + c + 4 * q);
                            a = __builtin_fmaf(xv.x, wr[b][4 * q], a);
                            a = __builtin_fmaf(xv.y, wr[b][4 * q + 1], a);
                            a = __builtin_fmaf(xv.z, wr[b][4 * q + 2], a);
                            a = __builtin_fmaf(xv.w, wr[b][4 * q + 3], a);
                        }
                        acc[r] = a;
                    }
                    load_wblock(wr[b], W, c + PROJ_PF * PROJ_CB, D, d_I, j);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r) ks[(g * RPT + r) * d_I + j] = bf16_nearest_finite(acc[r]);
    }
    __syncthreads();
    const int nch = d_I / 8;
    for (int i = tid; i < nr * nch; i += PROJ_THREADS) {
        const int r = i / nch, ch = i - r * nch;
        const int64_t dst = dst_row[row0 + r];
        if (dst < 0 || dst >= n_cache_rows) continue;
        kcache[((dst >> 6) * nch + ch) * 64 + (dst & 63)] =
            *reinterpret_cast<const uint4*>(ks + r * d_I + ch * 8);
    }
}

// One launch: workgroups [0, nq) quantise 256 (row, block) units each, the
// rest project 2*RPT rows each.
template <bool BF16, int RPT>
__global__ __launch_bounds__(PROJ_THREADS) void kv_write_project_kernel(
    const void* __restrict__ x, int64_t n_rows, int D, const int64_t* __restrict__ dst_row,
    int64_t n_cache_rows, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const float* __restrict__ W, int d_I, uint4* __restrict__ kcache, int64_t nq) {
    extern __shared__ float xs[];
    if (blockIdx.x < nq) {
        const int nblk = D / 16;
        const int64_t gid = static_cast<int64_t>(blockIdx.x) * PROJ_THREADS + threadIdx.x;
        if (gid >= n_rows * nblk) return;
        const int64_t row = gid / nblk;
        const int blk = static_cast<int>(gid % nblk);
        const int64_t dst = dst_row[row];
        if (dst < 0 || dst >= n_cache_rows) return;
        quantise_block<BF16>(x, row, blk, D, dst, codes, scales);
        return;
    }
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) - nq) * (2 * RPT);
    project_rows<BF16, RPT>(x, n_rows, D, dst_row, n_cache_rows, W, d_I, kcache, row0, xs);
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

size_t kv_project_lds_bytes(int D, int d_I, int rpt) {
    return static_cast<size_t>(2 * rpt) * D * sizeof(float) + static_cast<size_t>(2 * rpt) * d_I * 2;
}

bool kv_project_shape_supported(int D, int d_I) {
    return D % 16 == 0 && D > 0 && d_I % 8 == 0 && d_I > 0 && kv_project_lds_bytes(D, d_I, PROJ_MAX_RPT) <= 65536;
}

template <int RPT>
static hipError_t launch_project(const void* x, bool x_bf16, int64_t n_rows, int D, const int64_t* dst_row,
                                 int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const float* W, int d_I,
                                 void* kcache, hipStream_t st) {
    const int64_t nq = (n_rows * (D / 16) + PROJ_THREADS - 1) / PROJ_THREADS;
    const int64_t np = (n_rows + 2 * RPT - 1) / (2 * RPT);
    const dim3 grid(static_cast<unsigned>(nq + np));
    const size_t lds = kv_project_lds_bytes(D, d_I, RPT);
    uint4* kc = static_cast<uint4*>(kcache);
    if (x_bf16)
        kv_write_project_kernel<true, RPT><<<grid, PROJ_THREADS, lds, st>>>(x, n_rows, D, dst_row, n_cache_rows,
                                                                            codes, scales, W, d_I, kc, nq);
    else
        kv_write_project_kernel<false, RPT><<<grid, PROJ_THREADS, lds, st>>>(x, n_rows, D, dst_row, n_cache_rows,
                                                                             codes, scales, W, d_I, kc, nq);
    return hipGetLastError();
}

// A few rows (a decode token's batch): one row per thread, many workgroups.
// Thousands (a prefill chunk's entries): eight rows per thread, so each
// weight read serves eight fmas.
hipError_t launch_kv_write_project(const void* x, bool x_bf16, int64_t n_rows, int D, const int64_t* dst_row,
                                   int64_t n_cache_rows, uint8_t* codes, uint8_t* scales, const float* W,
                                   int d_I, void* kcache, hipStream_t st) {
    if (n_rows == 0) return hipSuccess;
    if (n_rows <= 1024)
        return launch_project<1>(x, x_bf16, n_rows, D, dst_row, n_cache_rows, codes, scales, W, d_I, kcache, st);
    return launch_project<PROJ_MAX_RPT>(x, x_bf16, n_rows, D, dst_row, n_cache_rows, codes, scales, W, d_I,
                                        kcache, st);
}

}  // namespace csa2
