// The decode Full layer's candidate pool and top-k with the indexer products
// on the matrix cores ("DeepSeek-V4.1-Flash KV Cache Compression" notes,
// sections 2-3: the Full layer scores every visible entry, builds the pool of
// the 2,048 best 8-entry blocks by block max, and takes its top-k).
//
// The indices and the pool must equal those chosen from the exact score
// (float32 fma chains over channels, then heads, in order).  As for prefill:
//  1. dscan_kernel computes s~ = sum_h w_h ReLU(q_h . k_j) with
//     v_mfma_f32_16x16x32_bf16 (A = the 8 heads' q rows, B = 16 keys), its
//     block maxima bm~ and the row's largest key norm Kmax.  With
//     A_t = sum_h |w_h| ||q_h||, every |s~_j - s_j| <= eps_t =
//     kEpsRel * A_t * Kmax + (underflow term): the bound of the prefill path
//     (bf16 products exact in float32, any-order float32 sums within
//     gamma_128 of the real value, Cauchy-Schwarz, ReLU 1-Lipschitz).  A
//     block max is 1-Lipschitz in the sup norm, so |bm~_b - bm_b| <= eps_t.
//  2. dselect_kernel, one workgroup per row:
//     pool: with tau~ the P_b-th largest bm~, blocks with bm~ > tau~ + 2 eps
//       are in the exact pool and blocks below tau~ - 2 eps are not (the
//       exact P_b-th block max is within eps of tau~); the blocks in between
//       get their exact block max from exact scores of their 8 positions and
//       fill the remaining places by (exact block max desc, block id asc);
//     top-k: the same argument over the pool's 8 * P_b positions with s~,
//       the band rescored exactly and ranked by (exact score desc, position
//       asc).  The Full top-k lies inside the exact pool (k <= P_b), so this
//       is the top-k of the whole row.
//     Every exact tie at either threshold lies in its band, so ties resolve
//     as in the definition.  A row whose band overflows its LDS budget is
//     redone from exact scores of the whole row (same result, slower).
#include "csa2_internal.h"

namespace csa2 {
namespace {
#include "select_util.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kHeads = 8, kDim = 128;
constexpr int kNch = kDim * 2 / 16;               // 16-byte chunks per indexer row
constexpr float kEpsRel = 4.0e-5f;
constexpr int kBandBlocks = 512;                  // pool band rescored exactly
constexpr int kBandPos = 2048;                    // top-k band rescored exactly
constexpr int kPoolCap = 2048;                    // largest P_b
constexpr int kScanThreads = 256;

struct DsArgs {
    const uint16_t* q;        // [B][8][128] bf16
    const float* w;           // [B][8]
    const uint8_t* kc;        // tiled indexer cache, cap rows per sequence (bf16)
    const int32_t* ctx_len;   // [B]
    int64_t cap;
    int64_t B;
    float* st;                // [B][cap] approximate (or, after a fallback, exact) scores
    float* bm;                // [B][nb]
    float* kmax;              // [B][nwg] largest squared key norm per scan workgroup
    int64_t nwg;              // scan workgroups per row
    int64_t nb;               // blocks per row = cap / 8
    int32_t P_b, k;
    int32_t* pool;            // [B][P_b]
    int32_t* idx;             // [B][k]
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float float_of_key(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}
__device__ __forceinline__ float next_up(float x) {
    if (x != x || x == __builtin_inff()) return x;
    if (x == 0.0f) return __uint_as_float(1u);
    const uint32_t u = __float_as_uint(x);
    return __uint_as_float(x > 0.0f ? u + 1u : u - 1u);
}
__device__ __forceinline__ float next_down(float x) { return -next_up(-x); }
__device__ __forceinline__ const uint4* kchunk(const uint8_t* kc, int64_t pos, int c) {
    return reinterpret_cast<const uint4*>(kc) + ((pos >> 6) * kNch + c) * 64 + (pos & 63);
}
__device__ __forceinline__ int64_t vis_of(const DsArgs& a, int64_t b) {
    const int64_t v = a.ctx_len[b];
    return v < a.cap ? (v > 0 ? v : 0) : a.cap;
}

// ---------------------------------------------------------------- scan
// Workgroup = 4 waves; wave w of workgroup (x, row) takes the 64-key cache
// tile 4x + w.  Per 16-key block j: lane l loads chunk 4s + l/16 of key
// 16j + l%16 for k-steps s = 0..3 (the B operand: channels 32s + 8(l/16) ..
// +7 of that key), and the four MFMAs give C[head][key] with lane l holding
// heads 4(l/16) + i of key l%16 (lanes >= 32: heads 8..15, all zero).
__global__ __launch_bounds__(kScanThreads) void dscan_kernel(DsArgs a) {
    __shared__ float wmax[kScanThreads / 64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = blockIdx.y;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + wv;
    const int64_t vis = vis_of(a, row);
    float nmax = 0.0f;
    if (tile * 64 < a.cap) {
    const uint8_t* kc = a.kc + row * a.cap * (kDim * 2);
    // A operand: q[head l%16][channels 32s + 8(l/16) .. +7], zero for heads >= 8
    bf16x8 qa[4];
    {
        const int h = lane & 15;
        const uint16_t* qr = a.q + (row * kHeads + (h < kHeads ? h : 0)) * kDim + 8 * (lane >> 4);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v = *reinterpret_cast<const uint4*>(qr + 32 * s);
            if (h >= kHeads) v = make_uint4(0u, 0u, 0u, 0u);
            qa[s] = __builtin_bit_cast(bf16x8, v);
        }
    }
    float wr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[i] = lane < 32 ? a.w[row * kHeads + 4 * (lane >> 4) + i] : 0.0f;
    // all 16 loads of the tile first (tile rows are always inside the cache)
    uint4 kv[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) kv[j][s] = *kchunk(kc, tile * 64 + 16 * j + (lane & 15), 4 * s + (lane >> 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        float ss = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, kv[j][s]), acc, 0, 0, 0);
            const uint32_t u[4] = {kv[j][s].x, kv[j][s].y, kv[j][s].z, kv[j][s].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ss = fmaf(bf16_lo(u[e]), bf16_lo(u[e]), ss);
                ss = fmaf(bf16_hi(u[e]), bf16_hi(u[e]), ss);
            }
        }
        // squared norm of key l%16: its four 32-channel parts sit in lanes
        // l, l^16, l^32, l^48
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        nmax = fmaxf(nmax, ss);
        // s~ of key l%16: heads 0..3 in lane l%16, heads 4..7 in lane l%16 + 16
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) p = fmaf(wr[i], fmaxf(acc[i], 0.0f), p);
        p += __shfl_xor(p, 16);
        const int64_t pos = tile * 64 + 16 * j + (lane & 15);
        const float v = pos < vis ? p : -__builtin_inff();
        if (lane < 16) a.st[row * a.cap + pos] = v;
        float mx = v;
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        mx = fmaxf(mx, __shfl_xor(mx, 4));
        if (mx == 0.0f) mx = 0.0f;
        if (lane < 16 && (lane & 7) == 0) a.bm[row * a.nb + (pos >> 3)] = mx;
    }
    // largest squared norm over the tile's keys (a tile with no visible key
    // does not count; its invisible keys only loosen the bound otherwise)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) nmax = fmaxf(nmax, __shfl_xor(nmax, off));
    if (tile * 64 >= vis) nmax = 0.0f;
    }
    // one slot per workgroup (no atomics: a whole row's workgroups would
    // otherwise queue on one address)
    if (lane == 0) wmax[wv] = nmax;
    __syncthreads();
    if (threadIdx.x == 0)
        a.kmax[row * a.nwg + blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// ---------------------------------------------------------------- select
// exact score of key row pos (q, w staged as float32 in LDS)
__device__ float exact_score(const float* qf, const float* wf, const uint8_t* kc, int64_t pos) {
    float d[kHeads];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) d[h] = 0.0f;
    for (int c = 0; c < kNch; ++c) {
        const uint4 v = *kchunk(kc, pos, c);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float k0 = bf16_lo(u[e]), k1 = bf16_hi(u[e]);
            const int ch = 8 * c + 2 * e;
#pragma unroll
            for (int h = 0; h < kHeads; ++h) {
                d[h] = fmaf(qf[h * kDim + ch], k0, d[h]);
                d[h] = fmaf(qf[h * kDim + ch + 1], k1, d[h]);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < kHeads; ++h) s = fmaf(wf[h], d[h] > 0.0f ? d[h] : 0.0f, s);
    return s;
}

struct SelectLds {
    SelLds sh;
    float qf[kHeads * kDim];
    float wf[kHeads];
    float eps;
    float kmax2;                       // largest squared key norm of the row
    uint32_t flags;                    // bit 0: fall back to exact scores
    uint32_t n_band;
    int32_t pool_s[kPoolCap];
    uint64_t band[kBandPos];           // (~exact key << 32) | id
    uint32_t band_key[kBandBlocks];    // exact block-max keys of band blocks
    uint32_t chosen[1024];             // bitmap: chosen band blocks / pool slots (32,768 bits)
};

__device__ __forceinline__ bool bit_of(const uint32_t* bm, int64_t i) { return (bm[i >> 5] >> (i & 31)) & 1u; }

// rank of band entry i among n distinct entries (ascending order of the
// 64-bit values = descending exact key, then ascending id)
__device__ __forceinline__ uint32_t band_rank(const uint64_t* band, uint32_t n, uint32_t i) {
    const uint64_t x = band[i];
    uint32_t r = 0;
    for (uint32_t j = 0; j < n; ++j) r += band[j] < x;
    return r;
}

template <int R1>
__global__ __launch_bounds__(kThreads) void dselect_kernel(DsArgs a) {
    __shared__ SelectLds L;
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t vis = vis_of(a, row);
    const uint8_t* kc = a.kc + row * a.cap * (kDim * 2);
    float* st = a.st + row * a.cap;
    float* bmr = a.bm + row * a.nb;
    int32_t* po = a.pool + row * static_cast<int64_t>(a.P_b);
    int32_t* o = a.idx + row * static_cast<int64_t>(a.k);
    const int P_b = a.P_b, k = a.k;
    const int64_t nbv = (vis + 7) / 8;                 // blocks with a visible position

    for (int i = tid; i < kHeads * kDim; i += kThreads)
        L.qf[i] = __uint_as_float(static_cast<uint32_t>(a.q[row * kHeads * kDim + i]) << 16);
    if (tid < kHeads) L.wf[tid] = a.w[row * kHeads + tid];
    if (tid == 0) L.flags = 0u;
    {
        // Kmax^2: the largest of the row's scan-workgroup slots
        float m = 0.0f;
        for (int64_t i = tid; i < a.nwg; i += kThreads) m = fmaxf(m, a.kmax[row * a.nwg + i]);
        for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
        if ((tid & 63) == 0) L.sh.wave_max[tid >> 6] = __float_as_uint(m);
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t m = 0u;
        for (int i = 0; i < kWaves; ++i) m = L.sh.wave_max[i] > m ? L.sh.wave_max[i] : m;
        L.kmax2 = __uint_as_float(m);
    }
    __syncthreads();
    if (tid < 64) {
        // eps_t from ||q_h|| (lanes 0..7), |w| and the row's Kmax
        float qn = 0.0f, wa = 0.0f;
        if (tid < kHeads) {
            float ss = 0.0f;
            for (int c = 0; c < kDim; ++c) ss = fmaf(L.qf[tid * kDim + c], L.qf[tid * kDim + c], ss);
            wa = fabsf(L.wf[tid]);
            qn = wa * sqrtf(ss);
        }
        for (int off = 1; off < 8; off <<= 1) {
            qn += __shfl_xor(qn, off);
            wa += __shfl_xor(wa, off);
        }
        if (tid == 0) {
            // the squared norm was summed in float32 (relative error far
            // below 2^-10): widen before the square root
            const float km = sqrtf(L.kmax2 * (1.0f + 0x1p-10f));
            L.eps = next_up(kEpsRel * qn * km + 0x1p-90f * km * wa + 0x1p-120f);
        }
    }
    for (int i = tid; i < 1024; i += kThreads) L.chosen[i] = 0u;
    __syncthreads();
    const float e2 = 2.0f * L.eps;

    // ------------------------------------------------ pool
    bool fallback = false;
    {
        const int64_t r0 = static_cast<int64_t>(tid) * R1;
        uint32_t kk[R1];
#pragma unroll
        for (int j = 0; j < R1; ++j) kk[j] = (r0 + j < a.nb) ? key_of(bmr[r0 + j]) : 0u;
        uint32_t TB = 0u, needB = 0u;
        uint32_t hi = 0u;
        if (nbv > P_b) {
            kth_key<R1>(kk, static_cast<uint32_t>(P_b), L.sh, TB, needB);
            const float tau = float_of_key(TB);
            hi = key_of(next_up(tau + e2));
            const uint32_t lo_raw = key_of(next_down(tau - e2));
            const uint32_t lo = lo_raw > 0u ? lo_raw : 1u;
            if (tid == 0) L.n_band = 0u;
            __syncthreads();
            uint32_t n_sure = 0;
#pragma unroll
            for (int j = 0; j < R1; ++j) {
                n_sure += kk[j] > hi;
                if (kk[j] != 0u && kk[j] >= lo && kk[j] <= hi) {
                    const uint32_t at = atomicAdd(&L.n_band, 1u);
                    if (at < static_cast<uint32_t>(kBandBlocks)) {
                        L.band[at] = static_cast<uint64_t>(r0 + j);
                        L.band_key[at] = 0u;
                    }
                }
            }
            uint32_t tot;
            block_excl_scan(n_sure, L.sh.wave_tot, tot);
            const uint32_t nband = L.n_band;
            if (nband > static_cast<uint32_t>(kBandBlocks) || tot >= static_cast<uint32_t>(P_b) ||
                tot + nband < static_cast<uint32_t>(P_b)) {
                fallback = true;
            } else {
                // exact block maxima of the band blocks: 8 positions each
                for (uint32_t i = tid; i < 8u * nband; i += kThreads) {
                    const int64_t blk = static_cast<int64_t>(L.band[i >> 3]);
                    const int64_t pos = blk * 8 + (i & 7);
                    const uint32_t ek = pos < vis ? key_of(exact_score(L.qf, L.wf, kc, pos)) : 0u;
                    atomicMax(&L.band_key[i >> 3], ek);
                }
                __syncthreads();
                for (uint32_t i = tid; i < nband; i += kThreads)
                    L.band[i] = (static_cast<uint64_t>(~L.band_key[i]) << 32) | L.band[i];
                __syncthreads();
                const uint32_t need_b = static_cast<uint32_t>(P_b) - tot;
                for (uint32_t i = tid; i < nband; i += kThreads) {
                    if (band_rank(L.band, nband, i) < need_b) {
                        const uint32_t blk = static_cast<uint32_t>(L.band[i]);
                        atomicOr(&L.chosen[blk >> 5], 1u << (blk & 31));
                    }
                }
                __syncthreads();
            }
        }
        if (!fallback) {
            // ordered emission of the pool (thread order = block order)
            uint32_t mine = 0;
#pragma unroll
            for (int j = 0; j < R1; ++j) {
                const bool take = nbv <= P_b ? (r0 + j < nbv) : (kk[j] > hi || bit_of(L.chosen, r0 + j));
                mine += take;
            }
            uint32_t tot;
            uint32_t at = block_excl_scan(mine, L.sh.wave_tot, tot);
#pragma unroll
            for (int j = 0; j < R1; ++j) {
                const bool take = nbv <= P_b ? (r0 + j < nbv) : (kk[j] > hi || bit_of(L.chosen, r0 + j));
                if (take) {
                    if (at < static_cast<uint32_t>(P_b)) {
                        po[at] = static_cast<int32_t>(r0 + j);
                        L.pool_s[at] = static_cast<int32_t>(r0 + j);
                    }
                    ++at;
                }
            }
            for (uint32_t i = tot + tid; i < static_cast<uint32_t>(P_b); i += kThreads) {
                po[i] = -1;
                L.pool_s[i] = -1;
            }
        }
    }
    // fallback is uniform: every thread saw the same shared values
    __syncthreads();

    // ------------------------------------------------ top-k inside the pool
    if (!fallback) {
        for (int i = tid; i < 1024; i += kThreads) L.chosen[i] = 0u;
        __syncthreads();
        const int b0 = 2 * tid;
        int32_t blk[2];
        uint32_t kk[16];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            blk[q] = b0 + q < P_b ? L.pool_s[b0 + q] : -1;
            const int64_t p0 = static_cast<int64_t>(blk[q] >= 0 ? blk[q] : 0) * 8;
            const float4 v0 = *reinterpret_cast<const float4*>(st + p0);
            const float4 v1 = *reinterpret_cast<const float4*>(st + p0 + 4);
            const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) kk[8 * q + e] = blk[q] >= 0 ? key_of(vv[e]) : 0u;
        }
        uint32_t T = 0u, need = 0u;
        const uint32_t k_eff = kth_key<16>(kk, static_cast<uint32_t>(k), L.sh, T, need);
        uint32_t hi = 0xffffffffu;
        bool all = k_eff < static_cast<uint32_t>(k);        // fewer visible positions than k: take all
        if (!all) {
            const float tau = float_of_key(T);
            hi = key_of(next_up(tau + e2));
            const uint32_t lo_raw = key_of(next_down(tau - e2));
            const uint32_t lo = lo_raw > 0u ? lo_raw : 1u;
            if (tid == 0) L.n_band = 0u;
            __syncthreads();
            uint32_t n_sure = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                n_sure += kk[j] > hi;
                if (kk[j] != 0u && kk[j] >= lo && kk[j] <= hi) {
                    const uint32_t at = atomicAdd(&L.n_band, 1u);
                    if (at < static_cast<uint32_t>(kBandPos)) L.band[at] = static_cast<uint64_t>(16 * tid + j);
                }
            }
            uint32_t tot;
            block_excl_scan(n_sure, L.sh.wave_tot, tot);
            const uint32_t nband = L.n_band;
            if (nband > static_cast<uint32_t>(kBandPos) || tot >= k_eff || tot + nband < k_eff) {
                fallback = true;
            } else {
                // band slots -> exact scores; rank by (exact desc, position asc):
                // slot order is position order inside the ascending pool
                for (uint32_t i = tid; i < nband; i += kThreads) {
                    const uint32_t slot = static_cast<uint32_t>(L.band[i]);
                    const int64_t pos = static_cast<int64_t>(L.pool_s[slot >> 3]) * 8 + (slot & 7);
                    const uint32_t ek = key_of(exact_score(L.qf, L.wf, kc, pos));
                    L.band[i] = (static_cast<uint64_t>(~ek) << 32) | slot;
                }
                __syncthreads();
                const uint32_t need_b = k_eff - tot;
                for (uint32_t i = tid; i < nband; i += kThreads) {
                    if (band_rank(L.band, nband, i) < need_b) {
                        const uint32_t slot = static_cast<uint32_t>(L.band[i]);
                        atomicOr(&L.chosen[slot >> 5], 1u << (slot & 31));
                    }
                }
                __syncthreads();
            }
        }
        if (!fallback) {
            uint32_t mine = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) mine += kk[j] != 0u && (all || kk[j] > hi || bit_of(L.chosen, 16 * tid + j));
            uint32_t tot;
            uint32_t at = block_excl_scan(mine, L.sh.wave_tot, tot);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (kk[j] != 0u && (all || kk[j] > hi || bit_of(L.chosen, 16 * tid + j))) {
                    if (at < static_cast<uint32_t>(k)) o[at] = blk[j >> 3] * 8 + (j & 7);
                    ++at;
                }
            }
            for (uint32_t i = tot + tid; i < static_cast<uint32_t>(k); i += kThreads) o[i] = -1;
        }
        __syncthreads();
    }
    if (!fallback) return;

    // ------------------------------------------------ exact fallback
    // exact scores and block maxima of the whole row, then the exact pool and
    // top-k with ordered emission (ties by id / position)
    for (int64_t i = tid; i < a.cap; i += kThreads) st[i] = i < vis ? exact_score(L.qf, L.wf, kc, i) : -__builtin_inff();
    __threadfence_block();
    __syncthreads();
    for (int64_t b = tid; b < a.nb; b += kThreads) {
        float m = -__builtin_inff();
        for (int e = 0; e < 8; ++e) m = fmaxf(m, st[b * 8 + e]);
        if (m == 0.0f) m = 0.0f;
        bmr[b] = m;
    }
    __threadfence_block();
    __syncthreads();
    {
        const int64_t r0 = static_cast<int64_t>(tid) * R1;
        uint32_t kk[R1];
#pragma unroll
        for (int j = 0; j < R1; ++j) kk[j] = (r0 + j < a.nb) ? key_of(bmr[r0 + j]) : 0u;
        const uint32_t got = select_run<R1>(kk, static_cast<uint32_t>(P_b), L.sh, [&](uint32_t r, int j) {
            po[r] = static_cast<int32_t>(r0) + j;
            L.pool_s[r] = static_cast<int32_t>(r0) + j;
        });
        for (int i = static_cast<int>(got) + tid; i < P_b; i += kThreads) {
            po[i] = -1;
            L.pool_s[i] = -1;
        }
    }
    __syncthreads();
    {
        const int b0 = 2 * tid;
        int32_t blk[2];
        uint32_t kk[16];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            blk[q] = b0 + q < P_b ? L.pool_s[b0 + q] : -1;
            const int64_t p0 = static_cast<int64_t>(blk[q] >= 0 ? blk[q] : 0) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) kk[8 * q + e] = blk[q] >= 0 ? key_of(st[p0 + e]) : 0u;
        }
        const uint32_t got = select_run<16>(kk, static_cast<uint32_t>(k), L.sh, [&](uint32_t r, int j) {
            o[r] = blk[j >> 3] * 8 + (j & 7);
        });
        for (int i = static_cast<int>(got) + tid; i < k; i += kThreads) o[i] = -1;
    }
}

}  // namespace

bool decode_select_supported(int64_t cap, int H_I, int d_I, int P_b, int k) {
    return H_I == kHeads && d_I == kDim && cap > 0 && cap % 64 == 0 && cap / 8 <= 32 * kThreads &&
           P_b >= 1 && P_b <= kPoolCap && k >= 1 && k <= P_b;
}

int64_t scan_wgs(int64_t cap) { return (cap / 64 + 3) / 4; }

size_t decode_select_workspace_bytes(int64_t B, int64_t cap) {
    const size_t st = (static_cast<size_t>(B) * cap * 4 + 255) / 256 * 256;
    const size_t bm = (static_cast<size_t>(B) * (cap / 8) * 4 + 255) / 256 * 256;
    const size_t km = (static_cast<size_t>(B) * scan_wgs(cap) * 4 + 255) / 256 * 256;
    return st + bm + km;
}

DsArgs make_args(const DecodeSelectLaunch& L, void* ws) {
    DsArgs a;
    a.q = static_cast<const uint16_t*>(L.q_idx);
    a.w = L.w;
    a.kc = static_cast<const uint8_t*>(L.k_idx);
    a.ctx_len = L.ctx_len;
    a.cap = L.cap;
    a.B = L.B;
    a.nb = L.cap / 8;
    a.P_b = L.P_b;
    a.k = L.k;
    a.pool = L.out_pool;
    a.idx = L.out_idx;
    char* p = static_cast<char*>(ws);
    a.st = reinterpret_cast<float*>(p); p += (static_cast<size_t>(L.B) * L.cap * 4 + 255) / 256 * 256;
    a.bm = reinterpret_cast<float*>(p); p += (static_cast<size_t>(L.B) * (L.cap / 8) * 4 + 255) / 256 * 256;
    a.kmax = reinterpret_cast<float*>(p);
    a.nwg = scan_wgs(L.cap);
    return a;
}

hipError_t launch_decode_scan(const DecodeSelectLaunch& L, void* ws, hipStream_t st) {
    if (L.B == 0) return hipSuccess;
    const DsArgs a = make_args(L, ws);
    const dim3 gs(static_cast<unsigned>(a.nwg), static_cast<unsigned>(L.B));
    dscan_kernel<<<gs, kScanThreads, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode_select(const DecodeSelectLaunch& L, void* ws, hipStream_t st) {
    if (L.B == 0) return hipSuccess;
    const DsArgs a = make_args(L, ws);
    if (a.nb <= 16 * kThreads)
        dselect_kernel<16><<<dim3(static_cast<unsigned>(L.B)), kThreads, 0, st>>>(a);
    else
        dselect_kernel<32><<<dim3(static_cast<unsigned>(L.B)), kThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace csa2
