// Full-mode top-k for a prefill chunk ("DeepSeek-V4.1-Flash KV Cache
// Compression" notes, sections 1-2: the encoder's Full layers score every
// visible compressed entry for each of the chunk's query tokens, m = 2).
//
// The indices must equal those chosen from the exact score (float32 fma
// chains over channels, then over heads, in order).  That order cannot be
// kept on the matrix cores, so the selection runs in two tiers:
//
//  1. score_mfma_kernel computes s~ = sum_h w_h ReLU(q_h . k_j) for a block of
//     queries x keys with v_mfma_f32_32x32x16_bf16 (bf16 products are exact
//     in float32; only the order and precision of the additions differ);
//  2. for each query row, |s~_j - s_j| <= eps_t for every key j, where
//         eps_t = kEpsRel * A_t * Kmax + (underflow term),
//         A_t   = sum_h |w_h| * ||q_h||_2,   Kmax = max_j ||k_j||_2.
//     Derivation: each dot product of n = 128 exact products summed in
//     float32 in any order, each addition rounded at least as well as
//     truncation (unit 2^-23), is within gamma_n * sum_c |q_c k_c| of the
//     real value (gamma_n = n 2^-23 / (1 - n 2^-23) = 1.53e-5), so the exact
//     chain and the matrix-core sum differ by at most 2 gamma_n ||q_h|| ||k_j||
//     (Cauchy-Schwarz); ReLU is 1-Lipschitz; the two 8-term head sums add
//     at most 2 gamma_8 (2^-24 unit) of sum_h |w_h| ||q_h|| ||k_j|| (1 + ...).
//     Total below 3.2e-5 * A_t * ||k_j||; kEpsRel = 4e-5 leaves margin for
//     the float32 norms themselves.
//     With tau~ the k-th largest s~ (the exact k-th score tau is within eps of
//     it): s~ > tau~ + 2 eps  =>  s > tau (chosen);  s~ < tau~ - 2 eps  =>
//     s < tau (not chosen); keys in between are rescored with the exact
//     chain, and the remaining slots go to them by (exact score desc,
//     position asc).  Every key whose exact score equals tau lies in that
//     band, so ties resolve exactly as in the definition.
//
// Rows whose candidate list or band does not fit the fixed LDS budget fall
// back to exact scores for the whole row (same result, slower).
//
// Scratch (per chunk of up to kChunkRows query rows): the s~ rows, a 4,096-bin
// histogram per row, and the candidate list per row.
#include "csa2_internal.h"

namespace csa2 {
namespace {
#include "select_util.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kHeads = 8, kDim = 128;          // indexer shape of the matrix-core path
constexpr int kNch = kDim * 2 / 16;            // 16-byte chunks per indexer row
constexpr int kBins = 4096;                    // coarse digit: key >> 20
constexpr int kCandCap = 12288;                // candidates per row kept for the final pass
constexpr int kBandCap = 2048;                 // band keys rescored in LDS
constexpr int kKCap = 4096;                    // largest k
constexpr int kChunkRows = 1024;               // query rows per scratch chunk
constexpr int kQB = 64;                        // queries per scoring workgroup
constexpr int kKeyTile = 32;
constexpr int kKeysPerWG = 4096;
constexpr float kEpsRel = 4.0e-5f;

struct PfArgs {
    const uint16_t* q;       // [T][8][128] bf16
    const float* w;          // [T][8]
    const uint8_t* kc;       // tiled indexer cache (bf16)
    int64_t cap;
    int32_t ctx_len;
    int64_t q_pos0;
    int32_t m;
    int32_t k;
    int64_t T;
};

__device__ __forceinline__ int64_t vis_of(const PfArgs& a, int64_t t) {
    const int64_t v = (a.q_pos0 + t + 1) / a.m;
    return v < a.ctx_len ? v : a.ctx_len;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// float value of a key (inverse of key_of for nonzero keys)
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

// 16-byte chunk c of indexer row `pos` in the tiled layout
__device__ __forceinline__ const uint4* kchunk(const uint8_t* kc, int64_t pos, int c) {
    return reinterpret_cast<const uint4*>(kc) + ((pos >> 6) * kNch + c) * 64 + (pos & 63);
}

// ---------------------------------------------------------------- norms
// Kmax = largest ||k_j|| over rows [0, n_rows), as float bits (non-negative
// floats order like their bit patterns).
__global__ __launch_bounds__(256) void knorm_max_kernel(const uint8_t* __restrict__ kc, int64_t n_rows,
                                                        uint32_t* __restrict__ kmax_bits) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    float nrm = 0.0f;
    if (j < n_rows) {
        float ss = 0.0f;
#pragma unroll 4
        for (int c = 0; c < kNch; ++c) {
            const uint4 v = *kchunk(kc, j, c);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = bf16_lo(u[e]), b = bf16_hi(u[e]);
                ss = fmaf(a, a, ss);
                ss = fmaf(b, b, ss);
            }
        }
        nrm = sqrtf(ss);
    }
    for (int off = 32; off > 0; off >>= 1) nrm = fmaxf(nrm, __shfl_xor(nrm, off));
    if ((threadIdx.x & 63) == 0) atomicMax(kmax_bits, __float_as_uint(nrm));
}

// eps_t per query row: kEpsRel * A_t * Kmax plus an absolute term for
// products that underflow float32 on the matrix cores.
__global__ __launch_bounds__(256) void eps_kernel(PfArgs a, const uint32_t* __restrict__ kmax_bits,
                                                  float* __restrict__ eps) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 32 + (threadIdx.x >> 3);
    const int h = threadIdx.x & 7;
    float qn = 0.0f, wa = 0.0f;
    if (t < a.T) {
        const uint4* qr = reinterpret_cast<const uint4*>(a.q + (t * kHeads + h) * kDim);
        float ss = 0.0f;
        for (int c = 0; c < kNch; ++c) {
            const uint4 v = qr[c];
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ss = fmaf(bf16_lo(u[e]), bf16_lo(u[e]), ss);
                ss = fmaf(bf16_hi(u[e]), bf16_hi(u[e]), ss);
            }
        }
        wa = fabsf(a.w[t * kHeads + h]);
        qn = wa * sqrtf(ss);
    }
    for (int off = 1; off < 8; off <<= 1) {
        qn += __shfl_xor(qn, off);
        wa += __shfl_xor(wa, off);
    }
    if (h == 0 && t < a.T) {
        const float km = __uint_as_float(*kmax_bits);
        eps[t] = next_up(kEpsRel * qn * km + 0x1p-90f * km * wa + 0x1p-120f);
    }
}

// ---------------------------------------------------------------- s~ rows
// Block = 8 waves x 8 queries (two 32-row M-tiles of 4 queries x 8 heads
// each) x kKeysPerWG keys, streamed in tiles of 32 keys through LDS
// (double-buffered).  A = q rows (registers), B = key rows (LDS).
// Output: st[(t - t0) * ld + j] for t in the chunk, j < n_cols; -inf where
// j >= vis(t).
__global__ __launch_bounds__(512) void score_mfma_kernel(PfArgs a, int64_t t0, int64_t t1, int64_t n_cols,
                                                         int64_t ld, float* __restrict__ st) {
    constexpr int KROW = kDim + 8;               // padded LDS row (bf16 elements)
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKeyTile * KROW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t qb = t0 + static_cast<int64_t>(blockIdx.y) * kQB + 8 * wv;   // wave's first query
    const int64_t j_begin = static_cast<int64_t>(blockIdx.x) * kKeysPerWG;
    int64_t j_end = j_begin + kKeysPerWG;
    if (j_end > n_cols) j_end = n_cols;
    const int n_tiles = static_cast<int>((j_end - j_begin + kKeyTile - 1) / kKeyTile);

    // q fragments: M-tile mt, row r = lane%32 -> query qb + 4mt + r/8, head r%8;
    // k-step s covers channels 16s + 8(lane/32) + 0..7
    bf16x8 qa[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        int64_t t = qb + 4 * mt + ((lane & 31) >> 3);
        if (t >= t1) t = t1 - 1;
        const uint16_t* qr = a.q + (t * kHeads + (lane & 7)) * kDim + 8 * (lane >> 5);
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qa[mt][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qr + 16 * s));
    }
    // head weights of the accumulator rows: reg r -> query r/4, head 4(lane/32) + r%4
    float wr[2][16];
    int64_t vis[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            int64_t t = qb + 4 * mt + qq;
            vis[mt][qq] = t < t1 ? vis_of(a, t) : 0;
            if (t >= t1) t = t1 - 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) wr[mt][4 * qq + i] = a.w[t * kHeads + 4 * (lane >> 5) + i];
        }
    }

    // key tile loader: thread -> (chunk c = tid / 32, key tid % 32)
    const int lc = tid >> 5, lk = tid & 31;
    auto load_tile = [&](int tile) -> uint4 {
        const int64_t pos = j_begin + static_cast<int64_t>(tile) * kKeyTile + lk;
        const int64_t p = pos < a.cap ? pos : 0;
        return *kchunk(a.kc, p, lc);
    };
    auto store_tile = [&](int buf, uint4 v) {
        *reinterpret_cast<uint4*>(&Ks[buf][lk * KROW + 8 * lc]) = v;
    };
    if (n_tiles > 0) store_tile(0, load_tile(0));
    __syncthreads();
    for (int tile = 0; tile < n_tiles; ++tile) {
        const int buf = tile & 1;
        uint4 nxt = make_uint4(0u, 0u, 0u, 0u);
        if (tile + 1 < n_tiles) nxt = load_tile(tile + 1);
        floatx16 acc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8 kb = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4*>(&Ks[buf][(lane & 31) * KROW + 16 * s + 8 * (lane >> 5)]));
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], kb, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], kb, acc[1], 0, 0, 0);
        }
        // epilogue: ReLU, head weights, the two 4-head halves joined across
        // lanes l and l^32
        const int64_t j = j_begin + static_cast<int64_t>(tile) * kKeyTile + (lane & 31);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            float part[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                float p = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) p = fmaf(wr[mt][4 * qq + i], fmaxf(acc[mt][4 * qq + i], 0.0f), p);
                part[qq] = p;
            }
            float full[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) full[qq] = part[qq] + __shfl_xor(part[qq], 32);
            // lanes < 32 write queries 0,1 of the tile, lanes >= 32 queries 2,3
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int qq = 2 * (lane >> 5) + e;
                const int64_t t = qb + 4 * mt + qq;
                if (t < t1 && j < j_end) {
                    const float v = (qq == 0 ? full[0] : qq == 1 ? full[1] : qq == 2 ? full[2] : full[3]);
                    const int64_t vq = (qq == 0 ? vis[mt][0] : qq == 1 ? vis[mt][1] : qq == 2 ? vis[mt][2] : vis[mt][3]);
                    st[(t - t0) * ld + j] = j < vq ? v : -__builtin_inff();
                }
            }
        }
        if (tile + 1 < n_tiles) store_tile(buf ^ 1, nxt);
        __syncthreads();
    }
}

// ---------------------------------------------------------------- selection
// Per-row candidate threshold: the 4,096-bin histogram gives the bin b* that
// holds the k-th s~; candidates are keys >= key_of(L), L = lower edge of b*
// minus 2 eps (rounded down), so every key within 2 eps of tau~ or above is
// one.  One 256-thread workgroup per row; thread t owns bins 4095-16t down
// to 4080-16t.
__global__ __launch_bounds__(256) void band_thresh_kernel(int64_t t0, PfArgs a, const float* __restrict__ eps,
                                                          const uint32_t* __restrict__ hist_all,
                                                          uint32_t* __restrict__ thr) {
    __shared__ uint32_t wsum[4];
    const int64_t r = blockIdx.x;
    const int64_t t = t0 + r;
    const int64_t vis = vis_of(a, t);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (vis <= a.k) {                                  // whole row chosen
        if (tid == 0) thr[r] = 1u;
        return;
    }
    const uint32_t need = static_cast<uint32_t>(a.k);
    const int hb = kBins - 16 - 16 * tid;
    uint32_t c[16], sum = 0;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(&hist_all[r * kBins + hb + i]);
        c[15 - i] = v.x; c[14 - i] = v.y; c[13 - i] = v.z; c[12 - i] = v.w;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c[i];                 // c[0] is the highest bin
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    const uint32_t excl = before + incl - sum;
    if (excl < need && excl + sum >= need) {
        uint32_t acc = excl;
        int bin = hb;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (acc + c[i] >= need) { bin = hb + 15 - i; break; }
            acc += c[i];
        }
        const float L = next_down(float_of_key(static_cast<uint32_t>(bin) << 20) - 2.0f * eps[t]);
        const uint32_t lk = key_of(L);
        thr[r] = lk > 0u ? lk : 1u;
    }
}

// Append (key, position) of every candidate (key >= thr[row]) to the row's
// list; one global atomic per wave.
__global__ __launch_bounds__(kThreads) void band_collect_kernel(const float* __restrict__ st, int64_t ld,
                                                                int64_t t0, PfArgs a,
                                                                const uint32_t* __restrict__ thr,
                                                                uint32_t* __restrict__ cnt,
                                                                uint2* __restrict__ cand) {
    constexpr int kPer = 16;
    constexpr int kChunk = kPer * kThreads;
    const int64_t r = blockIdx.y;
    const int64_t vis = vis_of(a, t0 + r);
    if (vis <= a.k) return;                           // whole row chosen: no candidates needed
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk;
    if (base >= vis) return;
    const float* s = st + r * ld;
    const uint32_t lkey = thr[r];
    const int lane = threadIdx.x & 63;
    uint32_t kk[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t i = base + j * kThreads + threadIdx.x;
        kk[j] = (i < vis) ? key_of(s[i]) : 0u;
    }
    uint64_t bal[kPer];
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        bal[j] = __ballot(kk[j] >= lkey);
        tot += static_cast<uint32_t>(__popcll(bal[j]));
    }
    if (tot == 0) return;
    uint32_t wb = 0;
    if (lane == 0) wb = atomicAdd(&cnt[r], tot);
    wb = __shfl(wb, 0);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const uint32_t off = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal[j] >> 32),
                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal[j]), 0u));
        const uint32_t at = wb + off;
        if (((bal[j] >> lane) & 1ull) && at < static_cast<uint32_t>(kCandCap)) {
            const int64_t i = base + j * kThreads + threadIdx.x;
            cand[r * kCandCap + at] = make_uint2(kk[j], static_cast<uint32_t>(i));
        }
        wb += static_cast<uint32_t>(__popcll(bal[j]));
    }
}

// exact score of key row pos for query row t (q, w staged as float32 in LDS)
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

__global__ __launch_bounds__(kThreads) void band_final_kernel(float* __restrict__ st, int64_t ld, int64_t t0,
                                                              PfArgs a, const float* __restrict__ eps,
                                                              const uint32_t* __restrict__ cnt,
                                                              const uint2* __restrict__ cand_all,
                                                              int32_t* __restrict__ out) {
    __shared__ uint2 cand[kCandCap];
    __shared__ uint64_t band[kBandCap];
    __shared__ uint32_t sel[kKCap];
    __shared__ float qf[kHeads * kDim];
    __shared__ float wf[kHeads];
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wave_tot[kWaves];
    __shared__ uint32_t res[2];
    __shared__ uint32_t counters[2];
    const int64_t r = blockIdx.x;
    const int64_t t = t0 + r;
    const int64_t vis = vis_of(a, t);
    const int k = a.k;
    int32_t* o = out + t * static_cast<int64_t>(k);
    const uint32_t k_eff = vis < k ? static_cast<uint32_t>(vis) : static_cast<uint32_t>(k);
    if (vis <= k) {                                   // every visible entry is chosen
        for (int64_t i = threadIdx.x; i < k; i += kThreads) o[i] = i < vis ? static_cast<int32_t>(i) : -1;
        return;
    }
    // query row in float32 (exact widening of bf16)
    for (int i = threadIdx.x; i < kHeads * kDim; i += kThreads) {
        const uint16_t b = a.q[t * kHeads * kDim + i];
        qf[i] = __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    if (threadIdx.x < kHeads) wf[threadIdx.x] = a.w[t * kHeads + threadIdx.x];
    const uint32_t C = cnt[r];
    bool fallback = C > static_cast<uint32_t>(kCandCap);
    if (!fallback) {
        for (uint32_t i = threadIdx.x; i < C; i += kThreads) cand[i] = cand_all[r * kCandCap + i];
        __syncthreads();
        // tau~: the k-th largest s~ (all keys at or above it are candidates)
        uint32_t T = 0, need = 0;
        auto get = [&](int64_t i) { return cand[i].x; };
        radix_select(get, C, k_eff, hist, res, T, need);
        const float tau = float_of_key(T);
        const float e2 = 2.0f * eps[t];
        const uint32_t hi_key = key_of(next_up(tau + e2));
        const uint32_t lo_key = key_of(next_down(tau - e2)) > 0u ? key_of(next_down(tau - e2)) : 1u;
        if (threadIdx.x < 2) counters[threadIdx.x] = 0;
        __syncthreads();
        // sure picks (s~ above the band) -> sel; band keys -> band
        for (uint32_t i = threadIdx.x; i < C; i += kThreads) {
            const uint2 c = cand[i];
            if (c.x > hi_key) {
                const uint32_t at = atomicAdd(&counters[0], 1u);
                if (at < static_cast<uint32_t>(kKCap)) sel[at] = c.y;
            } else if (c.x >= lo_key) {
                const uint32_t at = atomicAdd(&counters[1], 1u);
                if (at < static_cast<uint32_t>(kBandCap)) band[at] = c.y;
            }
        }
        __syncthreads();
        const uint32_t n_in = counters[0], n_band = counters[1];
        if (n_band > static_cast<uint32_t>(kBandCap) || n_in > k_eff || n_in + n_band < k_eff) {
            fallback = true;
        } else {
            // exact scores of the band keys; order by (score desc, position
            // asc) via an ascending sort of (~key << 32 | position)
            for (uint32_t i = threadIdx.x; i < n_band; i += kThreads) {
                const uint32_t pos = static_cast<uint32_t>(band[i]);
                const uint32_t ek = key_of(exact_score(qf, wf, a.kc, pos));
                band[i] = (static_cast<uint64_t>(~ek) << 32) | pos;
            }
            int p2 = 1;
            while (p2 < static_cast<int>(n_band)) p2 <<= 1;
            for (int i = threadIdx.x + static_cast<int>(n_band); i < p2; i += kThreads) band[i] = ~0ull;
            __syncthreads();
            for (int size = 2; size <= p2; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    for (int i = threadIdx.x; i < p2 / 2; i += kThreads) {
                        const int lo = 2 * i - (i & (stride - 1));
                        const int hi = lo + stride;
                        const bool up = ((lo & size) == 0);
                        const uint64_t x = band[lo], y = band[hi];
                        if ((x > y) == up) { band[lo] = y; band[hi] = x; }
                    }
                    __syncthreads();
                }
            }
            const uint32_t need_b = k_eff - n_in;
            for (uint32_t i = threadIdx.x; i < need_b; i += kThreads)
                sel[n_in + i] = static_cast<uint32_t>(band[i]);
            int q2 = 1;
            while (q2 < static_cast<int>(k_eff)) q2 <<= 1;
            for (int i = threadIdx.x + static_cast<int>(k_eff); i < q2; i += kThreads) sel[i] = 0xffffffffu;
            __syncthreads();
            bitonic_sort(sel, q2);
            for (uint32_t i = threadIdx.x; i < k_eff; i += kThreads) o[i] = static_cast<int32_t>(sel[i]);
        }
    }
    if (fallback) {
        // exact scores for the whole visible row (overwrites its s~ row)
        float* s = st + r * ld;
        __syncthreads();
        for (int64_t i = threadIdx.x; i < vis; i += kThreads) s[i] = exact_score(qf, wf, a.kc, i);
        __threadfence_block();
        __syncthreads();
        uint32_t T = 0, need = 0;
        auto get = [&](int64_t i) { return key_of(s[i]); };
        radix_select(get, vis, k_eff, hist, res, T, need);
        emit_ordered(get, vis, T, need, k_eff, nullptr, o, k, wave_tot);
    }
    for (int64_t i = k_eff + threadIdx.x; i < k; i += kThreads) o[i] = -1;
}

__global__ void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// per-row 12-bit histogram of s~ keys over [0, vis(t)); scores of one row
// spread over tens of bins, so plain LDS atomics rarely collide
__global__ __launch_bounds__(kThreads) void band_hist_kernel(const float* __restrict__ st, int64_t ld, int64_t t0,
                                                             PfArgs a, uint32_t* __restrict__ hist_all) {
    constexpr int kPer = 16;
    constexpr int kChunk = kPer * kThreads;
    __shared__ uint32_t hist[kBins];
    const int64_t r = blockIdx.y;
    const int64_t vis = vis_of(a, t0 + r);
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk;
    if (base >= vis || vis <= a.k) return;
    const float* s = st + r * ld;
    for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0;
    uint32_t kk[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t i = base + j * kThreads + threadIdx.x;
        kk[j] = (i < vis) ? key_of(s[i]) : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if (kk[j] != 0u) atomicAdd(&hist[kk[j] >> 20], 1u);
    __syncthreads();
    for (int i = threadIdx.x; i < kBins; i += kThreads)
        if (hist[i]) atomicAdd(&hist_all[r * kBins + i], hist[i]);
}

struct PfWs {
    uint32_t* kmax;
    float* eps;
    float* st;
    uint32_t* hist;     // [rows][kBins]
    uint32_t* cnt;      // [rows]
    uint32_t* thr;      // [rows]
    uint2* cand;        // [rows][kCandCap]
    int64_t ld;
};

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

PfWs carve(void* ws, int64_t T, int64_t n_cols) {
    PfWs w;
    char* p = static_cast<char*>(ws);
    const int64_t rows = T < kChunkRows ? T : kChunkRows;
    w.ld = (n_cols + 63) / 64 * 64;
    w.kmax = reinterpret_cast<uint32_t*>(p); p += 256;
    w.eps = reinterpret_cast<float*>(p); p += align256(static_cast<size_t>(T) * 4);
    w.st = reinterpret_cast<float*>(p); p += align256(static_cast<size_t>(rows) * w.ld * 4);
    w.hist = reinterpret_cast<uint32_t*>(p); p += align256(static_cast<size_t>(rows) * (kBins + 2) * 4);
    w.cnt = w.hist + rows * kBins;
    w.thr = w.cnt + rows;
    w.cand = reinterpret_cast<uint2*>(p); p += align256(static_cast<size_t>(rows) * kCandCap * 8);
    return w;
}

}  // namespace

int64_t prefill_cols(int64_t T, int32_t ctx_len, int64_t q_pos0, int32_t m) {
    if (T <= 0) return 0;
    int64_t v = (q_pos0 + T) / m;
    return v < ctx_len ? v : ctx_len;
}

size_t prefill_topk_workspace_bytes(int64_t T, int32_t ctx_len, int64_t q_pos0, int32_t m) {
    if (T <= 0) return 0;
    const int64_t n_cols = prefill_cols(T, ctx_len, q_pos0, m);
    const int64_t rows = T < kChunkRows ? T : kChunkRows;
    const int64_t ld = (n_cols + 63) / 64 * 64;
    return 256 + align256(static_cast<size_t>(T) * 4) + align256(static_cast<size_t>(rows) * ld * 4) +
           align256(static_cast<size_t>(rows) * (kBins + 2) * 4) + align256(static_cast<size_t>(rows) * kCandCap * 8);
}

int prefill_topk_max_k() { return kKCap; }

hipError_t launch_prefill_topk(const PrefillLaunch& L, void* ws, hipStream_t st) {
    if (L.T <= 0) return hipSuccess;
    PfArgs a;
    a.q = static_cast<const uint16_t*>(L.q);
    a.w = L.w;
    a.kc = static_cast<const uint8_t*>(L.k_idx);
    a.cap = L.cap;
    a.ctx_len = L.ctx_len;
    a.q_pos0 = L.q_pos0;
    a.m = L.m;
    a.k = L.k;
    a.T = L.T;
    const int64_t n_cols = prefill_cols(L.T, L.ctx_len, L.q_pos0, L.m);
    PfWs w = carve(ws, L.T, n_cols);
    zero_words_kernel<<<1, 64, 0, st>>>(w.kmax, 1);
    if (n_cols > 0)
        knorm_max_kernel<<<dim3(static_cast<unsigned>((n_cols + 255) / 256)), 256, 0, st>>>(a.kc, n_cols, w.kmax);
    eps_kernel<<<dim3(static_cast<unsigned>((L.T + 31) / 32)), 256, 0, st>>>(a, w.kmax, w.eps);
    for (int64_t t0 = 0; t0 < L.T; t0 += kChunkRows) {
        const int64_t t1 = t0 + kChunkRows < L.T ? t0 + kChunkRows : L.T;
        const int64_t rows = t1 - t0;
        const int64_t cols = prefill_cols(t1, L.ctx_len, L.q_pos0, L.m);
        const int64_t hwords = rows * (kBins + 1);      // histograms and candidate counts
        zero_words_kernel<<<dim3(static_cast<unsigned>((hwords + 255) / 256)), 256, 0, st>>>(w.hist, hwords);
        if (cols > 0) {
            const dim3 g1(static_cast<unsigned>((cols + kKeysPerWG - 1) / kKeysPerWG),
                          static_cast<unsigned>((rows + kQB - 1) / kQB));
            score_mfma_kernel<<<g1, 512, 0, st>>>(a, t0, t1, cols, w.ld, w.st);
            const dim3 g2(static_cast<unsigned>((cols + 16 * kThreads - 1) / (16 * kThreads)),
                          static_cast<unsigned>(rows));
            band_hist_kernel<<<g2, kThreads, 0, st>>>(w.st, w.ld, t0, a, w.hist);
            band_thresh_kernel<<<dim3(static_cast<unsigned>(rows)), 256, 0, st>>>(t0, a, w.eps, w.hist, w.thr);
            band_collect_kernel<<<g2, kThreads, 0, st>>>(w.st, w.ld, t0, a, w.thr, w.cnt, w.cand);
        }
        band_final_kernel<<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(w.st, w.ld, t0, a, w.eps, w.cnt,
                                                                                  w.cand, L.out);
    }
    return hipGetLastError();
}

}  // namespace csa2
