// Full-mode top-k for a prefill chunk ("DeepSeek-V4.1-Flash KV Cache
// Compression" notes, sections 1-2: the encoder's Full layers score every
// visible compressed entry for each of the chunk's query tokens, m = 2).
//
// The indices must equal those chosen from the exact score (float32 fma
// chains over channels, then over heads, in order).  That order cannot be
// kept on the matrix cores, so the selection runs in tiers:
//
//  1. Bound.  The matrix cores give s~ = sum_h w_h ReLU(q_h . k_j) with
//     v_mfma_f32_32x32x16_bf16 (bf16 products are exact in float32; only the
//     order and precision of the additions differ), and for every key j
//         |s~_j - s_j| <= eps_t = kEpsRel * A_t * Kmax + (underflow term),
//         A_t = sum_h |w_h| * ||q_h||_2,   Kmax = max_j ||k_j||_2.
//     Derivation: a dot product of n = 128 exact products summed in float32
//     in any order, each addition rounded at least as well as truncation
//     (unit 2^-23), is within gamma_n * sum_c |q_c k_c| of the real value
//     (gamma_n = n 2^-23 / (1 - n 2^-23) = 1.53e-5), so the exact chain and
//     the matrix-core sum differ by at most 2 gamma_n ||q_h|| ||k_j||
//     (Cauchy-Schwarz); ReLU is 1-Lipschitz; the two 8-term head sums add at
//     most 2 gamma_8 of sum_h |w_h| ||q_h|| ||k_j|| (1 + ...).  Total below
//     3.2e-5 * A_t * ||k_j||; kEpsRel = 4e-5 leaves margin for the float32
//     norms themselves.
//  2. Sample.  s~ of one 32-key block in every 512 keys (the block picked by
//     a hash of the group, so periodic structure cannot alias) gives each row a
//     lower key L_t: the lower edge of the radix bin that holds the sample's
//     j-th largest, j chosen so that about 3k keys of the whole row are
//     expected at or above it.
//  3. Candidates.  The full matrix-core pass keeps (s~, position) of every
//     key with s~ >= L_t; each workgroup owns a fixed slot range per row
//     (as many slots as it has keys), so no atomics are needed.
//  4. Final, per row: with C candidates, k <= C and tau~ the k-th largest
//     candidate s~ (then also the k-th of the whole row, since every other
//     key lies below L_t), one radix pass over the candidates gives a bin
//     [lo, hi] that holds tau~.  The exact k-th score tau then lies in
//     [lo - eps, hi + eps].  The check L_t <= lo - 2 eps shows that every key
//     within 2 eps of the bin or above is a candidate.  Then s~ > hi + 2 eps
//     => s > tau (chosen), s~ < lo - 2 eps => s < tau (not chosen); keys in
//     between (the band) are rescored with the exact chain and fill the
//     remaining slots by (exact score desc, position asc).  Every key whose
//     exact score equals tau lies in the band, so ties resolve exactly as in
//     the definition.
//
// A row that fails a check (too few or too many candidates, a band wider
// than the fixed LDS budget) is rescored exactly over its whole row and
// selected with the same radix routine as csa2_topk: same result, slower.
//
// Scratch per chunk of up to kChunkRows query rows: the sample's s~, and the
// candidate slots (8 bytes per (row, visible key) reserved, a few percent
// written), which a falling-back row reuses for its exact scores.
//
// Launch shape: the scoring grids are sized to whole rounds of one
// workgroup per CU, and numbered so the workgroups that read the same keys
// share an XCD's L2.
#include <type_traits>

#include "csa2_internal.h"

namespace csa2 {
namespace {
#include "select_util.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeads = 8, kDim = 128;          // indexer shape of the matrix-core path
constexpr int kNch = kDim * 2 / 16;            // 16-byte chunks per indexer row
constexpr int kCandCap = 12288;                // candidates per row staged in LDS
constexpr int kBandCap = 2048;                 // band keys rescored in LDS
constexpr int kKCap = 4096;                    // largest k
constexpr int kChunkRows = 1024;               // query rows per scratch chunk
constexpr int kQB = 64;                        // queries per scoring workgroup
constexpr int kSub = 32;                       // keys per MFMA column block
constexpr int kTileKeys = 128;                 // keys per LDS tile (4 column blocks)
constexpr int kMaxKeysPerWG = 16384;            // largest key range of a candidate workgroup
constexpr int kGroup = 512;                    // sample: one 32-key block per 512 keys
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

// ---------------------------------------------------------------- s~ blocks
// One workgroup = 8 waves x 8 queries (two 32-row M-tiles of 4 queries x 8
// heads each); A = q rows (registers), B = key rows from LDS.  Keys stream
// through LDS in tiles of 128 (double-buffered; the next tile's global loads
// are issued before the current tile's 64 MFMAs per wave).  Each 32-key
// column block ends in the epilogue: ReLU and head weights give per-lane
// partial sums over 4 heads, and one v_permlane32_swap pairs the halves, so
// lane l ends with s~ of key l%32 for query e (l < 32) or 2 + e (l >= 32) of
// M-tile mt, for e = 0, 1.
//
// Workgroup (bx, by) takes query block by and column blocks
// [bx * g.blocks, (bx + 1) * g.blocks).  The grid is 1-D and, with g.xcd,
// numbered so that the workgroups of one bx (which read the same keys) run on
// one XCD and share its L2: dispatch assigns workgroup L to XCD L % 8.
// SAMPLE: column block b is the hashed 32-key block of group b (kGroup keys
// per group); s~ goes to samp[row][32 * group + l%32] (-inf where invisible).
// Otherwise: column block b holds keys [32b, 32b + 32); the workgroup appends
// (s~ bits, position) for s~ >= L_row to the row's slots [bx * kpw, ...),
// kpw = 32 * g.blocks, in position order, and its count to counts[row][bx].
struct Geo {
    int64_t n_x;         // workgroups per query block that hold keys
    int32_t n_y;         // query blocks
    int32_t blocks;      // 32-key column blocks per workgroup (a multiple of 4)
    int32_t xcd;         // XCD-aware numbering (grid = roundup(n_x, 8) * n_y)
    int64_t cand_ld;     // candidate slots per row
    int64_t cnt_ld;      // count entries per row
};
// the top kSampBits bits of a multiplicative hash of the group index pick
// one of its kGroup / kSub blocks, so every block of a group can be sampled
constexpr int kSampBits = 4;
static_assert(kGroup / kSub == (1 << kSampBits), "the sample hash must cover every block of a group");
__device__ __forceinline__ int sample_block(int64_t group) {
    return static_cast<int>((static_cast<uint32_t>(group) * 0x9E3779B1u) >> (32 - kSampBits));
}

// float threshold of a row's candidate key: 1 -> -inf (every visible key),
// 0xffffffff -> +inf (none), else the float whose key it is
__device__ __forceinline__ float thr_float(uint32_t key) {
    if (key <= 1u) return -__builtin_inff();
    if (key == 0xffffffffu) return __builtin_inff();
    return float_of_key(key);
}

// ReLU as one integer max: non-negative floats order like their bit
// patterns, and every negative float (and -0) maps to +0
__device__ __forceinline__ float relu(float x) {
    const int i = __float_as_int(x);
    return __int_as_float(i > 0 ? i : 0);
}

template <bool SAMPLE>
__global__ __launch_bounds__(512) void score_mfma_kernel(PfArgs a, int64_t t0, int64_t t1, int64_t n_cols, Geo g,
                                                         float* __restrict__ samp, int64_t ld_s,
                                                         const uint32_t* __restrict__ thr,
                                                         uint32_t* __restrict__ counts, uint2* __restrict__ cand) {
    constexpr int KROW = kDim + 8;               // padded LDS row (bf16 elements)
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kTileKeys * KROW];
    int64_t bx;
    int by;
    {
        const int64_t L = blockIdx.x;
        if (g.xcd) {
            const int64_t i = L >> 3;
            bx = (L & 7) + 8 * (i / g.n_y);
            by = static_cast<int>(i % g.n_y);
        } else {
            bx = L % g.n_x;
            by = static_cast<int>(L / g.n_x);
        }
    }
    if (bx >= g.n_x) return;                     // padding of the XCD-aware grid
    const int n_tiles = g.blocks / (kTileKeys / kSub);
    const int tid = threadIdx.x, lane = tid & 63;
    const bool hi = lane >= 32;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t qb = t0 + static_cast<int64_t>(by) * kQB + 8 * wv;   // wave's first query

    // first key of column block b of this workgroup
    auto block_key = [&](int b) -> int64_t {
        const int64_t gb = bx * g.blocks + b;
        if (SAMPLE) return gb * kGroup + kSub * sample_block(gb);
        return gb * kSub;
    };

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
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            int64_t t = qb + 4 * mt + qq;
            if (t >= t1) t = t1 - 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) wr[mt][4 * qq + i] = a.w[t * kHeads + 4 * (lane >> 5) + i];
        }
    // per lane and (mt, e): its query's visible limit minus lane%32 (key
    // block jb is visible for this lane while jb < lim), threshold, and
    // where its row's values go (the sample row, or the workgroup's first
    // candidate slot of the row)
    int32_t lim[2][2];
    float thf[2][2];
    uint32_t soff[2][2];                 // SAMPLE: byte offset of this lane's sample slot 0 in the wave's buffer
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t t = qb + 4 * mt + (hi ? 2 + e : e);
            const bool ok = t < t1;
            const int64_t tc = ok ? t : t1 - 1;
            int64_t v = ok ? vis_of(a, t) : 0;
            if (v > n_cols) v = n_cols;
            lim[mt][e] = static_cast<int32_t>(v - (lane & 31));
            thf[mt][e] = SAMPLE ? 0.0f : thr_float(thr[tc - t0]);
            // rows past the chunk get an offset past the buffer, so their
            // stores are dropped
            soff[mt][e] = ok ? static_cast<uint32_t>(((t - qb) * ld_s + (lane & 31)) * 4) : 0x80000000u;
        }
    // the wave's 8 candidate rows (sample rows: SAMPLE) as one buffer (byte
    // range below 2^31, which the launch checks; rows past the chunk are
    // outside the range)
    int64_t rows_here = t1 - qb;
    rows_here = rows_here < 0 ? 0 : (rows_here > 8 ? 8 : rows_here);
    const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
        SAMPLE ? static_cast<void*>(samp + (qb < t1 ? qb - t0 : 0) * ld_s)
               : static_cast<void*>(cand + (qb < t1 ? qb - t0 : 0) * g.cand_ld),
        static_cast<short>(0), static_cast<int>(rows_here * (SAMPLE ? ld_s * 4 : g.cand_ld * 8)), 0x00020000);
    // uniform slot of the next candidate of wave row q (4mt + query) in the
    // wave's buffer: q * cand_ld + the workgroup's first slot + the count so far
    const uint32_t slot0 = static_cast<uint32_t>(bx * (kSub * g.blocks));
    uint32_t c_pos[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) c_pos[q] = static_cast<uint32_t>(q * g.cand_ld) + slot0;
    uint32_t hmask = hi ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(hmask));    // keep the masked xor below from becoming a select

    // tile loader: thread -> chunk c = tid / 32 of key (tid % 32) in each of
    // the tile's 4 column blocks.  Consecutive candidate tiles are 128 keys
    // (two 64-key cache tiles, 32 KiB) apart, so the addresses advance by a
    // constant; a tile reaching past the cache clamps per key.
    const int lc = tid >> 5, lk = tid & 31;
    uint4 n0, n1, n2, n3;
    // candidate pass: the workgroup's keys [kbase, cap) of the cache as one
    // buffer (reads past it return 0; such keys are never visible), chunk lc
    // of key lk at voff within a 64-key cache tile, the tile's four column
    // blocks at uniform offsets
    const int64_t kbase = SAMPLE ? 0 : bx * g.blocks * kSub;
    int64_t krem = SAMPLE ? 0 : (a.cap - kbase) * (kNch * 16);
    krem = krem < 0 ? 0 : (krem > 0x7fffffffLL ? 0x7fffffffLL : krem);
    const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.kc) + (SAMPLE ? 0 : kbase * (kNch * 16)), static_cast<short>(0),
        static_cast<int>(krem), 0x00020000);
    const int voff = (lc * 64 + lk) * 16;
    auto load_tile = [&](int tile) {
        if (!SAMPLE) {
            const int so = tile * (2 * kNch * 64 * 16);   // two cache tiles per candidate tile
            n0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krsrc, voff, so, 0));
            n1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krsrc, voff, so + 32 * 16, 0));
            n2 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krsrc, voff, so + kNch * 64 * 16, 0));
            n3 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krsrc, voff, so + (kNch * 64 + 32) * 16, 0));
        } else {
            int64_t p0 = block_key(4 * tile + 0) + lk, p1 = block_key(4 * tile + 1) + lk;
            int64_t p2 = block_key(4 * tile + 2) + lk, p3 = block_key(4 * tile + 3) + lk;
            n0 = *kchunk(a.kc, p0 < a.cap ? p0 : 0, lc);
            n1 = *kchunk(a.kc, p1 < a.cap ? p1 : 0, lc);
            n2 = *kchunk(a.kc, p2 < a.cap ? p2 : 0, lc);
            n3 = *kchunk(a.kc, p3 < a.cap ? p3 : 0, lc);
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* d = &Ks[buf][lk * KROW + 8 * lc];
        *reinterpret_cast<uint4*>(d) = n0;
        *reinterpret_cast<uint4*>(d + kSub * KROW) = n1;
        *reinterpret_cast<uint4*>(d + 2 * kSub * KROW) = n2;
        *reinterpret_cast<uint4*>(d + 3 * kSub * KROW) = n3;
    };
    // column block i of the tile in LDS buffer buf -> two 32 x 32 s tiles
    auto mfma_block = [&](int buf, int i, floatx16* acc) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8 kb = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4*>(&Ks[buf][(kSub * i + (lane & 31)) * KROW + 16 * s +
                                                                 8 * (lane >> 5)]));
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], kb, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], kb, acc[1], 0, 0, 0);
        }
    };
    // s~ of column block b (keys from jb) and what becomes of it; every block
    // is computed (loads of keys past the end read row 0) and invisible keys
    // are masked here
    // VIS false: every key of the block is visible to every row of the wave,
    // so no key needs the visibility test
    auto epilogue = [&](const floatx16* acc, int b, auto vis_tag) {
        constexpr bool VIS = decltype(vis_tag)::value;
        const int64_t jb = block_key(b);
        const int32_t jb32 = static_cast<int32_t>(jb < 0x7fffffff ? jb : 0x7fffffff);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            float part[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                float p = wr[mt][4 * qq] * relu(acc[mt][4 * qq]);
#pragma unroll
                for (int h = 1; h < 4; ++h) p = fmaf(wr[mt][4 * qq + h], relu(acc[mt][4 * qq + h]), p);
                part[qq] = p;
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[e]),
                                                                 __float_as_uint(part[2 + e]), false, false);
                const float v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                const bool vis_ok = !VIS || jb32 < lim[mt][e];
                if (SAMPLE) {
                    // unconditional: a slot past the row's groups is past the
                    // buffer (bit 31), and the hardware drops the store.  (A
                    // guarded store made the compiler wait for every store
                    // before the next tile's staging.)
                    const int64_t gi = jb / kGroup;
                    const uint32_t off = (soff[mt][e] + static_cast<uint32_t>(gi * kSub * 4)) |
                                         (gi * kSub < ld_s ? 0u : 0x80000000u);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vis_ok ? v : -__builtin_inff()), crsrc,
                                                          static_cast<int>(off), 0, 0);
                } else {
                    // (s~ bits, position) of taken keys go straight to the
                    // row's next slots, in position order: the lower half of
                    // the wave holds row qlo, the upper half row qhi.  Lanes
                    // that take nothing store past the buffer's range, which
                    // the hardware drops, so the store needs no branch.
                    // an invisible key compares as NaN, so the ballot is one compare
                    const float vt = vis_ok ? v : __builtin_nanf("");
                    const bool take = vt >= thf[mt][e];
                    const uint64_t bal = __builtin_amdgcn_ballot_w64(take);
                    const uint32_t blo = static_cast<uint32_t>(bal), bhi = static_cast<uint32_t>(bal >> 32);
                    const uint32_t n_lo = static_cast<uint32_t>(__builtin_popcount(blo));
                    const uint32_t n_hi = static_cast<uint32_t>(__builtin_popcount(bhi));
                    const int qlo = 4 * mt + e, qhi = 4 * mt + 2 + e;
                    // the upper lanes' prefix count includes the n_lo lower
                    // lanes, so their base is lowered by n_lo; the select of
                    // the two uniform bases is a masked xor
                    const uint32_t x = c_pos[qlo] ^ (c_pos[qhi] - n_lo);
                    const uint32_t base = c_pos[qlo] ^ (x & hmask);
                    const uint32_t at = __builtin_amdgcn_mbcnt_hi(bhi, __builtin_amdgcn_mbcnt_lo(blo, base));
                    // (every real offset is below 2^31; bit 31 marks the rest)
                    const uint32_t off = (at << 3) | (static_cast<uint32_t>(!take) << 31);
                    u32x2 val;
                    val[0] = __float_as_uint(v);
                    val[1] = static_cast<uint32_t>(jb32) + (lane & 31);
                    __builtin_amdgcn_raw_buffer_store_b64(val, crsrc, static_cast<int>(off), 0, 0);
                    c_pos[qlo] += n_lo;
                    c_pos[qhi] += n_hi;
                }
            }
        }
    };

    // software pipeline: the matrix products of column block b + 1 are
    // issued beside the epilogue of block b (two accumulator sets, blocks
    // alternate between them; 4 blocks per tile keep the parity per tile)
    floatx16 acc0[2], acc1[2];
    // one matrix product, then a share of the other block's epilogue: in-order
    // issue would otherwise run the 16 products first and the epilogue after
    auto interleave = [&]() {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);    // VALU
        }
    };
    // tile t + 1 is loaded into registers a whole tile ahead (before the last
    // block's candidate stores of tile t - 1), so the wait before its LDS
    // write covers only stores issued a tile earlier
    load_tile(0);
    store_tile(0);
    if (n_tiles > 1) load_tile(1);
    __syncthreads();
    mfma_block(0, 0, acc0);
    // the smallest visible count of the wave's rows (0 if a row lies past the
    // chunk): vis grows with t, so it is the first row's
    int64_t min_vis = qb + 7 < t1 ? vis_of(a, qb) : 0;
    if (min_vis > n_cols) min_vis = n_cols;
    auto tile_body = [&](int tile, auto vis_tag) {
        const int buf = tile & 1;
        mfma_block(buf, 1, acc1);
        epilogue(acc0, 4 * tile + 0, vis_tag);
        interleave();
        mfma_block(buf, 2, acc0);
        epilogue(acc1, 4 * tile + 1, vis_tag);
        interleave();
        mfma_block(buf, 3, acc1);
        epilogue(acc0, 4 * tile + 2, vis_tag);
        interleave();
        if (tile + 1 < n_tiles) store_tile(buf ^ 1);
        if (tile + 2 < n_tiles) load_tile(tile + 2);
        __syncthreads();
        if (tile + 1 < n_tiles) mfma_block(buf ^ 1, 0, acc0);
        epilogue(acc1, 4 * tile + 3, vis_tag);
    };
    // keys grow with the tile index: the leading tiles whose last key is
    // below min_vis run without the test, the rest with it
    int n_fast = 0;
    if (!SAMPLE) {
        const int64_t f = (min_vis / kSub - bx * g.blocks) / 4;
        n_fast = static_cast<int>(f < 0 ? 0 : (f > n_tiles ? n_tiles : f));
    }
    int tile = 0;
    for (; tile < n_fast; ++tile) tile_body(tile, std::false_type{});
    for (; tile < n_tiles; ++tile) tile_body(tile, std::true_type{});
    if (!SAMPLE && lane < 8) {
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) c = lane == q ? c_pos[q] - static_cast<uint32_t>(q * g.cand_ld) - slot0 : c;
        const int64_t t = qb + lane;
        if (t < t1) counts[(t - t0) * g.cnt_ld + bx] = c;
    }
}

// ---------------------------------------------------------------- threshold
// L_t per row: rows with vis <= k need no candidates (all chosen); rows with
// vis <= kCandCap take every visible key; otherwise L_t is the j-th largest
// sampled s~, j = round(target * n_s / vis) with n_s visible sampled keys and
// about target = min(3k, (k + kCandCap) / 2) keys expected at or above it.
// A sample row of up to kSampReg keys is selected from registers (16 per
// thread); longer rows are read from the workspace in radix passes.
constexpr int kSampReg = 16384;
constexpr int kSampPerThread = kSampReg / kThreads;
__global__ __launch_bounds__(kThreads) void sample_thresh_kernel(int64_t t0, PfArgs a, const float* __restrict__ samp,
                                                                 int64_t ld_s, uint32_t* __restrict__ thr) {
    __shared__ SelLds sh;
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wave_tot[kWaves];
    __shared__ uint32_t res[2];
    const int64_t r = blockIdx.x;
    const int64_t vis = vis_of(a, t0 + r);
    if (vis <= a.k) {
        if (threadIdx.x == 0) thr[r] = 0xffffffffu;
        return;
    }
    if (vis <= kCandCap) {
        if (threadIdx.x == 0) thr[r] = 1u;
        return;
    }
    int64_t n = (vis + kGroup - 1) / kGroup * kSub;
    if (n > ld_s) n = ld_s;
    const float* s = samp + r * ld_s;
    const double target = fmin(3.0 * a.k, 0.5 * (a.k + kCandCap));
    auto rank_of = [&](uint32_t n_s) {
        const double jd = target * static_cast<double>(n_s) / static_cast<double>(vis) + 0.5;
        uint32_t j = static_cast<uint32_t>(jd);
        if (j < 1u) j = 1u;
        if (j > n_s) j = n_s;
        return j;
    };
    uint32_t T = 1u;
    if (n <= kSampReg) {
        // slot i = j * kThreads + tid (0 = empty past n)
        uint32_t kk[kSampPerThread];
#pragma unroll
        for (int j = 0; j < kSampPerThread; ++j) {
            const int64_t i = static_cast<int64_t>(j) * kThreads + threadIdx.x;
            kk[j] = i < n ? key_of(s[i]) : 0u;
        }
        uint32_t mn, mx;
        const uint32_t n_s = sel_stats<kSampPerThread>(kk, sh, mn, mx);
        if (n_s > 0) {
            // L_t: the lower edge of the radix bin that holds the j-th
            // largest sample (at least j samples lie at or above it)
            uint32_t need = rank_of(n_s), hi_unused;
            sel_bracket<kSampPerThread>(kk, mn, mx, need, sh, T, hi_unused);
        }
    } else {
        auto get = [&](int64_t i) { return key_of(s[i]); };
        const uint32_t n_s = count_valid(get, n, wave_tot);
        uint32_t need = 0;
        if (n_s > 0) radix_select(get, n, rank_of(n_s), hist, res, T, need);
    }
    if (threadIdx.x == 0) thr[r] = T > 0u ? T : 1u;
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

// head h's channel chain of the same exact score: d_h with the channels in
// order (exact_score keeps all heads in one thread; this splits them over 8
// lanes, each chain unchanged)
__device__ float exact_head(const float* qf, const uint8_t* kc, int64_t pos, int h) {
    float d = 0.0f;
    const float* qh = qf + h * kDim;
#pragma unroll 4
    for (int c = 0; c < kNch; ++c) {
        const uint4 v = *kchunk(kc, pos, c);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ch = 8 * c + 2 * e;
            d = fmaf(qh[ch], bf16_lo(u[e]), d);
            d = fmaf(qh[ch + 1], bf16_hi(u[e]), d);
        }
    }
    return d;
}

constexpr int kCandPerThread = kCandCap / kThreads;   // candidates held in registers during selection
static_assert(kCandCap % kThreads == 0, "candidates split evenly over the threads");
static_assert(sizeof(SelLds) <= 4 * kCandCap + 12 * kBandCap, "selection LDS fits over the keys and band arrays");

__global__ __launch_bounds__(kThreads) void cand_final_kernel(int64_t t0, PfArgs a, const float* __restrict__ eps,
                                                              const uint32_t* __restrict__ thr,
                                                              const uint32_t* __restrict__ counts, int64_t cnt_ld,
                                                              int64_t cand_ld, int64_t kpw,
                                                              uint2* __restrict__ cand_all,
                                                              int32_t* __restrict__ out) {
    // candidate keys (s~ bits, then order keys), band entries and band
    // candidate indices; the selection's histograms take their place while
    // the keys are held in registers.  Positions stay put.
    __shared__ union CandLds {
        struct {
            uint32_t key[kCandCap];
            uint64_t band[kBandCap];
            uint32_t sel[kBandCap];
        } c;
        SelLds sh;
    } u_lds;
    __shared__ uint32_t cpos[kCandCap];
    uint32_t* ckey = u_lds.c.key;
    uint64_t* band = u_lds.c.band;
    uint32_t* sel = u_lds.c.sel;
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
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t* o = out + t * static_cast<int64_t>(k);
    const uint32_t k_eff = vis < k ? static_cast<uint32_t>(vis) : static_cast<uint32_t>(k);
    if (vis <= k) {                                   // every visible entry is chosen
        for (int64_t i = tid; i < k; i += kThreads) o[i] = i < vis ? static_cast<int32_t>(i) : -1;
        return;
    }
    // query row in float32 (exact widening of bf16)
    for (int i = tid; i < kHeads * kDim; i += kThreads) {
        const uint16_t b = a.q[t * kHeads * kDim + i];
        qf[i] = __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    if (tid < kHeads) wf[tid] = a.w[t * kHeads + tid];
    const uint32_t* crow = counts + r * cnt_ld;
    uint2* region = cand_all + r * cand_ld;
    const int64_t n_seg = (vis + kpw - 1) / kpw;   // workgroups that saw visible keys

    // total candidates
    // (the first kThreads counts stay in registers for the gather)
    const uint32_t cnt0 = tid < n_seg ? crow[tid] : 0u;
    uint32_t part = cnt0;
    for (int64_t sgi = tid + kThreads; sgi < n_seg; sgi += kThreads) part += crow[sgi];
    part = wave_sum(part);
    if (lane == 0) wave_tot[wv] = part;
    __syncthreads();
    uint32_t C = 0;
    for (int i = 0; i < kWaves; ++i) C += wave_tot[i];
    __syncthreads();
    const uint32_t L = thr[r];
    bool fallback = C > static_cast<uint32_t>(kCandCap) || C < k_eff;
    if (!fallback) {
        // gather the segments into LDS: hist[0..1023] = segment offsets,
        // hist[1024..2047] = counts, 1,024 segments at a time
        uint32_t running = 0;
        for (int64_t sb = 0; sb < n_seg; sb += kThreads) {
            const int64_t sgi = sb + tid;
            const uint32_t c = sb == 0 ? cnt0 : (sgi < n_seg ? crow[sgi] : 0u);
            const uint32_t incl = wave_incl_sum(c);
            if (lane == 63) wave_tot[wv] = incl;
            __syncthreads();
            uint32_t before = 0, tot = 0;
            for (int i = 0; i < kWaves; ++i) {
                before += i < wv ? wave_tot[i] : 0u;
                tot += wave_tot[i];
            }
            hist[tid] = running + before + incl - c;
            hist[1024 + tid] = c;
            __syncthreads();
            const int n_here = static_cast<int>(n_seg - sb < kThreads ? n_seg - sb : kThreads);
            for (int s = wv; s < n_here; s += kWaves) {
                const uint32_t so = hist[s], sc = hist[1024 + s];
                const uint2* src = region + (sb + s) * kpw;
                // eight loads in flight per lane, then their LDS writes
                for (uint32_t i0 = 0; i0 < sc; i0 += 64 * 8) {
                    uint2 cv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const uint32_t i = i0 + lane + 64 * u;
                        if (i < sc) cv[u] = src[i];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const uint32_t i = i0 + lane + 64 * u;
                        if (i < sc) {
                            ckey[so + i] = cv[u].x;
                            cpos[so + i] = cv[u].y;
                        }
                    }
                }
            }
            running += tot;
            __syncthreads();
        }
        // keys of s~ (candidates hold the float bits) into registers, slot
        // i = j * kThreads + tid (0 = empty past C)
        uint32_t kk[kCandPerThread];
#pragma unroll
        for (int j = 0; j < kCandPerThread; ++j) {
            const uint32_t i = static_cast<uint32_t>(j * kThreads + tid);
            kk[j] = i < C ? key_of(__uint_as_float(ckey[i])) : 0u;
        }
        __syncthreads();
        // [T_lo, T_hi]: one radix bin that holds tau~, the k-th largest s~ (of
        // the candidates, and of the row)
        uint32_t T_lo, T_hi;
        {
            uint32_t mn, mx, need = k_eff;
            sel_stats<kCandPerThread>(kk, u_lds.sh, mn, mx);
            sel_bracket<kCandPerThread>(kk, mn, mx, need, u_lds.sh, T_lo, T_hi);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kCandPerThread; ++j) {
            const uint32_t i = static_cast<uint32_t>(j * kThreads + tid);
            if (i < C) ckey[i] = kk[j];
        }
        __syncthreads();
        const float e2 = 2.0f * eps[t];
        const uint32_t hi_key = key_of(next_up(float_of_key(T_hi) + e2));
        const uint32_t lo_raw = key_of(next_down(float_of_key(T_lo) - e2));
        const uint32_t lo_key = lo_raw > 0u ? lo_raw : 1u;
        if (tid < 2) counters[tid] = 0;
        __syncthreads();
        if (lo_key < L) {
            fallback = true;                          // the band reaches below L_t
        } else {
            // sure picks (s~ above the band) are counted; band keys go to
            // band[] as candidate indices
            uint32_t n_sure = 0;
            for (uint32_t i = tid; i < C; i += kThreads) {
                const uint32_t ck = ckey[i];
                if (ck > hi_key) {
                    ++n_sure;
                } else if (ck >= lo_key) {
                    const uint32_t at = atomicAdd(&counters[1], 1u);
                    if (at < static_cast<uint32_t>(kBandCap)) band[at] = i;
                }
            }
            n_sure = wave_sum(n_sure);
            if (lane == 0) atomicAdd(&counters[0], n_sure);
            __syncthreads();
            const uint32_t n_in = counters[0], n_band = counters[1];
            if (n_band > static_cast<uint32_t>(kBandCap) || n_in > k_eff || n_in + n_band < k_eff) {
                fallback = true;
            } else {
                // exact scores of the band keys, ranked by (score desc,
                // position asc): entry = (~exact key << 32) | position, the
                // need_b smallest entries are chosen
                // (8 lanes per band key, lane h%8 running head h's chain;
                // the head sum is then taken in head order by the first)
                for (uint32_t i = tid >> 3; i < n_band; i += kThreads / 8) {
                    const uint32_t ci = static_cast<uint32_t>(band[i]);
                    const uint32_t pos = cpos[ci];
                    const int h = tid & 7;
                    const float d = exact_head(qf, a.kc, pos, h);
                    float sc = 0.0f;
#pragma unroll
                    for (int hh = 0; hh < kHeads; ++hh) {
                        const float dh = __shfl(d, (lane & ~7) + hh);
                        sc = fmaf(wf[hh], dh > 0.0f ? dh : 0.0f, sc);
                    }
                    if (h == 0) {
                        const uint32_t ek = key_of(sc);
                        band[i] = (static_cast<uint64_t>(~ek) << 32) | pos;
                        sel[i] = ci;
                    }
                }
                __syncthreads();
                const uint32_t need_b = k_eff - n_in;
                // rank of each band entry among the band (entries are distinct:
                // positions differ); chosen ones are marked by setting their
                // candidate key to ~0u (above every real key)
                for (uint32_t i = tid; i < n_band; i += kThreads) {
                    const uint64_t x = band[i];
                    uint32_t rank = 0;
                    for (uint32_t j2 = 0; j2 < n_band; ++j2) rank += band[j2] < x;
                    if (rank < need_b) ckey[sel[i]] = 0xffffffffu;
                }
                __syncthreads();
                // ordered emission: candidates are in position order
                // (thread tid owns candidates [tid * per, (tid + 1) * per),
                // so one workgroup scan orders every pick)
                const uint32_t per = (C + kThreads - 1) / kThreads;
                const uint32_t c0 = tid * per, c1 = c0 + per < C ? c0 + per : C;
                uint32_t mine = 0;
                for (uint32_t i = c0; i < c1; ++i) mine += ckey[i] > hi_key ? 1u : 0u;
                uint32_t tot;
                uint32_t at = block_excl_scan(mine, wave_tot, tot);
                for (uint32_t i = c0; i < c1; ++i) {
                    if (ckey[i] > hi_key) {
                        if (at < k_eff) o[at] = static_cast<int32_t>(cpos[i]);
                        ++at;
                    }
                }
            }
        }
    }
    if (fallback) {
        // exact scores for the whole visible row, kept in the row's slot
        // range (8 bytes reserved per visible key)
        float* s = reinterpret_cast<float*>(region);
        __syncthreads();
        for (int64_t i = tid; i < vis; i += kThreads) s[i] = exact_score(qf, wf, a.kc, i);
        __threadfence_block();
        __syncthreads();
        uint32_t T = 0, need = 0;
        auto get = [&](int64_t i) { return key_of(s[i]); };
        radix_select(get, vis, k_eff, hist, res, T, need);
        emit_ordered(get, vis, T, need, k_eff, nullptr, o, k, wave_tot);
    }
    for (int64_t i = k_eff + tid; i < k; i += kThreads) o[i] = -1;
}

__global__ void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

struct PfWs {
    uint32_t* kmax;
    float* eps;
    float* samp;        // [rows][ld_s]
    uint32_t* thr;      // [rows]
    uint32_t* counts;   // [rows][cnt_ld]
    uint2* cand;        // [rows][cand_ld]
    int64_t ld_s, cnt_ld, cand_ld;
};

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

struct PfSizes {
    int64_t rows, ld_s, cnt_ld, cand_ld;
    size_t kmax, eps, samp, thr, counts, cand;
    size_t total() const { return kmax + eps + samp + thr + counts + cand; }
};

// Candidate slots per row: a workgroup's slot range is its key range, and the
// ranges cover [0, cols) with less than one range (<= kMaxKeysPerWG keys) of
// overshoot.  Count entries per row: one per workgroup, at least 128 keys each.
PfSizes sizes_of(int64_t T, int64_t n_cols) {
    PfSizes z;
    z.rows = T < kChunkRows ? T : kChunkRows;
    z.ld_s = (n_cols + kGroup - 1) / kGroup * kSub;
    z.cnt_ld = (n_cols + kTileKeys - 1) / kTileKeys + 8;
    z.cand_ld = (n_cols + kTileKeys - 1) / kTileKeys * kTileKeys + kMaxKeysPerWG;
    z.kmax = 256;
    z.eps = align256(static_cast<size_t>(T) * 4);
    z.samp = align256(static_cast<size_t>(z.rows) * z.ld_s * 4);
    z.thr = align256(static_cast<size_t>(z.rows) * 4);
    z.counts = align256(static_cast<size_t>(z.rows) * z.cnt_ld * 4);
    z.cand = align256(static_cast<size_t>(z.rows) * z.cand_ld * 8);
    return z;
}

PfWs carve(void* ws, int64_t T, int64_t n_cols) {
    const PfSizes z = sizes_of(T, n_cols);
    PfWs w;
    char* p = static_cast<char*>(ws);
    w.kmax = reinterpret_cast<uint32_t*>(p); p += z.kmax;
    w.eps = reinterpret_cast<float*>(p); p += z.eps;
    w.samp = reinterpret_cast<float*>(p); p += z.samp;
    w.thr = reinterpret_cast<uint32_t*>(p); p += z.thr;
    w.counts = reinterpret_cast<uint32_t*>(p); p += z.counts;
    w.cand = reinterpret_cast<uint2*>(p); p += z.cand;
    w.ld_s = z.ld_s;
    w.cnt_ld = z.cnt_ld;
    w.cand_ld = z.cand_ld;
    return w;
}

int64_t cdiv(int64_t x, int64_t y) { return (x + y - 1) / y; }

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Split `units` column blocks (32 keys each) of n_y query blocks over
// workgroups of a multiple of 4 blocks, sized so the grid fills whole rounds
// of one workgroup per CU (about `per_wg` blocks each), numbered XCD-aware.
Geo make_geo(int64_t units, int n_y, int64_t per_wg, int64_t max_blocks, int n_cu) {
    Geo g;
    g.n_y = n_y;
    int64_t rounds = (units * n_y + per_wg * n_cu / 2) / (per_wg * n_cu);
    if (rounds < 1) rounds = 1;
    const int64_t want_x = (cdiv(n_cu * rounds, n_y) + 7) / 8 * 8;
    int64_t blocks = (cdiv(units, want_x) + 3) / 4 * 4;
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 4) blocks = 4;
    g.blocks = static_cast<int32_t>(blocks);
    g.n_x = cdiv(units, blocks);
    g.xcd = 1;
    g.cand_ld = 0;
    g.cnt_ld = 0;
    return g;
}

unsigned grid_of(const Geo& g) { return static_cast<unsigned>((g.n_x + 7) / 8 * 8 * g.n_y); }

}  // namespace

int64_t prefill_cols(int64_t T, int32_t ctx_len, int64_t q_pos0, int32_t m) {
    if (T <= 0) return 0;
    int64_t v = (q_pos0 + T) / m;
    return v < ctx_len ? v : ctx_len;
}

size_t prefill_topk_workspace_bytes(int64_t T, int32_t ctx_len, int64_t q_pos0, int32_t m) {
    if (T <= 0) return 0;
    return sizes_of(T, prefill_cols(T, ctx_len, q_pos0, m)).total();
}

int prefill_topk_max_k() { return kKCap; }

int64_t prefill_topk_max_cols() { return int64_t(1) << 24; }

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
    const int n_cu = cu_count();
    for (int64_t t0 = 0; t0 < L.T; t0 += kChunkRows) {
        const int64_t t1 = t0 + kChunkRows < L.T ? t0 + kChunkRows : L.T;
        const int64_t rows = t1 - t0;
        const int64_t cols = prefill_cols(t1, L.ctx_len, L.q_pos0, L.m);   // widest row of the chunk
        const int qblocks = static_cast<int>(cdiv(rows, kQB));
        if (cols > kCandCap) {
            if (8 * 4 * w.ld_s > 0x7fffffffLL) return hipErrorInvalidValue;   // a wave's sample rows as one buffer
            Geo gs = make_geo(cdiv(cols, kGroup), qblocks, 16, 1 << 20, n_cu);
            score_mfma_kernel<true><<<grid_of(gs), 512, 0, st>>>(a, t0, t1, cols, gs, w.samp, w.ld_s, nullptr,
                                                                  nullptr, nullptr);
        }
        sample_thresh_kernel<<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(t0, a, w.samp, w.ld_s, w.thr);
        int64_t kpw = kTileKeys;
        if (cols > 0) {
            Geo gc = make_geo(cdiv(cols, kSub), qblocks, 8192 / kSub, kMaxKeysPerWG / kSub, n_cu);
            gc.cand_ld = w.cand_ld;
            if (8 * 8 * w.cand_ld > 0x7fffffffLL) return hipErrorInvalidValue;
            gc.cnt_ld = w.cnt_ld;
            kpw = static_cast<int64_t>(gc.blocks) * kSub;
            score_mfma_kernel<false><<<grid_of(gc), 512, 0, st>>>(a, t0, t1, cols, gc, nullptr, 0, w.thr, w.counts,
                                                                   w.cand);
        }
        cand_final_kernel<<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(t0, a, w.eps, w.thr, w.counts,
                                                                                  w.cnt_ld, w.cand_ld, kpw, w.cand,
                                                                                  L.out);
    }
    return hipGetLastError();
}

}  // namespace csa2
