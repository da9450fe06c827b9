// Sparse-indexer scoring for gfx950 (decode Full scan, Reindex pool scan,
// and the plain per-query prefill scan).
//
// Score ("DeepSeek-V4.1-Flash KV Cache Compression" notes, sections 2-3, give
// the roles: a per-layer indexer Q scores an indexer K shared by all heads):
//     d_h = fma chain over channels c = 0..d_I-1 of q[h][c] * k[c]
//     s   = fma chain over heads h = 0..H_I-1 of w[h] * max(d_h, +0)
// in float32, exactly in this order, so every score is bit-reproducible and
// the top-k that follows is exact.  The chain forces one lane per (position,
// head) to walk all channels in order, so each lane owns whole key rows.
//
// Design (HBM stream, VALU co-limited at ~1,180 VALU ops per 256-byte row):
//  * The indexer-K cache is stored tiled (64 positions per tile, 16-byte
//    chunks chunk-major: chunk c of position p of tile t at
//    ((t * NCH + c) * 64 + p) * 16).  A wave reading chunk c of its 64
//    positions reads 1 KiB of contiguous memory, and every lane receives its
//    own row's chunk directly in registers: no LDS staging, no barriers.
//  * Each lane owns two positions (two tiles), so every broadcast query value
//    feeds two fmas and the bf16 -> f32 widening costs one op per channel.
//  * The query, transposed to [d_I][H_I] float32, sits in LDS and is read
//    with same-address (broadcast) 16-byte reads; LDS completions are in
//    order, so reads for the next channel overlap the current fmas.  Each
//    wave scores one unit of 128 positions.  The workgroup's threads load
//    the query, issue their first key loads, and only then stage the query
//    and meet the barrier, which waits for LDS and not for the key loads.
//  * The block max over 8 positions (candidate-pool input, notes section 3)
//    is fused: 8 consecutive lanes own one block.
#include <type_traits>

#include "csa2_internal.h"

namespace csa2 {
namespace {

#include "mxfp4_quant.h"

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnit = 128;          // positions per wave iteration (2 tiles of 64)

struct ScoreArgs {
    int64_t cap, Tq;
    const int32_t* ctx_len;
    const int64_t* q_pos;
    int m;
    const int32_t* pool; int P_b;
    int64_t ld, ld_bm;
    int64_t n_slots;          // slots written per row
    int64_t units_per_row;    // ceil(n_slots / kUnit)
    int units_per_wg;
    int q_bf16;
    // decode write in the same launch (knew == nullptr: none).  Workgroup
    // column gx_scan of row b writes sequence b's new entry: its MXFP4 row
    // from wx and its indexer key from knew (ROWB bytes per row), to flat
    // row wdst[b], which must lie in sequence b (else nothing is written).
    // Lanes scoring that position read the key from knew, so no workgroup
    // of the launch reads what another one writes.
    const uint8_t* knew;
    const void* wx; int wx_bf16; int wD;
    const int64_t* wdst;
    uint8_t* wcodes; uint8_t* wscales;
    int64_t gx_scan;
};

template <int HI, int DI, bool KBF16, bool WR, bool FULL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void score_kernel(const void* __restrict__ q_all,
                                                         const float* __restrict__ w_all,
                                                         const uint8_t* __restrict__ k_all,
                                                         float* __restrict__ scores,
                                                         float* __restrict__ block_max,
                                                         ScoreArgs a) {
    constexpr int ESZ = KBF16 ? 2 : 4;
    constexpr int ROWB = DI * ESZ;        // bytes per key row
    constexpr int NCH = ROWB / 16;        // 16-byte chunks per row
    constexpr int CPC = 16 / ESZ;         // channels per chunk
    constexpr int G = NCH >= 4 ? 4 : NCH;  // chunks per streamed group
    static_assert(NCH % G == 0, "chunk groups must tile the row");
    static_assert(HI % 4 == 0 || HI == 2, "head count must be 2 or a multiple of 4");
    __shared__ __attribute__((aligned(16))) float qs[DI * HI];   // [c][h]

    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t row = blockIdx.y;       // query row (b * Tq + tq)
    const int64_t b = row / a.Tq;

    if (WR && static_cast<int64_t>(blockIdx.x) == a.gx_scan) {
        // the write column (decode: Tq == 1, row == b): threads [0, D/16)
        // quantise one 16-channel block each, the next NCH threads copy one
        // 16-byte chunk of the indexer key into the tiled cache
        const int64_t dst = a.wdst[b];
        if (dst < b * a.cap || dst >= (b + 1) * a.cap) return;
        const int nblk = a.wD / 16;
        if (t < nblk) {
            float v[16];
            if (a.wx_bf16) load_block<true>(a.wx, b, t, a.wD, v);
            else load_block<false>(a.wx, b, t, a.wD, v);
            quantise_block(v, t, a.wD, dst, a.wcodes, a.wscales);
        } else if (t < nblk + NCH) {
            const int c = t - nblk;
            const uint4 val = *reinterpret_cast<const uint4*>(a.knew + b * ROWB + c * 16);
            *reinterpret_cast<uint4*>(const_cast<uint8_t*>(k_all) + (((dst >> 6) * NCH + c) * 64 + (dst & 63)) * 16) = val;
        }
        return;
    }

    // This thread's share of the query: channel qc, heads qh .. qh+QH-1,
    // which is one contiguous run of the [c][h] layout in LDS.  Full scan
    // (FULL, no pool): loaded raw first and staged only after the wave's
    // first key loads are issued, so the query and key latencies overlap (the
    // barrier waits for LDS only, not for the key loads).  Pool scan: staged
    // first, before the pool lookup.
    constexpr int QH = HI < 4 ? HI : 4;           // heads per thread
    constexpr int QT = DI * HI / QH;              // threads that stage the query
    static_assert(QT <= kThreads, "query staging fits the workgroup");
    const bool q_thr = t < QT;
    const int qc = t / (HI / QH), qh = (t % (HI / QH)) * QH;
    uint32_t qraw[QH];                            // bf16 held unshifted until staged
    if (q_thr) {
        const int64_t q0 = row * HI * DI + static_cast<int64_t>(qh) * DI + qc;
        if (a.q_bf16) {
#pragma unroll
            for (int j = 0; j < QH; ++j) qraw[j] = static_cast<const uint16_t*>(q_all)[q0 + j * DI];
        } else {
#pragma unroll
            for (int j = 0; j < QH; ++j) qraw[j] = static_cast<const uint32_t*>(q_all)[q0 + j * DI];
        }
    }
    auto stage_q = [&]() {
        if (q_thr) {
            float v[QH];
#pragma unroll
            for (int j = 0; j < QH; ++j) v[j] = __uint_as_float(a.q_bf16 ? qraw[j] << 16 : qraw[j]);
            float* dst = qs + qc * HI + qh;
            if constexpr (QH == 4)
                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            else
#pragma unroll
                for (int j = 0; j < QH; ++j) dst[j] = v[j];
        }
        __syncthreads();
    };
    if constexpr (!FULL) stage_q();
    float wh[HI];
#pragma unroll
    for (int h = 0; h < HI; ++h) wh[h] = w_all[row * HI + h];

    const uint8_t* kb = k_all + b * a.cap * ROWB;        // cap is a multiple of 64
    const int32_t* pool = FULL ? nullptr : a.pool + row * a.P_b;
    int64_t vis = a.ctx_len[b];
    if (a.q_pos) {
        const int64_t v2 = (a.q_pos[row] + 1) / a.m;
        vis = v2 < vis ? v2 : vis;
    }
    vis = vis < a.cap ? vis : a.cap;

    auto pos_of = [&](int64_t slot) -> int64_t {   // -1 when not a visible position
        if (slot >= a.n_slots) return -1;
        int64_t pos = slot;
        if (pool) {
            const int32_t blk = pool[slot >> 3];
            if (blk < 0) return -1;
            pos = static_cast<int64_t>(blk) * 8 + (slot & 7);
        }
        return pos < vis ? pos : -1;
    };

    // position of the entry this launch writes for sequence b (-1: none);
    // the unit holding it reads that row's key from knew (16-byte chunk
    // stride) instead of the tiled cache (1 KiB chunk stride)
    int64_t np = -1;
    if (WR) {
        const int64_t d = a.wdst[b] - b * a.cap;
        np = (d >= 0 && d < a.cap) ? d : -1;
    }
    const uint8_t* knew_row = WR ? a.knew + b * ROWB : nullptr;

    // one unit per wave (units_per_wg == kWaves); a wave past the row's last
    // unit stages its query share and meets the barrier, then stops
    const int64_t u = static_cast<int64_t>(blockIdx.x) * a.units_per_wg + wv;
    const bool has_unit = u < a.units_per_row;
    int64_t slot[2], pos[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        slot[p] = u * kUnit + p * 64 + lane;
        pos[p] = pos_of(slot[p]);        // -1 past the row's slots
    }
    const bool has_new = WR && np >= 0 && __ballot(pos[0] == np || pos[1] == np) != 0;   // wave-uniform
    // Stream the row chunks in groups of G; the group loop is not unrolled
    // so the compiler cannot hoist every load and query read at once.  Every
    // load is unconditional: invisible positions read row 0 of the sequence
    // and are masked when the score is written, and the last group's "next"
    // load repeats the last group, so no load sits in a lane-divergent
    // branch.  In the Full scan the first group goes out before the query is
    // staged (with the tiled addressing; the unit holding the new entry
    // reloads it with its own).
    const uint8_t* base[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int64_t pp = pos[p] < 0 ? 0 : pos[p];
        base[p] = kb + ((pp >> 6) * NCH * 64 + (pp & 63)) * 16;
    }
    uint4 cur[2][G];
    if constexpr (FULL) {
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int p = 0; p < 2; ++p) cur[p][j] = *reinterpret_cast<const uint4*>(base[p] + j * 1024);
        stage_q();
    }
    if (!has_unit) return;

    auto unit = [&](auto newrow) {
        constexpr bool NR = decltype(newrow)::value;
        int cstride[2] = {1024, 1024};
        constexpr int NG = NCH / G;
        auto load_group = [&](uint4 (&dst)[2][G], int g) {
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    dst[p][j] = *reinterpret_cast<const uint4*>(base[p] + (g * G + j) * (NR ? cstride[p] : 1024));
        };
        if (NR) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
                if (pos[p] == np) { base[p] = knew_row; cstride[p] = 16; }
        }
        if (FULL && NR) load_group(cur, 0);
        float acc[2][HI];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int h = 0; h < HI; ++h) acc[p][h] = 0.0f;
        auto fma_group = [&](const uint4 (&src)[2][G], int g) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int c = g * G + j;
                float kv[2][CPC];
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    if (KBF16) {
                        const uint32_t wd[4] = {src[p][j].x, src[p][j].y, src[p][j].z, src[p][j].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            kv[p][2 * e] = __uint_as_float(wd[e] << 16);
                            kv[p][2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
                        }
                    } else {
                        kv[p][0] = __uint_as_float(src[p][j].x); kv[p][1] = __uint_as_float(src[p][j].y);
                        kv[p][2] = __uint_as_float(src[p][j].z); kv[p][3] = __uint_as_float(src[p][j].w);
                    }
                }
#pragma unroll
                for (int e = 0; e < CPC; ++e) {
                    const int ch = c * CPC + e;
                    float qv[HI];
                    if (HI % 4 == 0) {
#pragma unroll
                        for (int h4 = 0; h4 < HI / 4; ++h4) {
                            const float4 q4 = *reinterpret_cast<const float4*>(&qs[ch * HI + 4 * h4]);
                            qv[4 * h4] = q4.x; qv[4 * h4 + 1] = q4.y; qv[4 * h4 + 2] = q4.z; qv[4 * h4 + 3] = q4.w;
                        }
                    } else {
#pragma unroll
                        for (int h = 0; h < HI; ++h) qv[h] = qs[ch * HI + h];
                    }
#pragma unroll
                    for (int h = 0; h < HI; ++h) {
                        acc[0][h] = __builtin_fmaf(qv[h], kv[0][e], acc[0][h]);
                        acc[1][h] = __builtin_fmaf(qv[h], kv[1][e], acc[1][h]);
                    }
                }
            }
        };
        if constexpr (FULL) {
            // One group's fmas run while the next group's loads are in
            // flight.  The scheduling barriers keep those loads ahead of the
            // fmas and the cur = nxt copy behind them: left alone, the
            // scheduler moves each chunk's copy up to where the matching chunk
            // of cur is consumed (or folds the pair into load-then-wait), and
            // the wave then waits for a load it has just issued.
#pragma unroll 1
            for (int g = 0; g < NG; ++g) {
                const int gn = g + 1 < NG ? g + 1 : g;
                uint4 nxt[2][G];
                load_group(nxt, gn);
                __builtin_amdgcn_sched_barrier(0);
                fma_group(cur, g);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                    for (int p = 0; p < 2; ++p) cur[p][j] = nxt[p][j];
            }
        } else {
            // Pool scan (rows gathered through the pool): each group's loads
            // all go out, then its fmas consume them, with the other waves of
            // the CU hiding the latency; a prefetched next group measured
            // slower here.
#pragma unroll 1
            for (int g = 0; g < NG; ++g) {
                load_group(cur, g);
                if constexpr (!NR) __builtin_amdgcn_sched_barrier(0);   // (spills in the new-entry unit)
                fma_group(cur, g);
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float s = 0.0f;
#pragma unroll
            for (int h = 0; h < HI; ++h) s = __builtin_fmaf(wh[h], acc[p][h] > 0.0f ? acc[p][h] : 0.0f, s);
            if (pos[p] < 0) s = -__builtin_inff();
            if (slot[p] < a.n_slots) scores[row * a.ld + slot[p]] = s;
            if (block_max) {
                float mx = s;
                mx = fmaxf(mx, __shfl_xor(mx, 1));
                mx = fmaxf(mx, __shfl_xor(mx, 2));
                mx = fmaxf(mx, __shfl_xor(mx, 4));
                if (mx == 0.0f) mx = 0.0f;
                const int64_t blk = slot[p] >> 3;
                if ((lane & 7) == 0 && blk < a.ld_bm) block_max[row * a.ld_bm + blk] = mx;
            }
        }
    };
    if (has_new) unit(std::true_type{});
    else unit(std::false_type{});
}

template <int HI, int DI, bool KBF16>
hipError_t launch_typed(const ScoreLaunch& p, hipStream_t st) {
    const int64_t rows = p.B * p.Tq;
    ScoreArgs a;
    a.cap = p.cap; a.Tq = p.Tq; a.ctx_len = p.ctx_len; a.q_pos = p.q_pos; a.m = p.m;
    a.pool = p.pool; a.P_b = p.P_b;
    a.ld = p.ld; a.ld_bm = p.ld_bm;
    a.n_slots = p.pool ? static_cast<int64_t>(p.P_b) * 8 : p.ld;
    a.units_per_row = (a.n_slots + kUnit - 1) / kUnit;
    a.q_bf16 = p.q_bf16;
    // one unit per wave: each workgroup reads 4 consecutive units (128 KiB
    // of keys at d_I = 128), so the workgroups in flight at any time read a
    // compact, moving window of the cache.  Measured at 1M entries x 64 rows
    // this reads 13% faster than fewer, longer workgroups (5.75 against
    // 5.05 TB/s); the query staging per workgroup costs 2 KiB.
    const int64_t upw = kWaves;
    a.units_per_wg = static_cast<int>(upw);
    const int64_t gx = (a.units_per_row + upw - 1) / upw;
    a.knew = static_cast<const uint8_t*>(p.knew);
    a.wx = p.wx; a.wx_bf16 = p.wx_bf16; a.wD = p.wD; a.wdst = p.wdst;
    a.wcodes = p.wcodes; a.wscales = p.wscales;
    a.gx_scan = gx;
    const int64_t gx_all = gx + (p.knew ? 1 : 0);   // one more column writes the new entries
    if (gx_all == 0 || rows == 0) return hipGetLastError();
    // the write's code paths are a separate instantiation, so a scan without
    // a write keeps its own register allocation
    const dim3 grid(static_cast<unsigned>(gx_all), static_cast<unsigned>(rows));
    const uint8_t* kx = static_cast<const uint8_t*>(p.k_idx);
    if (p.knew && !p.pool)
        score_kernel<HI, DI, KBF16, true, true><<<grid, kThreads, 0, st>>>(p.q_idx, p.w, kx, p.scores, p.block_max, a);
    else if (p.knew)
        score_kernel<HI, DI, KBF16, true, false><<<grid, kThreads, 0, st>>>(p.q_idx, p.w, kx, p.scores, p.block_max, a);
    else if (!p.pool)
        score_kernel<HI, DI, KBF16, false, true><<<grid, kThreads, 0, st>>>(p.q_idx, p.w, kx, p.scores, p.block_max, a);
    else
        score_kernel<HI, DI, KBF16, false, false><<<grid, kThreads, 0, st>>>(p.q_idx, p.w, kx, p.scores, p.block_max, a);
    return hipGetLastError();
}

}  // namespace

bool score_shape_supported(int H_I, int d_I) {
    return (H_I == 8 && d_I == 128) || (H_I == 2 && d_I == 32) || (H_I == 4 && d_I == 64);
}

hipError_t launch_score(const ScoreLaunch& p, hipStream_t st) {
#define CSA2_SCORE_CASE(HI, DI)                                                         \
    if (p.H_I == HI && p.d_I == DI)                                                     \
        return p.k_bf16 ? launch_typed<HI, DI, true>(p, st) : launch_typed<HI, DI, false>(p, st);
    CSA2_SCORE_CASE(8, 128)
    CSA2_SCORE_CASE(2, 32)
    CSA2_SCORE_CASE(4, 64)
#undef CSA2_SCORE_CASE
    return hipErrorInvalidValue;
}

}  // namespace csa2
