// Sparse-indexer scoring for gfx950 (decode Full scan, Reindex pool scan,
// and the plain per-query prefill scan).
//
// Score ("DeepSeek-V4.1-Flash KV Cache Compression" notes, sections 2-3, give
// the roles: a per-layer indexer Q scores an indexer K shared by all heads):
//     d_h = fma chain over channels c = 0..d_I-1 of q[h][c] * k[c]
//     s   = fma chain over heads h = 0..H_I-1 of w[h] * max(d_h, +0)
// in float32, exactly in this order, so every score is bit-reproducible and
// the top-k that follows is exact.
//
// Design (HBM-bound stream, VALU co-limited):
//  * one thread owns one position (one key row) and computes all H_I chains,
//    so each widened key value feeds H_I fmas and the bf16->f32 widening
//    costs one op per channel;
//  * the query is pre-transposed to [d_I][H_I] float32 so a channel's H_I
//    weights are one uniform 32-byte scalar load (SGPR operands of v_fma);
//  * key rows are streamed with coalesced 16-byte loads into registers one
//    256-row tile ahead, then stored to LDS with a 16-byte-chunk XOR swizzle
//    (chunk c of row r at c ^ (r % chunks)) so the per-thread row reads are
//    bank-conflict free;
//  * the block max over 8 positions (candidate-pool input, notes section 3)
//    is fused: 8 consecutive lanes own one block.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kTile = 256;   // positions per tile = threads per workgroup

struct ScoreArgs {
    const float* qT;    // [rows][d_I][H_I]
    const float* w;     // [rows][H_I]
    const uint8_t* k;   // [B][cap][d_I] raw bytes
    int64_t cap, Tq;
    const int32_t* ctx_len;
    const int64_t* q_pos;
    int m;
    const int32_t* pool; int P_b;
    float* scores; int64_t ld;
    float* block_max; int64_t ld_bm;
    int64_t n_slots;      // slots written per row
    int64_t tiles_per_row;
    int tiles_per_wg;
};

template <int HI, int DI, bool KBF16>
__global__ __launch_bounds__(kTile) void score_kernel(const float* __restrict__ qT_all,
                                                      const float* __restrict__ w_all,
                                                      const uint8_t* __restrict__ k_all,
                                                      float* __restrict__ scores,
                                                      float* __restrict__ block_max,
                                                      ScoreArgs a) {
    constexpr int ESZ = KBF16 ? 2 : 4;
    constexpr int ROWB = DI * ESZ;        // bytes per key row
    constexpr int NCH = ROWB / 16;        // 16-byte chunks per row
    constexpr int CPC = 16 / ESZ;         // channels per chunk
    constexpr int ROWS_PER_PASS = kTile / NCH;
    __shared__ uint4 tile[kTile * NCH];

    const int t = threadIdx.x;
    const int64_t row = blockIdx.y;       // query row (b * Tq + tq)
    const int64_t b = row / a.Tq;
    const float* qT = qT_all + row * (DI * HI);
    const float* w = w_all + row * HI;
    const uint8_t* kb = k_all + b * a.cap * ROWB;
    const int32_t* __restrict__ pool = a.pool ? a.pool + row * a.P_b : nullptr;

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

    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * a.tiles_per_wg;
    int64_t tile1 = tile0 + a.tiles_per_wg;
    if (tile1 > a.tiles_per_row) tile1 = a.tiles_per_row;

    uint4 stage[NCH];
    auto load_tile = [&](int64_t tl) {
        const int64_t base = tl * kTile;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int r = i * ROWS_PER_PASS + t / NCH;
            const int c = t % NCH;
            const int64_t pos = pos_of(base + r);
            if (pos >= 0)
                stage[i] = *reinterpret_cast<const uint4*>(kb + pos * ROWB + c * 16);
            else
                stage[i] = make_uint4(0, 0, 0, 0);
        }
    };

    if (tile0 < tile1) load_tile(tile0);
    for (int64_t tl = tile0; tl < tile1; ++tl) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int r = i * ROWS_PER_PASS + t / NCH;
            const int c = t % NCH;
            tile[r * NCH + (c ^ (r % NCH))] = stage[i];
        }
        __syncthreads();
        if (tl + 1 < tile1) load_tile(tl + 1);

        const int64_t slot = tl * kTile + t;
        const int64_t pos = pos_of(slot);
        float acc[HI];
#pragma unroll
        for (int h = 0; h < HI; ++h) acc[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint4 v = tile[t * NCH + (c ^ (t % NCH))];
            float kv[CPC];
            if (KBF16) {
                const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kv[2 * e] = __uint_as_float(wd[e] << 16);
                    kv[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
                }
            } else {
                kv[0] = __uint_as_float(v.x); kv[1] = __uint_as_float(v.y);
                kv[2] = __uint_as_float(v.z); kv[3] = __uint_as_float(v.w);
            }
#pragma unroll
            for (int e = 0; e < CPC; ++e) {
                const int ch = c * CPC + e;
#pragma unroll
                for (int h = 0; h < HI; ++h) acc[h] = __builtin_fmaf(qT[ch * HI + h], kv[e], acc[h]);
            }
        }
        float s = 0.0f;
#pragma unroll
        for (int h = 0; h < HI; ++h) s = __builtin_fmaf(w[h], acc[h] > 0.0f ? acc[h] : 0.0f, s);
        if (pos < 0) s = -__builtin_inff();
        if (slot < a.n_slots) scores[row * a.ld + slot] = s;

        if (block_max) {
            float mx = s;
            mx = fmaxf(mx, __shfl_xor(mx, 1));
            mx = fmaxf(mx, __shfl_xor(mx, 2));
            mx = fmaxf(mx, __shfl_xor(mx, 4));
            if (mx == 0.0f) mx = 0.0f;
            const int64_t blk = slot >> 3;
            if ((t & 7) == 0 && blk < a.ld_bm) block_max[row * a.ld_bm + blk] = mx;
        }
        __syncthreads();
    }
}

template <int HI, int DI>
__global__ __launch_bounds__(256) void transpose_q_kernel(const void* __restrict__ q, bool bf16,
                                                          int64_t rows, float* __restrict__ qT) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= rows * HI * DI) return;
    const int64_t r = gid / (HI * DI);
    const int rem = static_cast<int>(gid % (HI * DI));
    const int h = rem / DI, c = rem % DI;
    float v;
    if (bf16)
        v = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(q)[gid]) << 16);
    else
        v = static_cast<const float*>(q)[gid];
    qT[r * (HI * DI) + c * HI + h] = v;
}

template <int HI, int DI, bool KBF16>
hipError_t launch_typed(const ScoreLaunch& p, hipStream_t st) {
    const int64_t rows = p.B * p.Tq;
    {
        const int64_t n = rows * HI * DI;
        transpose_q_kernel<HI, DI><<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, st>>>(
            p.q_idx, p.q_bf16, rows, p.qT);
    }
    ScoreArgs a;
    a.qT = p.qT; a.w = p.w; a.k = static_cast<const uint8_t*>(p.k_idx);
    a.cap = p.cap; a.Tq = p.Tq; a.ctx_len = p.ctx_len; a.q_pos = p.q_pos; a.m = p.m;
    a.pool = p.pool; a.P_b = p.P_b;
    a.scores = p.scores; a.ld = p.ld; a.block_max = p.block_max; a.ld_bm = p.ld_bm;
    a.n_slots = p.pool ? static_cast<int64_t>(p.P_b) * 8 : p.ld;
    a.tiles_per_row = (a.n_slots + kTile - 1) / kTile;
    const int64_t total = a.tiles_per_row * rows;
    int64_t tpw = total / 2048;
    if (tpw < 1) tpw = 1;
    if (tpw > 64) tpw = 64;
    a.tiles_per_wg = static_cast<int>(tpw);
    const int64_t gx = (a.tiles_per_row + tpw - 1) / tpw;
    if (gx == 0 || rows == 0) return hipGetLastError();
    score_kernel<HI, DI, KBF16><<<dim3(static_cast<unsigned>(gx), static_cast<unsigned>(rows)),
                                  kTile, 0, st>>>(a.qT, a.w, a.k, a.scores, a.block_max, a);
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
