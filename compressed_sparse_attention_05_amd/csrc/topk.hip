// Exact top-k selection for gfx950 (Full-mode indices, Reindex indices and
// the candidate-pool block choice: "DeepSeek-V4.1-Flash KV Cache Compression"
// notes, sections 2-3).
//
// Order: score descending, then slot ascending; -0 ties with +0; -inf slots
// are never chosen.  Output: the chosen slots (or pool positions) in
// ascending order, then -1 padding.
//
// Scores map to monotone 32-bit keys (sign-flip transform; 0 never occurs
// for a finite score, so 0 marks an empty slot).  The exact k-th key T and
// the number need_T of slots equal to T still to take are found by radix
// selection; a slot is chosen when key > T, or key == T and fewer than
// need_T tied slots precede it.  Two paths:
//
//  * rows of up to 32,768 slots (pool scores, block maxima up to 256K
//    positions, Reindex pools, small contexts): one 1,024-thread workgroup
//    holds the row's keys in registers (a run of consecutive slots per
//    thread), resolves the k-th key with 13-bit radix passes that start
//    below the bits all keys share, and emits the chosen slots in slot order
//    with workgroup prefix counts (so ties resolve to the lowest slots and
//    the output is sorted without a sort);
//  * longer rows (the Full scan at 128K-1M): many workgroups per row build a
//    global 12-bit histogram, then every workgroup finds the threshold digit
//    and appends the (key, slot) pairs at or above it to a per-row candidate
//    list; one workgroup per row finishes the selection on the candidates
//    (two more LDS passes), gathers the chosen slots and sorts them.  When a
//    row's candidates or ties do not fit, that row falls back to passes over
//    the full row (exact, slower).
#include "csa2_internal.h"

namespace csa2 {
namespace {

#include "select_util.h"

constexpr int kSmallMax = 32768;       // slots staged in LDS by the one-workgroup path (== kSelMax)
constexpr int kChunk = 8192;           // slots per workgroup in the multi-workgroup passes
constexpr int kCandCap = 12288;        // candidates per row kept for the final pass
constexpr int kSortCap = 4096;         // largest k (and tie list) sorted in LDS
constexpr int kHistBins = 4096;        // first digit: key >> 20

// One-workgroup selection (select_run) lives in select_util.h.

// Keys of slots [i0, i0 + R) of a float row with n valid entries: 16-byte
// loads when the run is aligned and complete, else element loads.
template <int R>
__device__ __forceinline__ void load_run_keys(const float* __restrict__ row, int64_t i0, int64_t n,
                                              uint32_t (&kk)[R]) {
    const bool vec = ((reinterpret_cast<uintptr_t>(row + i0) & 15u) == 0) && i0 + R <= n;
    if (vec) {
#pragma unroll
        for (int j = 0; j < R; j += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + i0 + j);
            kk[j] = key_of(v.x); kk[j + 1] = key_of(v.y); kk[j + 2] = key_of(v.z); kk[j + 3] = key_of(v.w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < R; ++j) kk[j] = (i0 + j < n) ? key_of(row[i0 + j]) : 0u;
    }
}

// ---------------------------------------------------------------- small rows
// Rows of up to kSelMax slots: slot order, or pool slots (-> positions).
template <int R>
__global__ __launch_bounds__(kThreads) void topk_small_kernel(const float* __restrict__ scores, int64_t n,
                                                              int64_t ld, int k,
                                                              const int32_t* __restrict__ pool, int P_b,
                                                              int32_t* __restrict__ out) {
    __shared__ SelLds sh;
    const int64_t row = blockIdx.x;
    int32_t* o = out + row * static_cast<int64_t>(k);
    const int32_t* prow = pool ? pool + row * static_cast<int64_t>(P_b) : nullptr;
    uint32_t kk[R];
    const int r0 = threadIdx.x * R;
    load_run_keys<R>(scores + row * ld, r0, n, kk);
    int32_t blk[R / 8];
#pragma unroll
    for (int q = 0; q < R / 8; ++q) blk[q] = (prow && r0 / 8 + q < P_b) ? prow[r0 / 8 + q] : 0;
    const uint32_t got = select_run<R>(kk, static_cast<uint32_t>(k), sh, [&](uint32_t r, int j) {
        o[r] = prow ? blk[j >> 3] * 8 + (j & 7) : r0 + j;
    });
    for (int i = static_cast<int>(got) + threadIdx.x; i < k; i += kThreads) o[i] = -1;
}

// Full-mode top-k through the candidate pool: scores are in position order;
// slot s of the pool is position 8*pool[s/8] + s%8.  Thread t gathers the
// R/8 pool blocks of its run (two 16-byte loads per block when aligned).
template <int R>
__global__ __launch_bounds__(kThreads) void topk_from_pool_kernel(const float* __restrict__ scores, int64_t ld,
                                                                  const int32_t* __restrict__ pool, int P_b,
                                                                  int k, int32_t* __restrict__ out) {
    __shared__ SelLds sh;
    const int64_t row = blockIdx.x;
    const float* s = scores + row * ld;
    const int32_t* prow = pool + row * static_cast<int64_t>(P_b);
    int32_t* o = out + row * static_cast<int64_t>(k);
    const bool aligned = (reinterpret_cast<uintptr_t>(s) & 31u) == 0;
    constexpr int NB = R / 8;
    const int b0 = threadIdx.x * NB;
    int32_t blk[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) blk[q] = (b0 + q < P_b) ? prow[b0 + q] : -1;
    uint32_t kk[R];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int64_t p0 = static_cast<int64_t>(blk[q]) * 8;
        if (blk[q] >= 0 && aligned && p0 + 8 <= ld) {
            const float4 v0 = *reinterpret_cast<const float4*>(s + p0);
            const float4 v1 = *reinterpret_cast<const float4*>(s + p0 + 4);
            kk[8 * q + 0] = key_of(v0.x); kk[8 * q + 1] = key_of(v0.y);
            kk[8 * q + 2] = key_of(v0.z); kk[8 * q + 3] = key_of(v0.w);
            kk[8 * q + 4] = key_of(v1.x); kk[8 * q + 5] = key_of(v1.y);
            kk[8 * q + 6] = key_of(v1.z); kk[8 * q + 7] = key_of(v1.w);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                kk[8 * q + e] = (blk[q] >= 0 && p0 + e < ld) ? key_of(s[p0 + e]) : 0u;
        }
    }
    const uint32_t got = select_run<R>(kk, static_cast<uint32_t>(k), sh, [&](uint32_t r, int j) {
        o[r] = blk[j >> 3] * 8 + (j & 7);
    });
    for (int i = static_cast<int>(got) + threadIdx.x; i < k; i += kThreads) o[i] = -1;
}

// Candidate pool: the P_b best blocks by block max.  Up to kSelMax blocks
// directly; beyond that through super-blocks of 8 blocks (the P_b best
// blocks all lie in the P_b best super-blocks by super-block max, ties to
// the lower id), so both stages stay in one workgroup.
constexpr int kPoolMax = 2048;

template <int R>
__global__ __launch_bounds__(kThreads) void pool_kernel(const float* __restrict__ bmax, int64_t n_blocks,
                                                        int64_t ld, int P_b, int32_t* __restrict__ out) {
    __shared__ SelLds sh;
    const int64_t row = blockIdx.x;
    const float* bm = bmax + row * ld;
    int32_t* o = out + row * static_cast<int64_t>(P_b);
    const int64_t r0 = static_cast<int64_t>(threadIdx.x) * R;
    uint32_t kk[R];
    load_run_keys<R>(bm, r0, n_blocks, kk);
    const uint32_t got = select_run<R>(kk, static_cast<uint32_t>(P_b), sh,
                                       [&](uint32_t r, int j) { o[r] = static_cast<int32_t>(r0) + j; });
    for (int i = static_cast<int>(got) + threadIdx.x; i < P_b; i += kThreads) o[i] = -1;
}

// More than kSelMax blocks: stage 1 selects the P_b best super-blocks (8
// blocks each) by super-block max, stage 2 the P_b best blocks among their
// 8*P_b blocks.
template <int R, bool VEC>
__global__ __launch_bounds__(kThreads) void pool_super_kernel(const float* __restrict__ bmax, int64_t n_blocks,
                                                              int64_t ld, int P_b, int32_t* __restrict__ out) {
    __shared__ SelLds sh;
    __shared__ int32_t sup[kPoolMax];
    const int64_t row = blockIdx.x;
    const float* bm = bmax + row * ld;
    int32_t* o = out + row * static_cast<int64_t>(P_b);
    const int64_t r0 = static_cast<int64_t>(threadIdx.x) * R;
    {
        // stage 1: thread t owns super-blocks [tR, tR + R)
        uint32_t kk[R];
        if constexpr (VEC) {
            // Up to 16,384 super-blocks of a 16-byte aligned row (VEC): the
            // row is read coalesced (lane l of a wave takes the float4 of
            // maxima 4l .. 4l+3 of a 256-block stretch, two lanes per
            // super-block) with unconditional loads clamped to the row's whole
            // float4s, a batch of them in flight at once, and the super-block
            // keys are staged in LDS over the selection's histograms (16,384
            // keys, 64 KiB), then read back as runs.  With each thread reading
            // its own run directly, every load instruction touched 64 cache
            // lines and stage 1 took 18 us of a 40 us launch.
            static_assert(R == 16, "the staged keys fill the histograms at 16 per thread");
            static_assert(sizeof(sh.hist) >= 16 * kThreads * sizeof(uint32_t), "super-block keys fit the histograms");
            uint32_t* skey = &sh.hist[0][0];
            const int64_t n4 = n_blocks / 4;                 // whole float4s (n_blocks > 32,768 here)
            const float4* bm4 = reinterpret_cast<const float4*>(bm);
            constexpr int kBatch = 8;                       // float4s in flight per thread
#pragma unroll 1
            for (int m0 = 0; m0 < 2 * R; m0 += kBatch) {
                float4 raw[kBatch];
#pragma unroll
                for (int mm = 0; mm < kBatch; ++mm) {
                    const int64_t q = static_cast<int64_t>(m0 + mm) * kThreads + threadIdx.x;
                    raw[mm] = bm4[q < n4 ? q : n4 - 1];
                }
                __builtin_amdgcn_sched_barrier(0);    // every load of the batch goes out first
#pragma unroll
                for (int mm = 0; mm < kBatch; ++mm) {
                    const int64_t q = static_cast<int64_t>(m0 + mm) * kThreads + threadIdx.x;
                    const uint32_t a0 = key_of(raw[mm].x), a1 = key_of(raw[mm].y);
                    const uint32_t a2 = key_of(raw[mm].z), a3 = key_of(raw[mm].w);
                    const uint32_t m01 = a0 > a1 ? a0 : a1, m23 = a2 > a3 ? a2 : a3;
                    uint32_t mx = q < n4 ? (m01 > m23 ? m01 : m23) : 0u;
                    // the other half of this super-block is on the neighbour lane
                    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), 1));
                    mx = o > mx ? o : mx;
                    if ((threadIdx.x & 1) == 0) skey[q >> 1] = mx;
                }
            }
            if (n_blocks & 3) {
                // the last super-block ends in a partial float4: recompute it
                __syncthreads();
                if (threadIdx.x == 0) {
                    const int64_t sb = (n_blocks - 1) / 8;
                    uint32_t mx = 0u;
                    for (int64_t i = 8 * sb; i < n_blocks; ++i) {
                        const uint32_t k = key_of(bm[i]);
                        mx = k > mx ? k : mx;
                    }
                    skey[sb] = mx;
                }
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < R; j += 4) {
                const uint4 v = *reinterpret_cast<const uint4*>(&skey[r0 + j]);
                kk[j] = v.x; kk[j + 1] = v.y; kk[j + 2] = v.z; kk[j + 3] = v.w;
            }
            __syncthreads();                    // every read of the staged keys ends before the selection
        } else {
            // four super-blocks in flight
#pragma unroll
            for (int j = 0; j < R; ++j) {
                uint32_t e8[8];
                load_run_keys<8>(bm, (r0 + j) * 8, n_blocks, e8);
                uint32_t m = 0u;
#pragma unroll
                for (int e = 0; e < 8; ++e) m = e8[e] > m ? e8[e] : m;
                kk[j] = m;
                if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
        for (int i = threadIdx.x; i < P_b; i += kThreads) sup[i] = -1;
        __syncthreads();
        select_run<R>(kk, static_cast<uint32_t>(P_b), sh,
                      [&](uint32_t r, int j) { sup[r] = static_cast<int32_t>(r0) + j; });
        __syncthreads();
    }
    // stage 2: the 8*P_b blocks of the chosen super-blocks (ascending ids);
    // thread t takes slots [16t, 16t + 16) = super-blocks 2t and 2t+1
    uint32_t k2[16];
    int32_t sb2[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int si = 2 * threadIdx.x + q;
        sb2[q] = si < P_b ? sup[si] : -1;
        uint32_t e8[8];
        load_run_keys<8>(bm, static_cast<int64_t>(sb2[q] >= 0 ? sb2[q] : 0) * 8, n_blocks, e8);
#pragma unroll
        for (int e = 0; e < 8; ++e) k2[8 * q + e] = sb2[q] >= 0 ? e8[e] : 0u;
    }
    const uint32_t got = select_run<16>(k2, static_cast<uint32_t>(P_b), sh, [&](uint32_t r, int j) {
        o[r] = sb2[j >> 3] * 8 + (j & 7);
    });
    for (int i = static_cast<int>(got) + threadIdx.x; i < P_b; i += kThreads) o[i] = -1;
}

// ---------------------------------------------------------------- long rows
struct LongWs {
    uint32_t* hist;      // [rows][kHistBins]
    uint32_t* cnt;       // [rows]: candidates appended (may exceed the cap)
    uint32_t* nvalid;    // [rows]
    uint2* cand;         // [rows][kCandCap] (key, slot)
};

__global__ void topk_zero_kernel(uint32_t* __restrict__ p, int64_t n_words) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n_words) p[i] = 0u;
}

__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t n,
                                                             int64_t ld, LongWs ws) {
    __shared__ uint32_t hist[kHistBins];
    const int64_t row = blockIdx.y;
    const float* s = scores + row * ld;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk;
    uint32_t kk[kChunk / kThreads];
#pragma unroll
    for (int j = 0; j < kChunk / kThreads; ++j) {
        const int64_t i = base + j * kThreads + threadIdx.x;
        kk[j] = (i < n) ? key_of(s[i]) : 0u;
    }
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < kChunk / kThreads; ++j) {
        v += kk[j] != 0u;
        hist_inc(hist, kk[j] >> 20, kk[j] != 0u);
    }
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0 && v) atomicAdd(&ws.nvalid[row], v);
    __syncthreads();
    for (int i = threadIdx.x; i < kHistBins; i += kThreads)
        if (hist[i]) atomicAdd(&ws.hist[row * kHistBins + i], hist[i]);
}

__global__ __launch_bounds__(kThreads) void topk_collect_kernel(const float* __restrict__ scores, int64_t n,
                                                                int64_t ld, int k, LongWs ws) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t res[2];
    const int64_t row = blockIdx.y;
    const float* s = scores + row * ld;
    const uint32_t n_valid = ws.nvalid[row];
    const uint32_t k_eff = n_valid < static_cast<uint32_t>(k) ? n_valid : static_cast<uint32_t>(k);
    if (k_eff == 0) return;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk;
    uint32_t kk[kChunk / kThreads];
#pragma unroll
    for (int j = 0; j < kChunk / kThreads; ++j) {
        const int64_t i = base + j * kThreads + threadIdx.x;
        kk[j] = (i < n) ? key_of(s[i]) : 0u;
    }
    uint32_t hv[kHistBins / kThreads];
#pragma unroll
    for (int j = 0; j < kHistBins / kThreads; ++j) hv[j] = ws.hist[row * kHistBins + j * kThreads + threadIdx.x];
#pragma unroll
    for (int j = 0; j < kHistBins / kThreads; ++j) hist[j * kThreads + threadIdx.x] = hv[j];
    __syncthreads();
    find_digit(hist, kHistBins, k_eff, res);
    const uint32_t b1 = res[0];
    const int lane = threadIdx.x & 63;
    // one global atomic per wave for all of its candidates
    uint64_t bal[kChunk / kThreads];
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < kChunk / kThreads; ++j) {
        bal[j] = __ballot(kk[j] != 0u && (kk[j] >> 20) >= b1);
        tot += static_cast<uint32_t>(__popcll(bal[j]));
    }
    if (tot == 0) return;
    uint32_t wb = 0;
    if (lane == 0) wb = atomicAdd(&ws.cnt[row], tot);
    wb = rl(wb, 0);
#pragma unroll
    for (int j = 0; j < kChunk / kThreads; ++j) {
        const uint32_t off = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal[j] >> 32),
                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal[j]), 0u));
        const uint32_t at = wb + off;
        if (((bal[j] >> lane) & 1ull) && at < static_cast<uint32_t>(kCandCap)) {
            const int64_t i = base + j * kThreads + threadIdx.x;
            ws.cand[row * kCandCap + at] = make_uint2(kk[j], static_cast<uint32_t>(i));
        }
        wb += static_cast<uint32_t>(__popcll(bal[j]));
    }
}

__global__ __launch_bounds__(kThreads) void topk_final_kernel(const float* __restrict__ scores, int64_t n,
                                                              int64_t ld, int k,
                                                              const int32_t* __restrict__ pool, int P_b,
                                                              int32_t* __restrict__ out, LongWs ws) {
    __shared__ uint2 cand[kCandCap];
    __shared__ uint32_t sel[kSortCap];
    __shared__ uint32_t ties[kSortCap];
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wave_tot[kWaves];
    __shared__ uint32_t res[2];
    __shared__ uint32_t counters[2];
    const int64_t row = blockIdx.x;
    const float* s = scores + row * ld;
    int32_t* o = out + row * static_cast<int64_t>(k);
    const int32_t* prow = pool ? pool + row * static_cast<int64_t>(P_b) : nullptr;
    const uint32_t n_valid = ws.nvalid[row];
    const uint32_t k_eff = n_valid < static_cast<uint32_t>(k) ? n_valid : static_cast<uint32_t>(k);
    const uint32_t C = ws.cnt[row];
    bool fallback = (C > static_cast<uint32_t>(kCandCap)) || (k_eff > static_cast<uint32_t>(kSortCap));

    uint32_t T = 0, need = 0;
    if (k_eff > 0 && !fallback) {
        for (uint32_t b0 = 0; b0 < C; b0 += 4 * kThreads) {
            uint2 t[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t i = b0 + j * kThreads + threadIdx.x;
                t[j] = i < C ? ws.cand[row * kCandCap + i] : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t i = b0 + j * kThreads + threadIdx.x;
                if (i < C) cand[i] = t[j];
            }
        }
        __syncthreads();
        auto get = [&](int64_t i) { return cand[i].x; };
        radix_select(get, C, k_eff, hist, res, T, need);
        // gather: key > T into sel (unordered), key == T into ties
        if (threadIdx.x < 2) counters[threadIdx.x] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < C; i += kThreads) {
            const uint2 c = cand[i];
            if (c.x > T) {
                const uint32_t at = atomicAdd(&counters[0], 1u);
                if (at < static_cast<uint32_t>(kSortCap)) sel[at] = c.y;
            } else if (c.x == T) {
                const uint32_t at = atomicAdd(&counters[1], 1u);
                if (at < static_cast<uint32_t>(kSortCap)) ties[at] = c.y;
            }
        }
        __syncthreads();
        const uint32_t n_above = counters[0], n_ties = counters[1];
        if (n_ties > static_cast<uint32_t>(kSortCap)) {
            fallback = true;
        } else {
            if (need < n_ties) {       // keep the `need` lowest tied slots
                int p2 = 1;
                while (p2 < static_cast<int>(n_ties)) p2 <<= 1;
                for (int i = threadIdx.x + n_ties; i < p2; i += kThreads) ties[i] = 0xffffffffu;
                __syncthreads();
                bitonic_sort(ties, p2);
            }
            for (uint32_t i = threadIdx.x; i < need; i += kThreads) sel[n_above + i] = ties[i];
            int p2 = 1;
            while (p2 < static_cast<int>(k_eff)) p2 <<= 1;
            for (int i = threadIdx.x + k_eff; i < p2; i += kThreads) sel[i] = 0xffffffffu;
            __syncthreads();
            bitonic_sort(sel, p2);
            for (uint32_t i = threadIdx.x; i < k_eff; i += kThreads) {
                const uint32_t slot = sel[i];
                int64_t pos = slot;
                if (prow) pos = static_cast<int64_t>(prow[slot >> 3]) * 8 + (slot & 7);
                o[i] = static_cast<int32_t>(pos);
            }
        }
    }
    if (k_eff > 0 && fallback) {
        auto get = [&](int64_t i) { return key_of(s[i]); };
        radix_select(get, n, k_eff, hist, res, T, need);
        emit_ordered(get, n, T, need, k_eff, prow, o, k, wave_tot);
    }
    for (int64_t i = k_eff + threadIdx.x; i < k; i += kThreads) o[i] = -1;
}

// The Full layer's pool and its top-k, two workgroups per row that run side
// by side (workgroup 2r builds row r's pool, 2r + 1 its top-k).  Direct pool
// only (n_blocks <= kSelMax), R keys per thread for the block maxima.
//  * The pool workgroup selects the P_b best blocks and writes the pool.
//  * The top-k workgroup does not wait for it.  One radix pass over the block
//    maxima brackets the P_b-th largest maximum in [lo, hi]; every block
//    whose maximum is >= lo is a candidate.  The candidates hold the pool
//    (the pool's maxima are all >= the P_b-th largest, hence >= lo), and
//    the top-k over any set of positions between the pool and the whole
//    row equals the top-k over the pool (the identity behind
//    topk_from_pool_kernel), so the top-k is selected among the candidates'
//    scores.  When more than kCandBlocks blocks reach lo (many equal
//    maxima), the top-k workgroup finishes the exact pool selection itself
//    and uses the pool's blocks instead.
constexpr int kCandBlocks = 3072;      // candidate blocks of the top-k workgroup (3 per thread)

template <int R>
__global__ __launch_bounds__(kThreads) void pool_topk_kernel(const float* __restrict__ bmax, int64_t n_blocks,
                                                             int64_t ld_bm, int P_b, int32_t* __restrict__ pool,
                                                             const float* __restrict__ scores, int64_t ld,
                                                             int k, int32_t* __restrict__ out) {
    __shared__ SelLds sh;
    __shared__ int32_t cand_s[kCandBlocks];
    const int64_t row = blockIdx.x >> 1;
    const bool topk_wg = (blockIdx.x & 1) != 0;
    const int tid = threadIdx.x;
    const int64_t r0 = static_cast<int64_t>(tid) * R;
    int32_t* po = pool + row * static_cast<int64_t>(P_b);
    int32_t* o = out + row * static_cast<int64_t>(k);
    uint32_t kk[R];
    load_run_keys<R>(bmax + row * ld_bm, r0, n_blocks, kk);
    uint32_t mn, mx;
    const uint32_t n_valid = sel_stats<R>(kk, sh, mn, mx);
    const uint32_t kp = n_valid < static_cast<uint32_t>(P_b) ? n_valid : static_cast<uint32_t>(P_b);
    const int hb = kSelBins - 8 - 8 * tid;         // this thread's histogram bins
    uint32_t lb = 0, n_cand = kp;
    bool exact = !topk_wg;
    if (topk_wg) {
        if (kp == 0) {
            for (int i = tid; i < k; i += kThreads) o[i] = -1;
            return;
        }
        uint32_t need = kp, lo, hi;
        sel_bracket<R>(kk, mn, mx, need, sh, lo, hi);
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < R; ++j) mine += kk[j] != 0u && kk[j] >= lo;
        uint32_t n_br;
        uint32_t at = block_excl_scan(mine, sh.wave_tot, n_br);
        // every read of hist[0] (the bracket pass) ended before the scan's
        // barriers: clear this thread's bins for the next selection
        *reinterpret_cast<uint4*>(&sh.hist[0][hb]) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&sh.hist[0][hb + 4]) = make_uint4(0u, 0u, 0u, 0u);
        if (n_br <= static_cast<uint32_t>(kCandBlocks)) {
#pragma unroll
            for (int j = 0; j < R; ++j)
                if (kk[j] != 0u && kk[j] >= lo) cand_s[at++] = static_cast<int32_t>(r0) + j;
            lb = lo;
            n_cand = n_br;
        } else {
            exact = true;
            __syncthreads();
        }
    }
    if (exact && kp > 0) {
        // the exact pool: to HBM from the pool workgroup, to LDS from the
        // top-k workgroup
        uint32_t need = kp;
        const uint32_t T = sel_passes<R, true>(kk, mn, mx, need, sh);
        sel_emit<R>(kk, T, need, kp, sh, [&](uint32_t r, int j) {
            const int32_t b = static_cast<int32_t>(r0) + j;
            if (topk_wg) cand_s[r] = b; else po[r] = b;
        });
        lb = need == 0 ? T + 1u : T;
        // hist[0] was last read before sel_emit's barriers
        *reinterpret_cast<uint4*>(&sh.hist[0][hb]) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&sh.hist[0][hb + 4]) = make_uint4(0u, 0u, 0u, 0u);
    }
    if (!topk_wg) {
        for (int i = static_cast<int>(kp) + tid; i < P_b; i += kThreads) po[i] = -1;
        return;
    }
    __syncthreads();
    const float* s = scores + row * ld;
    const bool aligned = (reinterpret_cast<uintptr_t>(s) & 31u) == 0;
    constexpr int NB = kCandBlocks / kThreads;
    constexpr int R2 = 8 * NB;
    const int b0 = tid * NB;
    int32_t blk[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) blk[q] = (b0 + q < static_cast<int>(n_cand)) ? cand_s[b0 + q] : -1;
    uint32_t k2[R2];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int64_t p0 = static_cast<int64_t>(blk[q]) * 8;
        if (blk[q] >= 0 && aligned && p0 + 8 <= ld) {
            const float4 v0 = *reinterpret_cast<const float4*>(s + p0);
            const float4 v1 = *reinterpret_cast<const float4*>(s + p0 + 4);
            k2[8 * q + 0] = key_of(v0.x); k2[8 * q + 1] = key_of(v0.y);
            k2[8 * q + 2] = key_of(v0.z); k2[8 * q + 3] = key_of(v0.w);
            k2[8 * q + 4] = key_of(v1.x); k2[8 * q + 5] = key_of(v1.y);
            k2[8 * q + 6] = key_of(v1.z); k2[8 * q + 7] = key_of(v1.w);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                k2[8 * q + e] = (blk[q] >= 0 && p0 + e < ld) ? key_of(s[p0 + e]) : 0u;
        }
    }
    // With kp == P_b >= k, at least k candidate blocks have a maximum >= lb,
    // so at least k scores are >= lb and the k-th best is too: scores below
    // lb cannot be chosen and leave the selection as empty slots.  The rest
    // lie in [lb, mx] (no score exceeds the largest block maximum) and at
    // least k of them are nonempty, so the selection needs no count or range
    // pass of its own.  A short pool (fewer than P_b nonempty blocks) takes
    // the count and range of its scores first.
    uint32_t k_eff = static_cast<uint32_t>(k), key_lo = lb, key_hi = mx;
    if (kp == static_cast<uint32_t>(P_b) && lb != 0u) {
#pragma unroll
        for (int e = 0; e < R2; ++e) k2[e] = k2[e] >= lb ? k2[e] : 0u;
    } else {
        const uint32_t n2 = sel_stats<R2>(k2, sh, key_lo, key_hi);
        k_eff = n2 < k_eff ? n2 : k_eff;
    }
    if (k_eff > 0) {
        uint32_t need = k_eff;
        const uint32_t T = sel_passes<R2, true>(k2, key_lo, key_hi, need, sh);
        sel_emit<R2>(k2, T, need, k_eff, sh, [&](uint32_t r, int j) { o[r] = blk[j >> 3] * 8 + (j & 7); });
    }
    for (int i = static_cast<int>(k_eff) + tid; i < k; i += kThreads) o[i] = -1;
}

}  // namespace

bool pool_topk_supported(int64_t n_blocks, int P_b, int k) {
    return P_b <= kPoolMax && n_blocks <= kSelMax && k >= 1 && k <= P_b && 8 * static_cast<int64_t>(P_b) <= kSelMax;
}

hipError_t launch_pool_topk(const float* bmax, int64_t rows, int64_t n_blocks, int64_t ld_bm, int P_b,
                            int32_t* pool, const float* scores, int64_t ld, int k, int32_t* out, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(2 * rows));
    // the exact pool (P_b <= 2,048 blocks) always fits the candidate list
    static_assert(kPoolMax <= kCandBlocks && kCandBlocks % kThreads == 0, "candidate blocks");
    if (n_blocks <= 16 * kThreads)
        pool_topk_kernel<16><<<grid, kThreads, 0, st>>>(bmax, n_blocks, ld_bm, P_b, pool, scores, ld, k, out);
    else
        pool_topk_kernel<32><<<grid, kThreads, 0, st>>>(bmax, n_blocks, ld_bm, P_b, pool, scores, ld, k, out);
    return hipGetLastError();
}

hipError_t launch_topk_from_pool(const float* scores, int64_t rows, int64_t ld, const int32_t* pool, int P_b,
                                 int k, int32_t* out, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    if (8 * P_b <= 16 * kThreads)
        topk_from_pool_kernel<16><<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, ld, pool, P_b, k, out);
    else
        topk_from_pool_kernel<32><<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, ld, pool, P_b, k, out);
    return hipGetLastError();
}

bool pool_in_lds(int64_t n_blocks, int P_b) {
    return P_b <= kPoolMax && (n_blocks <= kSelMax || (n_blocks + 7) / 8 <= kSelMax);
}

hipError_t launch_pool(const float* bmax, int64_t rows, int64_t n_blocks, int64_t ld, int P_b, int32_t* out,
                       hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(rows));
    if (n_blocks <= 16 * kThreads)
        pool_kernel<16><<<grid, kThreads, 0, st>>>(bmax, n_blocks, ld, P_b, out);
    else if (n_blocks <= kSelMax)
        pool_kernel<32><<<grid, kThreads, 0, st>>>(bmax, n_blocks, ld, P_b, out);
    else if ((n_blocks + 7) / 8 <= 16 * kThreads && (reinterpret_cast<uintptr_t>(bmax) & 15u) == 0 && ld % 4 == 0)
        pool_super_kernel<16, true><<<grid, kThreads, 0, st>>>(bmax, n_blocks, ld, P_b, out);   // rows 16-byte aligned
    else if ((n_blocks + 7) / 8 <= 16 * kThreads)
        pool_super_kernel<16, false><<<grid, kThreads, 0, st>>>(bmax, n_blocks, ld, P_b, out);
    else
        pool_super_kernel<32, false><<<grid, kThreads, 0, st>>>(bmax, n_blocks, ld, P_b, out);
    return hipGetLastError();
}

size_t topk_workspace_bytes(int64_t rows, int64_t n) {
    if (n <= kSmallMax || rows == 0) return 0;
    const size_t words = static_cast<size_t>(rows) * (kHistBins + 2);
    return (words * 4 + 255) / 256 * 256 + static_cast<size_t>(rows) * kCandCap * sizeof(uint2);
}

hipError_t launch_topk(const float* scores, int64_t rows, int64_t n, int64_t ld, int k,
                       const int32_t* pool, int P_b, int32_t* out, void* ws, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    if (n <= kSmallMax) {
        if (n <= 16 * kThreads)
            topk_small_kernel<16><<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, n, ld, k, pool, P_b, out);
        else
            topk_small_kernel<32><<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, n, ld, k, pool, P_b, out);
        return hipGetLastError();
    }
    LongWs w;
    w.hist = static_cast<uint32_t*>(ws);
    w.cnt = w.hist + rows * kHistBins;
    w.nvalid = w.cnt + rows;
    const size_t words = static_cast<size_t>(rows) * (kHistBins + 2);
    w.cand = reinterpret_cast<uint2*>(static_cast<char*>(ws) + (words * 4 + 255) / 256 * 256);
    topk_zero_kernel<<<dim3(static_cast<unsigned>((words + 255) / 256)), 256, 0, st>>>(w.hist, static_cast<int64_t>(words));
    const unsigned chunks = static_cast<unsigned>((n + kChunk - 1) / kChunk);
    topk_hist_kernel<<<dim3(chunks, static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, n, ld, w);
    topk_collect_kernel<<<dim3(chunks, static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, n, ld, k, w);
    topk_final_kernel<<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, n, ld, k, pool, P_b, out, w);
    return hipGetLastError();
}

}  // namespace csa2
