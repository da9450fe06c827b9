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
//  * rows of up to 32,768 slots (pool scores, block maxima at 128K, small
//    contexts): one 1,024-thread workgroup stages the whole row of keys in
//    LDS, runs three histogram passes there, and emits the chosen slots in
//    slot order with wave-ballot prefix counts (so ties resolve to the lowest
//    slots and the output is sorted without a sort);
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

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kSmallMax = 32768;       // slots staged in LDS by the one-workgroup path (== kSelMax)
constexpr int kChunk = 8192;           // slots per workgroup in the multi-workgroup passes
constexpr int kCandCap = 12288;        // candidates per row kept for the final pass
constexpr int kSortCap = 4096;         // largest k (and tie list) sorted in LDS
constexpr int kHistBins = 4096;        // first digit: key >> 20

__device__ __forceinline__ uint32_t key_of(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0xff800000u) return 0u;      // -inf: empty
    if (u == 0x80000000u) u = 0u;         // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix of `flag` over the workgroup in thread order, plus the total.
__device__ __forceinline__ uint32_t block_excl_prefix(bool flag, uint32_t* wave_tot, uint32_t& total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const uint32_t in_wave = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u));
    if (lane == 0) wave_tot[wv] = static_cast<uint32_t>(__popcll(bal));
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const uint32_t c = wave_tot[i];
        before += (i < wv) ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + in_wave;
}

// Histogram increment with wave aggregation: up to four rounds in which the
// lanes sharing the lowest active lane's bin add their count with one atomic
// (scores crowd into a few bins, so plain LDS atomics would serialise),
// then the remaining lanes add one each.
__device__ __forceinline__ void hist_inc(uint32_t* hist, uint32_t bin, bool valid) {
    uint64_t active = __ballot(valid);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int round = 0; round < 4; ++round) {
        if (active == 0) return;
        const int leader = __builtin_ctzll(active);
        const uint32_t lb = __shfl(bin, leader);
        const uint64_t same = __ballot(valid && bin == lb) & active;
        if (lane == leader) atomicAdd(&hist[lb], static_cast<uint32_t>(__popcll(same)));
        active &= ~same;
    }
    if ((active >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Over bins [0, nbins) scanned from the top, find digit d with
// count(bins > d) < need <= count(bins >= d).  Result in res[0] (digit) and
// res[1] (count above).  Wave 0 works; all threads sync.
__device__ void find_digit(const uint32_t* hist, int nbins, uint32_t need, uint32_t* res) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = nbins / 64;
        const int hi_bin = nbins - 1 - lane * per;
        uint32_t sum = 0;
        for (int i = 0; i < per; ++i) sum += hist[hi_bin - i];
        uint32_t incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        const uint32_t excl = incl - sum;
        if (excl < need && incl >= need) {
            uint32_t acc = excl;
            for (int i = 0; i < per; ++i) {
                const uint32_t c = hist[hi_bin - i];
                if (acc + c >= need) {
                    res[0] = static_cast<uint32_t>(hi_bin - i);
                    res[1] = acc;
                    break;
                }
                acc += c;
            }
        }
    }
    __syncthreads();
}

// Ascending bitonic sort of n_pow2 (a power of two) uint32 values in LDS.
__device__ void bitonic_sort(uint32_t* a, int n_pow2) {
    for (int size = 2; size <= n_pow2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < n_pow2 / 2; i += kThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = ((lo & size) == 0);
                const uint32_t x = a[lo], y = a[hi];
                if ((x > y) == up) { a[lo] = y; a[hi] = x; }
            }
            __syncthreads();
        }
    }
}

// Three radix passes (11, 11, 10 bits) over keys get(i), i < n (0 = empty).
// Returns the exact k_eff-th largest key T and need = how many slots equal
// to T belong to the selection.  `hist` holds 2,048 bins.
template <class Get>
__device__ void radix_select(Get get, int64_t n, uint32_t k_eff, uint32_t* hist, uint32_t* res,
                             uint32_t& T, uint32_t& need) {
    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kBits[3] = {11, 11, 10};
    uint32_t prefix = 0;
    need = k_eff;
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = kShift[pass], nb = kBits[pass];
        const int nbins = 1 << nb;
        for (int i = threadIdx.x; i < nbins; i += kThreads) hist[i] = 0;
        __syncthreads();
        for (int64_t base = 0; base < n; base += 4 * kThreads) {
            uint32_t kk[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = base + j * kThreads + threadIdx.x;
                kk[j] = i < n ? get(i) : 0u;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool ok = kk[j] != 0u && (pass == 0 || (kk[j] >> (sh + nb)) == prefix);
                hist_inc(hist, (kk[j] >> sh) & (nbins - 1), ok);
            }
        }
        __syncthreads();
        find_digit(hist, nbins, need, res);
        prefix = (prefix << nb) | res[0];
        need -= res[1];
        __syncthreads();
    }
    T = prefix;
}

// Ordered emission: walk slots in order, keep key > T or the first `need`
// slots with key == T; write o[at] = slot (or pool position).
template <class Get>
__device__ void emit_ordered(Get get, int64_t n, uint32_t T, uint32_t need, uint32_t k_eff,
                             const int32_t* prow, int32_t* o, int k, uint32_t* wave_tot) {
    uint32_t ties_before = 0, written = 0;
    for (int64_t base = 0; base < n; base += kThreads) {
        const int64_t i = base + threadIdx.x;
        const uint32_t key = (i < n) ? get(i) : 0u;
        const bool tie = key != 0u && key == T;
        uint32_t tie_tot;
        const uint32_t tie_rank = ties_before + block_excl_prefix(tie, wave_tot, tie_tot);
        const bool sel = key != 0u && (key > T || (tie && tie_rank < need));
        uint32_t sel_tot;
        const uint32_t at = written + block_excl_prefix(sel, wave_tot, sel_tot);
        if (sel && at < static_cast<uint32_t>(k)) {
            int64_t pos = i;
            if (prow) pos = static_cast<int64_t>(prow[i >> 3]) * 8 + (i & 7);
            o[at] = static_cast<int32_t>(pos);
        }
        ties_before += tie_tot;
        written += sel_tot;
        if (written >= k_eff) break;
    }
}

template <class Get>
__device__ uint32_t count_valid(Get get, int64_t n, uint32_t* wave_tot) {
    uint32_t c = 0;
    for (int64_t base = 0; base < n; base += 4 * kThreads) {
        uint32_t kk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t i = base + j * kThreads + threadIdx.x;
            kk[j] = i < n ? get(i) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) c += kk[j] != 0u;
    }
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if ((threadIdx.x & 63) == 0) wave_tot[threadIdx.x >> 6] = c;
    __syncthreads();
    uint32_t tot = 0;
    for (int i = 0; i < kWaves; ++i) tot += wave_tot[i];
    __syncthreads();
    return tot;
}

// ------------------------------------------------- LDS selection core
// One 1,024-thread workgroup selects among up to kSelMax keys staged in
// LDS.  Radix passes use 8-bit digits and one private 256-bin histogram per
// wave (no cross-wave atomics; lanes of one wave meet only in crowded bins),
// merged per pass.  Emission: thread t owns the run of R consecutive slots
// [tR, tR + R); two workgroup scans give each thread its tie rank and output
// offset, and it writes its chosen slots in order.
constexpr int kSelMax = 32768;

struct alignas(16) SelLds {
    uint32_t keys[kSelMax];
    uint32_t hist[kWaves][256];
    uint32_t wave_tot[kWaves];
    uint32_t res[4];
};

// Workgroup exclusive scan of one uint32 per thread; returns the prefix and
// the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wave_tot, uint32_t& total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const uint32_t c = wave_tot[i];
        before += (i < wv) ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// Choose the k best of keys[0, n) (0 = empty) and call out(rank, slot) for
// each chosen slot in ascending slot order (rank = output position).
// Returns the number chosen (min(k, #nonempty)).  keys[n, 1024*R) must be
// zero, where R = run length (a multiple of 4).
template <class Out>
__device__ uint32_t select_core(SelLds& sh, int n, uint32_t k, Out out) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint32_t prefix = 0, need = 0, n_valid = 0;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int j = 0; j < 4; ++j) sh.hist[wv][lane * 4 + j] = 0u;
        __syncthreads();
        // Scores crowd into one or two digits (the top byte is sign and
        // exponent), so each wave first adds its two most common digits with
        // one ballot-counted atomic each; the remaining lanes add singly.
        for (int base = 0; base < n; base += kThreads) {
            const int i = base + tid;
            const uint32_t key = i < n ? sh.keys[i] : 0u;
            const bool ok = key != 0u && (pass == 0 || (key >> (shift + 8)) == prefix);
            const uint32_t bin = (key >> shift) & 255u;
            uint64_t act = __ballot(ok);
#pragma unroll
            for (int round = 0; round < 2; ++round) {
                if (act != 0) {
                    const int leader = __builtin_ctzll(act);
                    const uint32_t lb = __builtin_amdgcn_readlane(bin, leader);
                    const uint64_t same = __ballot(ok && bin == lb) & act;
                    if (lane == leader) atomicAdd(&sh.hist[wv][lb], static_cast<uint32_t>(__popcll(same)));
                    act &= ~same;
                }
            }
            if ((act >> lane) & 1ull) atomicAdd(&sh.hist[wv][bin], 1u);
        }
        __syncthreads();
        if (tid < 256) {
            uint32_t t = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) t += sh.hist[w][tid];
            sh.hist[0][tid] = t;
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns bins 255-4l .. 252-4l (descending)
            uint32_t c[4], sum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) { c[j] = sh.hist[0][255 - 4 * lane - j]; sum += c[j]; }
            uint32_t incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            uint32_t nd = need;
            if (pass == 0) {
                const uint32_t total = __shfl(incl, 63);
                nd = total < k ? total : k;
                if (lane == 0) sh.res[2] = total;
            }
            const uint32_t excl = incl - sum;
            if (nd > 0 && excl < nd && incl >= nd) {
                uint32_t acc = excl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (acc + c[j] >= nd) { sh.res[0] = 255u - 4u * lane - j; sh.res[1] = acc; break; }
                    acc += c[j];
                }
            }
            if (lane == 0) sh.res[3] = nd;
        }
        __syncthreads();
        if (pass == 0) {
            n_valid = sh.res[2];
            need = sh.res[3];
            if (need == 0) break;
        }
        prefix = (prefix << 8) | sh.res[0];
        need -= sh.res[1];
        __syncthreads();
    }
    const uint32_t k_eff = n_valid < k ? n_valid : k;
    if (k_eff == 0) return 0;
    const uint32_t T = prefix;
    const int R = ((n + kThreads * 4 - 1) / (kThreads * 4)) * 4;
    const int r0 = tid * R;
    uint32_t above = 0, ties = 0;
    for (int i = r0; i < r0 + R; i += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(&sh.keys[i]);
        const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) { above += kk[j] > T; ties += kk[j] == T; }
    }
    uint32_t tmp;
    const uint32_t ties_before = block_excl_scan(ties, sh.wave_tot, tmp);
    uint32_t take = need > ties_before ? need - ties_before : 0u;
    if (take > ties) take = ties;
    uint32_t at = block_excl_scan(above + take, sh.wave_tot, tmp);
    for (int i = r0; i < r0 + R; i += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(&sh.keys[i]);
        const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool tie_pick = kk[j] == T && take > 0;
            if (kk[j] > T || tie_pick) {
                if (tie_pick) --take;
                if (at < k) out(at, i + j);
                ++at;
            }
        }
    }
    __syncthreads();
    return k_eff;
}

// Zero keys[n, round_up(n, 4096)) so every run is fully defined.
__device__ __forceinline__ void pad_keys(SelLds& sh, int n) {
    const int padded = ((n + kThreads * 4 - 1) / (kThreads * 4)) * kThreads * 4;
    for (int i = n + threadIdx.x; i < padded; i += kThreads) sh.keys[i] = 0u;
}

// ---------------------------------------------------------------- small rows
// Rows of up to kSelMax slots: slot order, or pool slots (-> positions).
__global__ __launch_bounds__(kThreads) void topk_small_kernel(const float* __restrict__ scores, int64_t n,
                                                              int64_t ld, int k,
                                                              const int32_t* __restrict__ pool, int P_b,
                                                              int32_t* __restrict__ out) {
    __shared__ SelLds sh;
    const int64_t row = blockIdx.x;
    const float* s = scores + row * ld;
    int32_t* o = out + row * static_cast<int64_t>(k);
    const int32_t* prow = pool ? pool + row * static_cast<int64_t>(P_b) : nullptr;
    const int nn = static_cast<int>(n);
    for (int base = 0; base < nn; base += 8 * kThreads) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + j * kThreads + threadIdx.x;
            v[j] = i < nn ? s[i] : -__builtin_inff();
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + j * kThreads + threadIdx.x;
            if (i < nn) sh.keys[i] = key_of(v[j]);
        }
    }
    pad_keys(sh, nn);
    __syncthreads();
    const uint32_t got = select_core(sh, nn, static_cast<uint32_t>(k), [&](uint32_t r, int slot) {
        o[r] = prow ? prow[slot >> 3] * 8 + (slot & 7) : slot;
    });
    for (int i = static_cast<int>(got) + threadIdx.x; i < k; i += kThreads) o[i] = -1;
}

// Full-mode top-k through the candidate pool: scores are in position order;
// slot s of the pool is position 8*pool[s/8] + s%8.
__global__ __launch_bounds__(kThreads) void topk_from_pool_kernel(const float* __restrict__ scores, int64_t ld,
                                                                  const int32_t* __restrict__ pool, int P_b,
                                                                  int k, int32_t* __restrict__ out) {
    __shared__ SelLds sh;
    const int64_t row = blockIdx.x;
    const float* s = scores + row * ld;
    const int32_t* prow = pool + row * static_cast<int64_t>(P_b);
    int32_t* o = out + row * static_cast<int64_t>(k);
    const int n = 8 * P_b;
    for (int base = 0; base < n; base += 8 * kThreads) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + j * kThreads + threadIdx.x;
            v[j] = -__builtin_inff();
            if (i < n) {
                const int32_t b = prow[i >> 3];
                const int64_t pos = static_cast<int64_t>(b) * 8 + (i & 7);
                if (b >= 0 && pos < ld) v[j] = s[pos];
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + j * kThreads + threadIdx.x;
            if (i < n) sh.keys[i] = key_of(v[j]);
        }
    }
    pad_keys(sh, n);
    __syncthreads();
    const uint32_t got = select_core(sh, n, static_cast<uint32_t>(k), [&](uint32_t r, int slot) {
        o[r] = prow[slot >> 3] * 8 + (slot & 7);
    });
    for (int i = static_cast<int>(got) + threadIdx.x; i < k; i += kThreads) o[i] = -1;
}

// Candidate pool: the P_b best blocks by block max.  Up to kSelMax blocks
// directly; beyond that through super-blocks of 8 blocks (the P_b best
// blocks all lie in the P_b best super-blocks by super-block max, ties to
// the lower id), so both stages stay in LDS.
constexpr int kPoolMax = 2048;

__global__ __launch_bounds__(kThreads) void pool_kernel(const float* __restrict__ bmax, int64_t n_blocks,
                                                        int64_t ld, int P_b, int32_t* __restrict__ out) {
    __shared__ SelLds sh;
    __shared__ int32_t sup[kPoolMax];
    const int64_t row = blockIdx.x;
    const float* bm = bmax + row * ld;
    int32_t* o = out + row * static_cast<int64_t>(P_b);
    uint32_t got;
    if (n_blocks <= kSelMax) {
        const int n = static_cast<int>(n_blocks);
        for (int base = 0; base < n; base += 8 * kThreads) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = base + j * kThreads + threadIdx.x;
                v[j] = i < n ? bm[i] : -__builtin_inff();
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = base + j * kThreads + threadIdx.x;
                if (i < n) sh.keys[i] = key_of(v[j]);
            }
        }
        pad_keys(sh, n);
        __syncthreads();
        got = select_core(sh, n, static_cast<uint32_t>(P_b), [&](uint32_t r, int slot) { o[r] = slot; });
    } else {
        // stage 1: super-block keys = max of 8 block keys
        const int nsb = static_cast<int>((n_blocks + 7) / 8);
        for (int base = 0; base < nsb; base += 4 * kThreads) {
            float v[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sb = base + j * kThreads + threadIdx.x;
                const int64_t b0 = static_cast<int64_t>(sb) * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[j][e] = (sb < nsb && b0 + e < n_blocks) ? bm[b0 + e] : -__builtin_inff();
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sb = base + j * kThreads + threadIdx.x;
                if (sb >= nsb) continue;
                uint32_t m = 0u;
#pragma unroll
                for (int e = 0; e < 8; ++e) { const uint32_t kk = key_of(v[j][e]); m = kk > m ? kk : m; }
                sh.keys[sb] = m;
            }
        }
        pad_keys(sh, nsb);
        for (int i = threadIdx.x; i < P_b; i += kThreads) sup[i] = -1;
        __syncthreads();
        select_core(sh, nsb, static_cast<uint32_t>(P_b), [&](uint32_t r, int slot) { sup[r] = slot; });
        // stage 2: the 8*P_b blocks of the chosen super-blocks (ascending ids)
        const int n2 = 8 * P_b;
        for (int i = threadIdx.x; i < n2; i += kThreads) {
            const int32_t sb = sup[i >> 3];
            const int64_t b = static_cast<int64_t>(sb) * 8 + (i & 7);
            sh.keys[i] = (sb >= 0 && b < n_blocks) ? key_of(bm[b]) : 0u;
        }
        pad_keys(sh, n2);
        __syncthreads();
        got = select_core(sh, n2, static_cast<uint32_t>(P_b), [&](uint32_t r, int slot) {
            o[r] = sup[slot >> 3] * 8 + (slot & 7);
        });
    }
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
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
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
    wb = __shfl(wb, 0);
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

}  // namespace

hipError_t launch_topk_from_pool(const float* scores, int64_t rows, int64_t ld, const int32_t* pool, int P_b,
                                 int k, int32_t* out, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    topk_from_pool_kernel<<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, ld, pool, P_b, k, out);
    return hipGetLastError();
}

bool pool_in_lds(int64_t n_blocks, int P_b) {
    return P_b <= kPoolMax && (n_blocks <= kSelMax || (n_blocks + 7) / 8 <= kSelMax);
}

hipError_t launch_pool(const float* bmax, int64_t rows, int64_t n_blocks, int64_t ld, int P_b, int32_t* out,
                       hipStream_t st) {
    if (rows == 0) return hipSuccess;
    pool_kernel<<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(bmax, n_blocks, ld, P_b, out);
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
        topk_small_kernel<<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, n, ld, k, pool, P_b, out);
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
