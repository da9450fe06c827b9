// Workgroup-level selection helpers shared by the top-k kernels (1,024-thread
// workgroups).  Included by one translation unit each, inside an anonymous
// namespace, so every kernel file gets its own copy.
//
// Scores map to monotone 32-bit keys: key_of is strictly increasing in the
// score with -0 == +0, and 0 is reserved for an empty slot (-inf).
#pragma once

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;


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

