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

// ------------------------------------------------- one-workgroup selection
// Rows of up to kSelMax slots are selected by one 1,024-thread workgroup
// with the keys in registers: thread t holds the run of R consecutive slots
// [tR, tR + R) (R = 16 or 32).
//  1. The nonempty count, smallest and largest key give the bits all keys
//     share; radix passes start at the highest bit where they differ, so the
//     first 13-bit digit already spreads the keys over the bins (scores share
//     sign and most exponent bits, which a fixed top digit would spend a pass
//     on).  Two passes usually resolve the k-th key.
//  2. Each pass counts the keys that still match the resolved prefix into an
//     LDS histogram; a workgroup scan over the bins from the top finds the
//     digit holding the k-th key.
//  3. Emission: two workgroup scans give each thread its tie rank and output
//     offset, and it writes its chosen slots in order, so ties go to the
//     lowest slots and the output is sorted without a sort.
constexpr int kSelMax = 32768;
constexpr int kSelBits = 13;
constexpr int kSelBins = 1 << kSelBits;          // 8 bins per thread
static_assert(kSelBins == 8 * kThreads, "bin ownership assumes 8 bins per thread");

struct alignas(16) SelLds {
    uint32_t hist[kSelBins];
    uint32_t wave_tot[kWaves];
    uint32_t wave_min[kWaves];
    uint32_t wave_max[kWaves];
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

// Choose the k best keys of the workgroup's slots (thread t: slots
// [tR, tR + R) in kk, 0 = empty) and call out(rank, j) for each chosen slot
// tR + j in ascending slot order.  Returns min(k, #nonempty).
template <int R, class Out>
__device__ uint32_t select_run(const uint32_t (&kk)[R], uint32_t k, SelLds& sh, Out out) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

    // ---- 1. count, smallest and largest nonempty key
    uint32_t cnt = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        cnt += kk[j] != 0u;
        mn = (kk[j] != 0u && kk[j] < mn) ? kk[j] : mn;
        mx = kk[j] > mx ? kk[j] : mx;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        cnt += __shfl_xor(cnt, off);
        const uint32_t omn = __shfl_xor(mn, off), omx = __shfl_xor(mx, off);
        mn = omn < mn ? omn : mn;
        mx = omx > mx ? omx : mx;
    }
    if (lane == 0) { sh.wave_tot[wv] = cnt; sh.wave_min[wv] = mn; sh.wave_max[wv] = mx; }
    __syncthreads();
    uint32_t n_valid = 0;
    mn = 0xffffffffu; mx = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        n_valid += sh.wave_tot[w];
        mn = sh.wave_min[w] < mn ? sh.wave_min[w] : mn;
        mx = sh.wave_max[w] > mx ? sh.wave_max[w] : mx;
    }
    __syncthreads();
    const uint32_t k_eff = n_valid < k ? n_valid : k;
    if (k_eff == 0) return 0;

    // ---- 2. radix passes below the shared prefix
    uint32_t need = k_eff, T;
    if (mn == mx) {
        T = mn;                                    // every nonempty key is T
    } else {
        int top = 31 - __builtin_clz(mn ^ mx);     // highest bit not shared
        uint64_t known = static_cast<uint64_t>(mn) >> (top + 1);
        while (top >= 0) {
            const int nb = top + 1 < kSelBits ? top + 1 : kSelBits;
            const int shift = top + 1 - nb;
            const uint32_t dmask = (1u << nb) - 1u;
            // keys match the resolved prefix when their bits above `top`
            // equal it (all keys do before the first pass below bit 31)
            const bool match_all = top == 31;
            const int pshift = match_all ? 0 : top + 1;
            const uint32_t known32 = static_cast<uint32_t>(known);
            for (int i = tid; i < kSelBins; i += kThreads) sh.hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const bool ok = kk[j] != 0u && (match_all || (kk[j] >> pshift) == known32);
                if (ok) atomicAdd(&sh.hist[(kk[j] >> shift) & dmask], 1u);
                if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
            // thread t holds bins kSelBins-1-8t down to kSelBins-8-8t, so
            // thread order is descending bin order
            const int hb = kSelBins - 8 - 8 * tid;
            const uint4 lo = *reinterpret_cast<const uint4*>(&sh.hist[hb]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&sh.hist[hb + 4]);
            const uint32_t c[8] = {hi.w, hi.z, hi.y, hi.x, lo.w, lo.z, lo.y, lo.x};
            uint32_t sum = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) sum += c[i];
            uint32_t tot;
            const uint32_t excl = block_excl_scan(sum, sh.wave_tot, tot);
            if (excl < need && excl + sum >= need) {
                uint32_t acc = excl;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (acc + c[i] >= need) { sh.res[0] = hb + 7 - i; sh.res[1] = acc; break; }
                    acc += c[i];
                }
            }
            __syncthreads();
            known = (known << nb) | sh.res[0];
            need -= sh.res[1];
            top = shift - 1;
            __syncthreads();
        }
        T = static_cast<uint32_t>(known);
    }

    // ---- 3. ordered emission
    uint32_t above = 0, ties = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) { above += kk[j] > T; ties += kk[j] == T; }
    uint32_t tmp;
    const uint32_t ties_before = block_excl_scan(ties, sh.wave_tot, tmp);
    uint32_t take = need > ties_before ? need - ties_before : 0u;
    if (take > ties) take = ties;
    uint32_t at = block_excl_scan(above + take, sh.wave_tot, tmp);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const bool tie_pick = kk[j] == T && take > 0;
        if (kk[j] > T || tie_pick) {
            if (tie_pick) --take;
            if (at < k) out(at, j);
            ++at;
        }
        if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    return k_eff;
}

// Find the k-th largest key (and how many keys equal to it belong to the
// top k) of the workgroup's R-key runs, with the adaptive radix passes of
// select_run (stages 1 and 2 only).  Returns min(k, #nonempty).
template <int R>
__device__ uint32_t kth_key(const uint32_t (&kk)[R], uint32_t k, SelLds& sh, uint32_t& T_out, uint32_t& need_out) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint32_t cnt = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        cnt += kk[j] != 0u;
        mn = (kk[j] != 0u && kk[j] < mn) ? kk[j] : mn;
        mx = kk[j] > mx ? kk[j] : mx;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        cnt += __shfl_xor(cnt, off);
        const uint32_t omn = __shfl_xor(mn, off), omx = __shfl_xor(mx, off);
        mn = omn < mn ? omn : mn;
        mx = omx > mx ? omx : mx;
    }
    if (lane == 0) { sh.wave_tot[wv] = cnt; sh.wave_min[wv] = mn; sh.wave_max[wv] = mx; }
    __syncthreads();
    uint32_t n_valid = 0;
    mn = 0xffffffffu; mx = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        n_valid += sh.wave_tot[w];
        mn = sh.wave_min[w] < mn ? sh.wave_min[w] : mn;
        mx = sh.wave_max[w] > mx ? sh.wave_max[w] : mx;
    }
    __syncthreads();
    const uint32_t k_eff = n_valid < k ? n_valid : k;
    T_out = 0u; need_out = 0u;
    if (k_eff == 0) return 0;
    uint32_t need = k_eff, T;
    if (mn == mx) {
        T = mn;
    } else {
        int top = 31 - __builtin_clz(mn ^ mx);
        uint64_t known = static_cast<uint64_t>(mn) >> (top + 1);
        while (top >= 0) {
            const int nb = top + 1 < kSelBits ? top + 1 : kSelBits;
            const int shift = top + 1 - nb;
            const uint32_t dmask = (1u << nb) - 1u;
            const bool match_all = top == 31;
            const int pshift = match_all ? 0 : top + 1;
            const uint32_t known32 = static_cast<uint32_t>(known);
            for (int i = tid; i < kSelBins; i += kThreads) sh.hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const bool ok = kk[j] != 0u && (match_all || (kk[j] >> pshift) == known32);
                if (ok) atomicAdd(&sh.hist[(kk[j] >> shift) & dmask], 1u);
                if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
            const int hb = kSelBins - 8 - 8 * tid;
            const uint4 lo = *reinterpret_cast<const uint4*>(&sh.hist[hb]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&sh.hist[hb + 4]);
            const uint32_t c[8] = {hi.w, hi.z, hi.y, hi.x, lo.w, lo.z, lo.y, lo.x};
            uint32_t sum = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) sum += c[i];
            uint32_t tot;
            const uint32_t excl = block_excl_scan(sum, sh.wave_tot, tot);
            if (excl < need && excl + sum >= need) {
                uint32_t acc = excl;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (acc + c[i] >= need) { sh.res[0] = hb + 7 - i; sh.res[1] = acc; break; }
                    acc += c[i];
                }
            }
            __syncthreads();
            known = (known << nb) | sh.res[0];
            need -= sh.res[1];
            top = shift - 1;
            __syncthreads();
        }
        T = static_cast<uint32_t>(known);
    }
    T_out = T;
    need_out = need;
    return k_eff;
}
