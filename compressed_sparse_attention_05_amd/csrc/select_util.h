// Workgroup-level selection helpers shared by the top-k kernels (1,024-thread
// workgroups).  Included by one translation unit each, inside an anonymous
// namespace, so every kernel file gets its own copy.
//
// Scores map to monotone 32-bit keys: key_of is strictly increasing in the
// score with -0 == +0, and 0 is reserved for an empty slot (-inf).
#pragma once

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// ---- wave64 scans and reductions on the VALU.  Each step of __shfl_up /
// __shfl_xor is a ds_bpermute round trip through the LDS crossbar; here DPP
// row shifts scan each 16-lane row in four dependent VALU ops, and the four
// row totals come back through readlane.  Every caller runs them with the
// whole wave active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shift(uint32_t fill, uint32_t x) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(fill), static_cast<int>(x), CTRL, 0xf, 0xf, false));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

// inclusive prefix sums within each 16-lane row
__device__ __forceinline__ uint32_t row_incl_sum(uint32_t x) {
    x += dpp_shift<kRowShr1>(0u, x);
    x += dpp_shift<kRowShr2>(0u, x);
    x += dpp_shift<kRowShr4>(0u, x);
    x += dpp_shift<kRowShr8>(0u, x);
    return x;
}
__device__ __forceinline__ uint32_t rl(uint32_t x, int lane) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), lane));
}
// inclusive prefix sum over the wave in lane order
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
    x = row_incl_sum(x);
    const uint32_t r0 = rl(x, 15), r1 = rl(x, 31), r2 = rl(x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}
// wave-uniform sum, minimum and maximum
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
    x = row_incl_sum(x);
    return rl(x, 15) + rl(x, 31) + rl(x, 47) + rl(x, 63);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
    uint32_t y;
    y = dpp_shift<kRowShr1>(0xffffffffu, x); x = y < x ? y : x;
    y = dpp_shift<kRowShr2>(0xffffffffu, x); x = y < x ? y : x;
    y = dpp_shift<kRowShr4>(0xffffffffu, x); x = y < x ? y : x;
    y = dpp_shift<kRowShr8>(0xffffffffu, x); x = y < x ? y : x;
    const uint32_t a = rl(x, 15), b = rl(x, 31), c = rl(x, 47), d = rl(x, 63);
    const uint32_t ab = a < b ? a : b, cd = c < d ? c : d;
    return ab < cd ? ab : cd;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    uint32_t y;
    y = dpp_shift<kRowShr1>(0u, x); x = y > x ? y : x;
    y = dpp_shift<kRowShr2>(0u, x); x = y > x ? y : x;
    y = dpp_shift<kRowShr4>(0u, x); x = y > x ? y : x;
    y = dpp_shift<kRowShr8>(0u, x); x = y > x ? y : x;
    const uint32_t a = rl(x, 15), b = rl(x, 31), c = rl(x, 47), d = rl(x, 63);
    const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}


__device__ __forceinline__ uint32_t key_of(float v) { return order_key(v); }

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
        const uint32_t lb = rl(bin, leader);
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
        const uint32_t incl = wave_incl_sum(sum);
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
    c = wave_sum(c);
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
//     LDS histogram.  Thread t owns bins kSelBins-8-8t .. kSelBins-1-8t, so
//     thread order is descending bin order.  Every wave then finds the digit
//     holding the k-th key on its own (the wave totals locate the owning
//     wave, whose bins it rereads), so no result is published through LDS.
//     Two histograms alternate: a thread clears its bins of the other one
//     after the pass's first barrier, when every wave has finished reading
//     them, so a pass has two barriers.  When the digit's bin holds at most
//     kFinMax keys, they are appended to LDS instead and one wave ranks
//     them (each lane counts the bin's keys above and equal to its own), which
//     resolves the exact key for a fraction of another pass's cost.
//  3. Emission: one workgroup scan of (keys above T, keys equal to T) packed
//     into 16-bit halves gives each thread its output offset and its share
//     of the ties; it writes its chosen slots in order, so ties go to the
//     lowest slots and the output is sorted without a sort.
constexpr int kSelMax = 32768;
constexpr int kSelBits = 13;
constexpr int kSelBins = 1 << kSelBits;          // 8 bins per thread
static_assert(kSelBins == 8 * kThreads, "bin ownership assumes 8 bins per thread");
static_assert(kSelMax < 65536, "emission packs two counts into 16-bit halves");

constexpr int kFinMax = 64;                      // bin size finished by one wave

struct alignas(16) SelLds {
    uint32_t hist[2][kSelBins];
    uint32_t wave_tot[kWaves];
    uint32_t wave_min[kWaves];
    uint32_t wave_max[kWaves];
    uint32_t pass_tot[2][kWaves];
    uint32_t emit_tot[kWaves];
    uint32_t res[4];
    uint32_t fin[kFinMax];
    uint32_t fin_cnt;
};

// Workgroup exclusive scan of one uint32 per thread; returns the prefix and
// the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wave_tot, uint32_t& total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_sum(v);
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

// Stage 1: nonempty count, smallest and largest nonempty key of the
// workgroup; also clears this thread's bins of hist[0] for the first pass.
// One barrier; wave_tot/min/max are read only here.
template <int R>
__device__ __forceinline__ uint32_t sel_stats(const uint32_t (&kk)[R], SelLds& sh, uint32_t& mn_out, uint32_t& mx_out) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint32_t cnt = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        cnt += kk[j] != 0u;
        mn = (kk[j] != 0u && kk[j] < mn) ? kk[j] : mn;
        mx = kk[j] > mx ? kk[j] : mx;
    }
    cnt = wave_sum(cnt);
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) { sh.wave_tot[wv] = cnt; sh.wave_min[wv] = mn; sh.wave_max[wv] = mx; }
    {
        const int hb = kSelBins - 8 - 8 * tid;
        *reinterpret_cast<uint4*>(&sh.hist[0][hb]) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&sh.hist[0][hb + 4]) = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    uint32_t n_valid = 0;
    mn = 0xffffffffu; mx = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        n_valid += sh.wave_tot[w];
        mn = sh.wave_min[w] < mn ? sh.wave_min[w] : mn;
        mx = sh.wave_max[w] > mx ? sh.wave_max[w] : mx;
    }
    mn_out = mn; mx_out = mx;
    return n_valid;
}

// Stage 2: the exact need-th largest key T (need >= 1 nonempty keys exist)
// and, on return, need = how many keys equal to T belong to the selection.
// hist[0] must be clear (sel_stats); both histograms are left dirty.
// EARLY: stop as soon as the digit's bin holds exactly the keys still needed
// (then every key in it is chosen); the result is then one below the
// smallest key the resolved prefix allows, with need = 0, so "key > result"
// is exactly the selection.  Random scores reach that after two passes
// instead of running down to bit 0.  Without EARLY the result is the exact
// need-th key.
// sel_passes_from: the same passes when the keys that can hold the result
// are known to share the bits above `top` with value `known` (keys with other
// high bits are counted as above when larger, which the caller has already
// subtracted from need, or are never chosen when smaller).  hist[0] must be
// clear.
// MAXP: stop after that many passes; *rem_bits (when given) is then the
// number of low bits still unresolved below the returned prefix.  With
// MAXP > 1, a bin of at most kFinMax keys left after a pass is resolved
// exactly by one wave instead of further passes.
template <int R, bool EARLY = false, int MAXP = 32>
__device__ __forceinline__ uint32_t sel_passes_from(const uint32_t (&kk)[R], int top, uint64_t known, uint32_t& need,
                                                    SelLds& sh, int* rem_bits = nullptr) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int hb = kSelBins - 8 - 8 * tid;         // this thread's bins
    int buf = 0;
    for (int pass = 0; top >= 0 && pass < MAXP; ++pass) {
        const int nb = top + 1 < kSelBits ? top + 1 : kSelBits;
        const int shift = top + 1 - nb;
        const uint32_t dmask = (1u << nb) - 1u;
        // keys match the resolved prefix when their bits above `top` equal
        // it (all keys do before the first pass below bit 31)
        const bool match_all = top == 31;
        const int pshift = match_all ? 0 : top + 1;
        const uint32_t known32 = static_cast<uint32_t>(known);
        uint32_t* hist = sh.hist[buf];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const bool ok = kk[j] != 0u && (match_all || (kk[j] >> pshift) == known32);
            if (ok) atomicAdd(&hist[(kk[j] >> shift) & dmask], 1u);
            if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        // the other histogram was last read before this barrier: clear this
        // thread's bins of it for the next pass
        *reinterpret_cast<uint4*>(&sh.hist[buf ^ 1][hb]) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&sh.hist[buf ^ 1][hb + 4]) = make_uint4(0u, 0u, 0u, 0u);
        if (tid == 0) sh.fin_cnt = 0u;
        {
            const uint4 lo = *reinterpret_cast<const uint4*>(&hist[hb]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&hist[hb + 4]);
            uint32_t sum = lo.x + lo.y + lo.z + lo.w + hi.x + hi.y + hi.z + hi.w;
            sum = wave_sum(sum);
            if (lane == 0) sh.pass_tot[buf][wv] = sum;
        }
        __syncthreads();
        // the wave holding the need-th key (waves in descending bin order)
        uint32_t acc = 0;
        int W = kWaves - 1;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t t = sh.pass_tot[buf][w];
            if (W == kWaves - 1 && w < kWaves - 1) {
                if (acc + t >= need) W = w; else acc += t;
            }
        }
        W = __builtin_amdgcn_readfirstlane(W);
        acc = __builtin_amdgcn_readfirstlane(acc);
        // lane l rereads the bins of thread 64W + l
        const int hbw = kSelBins - 8 - 8 * (64 * W + lane);
        const uint4 lo = *reinterpret_cast<const uint4*>(&hist[hbw]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&hist[hbw + 4]);
        const uint32_t c[8] = {hi.w, hi.z, hi.y, hi.x, lo.w, lo.z, lo.y, lo.x};
        uint32_t s8 = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) s8 += c[i];
        const uint32_t incl = wave_incl_sum(s8);
        const uint32_t excl = acc + incl - s8;
        const bool mine = excl < need && excl + s8 >= need;
        uint32_t digit = 0, above = 0, in_bin = 0;
        if (mine) {
            uint32_t a = excl;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (a + c[i] >= need) {
                    digit = static_cast<uint32_t>(hbw + 7 - i); above = a; in_bin = c[i];
                    break;
                }
                a += c[i];
            }
        }
        const uint64_t bal = __ballot(mine);
        const int src = bal ? static_cast<int>(__builtin_ctzll(bal)) : 0;
        digit = rl(digit, src);
        above = rl(above, src);
        known = (known << nb) | digit;
        need -= above;
        in_bin = rl(in_bin, src);
        if (EARLY && shift > 0) {
            const uint32_t lowest = static_cast<uint32_t>(known) << shift;
            if (in_bin == need && lowest != 0u) {
                need = 0;
                return lowest - 1u;
            }
        }
        if (MAXP > 1 && shift > 0 && in_bin <= static_cast<uint32_t>(kFinMax)) {
            // the bin's keys (exactly in_bin of them) to LDS, in any order
            const uint32_t kp = static_cast<uint32_t>(known);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                if (kk[j] != 0u && (kk[j] >> shift) == kp) sh.fin[atomicAdd(&sh.fin_cnt, 1u)] = kk[j];
                if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
            if (wv == 0) {
                const uint32_t x = lane < static_cast<int>(in_bin) ? sh.fin[lane] : 0u;
                uint32_t gt = 0, eq = 0;
                for (int i = 0; i < static_cast<int>(in_bin); ++i) {
                    const uint32_t y = rl(x, i);
                    gt += y > x;
                    eq += y == x;
                }
                // the need-th largest: gt < need <= gt + eq (equal keys agree)
                const bool hit = lane < static_cast<int>(in_bin) && gt < need && gt + eq >= need;
                const uint64_t hb2 = __ballot(hit);
                const int at = hb2 ? static_cast<int>(__builtin_ctzll(hb2)) : 0;
                if (lane == 0) {
                    sh.res[2] = rl(x, at);
                    sh.res[3] = need - rl(gt, at);
                }
            }
            __syncthreads();
            need = sh.res[3];
            if (rem_bits) *rem_bits = 0;
            return sh.res[2];
        }
        top = shift - 1;
        buf ^= 1;
    }
    if (rem_bits) *rem_bits = top + 1;
    return static_cast<uint32_t>(known);
}

template <int R, bool EARLY = false>
__device__ __forceinline__ uint32_t sel_passes(const uint32_t (&kk)[R], uint32_t mn, uint32_t mx, uint32_t& need,
                                               SelLds& sh) {
    if (mn == mx) return mn;                       // every nonempty key is T
    const int top = 31 - __builtin_clz(mn ^ mx);   // highest bit not shared
    return sel_passes_from<R, EARLY>(kk, top, static_cast<uint64_t>(mn) >> (top + 1), need, sh);
}

// One histogram pass: on return the need-th largest key lies in [lo, hi]
// (lo == hi when every bit is resolved), and need is its rank among the keys
// of that range.
template <int R>
__device__ __forceinline__ void sel_bracket(const uint32_t (&kk)[R], uint32_t mn, uint32_t mx, uint32_t& need,
                                            SelLds& sh, uint32_t& lo, uint32_t& hi) {
    if (mn == mx) { lo = hi = mn; return; }
    const int top = 31 - __builtin_clz(mn ^ mx);
    int rem = 0;
    const uint32_t p = sel_passes_from<R, false, 1>(kk, top, static_cast<uint64_t>(mn) >> (top + 1), need, sh, &rem);
    lo = rem >= 32 ? 0u : p << rem;
    hi = rem >= 32 ? 0xffffffffu : (lo | ((1u << rem) - 1u));
}

// Stage 3, ordered emission of the keys above T plus the first `need` keys
// equal to T: one scan of (above << 16 | ties) gives each thread its output
// offset and its share of the ties; out(rank, j) for each chosen slot in
// ascending slot order.  Ends with a barrier.
template <int R, class Out>
__device__ __forceinline__ void sel_emit(const uint32_t (&kk)[R], uint32_t T, uint32_t need, uint32_t k, SelLds& sh,
                                         Out out) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint32_t above = 0, ties = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) { above += kk[j] > T; ties += kk[j] == T; }
    const uint32_t packed = (above << 16) | ties;
    const uint32_t incl = wave_incl_sum(packed);
    if (lane == 63) sh.emit_tot[wv] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) before += (i < wv) ? sh.emit_tot[i] : 0u;
    const uint32_t excl = before + incl - packed;
    const uint32_t above_before = excl >> 16, ties_before = excl & 0xffffu;
    uint32_t take = need > ties_before ? need - ties_before : 0u;
    if (take > ties) take = ties;
    uint32_t at = above_before + (need < ties_before ? need : ties_before);
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
}

// Choose the k best keys of the workgroup's slots (thread t: slots
// [tR, tR + R) in kk, 0 = empty) and call out(rank, j) for each chosen slot
// tR + j in ascending slot order.  Returns min(k, #nonempty).
// If lb is given, *lb is set to a key no larger than any chosen key (every
// chosen key is >= *lb; 0 when nothing is chosen); max_key receives the
// largest key.
template <int R, class Out>
__device__ uint32_t select_run(const uint32_t (&kk)[R], uint32_t k, SelLds& sh, Out out, uint32_t* lb = nullptr,
                               uint32_t* max_key = nullptr) {
    uint32_t mn, mx;
    const uint32_t n_valid = sel_stats<R>(kk, sh, mn, mx);
    if (max_key) *max_key = mx;
    const uint32_t k_eff = n_valid < k ? n_valid : k;
    if (lb) *lb = 0u;
    if (k_eff == 0) return 0;
    uint32_t need = k_eff;
    const uint32_t T = sel_passes<R, true>(kk, mn, mx, need, sh);
    if (lb) *lb = need == 0 ? T + 1u : T;
    sel_emit<R>(kk, T, need, k, sh, out);
    return k_eff;
}

// Find the k-th largest key (and how many keys equal to it belong to the
// top k) of the workgroup's R-key runs, with the adaptive radix passes of
// select_run (stages 1 and 2 only).  Returns min(k, #nonempty).
template <int R>
__device__ uint32_t kth_key(const uint32_t (&kk)[R], uint32_t k, SelLds& sh, uint32_t& T_out, uint32_t& need_out) {
    uint32_t mn, mx;
    const uint32_t n_valid = sel_stats<R>(kk, sh, mn, mx);
    const uint32_t k_eff = n_valid < k ? n_valid : k;
    T_out = 0u; need_out = 0u;
    if (k_eff == 0) { __syncthreads(); return 0; }
    uint32_t need = k_eff;
    T_out = sel_passes<R>(kk, mn, mx, need, sh);
    need_out = need;
    // callers reuse wave_tot (block_excl_scan) next
    __syncthreads();
    return k_eff;
}
