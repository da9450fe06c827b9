// Exact top-k selection for gfx950 (Full-mode indices, Reindex indices and
// the candidate-pool block choice: "DeepSeek-V4.1-Flash KV Cache Compression"
// notes, sections 2-3).
//
// Order: score descending, then slot ascending; -0 ties with +0; -inf slots
// are never chosen.  Output: the chosen slots (or pool positions) in
// ascending order, then -1 padding.
//
// Method: scores map to monotone 32-bit keys (sign-flip transform).  Three
// LDS-histogram radix passes (11, 11, 10 bits) find the exact k-th key T and
// how many of the slots equal to T are still needed (need_T).  A final pass
// walks the row in slot order, 1024 slots per step, and keeps a slot when
// key > T, or key == T and fewer than need_T tied slots came before it; two
// wave-ballot prefix counts per step give the tie rank and the output offset,
// so ties always resolve to the lowest slots and the output is sorted without
// a sort.
//
// One 1024-thread workgroup per row; the row is re-read from L2/HBM once per
// pass.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ bool key_of(float v, uint32_t& key) {
    uint32_t u = __float_as_uint(v);
    if (u == 0xff800000u) return false;   // -inf
    if (u == 0x80000000u) u = 0u;         // -0 -> +0
    key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return true;
}

// Exclusive prefix of `flag` over the workgroup in thread order, plus the
// total.  Uses one 64-bit ballot per wave and a 16-entry LDS exchange.
__device__ __forceinline__ uint32_t block_excl_prefix(bool flag, uint32_t* wave_tot,
                                                      uint32_t& total) {
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

// Given a histogram over `nbins` digits, find digit d (scanning from the top)
// where the count of keys with a larger digit is < need and including d is
// >= need.  Returns d and sets `above` to the count of larger digits.
// Executed by wave 0; result broadcast through LDS.
__device__ void find_digit(const uint32_t* hist, int nbins, uint32_t need, uint32_t* sh_res) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = nbins / 64;
        // lane 0 owns the top `per` bins
        const int hi_bin = nbins - 1 - lane * per;
        uint32_t sum = 0;
        for (int i = 0; i < per; ++i) sum += hist[hi_bin - i];
        // inclusive prefix over lanes (lane order = descending bins)
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
                    sh_res[0] = static_cast<uint32_t>(hi_bin - i);
                    sh_res[1] = acc;
                    break;
                }
                acc += c;
            }
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores, int64_t n,
                                                        int64_t ld, int k,
                                                        const int32_t* __restrict__ pool, int P_b,
                                                        int32_t* __restrict__ out) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wave_tot[kWaves];
    __shared__ uint32_t res[2];
    __shared__ uint32_t n_valid_sh;

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const float* s = scores + row * ld;
    int32_t* o = out + row * static_cast<int64_t>(k);
    const int32_t* prow = pool ? pool + row * static_cast<int64_t>(P_b) : nullptr;

    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kBits[3] = {11, 11, 10};
    uint32_t prefix = 0;     // digits fixed so far
    uint32_t need = 0;       // keys still to take at/below the current prefix
    uint32_t n_valid = 0;

    for (int pass = 0; pass < 3; ++pass) {
        const int sh = kShift[pass], nb = kBits[pass];
        const int nbins = 1 << nb;
        for (int i = tid; i < nbins; i += kThreads) hist[i] = 0;
        if (tid == 0) n_valid_sh = 0;
        __syncthreads();
        uint32_t my_valid = 0;
        for (int64_t i = tid; i < n; i += kThreads) {
            uint32_t key;
            if (!key_of(s[i], key)) continue;
            if (pass == 0) {
                ++my_valid;
            } else if ((key >> (sh + nb)) != prefix) {
                continue;
            }
            atomicAdd(&hist[(key >> sh) & (nbins - 1)], 1u);
        }
        if (pass == 0) {
            // count valid slots
            for (int off = 32; off > 0; off >>= 1) my_valid += __shfl_xor(my_valid, off);
            if ((tid & 63) == 0) atomicAdd(&n_valid_sh, my_valid);
        }
        __syncthreads();
        if (pass == 0) {
            n_valid = n_valid_sh;
            need = n_valid < static_cast<uint32_t>(k) ? n_valid : static_cast<uint32_t>(k);
            if (need == 0) break;
        }
        find_digit(hist, nbins, need, res);
        prefix = (prefix << nb) | res[0];
        need -= res[1];
        __syncthreads();
    }

    const uint32_t k_eff = n_valid < static_cast<uint32_t>(k) ? n_valid : static_cast<uint32_t>(k);
    if (k_eff > 0) {
        const uint32_t T = prefix;
        uint32_t ties_before = 0, written = 0;
        for (int64_t base = 0; base < n; base += kThreads) {
            const int64_t i = base + tid;
            uint32_t key = 0;
            const bool valid = (i < n) && key_of(s[i], key);
            const bool tie = valid && key == T;
            uint32_t tie_tot;
            const uint32_t tie_rank = ties_before + block_excl_prefix(tie, wave_tot, tie_tot);
            const bool sel = valid && (key > T || (tie && tie_rank < need));
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
    for (int64_t i = k_eff + tid; i < k; i += kThreads) o[i] = -1;
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t rows, int64_t n, int64_t ld, int k,
                       const int32_t* pool, int P_b, int32_t* out, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    topk_kernel<<<dim3(static_cast<unsigned>(rows)), kThreads, 0, st>>>(scores, n, ld, k, pool, P_b, out);
    return hipGetLastError();
}

}  // namespace csa2
