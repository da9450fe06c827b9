// Sparse attention over gathered MXFP4 main KV joined with the sliding-window
// KV, for gfx950 ("DeepSeek-V4.1-Flash: reading a model through its three
// memory costs", section 03: selected main-KV entries are combined with the
// local SWA KV before attention; "Notes on DeepSeek V4.1 Flash", post 4).
//
// Per query unit u (a decode sequence or a prefill token) and head h:
//     rows  = dequant(main[idx[u][j]]) for j < k (-1 skipped)  ++  SWA rows
//     out_h = softmax_j(sm_scale * q_h . row_j) . rows
// The latent (D channels) is both key and value; all heads share the rows.
//
// Work split: one workgroup = (unit, key split, block of 64 heads), 4 waves.
// Wave w owns head group hg = w & 1 (32 heads) and channel half dh = w >> 1.
// Keys stream in tiles of 32:
//  1. all 256 threads gather the tile's rows and dequantise them to fp16 into
//     LDS twice: key-major Kt[key][d] (for S) and Vt[step][grp][d][8 keys]
//     (for P.V, so every MFMA operand is one 16-byte LDS read);
//  2. S^T[key][head] over this wave's channel half with
//     v_mfma_f32_32x32x16_f16 (A = key rows, B = q in registers), then the
//     two channel halves are added through LDS (same order in both waves);
//  3. online softmax in base 2: each lane holds one head's 16 keys and its
//     partner lane (l ^ 32) the other 16, so the statistics need one
//     cross-lane max per tile;
//  4. O^T[d][head] += V^T P^T with the fp16-rounded probabilities taken
//     straight from the S accumulators: the MFMA k-slot order is chosen to
//     be the accumulator row order, so no shuffle is needed.  The running
//     sum uses the same rounded probabilities.
// Partial results of several key splits are merged by combine_kernel.
//
// Exactness: every MXFP4 value is an fp16 number (E2M1 times E4M3 has at
// most 5 significant bits, range 2^-10..2688) and bf16 q / SWA values in
// [2^-14, 65504] are fp16 numbers, so the operands are exact; MFMA sums in
// float32; only P is rounded (to fp16, relative 2^-11).
#include "csa2_internal.h"

namespace csa2 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kKT = 32;          // keys per tile
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    const uint16_t* q; int q_bf16;          // [units][H][D]
    const uint8_t* codes; const uint8_t* scales; int64_t cap; int64_t kv_unit_stride;
    const int32_t* idx; int k;
    const uint8_t* swa; int swa_bf16; int W;
    const int32_t* swa_len;
    int64_t q_pos0, swa_start; int prefill;
    int64_t units; int H;
    float c2;                                // sm_scale * log2(e)
    float* out;
    float* ws_o; float* ws_m; float* ws_l;   // partials (splits > 1)
    int splits, tiles_per_split, n_tiles;
};

__device__ __forceinline__ uint32_t f16_bits(float v) {
    _Float16 h = static_cast<_Float16>(v);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

// Non-negative finite E4M3 code -> float (exact).
__device__ __forceinline__ float e4m3_val(uint32_t c) {
    return (c < 8u) ? static_cast<float>(c) * 0x1p-9f
                    : __uint_as_float((c << 20) + (120u << 23));
}

// 8 MXFP4 nibbles (channels 0..7 of a code dword, channel 2i in the low
// nibble of byte i) times an fp16 scale -> 4 dwords of packed fp16 pairs
// (channel 2p low half, 2p+1 high half).  E2M1 magnitudes have a zero low
// byte in fp16, so a byte permute over the table of high bytes
// {00,38,3C,3E,40,42,44,46} does the lookup.
__device__ __forceinline__ void dequant8(uint32_t cw, uint32_t scale_h2, uint32_t out[4]) {
    const uint32_t tlo = 0x3E3C3800u, thi = 0x46444240u;
    const uint32_t hb_lo = __builtin_amdgcn_perm(thi, tlo, cw & 0x07070707u) |
                           ((cw & 0x08080808u) << 4);                 // channels 0,2,4,6
    const uint32_t hb_hi = __builtin_amdgcn_perm(thi, tlo, (cw >> 4) & 0x07070707u) |
                           (cw & 0x80808080u);                        // channels 1,3,5,7
    const half2v s = __builtin_bit_cast(half2v, scale_h2);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t sel = 0x0Cu | (static_cast<uint32_t>(p) << 8) | (0x0Cu << 16) |
                             (static_cast<uint32_t>(4 + p) << 24);
        const uint32_t pair = __builtin_amdgcn_perm(hb_hi, hb_lo, sel);
        out[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, pair) * s);
    }
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return f16_bits(a) | (f16_bits(b) << 16);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnArgs a) {
    constexpr int DH = D / 2;              // channels per wave (S partial and O slice)
    constexpr int SSTEPS = DH / 16;        // MFMA k-steps for S
    constexpr int MT = DH / 32;            // O^T row tiles per wave
    constexpr int KROW = D + 8;            // padded Kt row (halves)
    constexpr int CH = D / 8;              // 8-channel chunks per row
    // Kt is dead once S is formed, so the S partials ([4 waves][16][64]
    // float32) reuse its space.
    constexpr int KT_BYTES = kKT * KROW * 2;
    constexpr int SP_BYTES = 4 * 16 * 64 * 4;
    constexpr int KBUF = KT_BYTES > SP_BYTES ? KT_BYTES : SP_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char kbuf[KBUF];
    __shared__ __attribute__((aligned(16))) _Float16 Vt[kKT * D];
    __shared__ int kvalid[kKT];
    _Float16* Kt = reinterpret_cast<_Float16*>(kbuf);
    float* Spart = reinterpret_cast<float*>(kbuf);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int hg = wv & 1, dh = wv >> 1;
    const int64_t u = blockIdx.x;
    const int split = blockIdx.y;
    const int hb = blockIdx.z;
    const int hbase = hb * 64;

    // ---- unit geometry
    const int32_t* idx = a.idx + u * a.k;
    const int64_t kvbase = u * a.kv_unit_stride;
    const uint8_t* swa_rows;
    int n_swa;
    const int64_t swa_row_bytes = static_cast<int64_t>(D) * (a.swa_bf16 ? 2 : 4);
    if (a.prefill) {
        const int64_t i = a.q_pos0 + u;
        int64_t lo = i - a.W + 1;
        if (lo < a.swa_start) lo = a.swa_start;
        if (lo < 0) lo = 0;
        n_swa = static_cast<int>(i - lo + 1 > 0 ? i - lo + 1 : 0);
        swa_rows = a.swa + (lo - (a.q_pos0 - (a.W - 1))) * swa_row_bytes;
    } else {
        int sl = a.swa_len[u];
        n_swa = sl < a.W ? (sl > 0 ? sl : 0) : a.W;
        swa_rows = a.swa + u * static_cast<int64_t>(a.W) * swa_row_bytes;
    }
    const int n_slots = a.k + a.W;

    // ---- q fragments (B operand of S^T): head = hbase + 32hg + lane%32,
    // channels dh*DH + 16*st + 8*(lane/32) + 0..7
    half8 qf[SSTEPS];
    {
        const int head = hbase + 32 * hg + (lane & 31);
        const bool hv = head < a.H;
#pragma unroll
        for (int st = 0; st < SSTEPS; ++st) {
            const int d0 = dh * DH + 16 * st + 8 * (lane >> 5);
            uint32_t wd[4] = {0, 0, 0, 0};
            if (hv) {
                if (a.q_bf16) {
                    const uint4 v = *reinterpret_cast<const uint4*>(a.q + (u * a.H + head) * D + d0);
                    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        wd[e] = pack_h2(__uint_as_float(in[e] << 16), __uint_as_float(in[e] & 0xffff0000u));
                } else {
                    const float* qf32 = reinterpret_cast<const float*>(a.q) + (u * a.H + head) * D + d0;
                    const float4 x0 = *reinterpret_cast<const float4*>(qf32);
                    const float4 x1 = *reinterpret_cast<const float4*>(qf32 + 4);
                    wd[0] = pack_h2(x0.x, x0.y); wd[1] = pack_h2(x0.z, x0.w);
                    wd[2] = pack_h2(x1.x, x1.y); wd[3] = pack_h2(x1.z, x1.w);
                }
            }
            qf[st] = __builtin_bit_cast(half8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
        }
    }

    floatx16 o_acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[mt][r] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;

    const int t_begin = split * a.tiles_per_split;
    int t_end = t_begin + a.tiles_per_split;
    if (t_end > a.n_tiles) t_end = a.n_tiles;

    // dequant role of this thread: key group (step sg, group gg) = wave,
    // 8-channel chunk j = lane
    const int sg = wv >> 1, gg = wv & 1;
    const int j = lane;

    for (int tile = t_begin; tile < t_end; ++tile) {
        // ---------------- 1. gather + dequantise 32 rows
        if (j < CH) {
            uint32_t h[8][4];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int key = 16 * sg + 4 * gg + (i & 3) + 8 * (i >> 2);
                const int slot = tile * kKT + key;
                bool valid = false;
                if (slot < a.k) {
                    const int32_t row = idx[slot];
                    if (row >= 0 && row < a.cap) {
                        valid = true;
                        const int64_t rr = kvbase + row;
                        const uint32_t cw = *reinterpret_cast<const uint32_t*>(a.codes + rr * (D / 2) + 4 * j);
                        const uint32_t sc = a.scales[rr * (D / 16) + (j >> 1)] & 0x7fu;
                        const uint32_t s16 = f16_bits(e4m3_val(sc));
                        dequant8(cw, s16 | (s16 << 16), h[i]);
                    }
                } else if (slot < n_slots) {
                    const int r = slot - a.k;
                    if (r < n_swa) {
                        valid = true;
                        if (a.swa_bf16) {
                            const uint4 v = *reinterpret_cast<const uint4*>(swa_rows + r * swa_row_bytes + 16 * j);
                            const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                h[i][e] = pack_h2(__uint_as_float(in[e] << 16), __uint_as_float(in[e] & 0xffff0000u));
                        } else {
                            const float* f = reinterpret_cast<const float*>(swa_rows + r * swa_row_bytes) + 8 * j;
                            const float4 x0 = *reinterpret_cast<const float4*>(f);
                            const float4 x1 = *reinterpret_cast<const float4*>(f + 4);
                            h[i][0] = pack_h2(x0.x, x0.y); h[i][1] = pack_h2(x0.z, x0.w);
                            h[i][2] = pack_h2(x1.x, x1.y); h[i][3] = pack_h2(x1.z, x1.w);
                        }
                    }
                }
                if (!valid) { h[i][0] = h[i][1] = h[i][2] = h[i][3] = 0u; }
                if (j == 0) kvalid[key] = valid ? 1 : 0;
                *reinterpret_cast<uint4*>(&Kt[key * KROW + 8 * j]) =
                    make_uint4(h[i][0], h[i][1], h[i][2], h[i][3]);
            }
            // transpose 8 keys x 8 channels -> Vt[sg][gg][d][key i]
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t lo4[4], hi4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    lo4[q] = __builtin_amdgcn_perm(h[2 * q + 1][p], h[2 * q][p], 0x05040100u);
                    hi4[q] = __builtin_amdgcn_perm(h[2 * q + 1][p], h[2 * q][p], 0x07060302u);
                }
                _Float16* base = &Vt[((sg * 2 + gg) * D + 8 * j + 2 * p) * 8];
                *reinterpret_cast<uint4*>(base) = make_uint4(lo4[0], lo4[1], lo4[2], lo4[3]);
                *reinterpret_cast<uint4*>(base + 8) = make_uint4(hi4[0], hi4[1], hi4[2], hi4[3]);
            }
        }
        __syncthreads();

        // ---------------- 2. S^T partial over this wave's channel half
        floatx16 s_acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) s_acc[r] = 0.0f;
#pragma unroll
        for (int st = 0; st < SSTEPS; ++st) {
            const int d0 = dh * DH + 16 * st + 8 * (lane >> 5);
            const half8 kf = *reinterpret_cast<const half8*>(&Kt[(lane & 31) * KROW + d0]);
            s_acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[st], s_acc, 0, 0, 0);
        }
        int kv_ok[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) kv_ok[r] = kvalid[8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)];
        __syncthreads();   // everyone done reading Kt before Spart overwrites it
#pragma unroll
        for (int r = 0; r < 16; ++r) Spart[(wv * 16 + r) * 64 + lane] = s_acc[r];
        __syncthreads();
        float t2[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float s = Spart[(hg * 16 + r) * 64 + lane] + Spart[((hg + 2) * 16 + r) * 64 + lane];
            t2[r] = kv_ok[r] ? s * a.c2 : -__builtin_inff();
        }

        // ---------------- 3. online softmax (base 2)
        float tmax = t2[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, t2[r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        float alpha = 1.0f;
        uint32_t pk[8];
        float psum = 0.0f;
        if (m_new == -__builtin_inff()) {
#pragma unroll
            for (int q = 0; q < 8; ++q) pk[q] = 0u;
        } else {
            alpha = exp2f(m_run - m_new);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const _Float16 p0 = static_cast<_Float16>(exp2f(t2[2 * q] - m_new));
                const _Float16 p1 = static_cast<_Float16>(exp2f(t2[2 * q + 1] - m_new));
                psum += static_cast<float>(p0) + static_cast<float>(p1);
                pk[q] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, p0)) |
                        (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, p1)) << 16);
            }
        }
        m_run = m_new;
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o_acc[mt][r] *= alpha;

        // ---------------- 4. O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const half8 pf = __builtin_bit_cast(half8, make_uint4(pk[4 * ks], pk[4 * ks + 1],
                                                                  pk[4 * ks + 2], pk[4 * ks + 3]));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int d = dh * DH + 32 * mt + (lane & 31);
                const half8 vf = *reinterpret_cast<const half8*>(&Vt[((ks * 2 + (lane >> 5)) * D + d) * 8]);
                o_acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o_acc[mt], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---------------- epilogue
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const int head_local = 32 * hg + (lane & 31);
    const int head = hbase + head_local;
    if (a.splits == 1) {
        if (head < a.H) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            float* orow = a.out + (u * a.H + head) * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = dh * DH + 32 * mt + 8 * r4 + 4 * (lane >> 5);
                    *reinterpret_cast<float4*>(orow + d) =
                        make_float4(o_acc[mt][4 * r4] * inv, o_acc[mt][4 * r4 + 1] * inv,
                                    o_acc[mt][4 * r4 + 2] * inv, o_acc[mt][4 * r4 + 3] * inv);
                }
        }
    } else {
        const int64_t pidx = (u * gridDim.z + hb) * a.splits + split;
        float* po = a.ws_o + pidx * (64 * D);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) po[((wv * MT + mt) * 16 + r) * 64 + lane] = o_acc[mt][r];
        if (dh == 0 && lane < 32) {
            a.ws_m[pidx * 64 + head_local] = m_run;
            a.ws_l[pidx * 64 + head_local] = l_tot;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ws_o,
                                                      const float* __restrict__ ws_m,
                                                      const float* __restrict__ ws_l, int splits,
                                                      int H, int hblocks, float* __restrict__ out) {
    constexpr int DH = D / 2, MT = DH / 32;
    const int64_t ub = blockIdx.x;                 // unit * hblocks + hb
    const int e = blockIdx.y * 256 + threadIdx.x;  // head_local * D + d
    if (e >= 64 * D) return;
    const int head_local = e / D, d = e % D;
    const int hb = static_cast<int>(ub % hblocks);
    const int64_t u = ub / hblocks;
    const int head = hb * 64 + head_local;
    if (head >= H) return;
    const int hg = head_local / 32, dhh = d / DH, dd = d % DH;
    const int mt = dd / 32, x = dd % 32;
    const int r = 4 * (x / 8) + (x % 4);
    const int ln = 32 * ((x % 8) / 4) + (head_local % 32);
    const int wv = hg + 2 * dhh;
    const int64_t nat = ((wv * MT + mt) * 16 + r) * 64 + ln;
    float mstar = -__builtin_inff();
    for (int s = 0; s < splits; ++s) mstar = fmaxf(mstar, ws_m[(ub * splits + s) * 64 + head_local]);
    float num = 0.0f, den = 0.0f;
    if (mstar != -__builtin_inff()) {
        for (int s = 0; s < splits; ++s) {
            const int64_t p = ub * splits + s;
            const float ms = ws_m[p * 64 + head_local];
            if (ms == -__builtin_inff()) continue;
            const float wgt = exp2f(ms - mstar);
            num += wgt * ws_o[p * (64 * D) + nat];
            den += wgt * ws_l[p * 64 + head_local];
        }
    }
    out[(u * H + head) * D + d] = den > 0.0f ? num / den : 0.0f;
}

struct SplitPlan { int splits, tiles_per_split, n_tiles; };

SplitPlan plan(int64_t units, int H, int k, int W) {
    SplitPlan p;
    p.n_tiles = (k + W + kKT - 1) / kKT;
    const int64_t hblocks = (H + 63) / 64;
    const int64_t base = units * hblocks;
    int64_t want = (512 + base - 1) / base;          // aim for ~512 workgroups
    int64_t max_splits = (p.n_tiles + 3) / 4;        // keep >= 4 tiles per split
    if (want > max_splits) want = max_splits;
    if (want < 1) want = 1;
    p.tiles_per_split = static_cast<int>((p.n_tiles + want - 1) / want);
    if (p.tiles_per_split < 1) p.tiles_per_split = 1;
    p.splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
    if (p.splits < 1) p.splits = 1;
    return p;
}

template <int D>
hipError_t launch_d(const AttnLaunch& L, hipStream_t st) {
    const SplitPlan sp = plan(L.units, L.H, L.k, L.W);
    const int hblocks = (L.H + 63) / 64;
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(L.q); a.q_bf16 = L.q_bf16;
    a.codes = L.codes; a.scales = L.scales; a.cap = L.cap; a.kv_unit_stride = L.kv_unit_stride;
    a.idx = L.idx; a.k = L.k;
    a.swa = static_cast<const uint8_t*>(L.swa); a.swa_bf16 = L.swa_bf16; a.W = L.W;
    a.swa_len = L.swa_len; a.q_pos0 = L.q_pos0; a.swa_start = L.swa_start; a.prefill = L.prefill;
    a.units = L.units; a.H = L.H; a.c2 = L.sm_scale * kLog2e; a.out = L.out;
    a.splits = sp.splits; a.tiles_per_split = sp.tiles_per_split; a.n_tiles = sp.n_tiles;
    const int64_t nparts = L.units * hblocks * sp.splits;
    a.ws_o = L.ws;
    a.ws_m = L.ws ? L.ws + nparts * 64 * D : nullptr;
    a.ws_l = L.ws ? a.ws_m + nparts * 64 : nullptr;
    if (L.units == 0) return hipSuccess;
    attn_kernel<D><<<dim3(static_cast<unsigned>(L.units), sp.splits, hblocks), kThreads, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sp.splits == 1) return e;
    combine_kernel<D><<<dim3(static_cast<unsigned>(L.units * hblocks), (64 * D + 255) / 256), 256, 0, st>>>(
        a.ws_o, a.ws_m, a.ws_l, sp.splits, L.H, hblocks, L.out);
    return hipGetLastError();
}

}  // namespace

bool attn_shape_supported(int H, int D) {
    return (D == 512 && H > 0 && H % 64 == 0) || (D == 64 && H > 0 && H <= 64);
}

size_t attn_workspace_bytes(int64_t units, int H, int D, int k, int W) {
    const SplitPlan sp = plan(units, H, k, W);
    if (sp.splits == 1) return 0;
    const int64_t hblocks = (H + 63) / 64;
    const int64_t nparts = units * hblocks * sp.splits;
    return static_cast<size_t>(nparts) * (64 * static_cast<size_t>(D) + 128) * sizeof(float);
}

hipError_t launch_attn(const AttnLaunch& L, hipStream_t st) {
    if (L.D == 512) return launch_d<512>(L, st);
    if (L.D == 64) return launch_d<64>(L, st);
    return hipErrorInvalidValue;
}

}  // namespace csa2
