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
// Work split: one workgroup = (unit, key split, block of 64 heads), 2*NQ
// waves (8 at D = 512).  Wave w owns head group hg = w & 1 (32 heads) and
// channel slice dq = w >> 1 (D/NQ channels).  Keys stream in tiles of 32:
//  1. all threads gather the tile's rows (prefetched one tile ahead) and
//     dequantise them to fp16 into LDS twice: key-major Kt[key][d] (for S)
//     and Vt[step][grp][cell(d)][8 keys] (for P.V, so every MFMA operand is
//     one 16-byte LDS read; cell() is a bank swizzle);
//  2. S^T[key][head] over this wave's channel slice with
//     v_mfma_f32_32x32x16_f16 (A = key rows, B = q in registers), then the
//     NQ slices are added through LDS (same order in every wave);
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
constexpr int kMaxTilesPerSplit = 16;
constexpr int kCombineMaxSplits = 64;  // key splits one combine block can merge
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

// NQ = channel splits: the workgroup has 2*NQ waves; wave w owns head group
// hg = w & 1 (32 heads) and channel slice dq = w >> 1 (D/NQ channels) for
// both the S partial and its slice of O.
template <int D, int NQ, bool BF16>
__global__ __launch_bounds__(128 * NQ) void attn_kernel(AttnArgs a) {
    constexpr int NW = 2 * NQ;             // waves
    constexpr int NT = 64 * NW;            // threads
    constexpr int DQ = D / NQ;             // channels per wave
    constexpr int SSTEPS = DQ / 16;        // MFMA k-steps for the S partial
    constexpr int MT = DQ / 32;            // O^T row tiles per wave
    constexpr int KROW = D + 8;            // padded Kt row (halves)
    constexpr int CH = D / 8;              // 8-channel chunks per row
    constexpr int KPT = kKT / NW;          // keys dequantised per thread
    static_assert(DQ % 32 == 0 && (KPT == 4 || KPT == 8), "unsupported split");
    // Kt is dead once S is formed, so the S partials ([NW][16][64] float32)
    // reuse its space.
    constexpr int KT_BYTES = kKT * KROW * 2;
    constexpr int SP_BYTES = NW * 16 * 64 * 4;
    constexpr int KBUF = KT_BYTES > SP_BYTES ? KT_BYTES : SP_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char kbuf[KBUF];
    __shared__ __attribute__((aligned(16))) _Float16 Vt[kKT * D];
    // 0 for a key that holds a row, -inf for an empty slot: added to the
    // logits, so empty slots get probability exactly 0 without a branch
    __shared__ __attribute__((aligned(16))) float kmask[kKT];
    __shared__ int32_t idx_s[kKT * kMaxTilesPerSplit];
    _Float16* Kt = reinterpret_cast<_Float16*>(kbuf);
    float* Spart = reinterpret_cast<float*>(kbuf);

    // the wave index is uniform within a wave: make that explicit so every
    // decision derived from it (key slot, channel slice) is a scalar branch
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hg = wv & 1, dq = wv >> 1;
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
    // channels dq*DQ + 16*st + 8*(lane/32) + 0..7
    half8 qf[SSTEPS];
    {
        // loads from a clamped (always valid) head, masked afterwards, so no
        // load sits in a lane-divergent branch
        const int head = hbase + 32 * hg + (lane & 31);
        const bool hv = head < a.H;
        const int64_t qrow = (u * a.H + (hv ? head : 0)) * D;
        uint4 raw[SSTEPS][BF16 ? 1 : 2];
#pragma unroll
        for (int st = 0; st < SSTEPS; ++st) {
            const int d0 = dq * DQ + 16 * st + 8 * (lane >> 5);
            if (BF16) {
                raw[st][0] = *reinterpret_cast<const uint4*>(a.q + qrow + d0);
            } else {
                const float* qf32 = reinterpret_cast<const float*>(a.q) + qrow + d0;
                raw[st][0] = *reinterpret_cast<const uint4*>(qf32);
                raw[st][BF16 ? 0 : 1] = *reinterpret_cast<const uint4*>(qf32 + 4);
            }
        }
#pragma unroll
        for (int st = 0; st < SSTEPS; ++st) {
            uint32_t wd[4];
            if (BF16) {
                const uint32_t in[4] = {raw[st][0].x, raw[st][0].y, raw[st][0].z, raw[st][0].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    wd[e] = pack_h2(__uint_as_float(in[e] << 16), __uint_as_float(in[e] & 0xffff0000u));
            } else {
                const uint4 r1 = raw[st][BF16 ? 0 : 1];
                wd[0] = pack_h2(__uint_as_float(raw[st][0].x), __uint_as_float(raw[st][0].y));
                wd[1] = pack_h2(__uint_as_float(raw[st][0].z), __uint_as_float(raw[st][0].w));
                wd[2] = pack_h2(__uint_as_float(r1.x), __uint_as_float(r1.y));
                wd[3] = pack_h2(__uint_as_float(r1.z), __uint_as_float(r1.w));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) wd[e] = hv ? wd[e] : 0u;
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

    // index entries of the main-KV slots, staged kMaxTilesPerSplit tiles at
    // a time (window starting at tile win0)
    int win0 = t_begin;
    auto stage_idx = [&](int first_tile) {
        win0 = first_tile;
        for (int i = tid; i < kMaxTilesPerSplit * kKT; i += NT) {
            const int slot = first_tile * kKT + i;
            idx_s[i] = slot < a.k ? idx[slot] : -1;
        }
    };
    stage_idx(t_begin);
    __syncthreads();

    // dequant role: this wave covers KPT keys of the 8-key group g8 (step
    // sg = g8 >> 1, group gg = g8 & 1), slots i8 = i + 8 - ... of that group;
    // lane j handles channels 8j..8j+7.
    const int g8 = KPT == 8 ? wv : (wv >> 1);
    const int half = KPT == 8 ? 0 : (wv & 1);
    const int sg = g8 >> 1, gg = g8 & 1;
    const int j = lane;
    auto key_of_i = [&](int i) {
        const int i8 = half * 4 + i;
        return 16 * sg + 4 * gg + (i8 & 3) + 8 * (i8 >> 2);
    };

    // raw tile data for this thread's keys, prefetched one tile ahead:
    // kind 0 empty, 1 MXFP4 row (code word + scale byte), 2 window row (16
    // bytes of bf16 or 32 of float32).  Main and window rows use separate
    // registers so a load never has to wait for another load's register.
    constexpr int WWORDS = BF16 ? 4 : 8;
    uint32_t raw_cw[KPT], raw_sc[KPT], raw_sw[KPT][WWORDS];
    int raw_kind[KPT];
    // Every branch below is wave-uniform (it depends on the key slot only);
    // lanes past the row's chunk count load a clamped chunk and skip their
    // stores later, so no load sits in a lane-divergent branch.
    const int jl = j < CH ? j : 0;
    auto load_raw = [&](int tile) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int slot = tile * kKT + key_of_i(i);
            if (slot < a.k) {
                const int32_t row = __builtin_amdgcn_readfirstlane(idx_s[slot - win0 * kKT]);
                const bool ok = row >= 0 && row < a.cap;
                const int64_t rr = kvbase + (ok ? row : 0);
                raw_kind[i] = ok ? 1 : 0;
                raw_cw[i] = *reinterpret_cast<const uint32_t*>(a.codes + rr * (D / 2) + 4 * jl);
                raw_sc[i] = a.scales[rr * (D / 16) + (jl >> 1)];
            } else if (slot < n_slots && slot - a.k < n_swa) {
                const int r = slot - a.k;
                raw_kind[i] = 2;
                const uint4* src = reinterpret_cast<const uint4*>(swa_rows + r * swa_row_bytes + WWORDS * 4 * jl);
                const uint4 v0 = src[0];
                raw_sw[i][0] = v0.x; raw_sw[i][1] = v0.y; raw_sw[i][2] = v0.z; raw_sw[i][3] = v0.w;
                if (!BF16) {
                    const uint4 v1 = src[1];
                    raw_sw[i][WWORDS - 4] = v1.x; raw_sw[i][WWORDS - 3] = v1.y;
                    raw_sw[i][WWORDS - 2] = v1.z; raw_sw[i][WWORDS - 1] = v1.w;
                }
            } else {
                raw_kind[i] = 0;
            }
        }
    };

    // Vt cell of channel d: the low three bits are XORed with the next three,
    // so the dequantising lanes (channels 8j + c for lanes j) spread over all
    // banks instead of landing 128 bytes apart, while any 8 consecutive
    // channels read by the P.V operand still fill 8 distinct cells.
    auto vcell = [](int d) { return d ^ ((d >> 3) & 7); };

    // dequantise this thread's KPT keys (values in h) into Kt and Vt
    auto store_tile = [&](const uint32_t (&h)[KPT][4], const int (&kind)[KPT]) {
        if (j < CH) {
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int key = key_of_i(i);
                if (j == 0) kmask[key] = kind[i] != 0 ? 0.0f : -__builtin_inff();
                *reinterpret_cast<uint4*>(&Kt[key * KROW + 8 * j]) =
                    make_uint4(h[i][0], h[i][1], h[i][2], h[i][3]);
            }
            // transpose KPT keys x 8 channels into Vt[sg][gg][d][slot i8]
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t lo4[KPT / 2], hi4[KPT / 2];
#pragma unroll
                for (int q = 0; q < KPT / 2; ++q) {
                    lo4[q] = __builtin_amdgcn_perm(h[2 * q + 1][p], h[2 * q][p], 0x05040100u);
                    hi4[q] = __builtin_amdgcn_perm(h[2 * q + 1][p], h[2 * q][p], 0x07060302u);
                }
                const int grp = (sg * 2 + gg) * D;
                _Float16* lo_p = &Vt[(grp + vcell(8 * j + 2 * p)) * 8 + 4 * half];
                _Float16* hi_p = &Vt[(grp + vcell(8 * j + 2 * p + 1)) * 8 + 4 * half];
                if (KPT == 8) {
                    *reinterpret_cast<uint4*>(lo_p) = make_uint4(lo4[0], lo4[1], lo4[KPT / 2 - 2], lo4[KPT / 2 - 1]);
                    *reinterpret_cast<uint4*>(hi_p) = make_uint4(hi4[0], hi4[1], hi4[KPT / 2 - 2], hi4[KPT / 2 - 1]);
                } else {
                    *reinterpret_cast<uint2*>(lo_p) = make_uint2(lo4[0], lo4[KPT / 2 - 1]);
                    *reinterpret_cast<uint2*>(hi_p) = make_uint2(hi4[0], hi4[KPT / 2 - 1]);
                }
            }
        }
    };

    // S, online softmax and P.V for the tile currently in Kt/Vt
    auto tile_math = [&]() {
        // ---------------- 2. S^T partial over this wave's channel slice
        floatx16 s_acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) s_acc[r] = 0.0f;
#pragma unroll
        for (int st = 0; st < SSTEPS; ++st) {
            const int d0 = dq * DQ + 16 * st + 8 * (lane >> 5);
            const half8 kf = *reinterpret_cast<const half8*>(&Kt[(lane & 31) * KROW + d0]);
            s_acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[st], s_acc, 0, 0, 0);
        }
        float kmk[16];
        {
            const float4* km4 = reinterpret_cast<const float4*>(kmask);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                // rows 8*r4 + 4*(lane/32) + 0..3
                const float4 v = km4[2 * r4 + (lane >> 5)];
                kmk[4 * r4] = v.x; kmk[4 * r4 + 1] = v.y; kmk[4 * r4 + 2] = v.z; kmk[4 * r4 + 3] = v.w;
            }
        }
        __syncthreads();   // everyone done reading Kt before Spart overwrites it
        // partials as [wave][r/4][lane][4]: one 16-byte LDS access per 4 rows
        float4* Sp4 = reinterpret_cast<float4*>(Spart);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            Sp4[(wv * 4 + r4) * 64 + lane] = make_float4(s_acc[4 * r4], s_acc[4 * r4 + 1],
                                                         s_acc[4 * r4 + 2], s_acc[4 * r4 + 3]);
        __syncthreads();
        float t2[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            float4 sum = Sp4[(hg * 4 + r4) * 64 + lane];
#pragma unroll
            for (int qq = 1; qq < NQ; ++qq) {
                const float4 v = Sp4[((hg + 2 * qq) * 4 + r4) * 64 + lane];
                sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
            }
            t2[4 * r4] = fmaf(sum.x, a.c2, kmk[4 * r4]);
            t2[4 * r4 + 1] = fmaf(sum.y, a.c2, kmk[4 * r4 + 1]);
            t2[4 * r4 + 2] = fmaf(sum.z, a.c2, kmk[4 * r4 + 2]);
            t2[4 * r4 + 3] = fmaf(sum.w, a.c2, kmk[4 * r4 + 3]);
        }

        // ---------------- 3. online softmax (base 2) with a lazy reference:
        // probabilities are exp2(t - m_ref); m_ref moves (and O, l are
        // rescaled) only when some lane's tile max exceeds it by more than 8,
        // so p stays below 2^8 and the rescale is rare.  The final division
        // by l uses the same reference, so the result does not depend on it.
        float tmax = t2[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, t2[r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool grow = tmax > m_run + 8.0f || (m_run == -__builtin_inff() && tmax != -__builtin_inff());
        if (__ballot(grow) != 0) {
            const float m_new = grow ? tmax : m_run;
            const float alpha = (m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            if (m_new != m_run) {
                l_run *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o_acc[mt][r] *= alpha;
            }
            m_run = m_new;
        }
        uint32_t pk[8];
        float psum = 0.0f;
        if (m_run == -__builtin_inff()) {
#pragma unroll
            for (int q = 0; q < 8; ++q) pk[q] = 0u;
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                // v_exp_f32 directly: arguments are <= 8, and results too
                // small for fp16 become 0 either way
                const half2v ph = {static_cast<_Float16>(__builtin_amdgcn_exp2f(t2[2 * q] - m_run)),
                                   static_cast<_Float16>(__builtin_amdgcn_exp2f(t2[2 * q + 1] - m_run))};
                psum = __builtin_amdgcn_fdot2(ph, half2v{1.0f16, 1.0f16}, psum, false);
                pk[q] = __builtin_bit_cast(uint32_t, ph);
            }
        }
        l_run += psum;

        // ---------------- 4. O^T += V^T P^T over this wave's channel slice
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const half8 pf = __builtin_bit_cast(half8, make_uint4(pk[4 * ks], pk[4 * ks + 1],
                                                                  pk[4 * ks + 2], pk[4 * ks + 3]));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int d = dq * DQ + 32 * mt + (lane & 31);
                const half8 vf = *reinterpret_cast<const half8*>(&Vt[((ks * 2 + (lane >> 5)) * D + vcell(d)) * 8]);
                o_acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o_acc[mt], 0, 0, 0);
            }
        }
    };

    // ---- main tiles (every slot a main-KV slot): branch-free gathers
    // prefetched one tile ahead into registers no other path writes
    const int t_main_end = (a.k / kKT) < t_end ? (a.k / kKT) : t_end;
    uint32_t pm_cw[KPT], pm_sc[KPT];
    int pm_ok[KPT];
    auto load_main = [&](int tile) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int slot = tile * kKT + key_of_i(i);
            const int32_t row = __builtin_amdgcn_readfirstlane(idx_s[slot - win0 * kKT]);
            const bool ok = row >= 0 && row < a.cap;
            const int64_t rr = kvbase + (ok ? row : 0);
            pm_ok[i] = ok;
            pm_cw[i] = *reinterpret_cast<const uint32_t*>(a.codes + rr * (D / 2) + 4 * jl);
            pm_sc[i] = a.scales[rr * (D / 16) + (jl >> 1)];
        }
    };
    if (t_begin < t_main_end) load_main(t_begin);
    for (int tile = t_begin; tile < t_main_end; ++tile) {
        {
            uint32_t h[KPT][4];
            int kind[KPT];
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const uint32_t s16 = f16_bits(e4m3_val(pm_sc[i] & 0x7fu));
                dequant8(pm_cw[i], s16 | (s16 << 16), h[i]);
                // an empty slot keeps the (finite) values of the clamped row:
                // its logit is -inf, so it enters P.V with weight exactly 0
                kind[i] = pm_ok[i] ? 1 : 0;
            }
            store_tile(h, kind);
        }
        __syncthreads();
        if (tile + 1 < t_main_end) {                // in flight during this tile's math
            if (tile + 1 - win0 == kMaxTilesPerSplit) {
                stage_idx(tile + 1);
                __syncthreads();
            }
            load_main(tile + 1);
        }
        tile_math();
        __syncthreads();
    }

    // ---- remaining tiles (window rows, or a tile straddling the main/window
    // boundary): generic gather, not prefetched (at most a few tiles)
    for (int tile = t_begin > t_main_end ? t_begin : t_main_end; tile < t_end; ++tile) {
        if (tile - win0 >= kMaxTilesPerSplit) {
            stage_idx(tile);
            __syncthreads();
        }
        load_raw(tile);
        {
            uint32_t h[KPT][4];
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                if (raw_kind[i] == 1) {
                    const uint32_t s16 = f16_bits(e4m3_val(raw_sc[i] & 0x7fu));
                    dequant8(raw_cw[i], s16 | (s16 << 16), h[i]);
                } else if (raw_kind[i] == 2) {
                    if (BF16) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            h[i][e] = pack_h2(__uint_as_float(raw_sw[i][e] << 16),
                                              __uint_as_float(raw_sw[i][e] & 0xffff0000u));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            h[i][e] = pack_h2(__uint_as_float(raw_sw[i][2 * e]),
                                              __uint_as_float(raw_sw[i][2 * e + 1 < WWORDS ? 2 * e + 1 : 0]));
                    }
                } else {
                    h[i][0] = h[i][1] = h[i][2] = h[i][3] = 0u;
                }
            }
            store_tile(h, raw_kind);
        }
        __syncthreads();
        tile_math();
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
                    const int d = dq * DQ + 32 * mt + 8 * r4 + 4 * (lane >> 5);
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
        if (dq == 0 && lane < 32) {
            a.ws_m[pidx * 64 + head_local] = m_run;
            a.ws_l[pidx * 64 + head_local] = l_tot;
        }
    }
}

// Merge the key-split partials of one (unit, 64-head block): workgroup y
// covers one (wave, row-tile) block of the partial layout, i.e. 32 heads x
// 32 consecutive channels.  Reads are in the partials' own (coalesced)
// order; the result is transposed through LDS so the output rows are
// written as 128-byte runs.
template <int D, int NQ>
__global__ __launch_bounds__(1024) void combine_kernel(const float* __restrict__ ws_o,
                                                       const float* __restrict__ ws_m,
                                                       const float* __restrict__ ws_l, int splits,
                                                       int H, int hblocks, float* __restrict__ out) {
    constexpr int DQ = D / NQ, MT = DQ / 32;
    __shared__ float tile[32][33];
    __shared__ float wgt[kCombineMaxSplits][32];   // m_s, then exp2(m_s - m*), per split and head
    __shared__ float lsum[kCombineMaxSplits][32];
    __shared__ float inv_den[32];
    const int64_t ub = blockIdx.x;                 // unit * hblocks + hb
    const int wv = blockIdx.y / MT, mt = blockIdx.y % MT;
    const int hg = wv & 1, dqq = wv >> 1;
    const int t = threadIdx.x, r = t >> 6, ln = t & 63;
    const int hcol = ln & 31;
    const int dd = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
    const int64_t nat = ((wv * MT + mt) * 16 + r) * 64 + ln;
    const float* po = ws_o + ub * splits * static_cast<int64_t>(64 * D) + nat;
    constexpr int64_t PS = 64 * D;                 // partial stride
    // the first 16 splits' partials are loaded before the weights are
    // formed, so the two latencies overlap
    constexpr int kEarly = 16;
    float oe[kEarly];
#pragma unroll
    for (int i = 0; i < kEarly; ++i) oe[i] = i < splits ? po[i * PS] : 0.0f;
    // per-head split weights, once per block: thread t loads (split t/32,
    // head 32hg + t%32), then thread t < 32 reduces over the splits in LDS
    {
        const int h = t & 31;
        for (int s = t >> 5; s < splits; s += 32) {
            const int64_t p = (ub * splits + s) * 64 + 32 * hg + h;
            wgt[s][h] = ws_m[p];
            lsum[s][h] = ws_l[p];
        }
    }
    __syncthreads();
    if (t < 32) {
        float mstar = -__builtin_inff();
        for (int s = 0; s < splits; ++s) mstar = fmaxf(mstar, wgt[s][t]);
        float den = 0.0f;
        for (int s = 0; s < splits; ++s) {
            const float ms = wgt[s][t];
            const float w = (ms == -__builtin_inff()) ? 0.0f : exp2f(ms - mstar);
            wgt[s][t] = w;
            den += w * lsum[s][t];
        }
        inv_den[t] = den > 0.0f ? 1.0f / den : 0.0f;
    }
    __syncthreads();
    float num = 0.0f;
#pragma unroll
    for (int i = 0; i < kEarly; ++i) num += i < splits ? wgt[i][hcol] * oe[i] : 0.0f;
    int s = kEarly;
    for (; s + 8 <= splits; s += 8) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = po[(s + i) * PS];
#pragma unroll
        for (int i = 0; i < 8; ++i) num += wgt[s + i][hcol] * o[i];
    }
    for (; s < splits; ++s) num += wgt[s][hcol] * po[s * PS];
    tile[hcol][dd] = num * inv_den[hcol];
    __syncthreads();
    const int hb = static_cast<int>(ub % hblocks);
    const int64_t u = ub / hblocks;
    const int oh = t >> 5, od = t & 31;
    const int head = hb * 64 + 32 * hg + oh;
    if (head < H) out[(u * H + head) * D + dqq * DQ + 32 * mt + od] = tile[oh][od];
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
    if (want > kCombineMaxSplits) want = kCombineMaxSplits;
    if (want < 1) want = 1;
    p.tiles_per_split = static_cast<int>((p.n_tiles + want - 1) / want);
    if (p.tiles_per_split < 1) p.tiles_per_split = 1;
    p.splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
    if (p.splits < 1) p.splits = 1;
    return p;
}

template <int D, int NQ, bool BF16>
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
    attn_kernel<D, NQ, BF16><<<dim3(static_cast<unsigned>(L.units), sp.splits, hblocks), 128 * NQ, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sp.splits == 1) return e;
    combine_kernel<D, NQ><<<dim3(static_cast<unsigned>(L.units * hblocks), 2 * NQ * (D / NQ / 32)), 1024, 0, st>>>(
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
    if (L.q_bf16 != L.swa_bf16) return hipErrorInvalidValue;
    if (L.D == 512) return L.q_bf16 ? launch_d<512, 4, true>(L, st) : launch_d<512, 4, false>(L, st);
    if (L.D == 64) return L.q_bf16 ? launch_d<64, 2, true>(L, st) : launch_d<64, 2, false>(L, st);
    return hipErrorInvalidValue;
}

}  // namespace csa2
