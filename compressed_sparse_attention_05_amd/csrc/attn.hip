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
// Two kernels share the tile scheme (keys stream through LDS in tiles, the
// dequantised tile is stored once key-major, and P.V reads it transposed
// with ds_read_b64_tr_b16):
//  * attn_kernel<D, NQ> (D = 64): one workgroup =
//    (unit, key split, block of 64 heads), 2*NQ waves; wave w owns head group
//    hg = w & 1 and channel slice dq = w >> 1.  Per tile all waves gather and
//    dequantise, form S^T over their channel slice (the NQ slices added
//    through LDS), run the online softmax and add V^T P^T for their slice;
//  * attn_ws_kernel (D = 512, any number of units): warp-specialised, see
//    there.
// Common to both:
//  - S^T[key][head] with v_mfma_f32_32x32x16_f16 (A = key rows, B = q);
//  - online softmax in base 2 with a lazy reference: p = exp2(t - m_ref),
//    m_ref moves (and O, l are rescaled) only when a tile max exceeds it by
//    more than 8, so p < 2^8; the final division uses the same reference;
//  - O^T[d][head] += V^T P^T with the fp16-rounded probabilities taken
//    straight from the S accumulators (the MFMA k-slot order is chosen to be
//    the accumulator row order); the running sum uses the same rounded p.
// Partial results of several key splits are merged by combine_kernel.
//
// Exactness: every MXFP4 value is an fp16 number (E2M1 times E4M3 has at
// most 5 significant bits, range 2^-10..2688) and bf16 q / SWA values in
// [2^-14, 65504] are fp16 numbers, so the operands are exact; MFMA sums in
// float32; only P is rounded (to fp16, relative 2^-11).
#include <type_traits>

#include "csa2_internal.h"

namespace csa2 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

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
    // partials (splits > 1): each split's output divided by its own row sum,
    // as fp16, and its row max and row sum as fp32
    _Float16* ws_o; float* ws_m; float* ws_l;
    int splits, tiles_per_split, n_tiles;
};

__device__ __forceinline__ uint32_t f16_bits(float v) {
    _Float16 h = static_cast<_Float16>(v);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

// 8 MXFP4 nibbles (channels 0..7 of a code dword, channel 2i in the low
// nibble of byte i) times their E4M3 scale -> 4 dwords of packed fp16 pairs
// (channel 2p low half, 2p+1 high half), with the gfx950 converters: E2M1
// pairs to fp16 at unit scale (the converter applies only the exponent of its
// scale, so the E4M3 scale is a separate fp16 multiply) and the E4M3 scale
// byte to an fp16 pair.  Every step is exact: E2M1 times E4M3 has at most 5
// significant bits within fp16 range.  The scale code is clamped to 0x7e: an
// unwritten row's 0x7f (NaN in E4M3) must stay finite, since its zero weight
// only cancels finite values.
__device__ __forceinline__ void dequant8_hw(uint32_t cw, uint32_t sc, uint32_t out[4]) {
    uint32_t c = sc & 0x7fu;
    c = c < 0x7eu ? c : 0x7eu;
    const half2v s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c | (c << 8), 1.0f, false);
    const half2v v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0);
    const half2v v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1);
    const half2v v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2);
    const half2v v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3);
    out[0] = __builtin_bit_cast(uint32_t, v0 * s);
    out[1] = __builtin_bit_cast(uint32_t, v1 * s);
    out[2] = __builtin_bit_cast(uint32_t, v2 * s);
    out[3] = __builtin_bit_cast(uint32_t, v3 * s);
}

// 32 channels (a 16-byte code run) under their two scale bytes (sc: the
// bytes of channels 0..15 and 16..31): dequant8_hw four times, with each
// scale converted once.  out[4e + j]: channels 8e + 2j, 8e + 2j + 1.
__device__ __forceinline__ void dequant32_hw(const uint4& cw4, uint32_t sc, uint32_t (&out)[16]) {
    uint32_t c0 = sc & 0x7fu, c1 = (sc >> 8) & 0x7fu;
    c0 = c0 < 0x7eu ? c0 : 0x7eu;
    c1 = c1 < 0x7eu ? c1 : 0x7eu;
    const half2v s0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0 | (c0 << 8), 1.0f, false);
    const half2v s1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1 | (c1 << 8), 1.0f, false);
    const uint32_t cw[4] = {cw4.x, cw4.y, cw4.z, cw4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const half2v s = e < 2 ? s0 : s1;
        out[4 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 0) * s);
        out[4 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 1) * s);
        out[4 * e + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 2) * s);
        out[4 * e + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 3) * s);
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
    constexpr int KT = 8 * NW;             // keys per tile (64 at D = 512)
    constexpr int KPT = 8;                 // keys dequantised per thread
    constexpr int MK = KT / 32;            // 32-key row blocks of S^T per tile
    static_assert(DQ % 32 == 0, "unsupported split");
    // Kt holds the tile once, key-major; P.V reads it transposed
    // (ds_read_b64_tr_b16), so there is no second copy.
    __shared__ __attribute__((aligned(16))) _Float16 Kt[KT * KROW];
    __shared__ __attribute__((aligned(16))) float Spart[NW * MK * 16 * 64];
    // 0 for a key that holds a row, -inf for an empty slot: added to the
    // logits, so empty slots get probability exactly 0 without a branch
    __shared__ __attribute__((aligned(16))) float kmask[KT];
    __shared__ int32_t idx_s[KT * kMaxTilesPerSplit];

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
        for (int i = tid; i < kMaxTilesPerSplit * KT; i += NT) {
            const int slot = first_tile * KT + i;
            idx_s[i] = slot < a.k ? idx[slot] : -1;
        }
    };
    stage_idx(t_begin);
    __syncthreads();

    // dequant role: this wave covers KPT keys of the 8-key group g8 (step
    // sg = g8 >> 1, group gg = g8 & 1), slots i8 = i + 8 - ... of that group;
    // lane j handles channels 8j..8j+7.
    const int g8 = wv;
    const int half = 0;
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
            const int slot = tile * KT + key_of_i(i);
            if (slot < a.k) {
                const int32_t row = __builtin_amdgcn_readfirstlane(idx_s[slot - win0 * KT]);
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

    // dequantised KPT keys of this thread (values in h) into Kt
    auto store_tile = [&](const uint32_t (&h)[KPT][4], const int (&kind)[KPT]) {
        if (j < CH) {
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int key = key_of_i(i);
                if (j == 0) kmask[key] = kind[i] != 0 ? 0.0f : -__builtin_inff();
                *reinterpret_cast<uint4*>(&Kt[key * KROW + 8 * j]) =
                    make_uint4(h[i][0], h[i][1], h[i][2], h[i][3]);
            }
        }
    };

    // S, online softmax and P.V for the tile currently in Kt
    auto tile_math = [&]() {
        // ---------------- 2. S^T partial over this wave's channel slice, one
        // 32-key row block at a time
        floatx16 s_acc[MK];
#pragma unroll
        for (int mk = 0; mk < MK; ++mk) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s_acc[mk][r] = 0.0f;
#pragma unroll
            for (int st = 0; st < SSTEPS; ++st) {
                const int d0 = dq * DQ + 16 * st + 8 * (lane >> 5);
                const half8 kf = *reinterpret_cast<const half8*>(&Kt[(32 * mk + (lane & 31)) * KROW + d0]);
                s_acc[mk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[st], s_acc[mk], 0, 0, 0);
            }
        }
        // partials as [wave][mk][r/4][lane][4]: one 16-byte LDS access per 4 rows
        float4* Sp4 = reinterpret_cast<float4*>(Spart);
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                Sp4[((wv * MK + mk) * 4 + r4) * 64 + lane] =
                    make_float4(s_acc[mk][4 * r4], s_acc[mk][4 * r4 + 1], s_acc[mk][4 * r4 + 2], s_acc[mk][4 * r4 + 3]);
        __syncthreads();
        float t2[MK][16];
        const float4* km4 = reinterpret_cast<const float4*>(kmask);
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float4 sum = Sp4[((hg * MK + mk) * 4 + r4) * 64 + lane];
#pragma unroll
                for (int qq = 1; qq < NQ; ++qq) {
                    const float4 v = Sp4[(((hg + 2 * qq) * MK + mk) * 4 + r4) * 64 + lane];
                    sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
                }
                // rows 32*mk + 8*r4 + 4*(lane/32) + 0..3
                const float4 km = km4[8 * mk + 2 * r4 + (lane >> 5)];
                t2[mk][4 * r4] = fmaf(sum.x, a.c2, km.x);
                t2[mk][4 * r4 + 1] = fmaf(sum.y, a.c2, km.y);
                t2[mk][4 * r4 + 2] = fmaf(sum.z, a.c2, km.z);
                t2[mk][4 * r4 + 3] = fmaf(sum.w, a.c2, km.w);
            }

        // ---------------- 3. online softmax (base 2) with a lazy reference:
        // probabilities are exp2(t - m_ref); m_ref moves (and O, l are
        // rescaled) only when some lane's tile max exceeds it by more than 8,
        // so p stays below 2^8 and the rescale is rare.  The final division
        // by l uses the same reference, so the result does not depend on it.
        float tmax = t2[0][0];
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, t2[mk][r]);
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
        uint32_t pk[MK][8];
        float psum = 0.0f;
        if (m_run == -__builtin_inff()) {
#pragma unroll
            for (int mk = 0; mk < MK; ++mk)
#pragma unroll
                for (int q = 0; q < 8; ++q) pk[mk][q] = 0u;
        } else {
#pragma unroll
            for (int mk = 0; mk < MK; ++mk)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    // v_exp_f32 directly: arguments are <= 8, and results too
                    // small for fp16 become 0 either way
                    const half2v ph = {static_cast<_Float16>(__builtin_amdgcn_exp2f(t2[mk][2 * q] - m_run)),
                                       static_cast<_Float16>(__builtin_amdgcn_exp2f(t2[mk][2 * q + 1] - m_run))};
                    psum = __builtin_amdgcn_fdot2(ph, half2v{1.0f16, 1.0f16}, psum, false);
                    pk[mk][q] = __builtin_bit_cast(uint32_t, ph);
                }
        }
        l_run += psum;

        // ---------------- 4. O^T += V^T P^T over this wave's channel slice
#pragma unroll
        for (int ks = 0; ks < 2 * MK; ++ks) {
            const uint32_t* pp = &pk[ks >> 1][4 * (ks & 1)];
            const half8 pf = __builtin_bit_cast(half8, make_uint4(pp[0], pp[1], pp[2], pp[3]));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                // A = V^T[32 d][16 k-slots]; k-slot 8h + i holds key
                // 16ks + 4h + (i % 4) + 8(i / 4) (h = lane / 32), the order of
                // the P fragment.  In each 16-lane group g the transposed read
                // hands lane 16g + i' the elements i' % 4 of lanes 4e + i'/4
                // (e = 0..3), so lane 16g + j reads 4 channels of key
                // 16ks + 4(g/2) + j/4 (then 8 keys further for i >= 4).
                const int g = lane >> 4, j = lane & 15;
                const int key = 16 * ks + 4 * (g >> 1) + (j >> 2);
                const int d = dq * DQ + 32 * mt + 16 * (g & 1) + 4 * (j & 3);
                const short4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (short4v __attribute__((address_space(3)))*)(&Kt[key * KROW + d]));
                const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (short4v __attribute__((address_space(3)))*)(&Kt[(key + 8) * KROW + d]));
                const short8v vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                const half8 vf = __builtin_bit_cast(half8, vv);
                o_acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o_acc[mt], 0, 0, 0);
            }
        }
    };

    // ---- main tiles (every slot a main-KV slot): branch-free gathers
    // prefetched one tile ahead into registers no other path writes
    const int t_main_end = (a.k / KT) < t_end ? (a.k / KT) : t_end;
    uint32_t pm_cw[KPT], pm_sc[KPT];
    int pm_ok[KPT];
    auto load_main = [&](int tile) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int slot = tile * KT + key_of_i(i);
            const int32_t row = __builtin_amdgcn_readfirstlane(idx_s[slot - win0 * KT]);
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
                dequant8_hw(pm_cw[i], pm_sc[i], h[i]);
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
                    dequant8_hw(raw_cw[i], raw_sc[i], h[i]);
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
        _Float16* po = a.ws_o + pidx * (64 * D);
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                po[((wv * MT + mt) * 16 + r) * 64 + lane] = static_cast<_Float16>(o_acc[mt][r] * inv);
        if (dq == 0 && lane < 32) {
            a.ws_m[pidx * 64 + head_local] = m_run;
            a.ws_l[pidx * 64 + head_local] = l_tot;
        }
    }
}

// ---------------------------------------------------------------------------
// D = 512: warp-specialised tiles of 64 keys.  Eight waves in two roles:
//   S-waves 0..3 (head group hg = w & 1, key block kb = w >> 1): S^T for 32
//     keys x 32 heads over all 512 channels (32 MFMAs, q in registers), the
//     online softmax of that block and its P fragments;
//   D-waves 4..7 (channel slice dw = w - 4): O^T[128 d][64 heads] += V^T P^T
//     with V^T read transposed from Kt.
// A D-wave also gathers and dequantises its own 128 channels of every tile:
// those are the only channels it reads in P.V, so it can overwrite the tile
// it has just consumed with the next one as soon as its own P.V of it is
// done, without waiting for any other wave.  One barrier per tile:
//   S-waves: S(i) on Kt[i & 1] and the block max; the tile max with the
//            partner key block (a two-wave handshake in LDS); softmax -> P(i)
//   D-waves: O += V(i - 1) P(i - 1) from Kt[(i - 1) & 1]; then tile i + 1
//            into that buffer; then the gathers of tile i + 2 into registers
// With ILV (splits of many tiles) the D-waves instead dequantise tile i + 1
// inside P.V: group g right after the k-step that read keys 16g .. 16g + 15,
// the same keys it overwrites in this wave's channels, so the VALU work
// interleaves with the wave's own MFMAs.
// P, the rescale factors and their flags alternate between two LDS copies.
// Each role runs its own copy of the tile loop (the same barriers), so the
// two roles' registers are allocated separately.  No S partial sums cross
// waves (each S-wave covers all channels).  The gathers are buffer loads
// whose row offset is a plain integer (rows beyond the cache read zeros);
// one load path per instantiation, since a branch between buffer and global
// loads makes the compiler wait for every gather where the paths join.
// Start-up: the first main tile's gathers go out first (index entries
// straight from global memory), then the unit's q is read once by all 512
// threads in 1 KiB runs and staged in the second Kt buffer, from which each
// S-wave takes its fragments.  A split's generic tiles (window rows, or a
// tile that mixes main and window rows) come first and are loaded directly.
template <bool BF16, bool USE_BUF, bool ILV>
__global__ __launch_bounds__(512) void attn_ws_kernel(AttnArgs a) {
    constexpr int D = 512, KT = 64, KROW = D + 8, SSTEPS = D / 16;
    __shared__ __attribute__((aligned(16))) _Float16 Kt[2][KT * KROW];
    __shared__ __attribute__((aligned(16))) uint4 Pb[2][2][4][64];   // [parity][head group][k-step][lane]
    __shared__ __attribute__((aligned(16))) float kmask[2][KT];
    __shared__ float Lm[2][2][32];                                 // tile max [hg][kb][head]
    __shared__ float alpha_s[2][64];
    __shared__ int grow_s[2][2];
    __shared__ int pair_it[2][2];                                  // [hg][kb]: iteration whose Lm is posted
    __shared__ float Lsum[2][2][32];
    __shared__ float Mfin[64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool s_role = wv < 4;
    const int hg = wv & 1, kb = (wv >> 1) & 1;
    const int dw = wv & 3;
    const int64_t u = blockIdx.x;
    const int split = blockIdx.y;
    const int hb = blockIdx.z;
    const int hbase = hb * 64;

    // ---- unit geometry
    const int32_t* idx = a.idx + u * a.k;
    const int64_t kvbase = u * a.kv_unit_stride;
    const uint8_t* swa_rows;
    int n_swa;
    const int64_t swa_row_bytes = static_cast<int64_t>(D) * (BF16 ? 2 : 4);
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

    const int t_begin = split * a.tiles_per_split;
    int t_end = t_begin + a.tiles_per_split;
    if (t_end > a.n_tiles) t_end = a.n_tiles;
    const int n_it = t_end > t_begin ? t_end - t_begin : 0;
    const int t_main_end = a.k / KT;        // tiles made only of main-KV slots
    // iteration order: generic tiles first, then main tiles t_begin, ...
    const int t_first_gen = t_begin > t_main_end ? t_begin : t_main_end;
    const int n_gen = t_end > t_first_gen ? t_end - t_first_gen : 0;
    auto tile_of = [&](int it) { return it < n_gen ? t_first_gen + it : t_begin + (it - n_gen); };
    auto is_main = [&](int it) { return it >= n_gen; };

    // ---- D-wave slices: lane l takes key l / 4 + 16 g (g = 0..3) of a tile
    // and channels 128 dw + 32 (l % 4) .. + 31 of it: one 16-byte code load
    // and one 2-byte scale load per key
    const int sp = lane & 3, skey = lane >> 2;
    uint4 pm_c[4];
    uint32_t pm_s[4];
    uint32_t pm_ok = 0;                               // bit g: this lane's key of group g is a real row
    int32_t nidx[4];                                  // index entries of the next main tile to gather
    const __amdgpu_buffer_rsrc_t rc_codes = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.codes + kvbase * (D / 2)), static_cast<short>(0),
        USE_BUF ? static_cast<int>(a.cap * (D / 2)) : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rc_scales = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.scales + kvbase * (D / 16)), static_cast<short>(0),
        USE_BUF ? static_cast<int>(a.cap * (D / 16)) : 0, 0x00020000);
    int nidx_tile = -1;                               // the tile nidx holds (wave-uniform)
    auto load_idx = [&](int tile) {
#pragma unroll
        for (int g = 0; g < 4; ++g) nidx[g] = idx[tile * KT + skey + 16 * g];
        nidx_tile = tile;
    };
    auto gather_slice = [&]() {
        pm_ok = 0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const bool ok = nidx[g] >= 0 && nidx[g] < a.cap;
            const int32_t rw = ok ? nidx[g] : 0;
            pm_ok |= ok ? (1u << g) : 0u;
            if constexpr (USE_BUF) {
                pm_c[g] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rc_codes, rw * (D / 2) + 64 * dw + 16 * sp, 0, 0));
                pm_s[g] = __builtin_amdgcn_raw_buffer_load_b16(rc_scales, rw * (D / 16) + 8 * dw + 2 * sp, 0, 0);
            } else {
                const int64_t rr = kvbase + rw;
                pm_c[g] = *reinterpret_cast<const uint4*>(a.codes + rr * (D / 2) + 64 * dw + 16 * sp);
                pm_s[g] = *reinterpret_cast<const uint16_t*>(a.scales + rr * (D / 16) + 8 * dw + 2 * sp);
            }
        }
    };
    // gather main tile `it_` into registers, then fetch the next main
    // tile's index entries so the following gather need not wait for them
    auto gather_main = [&](int it_) {
        if (nidx_tile != tile_of(it_)) load_idx(tile_of(it_));
        gather_slice();
        if (it_ + 1 < n_it && is_main(it_ + 1)) load_idx(tile_of(it_ + 1));
    };
    // rows are KROW = 520 halves (1,040 bytes) apart, so the 16 keys of one
    // store instruction start 4 banks apart and its 64 lanes spread evenly
    // over the banks in the plain piece order
    auto dequant_group = [&](int buf, int g) {
        {
            const int key = skey + 16 * g;
            _Float16* dst = &Kt[buf][key * KROW + 128 * dw + 32 * sp];
            const uint32_t sc = pm_s[g];
            uint32_t c0 = sc & 0x7fu, c1 = (sc >> 8) & 0x7fu;
            c0 = c0 < 0x7eu ? c0 : 0x7eu;
            c1 = c1 < 0x7eu ? c1 : 0x7eu;
            const half2v s0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0 | (c0 << 8), 1.0f, false);
            const half2v s1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1 | (c1 << 8), 1.0f, false);
            const uint32_t cw[4] = {pm_c[g].x, pm_c[g].y, pm_c[g].z, pm_c[g].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const half2v sv = e < 2 ? s0 : s1;
                const uint32_t h0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 0) * sv);
                const uint32_t h1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 1) * sv);
                const uint32_t h2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 2) * sv);
                const uint32_t h3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 3) * sv);
                *reinterpret_cast<uint4*>(dst + 8 * e) = make_uint4(h0, h1, h2, h3);
            }
            // an empty slot keeps the finite values of the clamped row; its
            // logit is -inf, so it enters P.V with weight exactly 0
            if (dw == 0 && sp == 0) kmask[buf][key] = ((pm_ok >> g) & 1u) ? 0.0f : -__builtin_inff();
        }
    };
    auto dequant_slice = [&](int buf) {
#pragma unroll
        for (int g = 0; g < 4; ++g) dequant_group(buf, g);
    };
    // group g dequantised into registers (stored later by store_group, once
    // this wave's P.V reads of the buffer are done)
    auto dequant_regs = [&](int g, uint4 (&h)[4]) {
        const uint32_t sc = pm_s[g];
        uint32_t c0 = sc & 0x7fu, c1 = (sc >> 8) & 0x7fu;
        c0 = c0 < 0x7eu ? c0 : 0x7eu;
        c1 = c1 < 0x7eu ? c1 : 0x7eu;
        const half2v s0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0 | (c0 << 8), 1.0f, false);
        const half2v s1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1 | (c1 << 8), 1.0f, false);
        const uint32_t cw[4] = {pm_c[g].x, pm_c[g].y, pm_c[g].z, pm_c[g].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const half2v sv = e < 2 ? s0 : s1;
            h[e] = make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 0) * sv),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 1) * sv),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 2) * sv),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[e], 1.0f, 3) * sv));
        }
    };
    auto store_group = [&](int buf, int g, const uint4 (&h)[4]) {
        const int key = skey + 16 * g;
        _Float16* dst = &Kt[buf][key * KROW + 128 * dw + 32 * sp];
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<uint4*>(dst + 8 * e) = h[e];
        if (dw == 0 && sp == 0) kmask[buf][key] = ((pm_ok >> g) & 1u) ? 0.0f : -__builtin_inff();
    };
    // this D-wave's slice of any tile (main rows, window rows, empty
    // slots), loaded and stored at once; index entries from global memory
    auto load_generic_slice = [&](int tile, int buf) {
#pragma unroll 1
        for (int g = 0; g < 4; ++g) {
            const int key = skey + 16 * g;
            const int slot = tile * KT + key;
            uint32_t h[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) h[i] = 0u;
            bool valid = false;
            if (slot < a.k) {
                const int32_t row = idx[slot];
                valid = row >= 0 && row < a.cap;
                const int64_t rr = kvbase + (valid ? row : 0);
                const uint4 c4 = *reinterpret_cast<const uint4*>(a.codes + rr * (D / 2) + 64 * dw + 16 * sp);
                const uint32_t sc = *reinterpret_cast<const uint16_t*>(a.scales + rr * (D / 16) + 8 * dw + 2 * sp);
                dequant32_hw(c4, sc, h);
            } else if (slot < n_slots && slot - a.k < n_swa) {
                valid = true;
                const uint8_t* rp = swa_rows + static_cast<int64_t>(slot - a.k) * swa_row_bytes;
                if (BF16) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint4 v = *reinterpret_cast<const uint4*>(rp + 2 * (128 * dw + 32 * sp + 8 * e));
                        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            h[4 * e + j] = pack_h2(__uint_as_float(in[j] << 16), __uint_as_float(in[j] & 0xffff0000u));
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float* fp = reinterpret_cast<const float*>(rp) + 128 * dw + 32 * sp + 8 * e;
                        const uint4 v0 = *reinterpret_cast<const uint4*>(fp);
                        const uint4 v1 = *reinterpret_cast<const uint4*>(fp + 4);
                        h[4 * e] = pack_h2(__uint_as_float(v0.x), __uint_as_float(v0.y));
                        h[4 * e + 1] = pack_h2(__uint_as_float(v0.z), __uint_as_float(v0.w));
                        h[4 * e + 2] = pack_h2(__uint_as_float(v1.x), __uint_as_float(v1.y));
                        h[4 * e + 3] = pack_h2(__uint_as_float(v1.z), __uint_as_float(v1.w));
                    }
                }
            }
            _Float16* dst = &Kt[buf][key * KROW + 128 * dw + 32 * sp];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<uint4*>(dst + 8 * e) = make_uint4(h[4 * e], h[4 * e + 1], h[4 * e + 2], h[4 * e + 3]);
            if (dw == 0 && sp == 0) kmask[buf][key] = valid ? 0.0f : -__builtin_inff();
        }
    };

    // ---- start-up: the first main tile's rows (index entries straight
    // from global memory), q staged in Kt[1] by all threads
    if (!s_role && n_it > 0 && is_main(0)) gather_main(0);
    // q[u][hbase .. hbase + 63][0 .. 511] read once by all threads in 1 KiB
    // runs (thread t: 16-byte pieces t, t + 512, ...), staged as fp16 rows
    // of Kt[1] (the second tile buffer is free until phase 2 of the first
    // tile)
    {
        constexpr int QCH = 64 * D / 8;                    // 16-byte (bf16) or 32-byte (fp32) pieces
        const int64_t qbase = (u * a.H + hbase) * static_cast<int64_t>(D);
        uint32_t qh[QCH / 512][4];
#pragma unroll
        for (int r = 0; r < QCH / 512; ++r) {
            const int c = tid + 512 * r;                   // piece: head c / 64, channels 8 (c % 64) ..
            if (BF16) {
                const uint4 v = *reinterpret_cast<const uint4*>(a.q + qbase + 8 * static_cast<int64_t>(c));
                qh[r][0] = v.x; qh[r][1] = v.y; qh[r][2] = v.z; qh[r][3] = v.w;
            } else {
                const float* q32 = reinterpret_cast<const float*>(a.q) + qbase + 8 * static_cast<int64_t>(c);
                const uint4 v0 = *reinterpret_cast<const uint4*>(q32);
                const uint4 v1 = *reinterpret_cast<const uint4*>(q32 + 4);
                qh[r][0] = pack_h2(__uint_as_float(v0.x), __uint_as_float(v0.y));
                qh[r][1] = pack_h2(__uint_as_float(v0.z), __uint_as_float(v0.w));
                qh[r][2] = pack_h2(__uint_as_float(v1.x), __uint_as_float(v1.y));
                qh[r][3] = pack_h2(__uint_as_float(v1.z), __uint_as_float(v1.w));
            }
        }
#pragma unroll
        for (int r = 0; r < QCH / 512; ++r) {
            const int c = tid + 512 * r;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = BF16 ? pack_h2(__uint_as_float(qh[r][e] << 16), __uint_as_float(qh[r][e] & 0xffff0000u))
                            : qh[r][e];
            *reinterpret_cast<uint4*>(&Kt[1][(c >> 6) * KROW + 8 * (c & 63)]) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    if (tid < 4) pair_it[tid >> 1][tid & 1] = -1;
    __syncthreads();                                  // q staged

    // ---- role registers: R holds the q fragments of an S-wave (32 k-steps
    // x 4 dwords) or the O^T accumulators of a D-wave (4 d tiles x 2 head
    // tiles); a wave keeps one role for the whole kernel, so the two share
    // the same 128 registers
    floatx16 R[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) R[i][r] = 0.0f;
    auto qfrag = [&](int st) {
        const int b = 4 * (st & 3);
        return __builtin_bit_cast(half8, make_float4(R[st >> 2][b], R[st >> 2][b + 1], R[st >> 2][b + 2],
                                                     R[st >> 2][b + 3]));
    };
    float m_run = -__builtin_inff(), l_run = 0.0f;
    if (s_role) {
        // head 32hg + lane % 32 of the block, channels 16st + 8(lane / 32) ..
        const _Float16* qrow = &Kt[1][(32 * hg + (lane & 31)) * KROW + 8 * (lane >> 5)];
#pragma unroll
        for (int st = 0; st < SSTEPS; ++st) {
            const uint4 v = *reinterpret_cast<const uint4*>(qrow + 16 * st);
            R[st >> 2][4 * (st & 3)] = __uint_as_float(v.x);
            R[st >> 2][4 * (st & 3) + 1] = __uint_as_float(v.y);
            R[st >> 2][4 * (st & 3) + 2] = __uint_as_float(v.z);
            R[st >> 2][4 * (st & 3) + 3] = __uint_as_float(v.w);
        }
    }
    if (!s_role && n_it > 0) {
        if (is_main(0)) dequant_slice(0);
        else load_generic_slice(tile_of(0), 0);
        if (n_it > 1 && is_main(1)) gather_main(1);
    }
    __syncthreads();                                  // first tile in Kt[0], q taken

    // O^T += V^T P^T for the tile in Kt[buf] with the P fragments in Pb.
    // With deq, group ks of the next tile (in registers) is dequantised and
    // stored over keys 16ks .. 16ks + 15 of this wave's channels right after
    // k-step ks has read them: the VALU work then runs beside this wave's
    // own MFMAs instead of after them.
    auto pv_tile = [&](int buf, bool deq) {  // buf: also the parity of its P, alpha and grow flags
        if (grow_s[buf][0] | grow_s[buf][1]) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const float al = grow_s[buf][nt] ? alpha_s[buf][32 * nt + (lane & 31)] : 1.0f;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) R[2 * mt + nt][r] *= al;
            }
        }
        const int g = lane >> 4, jj = lane & 15;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const half8 pf0 = __builtin_bit_cast(half8, Pb[buf][0][ks][lane]);
            const half8 pf1 = __builtin_bit_cast(half8, Pb[buf][1][ks][lane]);
            // A = V^T[32 d][16 k-slots]: k-slot 8h + i holds key
            // 16ks + 4h + (i % 4) + 8(i / 4), h = lane / 32 (the P order); the
            // transposed read hands lane 16g + i' the element i' % 4 of lanes
            // 4e + i'/4 of its 16-lane group, so lane 16g + jj reads 4
            // channels of key 16ks + 4(g/2) + jj/4, and 8 keys further on.
            const int key = 16 * ks + 4 * (g >> 1) + (jj >> 2);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int d = 128 * dw + 32 * mt + 16 * (g & 1) + 4 * (jj & 3);
                const short4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (short4v __attribute__((address_space(3)))*)(&Kt[buf][key * KROW + d]));
                const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (short4v __attribute__((address_space(3)))*)(&Kt[buf][(key + 8) * KROW + d]));
                const short8v vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                const half8 vf = __builtin_bit_cast(half8, vv);
                R[2 * mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf0, R[2 * mt], 0, 0, 0);
                R[2 * mt + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf1, R[2 * mt + 1], 0, 0, 0);
            }
            if (deq) dequant_group(buf, ks);
            __builtin_amdgcn_sched_barrier(0);    // one k-step's fragments in registers at a time
        }
    };

    // one loop per role, so each role's registers are allocated on their own
    // (the same number of barriers in both)
    if (s_role) {
        for (int it = 0; it < n_it; ++it) {
            const int buf = it & 1;
            float t2[16];
            // two independent accumulation chains (even / odd k-steps) keep
            // the matrix core busy across the dependent MFMA latency
            floatx16 s_acc, s_acc2;
#pragma unroll
            for (int r = 0; r < 16; ++r) { s_acc[r] = 0.0f; s_acc2[r] = 0.0f; }
#pragma unroll
            for (int st = 0; st < SSTEPS; st += 2) {
                const half8 kf0 = *reinterpret_cast<const half8*>(
                    &Kt[buf][(32 * kb + (lane & 31)) * KROW + 16 * st + 8 * (lane >> 5)]);
                const half8 kf1 = *reinterpret_cast<const half8*>(
                    &Kt[buf][(32 * kb + (lane & 31)) * KROW + 16 * (st + 1) + 8 * (lane >> 5)]);
                s_acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf0, qfrag(st), s_acc, 0, 0, 0);
                s_acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf1, qfrag(st + 1), s_acc2, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s_acc[r] += s_acc2[r];
            const float4* km4 = reinterpret_cast<const float4*>(kmask[buf]);
            float bmax = -__builtin_inff();
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                // rows 32kb + 8r4 + 4(lane/32) + 0..3
                const float4 km = km4[8 * kb + 2 * r4 + (lane >> 5)];
                t2[4 * r4] = fmaf(s_acc[4 * r4], a.c2, km.x);
                t2[4 * r4 + 1] = fmaf(s_acc[4 * r4 + 1], a.c2, km.y);
                t2[4 * r4 + 2] = fmaf(s_acc[4 * r4 + 2], a.c2, km.z);
                t2[4 * r4 + 3] = fmaf(s_acc[4 * r4 + 3], a.c2, km.w);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, t2[r]);
            bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
            if (lane < 32) Lm[hg][kb][lane] = bmax;
            // post this key half's maximum, then wait for the other half's
            if (lane == 0) __hip_atomic_store(&pair_it[hg][kb], it, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            while (__hip_atomic_load(&pair_it[hg][kb ^ 1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != it)
                __builtin_amdgcn_s_sleep(1);
            // tile max over both key blocks (same value in both S-waves of
            // the head group); the reference moves only when it is exceeded
            // by more than 8, so p < 2^8 and rescales are rare
            const float tmax = fmaxf(Lm[hg][0][lane & 31], Lm[hg][1][lane & 31]);
            const bool grow = tmax > m_run + 8.0f || (m_run == -__builtin_inff() && tmax != -__builtin_inff());
            const bool any = __ballot(grow) != 0;
            float al = 1.0f;
            if (any) {
                const float m_new = grow ? tmax : m_run;
                al = (m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
                if (m_new != m_run) l_run *= al;
                m_run = m_new;
            }
            if (kb == 0) {
                if (lane < 32) alpha_s[buf][32 * hg + lane] = al;
                if (lane == 0) grow_s[buf][hg] = any ? 1 : 0;
            }
            uint32_t pk[8];
            float psum = 0.0f;
            if (m_run == -__builtin_inff()) {
#pragma unroll
                for (int q = 0; q < 8; ++q) pk[q] = 0u;
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const half2v ph = {static_cast<_Float16>(__builtin_amdgcn_exp2f(t2[2 * q] - m_run)),
                                       static_cast<_Float16>(__builtin_amdgcn_exp2f(t2[2 * q + 1] - m_run))};
                    psum = __builtin_amdgcn_fdot2(ph, half2v{1.0f16, 1.0f16}, psum, false);
                    pk[q] = __builtin_bit_cast(uint32_t, ph);
                }
            }
            l_run += psum;
            Pb[buf][hg][2 * kb][lane] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            Pb[buf][hg][2 * kb + 1][lane] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
            __syncthreads();
        }
    } else {
        // the iterations whose next tile is a window (generic) tile first,
        // then those whose next tile is a main tile (from the registers the
        // gather of two iterations before filled)
        const int it_gen_end = n_gen < n_it ? n_gen : n_it;   // next tile generic for it + 1 < n_gen
        int it = 0;
        for (; it + 1 < it_gen_end; ++it) {
            const int buf = it & 1;
            if (it > 0) pv_tile(buf ^ 1, false);
            load_generic_slice(tile_of(it + 1), buf ^ 1);
            if (it + 2 < n_it && is_main(it + 2)) gather_main(it + 2);
            __syncthreads();
        }
        if constexpr (!ILV) {
            // the first two groups of the next tile are dequantised into
            // registers before P.V, beside the S-waves' products (the VALU
            // and the matrix cores of a SIMD then overlap), and stored after it
            for (; it < n_it; ++it) {
                const int buf = it & 1;
                const bool next = it + 1 < n_it;
                uint4 dq0[4], dq1[4];
                if (next) {
                    dequant_regs(0, dq0);
                    dequant_regs(1, dq1);
                }
                if (it > 0) pv_tile(buf ^ 1, false);
                if (next) {
                    store_group(buf ^ 1, 0, dq0);
                    store_group(buf ^ 1, 1, dq1);
                    dequant_group(buf ^ 1, 2);
                    dequant_group(buf ^ 1, 3);
                }
                if (it + 2 < n_it) gather_main(it + 2);
                __syncthreads();
            }
        } else {
            // the next tile is dequantised inside P.V, group by group (the
            // first iteration has no P.V, the last no next tile: both peeled)
            if (it == 0 && n_it > 1) {
                dequant_slice(1);
                if (n_it > 2) gather_main(2);
                __syncthreads();
                it = 1;
            }
            for (; it + 1 < n_it; ++it) {
                const int buf = it & 1;
                pv_tile(buf ^ 1, true);
                if (it + 2 < n_it) gather_main(it + 2);
                __syncthreads();
            }
            if (it < n_it) {
                if (it > 0) pv_tile((it & 1) ^ 1, false);
                __syncthreads();
            }
        }
        if (n_it > 0) pv_tile((n_it - 1) & 1, false);
    }


    // ---------------- epilogue
    if (s_role) {
        const float lw = l_run + __shfl_xor(l_run, 32);
        if (lane < 32) {
            Lsum[hg][kb][lane] = lw;
            if (kb == 0) Mfin[32 * hg + lane] = m_run;
        }
    }
    __syncthreads();
    if (s_role) return;
    float l_tot[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) l_tot[nt] = Lsum[nt][0][lane & 31] + Lsum[nt][1][lane & 31];
    if (a.splits == 1) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int head = hbase + 32 * nt + (lane & 31);
            if (head >= a.H) continue;
            const float inv = l_tot[nt] > 0.0f ? 1.0f / l_tot[nt] : 0.0f;
            float* orow = a.out + (u * a.H + head) * D;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = 128 * dw + 32 * mt + 8 * r4 + 4 * (lane >> 5);
                    const floatx16& o = R[2 * mt + nt];
                    *reinterpret_cast<float4*>(orow + d) =
                        make_float4(o[4 * r4] * inv, o[4 * r4 + 1] * inv, o[4 * r4 + 2] * inv, o[4 * r4 + 3] * inv);
                }
        }
    } else {
        // partial layout of combine_kernel<512, 4>: block (w' = 2dw + nt, mt)
        const int64_t pidx = (u * gridDim.z + hb) * a.splits + split;
        _Float16* po = a.ws_o + pidx * (64 * D);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float inv = l_tot[nt] > 0.0f ? 1.0f / l_tot[nt] : 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    po[(((2 * dw + nt) * 4 + mt) * 16 + r) * 64 + lane] = static_cast<_Float16>(R[2 * mt + nt][r] * inv);
        }
        if (dw == 0 && lane < 32) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                a.ws_m[pidx * 64 + 32 * nt + lane] = Mfin[32 * nt + lane];
                a.ws_l[pidx * 64 + 32 * nt + lane] = l_tot[nt];
            }
        }
    }
}

// Merge the key-split partials of one (unit, 64-head block).  A block of
// the partial layout is one (wave, row-tile) pair: 32 heads (head group hg =
// wave & 1) x 32 consecutive channels.  Workgroup (ub, hg, g) merges `bpw`
// consecutive blocks of head group hg, so the per-head split weights are
// formed once for all of them; with many units bpw = 4 cuts the number of
// workgroups (each pays a fixed chain of dependent loads and barriers) by 4.
// Reads are in the partials' own (coalesced) order; each result block is
// transposed through LDS so the output rows are written as 128-byte runs.
template <int D, int NQ>
__global__ __launch_bounds__(1024) void combine_kernel(const _Float16* __restrict__ ws_o,
                                                       const float* __restrict__ ws_m,
                                                       const float* __restrict__ ws_l, int splits,
                                                       int H, int hblocks, int bpw, float* __restrict__ out) {
    constexpr int DQ = D / NQ, MT = DQ / 32;
    __shared__ float tile[32][33];
    __shared__ float wgt[kCombineMaxSplits][32];   // m_s, then exp2(m_s - m*), per split and head
    __shared__ float lsum[kCombineMaxSplits][32];
    __shared__ float inv_den[32];
    const int64_t ub = blockIdx.x;                 // unit * hblocks + hb
    const int hg = blockIdx.y;
    const int t = threadIdx.x, r = t >> 6, ln = t & 63;
    const int hcol = ln & 31;
    const int dd = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
    constexpr int64_t PS = 64 * D;                 // partial stride
    const _Float16* pbase = ws_o + ub * splits * static_cast<int64_t>(64 * D);
    const int hb = static_cast<int>(ub % hblocks);
    const int64_t u = ub / hblocks;
    const int oh = t >> 5, od = t & 31;
    const int head = hb * 64 + 32 * hg + oh;
    // block j of head group hg: dqq = j / MT, mt = j % MT, wave 2 dqq + hg
    auto block_ptr = [&](int j) {
        const int wv = 2 * (j / MT) + hg, mt = j % MT;
        return pbase + ((wv * MT + mt) * 16 + r) * 64 + ln;
    };
    const int j0 = blockIdx.z * bpw;
    // Loads are issued before the weights are formed, so the two latencies
    // overlap: with 4 blocks of at most 4 splits (many units), all 16 of
    // them; otherwise the first block's first 16 splits.
    const bool all16 = bpw == 4 && splits <= 4;
    constexpr int kEarly = 16;
    // raw 16-bit loads, one per register and widened where used, so no wait
    // follows the loads
    uint32_t oe[kEarly];
    auto h2f = [](uint32_t x) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(x))); };
    if (all16) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const _Float16* po = block_ptr(j0 + jj);
#pragma unroll
            for (int s = 0; s < 4; ++s)          // (unconditional loads of a clamped split)
                oe[4 * jj + s] = *reinterpret_cast<const uint16_t*>(po + (s < splits ? s : splits - 1) * PS);
        }
    } else {
        const _Float16* po = block_ptr(j0);
#pragma unroll
        for (int i = 0; i < kEarly; ++i) oe[i] = *reinterpret_cast<const uint16_t*>(po + (i < splits ? i : splits - 1) * PS);
    }
    // per-head split weights, once per workgroup: thread t loads (split
    // t/32, head 32hg + t%32), then thread t < 32 reduces over the splits
    {
        const int h = t & 31;
        for (int s = t >> 5; s < splits; s += 32) {
            const int64_t p = (ub * splits + s) * 64 + 32 * hg + h;
            wgt[s][h] = ws_m[p];
            lsum[s][h] = ws_l[p];
        }
    }
    __syncthreads();
    // waves 0..3: lane l of wave w takes head 8w + l % 8 and splits l / 8,
    // l / 8 + 8, ...; the eight lanes of a head then meet by shuffles
    if (t < 256) {
        const int h = 8 * (t >> 6) + (t & 7), s0 = (t & 63) >> 3;
        float mstar = -__builtin_inff();
        for (int s = s0; s < splits; s += 8) mstar = fmaxf(mstar, wgt[s][h]);
        mstar = fmaxf(mstar, __shfl_xor(mstar, 8));
        mstar = fmaxf(mstar, __shfl_xor(mstar, 16));
        mstar = fmaxf(mstar, __shfl_xor(mstar, 32));
        float den = 0.0f;
        for (int s = s0; s < splits; s += 8) {
            const float ms = wgt[s][h];
            const float w = (ms == -__builtin_inff()) ? 0.0f : exp2f(ms - mstar);
            // a split's partial is its output divided by its row sum
            wgt[s][h] = w * lsum[s][h];
            den += w * lsum[s][h];
        }
        den += __shfl_xor(den, 8);
        den += __shfl_xor(den, 16);
        den += __shfl_xor(den, 32);
        if ((t & 63) < 8) inv_den[h] = den > 0.0f ? 1.0f / den : 0.0f;
    }
    __syncthreads();
    auto emit = [&](int j, float num, bool first) {
        if (!first) __syncthreads();               // the previous block's tile has been written out
        tile[hcol][dd] = num * inv_den[hcol];
        __syncthreads();
        const int dqq = j / MT, mt = j % MT;
        if (head < H) out[(u * H + head) * D + dqq * DQ + 32 * mt + od] = tile[oh][od];
    };
    if (all16) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float num = 0.0f;
#pragma unroll
            for (int s = 0; s < 4; ++s) num += s < splits ? wgt[s][hcol] * h2f(oe[4 * jj + s]) : 0.0f;
            emit(j0 + jj, num, jj == 0);
        }
        return;
    }
    for (int jj = 0; jj < bpw; ++jj) {
        const int j = j0 + jj;
        const _Float16* po = block_ptr(j);
        float num = 0.0f;
        int s = 0;
        if (jj == 0) {
#pragma unroll
            for (int i = 0; i < kEarly; ++i) num += i < splits ? wgt[i][hcol] * h2f(oe[i]) : 0.0f;
            s = kEarly;
        }
        for (; s + 8 <= splits; s += 8) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = static_cast<float>(po[(s + i) * PS]);
#pragma unroll
            for (int i = 0; i < 8; ++i) num += wgt[s + i][hcol] * o[i];
        }
        for (; s < splits; ++s) num += wgt[s][hcol] * static_cast<float>(po[s * PS]);
        emit(j, num, jj == 0);
    }
}

struct SplitPlan { int splits, tiles_per_split, n_tiles; };

// splits of at least this many tiles run attn_ws_kernel with the next tile's
// dequantisation inside P.V (measured: prefill, one split of 34 tiles, 3.5-4.5%
// faster; 9-tile splits unchanged; 3-tile splits 0.9% slower)
constexpr int kIlvTiles = 16;

// keys per tile of attn_kernel<D, ...> (8 per thread, 8 * waves)
constexpr int tile_keys(int D) { return D == 512 ? 64 : 32; }

SplitPlan plan(int64_t units, int H, int k, int W, int KT) {
    SplitPlan p;
    p.n_tiles = (k + W + KT - 1) / KT;
    const int64_t hblocks = (H + 63) / 64;
    const int64_t base = units * hblocks;
    int64_t want = (512 + base - 1) / base;          // aim for ~512 workgroups
    const int min_tiles = 128 / KT;                  // keep >= 128 keys per split
    int64_t max_splits = (p.n_tiles + min_tiles - 1) / min_tiles;
    if (want > max_splits) want = max_splits;
    if (want > kCombineMaxSplits) want = kCombineMaxSplits;
    if (want < 1) want = 1;
    p.tiles_per_split = static_cast<int>((p.n_tiles + want - 1) / want);
    if (p.tiles_per_split < 1) p.tiles_per_split = 1;
    p.splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
    if (p.splits < 1) p.splits = 1;
    return p;
}

// The warp-specialised kernel runs one 512-thread workgroup per CU (its LDS
// use), so its key splits are chosen by rounds of kCUs workgroups: the cost
// of a plan is (rounds) x (tiles per split + about 2 tiles of start-up and
// write-out) plus the combine's reading of the partials.  Fixed at the
// MI355X CU count, so the workspace size never depends on the device.
constexpr int kCUs = 256;
// D = 512 always takes the warp-specialised kernel (at 4, 8 and 12 units
// too: 22.6, 24.6 and 26.8 us against 24.8, 27.1 and 29.2 us for the split
// kernel, attention and combine together); D = 64 the split kernel.
constexpr bool use_ws(int D) { return D == 512; }

SplitPlan plan_ws(int64_t units, int H, int k, int W, int KT) {
    SplitPlan best;
    best.n_tiles = (k + W + KT - 1) / KT;
    const int64_t hblocks = (H + 63) / 64;
    const int min_tiles = 128 / KT;
    int max_splits = (best.n_tiles + min_tiles - 1) / min_tiles;
    if (max_splits > kCombineMaxSplits) max_splits = kCombineMaxSplits;
    if (max_splits < 1) max_splits = 1;
    double best_cost = 1e300;
    best.splits = 1;
    best.tiles_per_split = best.n_tiles > 0 ? best.n_tiles : 1;
    for (int s = 1; s <= max_splits; ++s) {
        const int tps = (best.n_tiles + s - 1) / s;
        if (tps < 1) break;
        const int se = (best.n_tiles + tps - 1) / tps;
        const int64_t wgs = units * hblocks * se;
        const int64_t rounds = (wgs + kCUs - 1) / kCUs;
        const double cost = static_cast<double>(rounds) * (tps + 2) +
                            (se > 1 ? 0.5 * static_cast<double>(wgs) / kCUs : 0.0);
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best.splits = se;
            best.tiles_per_split = tps;
        }
    }
    return best;
}

template <int D, int NQ, bool BF16>
hipError_t launch_d(const AttnLaunch& L, hipStream_t st) {
    const SplitPlan sp = use_ws(D) ? plan_ws(L.units, L.H, L.k, L.W, tile_keys(D))
                                    : plan(L.units, L.H, L.k, L.W, tile_keys(D));
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
    // [nparts][64][D] fp16 partials, then [nparts][64] row maxima and sums
    a.ws_o = reinterpret_cast<_Float16*>(L.ws);
    a.ws_m = L.ws ? reinterpret_cast<float*>(reinterpret_cast<char*>(L.ws) + nparts * 64 * D * sizeof(_Float16)) : nullptr;
    a.ws_l = L.ws ? a.ws_m + nparts * 64 : nullptr;
    if (L.units == 0) return hipSuccess;
    if constexpr (use_ws(D)) {
        const dim3 grid(static_cast<unsigned>(L.units), sp.splits, hblocks);
        // long splits (the tile loop dominates) take the next tile's
        // dequantisation inside P.V; short ones keep it around P.V
        const bool ilv = sp.tiles_per_split >= kIlvTiles;
        const bool buf = L.cap * (D / 2) <= 0x7fffffffLL;
        if (buf && ilv) attn_ws_kernel<BF16, true, true><<<grid, 512, 0, st>>>(a);
        else if (buf) attn_ws_kernel<BF16, true, false><<<grid, 512, 0, st>>>(a);
        else if (ilv) attn_ws_kernel<BF16, false, true><<<grid, 512, 0, st>>>(a);
        else attn_ws_kernel<BF16, false, false><<<grid, 512, 0, st>>>(a);
    }
    else
        attn_kernel<D, NQ, BF16><<<dim3(static_cast<unsigned>(L.units), sp.splits, hblocks), 128 * NQ, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sp.splits == 1) return e;
    // blocks of one head group: NQ channel slices x (D / NQ / 32) row tiles
    constexpr int kGroupBlocks = NQ * (D / NQ / 32);
    const int64_t n_blocks = L.units * hblocks * 2 * kGroupBlocks;
    const int bpw = (n_blocks >= 4 * kCUs && kGroupBlocks % 4 == 0) ? 4 : 1;
    combine_kernel<D, NQ><<<dim3(static_cast<unsigned>(L.units * hblocks), 2, kGroupBlocks / bpw), 1024, 0, st>>>(
        a.ws_o, a.ws_m, a.ws_l, sp.splits, L.H, hblocks, bpw, L.out);
    return hipGetLastError();
}

}  // namespace

bool attn_shape_supported(int H, int D) {
    return (D == 512 && H > 0 && H % 64 == 0) || (D == 64 && H > 0 && H <= 64);
}

size_t attn_workspace_bytes(int64_t units, int H, int D, int k, int W) {
    const SplitPlan sp = use_ws(D) ? plan_ws(units, H, k, W, tile_keys(D)) : plan(units, H, k, W, tile_keys(D));
    if (sp.splits == 1) return 0;
    const int64_t hblocks = (H + 63) / 64;
    const int64_t nparts = units * hblocks * sp.splits;
    return static_cast<size_t>(nparts) * (64 * static_cast<size_t>(D) * sizeof(_Float16) + 128 * sizeof(float));
}

hipError_t launch_attn(const AttnLaunch& L, hipStream_t st) {
    if (L.q_bf16 != L.swa_bf16) return hipErrorInvalidValue;
    if (L.D == 512) return L.q_bf16 ? launch_d<512, 4, true>(L, st) : launch_d<512, 4, false>(L, st);
    if (L.D == 64) return L.q_bf16 ? launch_d<64, 2, true>(L, st) : launch_d<64, 2, false>(L, st);
    return hipErrorInvalidValue;
}

}  // namespace csa2
