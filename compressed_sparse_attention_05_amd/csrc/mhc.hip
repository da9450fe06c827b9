// Single-pass mHC block step for gfx950.
//
// "DeepSeek-V4.1-Flash KV Cache Compression" notes, section 6, and the summary
// page's Methodology item 4, equation (6): the residual stream is n parallel
// streams X_l in R^{n x d}, and
//     X_{l+1} = B_l X_l + C_l F_l(A_{l-1} X_l),   (A_l, B_l, C_l) = H(X_l).
// Shifting the input-mixing coefficient by one block lets one read of the
// streams do everything: this pass takes X_l, the block output f_l and the
// coefficients (A_l, B_l, C_l) the previous pass predicted, and writes
//     X_{l+1} = B_l X_l + C_l f_l                 (stored as bfloat16)
//     u_{l+1} = A_l X_{l+1}                        (the next block's input)
//     (A_{l+1}, B_{l+1}, C_{l+1}) = H(X_{l+1})
// moving n*d + d values in and n*d + d out: the (2n+2)d bound.  H (not
// defined on the pages) is read as the manifold-constrained hyper-connection
// form: z = (x . phi) / rms(x) over the flattened stored streams x, then
// A = sigmoid(a_pre z_A + b_A), C = 2 sigmoid(a_post z_C + b_C),
// B = Sinkhorn(exp(a_res z_B + b_B)) (rows, then columns, `iters` times).
//
// Design: HBM-bound streaming (10*d*2 bytes per token at n = 4).
//  * A workgroup owns 32 tokens; its 8 waves split the channels (d/8 each).
//    Lane (t, h) of a wave owns token t = lane % 32 and, per iteration of 32
//    channels, the 16 channels c0 + 16h .. c0 + 16h + 15 of every stream:
//    two 16-byte loads per stream, contiguous across the lane pair.
//  * The residual mix runs in float32 on the VALU; the result is rounded to
//    bfloat16 once, stored, and reused unchanged as the matrix-core operand
//    of the projection, for u and for the sum of squares.
//  * The projection z = x . phi (24 outputs, padded to 32) runs on
//    v_mfma_f32_32x32x16_bf16 with tokens as rows.  Its reduction order over
//    features is free, so each k-step takes the 16 channels the lane pair
//    already holds (lane half h supplies 8 of them) and phiT is read with the
//    same channel mapping.
//  * The epilogue sums the 8 waves' partial products and squares in LDS and
//    one thread per token finishes H.
#include "csa2_internal.h"

namespace csa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kN = 4;                      // streams
constexpr int kK = 2 * kN + kN * kN;       // 24 coefficient logits
constexpr int kTok = 32;                   // tokens per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChan = 32;                  // channels per lane pair per iteration

struct MhcArgs {
    const uint16_t* X; const uint16_t* f;
    const float* A; const float* B; const float* C;
    const uint16_t* phiT; const float* bias;
    float a_pre, a_post, a_res;
    int64_t T; int d; int iters;
    uint16_t* Xn; uint16_t* u; float* An; float* Bn; float* Cn;
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two floats -> packed bfloat16 pair (nearest, ties to even), low half first
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__global__ __launch_bounds__(kThreads) void mhc_step_kernel(MhcArgs a) {
    __shared__ float zp[kWaves][kTok][33];       // partial logits, padded rows
    __shared__ float sq[kWaves][2][kTok];        // partial sums of squares

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = lane & 31, h = lane >> 5;
    const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kTok;
    const int64_t tok = tok0 + t;
    const bool valid = tok < a.T;
    const int64_t tk = valid ? tok : a.T - 1;    // rows past the end reread the last token
    const int d = a.d;

    // this token's incoming coefficients
    float Ai[kN], Bi[kN][kN], Ci[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        Ai[i] = a.A[tk * kN + i];
        Ci[i] = a.C[tk * kN + i];
#pragma unroll
        for (int j = 0; j < kN; ++j) Bi[i][j] = a.B[(tk * kN + i) * kN + j];
    }
    // projection column of this lane (B operand): output o = lane % 32
    const int o = t;
    const bool o_ok = o < kK;
    const uint16_t* phi_row = a.phiT + static_cast<int64_t>(o_ok ? o : 0) * (kN * static_cast<int64_t>(d));

    const uint16_t* xrow = a.X + tk * kN * static_cast<int64_t>(d);
    const uint16_t* frow = a.f + tk * static_cast<int64_t>(d);
    uint16_t* xnrow = a.Xn + tk * kN * static_cast<int64_t>(d);
    uint16_t* urow = a.u + tk * static_cast<int64_t>(d);

    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    float ss = 0.0f;

    const int per_wave = d / kWaves;
    const int cw0 = wv * per_wave;
    for (int it = 0; it < per_wave / kChan; ++it) {
        const int c = cw0 + it * kChan + 16 * h;        // this lane's 16 channels
        uint4 xv[kN][2], fv[2];
#pragma unroll
        for (int i = 0; i < kN; ++i)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                xv[i][q] = *reinterpret_cast<const uint4*>(xrow + static_cast<int64_t>(i) * d + c + 8 * q);
#pragma unroll
        for (int q = 0; q < 2; ++q) fv[q] = *reinterpret_cast<const uint4*>(frow + c + 8 * q);
        uint4 pv[kN][2];
#pragma unroll
        for (int i = 0; i < kN; ++i)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                pv[i][q] = o_ok ? *reinterpret_cast<const uint4*>(phi_row + static_cast<int64_t>(i) * d + c + 8 * q)
                                : make_uint4(0u, 0u, 0u, 0u);

        float uo[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) uo[e] = 0.0f;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float fx[8], xx[kN][8];
            const uint32_t fw[4] = {fv[q].x, fv[q].y, fv[q].z, fv[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) { fx[2 * e] = bf_lo(fw[e]); fx[2 * e + 1] = bf_hi(fw[e]); }
#pragma unroll
            for (int j = 0; j < kN; ++j) {
                const uint32_t xw[4] = {xv[j][q].x, xv[j][q].y, xv[j][q].z, xv[j][q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) { xx[j][2 * e] = bf_lo(xw[e]); xx[j][2 * e + 1] = bf_hi(xw[e]); }
            }
#pragma unroll
            for (int i = 0; i < kN; ++i) {
                uint32_t ow[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v[2];
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const int ch = 2 * e + p;
                        float s = Ci[i] * fx[ch];
#pragma unroll
                        for (int j = 0; j < kN; ++j) s = __builtin_fmaf(Bi[i][j], xx[j][ch], s);
                        v[p] = s;
                    }
                    ow[e] = pack_bf16(v[0], v[1]);
                    // the stored (rounded) values feed u, the squares and the projection
                    const float r0 = bf_lo(ow[e]), r1 = bf_hi(ow[e]);
                    ss = __builtin_fmaf(r0, r0, ss);
                    ss = __builtin_fmaf(r1, r1, ss);
                    uo[8 * q + 2 * e] = __builtin_fmaf(Ai[i], r0, uo[8 * q + 2 * e]);
                    uo[8 * q + 2 * e + 1] = __builtin_fmaf(Ai[i], r1, uo[8 * q + 2 * e + 1]);
                }
                const uint4 packed = make_uint4(ow[0], ow[1], ow[2], ow[3]);
                if (valid)
                    *reinterpret_cast<uint4*>(xnrow + static_cast<int64_t>(i) * d + c + 8 * q) = packed;
                // k-step (stream i, q): this lane half supplies channels c + 8q .. +7
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, packed),
                                                              __builtin_bit_cast(bf16x8, pv[i][q]), acc, 0, 0, 0);
            }
        }
        if (valid) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint4 uw = make_uint4(pack_bf16(uo[8 * q], uo[8 * q + 1]), pack_bf16(uo[8 * q + 2], uo[8 * q + 3]),
                                            pack_bf16(uo[8 * q + 4], uo[8 * q + 5]),
                                            pack_bf16(uo[8 * q + 6], uo[8 * q + 7]));
                *reinterpret_cast<uint4*>(urow + c + 8 * q) = uw;
            }
        }
    }

    // ---- partial logits and squares -> LDS.  acc register r of lane l holds
    // token row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int r = 0; r < 16; ++r) zp[wv][8 * (r >> 2) + 4 * h + (r & 3)][o] = acc[r];
    sq[wv][h][t] = ss;
    __syncthreads();
    if (tid >= kTok) return;
    const int64_t tt = tok0 + tid;
    if (tt >= a.T) return;
    float z[kK];
#pragma unroll
    for (int k = 0; k < kK; ++k) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += zp[w][tid][k];
        z[k] = s;
    }
    float s2 = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s2 += sq[w][0][tid] + sq[w][1][tid];
    const float inv_r = 1.0f / sqrtf(s2 / static_cast<float>(kN * d) + 1e-6f);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        const float za = a.a_pre * (z[i] * inv_r) + a.bias[i];
        const float zc = a.a_post * (z[kN + i] * inv_r) + a.bias[kN + i];
        a.An[tt * kN + i] = 1.0f / (1.0f + expf(-za));
        a.Cn[tt * kN + i] = 2.0f / (1.0f + expf(-zc));
    }
    float M[kN][kN];
#pragma unroll
    for (int i = 0; i < kN; ++i)
#pragma unroll
        for (int j = 0; j < kN; ++j)
            M[i][j] = expf(a.a_res * (z[2 * kN + i * kN + j] * inv_r) + a.bias[2 * kN + i * kN + j]);
    for (int s = 0; s < a.iters; ++s) {
#pragma unroll
        for (int i = 0; i < kN; ++i) {
            float rs = 0.0f;
#pragma unroll
            for (int j = 0; j < kN; ++j) rs += M[i][j];
            const float inv = 1.0f / rs;
#pragma unroll
            for (int j = 0; j < kN; ++j) M[i][j] *= inv;
        }
#pragma unroll
        for (int j = 0; j < kN; ++j) {
            float cs = 0.0f;
#pragma unroll
            for (int i = 0; i < kN; ++i) cs += M[i][j];
            const float inv = 1.0f / cs;
#pragma unroll
            for (int i = 0; i < kN; ++i) M[i][j] *= inv;
        }
    }
#pragma unroll
    for (int i = 0; i < kN; ++i)
#pragma unroll
        for (int j = 0; j < kN; ++j) a.Bn[(tt * kN + i) * kN + j] = M[i][j];
}

}  // namespace

bool mhc_shape_supported(int n, int d) { return n == kN && d > 0 && d % (kWaves * kChan) == 0; }

hipError_t launch_mhc_step(const MhcLaunch& p, hipStream_t st) {
    if (p.T == 0) return hipSuccess;
    MhcArgs a;
    a.X = p.X; a.f = p.f; a.A = p.A; a.B = p.B; a.C = p.C; a.phiT = p.phiT; a.bias = p.bias;
    a.a_pre = p.alpha_pre; a.a_post = p.alpha_post; a.a_res = p.alpha_res;
    a.T = p.T; a.d = p.d; a.iters = p.iters;
    a.Xn = p.Xn; a.u = p.u; a.An = p.An; a.Bn = p.Bn; a.Cn = p.Cn;
    const dim3 grid(static_cast<unsigned>((p.T + kTok - 1) / kTok));
    mhc_step_kernel<<<grid, kThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace csa2
