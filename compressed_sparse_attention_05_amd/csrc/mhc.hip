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
//  * A workgroup owns 32 tokens and walks the channels in chunks of 128.
//    For the residual update, lane l of wave w owns token 4w + l/16 and the
//    8 channels 8(l%16) .. +7 of the chunk: each 16-byte load or store
//    instruction then covers four whole 256-byte row pieces (X streams, f,
//    X_next, u), so HBM sees full lines in both directions.
//  * The update runs in float32 on the VALU; the result is rounded to
//    bfloat16 once, stored, and reused unchanged for u, the sum of squares
//    and the projection.
//  * The projection z = x . phi (24 outputs, padded to 32) runs on
//    v_mfma_f32_32x32x16_bf16 with tokens as rows: the chunk's bfloat16
//    tile [32 tokens][4 x 128 features] is staged in LDS (rows padded by 16
//    bytes, so the operand reads spread over the banks) and each wave takes
//    4 of its 32 k-steps, reading phiT with the same feature mapping.
//  * Two chunks of global loads are kept in flight (a ring of two register
//    buffers) while a chunk is processed; the LDS tiles alternate, one
//    barrier per chunk.
//  * The epilogue sums the 8 waves' partial logits in LDS (reusing the tile)
//    and one thread per token finishes H.
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
constexpr int kCh = 128;                   // channels per chunk
constexpr int kFeat = kN * kCh;            // features per chunk (512)
constexpr int kRow = kFeat + 8;            // LDS tile row, bf16 elements (+16 bytes)
constexpr int kStepsPerWave = kFeat / 16 / kWaves;   // 4

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

union MhcLds {
    uint16_t tile[2][kTok * kRow];                // the chunk's X_next, bf16 (two chunks alternate)
    float zp[kWaves][kTok][33];                   // partial logits (epilogue)
};

__global__ __launch_bounds__(kThreads) void mhc_step_kernel(MhcArgs a) {
    __shared__ __attribute__((aligned(16))) MhcLds sh;
    __shared__ float sq[kTok];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kTok;
    const int d = a.d;

    // ---- update-stage ownership: token tv, channels 8e .. 8e+7 of a chunk
    const int tv = 4 * wv + (lane >> 4), e = lane & 15;
    const bool valid = tok0 + tv < a.T;
    const int64_t tk = valid ? tok0 + tv : a.T - 1;     // rows past the end reread the last token
    float Ai[kN], Bi[kN][kN], Ci[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        Ai[i] = a.A[tk * kN + i];
        Ci[i] = a.C[tk * kN + i];
#pragma unroll
        for (int j = 0; j < kN; ++j) Bi[i][j] = a.B[(tk * kN + i) * kN + j];
    }
    const uint16_t* xrow = a.X + tk * kN * static_cast<int64_t>(d) + 8 * e;
    const uint16_t* frow = a.f + tk * static_cast<int64_t>(d) + 8 * e;
    uint16_t* xnrow = a.Xn + tk * kN * static_cast<int64_t>(d) + 8 * e;
    uint16_t* urow = a.u + tk * static_cast<int64_t>(d) + 8 * e;

    // ---- projection-stage ownership: token row t = lane % 32, half h
    const int t = lane & 31, h = lane >> 5;
    const int o = t;
    const bool o_ok = o < kK;
    const uint16_t* phi_row = a.phiT + static_cast<int64_t>(o_ok ? o : 0) * (kN * static_cast<int64_t>(d));

    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    float ss = 0.0f;

    // two chunks of loads in flight: a ring of two register buffers
    auto load_chunk = [&](int c0, uint4 (&xv)[kN], uint4& fv, uint4 (&pv)[kStepsPerWave]) {
#pragma unroll
        for (int j = 0; j < kN; ++j) xv[j] = *reinterpret_cast<const uint4*>(xrow + static_cast<int64_t>(j) * d + c0);
        fv = *reinterpret_cast<const uint4*>(frow + c0);
#pragma unroll
        for (int s = 0; s < kStepsPerWave; ++s) {
            const int ft = (kStepsPerWave * wv + s) * 16 + 8 * h;     // feature in the chunk
            const int j = ft / kCh, cc = ft % kCh;
            pv[s] = o_ok ? *reinterpret_cast<const uint4*>(phi_row + static_cast<int64_t>(j) * d + c0 + cc)
                         : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    const int n_chunks = d / kCh;
    auto process = [&](int ch, uint4 (&xv)[kN], uint4& fv, uint4 (&pv)[kStepsPerWave]) {
        const int c0 = ch * kCh;
        uint4 xc[kN], fc = fv, pc[kStepsPerWave];
#pragma unroll
        for (int j = 0; j < kN; ++j) xc[j] = xv[j];
#pragma unroll
        for (int s = 0; s < kStepsPerWave; ++s) pc[s] = pv[s];
        if (ch + 2 < n_chunks) load_chunk(c0 + 2 * kCh, xv, fv, pv);

        // residual update of this lane's 4 x 8 values
        float fx[8], xx[kN][8];
        {
            const uint32_t fw[4] = {fc.x, fc.y, fc.z, fc.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) { fx[2 * q] = bf_lo(fw[q]); fx[2 * q + 1] = bf_hi(fw[q]); }
        }
#pragma unroll
        for (int j = 0; j < kN; ++j) {
            const uint32_t xw[4] = {xc[j].x, xc[j].y, xc[j].z, xc[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) { xx[j][2 * q] = bf_lo(xw[q]); xx[j][2 * q + 1] = bf_hi(xw[q]); }
        }
        float uo[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) uo[q] = 0.0f;
        uint4 outp[kN];
#pragma unroll
        for (int i = 0; i < kN; ++i) {
            uint32_t ow[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[2];
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int c = 2 * q + p;
                    float s = Ci[i] * fx[c];
#pragma unroll
                    for (int j = 0; j < kN; ++j) s = __builtin_fmaf(Bi[i][j], xx[j][c], s);
                    v[p] = s;
                }
                ow[q] = pack_bf16(v[0], v[1]);
                // the stored (rounded) values feed u, the squares and the projection
                const float r0 = bf_lo(ow[q]), r1 = bf_hi(ow[q]);
                ss = __builtin_fmaf(r0, r0, ss);
                ss = __builtin_fmaf(r1, r1, ss);
                uo[2 * q] = __builtin_fmaf(Ai[i], r0, uo[2 * q]);
                uo[2 * q + 1] = __builtin_fmaf(Ai[i], r1, uo[2 * q + 1]);
            }
            outp[i] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
            if (valid) *reinterpret_cast<uint4*>(xnrow + static_cast<int64_t>(i) * d + c0) = outp[i];
        }
        if (valid)
            *reinterpret_cast<uint4*>(urow + c0) = make_uint4(pack_bf16(uo[0], uo[1]), pack_bf16(uo[2], uo[3]),
                                                               pack_bf16(uo[4], uo[5]), pack_bf16(uo[6], uo[7]));

        // stage the chunk's tile, then this wave's 4 k-steps on the matrix cores.
        // Tiles alternate, so one barrier per chunk suffices: a wave writes
        // tile ch%2 only after the previous chunk's barrier, which every wave
        // reaches after its reads of that tile two chunks ago.
        uint16_t* tile = sh.tile[ch & 1];
#pragma unroll
        for (int i = 0; i < kN; ++i)
            *reinterpret_cast<uint4*>(&tile[tv * kRow + i * kCh + 8 * e]) = outp[i];
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kStepsPerWave; ++s) {
            const int ft = (kStepsPerWave * wv + s) * 16 + 8 * h;
            const uint4 xa = *reinterpret_cast<const uint4*>(&tile[t * kRow + ft]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa),
                                                          __builtin_bit_cast(bf16x8, pc[s]), acc, 0, 0, 0);
        }
    };
    uint4 xA[kN], fA, pA[kStepsPerWave], xB[kN], fB, pB[kStepsPerWave];
    load_chunk(0, xA, fA, pA);
    if (n_chunks > 1) load_chunk(kCh, xB, fB, pB);
    for (int ch = 0; ch < n_chunks; ch += 2) {
        process(ch, xA, fA, pA);
        if (ch + 1 < n_chunks) process(ch + 1, xB, fB, pB);
    }

    // ---- sums of squares: the 16 lanes of a token group
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if (e == 0) sq[tv] = ss;
    __syncthreads();                      // every tile read is done: reuse it for the logits
    // acc register r of lane l holds token row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int r = 0; r < 16; ++r) sh.zp[wv][8 * (r >> 2) + 4 * h + (r & 3)][o] = acc[r];
    __syncthreads();
    if (tid >= kTok) return;
    const int64_t tt = tok0 + tid;
    if (tt >= a.T) return;
    float z[kK];
#pragma unroll
    for (int k = 0; k < kK; ++k) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sh.zp[w][tid][k];
        z[k] = s;
    }
    const float inv_r = 1.0f / sqrtf(sq[tid] / static_cast<float>(kN * d) + 1e-6f);
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

bool mhc_shape_supported(int n, int d) { return n == kN && d > 0 && d % kCh == 0; }

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
