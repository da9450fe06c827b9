// MXFP4 quantisation of one 16-channel block ("DeepSeek-V4.1-Flash KV Cache
// Compression" notes, section 4; summary page, Methodology item 5): one E4M3
// (OCP FN) scale byte and 16 E2M1 nibbles, no second-level scale.
// scale = E4M3 nearest to amax/6 (ties to even, saturating at 448); element =
// E2M1 nearest to |x|/scale (ties to even, saturating at 6).  Every decision
// is an exact float32 comparison against a threshold that float32 holds
// exactly, so the bytes are reproducible on any device.
//
// Device helpers shared by the cache writers (the plain write kernel and the
// decode scan that writes the token's entry in the same launch).  Included
// inside namespace csa2 { namespace { ... } } of each translation unit.
#pragma once

// Value of a non-negative finite E4M3 code (0..126), exact in float32.
__device__ __forceinline__ float e4m3_nonneg(int c) {
    return (c < 8) ? static_cast<float>(c) * 0x1p-9f
                   : __uint_as_float((static_cast<uint32_t>(c) << 20) + (120u << 23));
}

// Nearest E4M3 code to amax/6, ties to even, saturating at 126 (448).
// Binary search for the largest code c with 6*v(c) <= amax (6*v(c) is exact),
// then the tie/round decision against 3*(v(c) + v(c+1)) (also exact).
__device__ __forceinline__ int scale_code(float amax) {
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (6.0f * e4m3_nonneg(mid) <= amax) lo = mid; else hi = mid - 1;
    }
    if (lo == 126) return 126;
    float t = 3.0f * (e4m3_nonneg(lo) + e4m3_nonneg(lo + 1));
    if (amax > t) return lo + 1;
    if (amax == t) return (lo & 1) ? lo + 1 : lo;
    return lo;
}

// E2M1 magnitude code (0..7) nearest to a/s: count the midpoints a exceeds,
// and at an exact midpoint pick the even code (midpoints 0.75, 1.75, 3.5
// round up to codes 2, 4, 6; 0.25, 1.25, 2.5, 5 round down to 0, 2, 4, 6).
__device__ __forceinline__ uint32_t mag_code(float a, float s) {
    const float t0 = s * 0.25f, t1 = s * 0.75f, t2 = s * 1.25f, t3 = s * 1.75f;
    const float t4 = s * 2.5f, t5 = s * 3.5f, t6 = s * 5.0f;
    uint32_t c = (a > t0) + (a > t1) + (a > t2) + (a > t3) + (a > t4) + (a > t5) + (a > t6);
    c += (a == t1) + (a == t3) + (a == t5);
    return c;
}

// The 16 channels of block `blk` of input row `row`, widened to float32.
template <bool BF16>
__device__ __forceinline__ void load_block(const void* __restrict__ x, int64_t row, int blk, int D, float (&v)[16]) {
    if (BF16) {
        const uint4* p = reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(x) + row * D + blk * 16);
        uint4 a = p[0], b = p[1];
        uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(
            static_cast<const float*>(x) + row * D + blk * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 f = p[i];
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
    }
}

// Quantise one 16-channel block v into flat cache row `dst`: scale byte,
// then eight code bytes (channel 2j in the low nibble).
__device__ __forceinline__ void quantise_block(const float (&v)[16], int blk, int D, int64_t dst,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int nblk = D / 16;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int sc = scale_code(amax);
    uint32_t lo = 0, hi = 0;
    if (sc != 0) {
        const float s = e4m3_nonneg(sc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t c = mag_code(fabsf(v[i]), s);
            if (v[i] < 0.0f && c != 0) c |= 8u;
            if (i < 8) lo |= c << (4 * i); else hi |= c << (4 * (i - 8));
        }
    }
    uint2* cp = reinterpret_cast<uint2*>(codes + dst * (D / 2) + blk * 8);
    *cp = make_uint2(lo, hi);
    scales[dst * nblk + blk] = static_cast<uint8_t>(sc);
}

