// W3G128 fused dequantize-and-multiply kernels for gfx950 (CDNA4), with the
// C ABI declared in include/qw3.h.
//
// Format (GSQ model card "Llama-3.1-70B-Instruct-3Bit-GSQ", "Storage layout"):
// a row of K weights is a little-endian bitstream of 3K bits packed into 3K/32
// int32 words, code k in stream bits [3k, 3k+3); one bf16 scale per 128
// weights; weight = scale * (code - 4).  A group of 128 codes is exactly 12
// words (48 bytes, three 16-byte loads) and a 32-code block is 3 words, so
// every group and block starts on a word boundary.
//
// Decode.  Two codes are turned into an exact fp16 pair with two VALU ops:
//   v = (window & mask) | 0x64006400   puts code a at mantissa bits [p,p+3) of
//                                      the low half and code b at [p',p'+3) of
//                                      the high half of two fp16 values 1024+..
//   q = fma(v, (2^-p, 2^-p'), -(1024*2^-p + 4, 1024*2^-p' + 4))
// which yields (a - 4, b - 4) exactly.  `window` is a 32-bit funnel shift of
// the 96-bit block.  The 16 pairs of a block come from 7 windows, three of
// which are the raw words, so a block of 32 codes costs 4 shifts + 16 and-or +
// 16 packed fma.  Which two codes share an fp16 pair does not matter for a dot
// product as long as the activations are paired the same way, so activations
// are converted once into the same pairing (kPairLo / kPairHi below).
//
// Activations.  x is bf16; the products use fp16 operands, so each group of
// 128 activations is scaled by a power of two 2^-e that brings its largest
// magnitude into [2^14, 2^15) and is then rounded to fp16.  bf16 has 8
// significant bits and fp16 11, so this is exact for every element within
// 2^31 of the group's largest; 2^e is multiplied back in fp32 together with
// the weight scale.  Every product q * x' is then exact and only the fp32
// accumulation rounds.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "qw3.h"

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;         // weights per scale
constexpr int kWordsPerGroup = 12;  // 128 * 3 / 32

// ----------------------------------------------------------- decode table --
// Code pairs of one 32-code block, in the order decode_block() emits them.
// Pair i holds code kPairLo[i] in its low fp16 half and kPairHi[i] in its high.
__device__ constexpr int kPairLo[16] = {0, 1, 2, 3, 4, 5, 12, 13, 14, 15, 16, 22, 23, 24, 25, 26};
__device__ constexpr int kPairHi[16] = {7, 6, 9, 8, 10, 11, 18, 17, 19, 21, 20, 28, 27, 29, 31, 30};

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
    h2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Exact (a-4, b-4) from a window holding code a at bits [P, P+3) and code b at
// bits [16+PP, 16+PP+3).
template <int P, int PP>
__device__ __forceinline__ h2_t q_pair(uint32_t win) {
    constexpr uint32_t kMask = (7u << P) | (7u << (16 + PP));
    constexpr h2_t kMul = {(_Float16)(1.0f / (1 << P)), (_Float16)(1.0f / (1 << PP))};
    constexpr h2_t kAdd = {(_Float16)(-(1024.0f / (1 << P) + 4.0f)),
                           (_Float16)(-(1024.0f / (1 << PP) + 4.0f))};
    const uint32_t v = (win & kMask) | 0x64006400u;
    return __builtin_elementwise_fma(as_h2(v), kMul, kAdd);
}

// The 32 codes of words (w0, w1, w2) as 16 exact fp16 pairs, pair order above.
__device__ __forceinline__ void decode_block(uint32_t w0, uint32_t w1, uint32_t w2, h2_t (&q)[16]) {
    const uint32_t s4 = __builtin_amdgcn_alignbit(w1, w0, 4);    // stream bits [4, 36)
    const uint32_t s12 = __builtin_amdgcn_alignbit(w1, w0, 12);  // [12, 44)
    const uint32_t s41 = __builtin_amdgcn_alignbit(w2, w1, 9);   // [41, 73)
    const uint32_t s71 = w2 >> 7;                                // [71, 96)
    q[0] = q_pair<0, 5>(w0);
    q[1] = q_pair<3, 2>(w0);
    q[2] = q_pair<2, 7>(s4);
    q[3] = q_pair<5, 4>(s4);
    q[4] = q_pair<0, 2>(s12);
    q[5] = q_pair<3, 5>(s12);
    q[6] = q_pair<4, 6>(w1);
    q[7] = q_pair<7, 3>(w1);
    q[8] = q_pair<1, 0>(s41);
    q[9] = q_pair<4, 6>(s41);
    q[10] = q_pair<7, 3>(s41);
    q[11] = q_pair<2, 4>(w2);
    q[12] = q_pair<5, 1>(w2);
    q[13] = q_pair<1, 0>(s71);
    q[14] = q_pair<4, 6>(s71);
    q[15] = q_pair<7, 3>(s71);
}

// acc + sum over the block of q * x', x' given as 16 fp16 pairs in pair order.
__device__ __forceinline__ float dot_block(uint32_t w0, uint32_t w1, uint32_t w2,
                                           const uint32_t *xp, float acc) {
    h2_t q[16];
    decode_block(w0, w1, w2, q);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = __builtin_amdgcn_fdot2(q[i], as_h2(xp[i]), acc, false);
    return acc;
}

// ---------------------------------------------------------------- DPP ------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Sum over aligned segments of T lanes (T a power of two <= 64).  The total
// lands in the last lane of each segment (and, for T <= 16, in all of them).
template <int T>
__device__ __forceinline__ float segment_sum(float v) {
    if constexpr (T >= 2) v += dpp_f32<kDppQuadXor1>(v);
    if constexpr (T >= 4) v += dpp_f32<kDppQuadXor2>(v);
    if constexpr (T >= 8) v += dpp_f32<kDppRowHalfMirror>(v);
    if constexpr (T >= 16) v += dpp_f32<kDppRowMirror>(v);
    if constexpr (T >= 32) v += dpp_f32<kDppRowBcast15, 0xA>(v);
    if constexpr (T >= 64) v += dpp_f32<kDppRowBcast31, 0xC>(v);
    return v;
}

// ------------------------------------------------- activation conversion --
// Largest |x| of 32 bf16 values (as a bf16 magnitude bit pattern).
__device__ __forceinline__ uint32_t absmax32(const uint4 (&xb)[4]) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d[4] = {xb[i].x, xb[i].y, xb[i].z, xb[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m = max(m, d[j] & 0x7FFFu);
            m = max(m, (d[j] >> 16) & 0x7FFFu);
        }
    }
    return m;
}

// Exponent e with (largest magnitude) * 2^-e in [2^14, 2^15).
__device__ __forceinline__ int group_exponent(uint32_t absmax_bits) {
    return __builtin_amdgcn_frexp_expf(bf16_to_f32(absmax_bits)) - 15;
}

// 32 bf16 values -> x * 2^-e as fp16, arranged as the 16 pairs of a block.
__device__ __forceinline__ void convert_block(const uint4 (&xb)[4], int e, uint32_t (&out)[16]) {
    _Float16 h[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d[4] = {xb[i].x, xb[i].y, xb[i].z, xb[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[8 * i + 2 * j] = (_Float16)ldexpf(bf16_to_f32(d[j] & 0xFFFFu), -e);
            h[8 * i + 2 * j + 1] = (_Float16)ldexpf(bf16_to_f32(d[j] >> 16), -e);
        }
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) out[p] = pack_h2(h[kPairLo[p]], h[kPairHi[p]]);
}

__device__ __forceinline__ void load_x32(const uint16_t *src, uint4 (&xb)[4]) {
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[i] = s[i];
}

// ------------------------------------------------------------- qpack -------
// One thread per (row, group): 128 codes in, 12 words out.
__global__ __launch_bounds__(256) void qpack_kernel(const uint8_t *__restrict__ codes,
                                                    uint32_t *__restrict__ packed, int64_t units) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(codes + u * kGroup);
    uint32_t words[kWordsPerGroup];
    uint64_t acc = 0;
    int nbits = 0, nw = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 v = src[i];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t c = (d[j >> 2] >> (8 * (j & 3))) & 7u;
            acc |= (uint64_t)c << nbits;
            nbits += 3;
            if (nbits >= 32) {
                words[nw++] = (uint32_t)acc;
                acc >>= 32;
                nbits -= 32;
            }
        }
    }
    uint4 *dst = reinterpret_cast<uint4 *>(packed + u * kWordsPerGroup);
    dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
    dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
    dst[2] = make_uint4(words[8], words[9], words[10], words[11]);
}

// ----------------------------------------------------------- qdequant -----
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One thread per (row, group): 12 words + 1 scale in, 128 bf16 out.
__global__ __launch_bounds__(256) void qdequant_kernel(const uint32_t *__restrict__ packed,
                                                       const uint16_t *__restrict__ scales,
                                                       uint16_t *__restrict__ w_out, int64_t units) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(packed + u * kWordsPerGroup);
    const uint4 a = src[0], b = src[1], c = src[2];
    const uint32_t w[kWordsPerGroup] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c.x, c.y, c.z, c.w};
    const float s = bf16_to_f32(scales[u]);
    uint4 *dst = reinterpret_cast<uint4 *>(w_out + u * kGroup);
#pragma unroll
    for (int o = 0; o < 16; ++o) {  // 8 outputs per 16-byte store
        uint32_t h[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int k = 8 * o + t;
            const int bit = 3 * k;
            const uint64_t pair = (bit >> 5) + 1 < kWordsPerGroup
                                      ? ((uint64_t)w[(bit >> 5) + 1] << 32) | w[bit >> 5]
                                      : (uint64_t)w[bit >> 5];
            const int c3 = (int)((pair >> (bit & 31)) & 7u);
            h[t] = f32_to_bf16_rne((float)(c3 - 4) * s);
        }
        dst[o] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                            h[6] | (h[7] << 16));
    }
}

// ------------------------------------------------------------ qgemv -------
// Batch-1 fused GEMV.  A team of T lanes owns one output row at a time; lane
// g of the team owns weight group g (128 weights = 12 words = 48 contiguous
// bytes), so a team's three 16-byte loads per lane cover the row contiguously.
// The lane's 128 activations stay in 64 VGPRs as fp16 pairs for the whole
// kernel ("x-stationary").  WG = T * R threads process R rows per iteration
// in a grid-stride loop, with the next row's loads issued before the current
// row is decoded.  The team's partial sums are reduced in a fixed order with
// DPP (T <= 64) or DPP + LDS (T > 64), so results are run-to-run identical.
template <int T>
struct GemvCfg {
    static constexpr int R = T >= 512 ? 1 : 512 / T;  // rows per iteration
    static constexpr int WGS = T * R;                  // threads per workgroup
    static constexpr int WAVES_PER_TEAM = T > 64 ? T / 64 : 1;
};

template <int T, bool kLdsX>
__global__ __launch_bounds__(GemvCfg<T>::WGS) void qgemv_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ packed,
    const uint16_t *__restrict__ scales, float *__restrict__ y, int64_t N, int G) {
    using Cfg = GemvCfg<T>;
    constexpr int R = Cfg::R;
    extern __shared__ uint32_t smem[];

    const int tid = threadIdx.x;
    const int gl = tid % T;  // weight group owned by this lane
    const int team = tid / T;
    const bool lane_on = gl < G;
    const int64_t W = (int64_t)G * kWordsPerGroup;
    const int64_t stride = (int64_t)gridDim.x * R;
    int64_t row = (int64_t)blockIdx.x * R + team;

    auto load_row = [&](int64_t r, uint4 &a0, uint4 &a1, uint4 &a2, uint32_t &s) {
        if (lane_on && r < N) {
            const uint4 *p = reinterpret_cast<const uint4 *>(packed + r * W + gl * kWordsPerGroup);
            a0 = p[0];
            a1 = p[1];
            a2 = p[2];
            s = scales[r * G + gl];
        } else {
            a0 = a1 = a2 = make_uint4(0, 0, 0, 0);
            s = 0;
        }
    };

    // First row in flight while the activations are converted.
    uint4 a0, a1, a2;
    uint32_t sa;
    load_row(row, a0, a1, a2, sa);

    uint32_t xp[64];
    int e = 0;
    if constexpr (kLdsX) {
        // The workgroup converts x once into LDS: 4 lanes (a quad) per group,
        // one 32-value block each, then every lane copies its group's pairs.
        uint32_t *xs = smem;                                        // [G][64] pairs
        int *xe = reinterpret_cast<int *>(smem + (size_t)G * 64);  // [G]
        for (int idx = tid; idx < 4 * G; idx += Cfg::WGS) {
            const int g = idx >> 2, blk = idx & 3;
            uint4 xb[4];
            load_x32(x + (size_t)g * kGroup + blk * 32, xb);
            uint32_t m = absmax32(xb);
            m = max(m, dpp_u32<kDppQuadXor1>(m));
            m = max(m, dpp_u32<kDppQuadXor2>(m));
            const int eg = group_exponent(m);
            uint32_t out[16];
            convert_block(xb, eg, out);
            uint4 *dst = reinterpret_cast<uint4 *>(xs + ((size_t)g * 4 + blk) * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
            if (blk == 0) xe[g] = eg;
        }
        __syncthreads();
        if (lane_on) {
            const uint4 *src = reinterpret_cast<const uint4 *>(xs + (size_t)gl * 64);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint4 v = src[i];
                xp[4 * i] = v.x;
                xp[4 * i + 1] = v.y;
                xp[4 * i + 2] = v.z;
                xp[4 * i + 3] = v.w;
            }
            e = xe[gl];
        } else {
#pragma unroll
            for (int i = 0; i < 64; ++i) xp[i] = 0;
        }
    } else {
        // Each lane converts its own group (two passes: max, then convert).
#pragma unroll
        for (int i = 0; i < 64; ++i) xp[i] = 0;
        if (lane_on) {
            const uint16_t *xg = x + (size_t)gl * kGroup;
            uint32_t m = 0;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                uint4 xb[4];
                load_x32(xg + blk * 32, xb);
                m = max(m, absmax32(xb));
            }
            e = group_exponent(m);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                uint4 xb[4];
                load_x32(xg + blk * 32, xb);
                uint32_t out[16];
                convert_block(xb, e, out);
#pragma unroll
                for (int p = 0; p < 16; ++p) xp[blk * 16 + p] = out[p];
            }
        }
    }

    float *red = reinterpret_cast<float *>(smem);  // T > 64 only; reused after xs
    int parity = 0;
    if constexpr (T > 64) __syncthreads();  // xs/xe fully consumed before reuse

    // WG-uniform trip count (the LDS reduction below needs every wave).
    for (int64_t base = (int64_t)blockIdx.x * R; base < N; base += stride) {
        uint4 b0, b1, b2;
        uint32_t sb;
        load_row(row + stride, b0, b1, b2, sb);

        float acc0 = 0.f, acc1 = 0.f;
        acc0 = dot_block(a0.x, a0.y, a0.z, xp + 0, acc0);
        acc1 = dot_block(a0.w, a1.x, a1.y, xp + 16, acc1);
        acc0 = dot_block(a1.z, a1.w, a2.x, xp + 32, acc0);
        acc1 = dot_block(a2.y, a2.z, a2.w, xp + 48, acc1);
        const float part = ldexpf(acc0 + acc1, e) * bf16_to_f32(sa);

        if constexpr (T <= 64) {
            const float tot = segment_sum<T>(part);
            if (gl == T - 1 && row < N) y[row] = tot;
        } else {
            const float wsum = segment_sum<64>(part);
            const int wave = tid >> 6;
            float *slot = red + parity * (Cfg::WGS / 64);
            if ((tid & 63) == 63) slot[wave] = wsum;
            __syncthreads();
            if (gl == 0 && row < N) {
                float tot = 0.f;
#pragma unroll
                for (int i = 0; i < Cfg::WAVES_PER_TEAM; ++i) tot += slot[team * Cfg::WAVES_PER_TEAM + i];
                y[row] = tot;
            }
            parity ^= 1;
        }
        a0 = b0;
        a1 = b1;
        a2 = b2;
        sa = sb;
        row += stride;
    }
}

// ----------------------------------------------- small-M matrix cores -----
// Activations for the matrix-core kernels: x[m][k] * 2^-e[g][m] as fp16 in the
// operand order of the 16x16x32 MFMA: for group g, token m and 32-code block
// j, 16 fp16 pairs in decode pair order (64 bytes).  Tokens m in [M, Mp) are
// zero.  One thread per (g, m, j); the four blocks of a group form a quad.
__global__ __launch_bounds__(256) void prep_x_kernel(const uint16_t *__restrict__ x,
                                                     uint4 *__restrict__ xq,
                                                     int16_t *__restrict__ xe, int M, int Mp,
                                                     int64_t K, int G) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t units = (int64_t)G * Mp * 4;
    if (idx >= units) return;  // units is a multiple of 4: whole quads exit together
    const int j = (int)(idx & 3);
    const int64_t gm = idx >> 2;
    const int m = (int)(gm % Mp);
    const int g = (int)(gm / Mp);
    uint32_t out[16];
    int eg = 0;
    if (m < M) {
        uint4 xb[4];
        load_x32(x + (int64_t)m * K + (int64_t)g * kGroup + j * 32, xb);
        uint32_t mx = absmax32(xb);
        mx = max(mx, dpp_u32<kDppQuadXor1>(mx));
        mx = max(mx, dpp_u32<kDppQuadXor2>(mx));
        eg = group_exponent(mx);
        convert_block(xb, eg, out);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) out[i] = 0;
    }
    uint4 *dst = xq + idx * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    if (j == 0) xe[(int64_t)g * Mp + m] = (int16_t)eg;
}

// Streaming small-M product on v_mfma_f32_16x16x32_f16.  One wave owns 16
// output rows and walks all groups.  Lane l works on row n0 + l%16 and block
// j = l/16 of each group: it decodes 32 codes (3 words) into the B operand
// (8 fp16 per MFMA, 4 MFMAs per group) while the A operand holds the same
// k-slots of x' for token l%16.  D[m][n] of one group is scaled by
// s[n][g] * 2^e[g][m] and added to the fp32 accumulator.  MT tiles of 16
// tokens share each decoded B operand, so the weights are read once.
template <int MT>
__global__ __launch_bounds__(256) void qgemm_mfma_kernel(const uint4 *__restrict__ xq,
                                                         const int16_t *__restrict__ xe,
                                                         const uint32_t *__restrict__ packed,
                                                         const uint16_t *__restrict__ scales,
                                                         float *__restrict__ y, int M, int Mp,
                                                         int64_t N, int G, int64_t y_ld) {
    const int lane = threadIdx.x & 63;
    const int64_t n0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16;
    if (n0 >= N) return;  // whole wave
    const int nl = lane & 15;
    const int jq = lane >> 4;
    const int64_t n = n0 + nl;
    const int64_t nrow = n < N ? n : N - 1;
    const int64_t W = (int64_t)G * kWordsPerGroup;
    const uint32_t *wrow = packed + nrow * W + jq * 3;
    const uint16_t *srow = scales + nrow * G;

    f4_t acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};

    for (int g = 0; g < G; ++g) {
        const uint32_t *wp = wrow + (int64_t)g * kWordsPerGroup;
        const uint32_t w0 = wp[0], w1 = wp[1], w2 = wp[2];
        const float s = bf16_to_f32(srow[g]);
        h2_t q[16];
        decode_block(w0, w1, w2, q);
        h8_t bop[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bop[t] = h8_t{q[4 * t].x, q[4 * t].y, q[4 * t + 1].x, q[4 * t + 1].y,
                          q[4 * t + 2].x, q[4 * t + 2].y, q[4 * t + 3].x, q[4 * t + 3].y};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            h8_t aop[4];
            if (mt * 16 + nl < M) {
                const uint4 *ap = xq + (((int64_t)g * Mp + mt * 16 + nl) * 4 + jq) * 4;
#pragma unroll
                for (int t = 0; t < 4; ++t) aop[t] = __builtin_bit_cast(h8_t, ap[t]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) aop[t] = h8_t{0, 0, 0, 0, 0, 0, 0, 0};
            }
            f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[t], bop[t], d, 0, 0, 0);
            const int16_t *ep = xe + (int64_t)g * Mp + mt * 16 + 4 * jq;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][r] += ldexpf(d[r], (int)ep[r]) * s;
        }
    }
    if (n >= N) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mt * 16 + 4 * jq + r;
            if (m < M) y[(int64_t)m * y_ld + n] = acc[mt][r];
        }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = 0.f;
}

// ------------------------------------------------------------ host side ---
thread_local char g_hip_error[256] = "no HIP error";

qw3_status hip_fail(hipError_t err) {
    snprintf(g_hip_error, sizeof g_hip_error, "%s (%d)", hipGetErrorString(err), (int)err);
    return QW3_ERR_HIP;
}

qw3_status check_launch() {
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? QW3_OK : hip_fail(err);
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

qw3_status check_shape(int64_t N, int64_t K) {
    if (N < 0 || K < 0 || K % kGroup != 0 || K > QW3_MAX_K || N > (int64_t(1) << 40)) return QW3_ERR_SHAPE;
    return QW3_OK;
}

std::mutex g_dev_mutex;
int g_cu_count[64];

qw3_status cu_count(int *out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err);
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (dev < 0 || dev >= 64) return hip_fail(hipErrorInvalidDevice);
    if (g_cu_count[dev] == 0) {
        int cus = 0;
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return hip_fail(err);
        g_cu_count[dev] = cus > 0 ? cus : 1;
    }
    *out = g_cu_count[dev];
    return QW3_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

qw3_status fill_zero(float *y, int64_t n, hipStream_t stream) {
    if (n == 0) return QW3_OK;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, y, n);
    return check_launch();
}

// LDS bytes of the x-stationary GEMV: fp16 pairs + exponents, or the
// cross-wave reduction slots, whichever is larger.
size_t gemv_lds_bytes(int G, int wgs, bool lds_x) {
    const size_t red = 2 * (size_t)(wgs / 64) * sizeof(float);
    const size_t xs = lds_x ? (size_t)G * 64 * 4 + (size_t)G * 4 : 0;
    return xs > red ? xs : red;
}

constexpr size_t kMaxLdsX = 64 * 1024;

template <int T>
qw3_status launch_gemv_t(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                         int64_t N, int G, hipStream_t stream) {
    using Cfg = GemvCfg<T>;
    int cus = 0;
    qw3_status st = cu_count(&cus);
    if (st != QW3_OK) return st;
    const bool lds_x = (size_t)G * 64 * 4 + (size_t)G * 4 <= kMaxLdsX;
    const size_t lds = gemv_lds_bytes(G, Cfg::WGS, lds_x);
    // Two resident workgroups per CU is what the register and LDS budget of
    // this kernel allows at up to 512 threads; more blocks only add tail.
    const int per_cu = Cfg::WGS <= 512 ? 2 : 1;
    int64_t blocks = ceil_div(N, Cfg::R);
    if (blocks > (int64_t)cus * per_cu) blocks = (int64_t)cus * per_cu;
    if (lds_x)
        hipLaunchKernelGGL((qgemv_kernel<T, true>), dim3((unsigned)blocks), dim3(Cfg::WGS), lds, stream, x,
                           packed, scales, y, N, G);
    else
        hipLaunchKernelGGL((qgemv_kernel<T, false>), dim3((unsigned)blocks), dim3(Cfg::WGS), lds, stream, x,
                           packed, scales, y, N, G);
    return check_launch();
}

qw3_status launch_gemv(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                       int64_t N, int64_t K, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    if (G <= 1) return launch_gemv_t<1>(x, packed, scales, y, N, G, stream);
    if (G <= 2) return launch_gemv_t<2>(x, packed, scales, y, N, G, stream);
    if (G <= 4) return launch_gemv_t<4>(x, packed, scales, y, N, G, stream);
    if (G <= 8) return launch_gemv_t<8>(x, packed, scales, y, N, G, stream);
    if (G <= 16) return launch_gemv_t<16>(x, packed, scales, y, N, G, stream);
    if (G <= 32) return launch_gemv_t<32>(x, packed, scales, y, N, G, stream);
    if (G <= 64) return launch_gemv_t<64>(x, packed, scales, y, N, G, stream);
    switch ((G + 63) / 64) {
        case 2: return launch_gemv_t<128>(x, packed, scales, y, N, G, stream);
        case 3: return launch_gemv_t<192>(x, packed, scales, y, N, G, stream);
        case 4: return launch_gemv_t<256>(x, packed, scales, y, N, G, stream);
        case 5: return launch_gemv_t<320>(x, packed, scales, y, N, G, stream);
        case 6: return launch_gemv_t<384>(x, packed, scales, y, N, G, stream);
        case 7: return launch_gemv_t<448>(x, packed, scales, y, N, G, stream);
        case 8: return launch_gemv_t<512>(x, packed, scales, y, N, G, stream);
        case 9: return launch_gemv_t<576>(x, packed, scales, y, N, G, stream);
        case 10: return launch_gemv_t<640>(x, packed, scales, y, N, G, stream);
        case 11: return launch_gemv_t<704>(x, packed, scales, y, N, G, stream);
        case 12: return launch_gemv_t<768>(x, packed, scales, y, N, G, stream);
        case 13: return launch_gemv_t<832>(x, packed, scales, y, N, G, stream);
        case 14: return launch_gemv_t<896>(x, packed, scales, y, N, G, stream);
        case 15: return launch_gemv_t<960>(x, packed, scales, y, N, G, stream);
        default: return launch_gemv_t<1024>(x, packed, scales, y, N, G, stream);
    }
}

// Small-M path: convert x once into scratch, then one streaming pass over W
// per chunk of up to 32 tokens.
qw3_status launch_gemm_small(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int mchunk = M > 16 ? 32 : 16;
    const size_t xq_bytes = (size_t)mchunk * (size_t)K * 2;
    const size_t xe_bytes = (size_t)G * mchunk * sizeof(int16_t);
    void *scratch = nullptr;
    hipError_t err = hipMallocAsync(&scratch, xq_bytes + xe_bytes, stream);
    if (err != hipSuccess) return hip_fail(err);
    uint4 *xq = reinterpret_cast<uint4 *>(scratch);
    int16_t *xe = reinterpret_cast<int16_t *>(static_cast<char *>(scratch) + xq_bytes);
    qw3_status st = QW3_OK;
    for (int64_t m0 = 0; m0 < M && st == QW3_OK; m0 += mchunk) {
        const int mc = (int)(M - m0 < mchunk ? M - m0 : mchunk);
        const int64_t units = (int64_t)G * mchunk * 4;
        hipLaunchKernelGGL(prep_x_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, stream,
                           x + m0 * K, xq, xe, mc, mchunk, K, G);
        st = check_launch();
        if (st != QW3_OK) break;
        const unsigned blocks = (unsigned)ceil_div(N, 64);
        if (mchunk == 16)
            hipLaunchKernelGGL(qgemm_mfma_kernel<1>, dim3(blocks), dim3(256), 0, stream, xq, xe, packed, scales,
                               y + m0 * N, mc, mchunk, N, G, N);
        else
            hipLaunchKernelGGL(qgemm_mfma_kernel<2>, dim3(blocks), dim3(256), 0, stream, xq, xe, packed, scales,
                               y + m0 * N, mc, mchunk, N, G, N);
        st = check_launch();
    }
    err = hipFreeAsync(scratch, stream);
    if (st == QW3_OK && err != hipSuccess) st = hip_fail(err);
    return st;
}

}  // namespace

// ------------------------------------------------------------------ C ABI --
extern "C" {

qw3_status qpack_uint3(const uint8_t *codes, int32_t *packed, int64_t N, int64_t K, void *hip_stream) {
    qw3_status st = check_shape(N, K);
    if (st != QW3_OK) return st;
    if (N == 0 || K == 0) return QW3_OK;
    if (!codes || !packed) return QW3_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(packed, 16)) return QW3_ERR_ALIGN;
    const int64_t units = N * (K / kGroup);
    hipLaunchKernelGGL(qpack_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0,
                       (hipStream_t)hip_stream, codes, reinterpret_cast<uint32_t *>(packed), units);
    return check_launch();
}

qw3_status qdequant_bf16(const int32_t *packed, const uint16_t *scales, uint16_t *w_out, int64_t N, int64_t K,
                         void *hip_stream) {
    qw3_status st = check_shape(N, K);
    if (st != QW3_OK) return st;
    if (N == 0 || K == 0) return QW3_OK;
    if (!packed || !scales || !w_out) return QW3_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(w_out, 16) || !aligned(scales, 2)) return QW3_ERR_ALIGN;
    const int64_t units = N * (K / kGroup);
    hipLaunchKernelGGL(qdequant_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0,
                       (hipStream_t)hip_stream, reinterpret_cast<const uint32_t *>(packed), scales, w_out, units);
    return check_launch();
}

qw3_status qgemv_w3g128(const uint16_t *x, const int32_t *packed, const uint16_t *scales, float *y, int64_t N,
                        int64_t K, void *hip_stream) {
    qw3_status st = check_shape(N, K);
    if (st != QW3_OK) return st;
    if (N == 0) return QW3_OK;
    if (!y) return QW3_ERR_NULL;
    if (!aligned(y, 4)) return QW3_ERR_ALIGN;
    if (K == 0) return fill_zero(y, N, (hipStream_t)hip_stream);
    if (!x || !packed || !scales) return QW3_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2)) return QW3_ERR_ALIGN;
    return launch_gemv(x, reinterpret_cast<const uint32_t *>(packed), scales, y, N, K, (hipStream_t)hip_stream);
}

qw3_status qgemm_w3g128_smallM(const uint16_t *x, const int32_t *packed, const uint16_t *scales, float *y,
                               int64_t M, int64_t N, int64_t K, void *hip_stream) {
    qw3_status st = check_shape(N, K);
    if (st != QW3_OK) return st;
    if (M < 0 || M > (int64_t(1) << 24)) return QW3_ERR_SHAPE;
    if (N == 0 || M == 0) return QW3_OK;
    if (!y) return QW3_ERR_NULL;
    if (!aligned(y, 4)) return QW3_ERR_ALIGN;
    if (K == 0) return fill_zero(y, M * N, (hipStream_t)hip_stream);
    if (!x || !packed || !scales) return QW3_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2)) return QW3_ERR_ALIGN;
    const uint32_t *pw = reinterpret_cast<const uint32_t *>(packed);
    if (M == 1) return launch_gemv(x, pw, scales, y, N, K, (hipStream_t)hip_stream);
    return launch_gemm_small(x, pw, scales, y, M, N, K, (hipStream_t)hip_stream);
}

const char *qstatus_str(qw3_status status) {
    switch (status) {
        case QW3_OK: return "ok";
        case QW3_ERR_NULL: return "a required pointer is NULL";
        case QW3_ERR_SHAPE: return "invalid shape (negative size, K % 128 != 0, or K > QW3_MAX_K)";
        case QW3_ERR_ALIGN: return "misaligned pointer (x/packed/codes/w_out need 16 bytes)";
        case QW3_ERR_HIP: return "HIP runtime error (see qw3_last_hip_error)";
        default: return "unknown status";
    }
}

const char *qw3_last_hip_error(void) { return g_hip_error; }

int qw3_abi_version(void) { return 1; }

}  // extern "C"
