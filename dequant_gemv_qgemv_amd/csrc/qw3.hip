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
//                                      the high half: fp16 values 1024 + a*2^p
//                                      and 1024 + b*2^p'
//   q = v - (1024 + 4*2^p, 1024 + 4*2^p')   (one v_pk_add_f16)
// which yields ((a - 4) * 2^p, (b - 4) * 2^p') exactly; the 2^-p factors are
// folded into the activations.  `window` is a 32-bit funnel shift of the
// 96-bit block.  The 16 pairs of a block come from 7 windows, three of which
// are the raw words, so a block of 32 codes costs 4 shifts + 16 and-or + 16
// packed adds.  Which two codes share a pair does not matter for a dot product
// as long as the activations are paired the same way, so activations are
// converted once into the same pairing (kPairs below).
//
// Activations.  x is bf16; the products use fp16 operands, so each group of
// 128 activations is scaled by a power of two 2^-e that brings its largest
// magnitude into [2^14, 2^15), and each element by its slot's 2^-p, and is
// then rounded to fp16.  bf16 has 8 significant bits and fp16 11, so this is
// exact for every element within 2^24 of the group's largest; 2^e is
// multiplied back in fp32 together with the weight scale.  Every product is
// then exact and only the fp32 accumulation rounds.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>
#include <type_traits>

#include "qw3.h"

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;         // weights per scale
constexpr int kWordsPerGroup = 12;  // 128 * 3 / 32

// ----------------------------------------------------------- decode table --
// The 16 code pairs of a 32-code block: window index (0: w0, 1: bits [4,36),
// 2: [12,44), 3: w1, 4: [41,73), 5: w2, 6: [71,96)), low code, high code, and
// their bit offsets p, p' inside the window's two 16-bit halves.  Every code
// 0..31 appears once; lo at 3*lo - start(win) = p, hi at 3*hi - start - 16 = p'.
struct PairSpec {
    int win, lo, hi, p, pp;
};
constexpr PairSpec kPairs[16] = {
    {0, 0, 7, 0, 5},   {0, 1, 6, 3, 2},   {1, 2, 9, 2, 7},   {1, 3, 8, 5, 4},
    {2, 4, 10, 0, 2},  {2, 5, 11, 3, 5},  {3, 12, 18, 4, 6}, {3, 13, 17, 7, 3},
    {4, 14, 19, 1, 0}, {4, 15, 21, 4, 6}, {4, 16, 20, 7, 3}, {5, 22, 28, 2, 4},
    {5, 23, 27, 5, 1}, {6, 24, 29, 1, 0}, {6, 25, 31, 4, 6}, {6, 26, 30, 7, 3}};
constexpr int kWinStart[7] = {0, 4, 12, 32, 41, 64, 71};

constexpr bool pairs_cover_block() {
    int seen = 0;
    for (int i = 0; i < 16; ++i) {
        const PairSpec ps = kPairs[i];
        if (3 * ps.lo - kWinStart[ps.win] != ps.p || 3 * ps.hi - kWinStart[ps.win] - 16 != ps.pp) return false;
        if (ps.p < 0 || ps.p > 7 || ps.pp < 0 || ps.pp > 7) return false;
        seen |= (1 << ps.lo) | (1 << ps.hi);
    }
    return seen == -1;
}
static_assert(pairs_cover_block(), "decode table must cover codes 0..31 once at valid offsets");

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
    h2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Exact ((a-4)*2^P, (b-4)*2^PP) from a window holding code a at bits [P, P+3)
// and code b at bits [16+PP, 16+PP+3).
// `magic` is 0x64006400 held in a VGPR (see magic_vgpr()): with the mask in an
// SGPR the and/or pair then issues as a single v_and_or_b32 (gfx9 VOP3 cannot
// encode two literal constants).
template <int P, int PP>
__device__ __forceinline__ h2_t q_pair(uint32_t win, uint32_t magic) {
    constexpr uint32_t kMask = (7u << P) | (7u << (16 + PP));
    constexpr h2_t kSub = {(_Float16)(1024.0f + 4.0f * (1 << P)), (_Float16)(1024.0f + 4.0f * (1 << PP))};
    const uint32_t v = (win & kMask) | magic;
    return as_h2(v) - kSub;
}

// 0x64006400 (two fp16 1024.0) in a VGPR the compiler cannot constant-fold.
__device__ __forceinline__ uint32_t magic_vgpr() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

template <int I>
__device__ __forceinline__ h2_t q_pair_i(const uint32_t (&win)[7], uint32_t magic) {
    constexpr PairSpec ps = kPairs[I];
    return q_pair<ps.p, ps.pp>(win[ps.win], magic);
}

// The 32 codes of words (w0, w1, w2) as 16 exact fp16 pairs, kPairs order.
__device__ __forceinline__ void decode_block(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t magic,
                                             h2_t (&q)[16]) {
    const uint32_t win[7] = {w0,
                             __builtin_amdgcn_alignbit(w1, w0, 4),
                             __builtin_amdgcn_alignbit(w1, w0, 12),
                             w1,
                             __builtin_amdgcn_alignbit(w2, w1, 9),
                             w2,
                             w2 >> 7};
    q[0] = q_pair_i<0>(win, magic);
    q[1] = q_pair_i<1>(win, magic);
    q[2] = q_pair_i<2>(win, magic);
    q[3] = q_pair_i<3>(win, magic);
    q[4] = q_pair_i<4>(win, magic);
    q[5] = q_pair_i<5>(win, magic);
    q[6] = q_pair_i<6>(win, magic);
    q[7] = q_pair_i<7>(win, magic);
    q[8] = q_pair_i<8>(win, magic);
    q[9] = q_pair_i<9>(win, magic);
    q[10] = q_pair_i<10>(win, magic);
    q[11] = q_pair_i<11>(win, magic);
    q[12] = q_pair_i<12>(win, magic);
    q[13] = q_pair_i<13>(win, magic);
    q[14] = q_pair_i<14>(win, magic);
    q[15] = q_pair_i<15>(win, magic);
}

// Pairs 4u .. 4u + 3 of a block (kPairs order), u a compile-time value after
// unrolling: the same values as decode_block, a quarter at a time.  Each
// quarter needs one funnel shift (windows 1, 2, 4, 6; windows 0, 3, 5 are the
// words themselves).
__device__ __forceinline__ void decode_quarter(int u, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t magic,
                                               h2_t (&q)[4]) {
    if (u == 0) {
        const uint32_t win[7] = {w0, __builtin_amdgcn_alignbit(w1, w0, 4), 0, 0, 0, 0, 0};
        q[0] = q_pair_i<0>(win, magic);
        q[1] = q_pair_i<1>(win, magic);
        q[2] = q_pair_i<2>(win, magic);
        q[3] = q_pair_i<3>(win, magic);
    } else if (u == 1) {
        const uint32_t win[7] = {0, 0, __builtin_amdgcn_alignbit(w1, w0, 12), w1, 0, 0, 0};
        q[0] = q_pair_i<4>(win, magic);
        q[1] = q_pair_i<5>(win, magic);
        q[2] = q_pair_i<6>(win, magic);
        q[3] = q_pair_i<7>(win, magic);
    } else if (u == 2) {
        const uint32_t win[7] = {0, 0, 0, 0, __builtin_amdgcn_alignbit(w2, w1, 9), w2, 0};
        q[0] = q_pair_i<8>(win, magic);
        q[1] = q_pair_i<9>(win, magic);
        q[2] = q_pair_i<10>(win, magic);
        q[3] = q_pair_i<11>(win, magic);
    } else {
        const uint32_t win[7] = {0, 0, 0, 0, 0, w2, w2 >> 7};
        q[0] = q_pair_i<12>(win, magic);
        q[1] = q_pair_i<13>(win, magic);
        q[2] = q_pair_i<14>(win, magic);
        q[3] = q_pair_i<15>(win, magic);
    }
}

// acc + sum over the block of q * x', x' given as 16 fp16 pairs in pair order.
__device__ __forceinline__ float dot_block(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t magic,
                                           const uint32_t *xp, float acc) {
    h2_t q[16];
    decode_block(w0, w1, w2, magic, q);
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

// 32 bf16 values -> x * 2^-(e + slot offset) as fp16, arranged as the 16
// pairs of a block (kPairs order).
__device__ __forceinline__ void convert_block(const uint4 (&xb)[4], int e, uint32_t (&out)[16]) {
    float f[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d[4] = {xb[i].x, xb[i].y, xb[i].z, xb[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[8 * i + 2 * j] = bf16_to_f32(d[j] & 0xFFFFu);
            f[8 * i + 2 * j + 1] = bf16_to_f32(d[j] >> 16);
        }
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const PairSpec ps = kPairs[p];
        out[p] = pack_h2((_Float16)ldexpf(f[ps.lo], -e - ps.p), (_Float16)ldexpf(f[ps.hi], -e - ps.pp));
    }
}

__device__ __forceinline__ void load_x32(const uint16_t *src, uint4 (&xb)[4]) {
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[i] = s[i];
}

// ------------------------------------------------------------- qpack -------
// One thread per (row, group): 128 codes in, 12 words out (grid-stride loop).
__device__ __forceinline__ void pack_group(const uint8_t *__restrict__ codes, uint32_t *__restrict__ packed,
                                           int64_t u) {
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

__global__ __launch_bounds__(256) void qpack_kernel(const uint8_t *__restrict__ codes,
                                                    uint32_t *__restrict__ packed, int64_t units) {
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256)
        pack_group(codes, packed, u);
}

// ------------------------------------- repack from 4-bit containers -------
// The intermediate that GSQ training writes (GSQ model card, "Storage
// layout": the 3-bit codebook padded into a 4-bit INT32 container): code k of
// a row in nibble k % 8 of word k / 8, least significant nibble first, its top
// bit padding.  A group of 128 codes is 16 container words in and 12 stream
// words out; one thread per group, grid-stride loop.
__device__ __forceinline__ void repack_group(const uint32_t *__restrict__ w4, uint32_t *__restrict__ packed,
                                             int64_t u) {
    const uint4 *src = reinterpret_cast<const uint4 *>(w4 + u * 16);
    uint32_t words[kWordsPerGroup];
    uint64_t acc = 0;
    int nbits = 0, nw = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t c = (d[j >> 3] >> (4 * (j & 7))) & 7u;
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

__global__ __launch_bounds__(256) void qrepack_w4c_kernel(const uint32_t *__restrict__ w4,
                                                          uint32_t *__restrict__ packed, int64_t units) {
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256)
        repack_group(w4, packed, u);
}

// ----------------------------------------------------------- qdequant -----
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Chunk i of 8 consecutive weights: group i / 16 (row-major groups: row n's
// group g is group n * G + g), from bit 24 * (i % 16) of it (at most two
// words), to one 16-byte store.
__device__ __forceinline__ void dequant_chunk(const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales,
                                              uint16_t *__restrict__ w_out, int64_t i) {
    const int64_t u = i >> 4;
    const int b0 = 24 * (int)(i & 15);
    const int j = b0 >> 5;
    const uint32_t *gw = packed + u * kWordsPerGroup;
    const uint32_t lo = gw[j];
    const uint32_t hi = gw[j < kWordsPerGroup - 1 ? j + 1 : j];  // the last chunk sits in word 11 alone
    const uint32_t field = (uint32_t)(((((uint64_t)hi) << 32) | lo) >> (b0 & 31));
    const float s = bf16_to_f32(scales[u]);
    uint32_t h[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) h[t] = f32_to_bf16_rne((float)((int)((field >> (3 * t)) & 7u) - 4) * s);
    reinterpret_cast<uint4 *>(w_out)[i] =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// Consecutive threads take consecutive chunks, so their 16-byte stores are
// contiguous; grid-stride loop for any size.
__global__ __launch_bounds__(256) void qdequant_kernel(const uint32_t *__restrict__ packed,
                                                       const uint16_t *__restrict__ scales,
                                                       uint16_t *__restrict__ w_out, int64_t chunks) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * 256)
        dequant_chunk(packed, scales, w_out, i);
}

// ------------------------------------------------------------ qgemv -------
// Batch-1 fused GEMV.  A team of T lanes owns one output row at a time; lane
// g of the team owns weight group g (128 weights = 12 words = 48 contiguous
// bytes), so the team's three 16-byte loads per lane cover the row
// contiguously.  The lane's 128 activations stay in 64 VGPRs as fp16 pairs
// for the whole kernel ("x-stationary").  R = WGS / T teams per workgroup walk
// the rows in a grid-stride loop.  Each lane keeps a ring of D rows in flight:
// the loads of row i + D are issued as soon as row i has been decoded, so the
// memory system always holds D rows per team (the GEMV is latency-bound
// without it).  Partial sums are reduced in a fixed order (DPP inside a wave,
// then LDS across waves), so results are run-to-run identical.
#ifndef QW3_GEMV_DEPTH
#define QW3_GEMV_DEPTH 3
#endif
constexpr int kGemvDepth = QW3_GEMV_DEPTH;
#ifndef QW3_GEMV_WGS
#define QW3_GEMV_WGS 256
#endif
constexpr int kGemvWGS = QW3_GEMV_WGS;  // threads per workgroup, teams of T <= 64
#ifdef QW3_GEMV_WAVES
#define QW3_GEMV_OCC __attribute__((amdgpu_waves_per_eu(QW3_GEMV_WAVES)))
#else
#define QW3_GEMV_OCC
#endif
constexpr size_t kMaxLdsX = 64 * 1024;

struct RowBuf {
    uint4 a, b, c;  // the lane's 12 words of the row
    uint32_t s;     // the lane's bf16 scale
};

// Loads the lane's 12 words and scale of row r.  Every load is issued
// unconditionally -- rows past the end read the last row, lanes without a
// group read the last group -- so the code between loads is straight-line and
// the compiler can wait for exactly the loads a step needs (s_waitcnt vmcnt(n))
// instead of draining every load in flight.  The extra rows are never stored
// and the extra groups meet zero activations.
#ifndef QW3_GEMV_NT
#define QW3_GEMV_NT 0
#endif
typedef unsigned u32x4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_words16(const uint32_t *p) {
#if QW3_GEMV_NT
    // Streaming data, read once: non-temporal loads keep it out of the caches.
    const u32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const uint4 *>(p);
#endif
}

__device__ __forceinline__ void load_row(const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales,
                                         int64_t r, int64_t N, int64_t W, int G, int g_load, RowBuf &rb) {
    const int64_t rr = r < N ? r : N - 1;
    const uint32_t *p = packed + rr * W + g_load * kWordsPerGroup;
    rb.a = load_words16(p);
    rb.b = load_words16(p + 4);
    rb.c = load_words16(p + 8);
    rb.s = scales[rr * G + g_load];
}

// sum_k q_k x'_k * 2^e * s over the lane's group of one row.
__device__ __forceinline__ float row_partial(const RowBuf &rb, const uint32_t (&xp)[64], int e, uint32_t magic) {
    const float a0 = dot_block(rb.a.x, rb.a.y, rb.a.z, magic, xp + 0, 0.f);
    const float a1 = dot_block(rb.a.w, rb.b.x, rb.b.y, magic, xp + 16, 0.f);
    const float a2 = dot_block(rb.b.z, rb.b.w, rb.c.x, magic, xp + 32, 0.f);
    const float a3 = dot_block(rb.c.y, rb.c.z, rb.c.w, magic, xp + 48, 0.f);
    return ldexpf((a0 + a1) + (a2 + a3), e) * bf16_to_f32(rb.s);
}

// Activation staging, LDS path.  The workgroup converts x once: 4 threads (a
// quad) per group, one 32-value block each, U blocks per thread at most; then
// every lane copies its own group's 64 pairs and exponent into registers.
// Issue (raw loads) and finish (convert, exchange) are split so the row loads
// can be issued in between.
template <int U>
struct XStage {
    uint4 raw[U][4];
};

template <int U>
__device__ __forceinline__ void xstage_issue(const uint16_t *__restrict__ x, int G, XStage<U> &st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int idx = threadIdx.x + u * blockDim.x;
        if (idx >= 4 * G) idx = 4 * G - 1;  // clamped: always issued
        load_x32(x + (size_t)(idx >> 2) * kGroup + (idx & 3) * 32, st.raw[u]);
    }
}

// LDS layout of the converted activations: xs4[q][g] holds pairs 4q..4q+3 of
// group g (16 bytes), q = 0..15, so that when lane g fetches its group the 64
// lanes of each ds_read_b128 touch 64 consecutive 16-byte chunks (no bank
// conflicts); exponents follow as int[G].
template <int U>
__device__ __forceinline__ void xstage_convert(const XStage<U> &st, int G, uint32_t *smem) {
    uint4 *xs4 = reinterpret_cast<uint4 *>(smem);                // [16][G]
    int *xe = reinterpret_cast<int *>(smem + (size_t)G * 64);  // [G]
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int idx = threadIdx.x + u * blockDim.x;  // quads share validity: 4G and blockDim are multiples of 4
        uint32_t m = absmax32(st.raw[u]);
        m = max(m, dpp_u32<kDppQuadXor1>(m));
        m = max(m, dpp_u32<kDppQuadXor2>(m));
        if (idx < 4 * G) {
            const int g = idx >> 2, blk = idx & 3;
            const int eg = group_exponent(m);
            uint32_t out[16];
            convert_block(st.raw[u], eg, out);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xs4[(size_t)(4 * blk + i) * G + g] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
            if (blk == 0) xe[g] = eg;
        }
    }
}

// After a barrier: this lane's pairs and exponent (zeros for lanes without a group).
__device__ __forceinline__ void xstage_fetch(const uint32_t *smem, int G, int gl, bool lane_on,
                                             uint32_t (&xp)[64], int &e) {
    const int *xe = reinterpret_cast<const int *>(smem + (size_t)G * 64);
    const int gs = lane_on ? gl : 0;
    const uint4 *xs4 = reinterpret_cast<const uint4 *>(smem);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint4 v = xs4[(size_t)i * G + gs];
        xp[4 * i] = lane_on ? v.x : 0u;
        xp[4 * i + 1] = lane_on ? v.y : 0u;
        xp[4 * i + 2] = lane_on ? v.z : 0u;
        xp[4 * i + 3] = lane_on ? v.w : 0u;
    }
    e = lane_on ? xe[gs] : 0;
}

// Activation staging without LDS (very long rows): each lane converts its own
// group in two passes (max, then convert).
__device__ __forceinline__ void xstage_lane(const uint16_t *__restrict__ x, int gl, bool lane_on,
                                            uint32_t (&xp)[64], int &e) {
    const uint16_t *xg = x + (size_t)(lane_on ? gl : 0) * kGroup;
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
        for (int p = 0; p < 16; ++p) xp[blk * 16 + p] = lane_on ? out[p] : 0u;
    }
    if (!lane_on) e = 0;
}

// Up to 4 weight matrices with the same K that share one activation vector
// (e.g. the q, k and v projections of a layer) in one launch (one activation
// staging): the workgroups are dealt to the matrices in proportion to their
// rows, so each workgroup works on one matrix and its pointers stay uniform.
constexpr int kMaxSegs = 4;
struct GemvSegs {
    const uint32_t *packed[kMaxSegs];
    const uint16_t *scales[kMaxSegs];
    float *y[kMaxSegs];
    int64_t rows[kMaxSegs];
    int blk_end[kMaxSegs];  // cumulative workgroup counts; unused entries repeat the total
};

template <typename P>
__device__ __forceinline__ P seg_pick(const P (&v)[kMaxSegs], int k) {
    return k == 0 ? v[0] : (k == 1 ? v[1] : (k == 2 ? v[2] : v[3]));
}

// Teams of T <= 64 lanes (T a power of two >= G): the reduction is DPP only.
// Order of the prologue: activation loads, then the first D rows, then the
// conversion (which waits only for the activation loads).
template <int T, bool MULTI, int D>
__global__ __launch_bounds__(kGemvWGS) QW3_GEMV_OCC void qgemv_small_kernel(const uint16_t *__restrict__ x,
                                                               const GemvSegs sg, int G, int lds_x) {
    constexpr int R = kGemvWGS / T;
    extern __shared__ uint32_t smem[];
    // This workgroup's matrix (workgroup-uniform) and its place among the
    // workgroups of that matrix.
    int kseg = 0, blk = blockIdx.x, nblk = gridDim.x;
    if constexpr (MULTI) {
        kseg = ((int)blockIdx.x >= sg.blk_end[0]) + ((int)blockIdx.x >= sg.blk_end[1]) +
               ((int)blockIdx.x >= sg.blk_end[2]);
        const int b0 = kseg == 0 ? 0 : seg_pick(sg.blk_end, kseg - 1);
        blk = blockIdx.x - b0;
        nblk = seg_pick(sg.blk_end, kseg) - b0;
    }
    const uint32_t *__restrict__ packed = MULTI ? seg_pick(sg.packed, kseg) : sg.packed[0];
    const uint16_t *__restrict__ scales = MULTI ? seg_pick(sg.scales, kseg) : sg.scales[0];
    float *__restrict__ y = MULTI ? seg_pick(sg.y, kseg) : sg.y[0];
    const int64_t N = MULTI ? seg_pick(sg.rows, kseg) : sg.rows[0];
    const int gl = threadIdx.x % T;
    const bool lane_on = gl < G;
    const int g_load = lane_on ? gl : G - 1;
    const int64_t W = (int64_t)G * kWordsPerGroup;
    const int64_t stride = (int64_t)nblk * R;
    const int64_t row0 = (int64_t)blk * R + threadIdx.x / T;
    auto load = [&](int64_t r, RowBuf &rb) { load_row(packed, scales, r, N, W, G, g_load, rb); };

    // Ring of E = D + 1 row buffers.  Step i first issues the loads of row
    // i + D into the buffer that step i - 1 finished with, then decodes row i:
    // D rows are in flight while a row is decoded (the scheduling barrier
    // keeps the compiler from sinking the loads behind the decode).
    constexpr int E = D + 1;
    uint32_t xp[64];
    int e = 0;
    RowBuf ring[E];
    if (lds_x) {
        XStage<1> st;  // 4G <= 256 <= blockDim: one block per thread
        xstage_issue<1>(x, G, st);
#pragma unroll
        for (int d = 0; d < D; ++d) load(row0 + d * stride, ring[d]);
        xstage_convert<1>(st, G, smem);
        __syncthreads();
        xstage_fetch(smem, G, gl, lane_on, xp, e);
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d) load(row0 + d * stride, ring[d]);
        xstage_lane(x, gl, lane_on, xp, e);
    }
    const uint32_t magic = magic_vgpr();

    for (int64_t row = row0; row < N; row += E * stride) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const int64_t r = row + i * stride;
            load(r + D * stride, ring[(i + D) % E]);
            __builtin_amdgcn_sched_barrier(0);
            const float part = row_partial(ring[i], xp, e, magic);
            const float tot = segment_sum<T>(part);
            if (gl == T - 1 && r < N) y[r] = tot;
        }
    }
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// only, so its global loads stay in flight across the barrier, and the
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Teams of T > 64 lanes, T a multiple of 32 (>= G): each half-wave sums its 32
// lanes with DPP, the half sums go through LDS, and lane 0 of the team adds
// its T/32 halves in order.  One barrier per D + 1 rows.  1024-thread
// workgroups (K > 65536) keep a single row in flight to stay within 128 VGPRs.  The LDS holds the
// converted activations first, then (after a barrier) the half sums.
// LDS_X: the converted activations fit in LDS (K <= 32768); otherwise each
// lane converts its own group.  A template parameter, so that one prologue
// reaches the loop and the loop's waits are exact.
template <int MAXWGS, int D, bool LDS_X>
__global__ __launch_bounds__(MAXWGS) QW3_GEMV_OCC void qgemv_big_kernel(const uint16_t *__restrict__ x,
                                                         const uint32_t *__restrict__ packed,
                                                         const uint16_t *__restrict__ scales,
                                                         float *__restrict__ y, int64_t N, int G, int T) {
    extern __shared__ uint32_t smem[];
    const int tid = threadIdx.x;
    const int wgs = blockDim.x;
    const int R = wgs / T;
    const int gl = tid % T;
    const int team = tid / T;
    const int halves = T / 32;
    const bool lane_on = gl < G;
    const int g_load = lane_on ? gl : G - 1;
    const int64_t W = (int64_t)G * kWordsPerGroup;
    const int64_t stride = (int64_t)gridDim.x * R;
    const int64_t row0 = (int64_t)blockIdx.x * R + team;

    // Issue-first ring of E = D + 1 row buffers, as in qgemv_small_kernel.
    constexpr int E = D + 1;
    uint32_t xp[64];
    int e = 0;
    RowBuf ring[E];
    if constexpr (LDS_X) {
        XStage<4> st;  // 4G <= 4 * blockDim (T >= G, blockDim >= T)
        xstage_issue<4>(x, G, st);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            __builtin_amdgcn_sched_barrier(0);  // rows issued in ring order
            load_row(packed, scales, row0 + d * stride, N, W, G, g_load, ring[d]);
        }
        __builtin_amdgcn_sched_barrier(0);
        xstage_convert<4>(st, G, smem);
        __syncthreads();
        xstage_fetch(smem, G, gl, lane_on, xp, e);
        __syncthreads();  // LDS is reused for the half sums below
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            load_row(packed, scales, row0 + d * stride, N, W, G, g_load, ring[d]);
        }
        __builtin_amdgcn_sched_barrier(0);
        xstage_lane(x, gl, lane_on, xp, e);
    }
    const uint32_t magic = magic_vgpr();

    float *red = reinterpret_cast<float *>(smem);  // [2][E][wgs/32]
    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * R; base < N; base += E * stride) {  // WG-uniform
        const int64_t row = base + team;
        float *slot = red + parity * E * (wgs / 32);
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const int64_t r = row + i * stride;
            load_row(packed, scales, r + D * stride, N, W, G, g_load, ring[(i + D) % E]);
            __builtin_amdgcn_sched_barrier(0);
            const float part = row_partial(ring[i], xp, e, magic);
            const float hs = segment_sum<32>(part);
            if ((tid & 31) == 31) slot[i * (wgs / 32) + (tid >> 5)] = hs;
        }
        // Half sums written (lgkmcnt) before the barrier; global loads stay in
        // flight (a __syncthreads fence would wait for them too).
        lds_barrier();
        if (gl == 0) {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const int64_t r = row + i * stride;
                if (r < N) {
                    float tot = 0.f;
                    for (int h = 0; h < halves; ++h) tot += slot[i * (wgs / 32) + team * halves + h];
                    y[r] = tot;
                }
            }
        }
        parity ^= 1;
    }
}

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. C - 1, each index a
// compile-time constant (register-ring slots must be static).
template <int I, int C, typename F>
__device__ __forceinline__ void static_for_from(F &&f) {
    if constexpr (I < C) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, C>(f);
    }
}
template <int C, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_from<0, C>(f);
}

// ------------------------------------- batch 1, K = 8192, on the matrix cores --
// The same fused GEMV with the dot products on v_mfma_f32_16x16x32_f16, which
// leaves two VALU ops per weight pair (the exact decode) instead of three.
// Workgroups of four waves walk 16-row tiles; wave w owns the 16 groups
// 16q + 4w + j (q, j = 0..3) of every row of a tile, so the four waves together
// cover K = 8192 and a tile's super-step q reads bytes [768q, 768q + 768) of
// each of its rows.  In super-step q, lane (n, j) (n = lane % 16, j = lane / 16)
// decodes group 16q + 4w + j of row n straight into the B operand (k chunk j
// of 8 weights, 4 MFMAs per 32-code block).  The A operand is x' and stays in
// 64 VGPRs for the whole kernel: row m = 4q' + j' of A carries the activations
// of group 16q' + 4w + j' in k chunk j' and zero elsewhere.  So output row
// 4q' + j' only ever sums products of group 16q' + 4w + j' activations; in
// super-step q the rows 4q..4q+3 hold the partial sums of groups 16q + 4w + r
// (r = 0..3) exactly apart, in lane row q, and the other 12 rows are discarded.
// Those four partials are multiplied by their group scale (and the
// activation exponent) and accumulated in fp32.  The wave's per-row partials
// are summed across lane rows with permlane swaps and across the four waves
// through LDS, in a fixed order, once per batch of tiles.  Loads run three
// super-steps ahead in a register ring, as in qgemv_small_kernel.
#ifndef QW3_MF_BATCH
#define QW3_MF_BATCH 8
#endif
#ifndef QW3_MF_ILV
#define QW3_MF_ILV 1
#endif
#ifndef QW3_MF_RING
#define QW3_MF_RING 4
#endif
#ifndef QW3_MF_AHEAD
#define QW3_MF_AHEAD 3
#endif
constexpr int kMfBatch = QW3_MF_BATCH;  // tiles per cross-wave reduction
constexpr int kMfRing = QW3_MF_RING;    // register ring slots (one super-step each)
constexpr int kMfAhead = QW3_MF_AHEAD;  // super-steps loaded ahead of the one decoded
#ifndef QW3_MF_PER_CU
#define QW3_MF_PER_CU 1
#endif
constexpr int kMfPerCu = QW3_MF_PER_CU;  // workgroups per CU
// LDS: the converted activations, then the partial sums [2][kMfBatch][WAVES][16].
template <int GPW, int WAVES>
constexpr size_t mf_lds() {
    return (size_t)GPW * WAVES * 64 * 4 + (size_t)GPW * WAVES * 4 + 2 * kMfBatch * WAVES * 16 * sizeof(float);
}
typedef unsigned u32x2v_t __attribute__((ext_vector_type(2)));
struct MfSlot {
    u32x4v_t a, b, c;  // the lane's 12 words of one group of one row
    u32x2v_t s;        // (super-steps 0 and 4) the bf16 scales of lane row j's four groups
};

// First of the four groups that wave w (of WAVES, GPW groups each) handles in
// super-step q.
template <int GPW, int WAVES>
__device__ __forceinline__ int mf_group(int w, int q) {
    return QW3_MF_ILV ? 4 * WAVES * q + 4 * w : GPW * w + 4 * q;
}

// GPW groups per wave: 16 (K = 8192, 4 waves) or 32 (K = 28672, 7 waves).  A
// wave then walks GPW / 4 super-steps per tile, and its activations are GPW /
// 16 A-operand sets: set a serves super-steps 4a .. 4a + 3 with rows
// m = 4(q mod 4) + j' as above.
template <int GPW, int WAVES, bool MULTI>
__global__ __launch_bounds__(64 * WAVES) void qgemv_mfma_kernel(const uint16_t *__restrict__ x, const GemvSegs sg) {
    constexpr int G = GPW * WAVES;
    constexpr int NS = GPW / 4;   // super-steps per tile
    constexpr int AS = GPW / 16;  // A-operand sets
    constexpr int XU = (4 * G + 64 * WAVES - 1) / (64 * WAVES);  // activation blocks per thread
    constexpr int64_t W = (int64_t)G * kWordsPerGroup;
    static_assert(NS % 4 == 0, "whole A-operand sets");
    extern __shared__ uint32_t smem[];
    float *red = reinterpret_cast<float *>(smem + G * 64 + G);  // [2][kMfBatch][WAVES][16 rows]
    int kseg = 0, blk = blockIdx.x, nblk = gridDim.x;
    if constexpr (MULTI) {
        kseg = ((int)blockIdx.x >= sg.blk_end[0]) + ((int)blockIdx.x >= sg.blk_end[1]) +
               ((int)blockIdx.x >= sg.blk_end[2]);
        const int b0 = kseg == 0 ? 0 : seg_pick(sg.blk_end, kseg - 1);
        blk = blockIdx.x - b0;
        nblk = seg_pick(sg.blk_end, kseg) - b0;
    }
    const uint32_t *__restrict__ packed = MULTI ? seg_pick(sg.packed, kseg) : sg.packed[0];
    const uint16_t *__restrict__ scales = MULTI ? seg_pick(sg.scales, kseg) : sg.scales[0];
    float *__restrict__ y = MULTI ? seg_pick(sg.y, kseg) : sg.y[0];
    const int64_t N = MULTI ? seg_pick(sg.rows, kseg) : sg.rows[0];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, lj = lane >> 4;
    const int64_t my_tiles = (((N + 15) >> 4) - blk + nblk - 1) / nblk;  // >= 1: at most one workgroup per tile
    // Unconditional loads (see load_row): tiles past the last re-read it, rows past N read row N - 1.
    auto load = [&](int64_t it, int q, MfSlot &sl) {
        it = it < my_tiles ? it : my_tiles - 1;
        int64_t r = (blk + it * nblk) * 16 + n;
        r = r < N ? r : N - 1;
        const u32x4v_t *p =
            reinterpret_cast<const u32x4v_t *>(packed + r * W + (mf_group<GPW, WAVES>(w, q) + lj) * kWordsPerGroup);
        sl.a = p[0];
        sl.b = p[1];
        sl.c = p[2];
        if (q % 4 == 0)
            sl.s = *reinterpret_cast<const u32x2v_t *>(scales + r * G + mf_group<GPW, WAVES>(w, q + lj));
    };
    // Steps are numbered s = NS * tile + q; step s lives in ring slot s % RS.
    // The body covers UT tiles, a whole number of ring cycles, so every slot
    // index is static.
    constexpr int RS = kMfRing, AH = kMfAhead;
    constexpr int UT = RS > NS ? RS / NS : 1;
    static_assert(AH < RS && (RS % NS == 0 || NS % RS == 0), "ring cycles must tile the super-steps");
    MfSlot ring[RS];
    XStage<XU> st;
    xstage_issue<XU>(x, G, st);
    // Issued strictly in ring order: the waits in the loop count on it.
#pragma unroll
    for (int s = 0; s < AH; ++s) {
        load(s / NS, s % NS, ring[s % RS]);
        __builtin_amdgcn_sched_barrier(0);
    }
    xstage_convert<XU>(st, G, smem);
    __syncthreads();
    h8_t xa[AS][16];  // step t = 4 * block + u: pairs 4u .. 4u + 3 of 32-code block `block`
    float fe[AS][4];  // 2^e of the groups whose partials this lane scales (lane row lj of each set)
    {
        const bool on = (n & 3) == lj;
        const uint4 *xs4 = reinterpret_cast<const uint4 *>(smem);
        const int *xe = reinterpret_cast<const int *>(smem + G * 64);
#pragma unroll
        for (int a = 0; a < AS; ++a) {
            const int ga = mf_group<GPW, WAVES>(w, 4 * a + (n >> 2)) + lj;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const uint4 v = xs4[t * G + ga];
                xa[a][t] = on ? __builtin_bit_cast(h8_t, v) : h8_t{0, 0, 0, 0, 0, 0, 0, 0};
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) fe[a][r] = ldexpf(1.0f, xe[mf_group<GPW, WAVES>(w, 4 * a + lj) + r]);
        }
    }
    const uint32_t magic = magic_vgpr();
    // Tile it0 + h, whose super-steps are ring steps h * NS + q.
    auto tile = [&](int64_t it0, auto hc) __attribute__((always_inline)) {
        constexpr int h = decltype(hc)::value;
        const int64_t it = it0 + h;
        float acc[4] = {0.f, 0.f, 0.f, 0.f}, sc[AS][4];
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            // refill the slot freed by the previous step with the step AH ahead
            const int u = h * NS + q;
            load(it0 + (u + AH) / NS, (u + AH) % NS, ring[(u + AH) % RS]);
            __builtin_amdgcn_sched_barrier(0);
            const MfSlot &sl = ring[u % RS];
            const int a = q / 4;
            if (q % 4 == 0) {
                sc[a][0] = bf16_to_f32(sl.s.x & 0xFFFFu) * fe[a][0];
                sc[a][1] = __uint_as_float(sl.s.x & 0xFFFF0000u) * fe[a][1];
                sc[a][2] = bf16_to_f32(sl.s.y & 0xFFFFu) * fe[a][2];
                sc[a][3] = __uint_as_float(sl.s.y & 0xFFFF0000u) * fe[a][3];
            }
            const uint32_t wd[12] = {sl.a.x, sl.a.y, sl.a.z, sl.a.w, sl.b.x, sl.b.y,
                                     sl.b.z, sl.b.w, sl.c.x, sl.c.y, sl.c.z, sl.c.w};
            f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                h2_t qd[16];
                decode_block(wd[3 * b], wd[3 * b + 1], wd[3 * b + 2], magic, qd);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const h8_t bop = {qd[4 * v].x,     qd[4 * v].y,     qd[4 * v + 1].x, qd[4 * v + 1].y,
                                      qd[4 * v + 2].x, qd[4 * v + 2].y, qd[4 * v + 3].x, qd[4 * v + 3].y};
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[a][4 * b + v], bop, d, 0, 0, 0);
                }
            }
            if (lj == q % 4) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(d[r], sc[a][r], acc[r]);
            }
        }
        // Row n's partial over the wave's groups: the four lane rows, then LDS.
        float part = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        const auto s32 =
            __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        part = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
        const auto s16 =
            __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        part = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
        const int bt = (int)(it % kMfBatch);
        float *rb = red + ((it / kMfBatch) & 1) * (kMfBatch * WAVES * 16);
        if (lj == 0) rb[(bt * WAVES + w) * 16 + n] = part;
        if (bt == kMfBatch - 1 || it == my_tiles - 1) {
            // The batch's partials are in LDS (lgkmcnt) before the barrier; the
            // loads of the next tiles stay in flight.  The other half of `red`
            // is written next, so one barrier per batch suffices.
            lds_barrier();
            const int i = threadIdx.x;
            if (i < (bt + 1) * 16) {
                const float *rr = rb + (i >> 4) * WAVES * 16 + (i & 15);
                float tot = rr[0];
#pragma unroll
                for (int v = 1; v < WAVES; ++v) tot += rr[16 * v];
                const int64_t row = (blk + (it - bt + (i >> 4)) * nblk) * 16 + (i & 15);
                if (row < N) y[row] = tot;
            }
        }
    };
    // Whole ring cycles in the loop, so its back edge always carries the same
    // pending loads (exact waits); a ragged last cycle follows it.
    int64_t it0 = 0;
    for (; it0 + UT <= my_tiles; it0 += UT)
        static_for<UT>([&](auto hc) __attribute__((always_inline)) { tile(it0, hc); });
    static_for<UT - 1>([&](auto hc) __attribute__((always_inline)) {
        if (it0 + decltype(hc)::value < my_tiles) tile(it0, hc);
    });
    // Slots whose loads (past the last tile) are still in flight at the loop's
    // exit and that the ragged cycle does not read: held until here, so their
    // registers are not reused -- which would first wait for those loads.
    if constexpr (UT > 1)
        static_for<RS>([&ring](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i >= NS * (UT - 1) && i < AH)
                asm volatile("" ::"v"(ring[i].a), "v"(ring[i].b), "v"(ring[i].c), "v"(ring[i].s));
        });
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
    const uint32_t magic = magic_vgpr();

    for (int g = 0; g < G; ++g) {
        const uint32_t *wp = wrow + (int64_t)g * kWordsPerGroup;
        const uint32_t w0 = wp[0], w1 = wp[1], w2 = wp[2];
        const float s = bf16_to_f32(srow[g]);
        h2_t q[16];
        decode_block(w0, w1, w2, magic, q);
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

// y[m][n] = sum over chunks c, in order, of part[c][m][n].
__global__ __launch_bounds__(256) void qgemm_chunk_sum_kernel(const float *__restrict__ part, float *__restrict__ y,
                                                            int64_t count, int C, int64_t chunk_stride) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    // Up to 8 chunks' loads in flight before their adds (a plain loop waits
    // for each load in turn); the adds stay in chunk order.
    constexpr int kBatch = 8;
    float tot = 0.f;
    for (int c0 = 0; c0 < C; c0 += kBatch) {
        float v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (c0 + k < C) v[k] = part[(int64_t)(c0 + k) * chunk_stride + i];
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (c0 + k < C) tot = c0 + k == 0 ? v[k] : tot + v[k];
    }
    y[i] = tot;
}

// ------------------------------ batched decode from registers, K-split, MFMA --
// Same decode and MFMAs as qgemm_bd_kernel (lane (n = l%16, j = l/16)
// decodes block j of each group of weight row n of a 16-row tile; 4 MFMAs
// per group, then D * s[n][g]), but the words come straight from
// global memory into registers: lane (n, j) loads all 48 bytes of group
// 4q + j of its row, so the 4 lanes of a row read 192 contiguous bytes, and
// a 4 x 4 transpose of 12-byte blocks across the 4 lanes (permlane32 and
// permlane16 swaps) then gives lane j block j of groups 4q..4q+3.  Each wave
// owns 8 consecutive groups (2 quads) of a chunk of K; tiles are prefetched
// one ahead in registers.  The activations of a wave's 8 groups share one
// exponent per token (prep_x_slice_kernel), so D * s[n][g] accumulates and
// the token exponent is applied once per tile.

// x' with one exponent per (token, 8-group slice): unit (slice, m, gi, b) =
// the 32 values of block b of group slice*8 + gi; the 32 units of a
// (slice, m) are one half-wave.  Stored as xq[((g*4 + t)*4 + b)*Mp + m]
// (t: the MFMA of the block), xe[slice*Mp + m]: the batched kernels' lane
// (m, b) = m + 16b reads xq[(g*4 + t)*64 + lane], so each of their operand
// loads is one contiguous kilobyte.
__global__ __launch_bounds__(256) void prep_x_slice_kernel(const uint16_t *__restrict__ x, uint4 *__restrict__ xq,
                                                           int16_t *__restrict__ xe, int M, int Mp, int64_t K,
                                                           int S) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t units = (int64_t)S * Mp * 32;
    if (idx >= units) return;  // units is a multiple of 32: whole half-waves exit together
    const int b = (int)(idx & 3);
    const int gi = (int)((idx >> 2) & 7);
    const int64_t sm = idx >> 5;
    const int m = (int)(sm % Mp);
    const int sl = (int)(sm / Mp);
    const int g = sl * 8 + gi;
    uint4 xb[4];
    if (m < M) {
        load_x32(x + (int64_t)m * K + (int64_t)g * kGroup + b * 32, xb);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xb[i] = make_uint4(0, 0, 0, 0);
    }
    uint32_t mx = absmax32(xb);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 32));
    const int e = m < M ? group_exponent(mx) : 0;
    uint32_t out[16];
    convert_block(xb, e, out);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xq[(((int64_t)g * 4 + i) * 4 + b) * Mp + m] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    if (gi == 0 && b == 0) xe[(int64_t)sl * Mp + m] = (int16_t)e;
}

// 4 x 4 transpose of 3-dword blocks across the lane rows j = l/16:
// in: b[k] = block k of lane row j's group; out: b[k] = block j of row k's.
__device__ __forceinline__ void quad_block_transpose(uint32_t (&b)[4][3]) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        // rows {0,1} <-> {2,3}: (b0, b2) and (b1, b3)
        auto r02 = __builtin_amdgcn_permlane32_swap(b[0][d], b[2][d], false, false);
        auto r13 = __builtin_amdgcn_permlane32_swap(b[1][d], b[3][d], false, false);
        // rows 0 <-> 1 and 2 <-> 3: (b0, b1) and (b2, b3)
        auto r01 = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
        auto r23 = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
        b[0][d] = r01[0];
        b[1][d] = r01[1];
        b[2][d] = r23[0];
        b[3][d] = r23[1];
    }
}

typedef unsigned u32x4m_t __attribute__((ext_vector_type(4)));
struct MtStage {
    u32x4m_t w[6];  // quad 0: w[0..2] (group 4*0 + j), quad 1: w[3..5] (group 4 + j)
    u32x4m_t s;     // bf16 scales of the wave's 8 groups for row n
};

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void qgemm_mt_kernel(const uint4 *__restrict__ xq,
                                                            const int16_t *__restrict__ xe,
                                                            const uint32_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scales,
                                                            float *__restrict__ out, int M, int64_t N, int G, int C,
                                                            int64_t out_chunk) {
    constexpr int Mp = 16;
    __shared__ __align__(16) unsigned char red[2][WAVES][64 * 16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int j = lane >> 4;
    const int chunk = (int)(blockIdx.x % C);
    const int64_t tb = blockIdx.x / C, TB = gridDim.x / C;
    const int g0 = (chunk * WAVES + wave) * 8;  // the wave's 8 groups
    const int64_t tiles = (N + 15) / 16;
    const int64_t my_tiles = (tiles - tb + TB - 1) / TB;  // >= 1
    const int64_t W = (int64_t)G * kWordsPerGroup;
    float *y = out + (int64_t)chunk * out_chunk;

    auto load_stage = [&](int64_t t, MtStage &st) {
        t = t < my_tiles ? t : my_tiles - 1;
        int64_t row = (tb + t * TB) * 16 + n;
        row = row < N ? row : N - 1;
        const uint32_t *rp = packed + row * W;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u32x4m_t *p = reinterpret_cast<const u32x4m_t *>(rp + (int64_t)(g0 + 4 * q + j) * kWordsPerGroup);
#pragma unroll
            for (int i = 0; i < 3; ++i) st.w[3 * q + i] = p[i];
        }
        const uint16_t *sp = scales + row * G + g0;
        st.s = u32x4m_t{(uint32_t)sp[0] | ((uint32_t)sp[1] << 16), (uint32_t)sp[2] | ((uint32_t)sp[3] << 16),
                        (uint32_t)sp[4] | ((uint32_t)sp[5] << 16), (uint32_t)sp[6] | ((uint32_t)sp[7] << 16)};
    };
    MtStage ring0, ring1;
    load_stage(0, ring0);

    h8_t xa[8][4];
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            xa[gi][u] = h8_t{0, 0, 0, 0, 0, 0, 0, 0};
            if (n < M) xa[gi][u] = __builtin_bit_cast(h8_t, xq[(((int64_t)(g0 + gi) * 4 + u) * 4 + j) * Mp + n]);
        }
    }
    // One activation exponent per (token, slice): D rows 4j..4j+3 are tokens.
    int et[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) et[r] = xe[(int64_t)(g0 / 8) * Mp + 4 * j + r];
    const uint32_t magic = magic_vgpr();

    auto tile = [&](int64_t t, const MtStage &st) {
        const uint32_t scw[4] = {st.s.x, st.s.y, st.s.z, st.s.w};
        f4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint32_t blk[4][3];
            const uint32_t wd[12] = {st.w[3 * q].x,     st.w[3 * q].y,     st.w[3 * q].z,     st.w[3 * q].w,
                                     st.w[3 * q + 1].x, st.w[3 * q + 1].y, st.w[3 * q + 1].z, st.w[3 * q + 1].w,
                                     st.w[3 * q + 2].x, st.w[3 * q + 2].y, st.w[3 * q + 2].z, st.w[3 * q + 2].w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int d = 0; d < 3; ++d) blk[k][d] = wd[3 * k + d];
            quad_block_transpose(blk);  // blk[k] = block j of group g0 + 4q + k
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int gi = 4 * q + k;
                h2_t qd[16];
                decode_block(blk[k][0], blk[k][1], blk[k][2], magic, qd);
                f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const h8_t bop = {qd[4 * u].x, qd[4 * u].y, qd[4 * u + 1].x, qd[4 * u + 1].y,
                                      qd[4 * u + 2].x, qd[4 * u + 2].y, qd[4 * u + 3].x, qd[4 * u + 3].y};
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[gi][u], bop, d, 0, 0, 0);
                }
                const uint32_t sw = scw[gi >> 1];
                const float sv = __uint_as_float((gi & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(d[r], sv, acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = ldexpf(acc[r], et[r]);
        *reinterpret_cast<f4_t *>(&red[t & 1][wave][lane * 16]) = acc;
        lds_barrier();  // LDS only: the next tile's loads stay in flight
        if (wave == (int)(t % WAVES)) {
            f4_t tot = *reinterpret_cast<const f4_t *>(&red[t & 1][0][lane * 16]);
#pragma unroll
            for (int w = 1; w < WAVES; ++w) tot += *reinterpret_cast<const f4_t *>(&red[t & 1][w][lane * 16]);
            const int64_t row = (tb + t * TB) * 16 + n;
            if (row < N) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * j + r < M) y[(int64_t)(4 * j + r) * N + row] = tot[r];
            }
        }
    };
    for (int64_t t = 0; t < my_tiles; t += 2) {
        load_stage(t + 1, ring1);
        __builtin_amdgcn_sched_barrier(0);
        tile(t, ring0);
        if (t + 1 >= my_tiles) break;  // workgroup-uniform
        load_stage(t + 2, ring0);
        __builtin_amdgcn_sched_barrier(0);
        tile(t + 1, ring1);
    }
}

// ----------------------- batched decode, a ring of 4-group steps (M <= 16) --
// The layout of qgemm_mt_kernel -- a wave owns 8 groups of a K chunk and 16
// tokens' activations in VGPRs; lane (n, j) loads group g0 + 4q + j of row n
// and a 4 x 4 block transpose gives it block j of each of the four groups --
// walked as 4-group super-steps (two per 16-row tile) through a ring of four
// register slots, the loads of a super-step issued two ahead (three ahead,
// with two waves per SIMD, put more bytes in flight than the memory system
// serves well and measured about 3 % slower).  The partial
// sums of a tile (token 4j + r, row n in lane (n, j), register r) go to LDS;
// every kMrBatch tiles one barrier lets the workgroup add its waves' partials
// in wave order and store them.  Scale rows must be 8-byte aligned (one
// 8-byte load per lane and super-step).
#ifndef QW3_MR_BATCH
#define QW3_MR_BATCH 4
#endif
constexpr int kMrBatch = QW3_MR_BATCH;
// TS sets of 16 tokens share each decoded block (TS = 2: 17..32 tokens in one
// pass over the weights); a wave then owns 8 / TS groups.
template <int WAVES, int TS>
constexpr size_t mr_lds() { return (size_t)2 * kMrBatch * WAVES * TS * 64 * 16; }
struct MrSlot {
    u32x4v_t w[3];  // group g0 + 4q + j of row n: 12 words
    u32x2v_t s;     // bf16 scales of groups g0 + 4q .. g0 + 4q + 3 of row n
};

template <int WAVES, int TS, bool XH>
__global__ __launch_bounds__(64 * WAVES) void qgemm_mr_kernel(const uint4 *__restrict__ xq,
                                                            const int16_t *__restrict__ xe,
                                                            const uint16_t *__restrict__ x,
                                                            const uint32_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scales,
                                                            float *__restrict__ out, int M, int64_t N, int G, int C,
                                                            int64_t out_chunk) {
    constexpr int Mp = 16 * TS;
    constexpr int GW = 8 / TS;   // groups per wave
    constexpr int NS = GW / 4;   // 4-group super-steps per tile
    constexpr int UT = 4 / NS;   // tiles per ring cycle (4 slots)
    extern __shared__ __align__(16) unsigned char lds[];  // [2][kMrBatch][WAVES][TS][64 lanes] x f4
    f4_t *red = reinterpret_cast<f4_t *>(lds);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int j = lane >> 4;
    const int chunk = (int)(blockIdx.x % C);
    const int64_t tb = blockIdx.x / C, TB = gridDim.x / C;
    const int g0 = (chunk * WAVES + wave) * GW;  // the wave's groups
    const int64_t my_tiles = (((N + 15) >> 4) - tb + TB - 1) / TB;  // >= 1: at most one tile block per tile
    const int64_t W = (int64_t)G * kWordsPerGroup;
    float *y = out + (int64_t)chunk * out_chunk;

    int et[TS][4];
    h8_t xa[GW][TS][4];
    [[maybe_unused]] uint4 xh[4][4];
    if constexpr (XH) {
        // Up to 8 tokens (TS = 1): the activations straight from x.  Lane
        // (n, j) reads block j of groups g0 + 4(n / 8) .. + 3 of token n % 8
        // (tokens past M read token M - 1; rows 8..15 of D are never stored),
        // so lanes n and n + 8 share the wave's 8 groups of one token.
        static_assert(!XH || TS == 1, "in-kernel conversion for one token set");
        const int64_t K = (int64_t)G * kGroup;
        const int t = (n & 7) < M ? (n & 7) : M - 1;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            load_x32(x + t * K + (int64_t)(g0 + 4 * (n >> 3) + k) * kGroup + 32 * j, xh[k]);
    } else {
        // The slice's activation exponents (one per token; the wave's groups lie
        // in one 8-group slice) through the scalar unit: they stay out of the
        // vector memory counter, whose waits in the loop count the ring's loads
        // exactly.  Lane row j scales tokens 16 ts + 4j .. 16 ts + 4j + 3.
        {
            const int *xs = reinterpret_cast<const int *>(xe + (int64_t)(g0 / 8) * Mp);
            int ew[8 * TS];
#pragma unroll
            for (int i = 0; i < 8 * TS; ++i) ew[i] = xs[i];
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int b = 8 * ts + r / 2;
                    const int w0 = j == 0 ? ew[b] : j == 1 ? ew[b + 2] : j == 2 ? ew[b + 4] : ew[b + 6];
                    et[ts][r] = (r & 1) ? (w0 >> 16) : (int)(int16_t)(w0 & 0xFFFF);
                }
        }
        // Activations first (L2-resident), then the ring: the loop's waits for
        // the ring count exactly.  Token slots past M read slot M - 1 again (their
        // rows of D are never stored), so a load touches only the lines of the M
        // real tokens.
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            const int m = 16 * ts + n < M ? 16 * ts + n : M - 1;
#pragma unroll
            for (int gi = 0; gi < GW; ++gi)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    xa[gi][ts][u] = __builtin_bit_cast(h8_t, xq[(((int64_t)(g0 + gi) * 4 + u) * 4 + j) * Mp + m]);
        }
    }
    // Unconditional loads: tiles past the last re-read it, rows past N read row N - 1.
    auto load = [&](int64_t t, int q, MrSlot &sl) {
        t = t < my_tiles ? t : my_tiles - 1;
        int64_t row = (tb + t * TB) * 16 + n;
        row = row < N ? row : N - 1;
        const u32x4v_t *p = reinterpret_cast<const u32x4v_t *>(packed + row * W + (int64_t)(g0 + 4 * q + j) * kWordsPerGroup);
        sl.w[0] = p[0];
        sl.w[1] = p[1];
        sl.w[2] = p[2];
        sl.s = *reinterpret_cast<const u32x2v_t *>(scales + row * G + g0 + 4 * q);
    };
    MrSlot ring[4];
    __builtin_amdgcn_sched_barrier(0);
    load(0, 0, ring[0]);
    __builtin_amdgcn_sched_barrier(0);
    load(1 / NS, 1 % NS, ring[1]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XH) {
        // One exponent per token over the slice (the largest |x| over lanes
        // n, n + 8 and the four lane rows).  Each lane converts its 4 groups;
        // a DPP row rotation by 8 brings the other 4 from lane n ^ 8, so
        // every lane holds all 8 groups of token n % 8.
        uint32_t mx = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) mx = max(mx, absmax32(xh[k]));
        mx = max(mx, dpp_u32<0x128>(mx));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
        const int e = group_exponent(mx);
        const bool lo = n < 8;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t o[16];
            convert_block(xh[k], e, o);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint4 own = make_uint4(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3]);
                const uint4 oth = make_uint4(dpp_u32<0x128>(o[4 * u]), dpp_u32<0x128>(o[4 * u + 1]),
                                             dpp_u32<0x128>(o[4 * u + 2]), dpp_u32<0x128>(o[4 * u + 3]));
                xa[k][0][u] = __builtin_bit_cast(h8_t, lo ? own : oth);
                xa[4 + k][0][u] = __builtin_bit_cast(h8_t, lo ? oth : own);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) et[0][r] = __shfl(e, 4 * j + r);
    }

    const uint32_t magic = magic_vgpr();
    f4_t acc[TS];
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) acc[ts] = f4_t{0.f, 0.f, 0.f, 0.f};
    // Tile c0 + h: ring steps u = NS h + q.  UT tiles are one ring cycle, so
    // the loop runs whole cycles (its back edge always carries the same
    // pending loads, and the waits stay exact) and a ragged last cycle follows.
    auto tile = [&](int64_t c0, auto hc) __attribute__((always_inline)) {
        constexpr int h = decltype(hc)::value;
        const int64_t t = c0 + h;
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int u = NS * h + q;
            load(c0 + (u + 2) / NS, (u + 2) % NS, ring[(u + 2) & 3]);
            __builtin_amdgcn_sched_barrier(0);
            const MrSlot &sl = ring[u];
            uint32_t blk[4][3];
            const uint32_t wd[12] = {sl.w[0].x, sl.w[0].y, sl.w[0].z, sl.w[0].w, sl.w[1].x, sl.w[1].y,
                                     sl.w[1].z, sl.w[1].w, sl.w[2].x, sl.w[2].y, sl.w[2].z, sl.w[2].w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int d = 0; d < 3; ++d) blk[k][d] = wd[3 * k + d];
            quad_block_transpose(blk);  // blk[k] = block j of group g0 + 4q + k
            const uint32_t scw[2] = {sl.s.x, sl.s.y};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                h2_t qd[16];
                decode_block(blk[k][0], blk[k][1], blk[k][2], magic, qd);
                f4_t d[TS];
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) d[ts] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const h8_t bop = {qd[4 * v].x,     qd[4 * v].y,     qd[4 * v + 1].x, qd[4 * v + 1].y,
                                      qd[4 * v + 2].x, qd[4 * v + 2].y, qd[4 * v + 3].x, qd[4 * v + 3].y};
#pragma unroll
                    for (int ts = 0; ts < TS; ++ts)
                        d[ts] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[4 * q + k][ts][v], bop, d[ts], 0, 0, 0);
                }
                const uint32_t sw = scw[k >> 1];
                const float sv = __uint_as_float((k & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
#pragma unroll
                for (int ts = 0; ts < TS; ++ts)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[ts][r] = fmaf(d[ts][r], sv, acc[ts][r]);
            }
            if (q == NS - 1) {
                // Tile t done: its partials (times the activation exponents) to LDS.
                const int bt = (int)(t % kMrBatch);
                f4_t *rb = red + ((t / kMrBatch) & 1) * (kMrBatch * WAVES * TS * 64);
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[ts][r] = ldexpf(acc[ts][r], et[ts][r]);
                    rb[((bt * WAVES + wave) * TS + ts) * 64 + lane] = acc[ts];
                    acc[ts] = f4_t{0.f, 0.f, 0.f, 0.f};
                }
                if (bt == kMrBatch - 1 || t == my_tiles - 1) {
                    // One barrier per batch; the other half of `red` is written
                    // next, and the loads in flight stay in flight.
                    lds_barrier();
                    // (tile, token set, lane, r) outputs, a fixed number of
                    // passes: a data-dependent store count would leave the
                    // compiler unsure of the memory counter and make it over-wait.
                    const int outs = (bt + 1) * 256 * TS;
                    constexpr int kPasses = (kMrBatch * 256 * TS + 64 * WAVES - 1) / (64 * WAVES);
#pragma unroll
                    for (int ps = 0; ps < kPasses; ++ps) {
                        const int i = threadIdx.x + ps * 64 * WAVES;
                        const int tt = i / (256 * TS), ts = (i >> 8) % TS, l = (i >> 2) & 63, r = i & 3;
                        const int tok = 16 * ts + 4 * (l >> 4) + r;
                        const int64_t row = (tb + (t - bt + tt) * TB) * 16 + (l & 15);
                        if (i < outs && tok < M && row < N) {
                            const float *src = reinterpret_cast<const float *>(rb + (tt * WAVES * TS + ts) * 64 + l) + r;
                            float tot = src[0];
#pragma unroll
                            for (int w = 1; w < WAVES; ++w) tot += src[w * TS * 64 * 4];
                            y[(int64_t)tok * N + row] = tot;
                        }
                    }
                }
            }
        }
    };
    int64_t c0 = 0;
    for (; c0 + UT <= my_tiles; c0 += UT) static_for<UT>([&](auto hc) __attribute__((always_inline)) { tile(c0, hc); });
    static_for<UT - 1>([&](auto hc) __attribute__((always_inline)) {
        if (c0 + decltype(hc)::value < my_tiles) tile(c0, hc);
    });
}

// ------------------------------------- batched decode, up to four tokens ----
// The batch-1 matrix-core layout with the four tokens in place of its four
// super-step slots.  In super-step q lane (n, j) decodes group g0 + 4q + j of
// row n straight into the B operand (k chunk j), as in qgemv_mfma_kernel, so
// no transpose across lanes is needed.  A-operand set q has row m = 4t + j'
// carrying token t's activations of group g0 + 4q + j' in k chunk j' and zero
// elsewhere, so after the super-step's 16 MFMAs rows 4t .. 4t + 3 -- lane row
// t's registers -- hold token t's partial sums of the four groups, exactly
// apart.  A wave owns the 8 groups of one activation slice (two sets, 128
// VGPRs) and walks 16-row tiles through the ring of qgemm_mr_kernel; the
// waves' partials meet in LDS every kMrBatch tiles and are added in wave
// order.  The kernel converts the activations itself, with one exponent per
// token over the wave's slice (a conversion launch in front measured slower).
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void qgemm_m4_kernel(const uint16_t *__restrict__ x,
                                                            const uint32_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scales,
                                                            float *__restrict__ out, int M, int64_t N, int G, int C,
                                                            int64_t out_chunk) {
    constexpr int GW = 8, NS = 2, UT = 2;
    extern __shared__ __align__(16) unsigned char lds[];  // [2][kMrBatch][WAVES][64 lanes] floats
    float *red = reinterpret_cast<float *>(lds);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int j = lane >> 4;
    const int chunk = (int)(blockIdx.x % C);
    const int64_t tb = blockIdx.x / C, TB = gridDim.x / C;
    const int g0 = (chunk * WAVES + wave) * GW;
    const int64_t my_tiles = (((N + 15) >> 4) - tb + TB - 1) / TB;
    const int64_t W = (int64_t)G * kWordsPerGroup;
    float *y = out + (int64_t)chunk * out_chunk;

    // The bf16 activations straight from x, before the ring's loads: the
    // four lanes n = 4t .. 4t + 3 of lane row j share token t and group
    // g0 + 4q + j, and lane n reads block n % 4 of it (tokens past M read
    // token M - 1, whose rows of D are not stored).
    int et;
    h8_t xa[NS][16];
    uint4 xb[NS][4];
    {
        const int64_t K = (int64_t)G * kGroup;
        const int t = (n >> 2) < M ? (n >> 2) : M - 1;
#pragma unroll
        for (int q = 0; q < NS; ++q) load_x32(x + t * K + (int64_t)(g0 + 4 * q + j) * kGroup + 32 * (n & 3), xb[q]);
    }
    // Unconditional loads: tiles past the last re-read it, rows past N read row N - 1.
    auto load = [&](int64_t t, int q, MrSlot &sl) {
        t = t < my_tiles ? t : my_tiles - 1;
        int64_t row = (tb + t * TB) * 16 + n;
        row = row < N ? row : N - 1;
        const u32x4v_t *p = reinterpret_cast<const u32x4v_t *>(packed + row * W + (int64_t)(g0 + 4 * q + j) * kWordsPerGroup);
        sl.w[0] = p[0];
        sl.w[1] = p[1];
        sl.w[2] = p[2];
        sl.s = *reinterpret_cast<const u32x2v_t *>(scales + row * G + g0 + 4 * q);
    };
    MrSlot ring[4];
    __builtin_amdgcn_sched_barrier(0);
    load(0, 0, ring[0]);
    __builtin_amdgcn_sched_barrier(0);
    load(0, 1, ring[1]);
    __builtin_amdgcn_sched_barrier(0);
    {
        // One exponent per token over the wave's slice: the largest |x| over
        // the token's 4 x 4 lanes (the quad: the group's blocks; lane ^ 16
        // and lane ^ 32: its groups) maps to [2^14, 2^15).  Each lane
        // converts its block; the quad then hands all four blocks to its lane
        // n % 4 = j (a DPP broadcast per dword), the only one whose row takes
        // k chunk j: the other rows are zero.  Lane row j accumulates token
        // j, held by lane 4j.
        uint32_t mx = 0;
#pragma unroll
        for (int q = 0; q < NS; ++q) mx = max(mx, absmax32(xb[q]));
        mx = max(mx, dpp_u32<kDppQuadXor1>(mx));
        mx = max(mx, dpp_u32<kDppQuadXor2>(mx));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
        const int e = group_exponent(mx);
        const bool on = (n & 3) == j;
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            uint32_t o[16];
            convert_block(xb[q], e, o);
            static_for<4>([&](auto bc) __attribute__((always_inline)) {
                constexpr int b = decltype(bc)::value;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 f = make_uint4(dpp_u32<0x55 * b>(o[4 * v]), dpp_u32<0x55 * b>(o[4 * v + 1]),
                                               dpp_u32<0x55 * b>(o[4 * v + 2]), dpp_u32<0x55 * b>(o[4 * v + 3]));
                    xa[q][4 * b + v] = on ? __builtin_bit_cast(h8_t, f) : h8_t{0, 0, 0, 0, 0, 0, 0, 0};
                }
            });
        }
        et = __shfl(e, 4 * j);
    }

    const uint32_t magic = magic_vgpr();
    float acc = 0.f;
    // Tile c0 + h: ring steps u = 2h + q (UT tiles are one ring cycle).
    auto tile = [&](int64_t c0, auto hc) __attribute__((always_inline)) {
        constexpr int h = decltype(hc)::value;
        const int64_t t = c0 + h;
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int u = NS * h + q;
            load(c0 + (u + 2) / NS, (u + 2) % NS, ring[(u + 2) & 3]);
            __builtin_amdgcn_sched_barrier(0);
            const MrSlot &sl = ring[u];
            const uint32_t wd[12] = {sl.w[0].x, sl.w[0].y, sl.w[0].z, sl.w[0].w, sl.w[1].x, sl.w[1].y,
                                     sl.w[1].z, sl.w[1].w, sl.w[2].x, sl.w[2].y, sl.w[2].z, sl.w[2].w};
            f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                h2_t qd[16];
                decode_block(wd[3 * b], wd[3 * b + 1], wd[3 * b + 2], magic, qd);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const h8_t bop = {qd[4 * v].x,     qd[4 * v].y,     qd[4 * v + 1].x, qd[4 * v + 1].y,
                                      qd[4 * v + 2].x, qd[4 * v + 2].y, qd[4 * v + 3].x, qd[4 * v + 3].y};
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[q][4 * b + v], bop, d, 0, 0, 0);
                }
            }
            // d[r]: token j, group g0 + 4q + r of row n
            acc = fmaf(d[0], bf16_to_f32(sl.s.x & 0xFFFFu), acc);
            acc = fmaf(d[1], __uint_as_float(sl.s.x & 0xFFFF0000u), acc);
            acc = fmaf(d[2], bf16_to_f32(sl.s.y & 0xFFFFu), acc);
            acc = fmaf(d[3], __uint_as_float(sl.s.y & 0xFFFF0000u), acc);
            if (q == NS - 1) {
                const int bt = (int)(t % kMrBatch);
                float *rb = red + ((t / kMrBatch) & 1) * (kMrBatch * WAVES * 64);
                rb[(bt * WAVES + wave) * 64 + lane] = ldexpf(acc, et);
                acc = 0.f;
                if (bt == kMrBatch - 1 || t == my_tiles - 1) {
                    lds_barrier();
                    // (tile, lane) outputs in a fixed number of passes
                    const int outs = (bt + 1) * 64;
                    constexpr int kPasses = (kMrBatch * 64 + 64 * WAVES - 1) / (64 * WAVES);
#pragma unroll
                    for (int ps = 0; ps < kPasses; ++ps) {
                        const int i = threadIdx.x + ps * 64 * WAVES;
                        const int tt = i >> 6, l = i & 63;
                        const int tok = l >> 4;
                        const int64_t row = (tb + (t - bt + tt) * TB) * 16 + (l & 15);
                        if (i < outs && tok < M && row < N) {
                            const float *src = rb + tt * WAVES * 64 + l;
                            float tot = src[0];
#pragma unroll
                            for (int w = 1; w < WAVES; ++w) tot += src[w * 64];
                            y[(int64_t)tok * N + row] = tot;
                        }
                    }
                }
            }
        }
    };
    int64_t c0 = 0;
    for (; c0 + UT <= my_tiles; c0 += UT) static_for<UT>([&](auto hc) __attribute__((always_inline)) { tile(c0, hc); });
    if (c0 < my_tiles) tile(c0, std::integral_constant<int, 0>{});
}
template <int WAVES>
constexpr size_t m4_lds() { return (size_t)2 * kMrBatch * WAVES * 64 * sizeof(float); }

// --------------------------------------------------- prefill (large M) tiles --
// Many tokens: an MFMA GEMM whose B tiles are decoded on the fly.  Because a
// decoded weight is reused by every token of the tile, the group scale is
// folded into the decoded value instead of being applied per group after the
// MFMAs: B = (c-4) * 2^p * s * 2^-E[n], exact in fp16 (3 + 8 significant
// bits) with E[n] chosen per row so that the row's largest scale maps to
// [8, 16).  A = x * 2^-(E[m] + p) in fp16 with one exponent per token (largest
// |x| of the token maps to [2^14, 2^15); exact down to 2^-28 of it).  The
// accumulators then hold sum_k x w * 2^-(E[m] + E[n]), rescaled once at the
// end.  Tiles are 128 tokens x 128 rows x one group (128 k) per step, double
// buffered in LDS; each wave owns 64 x 64 of the output (16 MFMA tiles).
// LDS rows (256 bytes = 16 chunks of 16 bytes) are stored with chunk index
// XOR (row & 15) so that the 16 lanes of a quarter-wave reading one chunk of
// 16 consecutive rows hit 16 different bank groups.

// Per token: E[m] and x' = x * 2^-(E[m] + p) in block pair order, zero rows
// for m >= M.  One workgroup per token.
__global__ __launch_bounds__(256) void prep_tile_x_kernel(const uint16_t *__restrict__ x, uint32_t *__restrict__ xq,
                                                          int *__restrict__ xe, int M, int64_t K) {
    __shared__ uint32_t wmax[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t units = K / 32;
    uint32_t *dst = xq + (int64_t)m * (K / 2);
    if (m >= M) {
        for (int64_t u = tid; u < units; u += 256) {
            uint4 *d4 = reinterpret_cast<uint4 *>(dst + u * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) d4[i] = make_uint4(0, 0, 0, 0);
        }
        if (tid == 0) xe[m] = 0;
        return;
    }
    const uint16_t *src = x + (int64_t)m * K;
    uint32_t mx = 0;
    for (int64_t u = tid; u < units; u += 256) {
        uint4 xb[4];
        load_x32(src + u * 32, xb);
        mx = max(mx, absmax32(xb));
    }
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const int e = group_exponent(mx);
    for (int64_t u = tid; u < units; u += 256) {
        uint4 xb[4];
        load_x32(src + u * 32, xb);
        uint32_t out[16];
        convert_block(xb, e, out);
        uint4 *d4 = reinterpret_cast<uint4 *>(dst + u * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) d4[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    }
    if (tid == 0) xe[m] = e;
}

constexpr int kTileBM = 128;
constexpr int kTileBN = 128;
constexpr int kTileRow = 256;  // bytes of one row of one group (128 fp16)
constexpr size_t kTileStage = (size_t)(kTileBM + kTileBN) * kTileRow;
constexpr size_t kTileLds = 2 * kTileStage + (size_t)kTileBN * 4;

__device__ __forceinline__ int tile_off(int row, int chunk) { return row * kTileRow + ((chunk ^ (row & 15)) << 4); }

// One pipeline stage of the tile GEMM held in registers: this thread's share
// of a group's activations (8 x 16 B) and of its packed words and scales
// (two 12-byte blocks).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

struct TileStage {
    u32x4_t a[8];  // native vector type: stays in registers (HIP's uint4 struct copies did not)
    uint32_t w[6];
    uint32_t s[2];
};

__device__ __forceinline__ void tile_load(TileStage &st, const uint32_t *a_src, const uint32_t *const (&b_w)[2],
                                          const uint16_t *const (&b_s)[2], int g) {
    const u32x4_t *ap = reinterpret_cast<const u32x4_t *>(a_src + (int64_t)g * 64);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.a[i] = ap[i];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t *wp = b_w[h] + (int64_t)g * kWordsPerGroup;
        st.w[3 * h] = wp[0];
        st.w[3 * h + 1] = wp[1];
        st.w[3 * h + 2] = wp[2];
        st.s[h] = b_s[h][g];
    }
}

// Activations as they are; weights decoded to (c-4) * 2^p * s * 2^-E[row].
__device__ __forceinline__ void tile_store(const TileStage &st, unsigned char *sa, int a_row, int a_half, int tid,
                                           int b_blk, const int (&b_e)[2], uint32_t magic) {
    unsigned char *sb = sa + (size_t)kTileBM * kTileRow;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t *>(sa + tile_off(a_row, a_half * 8 + i)) = st.a[i];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        h2_t q[16];
        decode_block(st.w[3 * h], st.w[3 * h + 1], st.w[3 * h + 2], magic, q);
        const _Float16 sv = (_Float16)ldexpf(bf16_to_f32(st.s[h]), -b_e[h]);
        const h2_t s2 = {sv, sv};
        const int rl = h * 64 + (tid >> 2);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 v = make_uint4(__builtin_bit_cast(uint32_t, q[4 * c] * s2),
                                       __builtin_bit_cast(uint32_t, q[4 * c + 1] * s2),
                                       __builtin_bit_cast(uint32_t, q[4 * c + 2] * s2),
                                       __builtin_bit_cast(uint32_t, q[4 * c + 3] * s2));
            *reinterpret_cast<uint4 *>(sb + tile_off(rl, 4 * b_blk + c)) = v;
        }
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void qgemm_tile_kernel(const uint32_t *__restrict__ xq, const int *__restrict__ xe,
                                                       const uint32_t *__restrict__ packed,
                                                       const uint16_t *__restrict__ scales, float *__restrict__ y,
                                                       int M, int MT, int64_t N, int G) {
    extern __shared__ __align__(16) unsigned char lds[];
    int *En = reinterpret_cast<int *>(lds + 2 * kTileStage);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    // Token-tile major: the workgroups in flight together share one token
    // tile, which then stays in each XCD's L2 while the weight tiles stream.
    const int64_t NT = (N + kTileBN - 1) / kTileBN;
    const int m_tile = (int)(blockIdx.x / NT);
    const int64_t n_tile = blockIdx.x - (int64_t)m_tile * NT;
    const int64_t n0 = n_tile * kTileBN;
    const int m0 = m_tile * kTileBM;
    const int64_t K = (int64_t)G * kGroup;
    const int64_t W = (int64_t)G * kWordsPerGroup;

    // Row exponents: the largest scale of each row maps to [8, 16).
    if (tid < kTileBN) {
        int64_t r = n0 + tid;
        r = r < N ? r : N - 1;
        uint32_t mx = 0;
        for (int g = 0; g < G; ++g) mx = max(mx, (uint32_t)scales[r * G + g] & 0x7FFFu);
        En[tid] = __builtin_amdgcn_frexp_expf(bf16_to_f32(mx)) - 4;
    }
    __syncthreads();

    // Loader roles.  A: token tid/2, 64 fp16 (half a group row) = 8 x 16 B.
    // B: rows tid/4 and 64 + tid/4, block tid%4 (12 bytes each).
    const int a_row = tid >> 1, a_half = tid & 1;
    const uint32_t *a_src = xq + (int64_t)(m0 + a_row) * (K / 2) + a_half * 32;
    const int b_blk = tid & 3;
    int64_t b_r[2];
    int b_e[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int rl = h * 64 + (tid >> 2);
        int64_t r = n0 + rl;
        b_r[h] = r < N ? r : N - 1;
        b_e[h] = En[rl];
    }
    // Register ring of 3 stages: the operands of group g + 2 are loaded while
    // group g is multiplied and group g + 1 is decoded into LDS, so two steps
    // of latency are hidden.  Loads are unconditional (clamped to the last
    // group) and the barrier waits for LDS only, so the loads stay in flight.
    TileStage ring0, ring1, ring2;
    const uint32_t *b_w[2] = {packed + b_r[0] * W + 3 * b_blk, packed + b_r[1] * W + 3 * b_blk};
    const uint16_t *b_s[2] = {scales + b_r[0] * G, scales + b_r[1] * G};
    const uint32_t magic = magic_vgpr();
#define QW3_RING(k_) ((k_) == 0 ? ring0 : ((k_) == 1 ? ring1 : ring2))
#define QW3_TILE_LOAD(k_, g_) tile_load(QW3_RING(k_), a_src, b_w, b_s, (g_))
#define QW3_TILE_STORE(k_, buf_) \
    tile_store(QW3_RING(k_), lds + (size_t)(buf_) * kTileStage, a_row, a_half, tid, b_blk, b_e, magic)

    f4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = f4_t{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, lc = lane >> 4;
    auto mfma_group = [&](int buf) {
        const unsigned char *sa = lds + (size_t)buf * kTileStage;
        const unsigned char *sb = sa + (size_t)kTileBM * kTileRow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            h8_t av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[i] = *reinterpret_cast<const h8_t *>(sa + tile_off(wm * 64 + 16 * i + lr, 4 * ks + lc));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                bv[jj] = *reinterpret_cast<const h8_t *>(sb + tile_off(wn * 64 + 16 * jj + lr, 4 * ks + lc));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[i], bv[jj], acc[i][jj], 0, 0, 0);
        }
    };

    QW3_TILE_LOAD(0, 0);
    QW3_TILE_LOAD(1, (1 < G ? 1 : G - 1));
    QW3_TILE_STORE(0, 0);
    lds_barrier();
    // Step g: load g + 2 into slot (g + 2) % 3, multiply buffer g % 2, decode
    // slot (g + 1) % 3 into buffer (g + 1) % 2, barrier.  Unrolled by 3 so the
    // slots are static; steps past the last group only keep the pipeline shape.
#define QW3_TILE_STEP(u_)                                                                       \
    do {                                                                                        \
        const int g_ = g + (u_);                                                                \
        const int gl_ = g_ + 2 < G ? g_ + 2 : G - 1;                                            \
        QW3_TILE_LOAD(((u_) + 2) % 3, gl_);                                                     \
        if (g_ < G) mfma_group(g_ & 1);                                                         \
        QW3_TILE_STORE(((u_) + 1) % 3, (g_ + 1) & 1);                                           \
        lds_barrier();                                                                          \
    } while (0)
    for (int g = 0; g < G; g += 3) {
        QW3_TILE_STEP(0);
        QW3_TILE_STEP(1);
        QW3_TILE_STEP(2);
    }
#undef QW3_TILE_STEP

    // the exponents of the lane's 16 tokens, loaded together (past M: the last)
    int xt[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = m0 + wm * 64 + 16 * i + 4 * lc + r;
            xt[i][r] = xe[tok < M ? tok : M - 1];
        }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int nl = wn * 64 + 16 * jj + lr;
        const int64_t row = n0 + nl;
        const int en = En[nl];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = m0 + wm * 64 + 16 * i + 4 * lc + r;
                if (tok < M && row < N) y[(int64_t)tok * N + row] = ldexpf(acc[i][jj][r], en + xt[i][r]);
            }
        }
    }
}
#undef QW3_TILE_LOAD
#undef QW3_TILE_STORE
#undef QW3_RING

// ------------------------------------------ prefill, 256 x 256 output tiles --
// Larger tiles for the MFMA-bound case.  Eight waves, two per SIMD, each
// owning 128 tokens x 64 weight rows (32 MFMA tiles of 16 x 16, 128
// accumulators): while one wave of a SIMD decodes, the other's MFMAs run.  Per
// group (128 k) and k-step each wave decodes a quarter block of each of its
// rows straight into the B operand registers -- lane (n, j) decodes block j
// of row n of each 16-row sub-tile, exactly (c-4) * 2^p, times the
// row-normalised scale s * 2^-E[n] (exact in fp16) -- so only the activations
// go through LDS: each group's 256 x 128
// fp16 tile is copied in by buffer loads to LDS one group ahead (XOR-swizzled
// rows, double buffered in two separate arrays, two groups per loop
// iteration, so the compiler can tell that the copy in flight and the reads
// of the other stage are disjoint and overlaps the reads with the MFMAs).
// K may be split into C chunks whose partial sums are added by
// qgemm_chunk_sum_kernel.
// s_waitcnt immediate that constrains vmcnt only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

#ifndef QW3_PF_MIN_M
#define QW3_PF_MIN_M 129
#endif
constexpr int kPfBM = 256, kPfBN = 256;
constexpr size_t kPfStage = (size_t)kPfBM * kTileRow;  // 64 KB of activations per group

typedef unsigned u32x3_t __attribute__((ext_vector_type(3)));
typedef __attribute__((address_space(3))) void pf_lds_void_t;

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void qgemm_pf_kernel(
    const uint32_t *__restrict__ xq, const int *__restrict__ xe, const uint32_t *__restrict__ packed,
    const uint16_t *__restrict__ scales, float *__restrict__ out, int M, int MT, int64_t N, int G, int C,
    int64_t out_chunk) {
    constexpr int NI = 4;  // 16-row sub-tiles per wave
    // The two activation stages as separate arrays: the copy into one and the
    // reads from the other are then provably disjoint, so the compiler neither
    // drains the copy before a read nor needs the reads hidden in asm.
    __shared__ __align__(16) unsigned char stage_a[kPfStage], stage_b[kPfStage];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;  // token half, row quarter
    const int lr = lane & 15, lc = lane >> 4;
    const int64_t NT = (N + kPfBN - 1) / kPfBN;
    const int chunk = (int)(blockIdx.x / (NT * MT));
    const int64_t rest = blockIdx.x - (int64_t)chunk * NT * MT;
    const int m_tile = (int)(rest / NT);
    const int64_t n_tile = rest - (int64_t)m_tile * NT;
    const int64_t n0 = n_tile * kPfBN;
    const int m0 = m_tile * kPfBM;
    const int Gc = G / C;
    const int gbeg = chunk * Gc;
    const int64_t K = (int64_t)G * kGroup;
    const int64_t W = (int64_t)G * kWordsPerGroup;
    float *y = out + (int64_t)chunk * out_chunk;

    int64_t rows[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int64_t r = n0 + wn * 16 * NI + 16 * i + lr;
        rows[i] = r < N ? r : N - 1;
    }
    int en[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        uint32_t mx = 0;
        for (int g = gbeg + lc; g < gbeg + Gc; g += 4) mx = max(mx, (uint32_t)scales[rows[i] * G + g] & 0x7FFFu);
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
        en[i] = __builtin_amdgcn_frexp_expf(bf16_to_f32(mx)) - 4;
    }
    // 64 copy instructions per group, 8 per wave: instruction blk fills LDS
    // bytes [1024 blk, +1024) = rows 4 blk + lane/16, physical chunk lane%16.
    // The 8 copies go through a buffer descriptor over this tile's 256 token
    // rows of x' (256 K / 2 words, at most 32 MiB): each lane's byte offset is
    // fixed for the whole kernel and the group's is a scalar, so no vector
    // address register is written per copy.  (With 64-bit addresses the
    // compiler reused one address register for all 8 copies and, before
    // writing it again, waited for all of them.)
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(xq + (int64_t)m0 * (K / 2)), (short)0, (int)(kPfBM * K * 2), 0x00020000);
    uint32_t dma_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int blk = 8 * wave + i;
        const int r = 4 * blk + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        dma_off[i] = (uint32_t)((r * (K / 2) + 4 * c) * 4);
    }
    auto dma_a = [&](int g, unsigned char *base) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int blk = 8 * wave + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (pf_lds_void_t *)(base + (size_t)blk * 1024), 16, dma_off[i],
                                                     g * 256, 0, 0);
        }
    };
    uint32_t wcur[NI][3], wnext[NI][3], scur[NI], snext[NI];
    auto load_w = [&](int g, uint32_t (&w)[NI][3], uint32_t (&sc)[NI]) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const u32x3_t v = *reinterpret_cast<const u32x3_t *>(packed + rows[i] * W + (int64_t)g * kWordsPerGroup + 3 * lc);
            w[i][0] = v.x;
            w[i][1] = v.y;
            w[i][2] = v.z;
            sc[i] = scales[rows[i] * G + g];
        }
    };
    f4_t acc[8][NI];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int i = 0; i < NI; ++i) acc[mi][i] = f4_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t magic = magic_vgpr();

    // Group g: A from `abuf`; the next group's copies go to `nbuf`.
    auto group = [&](int g, const unsigned char *abuf, unsigned char *nbuf) __attribute__((always_inline)) {
        const bool more = g + 1 < gbeg + Gc;
        const int gn = more ? g + 1 : g;
        // This group's scales first: converting them after the next group's
        // loads are issued made the compiler drain those loads first.
        h2_t sc2[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const _Float16 sv = (_Float16)ldexpf(bf16_to_f32(scur[i]), -en[i]);
            sc2[i] = h2_t{sv, sv};
            asm volatile("" : "+v"(sc2[i]));  // computed here, not sunk past the copies
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) dma_a(gn, nbuf);
        load_w(gn, wnext, snext);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            h8_t a[8];
#pragma unroll
            for (int mi = 0; mi < 8; ++mi)
                a[mi] = *reinterpret_cast<const h8_t *>(abuf + tile_off(wm * 128 + 16 * mi + lr, 4 * lc + u));
            h8_t bop[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                h2_t qd[4];
                decode_quarter(u, wcur[i][0], wcur[i][1], wcur[i][2], magic, qd);
                const h2_t p0 = qd[0] * sc2[i], p1 = qd[1] * sc2[i], p2 = qd[2] * sc2[i], p3 = qd[3] * sc2[i];
                bop[i] = h8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
            }
#pragma unroll
            for (int mi = 0; mi < 8; ++mi)
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    acc[mi][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mi], bop[i], acc[mi][i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            scur[i] = snext[i];
#pragma unroll
            for (int d = 0; d < 3; ++d) wcur[i][d] = wnext[i][d];
        }
        // the next group's copies have landed and every wave is done with abuf
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_barrier();
        // the copies' lane offsets stay in their registers for the next group
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(dma_off[i]));
    };

    dma_a(gbeg, stage_a);
    load_w(gbeg, wcur, scur);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    // two groups per iteration, so each one's stage is a fixed array
    for (int g = gbeg; g < gbeg + Gc; g += 2) {
        group(g, stage_a, stage_b);
        if (g + 1 < gbeg + Gc) group(g + 1, stage_b, stage_a);
    }
    // The exponents of the lane's 32 tokens, loaded together (tokens past M
    // read the last one): loaded next to each store, every store waited for
    // its own load.
    int xt[8][4];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = m0 + wm * 128 + 16 * mi + 4 * lc + r;
            xt[mi][r] = xe[tok < M ? tok : M - 1];
        }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int64_t row = n0 + wn * 16 * NI + 16 * i + lr;
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = m0 + wm * 128 + 16 * mi + 4 * lc + r;
                if (tok < M && row < N) y[(int64_t)tok * N + row] = ldexpf(acc[mi][i][r], en[i] + xt[mi][r]);
            }
        }
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

// Device workspace of the batched-decode and prefill paths (converted
// activations, K-chunk partial sums): one buffer per (device, stream), kept
// until the process ends and grown to the largest request.  Work on one
// stream runs in order, so the calls on that stream share its buffer; other
// streams get their own.  A stream-ordered allocation and release per call
// measured several microseconds per call; this costs nothing after the first
// call of a size.  Growing synchronizes the stream first (the old buffer may
// still be read by queued work), so under graph capture make one call of the
// same size beforehand.
struct Workspace {
    int dev;
    hipStream_t stream;
    void *ptr;
    size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;

qw3_status workspace(hipStream_t stream, size_t bytes, void **out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err);
    bytes = (bytes + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);  // whole MiB: fewer regrowths
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace *w = nullptr;
    for (auto &e : g_ws)
        if (e.dev == dev && e.stream == stream) w = &e;
    if (w && w->bytes >= bytes) {
        *out = w->ptr;
        return QW3_OK;
    }
    if (w) {
        err = hipStreamSynchronize(stream);
        if (err == hipSuccess) err = hipFree(w->ptr);
        if (err != hipSuccess) return hip_fail(err);
        w->ptr = nullptr;
        w->bytes = 0;
    } else {
        g_ws.push_back(Workspace{dev, stream, nullptr, 0});
        w = &g_ws.back();
    }
    err = hipMalloc(&w->ptr, bytes);
    if (err != hipSuccess) {
        w->ptr = nullptr;
        return hip_fail(err);
    }
    w->bytes = bytes;
    *out = w->ptr;
    return QW3_OK;
}

qw3_status fill_zero(float *y, int64_t n, hipStream_t stream) {
    if (n == 0) return QW3_OK;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, y, n);
    return check_launch();
}

// Workgroups of `kernel` that fit on one CU at `wgs` threads and `lds` bytes.
qw3_status blocks_per_cu(const void *kernel, int wgs, size_t lds, int *out) {
    int nb = 0;
    const hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, wgs, lds);
    if (err != hipSuccess) return hip_fail(err);
    *out = nb > 0 ? nb : 1;
    return QW3_OK;
}

#ifndef QW3_GEMV_BPC
#define QW3_GEMV_BPC 1
#endif
template <int T, bool MULTI>
qw3_status launch_gemv_small(const uint16_t *x, GemvSegs sg, int count, int G, hipStream_t stream) {
    constexpr int R = kGemvWGS / T;
    const size_t xs_bytes = (size_t)G * 64 * 4 + (size_t)G * 4;
    const bool lds_x = xs_bytes <= kMaxLdsX;
    const size_t lds = lds_x ? xs_bytes : 0;
    const void *kern = reinterpret_cast<const void *>(&qgemv_small_kernel<T, MULTI, kGemvDepth>);
    int cus = 0, per_cu = 0;
    qw3_status st = cu_count(&cus);
    if (st == QW3_OK) st = blocks_per_cu(kern, kGemvWGS, lds, &per_cu);
    if (st != QW3_OK) return st;
    if (QW3_GEMV_BPC > 0 && per_cu > QW3_GEMV_BPC) per_cu = QW3_GEMV_BPC;
    const int64_t budget = (int64_t)cus * per_cu;
    int64_t tot = 0;
    for (int i = 0; i < count; ++i) tot += sg.rows[i];
    // Workgroups per matrix: in proportion to its rows (rounded down, so the
    // total stays within one workgroup per CU), at least one for a non-empty
    // matrix, at most one per R rows.
    int64_t blocks = 0;
    for (int i = 0; i < kMaxSegs; ++i) {
        int64_t b = 0;
        if (i < count && sg.rows[i] > 0) {
            b = budget * sg.rows[i] / tot;
            const int64_t cap = ceil_div(sg.rows[i], R);
            b = b < 1 ? 1 : (b > cap ? cap : b);
        }
        blocks += b;
        sg.blk_end[i] = (int)blocks;
    }
    // Waves with at most two rows each keep one row in flight instead of
    // kGemvDepth (deeper rings would only re-read the last row).
    const int64_t rows_per_wave = ceil_div(tot, blocks * R);
    if (rows_per_wave <= 2)
        hipLaunchKernelGGL((qgemv_small_kernel<T, MULTI, 1>), dim3((unsigned)blocks), dim3(kGemvWGS), lds, stream, x,
                           sg, G, lds_x ? 1 : 0);
    else
        hipLaunchKernelGGL((qgemv_small_kernel<T, MULTI, kGemvDepth>), dim3((unsigned)blocks), dim3(kGemvWGS), lds,
                           stream, x, sg, G, lds_x ? 1 : 0);
    return check_launch();
}

template <bool MULTI>
qw3_status launch_gemv_small_any(const uint16_t *x, const GemvSegs &sg, int count, int G, hipStream_t stream) {
    if (G <= 1) return launch_gemv_small<1, MULTI>(x, sg, count, G, stream);
    if (G <= 2) return launch_gemv_small<2, MULTI>(x, sg, count, G, stream);
    if (G <= 4) return launch_gemv_small<4, MULTI>(x, sg, count, G, stream);
    if (G <= 8) return launch_gemv_small<8, MULTI>(x, sg, count, G, stream);
    if (G <= 16) return launch_gemv_small<16, MULTI>(x, sg, count, G, stream);
    if (G <= 32) return launch_gemv_small<32, MULTI>(x, sg, count, G, stream);
    return launch_gemv_small<64, MULTI>(x, sg, count, G, stream);
}

qw3_status launch_gemv_big(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                           int64_t N, int G, hipStream_t stream) {
    // Team of T >= G lanes, T a multiple of 32; the workgroup holds whole
    // waves and at most 1024 threads (T <= 1024 since K <= QW3_MAX_K).
    int T = 32 * ((G + 31) / 32);
    int R = T >= 512 ? 1 : 512 / T;
    int wgs = T * R;
    if (wgs % 64 != 0) {
        if (2 * wgs <= 1024) {
            R *= 2;
            wgs *= 2;
        } else {
            T = 64 * ((G + 63) / 64);
            R = 1;
            wgs = T;
        }
    }
    const size_t xs_bytes = (size_t)G * 64 * 4 + (size_t)G * 4;
    const bool lds_x = xs_bytes <= kMaxLdsX;
    constexpr int kBigD = kGemvDepth, kHugeD = 1;
    const size_t red_bytes = 2 * (size_t)((wgs <= 512 ? kBigD : kHugeD) + 1) * (wgs / 32) * sizeof(float);
    const size_t lds = (lds_x && xs_bytes > red_bytes) ? xs_bytes : red_bytes;
    const void *kern =
        wgs <= 512 ? (lds_x ? reinterpret_cast<const void *>(&qgemv_big_kernel<512, kBigD, true>)
                            : reinterpret_cast<const void *>(&qgemv_big_kernel<512, kBigD, false>))
                   : (lds_x ? reinterpret_cast<const void *>(&qgemv_big_kernel<1024, kHugeD, true>)
                            : reinterpret_cast<const void *>(&qgemv_big_kernel<1024, kHugeD, false>));
    int cus = 0, per_cu = 0;
    qw3_status st = cu_count(&cus);
    if (st == QW3_OK) st = blocks_per_cu(kern, wgs, lds, &per_cu);
    if (st != QW3_OK) return st;
    int64_t blocks = ceil_div(N, R);
    if (blocks > (int64_t)cus * per_cu) blocks = (int64_t)cus * per_cu;
    hipLaunchKernelGGL(reinterpret_cast<void (*)(const uint16_t *, const uint32_t *, const uint16_t *, float *,
                                                 int64_t, int, int)>(const_cast<void *>(kern)),
                       dim3((unsigned)blocks), dim3(wgs), lds, stream, x, packed, scales, y, N, G, T);
    return check_launch();
}

// The matrix-core GEMV: one workgroup per CU, workgroups dealt to the
// matrices in proportion to their 16-row tiles, at least one and at most one
// per tile each (4 waves x 16 groups at K = 8192).
#ifndef QW3_GEMV_MFMA
#define QW3_GEMV_MFMA 1
#endif
template <int GPW, int WAVES, bool MULTI>
qw3_status launch_gemv_mfma(const uint16_t *x, GemvSegs sg, int count, hipStream_t stream) {
    int cus = 0;
    const qw3_status st = cu_count(&cus);
    if (st != QW3_OK) return st;
    int64_t tiles[kMaxSegs], tot = 0;
    for (int i = 0; i < kMaxSegs; ++i) {
        tiles[i] = i < count ? ceil_div(sg.rows[i], 16) : 0;
        tot += tiles[i];
    }
    int64_t blocks = 0;
    for (int i = 0; i < kMaxSegs; ++i) {
        int64_t b = 0;
        if (tiles[i] > 0) {
            b = (int64_t)kMfPerCu * cus * tiles[i] / tot;
            b = b < 1 ? 1 : (b > tiles[i] ? tiles[i] : b);
        }
        blocks += b;
        sg.blk_end[i] = (int)blocks;
    }
    const size_t lds = mf_lds<GPW, WAVES>();
    hipLaunchKernelGGL((qgemv_mfma_kernel<GPW, WAVES, MULTI>), dim3((unsigned)blocks), dim3(64 * WAVES), lds, stream,
                       x, sg);
    return check_launch();
}

// Whether the matrix-core GEMV takes a matrix: K = 8192, scale rows 8-byte
// aligned (8-byte scale loads) and at least four 16-row tiles per CU (with
// fewer it is no faster than the lane-per-group kernel).  At K = 28672
// (7 waves x 32 groups) it measured no faster than qgemv_big_kernel on the
// 8192-row down projection, two tiles per CU, so it is not used there.  The
// choice depends on the matrix alone, so a matrix gets the same kernel -- and
// the same bits -- from qgemv_w3g128 and from qgemv_w3g128_multi.
bool gemv_mfma_takes(int G, const uint16_t *scales, int64_t N) {
    if (!QW3_GEMV_MFMA || G != 64 || N == 0 || !aligned(scales, 8)) return false;
    int cus = 0;
    if (cu_count(&cus) != QW3_OK) return false;
    return ceil_div(N, 16) >= 4 * (int64_t)cus;
}

qw3_status launch_gemv(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                       int64_t N, int64_t K, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    if (G <= 64) {
        GemvSegs sg = {};
        sg.packed[0] = packed;
        sg.scales[0] = scales;
        sg.y[0] = y;
        sg.rows[0] = N;
        if (gemv_mfma_takes(G, scales, N)) return launch_gemv_mfma<16, 4, false>(x, sg, 1, stream);
        return launch_gemv_small_any<false>(x, sg, 1, G, stream);
    }
    return launch_gemv_big(x, packed, scales, y, N, G, stream);
}

// Several matrices sharing x: one launch when rows fit one wave (K <= 8192),
// else one launch per matrix.
qw3_status launch_gemv_multi(const uint16_t *x, int count, const uint32_t *const *packed,
                             const uint16_t *const *scales, float *const *y, const int64_t *N, int64_t K,
                             hipStream_t stream) {
    const int G = (int)(K / kGroup);
    if (G > 64) {
        for (int i = 0; i < count; ++i) {
            if (N[i] == 0) continue;
            const qw3_status st = launch_gemv(x, packed[i], scales[i], y[i], N[i], K, stream);
            if (st != QW3_OK) return st;
        }
        return QW3_OK;
    }
    // The matrices the matrix-core kernel takes go in one launch, the others
    // in one launch of the lane-per-group kernel.
    for (int pass = 0; pass < 2; ++pass) {
        GemvSegs sg = {};
        int cnt = 0;
        for (int i = 0; i < count; ++i) {
            if (N[i] == 0 || gemv_mfma_takes(G, scales[i], N[i]) != (pass == 0)) continue;
            sg.packed[cnt] = packed[i];
            sg.scales[cnt] = scales[i];
            sg.y[cnt] = y[i];
            sg.rows[cnt] = N[i];
            ++cnt;
        }
        if (cnt == 0) continue;
        for (int i = cnt; i < kMaxSegs; ++i) {
            sg.packed[i] = sg.packed[cnt - 1];
            sg.scales[i] = sg.scales[cnt - 1];
            sg.y[i] = sg.y[cnt - 1];
            sg.rows[i] = 0;
        }
        const qw3_status st = pass == 0 ? launch_gemv_mfma<16, 4, true>(x, sg, cnt, stream)
                                        : launch_gemv_small_any<true>(x, sg, cnt, G, stream);
        if (st != QW3_OK) return st;
    }
    return QW3_OK;
}

// Prefill: convert x once (per-token exponent), then one tile GEMM launch.
qw3_status launch_gemm_tile(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int MT = (int)ceil_div(M, kTileBM);
    const int64_t Mp = (int64_t)MT * kTileBM;
    const size_t xq_bytes = (size_t)Mp * (size_t)K * 2;
    const size_t xe_bytes = (size_t)Mp * sizeof(int);
    void *scratch = nullptr;
    {
        const qw3_status ws = workspace(stream, xq_bytes + xe_bytes, &scratch);
        if (ws != QW3_OK) return ws;
    }
    uint32_t *xq = reinterpret_cast<uint32_t *>(scratch);
    int *xe = reinterpret_cast<int *>(static_cast<char *>(scratch) + xq_bytes);
    hipLaunchKernelGGL(prep_tile_x_kernel, dim3((unsigned)Mp), dim3(256), 0, stream, x, xq, xe, (int)M, K);
    qw3_status st = check_launch();
    if (st == QW3_OK) {
        const int64_t blocks = ceil_div(N, kTileBN) * MT;
        hipLaunchKernelGGL(qgemm_tile_kernel, dim3((unsigned)blocks), dim3(256), kTileLds, stream, xq, xe, packed,
                           scales, y, (int)M, MT, N, G);
        st = check_launch();
    }
    return st;
}

// Prefill on 256 x 256 tiles: convert x once (per-token exponent), one tile
// launch (K split into C chunks when the tiles alone would not fill the
// GPU), and a chunk sum.
qw3_status launch_gemm_pf(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int MT = (int)ceil_div(M, kPfBM);
    const int64_t NT = ceil_div(N, kPfBN);
    int cus = 0;
    qw3_status st = cu_count(&cus);
    if (st != QW3_OK) return st;
    int C = 1;
    while (NT * MT * C * 2 <= cus && G % (2 * C) == 0) C *= 2;
    const int64_t Mp = (int64_t)MT * kPfBM;
    const size_t xq_bytes = (size_t)Mp * (size_t)K * 2;
    const size_t xe_bytes = ((size_t)Mp * sizeof(int) + 255) / 256 * 256;
    const size_t part_bytes = C > 1 ? (size_t)C * (size_t)M * (size_t)N * sizeof(float) : 0;
    void *scratch = nullptr;
    {
        const qw3_status ws = workspace(stream, xq_bytes + xe_bytes + part_bytes, &scratch);
        if (ws != QW3_OK) return ws;
    }
    uint32_t *xq = reinterpret_cast<uint32_t *>(scratch);
    int *xe = reinterpret_cast<int *>(static_cast<char *>(scratch) + xq_bytes);
    float *part = reinterpret_cast<float *>(static_cast<char *>(scratch) + xq_bytes + xe_bytes);
    hipLaunchKernelGGL(prep_tile_x_kernel, dim3((unsigned)Mp), dim3(256), 0, stream, x, xq, xe, (int)M, K);
    st = check_launch();
    if (st == QW3_OK) {
        float *dst = C > 1 ? part : y;
        hipLaunchKernelGGL(qgemm_pf_kernel, dim3((unsigned)(NT * MT * C)), dim3(512), 0, stream, xq, xe, packed,
                           scales, dst, (int)M, MT, N, G, C, (int64_t)M * N);
        st = check_launch();
    }
    if (st == QW3_OK && C > 1) {
        const int64_t count = M * N;
        hipLaunchKernelGGL(qgemm_chunk_sum_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, stream, part, y,
                           count, C, count);
        st = check_launch();
    }
    return st;
}

// Batched decode from registers (tokens <= 16 per pass), K in chunks of
// WAVES x 8 groups.
#ifndef QW3_MT_RING
#define QW3_MT_RING 1
#endif
#ifndef QW3_MR_XH
#define QW3_MR_XH 1
#endif
// TS = 1: passes of up to 16 tokens, through the ring kernel when the scale
// rows are 8-byte aligned (it reads 8 bytes of scales at a time), else
// through qgemm_mt_kernel (2 bytes at a time).  TS = 2: 17..32 tokens in one
// pass of the ring kernel (two sets of 16 per decoded block, 4 groups per
// wave), scale rows 8-byte aligned.
template <int WAVES, int TS>
qw3_status launch_gemm_mt(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const bool ring = TS == 2 || (QW3_MT_RING && aligned(scales, 8));
    constexpr int Mp = 16 * TS;
    const int C = G / ((8 / TS) * WAVES);
    // Up to 6 tokens: the ring kernel converts the activations itself (at 8
    // it measured the same as the conversion launch).
    const bool xh = QW3_MR_XH && ring && TS == 1 && M <= 6;
    const size_t xq_bytes = xh ? 0 : (size_t)Mp * (size_t)K * 2;
    const size_t xe_bytes = xh ? 0 : ((size_t)(G / 8) * Mp * sizeof(int16_t) + 255) / 256 * 256;
    const size_t part_bytes = C > 1 ? (size_t)C * Mp * (size_t)N * sizeof(float) : 0;
    const void *kern = xh     ? reinterpret_cast<const void *>(&qgemm_mr_kernel<WAVES, TS, TS == 1>)
                       : ring ? reinterpret_cast<const void *>(&qgemm_mr_kernel<WAVES, TS, false>)
                              : reinterpret_cast<const void *>(&qgemm_mt_kernel<WAVES>);
    const size_t lds = ring ? mr_lds<WAVES, TS>() : 0;
    int cus = 0, per_cu = 0;
    qw3_status st = cu_count(&cus);
    if (st == QW3_OK) st = blocks_per_cu(kern, 64 * WAVES, lds, &per_cu);
    if (st != QW3_OK) return st;
    void *scratch = nullptr;
    if (xq_bytes + xe_bytes + part_bytes > 0) {
        const qw3_status ws = workspace(stream, xq_bytes + xe_bytes + part_bytes, &scratch);
        if (ws != QW3_OK) return ws;
    }
    uint4 *xq = reinterpret_cast<uint4 *>(scratch);
    int16_t *xe = reinterpret_cast<int16_t *>(static_cast<char *>(scratch) + xq_bytes);
    float *part = reinterpret_cast<float *>(static_cast<char *>(scratch) + xq_bytes + xe_bytes);
    const int64_t tiles = ceil_div(N, 16);
    int64_t tb = (int64_t)cus * per_cu / C;
    if (tb < 1) tb = 1;
    if (tb > tiles) tb = tiles;
    for (int64_t m0 = 0; m0 < M && st == QW3_OK; m0 += Mp) {
        const int mc = (int)(M - m0 < Mp ? M - m0 : Mp);
        if (!xh) {
            const int64_t units = (int64_t)(G / 8) * Mp * 32;
            hipLaunchKernelGGL(prep_x_slice_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, stream,
                               x + m0 * K, xq, xe, mc, Mp, K, G / 8);
            st = check_launch();
            if (st != QW3_OK) break;
        }
        float *dst = C > 1 ? part : y + m0 * N;
        if (xh)
            hipLaunchKernelGGL((qgemm_mr_kernel<WAVES, TS, TS == 1>), dim3((unsigned)(tb * C)), dim3(64 * WAVES), lds,
                               stream, xq, xe, x + m0 * K, packed, scales, dst, mc, N, G, C, (int64_t)Mp * N);
        else if (ring)
            hipLaunchKernelGGL((qgemm_mr_kernel<WAVES, TS, false>), dim3((unsigned)(tb * C)), dim3(64 * WAVES), lds,
                               stream, xq, xe, x + m0 * K, packed, scales, dst, mc, N, G, C, (int64_t)Mp * N);
        else
            hipLaunchKernelGGL(qgemm_mt_kernel<WAVES>, dim3((unsigned)(tb * C)), dim3(64 * WAVES), 0, stream, xq, xe,
                               packed, scales, dst, mc, N, G, C, (int64_t)Mp * N);
        st = check_launch();
        if (st != QW3_OK || C == 1) continue;
        const int64_t count = (int64_t)mc * N;
        hipLaunchKernelGGL(qgemm_chunk_sum_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, stream, part,
                           y + m0 * N, count, C, (int64_t)Mp * N);
        st = check_launch();
    }
    return st;
}

// Up to four tokens: qgemm_m4_kernel, WAVES x 8 groups per K chunk (scale
// rows 8-byte aligned).
#ifndef QW3_GEMM_M4
#define QW3_GEMM_M4 1
#endif
template <int WAVES>
qw3_status launch_gemm_m4(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream) {
    constexpr int Mp = 4;  // token slots of the partial sums
    const int G = (int)(K / kGroup);
    const int C = G / (8 * WAVES);
    const size_t part_bytes = C > 1 ? (size_t)C * Mp * (size_t)N * sizeof(float) : 0;
    const size_t lds = m4_lds<WAVES>();
    int cus = 0, per_cu = 0;
    qw3_status st = cu_count(&cus);
    if (st == QW3_OK)
        st = blocks_per_cu(reinterpret_cast<const void *>(&qgemm_m4_kernel<WAVES>), 64 * WAVES, lds, &per_cu);
    if (st != QW3_OK) return st;
    float *part = nullptr;
    if (part_bytes > 0) {
        void *scratch = nullptr;
        st = workspace(stream, part_bytes, &scratch);
        if (st != QW3_OK) return st;
        part = static_cast<float *>(scratch);
    }
    const int64_t tiles = ceil_div(N, 16);
    int64_t tb = (int64_t)cus * per_cu / C;
    if (tb < 1) tb = 1;
    if (tb > tiles) tb = tiles;
    hipLaunchKernelGGL(qgemm_m4_kernel<WAVES>, dim3((unsigned)(tb * C)), dim3(64 * WAVES), lds, stream, x, packed,
                       scales, C > 1 ? part : y, (int)M, N, G, C, (int64_t)Mp * N);
    st = check_launch();
    if (st != QW3_OK || C == 1) return st;
    const int64_t count = M * N;
    hipLaunchKernelGGL(qgemm_chunk_sum_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, stream, part, y,
                       count, C, (int64_t)Mp * N);
    return check_launch();
}

// Small-M path: convert x once into scratch, then one streaming pass over W
// per chunk of up to 32 tokens.
qw3_status launch_gemm_small(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    if (M > 32) {
        if (M >= QW3_PF_MIN_M) return launch_gemm_pf(x, packed, scales, y, M, N, K, stream);
        return launch_gemm_tile(x, packed, scales, y, M, N, K, stream);
    }
    // Batched decode: 17..32 tokens in one pass when the scale rows allow the
    // ring kernel (chunks of 8 waves x 4 groups); otherwise passes of up to
    // 16 tokens in chunks of 8 waves x 8 groups (or 7 x 8 when K = 28672).
    if (M <= 4 && QW3_GEMM_M4 && aligned(scales, 8)) {
        if (G % 64 == 0) return launch_gemm_m4<8>(x, packed, scales, y, M, N, K, stream);
        if (G % 56 == 0) return launch_gemm_m4<7>(x, packed, scales, y, M, N, K, stream);
    }
    if (M > 16 && QW3_MT_RING && aligned(scales, 8) && G % 32 == 0)
        return launch_gemm_mt<8, 2>(x, packed, scales, y, M, N, K, stream);
    if (G % 64 == 0) return launch_gemm_mt<8, 1>(x, packed, scales, y, M, N, K, stream);
    if (G % 56 == 0) return launch_gemm_mt<7, 1>(x, packed, scales, y, M, N, K, stream);
    const int mchunk = M > 16 ? 32 : 16;
    const size_t xq_bytes = (size_t)mchunk * (size_t)K * 2;
    const size_t xe_bytes = (size_t)G * mchunk * sizeof(int16_t);
    void *scratch = nullptr;
    {
        const qw3_status ws = workspace(stream, xq_bytes + xe_bytes, &scratch);
        if (ws != QW3_OK) return ws;
    }
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
    const int64_t blocks = ceil_div(units, 256);
    hipLaunchKernelGGL(qpack_kernel, dim3((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20))), dim3(256), 0,
                       (hipStream_t)hip_stream, codes, reinterpret_cast<uint32_t *>(packed), units);
    return check_launch();
}

qw3_status qrepack_w4c_uint3(const int32_t *w4, int32_t *packed, int64_t N, int64_t K, void *hip_stream) {
    qw3_status st = check_shape(N, K);
    if (st != QW3_OK) return st;
    if (N == 0 || K == 0) return QW3_OK;
    if (!w4 || !packed) return QW3_ERR_NULL;
    if (!aligned(w4, 16) || !aligned(packed, 16)) return QW3_ERR_ALIGN;
    const int64_t units = N * (K / kGroup);
    const int64_t blocks = ceil_div(units, 256);
    hipLaunchKernelGGL(qrepack_w4c_kernel, dim3((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20))), dim3(256), 0,
                       (hipStream_t)hip_stream, reinterpret_cast<const uint32_t *>(w4),
                       reinterpret_cast<uint32_t *>(packed), units);
    return check_launch();
}

qw3_status qdequant_bf16(const int32_t *packed, const uint16_t *scales, uint16_t *w_out, int64_t N, int64_t K,
                         void *hip_stream) {
    qw3_status st = check_shape(N, K);
    if (st != QW3_OK) return st;
    if (N == 0 || K == 0) return QW3_OK;
    if (!packed || !scales || !w_out) return QW3_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(w_out, 16) || !aligned(scales, 2)) return QW3_ERR_ALIGN;
    const int64_t chunks = N * (K / kGroup) * 16;  // 8 weights each
    const int64_t blocks = ceil_div(chunks, 256);
    hipLaunchKernelGGL(qdequant_kernel, dim3((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20))), dim3(256), 0,
                       (hipStream_t)hip_stream, reinterpret_cast<const uint32_t *>(packed), scales, w_out, chunks);
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

qw3_status qgemv_w3g128_multi(const uint16_t *x, int32_t count, const int32_t *const *packed,
                              const uint16_t *const *scales, float *const *y, const int64_t *N, int64_t K,
                              void *hip_stream) {
    if (count < 1 || count > QW3_MAX_MULTI) return QW3_ERR_SHAPE;
    if (!packed || !scales || !y || !N) return QW3_ERR_NULL;
    int64_t tot = 0;
    for (int i = 0; i < count; ++i) {
        const qw3_status st = check_shape(N[i], K);
        if (st != QW3_OK) return st;
        tot += N[i];
    }
    if (tot == 0) return QW3_OK;
    for (int i = 0; i < count; ++i) {
        if (N[i] == 0) continue;
        if (!y[i]) return QW3_ERR_NULL;
        if (!aligned(y[i], 4)) return QW3_ERR_ALIGN;
        if (K == 0) continue;
        if (!packed[i] || !scales[i]) return QW3_ERR_NULL;
        if (!aligned(packed[i], 16) || !aligned(scales[i], 2)) return QW3_ERR_ALIGN;
    }
    if (K == 0) {
        for (int i = 0; i < count; ++i) {
            if (N[i] == 0) continue;
            const qw3_status st = fill_zero(y[i], N[i], (hipStream_t)hip_stream);
            if (st != QW3_OK) return st;
        }
        return QW3_OK;
    }
    if (!x) return QW3_ERR_NULL;
    if (!aligned(x, 16)) return QW3_ERR_ALIGN;
    return launch_gemv_multi(x, count, reinterpret_cast<const uint32_t *const *>(packed), scales, y, N, K,
                             (hipStream_t)hip_stream);
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
