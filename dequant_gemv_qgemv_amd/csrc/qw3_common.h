#pragma once
// W3G128 fused dequantize-and-multiply for gfx950 (CDNA4): what every kernel
// of the library (C ABI in include/qw3.h) shares -- the format, the decode,
// the activation conversion and the exactness guard -- and the host helpers
// its two translation units share (qw3_gemv.hip: the batch-1 kernels;
// qw3.hip: everything else and the C ABI).
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
// Activations.  x is bf16; the products use fp16 operands, so each exponent
// set (a group of 128 activations at batch 1, an 8-group slice of a token in
// batched decode, a whole token in the prefill kernel) is scaled by a power of
// two 2^-e that brings its largest magnitude into [2^14, 2^15), each element
// by its slot's 2^-p (p <= 7), and rounded to fp16.  bf16 has 8 significant
// bits and fp16 11, so every element of magnitude at least 2^(e-7) lands in
// the fp16 normal range and converts exactly; 2^e is multiplied back in fp32
// together with the weight scale.  Those products are exact and only the fp32
// accumulation rounds.
//
// Exactness guard.  Smaller elements (about 2^21 or more below the largest of
// their set) may be rounded or flushed.  The conversion sums their magnitudes
// per (token, group) into D, which bounds what they can change in any output:
// |sum_k w_k (x_k - x'_k)| <= 4 sum_g |s_g| D_g.  When some D is non-zero a
// pass after the fast loop (fixup_outputs) evaluates that bound for every
// output the workgroup wrote and recomputes in fp32 the ones above 2^-21, so
// each output meets |y - y_exact| <= 1e-4 sum_k |w_k x_k| + 1e-6 whatever the
// spread of x.  The prefill kernel also folds the group scale into the fp16
// weight, exact while every scale of the row lies within 2^21 of its largest;
// other rows are recomputed by the same pass.  The fast loops are unchanged:
// the pass costs nothing when every D is zero and every row folds exactly.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "qw3.h"

// Device code: inline functions, templates and constants only, so each
// translation unit compiles just what its kernels use.
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

// Largest magnitude and smallest non-zero magnitude (0x10000 when all are
// zero) of 32 bf16 values, as bf16 magnitude bit patterns; packed 16-bit max
// and min, one of each per two values.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void block_stats(const uint4 (&xb)[4], uint32_t &mx, uint32_t &mn) {
    u16x2_t vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};
    const u16x2_t one = {1, 1};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d[4] = {xb[i].x, xb[i].y, xb[i].z, xb[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u16x2_t v = __builtin_bit_cast(u16x2_t, d[j] & 0x7FFF7FFFu);
            vmax = __builtin_elementwise_max(vmax, v);
            vmin = __builtin_elementwise_min(vmin, v - one);  // zero wraps to 0xFFFF
        }
    }
    mx = max((uint32_t)vmax.x, (uint32_t)vmax.y);
    mn = min((uint32_t)vmin.x, (uint32_t)vmin.y) + 1u;
}

// bf16 magnitude bits of 2^(e-7): elements at least this large convert to
// fp16 normals exactly under exponent e for every slot offset p <= 7.
__device__ __forceinline__ uint32_t exact_floor_bits(int e) {
    const int b = e + 120;  // biased bf16 exponent of 2^(e-7)
    if (b >= 1) return (uint32_t)min(b, 255) << 7;
    if (b >= -6) return 1u << (b + 6);  // a bf16 subnormal
    return 0u;
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

// Conversion error of a block: sum over its 32 values of |x - x'|, x' the
// value its fp16 operand stands for, fp16(x * 2^-(e+p)) * 2^(e+p) with the
// slot offset p of convert_block.  fp16 subnormals are kept by the conversion
// and by every fp16 product used here (measured on gfx950), so an element
// converts exactly unless its low bits fall below 2^-24 after scaling; each
// difference is exact in fp32.  Only called when the block has a value below
// 2^(e-7), the smallest that is surely exact.
__device__ __forceinline__ float conversion_error(const uint4 (&xb)[4], int e) {
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
    float err = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const PairSpec ps = kPairs[p];
        const float a = ldexpf(f[ps.lo], -e - ps.p), b = ldexpf(f[ps.hi], -e - ps.pp);
        err += ldexpf(fabsf(a - (float)(_Float16)a), e + ps.p);
        err += ldexpf(fabsf(b - (float)(_Float16)b), e + ps.pp);
    }
    return err;
}

__device__ __forceinline__ void load_x32(const uint16_t *src, uint4 (&xb)[4]) {
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[i] = s[i];
}

// ------------------------------------------------------- exact fixup pass --
// Outputs whose bound 4 sum_g |s_g| D_g exceeds kFixBudget are recomputed by
// exact_output.  The budget leaves half of the 1e-6 absolute term of the
// accuracy bound for the fast path's own fp32 rounding.
constexpr float kFixBudget = 0x1p-21f;
constexpr int kNzCap = 128;  // compacted list of groups with a non-zero D

// sum_{g0 <= g < g1} s[g] * sum_{k in g} (c_k - 4) x_k in fp32 by one thread,
// read the plain way: code i of a 32-code block is bits [3i, 3i + 3) of its
// three little-endian words.  Each product (c - 4) x is exact in fp32; a
// group's 128 products are added in order, the group sums (times their
// scale) in runs of 32 groups, the runs in order.
__device__ __forceinline__ float exact_output(const uint16_t *__restrict__ xrow, const uint32_t *__restrict__ wrow,
                                           const uint16_t *__restrict__ srow, int g0, int g1) {
    float tot = 0.f;
    for (int gb = g0; gb < g1; gb += 32) {
        const int ge = min(gb + 32, g1);
        float run = 0.f;
        for (int g = gb; g < ge; ++g) {
            const uint32_t *gw = wrow + (int64_t)g * kWordsPerGroup;
            float acc = 0.f;
            for (int b = 0; b < 4; ++b) {
                const uint32_t w[4] = {gw[3 * b], gw[3 * b + 1], gw[3 * b + 2], 0u};
                uint4 xb[4];
                load_x32(xrow + (int64_t)g * kGroup + 32 * b, xb);
                const uint32_t xw[16] = {xb[0].x, xb[0].y, xb[0].z, xb[0].w, xb[1].x, xb[1].y, xb[1].z, xb[1].w,
                                         xb[2].x, xb[2].y, xb[2].z, xb[2].w, xb[3].x, xb[3].y, xb[3].z, xb[3].w};
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    const int bit = 3 * i;
                    const uint32_t c = __builtin_amdgcn_alignbit(w[(bit >> 5) + 1], w[bit >> 5], bit & 31) & 7u;
                    const float xv = bf16_to_f32((i & 1) ? (xw[i >> 1] >> 16) : (xw[i >> 1] & 0xFFFFu));
                    acc = fmaf((float)((int)c - 4), xv, acc);
                }
            }
            run = fmaf(acc, bf16_to_f32(srow[g]), run);
        }
        tot += run;
    }
    return tot;
}

// Whether folding the scales of row srow[g0..g1) into fp16 weights as
// s * 2^-E, E chosen so that the largest maps to [8, 16), is inexact for some
// non-zero scale: exact iff s * 2^-E >= 2^-17 (8 significant bits then sit at
// or above fp16's smallest subnormal, and so do the products with (c-4) 2^p).
__device__ __forceinline__ bool fold_inexact(const uint16_t *__restrict__ srow, int g0, int g1) {
    uint32_t mx = 0, mn = 0x10000u;
    for (int g = g0; g < g1; ++g) {
        const uint32_t b = srow[g] & 0x7FFFu;
        mx = max(mx, b);
        if (b) mn = min(mn, b);
    }
    if (mx == 0) return false;
    const int E = __builtin_amdgcn_frexp_expf(bf16_to_f32(mx)) - 4;
    return bf16_to_f32(mn) < ldexpf(1.0f, E - 17);
}

// The rows a workgroup wrote: blocks blk, blk + nblk, blk + 2 nblk, ... of R
// consecutive rows each, rows past N dropped.
struct BlockRows {
    int64_t blk, nblk, R, N;
    __device__ int64_t count() const {
        const int64_t nb = (N + R - 1) / R;
        return blk < nb ? ((nb - blk + nblk - 1) / nblk) * R : 0;
    }
    __device__ int64_t row(int64_t i) const {
        const int64_t r = (blk + (i / R) * nblk) * R + i % R;
        return r < N ? r : -1;
    }
};

// Wave 0 lists in nz[0..) the groups g in [g0, g1) with any_d(g); nz[kNzCap]
// receives their count (which may exceed kNzCap).  All threads of the
// workgroup call it (it ends with a barrier).
template <class AnyD>
__device__ __forceinline__ int build_nz(int g0, int g1, AnyD any_d, int *nz) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int cnt = 0;
        for (int base = g0; base < g1; base += 64) {
            const int g = base + lane;
            const bool f = g < g1 && any_d(g);
            const uint64_t bal = __ballot(f);
            const int pos = cnt + __popcll(bal & ((uint64_t(1) << lane) - 1));
            if (f && pos < kNzCap) nz[pos] = g;
            cnt += __popcll(bal);
        }
        if (lane == 0) nz[kNzCap] = cnt;
    }
    __syncthreads();
    return nz[kNzCap];
}

// The fixup pass over the outputs out[m * ldo + r] (tokens m < Mt, x row m at
// x + m * ldx; rows r of `rows`) computed over the groups [g0, g1): with D(m, g)
// = d_at(m, g), the outputs whose bound exceeds kFixBudget -- and, with `fold`,
// every output of a row whose scales do not fold exactly -- are recomputed by
// exact_output.  nz / nnz list the groups with a non-zero D (nz == nullptr or
// nnz > kNzCap: every group of the range).  Threads tid, tid + nthr, ... take
// one row each.  The caller orders the fast path's stores before this pass.
template <int TB, class DAt>
__device__ __forceinline__ void fixup_outputs(const uint16_t *__restrict__ x, int64_t ldx, int Mt,
                              const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales, int G,
                              int g0, int g1, const BlockRows &rows, DAt d_at, const int *nz, int nnz, bool fold,
                              float *__restrict__ out, int64_t ldo, int tid, int nthr) {
    const int64_t W = (int64_t)G * kWordsPerGroup;
    const bool dense = nz == nullptr || nnz > kNzCap;
    const int ne = dense ? g1 - g0 : nnz;
    const int64_t nrows = rows.count();
    for (int64_t i = tid; i < nrows; i += nthr) {
        const int64_t r = rows.row(i);
        if (r < 0) continue;
        const uint16_t *srow = scales + r * G;
        const bool all = fold && fold_inexact(srow, g0, g1);
        for (int m0 = 0; m0 < Mt; m0 += TB) {
            float b[TB];
#pragma unroll
            for (int t = 0; t < TB; ++t) b[t] = 0.f;
            if (!all) {
                for (int e = 0; e < ne; ++e) {
                    const int g = dense ? g0 + e : nz[e];
                    const float s = fabsf(bf16_to_f32(srow[g]));
#pragma unroll
                    for (int t = 0; t < TB; ++t)
                        if (m0 + t < Mt) b[t] = fmaf(s, d_at(m0 + t, g), b[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const int m = m0 + t;
                if (m < Mt && (all || !(4.0f * b[t] <= kFixBudget)))
                    out[(int64_t)m * ldo + r] = exact_output(x + (int64_t)m * ldx, packed + r * W, srow, g0, g1);
            }
        }
    }
}

typedef unsigned u32x4v_t __attribute__((ext_vector_type(4)));

// The same for the batched kernels that convert in-kernel: tokens t < M (x
// row t at x + t * K), one exponent per (token, 8-group slice), the slices of
// groups [g0, g0 + 8 S): xd[t][g - g0].  Half a wave per (token, slice).
__device__ __forceinline__ void slice_errors(const uint16_t *__restrict__ x, int64_t K, int M, int g0, int S,
                                             float *xd) {
    const int units = M * S * 32;
    for (int u = threadIdx.x; u < units; u += blockDim.x) {  // units and blockDim are multiples of 32
        const int b = u & 3, gi = (u >> 2) & 7, ts = u >> 5;
        const int t = ts / S, sl = ts % S;
        uint4 xb[4];
        load_x32(x + t * K + (int64_t)(g0 + 8 * sl + gi) * kGroup + 32 * b, xb);
        uint32_t m, mn;
        block_stats(xb, m, mn);
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 32));
        float d = conversion_error(xb, group_exponent(m));
        d += dpp_f32<kDppQuadXor1>(d);
        d += dpp_f32<kDppQuadXor2>(d);
        if (b == 0) xd[t * (8 * S) + 8 * sl + gi] = d;
    }
    __syncthreads();
}

// One word per wave in LDS: whether any lane of the wave passed `mine`.
__device__ __forceinline__ void publish_flag(bool mine, uint32_t *flags) {
    const uint64_t bal = __ballot(mine);
    if ((threadIdx.x & 63) == 0) flags[threadIdx.x >> 6] = bal != 0 ? 1u : 0u;
}
__device__ __forceinline__ bool any_flag(const uint32_t *flags) {
    uint32_t f = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) f |= flags[w];
    return f != 0;
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// only, so its global loads stay in flight across the barrier, and the
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

typedef unsigned u32x2v_t __attribute__((ext_vector_type(2)));

}  // namespace

// ------------------------------------------------------------ host side ---
// Host helpers of both translation units; hidden, so nothing here is exported
// beside the C ABI.  The inline variables have one definition in the library.
namespace __attribute__((visibility("hidden"))) qw3_shared {

inline thread_local char g_hip_error[256] = "no HIP error";  // message of the last QW3_ERR_HIP on this thread

inline qw3_status hip_fail(hipError_t err) {
    snprintf(g_hip_error, sizeof g_hip_error, "%s (%d)", hipGetErrorString(err), (int)err);
    return QW3_ERR_HIP;
}

inline qw3_status check_launch() {
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? QW3_OK : hip_fail(err);
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline qw3_status check_shape(int64_t N, int64_t K) {
    if (N < 0 || K < 0 || K % kGroup != 0 || K > QW3_MAX_K || N > (int64_t(1) << 40)) return QW3_ERR_SHAPE;
    return QW3_OK;
}

inline std::mutex g_dev_mutex;  // guards the per-device tables
inline int g_cu_count[64];

inline qw3_status cu_count(int *out) {
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

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups of `kernel` that fit on one CU at `wgs` threads and `lds` bytes.
inline qw3_status blocks_per_cu(const void *kernel, int wgs, size_t lds, int *out) {
    int nb = 0;
    const hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, wgs, lds);
    if (err != hipSuccess) return hip_fail(err);
    *out = nb > 0 ? nb : 1;
    return QW3_OK;
}

// The batch-1 launches (qw3_gemv.hip).  launch_gemv: y = dequant(W) x for M
// tokens, token m reading x + m K and writing y + m N (M > 1 only for the
// batch-invariant product).  launch_gemv_multi: several matrices that share
// x.  Arguments are checked by the caller.
qw3_status launch_gemv(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y, int64_t N,
                       int64_t K, hipStream_t stream, int M = 1);
qw3_status launch_gemv_multi(const uint16_t *x, int count, const uint32_t *const *packed,
                             const uint16_t *const *scales, float *const *y, const int64_t *N, int64_t K,
                             hipStream_t stream);

}  // namespace qw3_shared
