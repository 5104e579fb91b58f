// W3G128 fused dequantize-and-multiply for gfx950 (CDNA4): the batched-decode
// and prefill kernels, the format utilities (qpack, repack, qdequant) and the
// C ABI declared in include/qw3.h.  The format, decode, activation conversion
// and exactness guard shared by every kernel are in qw3_common.h; the batch-1
// kernels in qw3_gemv.hip.
#include <vector>

#include "qw3_common.h"

using namespace qw3_shared;

namespace {

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

// ----------------------------------------------- small-M matrix cores -----
// Activations for the matrix-core kernels: x[m][k] * 2^-e[g][m] as fp16 in the
// operand order of the 16x16x32 MFMA: for group g, token m and 32-code block
// j, 16 fp16 pairs in decode pair order (64 bytes).  Tokens m in [M, Mp) are
// zero.  One thread per (g, m, j); the four blocks of a group form a quad.
// xe[g][m] = 2 e + (1 if the group's error mass is non-zero), the mass itself
// in xd[g][m].
__global__ __launch_bounds__(256) void prep_x_kernel(const uint16_t *__restrict__ x,
                                                     uint4 *__restrict__ xq,
                                                     int16_t *__restrict__ xe, float *__restrict__ xd, int M,
                                                     int Mp, int64_t K, int G) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t units = (int64_t)G * Mp * 4;
    if (idx >= units) return;  // units is a multiple of 4: whole quads exit together
    const int j = (int)(idx & 3);
    const int64_t gm = idx >> 2;
    const int m = (int)(gm % Mp);
    const int g = (int)(gm / Mp);
    uint32_t out[16];
    int eg = 0;
    float d = 0.f;
    if (m < M) {
        uint4 xb[4];
        load_x32(x + (int64_t)m * K + (int64_t)g * kGroup + j * 32, xb);
        uint32_t mx, mn;
        block_stats(xb, mx, mn);
        mx = max(mx, dpp_u32<kDppQuadXor1>(mx));
        mx = max(mx, dpp_u32<kDppQuadXor2>(mx));
        eg = group_exponent(mx);
        if (mn < exact_floor_bits(eg)) d = conversion_error(xb, eg);  // rare
        convert_block(xb, eg, out);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) out[i] = 0;
    }
    d += dpp_f32<kDppQuadXor1>(d);
    d += dpp_f32<kDppQuadXor2>(d);
    uint4 *dst = xq + idx * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    if (j == 0) {
        xe[(int64_t)g * Mp + m] = (int16_t)(2 * eg + (d != 0.f ? 1 : 0));
        xd[(int64_t)g * Mp + m] = d;
    }
}

// Batched decode for any K (the path of K / 128 not a multiple of 8, where no
// whole 8-group activation slices exist), on v_mfma_f32_16x16x32_f16.  One
// workgroup of 8 waves per 16-row tile; wave w takes groups w, w + 8, ... of
// the tile.  Lane l works on row n0 + l%16 and block j = l/16 of each group:
// it decodes 32 codes (3 words) into the B operand (8 fp16 per MFMA, 4 MFMAs
// per group) while the A operand holds the same k-slots of x' for token l%16.
// D[m][n] of one group is scaled by s[n][g] * 2^e[g][m] and added to the fp32
// accumulator.  MT sets of 16 tokens share each decoded B operand, so the
// weights are read once.  Each wave keeps its next groups' words, scale, A
// operands and exponents in a 3-slot register ring, loaded two groups ahead
// (loads past its last group re-read that group, so the waits stay exact);
// the 8 waves' accumulators meet in LDS and are added in wave order.
typedef unsigned u32x3g_t __attribute__((ext_vector_type(3)));
template <int MT>
struct MfSlotG {
    u32x3g_t w;        // block j of the group of row n
    uint32_t s;        // its bf16 scale (low half)
    h8_t a[MT][4];     // A operands: x' of token 16 mt + n, block j
    uint32_t e[MT][2]; // exponents (2 e + flag) of tokens 16 mt + 4 j .. + 3
};
template <int MT>
__global__ __launch_bounds__(512) void qgemm_mfma_kernel(const uint4 *__restrict__ xq,
                                                         const int16_t *__restrict__ xe,
                                                         const float *__restrict__ xd,
                                                         const uint16_t *__restrict__ x,
                                                         const uint32_t *__restrict__ packed,
                                                         const uint16_t *__restrict__ scales,
                                                         float *__restrict__ y, int M, int Mp,
                                                         int64_t N, int G, int64_t y_ld) {
    constexpr int WAVES = 8;
    __shared__ __align__(16) f4_t red[WAVES][MT][64];
    __shared__ uint32_t flags[16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wblk = blockIdx.x;
    const int64_t n0 = wblk * 16;  // the grid has ceil(N / 16) workgroups
    const int nl = lane & 15;
    const int jq = lane >> 4;
    const int64_t n = n0 + nl;
    const int64_t nrow = n < N ? n : N - 1;
    const int64_t W = (int64_t)G * kWordsPerGroup;
    const uint32_t *wrow = packed + nrow * W + jq * 3;
    const uint16_t *srow = scales + nrow * G;
    const int steps = (G - wave + WAVES - 1) / WAVES;  // this wave's groups (0 when wave >= G)

    auto load = [&](int i, MfSlotG<MT> &sl) {
        int g = wave + WAVES * i;
        g = g < G ? g : G - 1;
        sl.w = *reinterpret_cast<const u32x3g_t *>(wrow + (int64_t)g * kWordsPerGroup);
        sl.s = srow[g];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint4 *ap = xq + (((int64_t)g * Mp + mt * 16 + nl) * 4 + jq) * 4;
#pragma unroll
            for (int t = 0; t < 4; ++t) sl.a[mt][t] = __builtin_bit_cast(h8_t, ap[t]);
            const uint2 ev = *reinterpret_cast<const uint2 *>(xe + (int64_t)g * Mp + mt * 16 + 4 * jq);
            sl.e[mt][0] = ev.x;
            sl.e[mt][1] = ev.y;
        }
    };
    f4_t acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t magic = magic_vgpr();
    int small = 0;
    auto step = [&](const MfSlotG<MT> &sl) __attribute__((always_inline)) {
        h2_t q[16];
        decode_block(sl.w.x, sl.w.y, sl.w.z, magic, q);
        const float s = bf16_to_f32(sl.s & 0xFFFFu);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const h8_t bop = {q[4 * t].x,     q[4 * t].y,     q[4 * t + 1].x, q[4 * t + 1].y,
                                  q[4 * t + 2].x, q[4 * t + 2].y, q[4 * t + 3].x, q[4 * t + 3].y};
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(sl.a[mt][t], bop, d, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t ew = sl.e[mt][r >> 1];
                const int ev = (r & 1) ? (int)ew >> 16 : (int)(int16_t)(ew & 0xFFFFu);
                small |= ev & 1;
                acc[mt][r] += ldexpf(d[r], ev >> 1) * s;
            }
        }
    };
    MfSlotG<MT> ring[3];
    __builtin_amdgcn_sched_barrier(0);
    load(0, ring[0]);
    __builtin_amdgcn_sched_barrier(0);
    load(1, ring[1]);
    __builtin_amdgcn_sched_barrier(0);
    int i = 0;
    for (; i + 3 <= steps; i += 3) {  // wave-uniform
        load(i + 2, ring[2]);
        __builtin_amdgcn_sched_barrier(0);
        step(ring[0]);
        load(i + 3, ring[0]);
        __builtin_amdgcn_sched_barrier(0);
        step(ring[1]);
        load(i + 4, ring[1]);
        __builtin_amdgcn_sched_barrier(0);
        step(ring[2]);
    }
    if (i < steps) step(ring[0]);
    if (i + 1 < steps) step(ring[1]);

    publish_flag(small != 0, flags);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][mt][lane] = acc[mt];
    __syncthreads();
    // (set, lane row, r, row) outputs, rows fastest; waves added in order.
    for (int o = threadIdx.x; o < 256 * MT; o += 512) {
        const int row16 = o & 15, r = (o >> 4) & 3, jj = (o >> 6) & 3, mt = o >> 8;
        const int tok = mt * 16 + 4 * jj + r;
        const int64_t row = n0 + row16;
        if (tok < M && row < N) {
            const float *src = reinterpret_cast<const float *>(&red[0][mt][16 * jj + row16]) + r;
            float tot = src[0];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) tot += src[w * MT * 64 * 4];
            y[(int64_t)tok * y_ld + row] = tot;
        }
    }
    if (any_flag(flags)) {  // workgroup-uniform (published before the barrier), rare
        __syncthreads();
        fixup_outputs<4>(x, (int64_t)G * kGroup, M, packed, scales, G, 0, G, BlockRows{wblk, (int64_t)gridDim.x, 16, N},
                         [&](int m, int g) { return xd[(int64_t)g * Mp + m]; }, nullptr, 0, false, y, y_ld,
                         threadIdx.x, blockDim.x);
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
// loads is one contiguous kilobyte.  xe holds 2 e + (1 if some group of the
// slice has a non-zero error mass for token m); the masses go to xd[g][m].
__global__ __launch_bounds__(256) void prep_x_slice_kernel(const uint16_t *__restrict__ x, uint4 *__restrict__ xq,
                                                           int16_t *__restrict__ xe, float *__restrict__ xd, int M,
                                                           int Mp, int64_t K, int S) {
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
    uint32_t mx, mn;
    block_stats(xb, mx, mn);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 32));
    const int e = m < M ? group_exponent(mx) : 0;
    float d = (m < M && mn < exact_floor_bits(e)) ? conversion_error(xb, e) : 0.f;  // rare
    const bool any = (__ballot(d != 0.f) >> (threadIdx.x & 32)) & 0xFFFFFFFFull;  // this half-wave
    d += dpp_f32<kDppQuadXor1>(d);
    d += dpp_f32<kDppQuadXor2>(d);
    uint32_t out[16];
    convert_block(xb, e, out);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xq[(((int64_t)g * 4 + i) * 4 + b) * Mp + m] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    if (b == 0) xd[(int64_t)g * Mp + m] = d;
    if (gi == 0 && b == 0) xe[(int64_t)sl * Mp + m] = (int16_t)(2 * e + (any ? 1 : 0));
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
                                                            const float *__restrict__ xd,
                                                            const uint16_t *__restrict__ x,
                                                            const uint32_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scales,
                                                            float *__restrict__ out, int M, int64_t N, int G, int C,
                                                            int64_t out_chunk) {
    constexpr int Mp = 16;
    __shared__ __align__(16) unsigned char red[2][WAVES][64 * 16];
    __shared__ uint32_t flags[16];
    __shared__ int nz[kNzCap + 1];
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
    // The low bit of each entry flags a non-zero error mass.
    int et[4], small = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int v = xe[(int64_t)(g0 / 8) * Mp + 4 * j + r];
        small |= v & 1;
        et[r] = v >> 1;
    }
    publish_flag(small != 0, flags);
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
    if (any_flag(flags)) {  // workgroup-uniform (the loop's barriers published the flags), rare
        __syncthreads();
        const int gc0 = chunk * WAVES * 8, gc1 = gc0 + WAVES * 8;
        auto d_at = [&](int m, int g) { return xd[(int64_t)g * Mp + m]; };
        const int nnz = build_nz(gc0, gc1, [&](int g) {
            bool f = false;
            for (int m = 0; m < M; ++m) f |= d_at(m, g) != 0.f;
            return f;
        }, nz);
        fixup_outputs<8>(x, (int64_t)G * kGroup, M, packed, scales, G, gc0, gc1, BlockRows{tb, TB, 16, N}, d_at, nz,
                         nnz, false, y, N, threadIdx.x, blockDim.x);
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
constexpr int kMrBatch = 4;  // tiles per cross-wave reduction
// TS sets of 16 tokens share each decoded block (TS = 2: 17..32 tokens in one
// pass over the weights); a wave then owns 8 / TS groups.
// LDS: the partial sums [2][kMrBatch][WAVES][TS][64 lanes] x f4, then 16
// wave flags and the fixup's group list.
template <int WAVES, int TS>
constexpr size_t mr_red_bytes() { return (size_t)2 * kMrBatch * WAVES * TS * 64 * 16; }
template <int WAVES, int TS>
constexpr size_t mr_lds() { return mr_red_bytes<WAVES, TS>() + ((size_t)16 + kNzCap + 1) * 4; }
struct MrSlot {
    u32x4v_t w[3];  // group g0 + 4q + j of row n: 12 words
    u32x2v_t s;     // bf16 scales of groups g0 + 4q .. g0 + 4q + 3 of row n
};

template <int WAVES, int TS>
__global__ __launch_bounds__(64 * WAVES) void qgemm_mr_kernel(const uint4 *__restrict__ xq,
                                                            const int16_t *__restrict__ xe,
                                                            const float *__restrict__ xd,
                                                            const uint16_t *__restrict__ x,
                                                            const uint32_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scales,
                                                            float *__restrict__ out, int M, int64_t N, int G, int C,
                                                            int64_t out_chunk) {
    constexpr int Mp = 16 * TS;
    constexpr int GW = 8 / TS;   // groups per wave
    constexpr int NS = GW / 4;   // 4-group super-steps per tile
    constexpr int UT = 4 / NS;   // tiles per ring cycle (4 slots)
    extern __shared__ __align__(16) unsigned char lds[];  // mr_lds()
    f4_t *red = reinterpret_cast<f4_t *>(lds);
    uint32_t *flags = reinterpret_cast<uint32_t *>(lds + mr_red_bytes<WAVES, TS>());
    int *nz = reinterpret_cast<int *>(flags + 16);
    int small = 0;  // some error mass of this lane's tokens and groups is non-zero
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
                const int v = (r & 1) ? (w0 >> 16) : (int)(int16_t)(w0 & 0xFFFF);
                small |= v & 1;  // the low bit flags a non-zero error mass
                et[ts][r] = v >> 1;
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
    publish_flag(small != 0, flags);  // read after the loop's barriers
    int64_t c0 = 0;
    for (; c0 + UT <= my_tiles; c0 += UT) static_for<UT>([&](auto hc) __attribute__((always_inline)) { tile(c0, hc); });
    static_for<UT - 1>([&](auto hc) __attribute__((always_inline)) {
        if (c0 + decltype(hc)::value < my_tiles) tile(c0, hc);
    });
    if (any_flag(flags)) {  // workgroup-uniform, rare
        __syncthreads();
        const int gc0 = chunk * WAVES * GW, gc1 = gc0 + WAVES * GW;
        auto d_at = [&](int m, int g) { return xd[(int64_t)g * Mp + m]; };
        const int nnz = build_nz(gc0, gc1, [&](int g) {
            bool f = false;
            for (int m = 0; m < M; ++m) f |= d_at(m, g) != 0.f;
            return f;
        }, nz);
        fixup_outputs<8>(x, (int64_t)G * kGroup, M, packed, scales, G, gc0, gc1, BlockRows{tb, TB, 16, N}, d_at, nz,
                         nnz, false, y, N, threadIdx.x, blockDim.x);
    }
}

// ------------------------------------- batched decode, up to eight tokens ---
// The batch-1 matrix-core layout with the tokens in place of its four
// super-step slots.  In super-step q lane (n, j) loads group g0 + 4q + j of
// row n (48 bytes), as in qgemv_mfma_kernel.
// TOK = 4: the lane decodes that group straight into the B operand (k chunk
// j), so no exchange across lanes is needed.  A-operand set q has row
// m = 4t + j' carrying token t's activations of group g0 + 4q + j' in k chunk
// j' and zero elsewhere, so after the super-step's 16 MFMAs rows 4t .. 4t + 3
// -- lane row t's registers -- hold token t's partial sums of the four groups,
// exactly apart.
// TOK = 8: one v_permlane32_swap per word pairs half-groups across lane rows:
// afterwards lane rows 0 and 2 hold the two halves (blocks 2-3 and 0-1) of
// group 4q and rows 1 and 3 those of group 4q + 1 (set 0), and a second
// register set holds groups 4q + 2 and 4q + 3 the same way (set 1).  Each set
// takes 8 MFMAs whose A row m = 2t + g' carries token t's activations in the
// k chunks j' with j' % 2 == g' (group 4q + 2 set + g') and zero in the
// others, so D rows 2t, 2t + 1 hold token t's partials of the set's two
// groups, and lane row j' accumulates tokens 2j' and 2j' + 1.  The same 16
// MFMAs and the same decode per super-step as TOK = 4, twice the tokens.
// A wave owns the 8 groups of one activation slice (128 VGPRs of A operands
// either way) and walks 16-row tiles through the ring of qgemm_mr_kernel; the
// waves' partials meet in LDS every kMrBatch tiles and are added in wave
// order.  The kernel converts the activations itself, with one exponent per
// token over the wave's slice (a conversion launch in front measured slower).
template <int WAVES, int TOK>
__global__ __launch_bounds__(64 * WAVES) void qgemm_m4_kernel(const uint16_t *__restrict__ x,
                                                            const uint32_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scales,
                                                            float *__restrict__ out, int M, int64_t N, int G, int C,
                                                            int64_t out_chunk) {
    static_assert(TOK == 4 || TOK == 8, "four or eight token slots");
    constexpr int GW = 8, NS = 2, UT = 2;
    constexpr int R2 = TOK / 4;  // tokens per lane row and lane
    extern __shared__ __align__(16) unsigned char lds[];  // [2][kMrBatch][WAVES][R2][64 lanes] floats, then the guard's
    float *red = reinterpret_cast<float *>(lds);
    float *xdl = red + 2 * kMrBatch * WAVES * 64 * R2;                         // D [TOK tokens][WAVES * GW groups]
    uint32_t *flags = reinterpret_cast<uint32_t *>(xdl + TOK * WAVES * GW);  // per wave
    int *nz = reinterpret_cast<int *>(flags + 16);
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

    // The bf16 activations straight from x, before the ring's loads (tokens
    // past M read token M - 1, whose rows of D are not stored).
    // TOK = 4: the four lanes n = 4t .. 4t + 3 of lane row j share token t
    // and group g0 + 4q + j, and lane n reads block n % 4 of it.
    // TOK = 8: lanes n = 2t, 2t + 1 of lane row j share token t; the one with
    // n % 2 == j % 2 (whose A rows take lane row j's k chunk) reads blocks
    // bb + (2 if j < 2 else 0) of group g0 + 4q + j % 2 (set 0), its
    // neighbour the same blocks of group g0 + 4q + 2 + j % 2 (set 1).
    constexpr int XB = TOK == 4 ? NS : 2 * NS;  // blocks per lane
    int et[R2];
    h8_t xa[NS][16];
    uint4 xb[XB][4];
    {
        const int64_t K = (int64_t)G * kGroup;
        if constexpr (TOK == 4) {
            const int t = (n >> 2) < M ? (n >> 2) : M - 1;
#pragma unroll
            for (int q = 0; q < NS; ++q)
                load_x32(x + t * K + (int64_t)(g0 + 4 * q + j) * kGroup + 32 * (n & 3), xb[q]);
        } else {
            const int t = (n >> 1) < M ? (n >> 1) : M - 1;
            const int gs = ((n & 1) == (j & 1) ? 0 : 2) + (j & 1);
            const int b0 = j < 2 ? 2 : 0;
#pragma unroll
            for (int q = 0; q < NS; ++q)
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
                    load_x32(x + t * K + (int64_t)(g0 + 4 * q + gs) * kGroup + 32 * (b0 + bb), xb[2 * q + bb]);
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
    load(0, 1, ring[1]);
    __builtin_amdgcn_sched_barrier(0);
    {
        // One exponent per token over the wave's slice: the largest |x| over
        // the token's lanes (TOK = 4: the quad -- the group's blocks -- and
        // lane ^ 16, lane ^ 32 -- its groups; TOK = 8: lane ^ 1 and the lane
        // rows) maps to [2^14, 2^15).
        uint32_t mx = 0, mnq[XB];
#pragma unroll
        for (int i = 0; i < XB; ++i) {
            uint32_t bm;
            block_stats(xb[i], bm, mnq[i]);
            mx = max(mx, bm);
        }
        mx = max(mx, dpp_u32<kDppQuadXor1>(mx));
        if constexpr (TOK == 4) mx = max(mx, dpp_u32<kDppQuadXor2>(mx));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
        const int e = group_exponent(mx);
        // The guard's cheap test (a value below the slice's exact range).
        bool small = false;
#pragma unroll
        for (int i = 0; i < XB; ++i) small |= mnq[i] < exact_floor_bits(e);
        publish_flag(small, flags);
        if constexpr (TOK == 4) {
            // Each lane converts its block; the quad then hands all four
            // blocks to its lane n % 4 = j (a DPP broadcast per dword), the
            // only one whose row takes k chunk j: the other rows are zero.
            // Lane row j accumulates token j, held by lane 4j.
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
            et[0] = __shfl(e, 4 * j);
        } else {
            // Each lane converts its four blocks; the lane with n % 2 == j % 2
            // keeps its own (set 0) and takes its neighbour's (set 1, a DPP
            // swap of adjacent lanes); the other lane's rows are zero.
            // xa[q][8 set + 4 bb + v]; lane row j accumulates tokens 2j and
            // 2j + 1, held by lanes 4j and 4j + 2.
            const bool on = (n & 1) == (j & 1);
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int q = i >> 1, bb = i & 1;
                uint32_t o[16];
                convert_block(xb[i], e, o);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 own = make_uint4(o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]);
                    const uint4 nb = make_uint4(dpp_u32<kDppQuadXor1>(o[4 * v]), dpp_u32<kDppQuadXor1>(o[4 * v + 1]),
                                                dpp_u32<kDppQuadXor1>(o[4 * v + 2]),
                                                dpp_u32<kDppQuadXor1>(o[4 * v + 3]));
                    xa[q][4 * bb + v] = on ? __builtin_bit_cast(h8_t, own) : h8_t{0, 0, 0, 0, 0, 0, 0, 0};
                    xa[q][8 + 4 * bb + v] = on ? __builtin_bit_cast(h8_t, nb) : h8_t{0, 0, 0, 0, 0, 0, 0, 0};
                }
            }
            et[0] = __shfl(e, 4 * j);
            et[1] = __shfl(e, 4 * j + 2);
        }
    }

    const uint32_t magic = magic_vgpr();
    float acc[R2];
#pragma unroll
    for (int r = 0; r < R2; ++r) acc[r] = 0.f;
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
            if constexpr (TOK == 4) {
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
                acc[0] = fmaf(d[0], bf16_to_f32(sl.s.x & 0xFFFFu), acc[0]);
                acc[0] = fmaf(d[1], __uint_as_float(sl.s.x & 0xFFFF0000u), acc[0]);
                acc[0] = fmaf(d[2], bf16_to_f32(sl.s.y & 0xFFFFu), acc[0]);
                acc[0] = fmaf(d[3], __uint_as_float(sl.s.y & 0xFFFF0000u), acc[0]);
            } else {
                // hw[0] (set 0): rows 0, 2 hold group 4q, rows 1, 3 group
                // 4q + 1; hw[1] (set 1): groups 4q + 2 and 4q + 3.  Rows 0, 1
                // hold blocks 2-3 of their group, rows 2, 3 blocks 0-1.
                uint32_t hw[2][6];
#pragma unroll
                for (int w = 0; w < 6; ++w) {
                    const auto r = __builtin_amdgcn_permlane32_swap(wd[6 + w], wd[w], false, false);
                    hw[0][w] = r[0];
                    hw[1][w] = r[1];
                }
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb) {
                        h2_t qd[16];
                        decode_block(hw[st][3 * bb], hw[st][3 * bb + 1], hw[st][3 * bb + 2], magic, qd);
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const h8_t bop = {qd[4 * v].x,     qd[4 * v].y,     qd[4 * v + 1].x, qd[4 * v + 1].y,
                                              qd[4 * v + 2].x, qd[4 * v + 2].y, qd[4 * v + 3].x, qd[4 * v + 3].y};
                            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[q][8 * st + 4 * bb + v], bop, d, 0, 0, 0);
                        }
                    }
                    // d[2r + g]: token 2j + r, group g0 + 4q + 2 st + g of row n
                    const uint32_t sw = st ? sl.s.y : sl.s.x;
                    const float s_lo = bf16_to_f32(sw & 0xFFFFu), s_hi = __uint_as_float(sw & 0xFFFF0000u);
                    acc[0] = fmaf(d[0], s_lo, acc[0]);
                    acc[0] = fmaf(d[1], s_hi, acc[0]);
                    acc[1] = fmaf(d[2], s_lo, acc[1]);
                    acc[1] = fmaf(d[3], s_hi, acc[1]);
                }
            }
            if (q == NS - 1) {
                const int bt = (int)(t % kMrBatch);
                float *rb = red + ((t / kMrBatch) & 1) * (kMrBatch * WAVES * 64 * R2);
#pragma unroll
                for (int r = 0; r < R2; ++r) {
                    rb[((bt * WAVES + wave) * R2 + r) * 64 + lane] = ldexpf(acc[r], et[r]);
                    acc[r] = 0.f;
                }
                if (bt == kMrBatch - 1 || t == my_tiles - 1) {
                    lds_barrier();
                    // (tile, token of the lane, lane) outputs in a fixed number of passes
                    const int outs = (bt + 1) * 64 * R2;
                    constexpr int kPasses = (kMrBatch * 64 * R2 + 64 * WAVES - 1) / (64 * WAVES);
#pragma unroll
                    for (int ps = 0; ps < kPasses; ++ps) {
                        const int i = threadIdx.x + ps * 64 * WAVES;
                        const int tt = i / (64 * R2), r = (i >> 6) % R2, l = i & 63;
                        const int tok = R2 * (l >> 4) + r;
                        const int64_t row = (tb + (t - bt + tt) * TB) * 16 + (l & 15);
                        if (i < outs && tok < M && row < N) {
                            const float *src = rb + (tt * WAVES * R2 + r) * 64 + l;
                            float tot = src[0];
#pragma unroll
                            for (int w = 1; w < WAVES; ++w) tot += src[w * R2 * 64];
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
    if (any_flag(flags)) {  // workgroup-uniform (the loop's barriers published the flags), rare
        __syncthreads();
        const int gc0 = chunk * WAVES * GW, gc1 = gc0 + WAVES * GW;
        slice_errors(x, (int64_t)G * kGroup, M, gc0, WAVES, xdl);
        auto d_at = [&](int m, int g) { return xdl[m * (WAVES * GW) + (g - gc0)]; };
        const int nnz = build_nz(gc0, gc1, [&](int g) {
            bool f = false;
            for (int m = 0; m < M; ++m) f |= d_at(m, g) != 0.f;
            return f;
        }, nz);
        fixup_outputs<4>(x, (int64_t)G * kGroup, M, packed, scales, G, gc0, gc1, BlockRows{tb, TB, 16, N}, d_at, nz,
                         nnz, false, y, N, threadIdx.x, blockDim.x);
    }
}
template <int WAVES, int TOK>
constexpr size_t m4_lds() {
    return (size_t)2 * kMrBatch * WAVES * 64 * (TOK / 4) * sizeof(float) + ((size_t)TOK * WAVES * 8 + 16 + kNzCap + 1) * 4;
}

// --------------------------------------------------- prefill (large M) tiles --
// Many tokens: an MFMA GEMM whose B tiles are decoded on the fly.  Because a
// decoded weight is reused by every token of the tile, the group scale is
// folded into the decoded value instead of being applied per group after the
// MFMAs: B = (c-4) * 2^p * s * 2^-E[n], exact in fp16 (3 + 8 significant
// bits) with E[n] chosen per row so that the row's largest scale maps to
// [8, 16).  A = x * 2^-(E[m] + p) in fp16 with one exponent per token (largest
// |x| of the token maps to [2^14, 2^15); exact down to 2^-28 of it).  The
// accumulators then hold sum_k x w * 2^-(E[m] + E[n]), rescaled once at the
// end.  The activation tiles go through LDS one group (128 k) at a time;
// LDS rows (256 bytes = 16 chunks of 16 bytes) are stored with chunk index
// XOR (row & 15) so that the 16 lanes of a quarter-wave reading one chunk of
// 16 consecutive rows hit 16 different bank groups.

// Per token: E[m] and x' = x * 2^-(E[m] + p) in block pair order, zero rows
// for m >= M; the error masses of the guard per group, xd[m][g], and their
// sum over the token, dtot[m].  One workgroup per token.
__global__ __launch_bounds__(256) void prep_tile_x_kernel(const uint16_t *__restrict__ x, uint32_t *__restrict__ xq,
                                                          int *__restrict__ xe, float *__restrict__ xd,
                                                          float *__restrict__ dtot, int M, int64_t K) {
    __shared__ uint32_t wmax[4];
    __shared__ float wsum[4];
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
        if (tid == 0) {
            xe[m] = 0;
            dtot[m] = 0.f;
        }
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
    const uint32_t floor_bits = exact_floor_bits(e);
    float dsum = 0.f;
    for (int64_t u = tid; u < units; u += 256) {  // units = 4 G: quads of threads are groups
        uint4 xb[4];
        load_x32(src + u * 32, xb);
        uint32_t bm, bn;
        block_stats(xb, bm, bn);
        float d = bn < floor_bits ? conversion_error(xb, e) : 0.f;  // rare
        dsum += d;
        d += dpp_f32<kDppQuadXor1>(d);
        d += dpp_f32<kDppQuadXor2>(d);
        if ((u & 3) == 0) xd[(int64_t)m * (K / kGroup) + (u >> 2)] = d;
        uint32_t out[16];
        convert_block(xb, e, out);
        uint4 *d4 = reinterpret_cast<uint4 *>(dst + u * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) d4[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    }
    for (int off = 32; off >= 1; off >>= 1) dsum += __shfl_xor(dsum, off);
    if ((tid & 63) == 0) wsum[tid >> 6] = dsum;
    __syncthreads();
    if (tid == 0) {
        xe[m] = e;
        dtot[m] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    }
}

// The fixup pass of one prefill workgroup, out of line so that the main
// kernel's registers stay with its MFMA loop: tokens [0, mt) of the tile (x,
// xd and y already offset to its first token), rows of `rows`, groups
// [g0, g1), every row's fold checked.  All threads call it.
__device__ __noinline__ void fixup_tile_call(const uint16_t *x, int64_t K, int mt, const uint32_t *packed,
                                             const uint16_t *scales, int G, int g0, int g1, BlockRows rows,
                                             const float *xd, int *nz, float *y, int64_t ldo) {
    auto d_at = [&](int m, int g) { return xd[(int64_t)m * G + g]; };
    const int nnz = build_nz(g0, g1, [&](int g) {
        bool f = false;
        for (int m = 0; m < mt; ++m) f |= d_at(m, g) != 0.f;
        return f;
    }, nz);
    fixup_outputs<8>(x, K, mt, packed, scales, G, g0, g1, rows, d_at, nz, nnz, true, y, ldo, threadIdx.x, blockDim.x);
}

// Whether the prefill kernel's fast result may be outside the accuracy bound
// for an output of row set / token set whose largest row exponent is en_max
// (largest scale below 2^(en_max + 4)) and whose largest token error mass is
// dmax: 4 s D > budget.
__device__ __forceinline__ bool tile_coarse_flag(int en_max, float dmax) {
    return dmax > 0.f && !(4.0f * ldexpf(dmax, en_max + 4) <= kFixBudget);
}

constexpr int kTileRow = 256;  // bytes of one LDS row: one token's group (128 fp16)

__device__ __forceinline__ int tile_off(int row, int chunk) { return row * kTileRow + ((chunk ^ (row & 15)) << 4); }


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

constexpr int kPfMinM = 129;  // fewest tokens that take the 256 x 256 tiles
constexpr int kPfBM = 256, kPfBN = 256;
constexpr size_t kPfStage = (size_t)kPfBM * kTileRow;  // 64 KB of activations per group

typedef unsigned u32x3_t __attribute__((ext_vector_type(3)));
typedef __attribute__((address_space(3))) void pf_lds_void_t;

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void qgemm_pf_kernel(
    const uint32_t *__restrict__ xq, const int *__restrict__ xe, const float *__restrict__ xd,
    const float *__restrict__ dtot, const uint16_t *__restrict__ x, const uint32_t *__restrict__ packed,
    const uint16_t *__restrict__ scales, float *__restrict__ out, int M, int MT, int64_t N, int G, int C,
    int64_t out_chunk) {
    constexpr int NI = 4;  // 16-row sub-tiles per wave
    // The two activation stages as separate arrays: the copy into one and the
    // reads from the other are then provably disjoint, so the compiler neither
    // drains the copy before a read nor needs the reads hidden in asm.
    __shared__ __align__(16) unsigned char stage_a[kPfStage], stage_b[kPfStage];
    __shared__ uint32_t flags[16];
    __shared__ int nz[kNzCap + 1];
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
    // Row exponents over the chunk (largest scale -> [8, 16)); a row whose
    // smallest non-zero scale lies below 2^(E - 17) does not fold exactly
    // (fold_inexact) and is recomputed after the loop.
    int en[NI];
    bool need = false;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        uint32_t mx = 0, mn = 0x10000u;
        for (int g = gbeg + lc; g < gbeg + Gc; g += 4) {
            const uint32_t b = (uint32_t)scales[rows[i] * G + g] & 0x7FFFu;
            mx = max(mx, b);
            if (b) mn = min(mn, b);
        }
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, 16));
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, 32));
        en[i] = __builtin_amdgcn_frexp_expf(bf16_to_f32(mx)) - 4;
        need |= mx != 0 && bf16_to_f32(mn) < ldexpf(1.0f, en[i] - 17);
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

    // The guard, decided before the loop: a row that does not fold exactly, or
    // a token error mass of the tile large enough to matter against this
    // wave's rows (4 tokens per lane, then the wave's maxima).
    {
        float dmax = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = m0 + 4 * lane + r;
            dmax = fmaxf(dmax, dtot[tok < M ? tok : M - 1]);
        }
        int en_max = max(max(en[0], en[1]), max(en[2], en[3]));
        for (int off = 32; off >= 1; off >>= 1) {
            dmax = fmaxf(dmax, __shfl_xor(dmax, off));
            en_max = max(en_max, __shfl_xor(en_max, off));
        }
        publish_flag(need || tile_coarse_flag(en_max, dmax), flags);
    }
    dma_a(gbeg, stage_a);
    load_w(gbeg, wcur, scur);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    const bool fix = __builtin_amdgcn_readfirstlane(any_flag(flags) ? 1 : 0) != 0;
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
    if (fix) {  // workgroup-uniform, rare
        __syncthreads();  // orders the stores above before the fixup's
        fixup_tile_call(x + (int64_t)m0 * K, K, M - m0 < kPfBM ? M - m0 : kPfBM, packed, scales, G, gbeg, gbeg + Gc,
                        BlockRows{n_tile, NT, kPfBN, N}, xd + (int64_t)m0 * G, nz, y + (int64_t)m0 * N, N);
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = 0.f;
}

// ------------------------------------------------------------ host side ---
// Device scratch of the batched-decode and prefill paths: converted
// activations, the guard's error masses and K-chunk partial sums.
//
// One buffer per (device, stream handle).  The first call on a stream
// allocates it (hipMalloc, whole MiB); a later call that needs more allocates
// one at least twice as large and keeps the old one allocated until the
// process ends, because work queued earlier -- or a graph captured earlier --
// may still use it: nothing is ever freed or synchronized.  A call that would
// allocate while its stream is being captured returns QW3_ERR_CAPTURE.
// Calls on one stream run in order and share its buffer; other streams get
// their own.  Streams are told apart by handle (the HIP runtime the library
// runs under offers no stream id), so a stream created at the address of a
// destroyed one inherits its buffer: the header asks callers to let a
// stream's work finish before destroying it.  (A stream-ordered allocation
// per call measured 4-8 us per call.)
struct Workspace {
    int dev;
    hipStream_t stream;
    void *ptr;
    size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;
std::vector<void *> g_ws_retired;  // superseded buffers, held until the process ends

bool stream_capturing(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return cs != hipStreamCaptureStatusNone;
}

qw3_status workspace(hipStream_t stream, size_t bytes, void **out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace *w = nullptr;
    for (auto &e : g_ws)
        if (e.dev == dev && e.stream == stream) w = &e;
    if (w && w->bytes >= bytes) {
        *out = w->ptr;
        return QW3_OK;
    }
    if (stream_capturing(stream)) return QW3_ERR_CAPTURE;
    size_t grow = (bytes + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);
    if (w && grow < 2 * w->bytes) grow = 2 * w->bytes;
    void *p = nullptr;
    err = hipMalloc(&p, grow);
    if (err != hipSuccess) return hip_fail(err);
    if (w) {
        g_ws_retired.push_back(w->ptr);
        w->ptr = p;
        w->bytes = grow;
    } else {
        g_ws.push_back(Workspace{dev, stream, p, grow});
    }
    *out = p;
    return QW3_OK;
}

// Static source, for callers that cannot allocate (qgemm_w3g128_smallM_noalloc):
// the file-scope array `scratch`, one copy per device for the life of the
// process.  On the host its name is only a stand-in; the device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and used everywhere instead.  Calls on one device share the array,
// so calls that overlap on one device race; every byte a call reads from it
// is written earlier by the same call, so nothing needs clearing.
constexpr size_t kScratchBytes = size_t(QW3_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kScratchBytes];
void *g_scratch_ptr[64];

qw3_status static_scratch(size_t bytes, void **out) {
    if (bytes > kScratchBytes) return QW3_ERR_SCRATCH;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err);
    if (dev < 0 || dev >= 64) return hip_fail(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return hip_fail(err);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QW3_OK;
}

// Where a call takes its scratch from.
struct ScratchSrc {
    hipStream_t stream;
    bool fixed;  // the static array instead of the per-stream workspace
    qw3_status get(size_t bytes, void **out) const {
        return fixed ? static_scratch(bytes, out) : workspace(stream, bytes, out);
    }
};

// Carves consecutive 256-byte-aligned pieces out of one scratch buffer.
struct Carve {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~size_t(255);
        return at;
    }
};

qw3_status fill_zero(float *y, int64_t n, hipStream_t stream) {
    if (n == 0) return QW3_OK;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, y, n);
    return check_launch();
}


// Scratch of the per-token conversion of Mp tokens: x' [Mp][K] fp16, the
// exponents [Mp], the token error masses [Mp] and the group masses [Mp][G].
struct TileX {
    uint32_t *xq;
    int *xe;
    float *dtot, *xd;
};
size_t tile_x_layout(int64_t Mp, int64_t K, Carve &cv, size_t (&at)[4]) {
    at[0] = cv.take((size_t)Mp * (size_t)K * 2);
    at[1] = cv.take((size_t)Mp * sizeof(int));
    at[2] = cv.take((size_t)Mp * sizeof(float));
    at[3] = cv.take((size_t)Mp * (size_t)(K / kGroup) * sizeof(float));
    return cv.off;
}
TileX tile_x_at(void *base, const size_t (&at)[4]) {
    char *b = static_cast<char *>(base);
    return TileX{reinterpret_cast<uint32_t *>(b + at[0]), reinterpret_cast<int *>(b + at[1]),
                 reinterpret_cast<float *>(b + at[2]), reinterpret_cast<float *>(b + at[3])};
}

// Prefill on 256 x 256 tiles: convert x once (per-token exponent), one tile
// launch (K split into C chunks when the tiles alone would not fill the
// GPU), and a chunk sum.
qw3_status launch_gemm_pf(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y, int64_t M,
                          int64_t N, int64_t K, const ScratchSrc &src) {
    const int G = (int)(K / kGroup);
    const int MT = (int)ceil_div(M, kPfBM);
    const int64_t NT = ceil_div(N, kPfBN);
    int cus = 0;
    qw3_status st = cu_count(&cus);
    if (st != QW3_OK) return st;
    int C = 1;
    while (NT * MT * C * 2 <= cus && G % (2 * C) == 0) C *= 2;
    const int64_t Mp = (int64_t)MT * kPfBM;
    Carve cv;
    size_t at[4];
    tile_x_layout(Mp, K, cv, at);
    const size_t part_at = cv.take(C > 1 ? (size_t)C * (size_t)M * (size_t)N * sizeof(float) : 0);
    void *base = nullptr;
    st = src.get(cv.off, &base);
    if (st != QW3_OK) return st;
    const TileX tx = tile_x_at(base, at);
    float *part = reinterpret_cast<float *>(static_cast<char *>(base) + part_at);
    hipLaunchKernelGGL(prep_tile_x_kernel, dim3((unsigned)Mp), dim3(256), 0, src.stream, x, tx.xq, tx.xe, tx.xd,
                       tx.dtot, (int)M, K);
    st = check_launch();
    if (st == QW3_OK) {
        float *dst = C > 1 ? part : y;
        hipLaunchKernelGGL(qgemm_pf_kernel, dim3((unsigned)(NT * MT * C)), dim3(512), 0, src.stream, tx.xq, tx.xe,
                           tx.xd, tx.dtot, x, packed, scales, dst, (int)M, MT, N, G, C, (int64_t)M * N);
        st = check_launch();
    }
    if (st == QW3_OK && C > 1) {
        const int64_t count = M * N;
        hipLaunchKernelGGL(qgemm_chunk_sum_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, src.stream,
                           part, y, count, C, count);
        st = check_launch();
    }
    return st;
}

// Batched decode from registers (tokens <= 16 per pass), K in chunks of
// WAVES x 8 groups.
// TS = 1: passes of up to 16 tokens, through the ring kernel when the scale
// rows are 8-byte aligned (it reads 8 bytes of scales at a time), else
// through qgemm_mt_kernel (2 bytes at a time).  TS = 2: 17..32 tokens in one
// pass of the ring kernel (two sets of 16 per decoded block, 4 groups per
// wave), scale rows 8-byte aligned.
template <int WAVES, int TS>
qw3_status launch_gemm_mt(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y, int64_t M,
                          int64_t N, int64_t K, const ScratchSrc &src) {
    const int G = (int)(K / kGroup);
    const bool ring = TS == 2 || aligned(scales, 8);
    constexpr int Mp = 16 * TS;
    const int C = G / ((8 / TS) * WAVES);
    Carve cv;
    const size_t xq_at = cv.take((size_t)Mp * (size_t)K * 2);
    const size_t xe_at = cv.take((size_t)(G / 8) * Mp * sizeof(int16_t));
    const size_t xd_at = cv.take((size_t)G * Mp * sizeof(float));
    const size_t part_at = cv.take(C > 1 ? (size_t)C * Mp * (size_t)N * sizeof(float) : 0);
    const void *kern = ring ? reinterpret_cast<const void *>(&qgemm_mr_kernel<WAVES, TS>)
                            : reinterpret_cast<const void *>(&qgemm_mt_kernel<WAVES>);
    const size_t lds = ring ? mr_lds<WAVES, TS>() : 0;
    int cus = 0, per_cu = 0;
    qw3_status st = cu_count(&cus);
    if (st == QW3_OK) st = blocks_per_cu(kern, 64 * WAVES, lds, &per_cu);
    if (st != QW3_OK) return st;
    void *base = nullptr;
    st = src.get(cv.off, &base);
    if (st != QW3_OK) return st;
    char *b = static_cast<char *>(base);
    uint4 *xq = reinterpret_cast<uint4 *>(b + xq_at);
    int16_t *xe = reinterpret_cast<int16_t *>(b + xe_at);
    float *xd = reinterpret_cast<float *>(b + xd_at);
    float *part = reinterpret_cast<float *>(b + part_at);
    const int64_t tiles = ceil_div(N, 16);
    int64_t tb = (int64_t)cus * per_cu / C;
    if (tb < 1) tb = 1;
    if (tb > tiles) tb = tiles;
    const hipStream_t stream = src.stream;
    for (int64_t m0 = 0; m0 < M && st == QW3_OK; m0 += Mp) {
        const int mc = (int)(M - m0 < Mp ? M - m0 : Mp);
        const int64_t units = (int64_t)(G / 8) * Mp * 32;
        hipLaunchKernelGGL(prep_x_slice_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, stream,
                           x + m0 * K, xq, xe, xd, mc, Mp, K, G / 8);
        st = check_launch();
        if (st != QW3_OK) break;
        float *dst = C > 1 ? part : y + m0 * N;
        if (ring)
            hipLaunchKernelGGL((qgemm_mr_kernel<WAVES, TS>), dim3((unsigned)(tb * C)), dim3(64 * WAVES), lds,
                               stream, xq, xe, xd, x + m0 * K, packed, scales, dst, mc, N, G, C, (int64_t)Mp * N);
        else
            hipLaunchKernelGGL(qgemm_mt_kernel<WAVES>, dim3((unsigned)(tb * C)), dim3(64 * WAVES), 0, stream, xq, xe,
                               xd, x + m0 * K, packed, scales, dst, mc, N, G, C, (int64_t)Mp * N);
        st = check_launch();
        if (st != QW3_OK || C == 1) continue;
        const int64_t count = (int64_t)mc * N;
        hipLaunchKernelGGL(qgemm_chunk_sum_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, stream, part,
                           y + m0 * N, count, C, (int64_t)Mp * N);
        st = check_launch();
    }
    return st;
}

// Up to TOK (4 or 8) tokens: qgemm_m4_kernel, WAVES x 8 groups per K chunk
// (scale rows 8-byte aligned).
template <int WAVES, int TOK>
qw3_status launch_gemm_m4(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y, int64_t M,
                          int64_t N, int64_t K, const ScratchSrc &src) {
    constexpr int Mp = TOK;  // token slots of the partial sums
    const int G = (int)(K / kGroup);
    const int C = G / (8 * WAVES);
    const size_t part_bytes = C > 1 ? (size_t)C * Mp * (size_t)N * sizeof(float) : 0;
    const size_t lds = m4_lds<WAVES, TOK>();
    int cus = 0, per_cu = 0;
    qw3_status st = cu_count(&cus);
    if (st == QW3_OK)
        st = blocks_per_cu(reinterpret_cast<const void *>(&qgemm_m4_kernel<WAVES, TOK>), 64 * WAVES, lds, &per_cu);
    if (st != QW3_OK) return st;
    float *part = nullptr;
    if (part_bytes > 0) {
        void *base = nullptr;
        st = src.get(part_bytes, &base);
        if (st != QW3_OK) return st;
        part = static_cast<float *>(base);
    }
    const int64_t tiles = ceil_div(N, 16);
    int64_t tb = (int64_t)cus * per_cu / C;
    if (tb < 1) tb = 1;
    if (tb > tiles) tb = tiles;
    hipLaunchKernelGGL((qgemm_m4_kernel<WAVES, TOK>), dim3((unsigned)(tb * C)), dim3(64 * WAVES), lds, src.stream, x,
                       packed, scales, C > 1 ? part : y, (int)M, N, G, C, (int64_t)Mp * N);
    st = check_launch();
    if (st != QW3_OK || C == 1) return st;
    const int64_t count = M * N;
    hipLaunchKernelGGL(qgemm_chunk_sum_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, src.stream, part, y,
                       count, C, (int64_t)Mp * N);
    return check_launch();
}

// Waves per workgroup of the batched-decode kernels, whose waves own 8 groups
// (one activation slice) each: the largest w <= 8 with G a multiple of 8 w,
// so that a workgroup's w slices tile K exactly (K = 8192: 8, 28672: 7,
// 4096: 4, 53248: 4); 0 when G is not a multiple of 8.
int slice_waves(int G) {
    if (G % 8 != 0) return 0;
    for (int w = 8; w > 1; --w)
        if ((G / 8) % w == 0) return w;
    return 1;
}

// f(std::integral_constant<int, w>{}) for w = 1..8.
template <class F>
qw3_status with_waves(int w, F &&f) {
    switch (w) {
        case 8: return f(std::integral_constant<int, 8>{});
        case 7: return f(std::integral_constant<int, 7>{});
        case 6: return f(std::integral_constant<int, 6>{});
        case 5: return f(std::integral_constant<int, 5>{});
        case 4: return f(std::integral_constant<int, 4>{});
        case 3: return f(std::integral_constant<int, 3>{});
        case 2: return f(std::integral_constant<int, 2>{});
        case 1: return f(std::integral_constant<int, 1>{});
        default: return QW3_ERR_SHAPE;
    }
}

// Small-M path: convert x once into scratch, then one streaming pass over W
// per chunk of up to 32 tokens.
qw3_status launch_gemm_small(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                             int64_t M, int64_t N, int64_t K, const ScratchSrc &src) {
    const int G = (int)(K / kGroup);
    const int w = slice_waves(G);
    if (M >= kPfMinM) return launch_gemm_pf(x, packed, scales, y, M, N, K, src);
    // Batched decode, and 33..128 tokens in passes over the weights (against
    // one 128-token tile GEMM, since removed: gate_proj M = 64 66 us against
    // 140, down_proj 68 against 458, q_proj 37 against 139).  With 8-byte aligned scale rows:
    // up to 4 and up to 8 tokens in the batch-1 layout, converting the
    // activations in the kernel (8 tokens: about 1 us faster than the ring
    // kernel with its conversion launch on both MLP shapes); 17 and more
    // tokens in passes of 32 through the ring kernel (chunks of 8 waves x 4
    // groups).  Otherwise passes of up to 16 tokens in chunks of w waves x 8
    // groups (slice_waves: 8 at K = 8192, 7 at 28672).  The 4- and 8-token
    // kernels and the 16-token passes need K / 1024 whole; other K take
    // qgemm_mfma_kernel in passes of 16 or 32.
    if (w > 0 && M <= 8 && aligned(scales, 8)) {
        if (M <= 4)
            return with_waves(w, [&](auto wc) { return launch_gemm_m4<decltype(wc)::value, 4>(x, packed, scales, y, M, N, K, src); });
        return with_waves(w, [&](auto wc) { return launch_gemm_m4<decltype(wc)::value, 8>(x, packed, scales, y, M, N, K, src); });
    }
    if (M > 16 && aligned(scales, 8) && G % 32 == 0) return launch_gemm_mt<8, 2>(x, packed, scales, y, M, N, K, src);
    if (w > 0)
        return with_waves(w, [&](auto wc) { return launch_gemm_mt<decltype(wc)::value, 1>(x, packed, scales, y, M, N, K, src); });
    const int mchunk = M > 16 ? 32 : 16;
    Carve cv;
    const size_t xq_at = cv.take((size_t)mchunk * (size_t)K * 2);
    const size_t xe_at = cv.take((size_t)G * mchunk * sizeof(int16_t));
    const size_t xd_at = cv.take((size_t)G * mchunk * sizeof(float));
    void *base = nullptr;
    qw3_status st = src.get(cv.off, &base);
    if (st != QW3_OK) return st;
    char *b = static_cast<char *>(base);
    uint4 *xq = reinterpret_cast<uint4 *>(b + xq_at);
    int16_t *xe = reinterpret_cast<int16_t *>(b + xe_at);
    float *xd = reinterpret_cast<float *>(b + xd_at);
    for (int64_t m0 = 0; m0 < M && st == QW3_OK; m0 += mchunk) {
        const int mc = (int)(M - m0 < mchunk ? M - m0 : mchunk);
        const int64_t units = (int64_t)G * mchunk * 4;
        hipLaunchKernelGGL(prep_x_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, src.stream,
                           x + m0 * K, xq, xe, xd, mc, mchunk, K, G);
        st = check_launch();
        if (st != QW3_OK) break;
        const unsigned blocks = (unsigned)ceil_div(N, 16);
        if (mchunk == 16)
            hipLaunchKernelGGL(qgemm_mfma_kernel<1>, dim3(blocks), dim3(512), 0, src.stream, xq, xe, xd, x + m0 * K,
                               packed, scales, y + m0 * N, mc, mchunk, N, G, N);
        else
            hipLaunchKernelGGL(qgemm_mfma_kernel<2>, dim3(blocks), dim3(512), 0, src.stream, xq, xe, xd, x + m0 * K,
                               packed, scales, y + m0 * N, mc, mchunk, N, G, N);
        st = check_launch();
    }
    return st;
}

// Validation shared by the two batched entry points.
qw3_status check_gemm_args(const uint16_t *x, const int32_t *packed, const uint16_t *scales, const float *y,
                           int64_t M, int64_t N, int64_t K) {
    qw3_status st = check_shape(N, K);
    if (st != QW3_OK) return st;
    if (M < 0 || M > (int64_t(1) << 24)) return QW3_ERR_SHAPE;
    if (N == 0 || M == 0) return QW3_OK;
    if (!y) return QW3_ERR_NULL;
    if (!aligned(y, 4)) return QW3_ERR_ALIGN;
    if (K == 0) return QW3_OK;
    if (!x || !packed || !scales) return QW3_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2)) return QW3_ERR_ALIGN;
    return QW3_OK;
}

qw3_status run_gemm(const uint16_t *x, const int32_t *packed, const uint16_t *scales, float *y, int64_t M, int64_t N,
                    int64_t K, const ScratchSrc &src) {
    const qw3_status st = check_gemm_args(x, packed, scales, y, M, N, K);
    if (st != QW3_OK || N == 0 || M == 0) return st;
    if (K == 0) return fill_zero(y, M * N, src.stream);
    const uint32_t *pw = reinterpret_cast<const uint32_t *>(packed);
    if (M == 1) return launch_gemv(x, pw, scales, y, N, K, src.stream);
    return launch_gemm_small(x, pw, scales, y, M, N, K, src);
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

qw3_status qgemm_w3g128_batch_invariant(const uint16_t *x, const int32_t *packed, const uint16_t *scales,
                                        float *y, int64_t M, int64_t N, int64_t K, void *hip_stream) {
    qw3_status st = check_shape(N, K);
    if (st != QW3_OK) return st;
    if (M < 0 || M > QW3_MAX_BATCH_INVARIANT_M) return QW3_ERR_SHAPE;
    if (N == 0 || M == 0) return QW3_OK;
    if (!y) return QW3_ERR_NULL;
    if (!aligned(y, 4)) return QW3_ERR_ALIGN;
    if (K == 0) return fill_zero(y, M * N, (hipStream_t)hip_stream);
    if (!x || !packed || !scales) return QW3_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2)) return QW3_ERR_ALIGN;
    return launch_gemv(x, reinterpret_cast<const uint32_t *>(packed), scales, y, N, K, (hipStream_t)hip_stream,
                       (int)M);
}

qw3_status qgemm_w3g128_smallM(const uint16_t *x, const int32_t *packed, const uint16_t *scales, float *y,
                               int64_t M, int64_t N, int64_t K, void *hip_stream) {
    return run_gemm(x, packed, scales, y, M, N, K, ScratchSrc{(hipStream_t)hip_stream, false});
}

qw3_status qgemm_w3g128_smallM_noalloc(const uint16_t *x, const int32_t *packed, const uint16_t *scales, float *y,
                                       int64_t M, int64_t N, int64_t K, void *hip_stream) {
    return run_gemm(x, packed, scales, y, M, N, K, ScratchSrc{(hipStream_t)hip_stream, true});
}

const char *qstatus_str(qw3_status status) {
    switch (status) {
        case QW3_OK: return "ok";
        case QW3_ERR_NULL: return "a required pointer is NULL";
        case QW3_ERR_SHAPE: return "invalid shape (negative size, K % 128 != 0, or K > QW3_MAX_K)";
        case QW3_ERR_ALIGN: return "misaligned pointer (x/packed/codes/w_out need 16 bytes)";
        case QW3_ERR_HIP: return "HIP runtime error (see qw3_last_hip_error)";
        case QW3_ERR_CAPTURE: return "the stream's workspace would have to grow during graph capture";
        case QW3_ERR_SCRATCH: return "the call needs more than the static scratch (QW3_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

const char *qw3_last_hip_error(void) { return g_hip_error; }

int qw3_abi_version(void) { return 1; }

}  // extern "C"
