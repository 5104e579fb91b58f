// Batch-1 kernels of the W3G128 library: qgemv_w3g128, qgemv_w3g128_multi
// and the batch-invariant product (C ABI in qw3.hip).  A translation unit of
// its own so that its instruction scheduling is chosen apart from the batched
// and prefill kernels: the build compiles it with the max-ilp machine
// scheduler, which measured faster on these kernels and slower on the others.
#include "qw3_common.h"

using namespace qw3_shared;

namespace {

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
constexpr int kGemvDepth = 3;    // rows in flight per team
constexpr int kGemvWGS = 256;     // threads per workgroup, teams of T <= 64
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
__device__ __forceinline__ uint4 load_words16(const uint32_t *p) { return *reinterpret_cast<const uint4 *>(p); }

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
// conflicts); exponents follow as int[G].  Returns whether this thread saw a
// value below its group's surely-exact range (the guard's cheap test; the
// conversion error itself is computed only then, by group_errors).
template <int U>
__device__ __forceinline__ bool xstage_convert(const XStage<U> &st, int G, uint32_t *smem) {
    uint4 *xs4 = reinterpret_cast<uint4 *>(smem);                // [16][G]
    int *xe = reinterpret_cast<int *>(smem + (size_t)G * 64);  // [G]
    bool small = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int idx = threadIdx.x + u * blockDim.x;  // quads share validity: 4G and blockDim are multiples of 4
        uint32_t m, mn;
        block_stats(st.raw[u], m, mn);
        m = max(m, dpp_u32<kDppQuadXor1>(m));
        m = max(m, dpp_u32<kDppQuadXor2>(m));
        if (idx < 4 * G) {
            const int g = idx >> 2, blk = idx & 3;
            const int eg = group_exponent(m);
            small |= mn < exact_floor_bits(eg);
            uint32_t out[16];
            convert_block(st.raw[u], eg, out);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xs4[(size_t)(4 * blk + i) * G + g] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
            if (blk == 0) xe[g] = eg;
        }
    }
    return small;
}

// The guard's error masses of a batch-1 activation vector, one exponent per
// group as in the staging: xd[g] = conversion_error summed over group g.  All
// threads of the workgroup call it (it ends with a barrier).
__device__ __forceinline__ void group_errors(const uint16_t *__restrict__ x, int G, float *xd) {
    for (int u = threadIdx.x; u < 4 * G; u += blockDim.x) {  // a quad of threads per group
        uint4 xb[4];
        load_x32(x + (size_t)(u >> 2) * kGroup + (u & 3) * 32, xb);
        uint32_t m, mn;
        block_stats(xb, m, mn);
        m = max(m, dpp_u32<kDppQuadXor1>(m));
        m = max(m, dpp_u32<kDppQuadXor2>(m));
        float d = conversion_error(xb, group_exponent(m));
        d += dpp_f32<kDppQuadXor1>(d);
        d += dpp_f32<kDppQuadXor2>(d);
        if ((u & 3) == 0) xd[u >> 2] = d;
    }
    __syncthreads();
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
// group in two passes (max, then convert).  Returns the guard's cheap test
// for the group (a value below its surely-exact range).
__device__ __forceinline__ bool xstage_lane(const uint16_t *__restrict__ x, int gl, bool lane_on,
                                            uint32_t (&xp)[64], int &e) {
    const uint16_t *xg = x + (size_t)(lane_on ? gl : 0) * kGroup;
    uint32_t m = 0, mn = 0x10000u;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        uint4 xb[4];
        load_x32(xg + blk * 32, xb);
        uint32_t bm, bn;
        block_stats(xb, bm, bn);
        m = max(m, bm);
        mn = min(mn, bn);
    }
    e = group_exponent(m);
    const bool small = lane_on && mn < exact_floor_bits(e);
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
    return small;
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
// LDS words of the batch-1 staging for G groups: xs4 [16][G] x 16 B and xe [G],
// then xd [G] (error masses), 16 wave flags and the fixup's group list.
__host__ __device__ constexpr size_t stage_words(int G) { return (size_t)G * 66 + 16 + kNzCap + 1; }

template <int T, bool MULTI, int D>
__global__ __launch_bounds__(kGemvWGS) void qgemv_small_kernel(const uint16_t *__restrict__ x,
                                                               const GemvSegs sg, int G) {
    constexpr int R = kGemvWGS / T;
    extern __shared__ uint32_t smem[];
    x += (int64_t)blockIdx.y * G * kGroup;  // token blockIdx.y (one token unless batch-invariant)
    float *xd = reinterpret_cast<float *>(smem + (size_t)G * 65);
    uint32_t *flags = smem + (size_t)G * 66;
    int *nz = reinterpret_cast<int *>(flags + 16);
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
    const int64_t N = MULTI ? seg_pick(sg.rows, kseg) : sg.rows[0];
    float *__restrict__ y = (MULTI ? seg_pick(sg.y, kseg) : sg.y[0]) + (int64_t)blockIdx.y * N;
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
    {
        XStage<1> st;  // 4G <= 256 <= blockDim: one block per thread
        xstage_issue<1>(x, G, st);
#pragma unroll
        for (int d = 0; d < D; ++d) load(row0 + d * stride, ring[d]);
        publish_flag(xstage_convert<1>(st, G, smem), flags);
        __syncthreads();
        xstage_fetch(smem, G, gl, lane_on, xp, e);
    }
    const bool fix = __builtin_amdgcn_readfirstlane(any_flag(flags) ? 1 : 0) != 0;  // the guard, workgroup-uniform
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
    if (fix) {  // rare
        __syncthreads();
        group_errors(x, G, xd);
        const int nnz = build_nz(0, G, [&](int g) { return xd[g] != 0.f; }, nz);
        fixup_outputs<1>(x, 0, 1, packed, scales, G, 0, G, BlockRows{blk, nblk, R, N},
                         [&](int, int g) { return xd[g]; }, nz, nnz, false, y, 0, threadIdx.x, blockDim.x);
    }
}


// Teams of T > 64 lanes, T a multiple of 32 (>= G): each half-wave sums its 32
// lanes with DPP, the half sums go through LDS, and lane 0 of the team adds
// its T/32 halves in order.  One barrier per D + 1 rows.  1024-thread
// workgroups (K > 65536) keep a single row in flight to stay within 128 VGPRs.  The LDS holds the
// converted activations first, then (after a barrier) the half sums.
// LDS_X: the converted activations fit in LDS (K <= 32768); otherwise each
// lane converts its own group.  A template parameter, so that one prologue
// reaches the loop and the loop's waits are exact.
// The batch-1 fixup out of line, for kernels held to 128 VGPRs (1024-thread
// workgroups), where the inlined pass would crowd the main loop's registers.
__device__ __noinline__ void fixup_m1_call(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                                           int G, BlockRows rows, const float *xd, const int *nz, int nnz, int tid,
                                           int nthr) {
    fixup_outputs<1>(x, 0, 1, packed, scales, G, 0, G, rows, [&](int, int g) { return xd[g]; }, nz, nnz, false, y, 0,
                     tid, nthr);
}

constexpr int kBigRedWords = 256;  // half-sum slots of qgemv_big_kernel: 2 (E <= 4) x E x (<= 32 halves)
// LDS words of qgemv_big_kernel: the staging (LDS_X) or the half sums, then
// xd [G], 16 wave flags and the fixup's group list.
__host__ __device__ constexpr size_t big_xd_at(int G, bool lds_x) { return lds_x ? (size_t)G * 65 : kBigRedWords; }
__host__ __device__ constexpr size_t big_words(int G, bool lds_x) { return big_xd_at(G, lds_x) + G + 16 + kNzCap + 1; }

template <int MAXWGS, int D, bool LDS_X>
__global__ __launch_bounds__(MAXWGS) void qgemv_big_kernel(const uint16_t *__restrict__ x,
                                                         const uint32_t *__restrict__ packed,
                                                         const uint16_t *__restrict__ scales,
                                                         float *__restrict__ y, int64_t N, int G, int T) {
    extern __shared__ uint32_t smem[];
    x += (int64_t)blockIdx.y * G * kGroup;  // token blockIdx.y (one token unless batch-invariant)
    y += (int64_t)blockIdx.y * N;
    float *xd = reinterpret_cast<float *>(smem + big_xd_at(G, LDS_X));
    uint32_t *flags = smem + big_xd_at(G, LDS_X) + G;
    int *nz = reinterpret_cast<int *>(flags + 16);
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
    static_assert(2 * E * 32 <= kBigRedWords, "half-sum slots");
    uint32_t xp[64];
    int e = 0;
    RowBuf ring[E];
    bool fix = false;
    if constexpr (LDS_X) {
        XStage<4> st;  // 4G <= 4 * blockDim (T >= G, blockDim >= T)
        xstage_issue<4>(x, G, st);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            __builtin_amdgcn_sched_barrier(0);  // rows issued in ring order
            load_row(packed, scales, row0 + d * stride, N, W, G, g_load, ring[d]);
        }
        __builtin_amdgcn_sched_barrier(0);
        publish_flag(xstage_convert<4>(st, G, smem), flags);
        __syncthreads();
        xstage_fetch(smem, G, gl, lane_on, xp, e);
        fix = __builtin_amdgcn_readfirstlane(any_flag(flags) ? 1 : 0) != 0;  // the guard, workgroup-uniform
        __syncthreads();  // LDS is reused for the half sums below
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            load_row(packed, scales, row0 + d * stride, N, W, G, g_load, ring[d]);
        }
        __builtin_amdgcn_sched_barrier(0);
        publish_flag(xstage_lane(x, gl, lane_on, xp, e), flags);  // read after the loop's barriers
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
    if (!LDS_X) fix = any_flag(flags);  // published before the loop's barriers
    if (fix) {  // workgroup-uniform, rare
        __syncthreads();
        group_errors(x, G, xd);
        const int nnz = build_nz(0, G, [&](int g) { return xd[g] != 0.f; }, nz);
        const BlockRows rows{(int64_t)blockIdx.x, (int64_t)gridDim.x, R, N};
        if constexpr (MAXWGS > 512)
            fixup_m1_call(x, packed, scales, y, G, rows, xd, nz, nnz, tid, wgs);
        else
            fixup_outputs<1>(x, 0, 1, packed, scales, G, 0, G, rows, [&](int, int g) { return xd[g]; }, nz, nnz, false,
                             y, 0, tid, wgs);
    }
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
constexpr int kMfBatch = 8;  // tiles per cross-wave reduction
constexpr int kMfRing = 4;   // register ring slots (one super-step each)
constexpr int kMfAhead = 3;  // super-steps loaded ahead of the one decoded
// LDS: the converted activations (xs4, xe), the partial sums
// [2][kMfBatch][WAVES][16], then xd [G], 16 wave flags and the fixup's list.
template <int WAVES>
constexpr size_t mf_red_words() { return (size_t)2 * kMfBatch * WAVES * 16; }
template <int GPW, int WAVES>
constexpr size_t mf_lds() {
    return ((size_t)GPW * WAVES * 66 + mf_red_words<WAVES>() + 16 + kNzCap + 1) * 4;
}
struct MfSlot {
    u32x4v_t a, b, c;  // the lane's 12 words of one group of one row
    u32x2v_t s;        // (super-steps 0 and 4) the bf16 scales of lane row j's four groups
};

// First of the four groups that wave w (of WAVES, GPW groups each) handles in
// super-step q.
template <int GPW, int WAVES>
__device__ __forceinline__ int mf_group(int w, int q) {
    return 4 * WAVES * q + 4 * w;
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
    float *xd = reinterpret_cast<float *>(smem + G * 65 + mf_red_words<WAVES>());
    uint32_t *flags = smem + G * 66 + mf_red_words<WAVES>();
    int *nz = reinterpret_cast<int *>(flags + 16);
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
    const int64_t N = MULTI ? seg_pick(sg.rows, kseg) : sg.rows[0];
    // token blockIdx.y (one token unless batch-invariant)
    float *__restrict__ y = (MULTI ? seg_pick(sg.y, kseg) : sg.y[0]) + (int64_t)blockIdx.y * N;
    x += (int64_t)blockIdx.y * G * kGroup;
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
    publish_flag(xstage_convert<XU>(st, G, smem), flags);
    __syncthreads();
    const bool fix = __builtin_amdgcn_readfirstlane(any_flag(flags) ? 1 : 0) != 0;  // the guard, workgroup-uniform
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
    if (fix) {  // rare
        __syncthreads();
        group_errors(x, G, xd);
        const int nnz = build_nz(0, G, [&](int g) { return xd[g] != 0.f; }, nz);
        fixup_outputs<1>(x, 0, 1, packed, scales, G, 0, G, BlockRows{blk, nblk, 16, N},
                         [&](int, int g) { return xd[g]; }, nz, nnz, false, y, 0, threadIdx.x, blockDim.x);
    }
}

template <int T, bool MULTI>
qw3_status launch_gemv_small(const uint16_t *x, GemvSegs sg, int count, int G, hipStream_t stream, int M) {
    constexpr int R = kGemvWGS / T;
    const size_t lds = stage_words(G) * 4;
    const void *kern = reinterpret_cast<const void *>(&qgemv_small_kernel<T, MULTI, kGemvDepth>);
    int cus = 0, per_cu = 0;
    qw3_status st = cu_count(&cus);
    if (st == QW3_OK) st = blocks_per_cu(kern, kGemvWGS, lds, &per_cu);
    if (st != QW3_OK) return st;
    if (per_cu > 1) per_cu = 1;  // one workgroup per CU: more bytes in flight measured slower
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
        hipLaunchKernelGGL((qgemv_small_kernel<T, MULTI, 1>), dim3((unsigned)blocks, (unsigned)M), dim3(kGemvWGS),
                           lds, stream, x, sg, G);
    else
        hipLaunchKernelGGL((qgemv_small_kernel<T, MULTI, kGemvDepth>), dim3((unsigned)blocks, (unsigned)M),
                           dim3(kGemvWGS), lds, stream, x, sg, G);
    return check_launch();
}

template <bool MULTI>
qw3_status launch_gemv_small_any(const uint16_t *x, const GemvSegs &sg, int count, int G, hipStream_t stream,
                                 int M = 1) {
    if (G <= 1) return launch_gemv_small<1, MULTI>(x, sg, count, G, stream, M);
    if (G <= 2) return launch_gemv_small<2, MULTI>(x, sg, count, G, stream, M);
    if (G <= 4) return launch_gemv_small<4, MULTI>(x, sg, count, G, stream, M);
    if (G <= 8) return launch_gemv_small<8, MULTI>(x, sg, count, G, stream, M);
    if (G <= 16) return launch_gemv_small<16, MULTI>(x, sg, count, G, stream, M);
    if (G <= 32) return launch_gemv_small<32, MULTI>(x, sg, count, G, stream, M);
    return launch_gemv_small<64, MULTI>(x, sg, count, G, stream, M);
}

qw3_status launch_gemv_big(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                           int64_t N, int G, hipStream_t stream, int M) {
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
    const bool lds_x = (size_t)G * 65 * 4 <= kMaxLdsX;
    constexpr int kBigD = kGemvDepth, kHugeD = 1;
    const size_t lds = big_words(G, lds_x) * 4;
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
                       dim3((unsigned)blocks, (unsigned)M), dim3(wgs), lds, stream, x, packed, scales, y, N, G, T);
    return check_launch();
}

// The matrix-core GEMV: one workgroup per CU, workgroups dealt to the
// matrices in proportion to their 16-row tiles, at least one and at most one
// per tile each (4 waves x 16 groups at K = 8192).
template <int GPW, int WAVES, bool MULTI>
qw3_status launch_gemv_mfma(const uint16_t *x, GemvSegs sg, int count, hipStream_t stream, int M = 1) {
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
            b = (int64_t)cus * tiles[i] / tot;
            b = b < 1 ? 1 : (b > tiles[i] ? tiles[i] : b);
        }
        blocks += b;
        sg.blk_end[i] = (int)blocks;
    }
    const size_t lds = mf_lds<GPW, WAVES>();
    hipLaunchKernelGGL((qgemv_mfma_kernel<GPW, WAVES, MULTI>), dim3((unsigned)blocks, (unsigned)M), dim3(64 * WAVES),
                       lds, stream, x, sg);
    return check_launch();
}

// Whether the matrix-core GEMV takes a matrix: K = 8192 (4 waves x 16 groups)
// or 16384 (4 waves x 32 groups), scale rows 8-byte aligned (8-byte scale
// loads) and at least four 16-row tiles per CU (with fewer it is no faster
// than the lane-per-group kernel).  At K = 28672
// (7 waves x 32 groups) it measured no faster than qgemv_big_kernel on the
// 8192-row down projection, two tiles per CU, so it is not used there.  The
// choice depends on the matrix alone, so a matrix gets the same kernel -- and
// the same bits -- from qgemv_w3g128 and from qgemv_w3g128_multi.
bool gemv_mfma_takes(int G, const uint16_t *scales, int64_t N) {
    if ((G != 64 && G != 128) || N == 0 || !aligned(scales, 8)) return false;
    int cus = 0;
    if (cu_count(&cus) != QW3_OK) return false;
    return ceil_div(N, 16) >= 4 * (int64_t)cus;
}

}  // namespace

// M > 1 (the batch-invariant product): the same launch with a token grid
// dimension, token m reading x + m K and writing y + m N.
qw3_status qw3_shared::launch_gemv(const uint16_t *x, const uint32_t *packed, const uint16_t *scales, float *y,
                                   int64_t N, int64_t K, hipStream_t stream, int M) {
    const int G = (int)(K / kGroup);
    if (gemv_mfma_takes(G, scales, N)) {
        GemvSegs sg = {};
        sg.packed[0] = packed;
        sg.scales[0] = scales;
        sg.y[0] = y;
        sg.rows[0] = N;
        return G == 64 ? launch_gemv_mfma<16, 4, false>(x, sg, 1, stream, M)
                       : launch_gemv_mfma<32, 4, false>(x, sg, 1, stream, M);
    }
    if (G <= 64) {
        GemvSegs sg = {};
        sg.packed[0] = packed;
        sg.scales[0] = scales;
        sg.y[0] = y;
        sg.rows[0] = N;
        return launch_gemv_small_any<false>(x, sg, 1, G, stream, M);
    }
    return launch_gemv_big(x, packed, scales, y, N, G, stream, M);
}

// Several matrices sharing x: one launch when rows fit one wave (K <= 8192),
// else one launch per matrix.
qw3_status qw3_shared::launch_gemv_multi(const uint16_t *x, int count, const uint32_t *const *packed,
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
