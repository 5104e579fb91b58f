/*
 * qw3.h -- C ABI of the W3G128 fused dequantize-and-multiply library (gfx950).
 *
 * W3G128 is the weight format of the GSQ model card
 * "Llama-3.1-70B-Instruct-3Bit-GSQ" (sections "Quantization details" and
 * "Storage layout"): a Linear layer with original weight [N = out_features,
 * K = in_features] is stored as
 *   packed  int32 [N, 3K/32]   exact-width 3-bit codes, no padding
 *   scales  bf16  [N, K/128]   one scale per group of 128 inputs
 * with a symmetric integer codebook times the group scale and no zero point.
 * This library reads it as follows (readings of points the card leaves open):
 *   - each row is one little-endian bitstream: code k of row n occupies stream
 *     bits 3k (least significant) to 3k+2, and stream bit j is bit (j mod 32)
 *     of word (j div 32) of that row; the int32 container is read as raw bits;
 *   - code c in 0..7 stands for the integer q = c - 4, so the weight is
 *     w[n][k] = scales[n][k / 128] * (c[n][k] - 4).
 * The fused operation is Y = X * dequant(W)^T (GLQ README, section
 * "Inference kernels"), computed without ever writing the dense weight.
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     never frees them.  Arrays are row-major and contiguous.
 *   - bf16 values are passed as their raw 16-bit patterns (uint16_t).
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL means the default
 *     stream) and returns without waiting for it; outputs are overwritten,
 *     never accumulated into.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     error status means nothing was launched and no output was touched.
 *     QW3_ERR_HIP means the HIP runtime refused a launch or an allocation
 *     (the message of the last HIP error is kept by qw3_last_hip_error()).
 *   - Shapes: 0 <= N, 0 <= M, 0 <= K <= QW3_MAX_K and K % 128 == 0.  A size
 *     of zero is valid and enqueues no work (for K == 0 the outputs of the
 *     products are filled with zeros, the value of an empty sum).
 *   - Alignment: `codes`, `packed`, `x` and `w_out` must be 16-byte aligned,
 *     `scales` 2-byte and `y` 4-byte aligned, else QW3_ERR_ALIGN.
 *   - Each call is deterministic: the same inputs give bit-identical outputs
 *     on every run (all reductions run in a fixed order, no atomics).
 *   - Inputs must be finite; NaN or Inf in x or scales give unspecified y.
 *     The products also assume every |s| * |x| below 2^100 and every
 *     sum_k |x_k w_k| below 2^120 (far inside fp32), so that no partial sum
 *     overflows; outside that y is unspecified.
 *   - Accuracy of the products, for every input in that domain whatever the
 *     spread of magnitudes within x or within a row's scales:
 *       |y - sum_k x_k w_k| <= 1e-4 * sum_k |x_k w_k| + 1e-6   per output.
 *     The fast paths multiply fp16 operands; the elements that their
 *     conversion may round (activations about 2^21 below the largest of their
 *     exponent set, scales more than 2^21 below the largest of their row on
 *     the many-token tiles) are tracked, and every output whose error bound
 *     could exceed 2^-21 is recomputed in fp32 by the same call.
 */
#ifndef QW3_H
#define QW3_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int qw3_status;

enum {
    QW3_OK = 0,
    QW3_ERR_NULL = -1,  /* a required pointer is NULL                        */
    QW3_ERR_SHAPE = -2, /* negative size, K % 128 != 0, or K > QW3_MAX_K      */
    QW3_ERR_ALIGN = -3, /* a pointer is not aligned as stated above           */
    QW3_ERR_HIP = -4,   /* the HIP runtime reported an error                  */
    QW3_ERR_CAPTURE = -5, /* qgemm_w3g128_smallM would have to allocate its
                             workspace while the stream is being captured      */
    QW3_ERR_SCRATCH = -6  /* qgemm_w3g128_smallM_noalloc needs more than
                             QW3_NOALLOC_SCRATCH_BYTES of scratch               */
};

/* Largest supported in_features (1024 groups of 128). */
#define QW3_MAX_K 131072

/*
 * qpack_uint3 -- pack 3-bit codes into the exact-width int32 stream.
 *   codes  [N, K] uint8, values 0..7 (only the low 3 bits of each byte are
 *          used; larger values are a caller error)
 *   packed [N, 3K/32] int32, written
 * Storage layout of the GSQ model card: the codes are packed at their exact
 * 3-bit width with no padding bits, so a [28672, 8192] weight becomes
 * [28672, 768] words.
 */
qw3_status qpack_uint3(const uint8_t *codes, int32_t *packed, int64_t N, int64_t K,
                       void *hip_stream);

/*
 * qrepack_w4c_uint3 -- repack the 4-bit-container intermediate into the
 * exact-width stream.
 *   w4     [N, K/8] int32: the codes as GSQ training writes them before the
 *          checkpoint is re-packed (GSQ model card, "Storage layout": training
 *          first keeps each 3-bit code in a 4-bit slot of int32 words).  Reading taken: code
 *          k of a row is nibble k % 8 of word k / 8 of that row, least
 *          significant nibble first, in the nibble's low 3 bits; the top bit of
 *          each nibble is padding and ignored.
 *   packed [N, 3K/32] int32, written: the same codes, exactly as qpack_uint3
 *          stores them.
 * Both pointers 16-byte aligned.  Validation and errors as for qpack_uint3.
 */
qw3_status qrepack_w4c_uint3(const int32_t *w4, int32_t *packed, int64_t N, int64_t K,
                             void *hip_stream);

/*
 * qdequant_bf16 -- expand packed codes into a dense bf16 weight.
 *   packed [N, 3K/32] int32, scales [N, K/128] bf16
 *   w_out  [N, K] bf16, written: w_out[n][k] = RNE_bf16(scales[n][k/128] * (c - 4))
 * The product is exact in fp32 and rounded once to bf16, nearest-even.  This
 * is the dense "dequantize then matmul" branch of the GLQ README ("How it
 * works": CPU and fallback paths dequantize instead of fusing).
 */
qw3_status qdequant_bf16(const int32_t *packed, const uint16_t *scales, uint16_t *w_out,
                         int64_t N, int64_t K, void *hip_stream);

/*
 * qgemv_w3g128 -- fused batch-1 product y = dequant(W) x.
 *   x [K] bf16, packed [N, 3K/32] int32, scales [N, K/128] bf16
 *   y [N] float32, written: y[n] = sum_k x[k] * scales[n][k/128] * (c[n][k] - 4)
 * The packed weights are streamed from memory once; the dense weight is never
 * formed (GLQ README, "Inference kernels").  fp32 accumulation; the result is
 * within 1e-4 * sum_k |x[k] w[n][k]| + 1e-6 of the exact sum (see the
 * accuracy note above).  Uses no device memory beyond its arguments.
 */
qw3_status qgemv_w3g128(const uint16_t *x, const int32_t *packed, const uint16_t *scales,
                        float *y, int64_t N, int64_t K, void *hip_stream);

/* Largest number of matrices in one qgemv_w3g128_multi call. */
#define QW3_MAX_MULTI 4

/*
 * qgemv_w3g128_multi -- qgemv_w3g128 for `count` (1..QW3_MAX_MULTI) matrices
 * that share one activation vector and the same K, e.g. the q, k and v
 * projections of a decoder layer, in one launch (one activation staging):
 *   x [K] bf16; for i < count: packed[i] [N[i], 3K/32] int32,
 *   scales[i] [N[i], K/128] bf16, y[i] [N[i]] float32, written.
 * `packed`, `scales`, `y` and `N` are HOST arrays of `count` entries holding
 * device pointers (and row counts).  Each y[i] equals what qgemv_w3g128 gives
 * for matrix i, bit for bit.  Validation and errors as for qgemv_w3g128 (a
 * count outside 1..QW3_MAX_MULTI is QW3_ERR_SHAPE); N[i] == 0 skips matrix i.
 * For K > 8192 the matrices are launched one after another.
 */
qw3_status qgemv_w3g128_multi(const uint16_t *x, int32_t count, const int32_t *const *packed,
                              const uint16_t *const *scales, float *const *y, const int64_t *N,
                              int64_t K, void *hip_stream);

/*
 * qgemm_w3g128_smallM -- fused product for M activation rows, Y = X dequant(W)^T.
 *   x [M, K] bf16 (row stride K), packed [N, 3K/32] int32, scales [N, K/128] bf16
 *   y [M, N] float32, written: y[m][n] = sum_k x[m][k] * scales[n][k/128] * (c[n][k] - 4)
 * Any M >= 0 is accepted.  M == 1 runs the batch-1 kernel; small M streams
 * the weights once for the whole batch through bf16-exact fp16 matrix-core
 * products; large M (prefill) runs a tiled matrix-core kernel.  Same accuracy
 * bound as qgemv_w3g128.
 *
 * Workspace.  The call uses device scratch owned by the library, one buffer
 * per (device, stream handle): the
 * activations converted to fp16 (2 bytes per element, M rounded up to 16 or
 * 32 per pass, or to whole 256-token tiles), per-group error masses
 * (4 bytes per token and group) and, when K is split across workgroups, fp32
 * partial sums (4 bytes per output element and K chunk).  Exceptions: M == 1
 * uses none; 2 <= M <= 8 with 8-byte aligned scale rows and K a multiple of
 * 1024 converts the activations inside the kernel and uses only the partial
 * sums, and only when K is split: into K / (1024 w) chunks, w the largest of
 * 1..8 dividing K / 1024 (K = 8192 or 4096: one chunk, no workspace;
 * K = 28672: w = 7, four chunks).
 *   - The first call on a stream allocates its buffer (hipMalloc).  A later
 *     call that needs more allocates a buffer at least twice as large; the
 *     superseded one is never freed or reused while the process runs, so work
 *     queued earlier and graphs captured earlier stay valid.  Buffers are held
 *     until the process ends.  The library never synchronizes a stream.
 *   - Calls on one stream run in order and share its buffer; calls on
 *     different streams use different buffers and may overlap.  Streams are
 *     told apart by handle: before destroying a stream that has calls of this
 *     library queued, wait for them (hipStreamSynchronize), since a stream
 *     created later at the same address takes over the same buffer.
 *   - Graph capture: a call captured on a stream uses that stream's buffer as
 *     it is at capture time.  If the buffer would have to grow during capture
 *     the call returns QW3_ERR_CAPTURE and enqueues nothing; make one call of
 *     the largest size on the stream before capturing.  Replays stay valid
 *     after later, larger calls on the stream (the old buffer is kept).
 */
qw3_status qgemm_w3g128_smallM(const uint16_t *x, const int32_t *packed,
                               const uint16_t *scales, float *y, int64_t M, int64_t N,
                               int64_t K, void *hip_stream);

/* Largest M of one qgemm_w3g128_batch_invariant call. */
#define QW3_MAX_BATCH_INVARIANT_M 65535

/*
 * qgemm_w3g128_batch_invariant -- the M-row product with every row computed
 * exactly as the batch-1 product computes it.  The GLQ README ("Inference
 * kernels") ties its fixed-order reductions to reproducible outputs at batch
 * 1 and in batched prefill.  qgemm_w3g128_smallM is deterministic run to run,
 * but its batched and tiled kernels add a row's products in other orders than
 * the batch-1 kernel, so its rows agree with qgemv_w3g128 only within the
 * accuracy bound; here a row's bits do not depend on the batch.
 *   x [M, K] bf16 (row stride K), packed [N, 3K/32] int32, scales [N, K/128] bf16
 *   y [M, N] float32, written: row m equals, bit for bit, what qgemv_w3g128
 *   writes for x row m (the same kernel with a token grid dimension, in one
 *   launch).
 * It reads the weights once per row of x (M times the batch-1 traffic, partly
 * served from the caches), so it is for callers that need outputs independent
 * of the batch, not for throughput.  0 <= M <= QW3_MAX_BATCH_INVARIANT_M,
 * else QW3_ERR_SHAPE; other validation, alignment and errors as for
 * qgemv_w3g128.  Uses no device memory beyond its arguments.
 */
qw3_status qgemm_w3g128_batch_invariant(const uint16_t *x, const int32_t *packed,
                                        const uint16_t *scales, float *y, int64_t M, int64_t N,
                                        int64_t K, void *hip_stream);

/* Device scratch of qgemm_w3g128_smallM_noalloc, per device (128 MiB). */
#define QW3_NOALLOC_SCRATCH_BYTES (128ull << 20)

/*
 * qgemm_w3g128_smallM_noalloc -- qgemm_w3g128_smallM for callers that cannot
 * allocate device memory: code under graph capture that has not sized a
 * workspace, tight serving loops, harnesses that forbid hipMalloc.
 *   Same arguments, layout, validation, accuracy and results as
 *   qgemm_w3g128_smallM (the same kernels; bit-identical outputs).
 *   Scratch comes from a static device array of QW3_NOALLOC_SCRATCH_BYTES
 *   that the library holds on every device it runs on until the process
 *   ends; the call itself never allocates, frees or synchronizes.  A call
 *   that needs more scratch returns QW3_ERR_SCRATCH and enqueues nothing.
 *   Needs, in bytes (Mp = M rounded up to 16 or 32 per batched pass, or to
 *   whole 256-token tiles; G = K / 128; C = K chunks):
 *     batched decode  2 Mp K + 5 G Mp + 4 C Mp N   (about 9 MiB for 32 tokens
 *                     against either MLP matrix of a 70B layer);
 *     prefill         2 Mp K + 4 Mp (G + 2) + 4 C M N  (about 97 MiB for 512
 *                     tokens against an 8192 x 28672 matrix).
 *   All calls on one device share the array: calls that overlap in time on
 *   one device (different streams, or graph replays) race and must be
 *   ordered by the caller.
 */
qw3_status qgemm_w3g128_smallM_noalloc(const uint16_t *x, const int32_t *packed,
                                       const uint16_t *scales, float *y, int64_t M, int64_t N,
                                       int64_t K, void *hip_stream);

/* Text for a status code (static storage, never NULL). */
const char *qstatus_str(qw3_status status);

/* Text of the last HIP error seen by this library in the calling thread. */
const char *qw3_last_hip_error(void);

/* ABI version of this header (increments on incompatible change). */
int qw3_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QW3_H */
