"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Packing and dequantization must match the oracle bit for bit.  Products must
satisfy |y_gpu - y_ref| <= 1e-4 * a + 1e-6 per element, where y_ref is the
oracle's fp64 sum with exact products and a = sum_k |x_k w_k| (the tolerance
the workload statement fixes).  Inputs come from `synth` (seeded); the oracle
packs its own copy of the codes, so the two sides share only the raw draws.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

RTOL = 1e-4
ATOL = 1e-6


def q():
    import dequant_gemv_qgemv_amd as mod
    return mod


def say(*args):
    print("[gpu-case]", *args, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def assert_close(y_gpu, y_ref, a, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    err = np.abs(y_gpu - y_ref)
    bound = RTOL * a + ATOL
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d outside |err| <= 1e-4*a + 1e-6; first %s: gpu %s ref %s a %s"
                             % (what, int(bad.sum()), bad.size, idx.tolist(),
                                [y_gpu[tuple(i)] for i in idx], [y_ref[tuple(i)] for i in idx],
                                [a[tuple(i)] for i in idx]))


def gpu_pack(codes: np.ndarray) -> torch.Tensor:
    return q().qpack_uint3(dev(codes))


# ------------------------------------------------------------ pack/dequant --

PACK_SHAPES = [(256, 1024), (37, 384), (1, 128), (5, 28672), (300, 256), (3, 131072)]


@pytest.mark.parametrize("n,k", PACK_SHAPES)
def test_qpack_bit_exact(n, k):
    say("qpack", n, k)
    c = synth.codes_all8(1000 + n + k, n, k)
    got = host(gpu_pack(c)).view(np.uint32)
    assert np.array_equal(got, oracle.pack(c))


def test_qpack_tiny_case_and_golden_rows():
    c, _, _ = synth.tiny_case()
    say("qpack tiny")
    assert np.array_equal(host(gpu_pack(c)).view(np.uint32), oracle.pack(c))
    rows = np.stack([np.full(128, 4, np.uint8), np.full(128, 7, np.uint8), np.zeros(128, np.uint8),
                     (np.arange(128) % 8).astype(np.uint8)])
    assert np.array_equal(host(gpu_pack(rows)).view(np.uint32), oracle.pack(rows))


# 4-bit-container intermediate (GSQ model card, "Storage layout" note), random
# words: every nibble value, padding bits included.
@pytest.mark.parametrize("n,k", [(256, 1024), (37, 384), (1, 128), (5, 28672), (300, 256), (3, 131072)])
def test_qrepack_w4c_bit_exact(n, k):
    say("qrepack_w4c", n, k)
    rng = np.random.default_rng(900 + k)
    w4 = rng.integers(0, 2 ** 32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
    got = host(q().qrepack_w4c_uint3(dev(w4))).view(np.uint32)
    assert np.array_equal(got, oracle.repack_w4c(w4))


def test_qrepack_w4c_then_gemv_matches_pack_path():
    """Repacked containers drive the GEMV exactly like codes packed directly."""
    n, k = 300, 8192
    c = synth.codes_all8(910, n, k)
    s = synth.scales(911, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(912, 1, k)
    sh = (4 * np.arange(8)).astype(np.uint32)
    w4 = (c.reshape(n, k // 8, 8).astype(np.uint32) << sh).sum(axis=2, dtype=np.uint64).astype(np.uint32)
    w4 |= np.uint32(0x88888888)  # padding bits set: ignored
    say("qrepack_w4c then qgemv")
    packed = q().qrepack_w4c_uint3(dev(w4))
    assert np.array_equal(host(packed).view(np.uint32), oracle.pack(c))
    y = host(q().qgemv_w3g128(dev(x.reshape(-1)), packed, dev(s)))
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "repacked gemv")


@pytest.mark.parametrize("n,k", [(256, 1024), (37, 384), (7, 28672), (2, 131072)])
def test_qdequant_bit_exact(n, k):
    say("qdequant", n, k)
    c = synth.codes_all8(2000 + n, n, k)
    s = synth.scales(2100 + n, n, k // 128, sigma=0.7, eps=1e-3)
    packed = gpu_pack(c)
    w = host(q().qdequant_bf16(packed, dev(s))).view(np.uint16)
    assert np.array_equal(w, oracle.dequant_bf16(oracle.pack(c), s, k))


def test_qdequant_negative_and_tiny_scales():
    n, k = 16, 256
    c = synth.codes_all8(7, n, k)
    s = synth.f32_to_bf16_bits(np.random.default_rng(8).standard_normal((n, 2)).astype(np.float32) * 1e-30)
    say("qdequant signed tiny scales")
    w = host(q().qdequant_bf16(gpu_pack(c), dev(s))).view(np.uint16)
    assert np.array_equal(w, oracle.dequant_bf16(oracle.pack(c), s, k))


# ------------------------------------------------------------------ GEMV ---

def run_gemv(c, s, x):
    n, k = c.shape
    packed = gpu_pack(c)
    return host(q().qgemv_w3g128(dev(x.reshape(-1)), packed, dev(s)))


def ref_gemv(c, s, x):
    y, a = oracle.gemm(x.reshape(1, -1), oracle.pack(c), s, c.shape[1])
    return y[0], a[0]


def test_qgemv_tiny_case():
    c, s, x = synth.tiny_case()
    say("qgemv tiny 256x1024")
    y = run_gemv(c, s, x)
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "tiny")


# G = K/128 values that hit every team size of the GEMV kernel, ragged N
GEMV_SHAPES = [(1, 128), (37, 256), (5, 384), (40, 640), (33, 1152), (17, 2176), (70, 4096),
               (9, 8064), (300, 8192), (11, 8320), (6, 12800), (8, 28672), (3, 38400),
               (4, 65536), (2, 131072)]


@pytest.mark.parametrize("n,k", GEMV_SHAPES)
def test_qgemv_parity_all_codes(n, k):
    say("qgemv", n, k)
    c = synth.codes_all8(3000 + k, n, k)
    s = synth.scales(3100 + k, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(3200 + k, 1, k)
    y = run_gemv(c, s, x)
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "qgemv %dx%d" % (n, k))


def test_qgemv_zero_rows_and_one_hot():
    n, k = 64, 1024
    c = np.full((n, k), 4, dtype=np.uint8)
    c[1::2, 5] = 7  # odd rows: one weight, q = +3
    s = synth.scales(41, n, k // 128, sigma=0.1, eps=1e-3)
    x = synth.activations(42, 1, k)
    say("qgemv zero rows")
    y = run_gemv(c, s, x)
    assert np.all(y[0::2] == 0.0)
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "zero rows")
    xh = np.zeros((1, k), dtype=np.uint16)
    xh[0, 5] = 0x4040  # 3.0
    y = run_gemv(c, s, xh)
    sf = synth.bf16_bits_to_f32(s)
    assert np.all(y[1::2] == 9.0 * sf[1::2, 0])  # exact: 3 * 3 * s


def test_qgemv_wide_activation_range():
    """Per-group exponent handling: huge, tiny and mixed magnitudes."""
    n, k = 48, 1024
    c = synth.codes_all8(51, n, k)
    s = synth.scales(52, n, k // 128, sigma=0.05, eps=1e-3)
    rng = np.random.default_rng(53)
    xf = rng.standard_normal(k).astype(np.float32)
    xf[:128] *= np.float32(2.0 ** 60)
    xf[128:256] *= np.float32(2.0 ** -60)
    xf[256:384] *= np.exp2(rng.integers(-12, 12, 128)).astype(np.float32)  # 24 binades in one group
    xf[384:512] = 0.0
    x = synth.f32_to_bf16_bits(xf)
    say("qgemv wide range")
    y = run_gemv(c, s, x)
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "wide range")


def test_qgemv_k_zero_and_n_zero():
    mod = q()
    say("qgemv K=0 / N=0")
    packed = torch.empty((5, 0), dtype=torch.int32, device="cuda")
    scales = torch.empty((5, 0), dtype=torch.int16, device="cuda")
    x = torch.empty((0,), dtype=torch.int16, device="cuda")
    y = torch.full((5,), 7.0, device="cuda")
    mod.qgemv_w3g128(x, packed, scales, out=y)
    assert host(y).tolist() == [0.0] * 5
    y0 = mod.qgemv_w3g128(torch.zeros(1024, dtype=torch.int16, device="cuda"),
                          torch.empty((0, 96), dtype=torch.int32, device="cuda"),
                          torch.empty((0, 8), dtype=torch.int16, device="cuda"))
    assert y0.shape == (0,)


def test_qgemv_deterministic():
    n, k = 4096, 8192
    c = synth.codes(61, n, k)
    s = synth.scales(62, n, k // 128)
    x = synth.activations(63, 1, k)
    say("qgemv determinism")
    packed, sd, xd = gpu_pack(c), dev(s), dev(x.reshape(-1))
    y1 = host(q().qgemv_w3g128(xd, packed, sd))
    y2 = host(q().qgemv_w3g128(xd, packed, sd))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_binding_rejects_misaligned_view():
    mod = q()
    k = 1024
    big = torch.zeros(k + 8, dtype=torch.int16, device="cuda")
    packed = torch.zeros((4, 96), dtype=torch.int32, device="cuda")
    scales = torch.zeros((4, 8), dtype=torch.int16, device="cuda")
    say("qgemv misaligned")
    with pytest.raises(mod.Qw3Error) as ei:
        mod.qgemv_w3g128(big[1:k + 1], packed, scales)
    assert ei.value.status == mod.QW3_ERR_ALIGN


# ------------------------------------ batch 1 on the matrix cores, K = 8192 --
# qgemv_w3g128 runs its matrix-core kernel for K = 8192 when the matrix has at
# least four 16-row tiles per CU (N >= 16384 rows on a 256-CU part) and its
# scale rows are 8-byte aligned; these cases are sized to take it.

MF_K = 8192


# (K = 16384: 32 groups per wave; the K = 28672 cases check the lane-per-group
# kernel at the same sizes; 16300 rows at K = 16384 stay below four tiles per CU)
@pytest.mark.parametrize("n,k", [(16411, MF_K), (17000, MF_K), (16400, 16384), (16300, 16384), (8200, 28672),
                                 (8213, 28672)])
def test_qgemv_mfma_parity_all_codes(n, k):
    say("qgemv matrix cores", n, k)
    c = synth.codes_all8(7000 + n, n, k)
    s = synth.scales(7100 + n, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(7200 + n, 1, k)
    y = run_gemv(c, s, x)
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "qgemv matrix cores %dx%d" % (n, k))


def test_qgemv_mfma_zero_rows_and_one_hot():
    """Rows of code 4 give exact zeros; one nonzero weight per row, anywhere
    in the row, gives the exact product."""
    n = 16400
    c = np.full((n, MF_K), 4, dtype=np.uint8)
    odd = np.arange(1, n, 2)
    col = (odd * 131) % MF_K  # every group, block and pair slot
    c[odd, col] = 7  # q = +3
    s = synth.scales(71, n, MF_K // 128, sigma=0.1, eps=1e-3)
    say("qgemv matrix cores zero rows")
    x3 = np.full((1, MF_K), 0x4040, dtype=np.uint16)  # 3.0 everywhere
    y = run_gemv(c, s, x3)
    assert np.all(y[0::2] == 0.0)
    sf = synth.bf16_bits_to_f32(s)
    assert np.array_equal(y[odd], (9.0 * sf[odd, col // 128]).astype(np.float32))
    x = synth.activations(72, 1, MF_K)
    y = run_gemv(c, s, x)
    assert np.all(y[0::2] == 0.0)
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "matrix cores one-hot")


def test_qgemv_mfma_wide_activation_range():
    n = 16400
    c = synth.codes_all8(73, n, MF_K)
    s = synth.scales(74, n, MF_K // 128, sigma=0.05, eps=1e-3)
    rng = np.random.default_rng(75)
    xf = rng.standard_normal(MF_K).astype(np.float32)
    xf[:128] *= np.float32(2.0 ** 60)
    xf[128:256] *= np.float32(2.0 ** -60)
    xf[256:384] *= np.exp2(rng.integers(-12, 12, 128)).astype(np.float32)
    xf[384:512] = 0.0
    xf[4096:4224] *= np.float32(2.0 ** -100)
    x = synth.f32_to_bf16_bits(xf)
    say("qgemv matrix cores wide range")
    y = run_gemv(c, s, x)
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "matrix cores wide range")


@pytest.mark.parametrize("offset_elems", [4, 1])
def test_qgemv_mfma_scale_views(offset_elems):
    """Scales 8-byte aligned but not 16 (matrix cores), and only 2-byte aligned
    (the lane-per-group kernel takes the matrix): both match the oracle."""
    n = 16400
    c = synth.codes(76, n, MF_K)
    s = synth.scales(77, n, MF_K // 128)
    x = synth.activations(78, 1, MF_K)
    packed, xd = gpu_pack(c), dev(x.reshape(-1))
    base = torch.zeros(n * 64 + 8, dtype=torch.int16, device="cuda")
    view = base[offset_elems:offset_elems + n * 64].view(n, 64)
    view.copy_(dev(s))
    say("qgemv matrix cores scale view offset", offset_elems)
    y = host(q().qgemv_w3g128(xd, packed, view))
    yr, a = ref_gemv(c, s, x)
    assert_close(y, yr, a, "scale view +%d" % offset_elems)
    y_al = host(q().qgemv_w3g128(xd, packed, dev(s)))
    if offset_elems == 4:
        assert np.array_equal(y.view(np.uint32), y_al.view(np.uint32))


def test_qgemv_mfma_deterministic():
    n = 16400
    c = synth.codes(79, n, MF_K)
    s = synth.scales(80, n, MF_K // 128)
    x = synth.activations(81, 1, MF_K)
    say("qgemv matrix cores determinism")
    packed, sd, xd = gpu_pack(c), dev(s), dev(x.reshape(-1))
    y1 = host(q().qgemv_w3g128(xd, packed, sd))
    y2 = host(q().qgemv_w3g128(xd, packed, sd))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


# -------------------------------------------------- several matrices, one x --

@pytest.mark.parametrize("k,ns", [(8192, (300, 40, 40)), (1024, (5, 0, 77, 130)), (2048, (64,)),
                                  (28672, (40, 24)), (8192, (16411, 300, 0, 17000)), (8192, (16400, 16411))])
def test_qgemv_multi_matches_single(k, ns):
    say("qgemv multi", k, ns)
    x = synth.activations(5000 + k, 1, k)
    xd = dev(x.reshape(-1))
    mats = []
    for i, n in enumerate(ns):
        c = synth.codes_all8(5100 + i, n, k)
        s = synth.scales(5200 + i, n, k // 128, sigma=0.02, eps=1e-3)
        mats.append((c, s, gpu_pack(c), dev(s)))
    ys = [host(o) for o in q().qgemv_w3g128_multi(xd, [(p, sd) for _, _, p, sd in mats])]
    for (c, s, p, sd), y in zip(mats, ys):
        assert np.array_equal(y.view(np.uint32), host(q().qgemv_w3g128(xd, p, sd)).view(np.uint32))
        if c.shape[0]:
            yr, a = oracle.gemm(x, oracle.pack(c), s, k)
            assert_close(y[None, :], yr, a, "multi")


# ----------------------------------------------- batch-invariant product --

@pytest.mark.parametrize("m,n,k", [(1, 37, 256), (5, 300, 1024), (3, 130, 8192), (4, 16400, 8192),
                                   (2, 16400, 16384), (7, 200, 28672), (2, 9, 131072)])
def test_batch_invariant_rows_equal_gemv(m, n, k):
    """Every row of qgemm_w3g128_batch_invariant equals qgemv_w3g128 on that
    activation row bit for bit (the lane-per-group, matrix-core and long-row
    kernels), and the rows meet the tolerance against the oracle."""
    say("batch invariant", m, n, k)
    c = synth.codes_all8(5300 + m, n, k)
    s = synth.scales(5301 + m, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(5302 + m, m, k)
    p, sd, xd = gpu_pack(c), dev(s), dev(x)
    y = host(q().qgemm_w3g128_batch_invariant(xd, p, sd))
    for r in range(m):
        yr1 = host(q().qgemv_w3g128(xd[r].contiguous(), p, sd))
        assert np.array_equal(y[r].view(np.uint32), yr1.view(np.uint32)), r
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "batch invariant")


def test_batch_invariant_largest_m():
    """M = QW3_MAX_BATCH_INVARIANT_M rows (one grid row per token): every row
    against the oracle, a sample of rows bit for bit against qgemv_w3g128."""
    m, n, k = q().QW3_MAX_BATCH_INVARIANT_M, 3, 256
    say("batch invariant, largest M", m)
    c = synth.codes_all8(5320, n, k)
    s = synth.scales(5321, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(5322, m, k)
    p, sd, xd = gpu_pack(c), dev(s), dev(x)
    y = host(q().qgemm_w3g128_batch_invariant(xd, p, sd))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "batch invariant, largest M")
    for r in (0, 1, 4097, m // 2, m - 2, m - 1):
        assert np.array_equal(y[r].view(np.uint32), host(q().qgemv_w3g128(xd[r].contiguous(), p, sd)).view(np.uint32))


def test_batch_invariant_wide_range_rows_take_the_fixup():
    """Rows whose activations defeat the fast conversion (large values on
    code-4 weights, tiny ones elsewhere) go through the exact recompute in
    the batch-1 kernel; their rows still equal qgemv_w3g128's and meet the
    tolerance, next to ordinary rows."""
    m, n, k = 3, 64, 1024
    rng = np.random.default_rng(5310)
    c = rng.integers(0, 8, size=(n, k)).astype(np.uint8)
    c[:, ::8] = 4
    s = synth.scales(5311, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(5312, m, k)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    xf[1] *= 2.0 ** -22
    xf[1, ::8] = rng.standard_normal(k // 8) * 2.0 ** 12
    x = synth.f32_to_bf16_bits(xf.astype(np.float32))
    p, sd, xd = gpu_pack(c), dev(s), dev(x)
    y = host(q().qgemm_w3g128_batch_invariant(xd, p, sd))
    for r in range(m):
        assert np.array_equal(y[r].view(np.uint32), host(q().qgemv_w3g128(xd[r].contiguous(), p, sd)).view(np.uint32))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "batch invariant, wide range")


def test_qgemv_multi_qkv_full_size():
    names = ("q_proj", "k_proj", "v_proj")
    k = synth.LAYER_70B["q_proj"][1]
    x = synth.layer_x(1, k)
    xd = dev(x.reshape(-1))
    mats = [synth.layer_weights(nm) for nm in names]
    packed = [gpu_pack(c) for c, _ in mats]
    say("qgemv multi q/k/v full size")
    ys = q().qgemv_w3g128_multi(xd, [(p, dev(s)) for p, (_, s) in zip(packed, mats)])
    for (c, s), y in zip(mats, ys):
        yr, a = oracle.gemm(x, oracle.pack(c), s, k)
        assert_close(host(y)[None, :], yr, a, "multi full size")


# ------------------------------------------------------------- small M ----

@pytest.mark.parametrize("m", [2, 3, 4, 5, 7, 8, 16, 17, 31, 32, 33, 64, 100])
@pytest.mark.parametrize("n,k", [(200, 1024), (70, 8192), (24, 28672)])
def test_qgemm_parity(m, n, k):
    say("qgemm", m, n, k)
    c = synth.codes_all8(4000 + n + k, n, k)
    s = synth.scales(4100 + k, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(4200 + m, m, k)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), dev(s)))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "qgemm M=%d %dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(5, 48, 16384), (16, 40, 7168), (9, 33, 57344),
                                   (24, 48, 16384), (20, 33, 57344), (32, 40, 4096), (17, 30, 7168),
                                   (4, 48, 16384), (3, 33, 57344), (2, 40, 7168), (4, 24, 28672),
                                   (6, 48, 16384), (8, 33, 57344), (7, 40, 4096)])
def test_qgemm_chunked_k(m, n, k):
    # K split over several workgroup chunks (partial sums added in a second
    # pass); 17..32 tokens take one pass of two token sets when K / 128 is a
    # multiple of 32 (16384: 4 chunks, 57344: 14, 4096: 1) and passes of 16
    # otherwise (7168, and 5..16 tokens); up to 4 tokens take the four-token
    # kernel in chunks of 64 groups (16384: 2, 57344: 7) or 56 (7168: 1,
    # 28672: 4)
    say("qgemm chunked", m, n, k)
    c = synth.codes_all8(4300 + k, n, k)
    s = synth.scales(4400 + k, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(4500 + m, m, k)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), dev(s)))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "qgemm chunked M=%d %dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k,off", [(9, 28672, 8192, 0), (16, 26000, 2048, 0), (12, 30001, 4096, 1),
                                       (3, 28672, 2048, 1), (13, 32768, 2048, 4), (16, 25000, 28672, 0)])
def test_qgemm_many_tiles_per_cu(m, n, k, off):
    """Batched decode on matrices of 25000..32768 rows (7 or 8 tiles of 16
    rows per CU), every output compared: ragged N, 2- and 8-byte aligned
    scale views (offset by 1 or 4 elements), K = 2048 .. 28672."""
    say("qgemm many tiles per CU", m, n, k, "scale offset", off)
    c = synth.codes_all8(5000 + m + n, n, k)
    s = synth.scales(5001 + k, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(5002 + m, m, k)
    big = torch.zeros(s.size + 8, dtype=torch.int16, device="cuda")
    big[off:off + s.size] = torch.from_numpy(s.reshape(-1).view(np.int16)).cuda()
    sv = big[off:off + s.size].view(n, k // 128)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), sv))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "qgemm many tiles M=%d %dx%d" % (m, n, k))


@pytest.mark.parametrize("m", [2, 7, 16, 17, 32])
@pytest.mark.parametrize("n,k", [(2048, 11008), (45, 384), (300, 640), (37, 2944)])
def test_qgemm_any_k(m, n, k):
    """K / 128 not a multiple of 8 (SmolLM3-3B's down_proj K = 11008 is 86
    groups): the workgroup-per-tile kernel with 8 waves over the groups, fewer
    groups than waves included (K = 384, 640), every output."""
    say("qgemm any K", m, n, k)
    c = synth.codes_all8(5200 + n + k, n, k)
    s = synth.scales(5201 + k, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(5202 + m, m, k)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), dev(s)))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "qgemm any K M=%d %dx%d" % (m, n, k))


@pytest.mark.parametrize("m", [3, 8, 16, 40])
@pytest.mark.parametrize("n,k", [(50, 2048), (40, 3072), (300, 4096), (36, 5120), (64, 6144), (20, 53248)])
def test_qgemm_slice_waves(m, n, k):
    """The batched kernels with 2..6 waves per workgroup (K / 1024 = 2, 3, 4, 5,
    6 and 52: one 8-group slice per wave, the largest wave count up to 8 that
    tiles K; K = 53248 in 13 K chunks), up to 8 tokens in the batch-1 layout,
    16-token passes, and 40 tokens in passes of 32 or 16."""
    say("qgemm slice waves", m, n, k)
    c = synth.codes_all8(5100 + n + k, n, k)
    s = synth.scales(5101 + k, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(5102 + m, m, k)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), dev(s)))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "qgemm slice waves M=%d %dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(300, 72, 1024), (129, 300, 2048), (520, 260, 4096)])
def test_qgemm_large_m_tiles(m, n, k):
    # ragged 256-token and 256-row tiles, K split into chunks
    say("qgemm large M", m, n, k)
    c = synth.codes_all8(4700 + n + k, n, k)
    s = synth.scales(4800 + k, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(4900 + m, m, k)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), dev(s)))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "qgemm large M=%d %dx%d" % (m, n, k))


@pytest.mark.parametrize("m", [3, 6, 24])
@pytest.mark.parametrize("off", [1, 4])
def test_qgemm_scales_view_not_16_byte_aligned(off, m):
    """Scale views 2-byte aligned (read two bytes at a time: passes of 16
    tokens) and 8-byte aligned but not 16 (the 8-byte scale loads of the
    ring and four-token kernels; 24 tokens in one pass)."""
    n, k = 40, 8192
    c = synth.codes_all8(4600, n, k)
    s = synth.scales(4601, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(4602, m, k)
    say("qgemm scales offset by %d elements" % off)
    big = torch.zeros(s.size + 8, dtype=torch.int16, device="cuda")
    big[off:off + s.size] = torch.from_numpy(s.reshape(-1).view(np.int16)).cuda()
    sv = big[off:off + s.size].view(n, k // 128)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), sv))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "qgemm scales view")


@pytest.mark.parametrize("m", [3, 9, 20, 40, 130])
def test_qgemm_max_k(m):
    """K = 131072, the largest accepted: 16, 32 or more K chunks on the
    batched paths, 1024 groups per row on the tile and prefill paths."""
    n, k = 24, 131072
    c = synth.codes_all8(4900 + m, n, k)
    s = synth.scales(4901, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(4902 + m, m, k)
    say("qgemm K = %d, M = %d" % (k, m))
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), dev(s)))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "qgemm max K M=%d" % m)


def _random_shapes(count, seed):
    """Seeded (M, N, K) across every dispatch rule: M = 1, up to 4 tokens,
    passes of 16 and 32, the 128-row tiles and the prefill tiles; K / 128 a
    multiple of 64, 56 or 32, or none of them; ragged N.  N shrinks so that
    the oracle's M N K stays near 3e8 multiply-adds."""
    rng = np.random.default_rng(seed)
    ms = [1, 2, 3, 4, 5, 8, 11, 16, 17, 23, 32, 33, 70, 129, 160]
    gs = [1, 2, 3, 7, 8, 28, 32, 56, 64, 96, 112, 128, 224]
    out = []
    for _ in range(count):
        m = int(rng.choice(ms))
        k = 128 * int(rng.choice(gs))
        n = int(rng.integers(1, 600))
        n = max(1, min(n, int(3e8 // (m * k))))
        out.append((m, n, k))
    return out


@pytest.mark.parametrize("m,n,k", _random_shapes(48, 20261203))
def test_qgemm_random_shapes(m, n, k):
    seed = m * 1000003 + n * 131 + k
    c = synth.codes_all8(seed, n, k)
    s = synth.scales(seed + 1, n, k // 128, sigma=0.02, eps=1e-3)
    x = synth.activations(seed + 2, m, k)
    say("qgemm random shape", m, n, k)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), dev(s)))
    yr, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y, yr, a, "random shape M=%d %dx%d" % (m, n, k))


def test_qgemm_m1_is_gemv_and_rows_repeat():
    n, k = 100, 2048
    c = synth.codes(71, n, k)
    s = synth.scales(72, n, k // 128)
    x1 = synth.activations(73, 1, k)
    packed, sd = gpu_pack(c), dev(s)
    say("qgemm M=1 / repeated rows")
    y1 = host(q().qgemm_w3g128_smallM(dev(x1), packed, sd))
    yv = host(q().qgemv_w3g128(dev(x1.reshape(-1)), packed, sd))
    assert np.array_equal(y1[0].view(np.uint32), yv.view(np.uint32))
    xr = np.repeat(x1, 20, axis=0)
    yr = host(q().qgemm_w3g128_smallM(dev(xr), packed, sd))
    assert all(np.array_equal(yr[i].view(np.uint32), yr[0].view(np.uint32)) for i in range(20))
    ref, a = oracle.gemm(x1, oracle.pack(c), s, k)
    assert_close(yr[0], ref[0], a[0], "repeated row")


# One pass of 16 tokens; 32 tokens in one pass with K in two chunks; seven
# K chunks (K = 28672); the prefill tiles with K split.
@pytest.mark.parametrize("m,n,k", [(16, 512, 8192), (32, 512, 8192), (24, 64, 28672), (300, 256, 4096)])
def test_qgemm_deterministic(m, n, k):
    c = synth.codes(81, n, k)
    s = synth.scales(82, n, k // 128)
    x = synth.activations(83, m, k)
    packed, sd, xd = gpu_pack(c), dev(s), dev(x)
    say("qgemm determinism", m, n, k)
    y1 = host(q().qgemm_w3g128_smallM(xd, packed, sd))
    y2 = host(q().qgemm_w3g128_smallM(xd, packed, sd))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    ref, a = oracle.gemm(x, oracle.pack(c), s, k)
    assert_close(y1, ref, a, "determinism case")


# --------------------------------------------- full 70B-layer shapes -------
# Every output row is compared (the oracle takes about 40 ms per projection
# and token on 16 host threads), except at M = 512, where every 8th row plus
# the first and last row of every 256-row tile are.

@functools.lru_cache(maxsize=1)
def layer(name):
    return synth.layer_weights(name)


def check_layer_full(name, ms):
    c, s = layer(name)
    n, k = c.shape
    packed = gpu_pack(c)
    words = oracle.pack(c)
    assert np.array_equal(host(packed).view(np.uint32), words), "packed words differ"
    sd = dev(s)
    for m in ms:
        x = synth.layer_x(m, k)
        say("layer", name, "M=%d" % m, n, k, "all rows")
        if m == 1:
            y = host(q().qgemv_w3g128(dev(x.reshape(-1)), packed, sd))[None, :]
        else:
            y = host(q().qgemm_w3g128_smallM(dev(x), packed, sd))
        yr, a = oracle.gemm(x, words, s, k)
        assert_close(y, yr, a, "%s M=%d" % (name, m))


@pytest.mark.parametrize("name", ["q_proj", "k_proj", "v_proj", "o_proj", "up_proj"])
def test_layer_projection_b1_full_size(name):
    check_layer_full(name, [1])


@pytest.mark.parametrize("name", ["gate_proj", "down_proj"])
def test_gate_down_b1_and_batched_full_size(name):
    """Batch 1 and batched decode M = 4, 6, 8, 16, 32, every output."""
    check_layer_full(name, [1, 4, 6, 8, 16, 32])


@pytest.mark.parametrize("name", ["gate_proj", "down_proj"])
def test_prefill_m512_full_size(name):
    c, s = layer(name)
    n, k = c.shape
    m = 512
    x = synth.layer_x(m, k)
    say("prefill", name, m, n, k)
    y = host(q().qgemm_w3g128_smallM(dev(x), gpu_pack(c), dev(s)))
    rows = np.unique(np.concatenate([np.arange(0, n, 8), np.arange(0, n, 256), np.arange(255, n, 256), [n - 1]]))
    yr, a = oracle.gemm(x, oracle.pack(c[rows]), s[rows], k)
    assert_close(y[:, rows], yr, a, "prefill %s" % name)


# ------------------------------------------------------- graph capture ----

def test_graph_capture_replays_match_eager():
    """The product calls captured in a HIP graph on a user stream (after one
    call of each size on that stream, so nothing is allocated while
    capturing), replayed three times with new activations copied into the
    captured buffers between replays: every replay equals the eager calls
    bit for bit.  Covers batch 1, up to 4 tokens, 16 and 32 tokens (K in two
    chunks plus the chunk sum) and the prefill tiles."""
    n, k = 96, 8192
    c = synth.codes_all8(8100, n, k)
    s = synth.scales(8101, n, k // 128, sigma=0.02, eps=1e-3)
    packed, sd = gpu_pack(c), dev(s)
    ms = [1, 3, 16, 32, 300]
    say("graph capture", ms)
    xs = [torch.zeros((m, k), dtype=torch.int16, device="cuda") for m in ms]
    ys = [torch.zeros((m, n), dtype=torch.float32, device="cuda") for m in ms]

    def calls():
        for x, y in zip(xs, ys):
            if x.shape[0] == 1:
                q().qgemv_w3g128(x.view(-1), packed, sd, out=y.view(-1))
            else:
                q().qgemm_w3g128_smallM(x, packed, sd, out=y)

    def load(seed):
        for i, (x, m) in enumerate(zip(xs, ms)):
            x.copy_(dev(synth.activations(seed + i, m, k)))

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        load(8200)
        calls()  # sizes the workspace of this stream before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        seed = 8300 + 10 * rep
        with torch.cuda.stream(stream):
            load(seed)
            calls()
        torch.cuda.synchronize()
        eager = [host(y).copy() for y in ys]
        for y in ys:
            y.fill_(float("nan"))
        with torch.cuda.stream(stream):
            load(seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for m, y, e in zip(ms, ys, eager):
            assert np.array_equal(host(y).view(np.uint32), e.view(np.uint32)), \
                "graph replay %d differs from the eager call at M=%d" % (rep, m)


def test_streams_have_their_own_workspace():
    """Batched calls queued on two streams at once (different M, so the
    workspaces differ in size and layout, K split so partial sums are
    staged) give the same results as calls made one at a time; a later,
    larger call on one stream grows only that stream's workspace."""
    n, k = 200, 16384
    c = synth.codes_all8(8500, n, k)
    s = synth.scales(8501, n, k // 128, sigma=0.02, eps=1e-3)
    packed, sd = gpu_pack(c), dev(s)
    say("two streams")
    cases = [(16, 8502), (32, 8503), (9, 8504), (24, 8505)]
    xs = [dev(synth.activations(seed, m, k)) for m, seed in cases]
    ref = [host(q().qgemm_w3g128_smallM(x, packed, sd)) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda") for m, _ in cases]
    torch.cuda.synchronize()
    for rep in range(3):
        for i, (x, y) in enumerate(zip(xs, outs)):
            with torch.cuda.stream(streams[i % 2]):
                q().qgemm_w3g128_smallM(x, packed, sd, out=y)
        torch.cuda.synchronize()
        for i, (y, r) in enumerate(zip(outs, ref)):
            assert np.array_equal(host(y).view(np.uint32), r.view(np.uint32)), "stream case %d, pass %d" % (i, rep)
            y.fill_(float("nan"))
    big = dev(synth.activations(8506, 300, k))
    with torch.cuda.stream(streams[0]):
        yb = q().qgemm_w3g128_smallM(big, packed, sd)
    torch.cuda.synchronize()
    yr, a = oracle.gemm(synth.activations(8506, 300, k), oracle.pack(c), s, k)
    assert_close(host(yb), yr, a, "grown workspace")


def test_graph_replay_survives_workspace_growth():
    """A graph captured at 16 tokens on a stream (K split: converted
    activations and partial sums in the stream's workspace), then an eager
    300-token call on the same stream that grows the workspace: replays still
    equal the eager 16-token call bit for bit (the superseded buffer is kept,
    never freed)."""
    n, k = 200, 16384
    c = synth.codes_all8(8600, n, k)
    s = synth.scales(8601, n, k // 128, sigma=0.02, eps=1e-3)
    packed, sd = gpu_pack(c), dev(s)
    x16 = torch.zeros((16, k), dtype=torch.int16, device="cuda")
    y16 = torch.zeros((16, n), dtype=torch.float32, device="cuda")
    x300 = dev(synth.activations(8602, 300, k))
    stream = torch.cuda.Stream()
    say("graph replay after workspace growth")
    with torch.cuda.stream(stream):
        x16.copy_(dev(synth.activations(8603, 16, k)))
        q().qgemm_w3g128_smallM(x16, packed, sd, out=y16)  # sizes the workspace for 16 tokens
    torch.cuda.synchronize()
    eager16 = host(y16).copy()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        q().qgemm_w3g128_smallM(x16, packed, sd, out=y16)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        y300 = q().qgemm_w3g128_smallM(x300, packed, sd)  # grows this stream's workspace
    torch.cuda.synchronize()
    for rep in range(3):
        y16.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y16).view(np.uint32), eager16.view(np.uint32)), "replay %d after growth" % rep
        with torch.cuda.stream(stream):
            q().qgemm_w3g128_smallM(x300, packed, sd, out=y300)  # eager work on the grown buffer between replays
        torch.cuda.synchronize()
    yr, a = oracle.gemm(synth.activations(8602, 300, k), oracle.pack(c), s, k)
    assert_close(host(y300), yr, a, "after growth")


def test_capture_that_would_grow_the_workspace_is_refused():
    """On a stream with no workspace yet, a captured call that would have to
    allocate returns QW3_ERR_CAPTURE and enqueues nothing; after one eager
    call of that size the same capture works."""
    n, k = 64, 16384
    c = synth.codes(8700, n, k)
    s = synth.scales(8701, n, k // 128)
    packed, sd = gpu_pack(c), dev(s)
    x = dev(synth.activations(8702, 16, k))
    y = torch.zeros((16, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    say("capture refused before the workspace exists")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(q().Qw3Error) as ei:
        with torch.cuda.graph(graph, stream=stream):
            q().qgemm_w3g128_smallM(x, packed, sd, out=y)
    assert ei.value.status == q().QW3_ERR_CAPTURE
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        q().qgemm_w3g128_smallM(x, packed, sd, out=y)
    torch.cuda.synchronize()
    eager = host(y).copy()
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2, stream=stream):
        q().qgemm_w3g128_smallM(x, packed, sd, out=y)
    y.fill_(0.0)
    torch.cuda.synchronize()
    graph2.replay()
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint32), eager.view(np.uint32))
