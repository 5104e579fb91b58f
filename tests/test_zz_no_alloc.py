"""qgemm_w3g128_smallM_noalloc: the batched product for callers that cannot
allocate, with its scratch in the library's static device array.

Through the C ABI, two calls in a row on each case (the second with a smaller
input, so it reads scratch the first one wrote): each output equals what
qgemm_w3g128_smallM gives for the same inputs, bit for bit (the same kernels),
and so meets the oracle's bound |y - y_ref| <= 1e-4 * sum |w x| + 1e-6.
A call that needs more than the static array is refused before any launch.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def q():
    import dequant_gemv_qgemv_amd as mod
    return mod


def say(*args):
    print("[gpu-case]", *args, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def noalloc_raw(x, packed, scales, y):
    """The entry point itself, through ctypes (no binding logic)."""
    lib = q().raw()
    m, k = x.shape
    n = packed.shape[0]
    st = lib.qgemm_w3g128_smallM_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(packed.data_ptr()),
                                         ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                         m, n, k, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == q().QW3_OK, q().qstatus_str(st)


# (first M, second M, N, K, scale offset): the ring kernel with a K split, the
# in-kernel conversion (5 and 3 tokens, K = 28672), the 2-byte scale reader
# (16-token passes) and the prefill tiles with K split.
CASES = [(32, 9, 1024, 8192, 0), (16, 5, 512, 28672, 0), (12, 3, 300, 8192, 1), (512, 200, 512, 4096, 0)]


@pytest.mark.parametrize("m1,m2,n,k,off", CASES)
def test_noalloc_matches_allocating_entry(m1, m2, n, k, off):
    c = synth.codes_all8(9100 + n, n, k)
    s = synth.scales(9101 + n, n, k // 128, sigma=0.02, eps=1e-3)
    packed = q().qpack_uint3(dev(c))
    if off:
        big = torch.zeros(s.size + 8, dtype=torch.int16, device="cuda")
        big[off:off + s.size] = dev(s.reshape(-1))
        sd = big[off:off + s.size].view(n, k // 128)
    else:
        sd = dev(s)
    words = oracle.pack(c)
    for m in (m1, m2):
        x = synth.activations(9200 + m, m, k)
        xd = dev(x)
        say("noalloc", "M=%d N=%d K=%d scale offset %d" % (m, n, k, off))
        y_na = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        noalloc_raw(xd, packed, sd, y_na)
        y_ref_gpu = q().qgemm_w3g128_smallM(xd, packed, sd)
        got, want = host(y_na), host(y_ref_gpu)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "M=%d differs from qgemm_w3g128_smallM" % m
        yr, a = oracle.gemm(x, words, s, k)
        assert np.all(np.abs(got.astype(np.float64) - yr) <= 1e-4 * a + 1e-6)


def test_noalloc_refuses_oversized_call():
    """4096 prefill tokens against an 8192 x 28672 matrix need 224 MiB of
    converted activations alone: refused with QW3_ERR_SCRATCH before any
    launch (the buffers are small stand-ins that are never read)."""
    lib = q().raw()
    m, n, k = 4096, 8192, 28672
    assert 2 * m * k > 1.5 * q().QW3_NOALLOC_SCRATCH_BYTES  # refused on the host, never launched
    buf = torch.zeros(4096, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    say("noalloc oversized")
    st = lib.qgemm_w3g128_smallM_noalloc(p, p, p, p, m, n, k, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == q().QW3_ERR_SCRATCH
