"""CPU checks of the C ABI: the library loads, exports what include/qw3.h
declares, and rejects bad arguments on the host before touching the GPU.

Every call here fails validation, so no HIP work is ever enqueued; the fake
pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import dequant_gemv_qgemv_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qw3.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)  # preprocessor lines
    return sorted(set(re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_four_operations():
    fns = header_functions()
    for name in ("qpack_uint3", "qdequant_bf16", "qgemv_w3g128", "qgemm_w3g128_smallM"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q.library_path())
    fns = header_functions()
    assert fns
    for name in fns:
        assert hasattr(lib, name), name
    assert set(fns) == set(q.exported_symbols())


def test_abi_version_and_status_strings():
    assert q.raw().qw3_abi_version() == 1
    for st in (q.QW3_OK, q.QW3_ERR_NULL, q.QW3_ERR_SHAPE, q.QW3_ERR_ALIGN, q.QW3_ERR_HIP, q.QW3_ERR_CAPTURE,
               q.QW3_ERR_SCRATCH):
        assert q.qstatus_str(st)
    assert q.qstatus_str(12345) == "unknown status"


# fake, never-dereferenced device addresses
A16 = ctypes.c_void_p(0x10000)
A16B = ctypes.c_void_p(0x20000)
A16C = ctypes.c_void_p(0x30000)
A16D = ctypes.c_void_p(0x40000)
MIS = ctypes.c_void_p(0x10008)  # 8-byte, not 16-byte, aligned
ODD = ctypes.c_void_p(0x10001)
NULL = ctypes.c_void_p(0)
S = ctypes.c_void_p(0)  # default stream


@pytest.mark.parametrize("n,k", [(-1, 128), (4, -128), (4, 100), (4, 129), (4, q.QW3_MAX_K + 128)])
def test_bad_shapes(n, k):
    lib = q.raw()
    assert lib.qpack_uint3(A16, A16B, n, k, S) == q.QW3_ERR_SHAPE
    assert lib.qrepack_w4c_uint3(A16, A16B, n, k, S) == q.QW3_ERR_SHAPE
    assert lib.qdequant_bf16(A16, A16B, A16C, n, k, S) == q.QW3_ERR_SHAPE
    assert lib.qgemv_w3g128(A16, A16B, A16C, A16D, n, k, S) == q.QW3_ERR_SHAPE
    assert lib.qgemm_w3g128_smallM(A16, A16B, A16C, A16D, 2, n, k, S) == q.QW3_ERR_SHAPE
    assert lib.qgemm_w3g128_smallM_noalloc(A16, A16B, A16C, A16D, 2, n, k, S) == q.QW3_ERR_SHAPE
    assert lib.qgemm_w3g128_batch_invariant(A16, A16B, A16C, A16D, 2, n, k, S) == q.QW3_ERR_SHAPE


def test_bad_m():
    assert q.raw().qgemm_w3g128_smallM(A16, A16B, A16C, A16D, -1, 4, 128, S) == q.QW3_ERR_SHAPE
    assert q.raw().qgemm_w3g128_smallM_noalloc(A16, A16B, A16C, A16D, -1, 4, 128, S) == q.QW3_ERR_SHAPE
    lib = q.raw()
    assert lib.qgemm_w3g128_batch_invariant(A16, A16B, A16C, A16D, -1, 4, 128, S) == q.QW3_ERR_SHAPE
    # one token per grid row: at most QW3_MAX_BATCH_INVARIANT_M rows
    assert lib.qgemm_w3g128_batch_invariant(A16, A16B, A16C, A16D, 65536, 4, 128, S) == q.QW3_ERR_SHAPE


def test_null_pointers():
    lib = q.raw()
    assert lib.qpack_uint3(NULL, A16B, 4, 128, S) == q.QW3_ERR_NULL
    assert lib.qpack_uint3(A16, NULL, 4, 128, S) == q.QW3_ERR_NULL
    assert lib.qrepack_w4c_uint3(NULL, A16B, 4, 128, S) == q.QW3_ERR_NULL
    assert lib.qrepack_w4c_uint3(A16, NULL, 4, 128, S) == q.QW3_ERR_NULL
    assert lib.qdequant_bf16(NULL, A16B, A16C, 4, 128, S) == q.QW3_ERR_NULL
    assert lib.qdequant_bf16(A16, NULL, A16C, 4, 128, S) == q.QW3_ERR_NULL
    assert lib.qdequant_bf16(A16, A16B, NULL, 4, 128, S) == q.QW3_ERR_NULL
    for i in range(4):
        args = [A16, A16B, A16C, A16D]
        args[i] = NULL
        assert lib.qgemv_w3g128(*args, 4, 128, S) == q.QW3_ERR_NULL
        assert lib.qgemm_w3g128_smallM(*args, 3, 4, 128, S) == q.QW3_ERR_NULL
        assert lib.qgemm_w3g128_smallM_noalloc(*args, 3, 4, 128, S) == q.QW3_ERR_NULL
        assert lib.qgemm_w3g128_batch_invariant(*args, 3, 4, 128, S) == q.QW3_ERR_NULL


def test_misaligned_pointers():
    lib = q.raw()
    assert lib.qpack_uint3(MIS, A16B, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qpack_uint3(A16, MIS, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qrepack_w4c_uint3(MIS, A16B, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qrepack_w4c_uint3(A16, MIS, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qdequant_bf16(MIS, A16B, A16C, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qdequant_bf16(A16, ODD, A16C, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qdequant_bf16(A16, A16B, MIS, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qgemv_w3g128(MIS, A16B, A16C, A16D, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qgemv_w3g128(A16, MIS, A16C, A16D, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qgemv_w3g128(A16, A16B, ODD, A16D, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qgemv_w3g128(A16, A16B, A16C, ctypes.c_void_p(0x40002), 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qgemm_w3g128_smallM(MIS, A16B, A16C, A16D, 3, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qgemm_w3g128_smallM_noalloc(MIS, A16B, A16C, A16D, 3, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qgemm_w3g128_batch_invariant(MIS, A16B, A16C, A16D, 3, 4, 128, S) == q.QW3_ERR_ALIGN
    assert lib.qgemm_w3g128_batch_invariant(A16, A16B, A16C, ctypes.c_void_p(0x40002), 3, 4, 128, S) == q.QW3_ERR_ALIGN


def test_empty_sizes_enqueue_nothing():
    lib = q.raw()
    # N == 0 or M == 0: valid and nothing to do, even with NULL pointers
    assert lib.qpack_uint3(NULL, NULL, 0, 128, S) == q.QW3_OK
    assert lib.qrepack_w4c_uint3(NULL, NULL, 0, 128, S) == q.QW3_OK
    assert lib.qdequant_bf16(NULL, NULL, NULL, 0, 1024, S) == q.QW3_OK
    assert lib.qgemv_w3g128(NULL, NULL, NULL, NULL, 0, 1024, S) == q.QW3_OK
    assert lib.qgemm_w3g128_smallM(NULL, NULL, NULL, NULL, 0, 5, 1024, S) == q.QW3_OK
    assert lib.qgemm_w3g128_smallM_noalloc(NULL, NULL, NULL, NULL, 0, 5, 1024, S) == q.QW3_OK
    assert lib.qgemm_w3g128_smallM(NULL, NULL, NULL, NULL, 5, 0, 1024, S) == q.QW3_OK
    assert lib.qgemm_w3g128_smallM_noalloc(NULL, NULL, NULL, NULL, 5, 0, 1024, S) == q.QW3_OK
    assert lib.qgemm_w3g128_batch_invariant(NULL, NULL, NULL, NULL, 0, 5, 1024, S) == q.QW3_OK
    assert lib.qgemm_w3g128_batch_invariant(NULL, NULL, NULL, NULL, 5, 0, 1024, S) == q.QW3_OK


def test_quantization_config_descriptor():
    good = {"quant_method": "humming", "b_dtype": "uint3", "weight_scale_group_size": 128,
            "weight_scale_type": "group", "has_zero_point": False,
            "ignore": ["lm_head", "embed_tokens"]}
    q.check_quantization_config(good)
    for key, bad in [("quant_method", "gptq"), ("b_dtype", "uint4"), ("weight_scale_group_size", 64),
                     ("weight_scale_type", "channel"), ("has_zero_point", True),
                     ("weight_scale_group_size", 128.0)]:
        cfg = dict(good)
        cfg[key] = bad
        with pytest.raises(ValueError):
            q.check_quantization_config(cfg)
    cfg = dict(good)
    del cfg["b_dtype"]
    with pytest.raises(ValueError):
        q.check_quantization_config(cfg)


def _arr(ctype, vals):
    return (ctype * len(vals))(*vals)


def test_multi_validation():
    lib = q.raw()
    lib.qgemv_w3g128_multi.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    P = _arr(ctypes.c_void_p, [0x10000, 0x20000])
    Sc = _arr(ctypes.c_void_p, [0x30000, 0x40000])
    Y = _arr(ctypes.c_void_p, [0x50000, 0x60000])
    n = _arr(ctypes.c_int64, [4, 8])
    assert lib.qgemv_w3g128_multi(A16, 0, P, Sc, Y, n, 128, S) == q.QW3_ERR_SHAPE
    assert lib.qgemv_w3g128_multi(A16, q.QW3_MAX_MULTI + 1, P, Sc, Y, n, 128, S) == q.QW3_ERR_SHAPE
    assert lib.qgemv_w3g128_multi(A16, 2, None, Sc, Y, n, 128, S) == q.QW3_ERR_NULL
    assert lib.qgemv_w3g128_multi(A16, 2, P, Sc, Y, None, 128, S) == q.QW3_ERR_NULL
    assert lib.qgemv_w3g128_multi(A16, 2, P, Sc, Y, _arr(ctypes.c_int64, [4, -1]), 128, S) == q.QW3_ERR_SHAPE
    assert lib.qgemv_w3g128_multi(A16, 2, P, Sc, Y, n, 100, S) == q.QW3_ERR_SHAPE
    assert lib.qgemv_w3g128_multi(NULL, 2, P, Sc, Y, n, 128, S) == q.QW3_ERR_NULL
    assert lib.qgemv_w3g128_multi(MIS, 2, P, Sc, Y, n, 128, S) == q.QW3_ERR_ALIGN
    Pm = _arr(ctypes.c_void_p, [0x10000, 0x20008])
    assert lib.qgemv_w3g128_multi(A16, 2, Pm, Sc, Y, n, 128, S) == q.QW3_ERR_ALIGN
    Yn = _arr(ctypes.c_void_p, [0x50000, 0])
    assert lib.qgemv_w3g128_multi(A16, 2, P, Sc, Yn, n, 128, S) == q.QW3_ERR_NULL
    # all matrices empty: valid, nothing enqueued
    z = _arr(ctypes.c_int64, [0, 0])
    assert lib.qgemv_w3g128_multi(NULL, 2, P, Sc, Y, z, 128, S) == q.QW3_OK
