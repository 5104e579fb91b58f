"""Reference oracle for the W3G128 format -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import it, and it imports nothing from them.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one bit and one term at a
time); this module only compiles it with gcc and marshals numpy arrays through
ctypes.  Definitions follow the GSQ model card "Llama-3.1-70B-Instruct-3Bit-GSQ"
(sections "Quantization details" and "Storage layout"): int32 ``weight``
[N, 3K/32] of exact-width 3-bit codes, bf16 ``weight_scale`` [N, K/128], a
symmetric integer codebook times the group scale, no zero point.  The product
the fused kernels compute is Y = X * dequant(W)^T (GLQ README, section
"Inference kernels").

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
that do not come from this code: the sizes the card prints, hand-derived packed
words, numpy's own bit packer, exact rational arithmetic and closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle_w3.so")
# The mutation test (tests/test_oracle_mutants.py) points this at deliberately
# broken copies of the oracle to show that the pins catch them.
_LIB_OVERRIDE = os.environ.get("W3_ORACLE_LIB_UNDER_TEST")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle_w3.so with gcc (OpenMP over rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_words_per_row.argtypes = [i64]
    lib.oracle_words_per_row.restype = i64
    lib.oracle_groups_per_row.argtypes = [i64]
    lib.oracle_groups_per_row.restype = i64
    lib.oracle_pack.argtypes = [vp, vp, i64, i64]
    lib.oracle_pack.restype = ctypes.c_int
    lib.oracle_unpack.argtypes = [vp, vp, i64, i64]
    lib.oracle_unpack.restype = ctypes.c_int
    lib.oracle_repack_w4c.argtypes = [vp, vp, i64, i64]
    lib.oracle_repack_w4c.restype = ctypes.c_int
    lib.oracle_dequant_bf16.argtypes = [vp, vp, vp, i64, i64]
    lib.oracle_dequant_bf16.restype = ctypes.c_int
    lib.oracle_gemm_rows.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp]
    lib.oracle_gemm_rows.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


def words_per_row(K: int) -> int:
    return int(_load().oracle_words_per_row(K))


def groups_per_row(K: int) -> int:
    return int(_load().oracle_groups_per_row(K))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def pack(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [N, K] (0..7) -> uint32 words [N, 3K/32], LSB-first stream."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    N, K = codes.shape
    out = np.empty((N, max(words_per_row(K), 0)), dtype=np.uint32)
    _check(_load().oracle_pack(_ptr(codes), _ptr(out), N, K), "pack")
    return out


def unpack(words: np.ndarray, K: int) -> np.ndarray:
    """uint32/int32 words [N, 3K/32] -> uint8 codes [N, K]."""
    words = np.ascontiguousarray(words).view(np.uint32)
    N = words.shape[0]
    assert words.shape[1] == words_per_row(K)
    out = np.empty((N, K), dtype=np.uint8)
    _check(_load().oracle_unpack(_ptr(words), _ptr(out), N, K), "unpack")
    return out


def repack_w4c(w4: np.ndarray) -> np.ndarray:
    """uint32/int32 4-bit-container words [N, K/8] -> uint32 words [N, 3K/32].

    Reading (see oracle.c): nibble k % 8 of word k / 8, least significant
    first, holds code k in its low 3 bits; the top bit is padding."""
    w4 = np.ascontiguousarray(w4).view(np.uint32)
    N, K8 = w4.shape
    K = 8 * K8
    out = np.empty((N, max(words_per_row(K), 0)), dtype=np.uint32)
    _check(_load().oracle_repack_w4c(_ptr(w4), _ptr(out), N, K), "repack_w4c")
    return out


def dequant_bf16(words: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """words [N, 3K/32] + bf16 bits [N, K/128] -> bf16 bits uint16 [N, K]."""
    words = np.ascontiguousarray(words).view(np.uint32)
    scales = np.ascontiguousarray(scales).view(np.uint16)
    N = words.shape[0]
    assert scales.shape == (N, groups_per_row(K))
    out = np.empty((N, K), dtype=np.uint16)
    _check(_load().oracle_dequant_bf16(_ptr(words), _ptr(scales), _ptr(out), N, K),
           "dequant_bf16")
    return out


def gemm(x: np.ndarray, words: np.ndarray, scales: np.ndarray, K: int, rows=None):
    """fp64 Y = X * dequant(W)^T over the listed output rows.

    x: bf16 bits uint16 [M, K]; words [N, 3K/32]; scales bf16 bits [N, K/128].
    Returns (y, a), both float64 [M, len(rows)]: y the exact-product fp64 sum
    and a the sum of absolute terms (the scale of the GPU tolerance).
    """
    x = np.ascontiguousarray(x).view(np.uint16)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    words = np.ascontiguousarray(words).view(np.uint32)
    scales = np.ascontiguousarray(scales).view(np.uint16)
    M = x.shape[0]
    N = words.shape[0]
    assert x.shape[1] == K and words.shape[1] == words_per_row(K)
    assert scales.shape == (N, groups_per_row(K))
    if rows is None:
        rows = np.arange(N, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((M, rows.size), dtype=np.float64)
    a = np.empty((M, rows.size), dtype=np.float64)
    _check(_load().oracle_gemm_rows(_ptr(x), _ptr(words), _ptr(scales), _ptr(rows),
                                    rows.size, M, N, K, _ptr(y), _ptr(a)), "gemm")
    return y, a
