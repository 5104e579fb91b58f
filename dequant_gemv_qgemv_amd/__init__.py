"""Python binding of the W3G128 HIP library (libqw3.so, C ABI in include/qw3.h).

This module only marshals arguments: it checks dtypes, devices, shapes and
contiguity of PyTorch tensors, passes their device pointers and the current
HIP stream to the C entry points of the same names, and turns a non-zero
status into an exception.  Every step of the computation runs in the HIP
kernels; there is no CPU or PyTorch fallback, and importing this package fails
loudly when the library has not been built.

Format: GSQ model card "Llama-3.1-70B-Instruct-3Bit-GSQ", sections
"Quantization details" and "Storage layout" -- int32 ``weight`` [N, 3K/32] of
exact-width 3-bit codes, bf16 ``weight_scale`` [N, K/128], weight =
scale * (code - 4), no zero point.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "qpack_uint3",
    "qrepack_w4c_uint3",
    "qdequant_bf16",
    "qgemv_w3g128",
    "qgemv_w3g128_multi",
    "qgemm_w3g128_smallM",
    "qgemm_w3g128_smallM_noalloc",
    "qstatus_str",
    "check_quantization_config",
    "library_path",
    "exported_symbols",
    "Qw3Error",
    "QW3_OK",
    "QW3_ERR_NULL",
    "QW3_ERR_SHAPE",
    "QW3_ERR_ALIGN",
    "QW3_ERR_HIP",
    "QW3_ERR_CAPTURE",
    "QW3_ERR_SCRATCH",
    "QW3_NOALLOC_SCRATCH_BYTES",
    "QW3_MAX_K",
    "QW3_MAX_MULTI",
    "QW3_MAX_BATCH_INVARIANT_M",
]

QW3_OK, QW3_ERR_NULL, QW3_ERR_SHAPE, QW3_ERR_ALIGN, QW3_ERR_HIP, QW3_ERR_CAPTURE, QW3_ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6
QW3_NOALLOC_SCRATCH_BYTES = 128 << 20
QW3_MAX_K = 131072
QW3_MAX_MULTI = 4
QW3_MAX_BATCH_INVARIANT_M = 65535
GROUP = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqw3.so")
_EXPORTS = ("qpack_uint3", "qrepack_w4c_uint3", "qdequant_bf16", "qgemv_w3g128", "qgemv_w3g128_multi",
            "qgemm_w3g128_smallM", "qgemm_w3g128_smallM_noalloc", "qgemm_w3g128_batch_invariant", "qstatus_str",
            "qw3_last_hip_error",
            "qw3_abi_version")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        "libqw3.so is not built (expected at %s); run __graft_entry__.build() or "
        "python dequant_gemv_qgemv_amd/_build.py" % _LIB_PATH)

_lib = ctypes.CDLL(_LIB_PATH)
_i64, _vp = ctypes.c_int64, ctypes.c_void_p
_lib.qpack_uint3.argtypes = [_vp, _vp, _i64, _i64, _vp]
_lib.qrepack_w4c_uint3.argtypes = [_vp, _vp, _i64, _i64, _vp]
_lib.qdequant_bf16.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp]
_lib.qgemv_w3g128.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _vp]
_lib.qgemm_w3g128_smallM.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.qgemm_w3g128_smallM_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.qgemm_w3g128_batch_invariant.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.qgemv_w3g128_multi.argtypes = [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _i64, _vp]
for _name in ("qpack_uint3", "qrepack_w4c_uint3", "qdequant_bf16", "qgemv_w3g128", "qgemv_w3g128_multi",
              "qgemm_w3g128_smallM", "qgemm_w3g128_smallM_noalloc"):
    getattr(_lib, _name).restype = ctypes.c_int
_lib.qstatus_str.argtypes = [ctypes.c_int]
_lib.qstatus_str.restype = ctypes.c_char_p
_lib.qw3_last_hip_error.argtypes = []
_lib.qw3_last_hip_error.restype = ctypes.c_char_p
_lib.qw3_abi_version.argtypes = []
_lib.qw3_abi_version.restype = ctypes.c_int


class Qw3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = "%s: %s" % (where, qstatus_str(status))
        if status == QW3_ERR_HIP:
            msg += " [%s]" % _lib.qw3_last_hip_error().decode()
        super().__init__(msg)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def exported_symbols():
    """Names this binding expects the library to export."""
    return _EXPORTS


def raw():
    """The ctypes handle of libqw3.so (for pointer-level tests)."""
    return _lib


def qstatus_str(status: int) -> str:
    return _lib.qstatus_str(int(status)).decode()


def _check(status: int, where: str):
    if status != QW3_OK:
        raise Qw3Error(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtypes, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s must have dtype in %s, got %s" % (name, dtypes, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (name, t.device))
    if t.dim() != ndim:
        raise ValueError("%s must be %d-D, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _k_from_packed(packed: torch.Tensor) -> int:
    w = packed.shape[1]
    if (32 * w) % 3 != 0:
        raise ValueError("packed has %d words per row, not 3K/32 for any K" % w)
    return (32 * w) // 3


def _check_weight(packed: torch.Tensor, scales: torch.Tensor):
    _need(packed, "packed", (torch.int32,), 2)
    _need(scales, "scales", _BF16, 2)
    if packed.device != scales.device:
        raise ValueError("packed and scales are on different devices")
    n = packed.shape[0]
    k = _k_from_packed(packed)
    if tuple(scales.shape) != (n, k // GROUP):
        raise ValueError("scales shape %s does not match packed %s (expected [%d, %d])"
                         % (tuple(scales.shape), tuple(packed.shape), n, k // GROUP))
    return n, k


def qpack_uint3(codes: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """uint8 codes [N, K] (0..7) -> int32 packed [N, 3K/32]."""
    _need(codes, "codes", (torch.uint8,), 2)
    n, k = codes.shape
    if k % GROUP:
        raise ValueError("K = %d is not a multiple of %d" % (k, GROUP))
    if out is None:
        out = torch.empty((n, 3 * k // 32), dtype=torch.int32, device=codes.device)
    _need(out, "out", (torch.int32,), 2)
    if tuple(out.shape) != (n, 3 * k // 32):
        raise ValueError("out must have shape [%d, %d]" % (n, 3 * k // 32))
    with torch.cuda.device(codes.device):
        _check(_lib.qpack_uint3(_ptr(codes), _ptr(out), n, k, _stream()), "qpack_uint3")
    return out


def qrepack_w4c_uint3(w4: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """int32 4-bit-container codes [N, K/8] (code k in nibble k % 8 of word
    k / 8, low 3 bits) -> int32 packed [N, 3K/32]."""
    _need(w4, "w4", (torch.int32,), 2)
    n, k = w4.shape[0], 8 * w4.shape[1]
    if out is None:
        out = torch.empty((n, 3 * k // 32), dtype=torch.int32, device=w4.device)
    _need(out, "out", (torch.int32,), 2)
    if tuple(out.shape) != (n, 3 * k // 32) or out.device != w4.device:
        raise ValueError("out must be int32 [%d, %d] on %s" % (n, 3 * k // 32, w4.device))
    with torch.cuda.device(w4.device):
        _check(_lib.qrepack_w4c_uint3(_ptr(w4), _ptr(out), n, k, _stream()), "qrepack_w4c_uint3")
    return out


def qdequant_bf16(packed: torch.Tensor, scales: torch.Tensor,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """packed [N, 3K/32] + bf16 scales [N, K/128] -> bf16 weight [N, K]."""
    n, k = _check_weight(packed, scales)
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=packed.device)
    _need(out, "out", _BF16, 2)
    if tuple(out.shape) != (n, k):
        raise ValueError("out must have shape [%d, %d]" % (n, k))
    with torch.cuda.device(packed.device):
        _check(_lib.qdequant_bf16(_ptr(packed), _ptr(scales), _ptr(out), n, k, _stream()),
               "qdequant_bf16")
    return out


def qgemv_w3g128(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """y[N] = dequant(W) x for bf16 x [K]; returns float32 [N]."""
    n, k = _check_weight(packed, scales)
    _need(x, "x", _BF16, 1)
    if x.shape[0] != k or x.device != packed.device:
        raise ValueError("x must be [%d] on %s" % (k, packed.device))
    if out is None:
        out = torch.empty((n,), dtype=torch.float32, device=packed.device)
    _need(out, "out", (torch.float32,), 1)
    if out.shape[0] != n:
        raise ValueError("out must be [%d]" % n)
    with torch.cuda.device(packed.device):
        _check(_lib.qgemv_w3g128(_ptr(x), _ptr(packed), _ptr(scales), _ptr(out), n, k, _stream()),
               "qgemv_w3g128")
    return out


def qgemv_w3g128_multi(x: torch.Tensor, weights, outs=None):
    """qgemv_w3g128 for several matrices sharing x and K, in one launch.

    weights: sequence of (packed, scales) pairs (1..QW3_MAX_MULTI); returns the
    list of float32 outputs [N_i] (or fills `outs`)."""
    weights = list(weights)
    if not 1 <= len(weights) <= QW3_MAX_MULTI:
        raise ValueError("1..%d matrices per call" % QW3_MAX_MULTI)
    shapes = [_check_weight(p, s) for p, s in weights]
    k = shapes[0][1]
    if any(kk != k for _, kk in shapes):
        raise ValueError("all matrices must have the same K")
    dev = weights[0][0].device
    if any(p.device != dev for p, _ in weights):
        raise ValueError("all matrices must be on one device")
    _need(x, "x", _BF16, 1)
    if x.shape[0] != k or x.device != dev:
        raise ValueError("x must be [%d] on %s" % (k, dev))
    if outs is None:
        outs = [torch.empty((n,), dtype=torch.float32, device=dev) for n, _ in shapes]
    outs = list(outs)
    if len(outs) != len(weights):
        raise ValueError("one output per matrix")
    for (n, _), o in zip(shapes, outs):
        _need(o, "out", (torch.float32,), 1)
        if o.shape[0] != n or o.device != dev:
            raise ValueError("out must be [%d] on %s" % (n, dev))
    cnt = len(weights)
    arr_p = (ctypes.c_void_p * cnt)(*[_ptr(p) for p, _ in weights])
    arr_s = (ctypes.c_void_p * cnt)(*[_ptr(s) for _, s in weights])
    arr_y = (ctypes.c_void_p * cnt)(*[_ptr(o) for o in outs])
    arr_n = (ctypes.c_int64 * cnt)(*[n for n, _ in shapes])
    with torch.cuda.device(dev):
        _check(_lib.qgemv_w3g128_multi(_ptr(x), cnt, arr_p, arr_s, arr_y, arr_n, k, _stream()),
               "qgemv_w3g128_multi")
    return outs


def qgemm_w3g128_smallM(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] = X dequant(W)^T for bf16 X [M, K]; returns float32 [M, N]."""
    n, k = _check_weight(packed, scales)
    _need(x, "x", _BF16, 2)
    m = x.shape[0]
    if x.shape[1] != k or x.device != packed.device:
        raise ValueError("x must be [M, %d] on %s" % (k, packed.device))
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=packed.device)
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (m, n):
        raise ValueError("out must be [%d, %d]" % (m, n))
    with torch.cuda.device(packed.device):
        _check(_lib.qgemm_w3g128_smallM(_ptr(x), _ptr(packed), _ptr(scales), _ptr(out), m, n, k,
                                        _stream()), "qgemm_w3g128_smallM")
    return out


def qgemm_w3g128_smallM_noalloc(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                                out: torch.Tensor) -> torch.Tensor:
    """qgemm_w3g128_smallM without any device allocation: the caller passes
    `out` (float32 [M, N]) and the library's static scratch is used."""
    n, k = _check_weight(packed, scales)
    _need(x, "x", _BF16, 2)
    m = x.shape[0]
    if x.shape[1] != k or x.device != packed.device:
        raise ValueError("x must be [M, %d] on %s" % (k, packed.device))
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (m, n) or out.device != packed.device:
        raise ValueError("out must be [%d, %d] on %s" % (m, n, packed.device))
    with torch.cuda.device(packed.device):
        _check(_lib.qgemm_w3g128_smallM_noalloc(_ptr(x), _ptr(packed), _ptr(scales), _ptr(out), m, n, k,
                                                _stream()), "qgemm_w3g128_smallM_noalloc")
    return out


def qgemm_w3g128_batch_invariant(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                                 out: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] = X dequant(W)^T with row m bit-identical to qgemv_w3g128(X[m]);
    reads the weights once per row of X."""
    n, k = _check_weight(packed, scales)
    _need(x, "x", _BF16, 2)
    m = x.shape[0]
    if x.shape[1] != k or x.device != packed.device:
        raise ValueError("x must be [M, %d] on %s" % (k, packed.device))
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=packed.device)
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (m, n) or out.device != packed.device:
        raise ValueError("out must be [%d, %d] on %s" % (m, n, packed.device))
    with torch.cuda.device(packed.device):
        _check(_lib.qgemm_w3g128_batch_invariant(_ptr(x), _ptr(packed), _ptr(scales), _ptr(out), m, n, k,
                                                 _stream()), "qgemm_w3g128_batch_invariant")
    return out


# Format descriptor of the checkpoint's config.json (GSQ model card, section
# "Storage layout"): only this combination is decoded by the kernels above.
_EXPECTED_CONFIG = {
    "quant_method": "humming",
    "b_dtype": "uint3",
    "weight_scale_group_size": 128,
    "weight_scale_type": "group",
    "has_zero_point": False,
}


def check_quantization_config(cfg: dict) -> None:
    """Raise ValueError unless `cfg` describes the W3G128 layout these kernels read."""
    for key, want in _EXPECTED_CONFIG.items():
        if key not in cfg:
            raise ValueError("quantization_config lacks %r" % key)
        got = cfg[key]
        if type(got) is not type(want) or got != want:
            raise ValueError("quantization_config[%r] = %r; only %r is supported" % (key, got, want))
