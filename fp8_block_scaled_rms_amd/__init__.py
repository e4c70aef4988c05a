"""fp8q: the FP8 quantized linear layer of LLM inference on MI355X (gfx950).

Thin ctypes binding over the C ABI declared in include/fp8q.h.  The binding
only marshals arguments: every step of the computation runs in the HIP
kernels of libfp8q.so.  PyTorch provides device memory and the current
stream; there is no fallback of any kind, and every call raises if the
library is missing or returns a non-OK status.

Functions named fp8q_* mirror the C entry points one to one (outputs first,
tensors in, sizes taken from the tensors).  The lower-case helpers
(rmsnorm_quant, silu_mul_quant, quant, scaled_mm, scaled_mm_blockwise)
allocate the outputs and the workspace with torch and call them.

Data types: bf16 tensors are torch.bfloat16; e4m3 tensors are torch.uint8
(raw OCP e4m3 bytes; ``t.view(torch.float8_e4m3fn)`` reinterprets them);
int8 tensors (the W8A8 INT8 functions, *_int8) are torch.int8; scales are
torch.float32.
"""
from __future__ import annotations

import ctypes
import os

import torch

PER_TOKEN = 0
GROUP128 = 1
PER_TENSOR_STATIC = 2
PER_TOKEN_UE8M0 = 3
GROUP128_UE8M0 = 4
OP_SCALED_MM = 0
OP_SCALED_MM_BLOCKWISE = 1
OP_SCALED_MM_INT8 = 2
OP_SCALED_MM_BLOCKWISE_UE8M0 = 3

_HERE = os.path.dirname(os.path.abspath(__file__))
# FP8Q_LIB may name another build of the same library (the host-sanitizer
# build the CPU tests use); there is no fallback if the file is missing
LIB_PATH = os.environ.get("FP8Q_LIB") or os.path.join(_HERE, "libfp8q.so")

_STATUS = {
    0: "FP8Q_OK", 1: "FP8Q_ERR_INVALID_ARG", 2: "FP8Q_ERR_UNSUPPORTED_SHAPE",
    3: "FP8Q_ERR_ALIGNMENT", 4: "FP8Q_ERR_WORKSPACE", 5: "FP8Q_ERR_NO_DEVICE",
    6: "FP8Q_ERR_ARCH", 7: "FP8Q_ERR_HIP", 8: "FP8Q_ERR_BAD_MODE", 9: "FP8Q_ERR_BAD_CONFIG",
}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t
_PI = ctypes.POINTER(ctypes.c_int)

# name -> (restype, argtypes); the C declarations are in include/fp8q.h
SIGNATURES = {
    "fp8q_rmsnorm_quant": (_INT, [_P, _P, _P, _P, _I64, _I64, _F32, _INT, _P]),
    "fp8q_silu_mul_quant": (_INT, [_P, _P, _P, _I64, _I64, _INT, _P]),
    "fp8q_quant": (_INT, [_P, _P, _P, _I64, _I64, _INT, _P]),
    "fp8q_scaled_mm": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "fp8q_scaled_mm_blockwise": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "fp8q_workspace_size": (_SZ, [_INT, _I64, _I64, _I64]),
    "fp8q_scaled_mm_blockwise_noalloc": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "fp8q_gemm_num_configs": (_INT, []),
    "fp8q_gemm_config_name": (ctypes.c_char_p, [_INT]),
    "fp8q_gemm_config_for": (_INT, [_INT, _I64, _I64, _I64]),
    "fp8q_workspace_size_cfg": (_SZ, [_INT, _I64, _I64, _I64]),
    "fp8q_scaled_mm_cfg": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _INT, _P]),
    "fp8q_scaled_mm_blockwise_cfg": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ,
                                            _INT, _P]),
    "fp8q_rmsnorm_quant_int8": (_INT, [_P, _P, _P, _P, _I64, _I64, _F32, _INT, _P]),
    "fp8q_silu_mul_quant_int8": (_INT, [_P, _P, _P, _I64, _I64, _INT, _P]),
    "fp8q_quant_int8": (_INT, [_P, _P, _P, _I64, _I64, _INT, _P]),
    "fp8q_scaled_mm_int8": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "fp8q_scaled_mm_int8_cfg": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _INT,
                                       _P]),
    "fp8q_scaled_mm_blockwise_ue8m0": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ,
                                              _P]),
    "fp8q_scaled_mm_blockwise_ue8m0_cfg": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P,
                                                  _SZ, _INT, _P]),
    "fp8q_scaled_mm_blockwise_silu_quant": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                                                   _P]),
    "fp8q_cvt_e4m3": (_INT, [_P, _P, _I64, _P]),
    "fp8q_silu": (_INT, [_P, _P, _I64, _P]),
    "fp8q_quant_launch_config": (_INT, [_INT, _INT, _I64, _I64, _INT, _PI, _PI, _PI]),
    "fp8q_status_string": (ctypes.c_char_p, [_INT]),
    # ceiling probes (include/fp8q_probe.h)
    "fp8q_probe_mfma": (_INT, [_INT, _I64, _INT, _P, _P, _P]),
    "fp8q_probe_mfma_flops_per_iter": (_I64, [_INT]),
    "fp8q_probe_stream": (_INT, [_INT, _P, _P, _I64, _INT, _P]),
    "fp8q_last_hip_error": (_INT, []),
    "fp8q_version": (_INT, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfp8q.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp8_block_scaled_rms_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class Fp8qError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().fp8q_status_string(status).decode()
        if status == 7:
            msg += f" (hipError {lib().fp8q_last_hip_error()})"
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != 0:
        raise Fp8qError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(t: torch.Tensor, dtypes, what: str):
    if t.dtype not in dtypes:
        raise TypeError(f"{what}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")


def _shape(t: torch.Tensor, shape, what: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _numel(t: torch.Tensor, n: int, what: str):
    if t.numel() != n:
        raise ValueError(f"{what}: {t.numel()} elements, expected {n}")


def _one_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1 or next(iter(devs)).type != "cuda":
        raise ValueError(f"tensors must share one GPU device, got {sorted(map(str, devs))}")


def _scale_numel(M: int, K: int, mode: int) -> int:
    if mode in (PER_TOKEN, PER_TOKEN_UE8M0):
        return M
    if mode == PER_TENSOR_STATIC:
        return 1
    return M * (K // 128)


def _check_quant(q, scale, x, M, K, mode, what, w=None):
    """The caller's tensors must match the sizes passed to the library (the C
    interface only sees pointers)."""
    _shape(q, (M, K), f"{what}: q")
    _numel(scale, _scale_numel(M, K, mode), f"{what}: scale")
    if w is not None:
        _shape(w, (K,), f"{what}: w")
    _one_device(q, scale, x, w)


def _check_gemm(y, a, b, sa, sb, ws, n_sa, n_sb, what):
    M, K = a.shape
    N = b.shape[0]
    _shape(b, (N, K), f"{what}: b")
    _shape(y, (M, N), f"{what}: y")
    _numel(sa, n_sa, f"{what}: sa")
    _numel(sb, n_sb, f"{what}: sb")
    _one_device(y, a, b, sa, sb, ws)


_E4M3 = (torch.uint8, torch.float8_e4m3fn)
_I8 = (torch.int8,)
_BF16 = (torch.bfloat16,)
_F32T = (torch.float32,)


# ------------------------------------------------------------- C mirrors --

def fp8q_rmsnorm_quant(q, scale, x, w, eps: float, mode: int, stream=None) -> None:
    _need(q, _E4M3, "q"); _need(scale, _F32T, "scale"); _need(x, _BF16, "x"); _need(w, _BF16, "w")
    M, K = x.shape
    _check_quant(q, scale, x, M, K, mode, "fp8q_rmsnorm_quant", w)
    _check(lib().fp8q_rmsnorm_quant(_ptr(q), _ptr(scale), _ptr(x), _ptr(w), M, K, eps, mode,
                                    _stream(stream)), "fp8q_rmsnorm_quant")


def fp8q_silu_mul_quant(q, scale, gate_up, mode: int, stream=None) -> None:
    _need(q, _E4M3, "q"); _need(scale, _F32T, "scale"); _need(gate_up, _BF16, "gate_up")
    M, twoD = gate_up.shape
    if twoD % 2:
        raise ValueError("fp8q_silu_mul_quant: gate_up needs an even number of columns")
    _check_quant(q, scale, gate_up, M, twoD // 2, mode, "fp8q_silu_mul_quant")
    _check(lib().fp8q_silu_mul_quant(_ptr(q), _ptr(scale), _ptr(gate_up), M, twoD // 2, mode,
                                     _stream(stream)), "fp8q_silu_mul_quant")


def fp8q_quant(q, scale, x, mode: int, stream=None) -> None:
    _need(q, _E4M3, "q"); _need(scale, _F32T, "scale"); _need(x, _BF16, "x")
    M, K = x.shape
    _check_quant(q, scale, x, M, K, mode, "fp8q_quant")
    _check(lib().fp8q_quant(_ptr(q), _ptr(scale), _ptr(x), M, K, mode, _stream(stream)),
           "fp8q_quant")


def fp8q_scaled_mm(y, a, b, sa, sb, ws=None, cfg: int | None = None, stream=None) -> None:
    _need(y, _BF16, "y"); _need(a, _E4M3, "a"); _need(b, _E4M3, "b")
    _need(sa, _F32T, "sa"); _need(sb, _F32T, "sb")
    M, K = a.shape
    N = b.shape[0]
    _check_gemm(y, a, b, sa, sb, ws, M, N, "fp8q_scaled_mm")
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    if cfg is None:
        rc = lib().fp8q_scaled_mm(_ptr(y), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M, N, K,
                                  _ptr(ws), wsb, _stream(stream))
    else:
        rc = lib().fp8q_scaled_mm_cfg(_ptr(y), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M, N, K,
                                      _ptr(ws), wsb, cfg, _stream(stream))
    _check(rc, "fp8q_scaled_mm")


def fp8q_scaled_mm_blockwise(y, a, b, sa, sb, ws=None, cfg: int | None = None,
                             stream=None) -> None:
    _need(y, _BF16, "y"); _need(a, _E4M3, "a"); _need(b, _E4M3, "b")
    _need(sa, _F32T, "sa"); _need(sb, _F32T, "sb")
    M, K = a.shape
    N = b.shape[0]
    _check_gemm(y, a, b, sa, sb, ws, M * (K // 128), (N // 128) * (K // 128),
                "fp8q_scaled_mm_blockwise")
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    if cfg is None:
        rc = lib().fp8q_scaled_mm_blockwise(_ptr(y), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M, N,
                                            K, _ptr(ws), wsb, _stream(stream))
    else:
        rc = lib().fp8q_scaled_mm_blockwise_cfg(_ptr(y), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M,
                                                N, K, _ptr(ws), wsb, cfg, _stream(stream))
    _check(rc, "fp8q_scaled_mm_blockwise")


def fp8q_scaled_mm_blockwise_noalloc(y, a, b, sa, sb, stream=None) -> None:
    """fp8q_scaled_mm_blockwise with the split-K partials in the library's
    per-GPU scratch array (no workspace argument, nothing allocated)."""
    _need(y, _BF16, "y"); _need(a, _E4M3, "a"); _need(b, _E4M3, "b")
    _need(sa, _F32T, "sa"); _need(sb, _F32T, "sb")
    M, K = a.shape
    N = b.shape[0]
    _check_gemm(y, a, b, sa, sb, None, M * (K // 128), (N // 128) * (K // 128),
                "fp8q_scaled_mm_blockwise_noalloc")
    _check(lib().fp8q_scaled_mm_blockwise_noalloc(_ptr(y), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb),
                                                  M, N, K, _stream(stream)),
           "fp8q_scaled_mm_blockwise_noalloc")


def fp8q_scaled_mm_blockwise_ue8m0(y, a, b, sa, sb, ws=None, cfg: int | None = None,
                                   stream=None) -> None:
    _need(y, _BF16, "y"); _need(a, _E4M3, "a"); _need(b, _E4M3, "b")
    _need(sa, _F32T, "sa"); _need(sb, _F32T, "sb")
    M, K = a.shape
    N = b.shape[0]
    _check_gemm(y, a, b, sa, sb, ws, M * (K // 128), (N // 128) * (K // 128),
                "fp8q_scaled_mm_blockwise_ue8m0")
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    if cfg is None:
        rc = lib().fp8q_scaled_mm_blockwise_ue8m0(_ptr(y), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb),
                                                  M, N, K, _ptr(ws), wsb, _stream(stream))
    else:
        rc = lib().fp8q_scaled_mm_blockwise_ue8m0_cfg(_ptr(y), _ptr(a), _ptr(b), _ptr(sa),
                                                      _ptr(sb), M, N, K, _ptr(ws), wsb, cfg,
                                                      _stream(stream))
    _check(rc, "fp8q_scaled_mm_blockwise_ue8m0")


def fp8q_scaled_mm_blockwise_silu_quant(q, scale, a, b, sa, sb, stream=None) -> None:
    _need(q, _E4M3, "q"); _need(scale, _F32T, "scale"); _need(a, _E4M3, "a")
    _need(b, _E4M3, "b"); _need(sa, _F32T, "sa"); _need(sb, _F32T, "sb")
    M, K = a.shape
    N = b.shape[0]
    what = "fp8q_scaled_mm_blockwise_silu_quant"
    if N % 2:
        raise ValueError(f"{what}: b needs an even number of rows (gate rows, then up rows)")
    _shape(b, (N, K), f"{what}: b")
    _shape(q, (M, N // 2), f"{what}: q")
    _numel(scale, M * (N // 2 // 128), f"{what}: scale")
    _numel(sa, M * (K // 128), f"{what}: sa")
    _numel(sb, (N // 128) * (K // 128), f"{what}: sb")
    _one_device(q, scale, a, sa, b, sb)
    _check(lib().fp8q_scaled_mm_blockwise_silu_quant(_ptr(q), _ptr(scale), _ptr(a), _ptr(b),
                                                     _ptr(sa), _ptr(sb), M, N, K,
                                                     _stream(stream)), what)


def fp8q_rmsnorm_quant_int8(q, scale, x, w, eps: float, mode: int, stream=None) -> None:
    _need(q, _I8, "q"); _need(scale, _F32T, "scale"); _need(x, _BF16, "x"); _need(w, _BF16, "w")
    M, K = x.shape
    _check_quant(q, scale, x, M, K, mode, "fp8q_rmsnorm_quant_int8", w)
    _check(lib().fp8q_rmsnorm_quant_int8(_ptr(q), _ptr(scale), _ptr(x), _ptr(w), M, K, eps, mode,
                                         _stream(stream)), "fp8q_rmsnorm_quant_int8")


def fp8q_silu_mul_quant_int8(q, scale, gate_up, mode: int, stream=None) -> None:
    _need(q, _I8, "q"); _need(scale, _F32T, "scale"); _need(gate_up, _BF16, "gate_up")
    M, twoD = gate_up.shape
    if twoD % 2:
        raise ValueError("fp8q_silu_mul_quant_int8: gate_up needs an even number of columns")
    _check_quant(q, scale, gate_up, M, twoD // 2, mode, "fp8q_silu_mul_quant_int8")
    _check(lib().fp8q_silu_mul_quant_int8(_ptr(q), _ptr(scale), _ptr(gate_up), M, twoD // 2,
                                          mode, _stream(stream)), "fp8q_silu_mul_quant_int8")


def fp8q_quant_int8(q, scale, x, mode: int, stream=None) -> None:
    _need(q, _I8, "q"); _need(scale, _F32T, "scale"); _need(x, _BF16, "x")
    M, K = x.shape
    _check_quant(q, scale, x, M, K, mode, "fp8q_quant_int8")
    _check(lib().fp8q_quant_int8(_ptr(q), _ptr(scale), _ptr(x), M, K, mode, _stream(stream)),
           "fp8q_quant_int8")


def fp8q_scaled_mm_int8(y, a, b, sa, sb, ws=None, cfg: int | None = None, stream=None) -> None:
    _need(y, _BF16, "y"); _need(a, _I8, "a"); _need(b, _I8, "b")
    _need(sa, _F32T, "sa"); _need(sb, _F32T, "sb")
    M, K = a.shape
    N = b.shape[0]
    _check_gemm(y, a, b, sa, sb, ws, M, N, "fp8q_scaled_mm_int8")
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    if cfg is None:
        rc = lib().fp8q_scaled_mm_int8(_ptr(y), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M, N, K,
                                       _ptr(ws), wsb, _stream(stream))
    else:
        rc = lib().fp8q_scaled_mm_int8_cfg(_ptr(y), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M, N,
                                           K, _ptr(ws), wsb, cfg, _stream(stream))
    _check(rc, "fp8q_scaled_mm_int8")


def fp8q_workspace_size(op: int, M: int, N: int, K: int, cfg: int | None = None) -> int:
    if cfg is None:
        return lib().fp8q_workspace_size(op, M, N, K)
    return lib().fp8q_workspace_size_cfg(cfg, M, N, K)


def fp8q_gemm_num_configs() -> int:
    return lib().fp8q_gemm_num_configs()


def fp8q_gemm_config_name(cfg: int) -> str:
    n = lib().fp8q_gemm_config_name(cfg)
    return n.decode() if n else None


def fp8q_gemm_config_for(op: int, M: int, N: int, K: int) -> int:
    return lib().fp8q_gemm_config_for(op, M, N, K)


def fp8q_cvt_e4m3(q, x, stream=None) -> None:
    _need(q, _E4M3, "q"); _need(x, _F32T, "x")
    _numel(q, x.numel(), "fp8q_cvt_e4m3: q")
    _one_device(q, x)
    _check(lib().fp8q_cvt_e4m3(_ptr(q), _ptr(x), x.numel(), _stream(stream)), "fp8q_cvt_e4m3")


def fp8q_silu(y, g, stream=None) -> None:
    _need(y, _F32T, "y"); _need(g, _BF16, "g")
    _numel(y, g.numel(), "fp8q_silu: y")
    _one_device(y, g)
    _check(lib().fp8q_silu(_ptr(y), _ptr(g), g.numel(), _stream(stream)), "fp8q_silu")


def fp8q_version() -> int:
    return lib().fp8q_version()


FRONT_IDENT, FRONT_RMSNORM, FRONT_SILU = 0, 1, 2


def fp8q_quant_launch_config(front_end: int, mode: int, M: int, K: int, num_cus: int):
    """(threads per unit, chunks per thread, workgroups) of a quantizer call."""
    v = [ctypes.c_int(0) for _ in range(3)]
    _check(lib().fp8q_quant_launch_config(front_end, mode, M, K, num_cus,
                                          *[ctypes.byref(x) for x in v]),
           "fp8q_quant_launch_config")
    return tuple(x.value for x in v)


# --------------------------------------------------- allocating helpers --

def _scale_shape(M: int, K: int, mode: int):
    if mode in (PER_TOKEN, PER_TOKEN_UE8M0):
        return (M,)
    if mode == PER_TENSOR_STATIC:
        return (1,)
    return (M, K // 128)


def _scale_arg(M, K, mode, scale, device):
    """The scale tensor: allocated for the dynamic modes, the caller's
    one-element fp32 tensor for the static mode."""
    if mode == PER_TENSOR_STATIC:
        if scale is None:
            raise ValueError("the static mode needs scale=<one-element fp32 tensor>")
        return scale
    return torch.empty(_scale_shape(M, K, mode), dtype=torch.float32, device=device)


def rmsnorm_quant(x: torch.Tensor, w: torch.Tensor, eps: float, mode: int, stream=None,
                  scale=None):
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = _scale_arg(M, K, mode, scale, x.device)
    fp8q_rmsnorm_quant(q, s, x, w, eps, mode, stream)
    return q, s


def silu_mul_quant(gate_up: torch.Tensor, mode: int, stream=None, scale=None):
    M, twoD = gate_up.shape
    D = twoD // 2
    q = torch.empty((M, D), dtype=torch.uint8, device=gate_up.device)
    s = _scale_arg(M, D, mode, scale, gate_up.device)
    fp8q_silu_mul_quant(q, s, gate_up, mode, stream)
    return q, s


def quant(x: torch.Tensor, mode: int, stream=None, scale=None):
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = _scale_arg(M, K, mode, scale, x.device)
    fp8q_quant(q, s, x, mode, stream)
    return q, s


def _int8_out(M, K, mode, scale, device):
    q = torch.empty((M, K), dtype=torch.int8, device=device)
    if mode == PER_TENSOR_STATIC:
        if scale is None:
            raise ValueError("the static mode needs scale=<one-element fp32 tensor>")
        return q, scale
    return q, torch.empty((M,), dtype=torch.float32, device=device)


def rmsnorm_quant_int8(x, w, eps: float, mode: int, stream=None, scale=None):
    q, s = _int8_out(x.shape[0], x.shape[1], mode, scale, x.device)
    fp8q_rmsnorm_quant_int8(q, s, x, w, eps, mode, stream)
    return q, s


def silu_mul_quant_int8(gate_up, mode: int, stream=None, scale=None):
    q, s = _int8_out(gate_up.shape[0], gate_up.shape[1] // 2, mode, scale, gate_up.device)
    fp8q_silu_mul_quant_int8(q, s, gate_up, mode, stream)
    return q, s


def quant_int8(x, mode: int, stream=None, scale=None):
    q, s = _int8_out(x.shape[0], x.shape[1], mode, scale, x.device)
    fp8q_quant_int8(q, s, x, mode, stream)
    return q, s


def scaled_mm_blockwise_silu_quant(a, b, sa, sb, stream=None):
    """(q [M, N/2] e4m3, scale [M, N/256] fp32) of silu_mul_quant (group
    128) applied to the blockwise product with the gate rows b[:N/2] and the
    up rows b[N/2:], in one kernel."""
    M, N = a.shape[0], b.shape[0]
    q = torch.empty((M, N // 2), dtype=torch.uint8, device=a.device)
    s = torch.empty((M, N // 2 // 128), dtype=torch.float32, device=a.device)
    fp8q_scaled_mm_blockwise_silu_quant(q, s, a, b, sa, sb, stream)
    return q, s


def scaled_mm_blockwise_ue8m0(a, b, sa, sb, cfg: int | None = None, stream=None):
    M, N = a.shape[0], b.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    ws = _workspace(OP_SCALED_MM_BLOCKWISE_UE8M0, M, N, a.shape[1], a.device, cfg)
    fp8q_scaled_mm_blockwise_ue8m0(y, a, b, sa, sb, ws, cfg, stream)
    return y


def scaled_mm_int8(a, b, sa, sb, cfg: int | None = None, stream=None):
    M, N = a.shape[0], b.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    ws = _workspace(OP_SCALED_MM_INT8, M, N, a.shape[1], a.device, cfg)
    fp8q_scaled_mm_int8(y, a, b, sa, sb, ws, cfg, stream)
    return y


def _workspace(op, M, N, K, device, cfg=None):
    nbytes = fp8q_workspace_size(op, M, N, K, cfg)
    if nbytes == 0:
        return None
    return torch.empty(((nbytes + 3) // 4,), dtype=torch.float32, device=device)


def scaled_mm(a, b, sa, sb, cfg: int | None = None, stream=None):
    M, N = a.shape[0], b.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    ws = _workspace(OP_SCALED_MM, M, N, a.shape[1], a.device, cfg)
    fp8q_scaled_mm(y, a, b, sa, sb, ws, cfg, stream)
    return y


def scaled_mm_blockwise(a, b, sa, sb, cfg: int | None = None, stream=None):
    M, N = a.shape[0], b.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    ws = _workspace(OP_SCALED_MM_BLOCKWISE, M, N, a.shape[1], a.device, cfg)
    fp8q_scaled_mm_blockwise(y, a, b, sa, sb, ws, cfg, stream)
    return y
