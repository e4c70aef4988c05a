"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before touching any device.

Pointers passed here are fake (never dereferenced): every call either fails
validation on the host, or -- only where no GPU is present -- stops at the
device check with FP8Q_ERR_NO_DEVICE.
"""
import ctypes
import os
import re

import pytest
import torch

import fp8_block_scaled_rms_amd as fq

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")

OK, INVALID, SHAPE, ALIGN, WS, NODEV, ARCH, HIP, MODE, CFG = range(10)

A, B, C, D, E = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000  # 16-byte aligned fakes


def _declared_functions():
    """Every function declared in include/*.h."""
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(fp8q_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def _no_gpu():
    return torch.cuda.device_count() == 0


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fq.LIB_PATH)
    names = _declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    # and the binding declares a signature for each of them
    assert set(names) == set(fq.SIGNATURES)


def test_version_and_status_strings():
    L = fq.lib()
    assert L.fp8q_version() == 200
    for s in range(10):
        assert L.fp8q_status_string(s)
    assert L.fp8q_status_string(99) == b"unknown status"


def test_quant_argument_checks():
    L = fq.lib()
    rms = L.fp8q_rmsnorm_quant
    assert rms(A, B, C, D, -1, 256, 1e-6, 1, None) == INVALID
    assert rms(A, B, C, D, 4, 0, 1e-6, 1, None) == INVALID
    assert rms(A, B, C, D, 4, 256, 1e-6, 5, None) == MODE
    assert rms(A, B, C, D, 4, 256, 1e-6, -1, None) == MODE
    assert rms(A, B, C, D, 4, 200, 1e-6, 4, None) == SHAPE       # K % 128 (group, UE8M0)
    assert rms(A, B, C, D, 4, 200, 1e-6, 3, None) != SHAPE       # K % 8 suffices per token
    assert rms(A, B, C, D, 4, 200, 1e-6, 2, None) != SHAPE       # and for the static mode
    assert rms(A, 0, C, D, 4, 256, 1e-6, 2, None) == INVALID     # static mode reads scale
    assert rms(A, B, C, D, 0, 256, 1e-6, 1, None) == OK          # M == 0: no-op
    assert rms(0, 0, 0, 0, 0, 256, 1e-6, 1, None) == OK          # not inspected
    assert rms(0, B, C, D, 4, 256, 1e-6, 1, None) == INVALID
    assert rms(A, B, C, 0, 4, 256, 1e-6, 1, None) == INVALID
    assert rms(A + 8, B, C, D, 4, 256, 1e-6, 1, None) == ALIGN
    assert rms(A, B, C, D + 2, 4, 256, 1e-6, 1, None) == ALIGN
    assert rms(A, B, C, D, 4, 200, 1e-6, 1, None) == SHAPE       # K % 128 (group)
    assert rms(A, B, C, D, 4, 12, 1e-6, 0, None) == SHAPE        # K % 8 (per token)
    assert rms(A, B, C, D, 4, 65536, 1e-6, 0, None) == SHAPE     # K too large
    assert rms(A, B, C, D, 4, 256, 0.0, 1, None) == INVALID      # eps
    assert rms(A, B, C, D, 4, 256, float("inf"), 1, None) == INVALID
    assert rms(A, B, C, D, 4, 256, float("nan"), 1, None) == INVALID
    silu = L.fp8q_silu_mul_quant
    assert silu(A, B, C, 4, 0, 1, None) == INVALID
    assert silu(A, B, C, 4, 100, 1, None) == SHAPE
    assert silu(A, B, C + 4, 4, 128, 1, None) == ALIGN
    assert silu(A, B, C, 4, 128, 7, None) == MODE
    q = L.fp8q_quant
    assert q(A, B, C, 4, 136, 1, None) == SHAPE
    assert q(A, 0, C, 4, 128, 1, None) == INVALID


def test_gemm_argument_checks():
    L = fq.lib()
    mm = L.fp8q_scaled_mm
    bw = L.fp8q_scaled_mm_blockwise
    assert mm(A, B, C, D, E, 0, 256, 256, None, 0, None) == OK
    assert mm(A, B, C, D, E, -1, 256, 256, None, 0, None) == INVALID
    assert mm(A, B, C, D, E, 4, 200, 256, None, 0, None) == SHAPE
    assert mm(A, B, C, D, E, 4, 256, 100, None, 0, None) == SHAPE
    assert mm(A, B, C, D, E, 4, 0, 256, None, 0, None) == INVALID
    assert mm(A + 2, B, C, D, E, 4, 256, 256, None, 0, None) == ALIGN
    assert bw(A, B, C, D, 0, 4, 256, 256, None, 0, None) == INVALID
    assert bw(A, B, C, D, E + 4, 4, 256, 256, None, 0, None) == ALIGN
    # forced variants
    n = L.fp8q_gemm_num_configs()
    assert n > 4
    assert L.fp8q_scaled_mm_cfg(A, B, C, D, E, 4, 256, 256, None, 0, n, None) == CFG
    # a skinny variant cannot take more tokens than its fragment count
    sk = next(i for i in range(n) if "_skinny_t1_" in fq.fp8q_gemm_config_name(i))
    assert L.fp8q_scaled_mm_cfg(A, B, C, D, E, 17, 256, 256, None, 0, sk, None) == CFG
    # a skinny variant covering wk*j = 8 K blocks per workgroup needs a
    # workspace of split = ceil(K/128 / 8) fp32 partials once K > 1024
    sp = next(i for i in range(n) if fq.fp8q_gemm_config_name(i) == "f16_skinny_t1_r1_k4_j2")
    assert L.fp8q_workspace_size_cfg(sp, 8, 256, 1024) == 0
    need = L.fp8q_workspace_size_cfg(sp, 8, 256, 4096)
    assert need == 4 * 8 * 256 * 4
    assert L.fp8q_scaled_mm_cfg(A, B, C, D, E, 8, 256, 4096, None, 0, sp, None) == WS
    assert L.fp8q_scaled_mm_cfg(A, B, C, D, E, 8, 256, 4096, A, need - 1, sp, None) == WS


def test_fused_silu_quant_gemm_argument_checks():
    L = fq.lib()
    f = L.fp8q_scaled_mm_blockwise_silu_quant
    # (q, scale, a, b, sa, sb, M, N, K, stream)
    assert f(A, B, C, D, E, A, 0, 256, 256, None) == OK              # M == 0: no-op
    assert f(0, 0, 0, 0, 0, 0, 0, 256, 256, None) == OK              # not inspected
    assert f(A, B, C, D, E, A, -1, 256, 256, None) == INVALID
    assert f(A, B, C, D, E, A, 4, 0, 256, None) == INVALID
    assert f(A, B, C, D, E, A, 4, 384, 256, None) == SHAPE           # N/2 not whole groups
    assert f(A, B, C, D, E, A, 4, 256, 100, None) == SHAPE           # K % 128
    assert f(A, 0, C, D, E, A, 4, 256, 256, None) == INVALID         # scale
    assert f(A, B + 4, C, D, E, A, 4, 256, 256, None) == ALIGN
    assert f(A, B, C, D, 0, A, 4, 256, 256, None) == INVALID         # sa
    # a tile's rows are addressed with 32-bit byte offsets from its first
    # gate row: (N/2 + 128) * K must stay below 2^32
    assert f(A, B, C, D, E, A, 4, 2 * (2**20 - 128), 4096, None) == SHAPE
    assert f(A, B, C, D, E, A, 4, 2**22, 2**22, None) == SHAPE       # K > 2^22


def test_noalloc_gemm_argument_checks():
    L = fq.lib()
    f = L.fp8q_scaled_mm_blockwise_noalloc
    assert f(A, B, C, D, E, 0, 256, 256, None) == OK
    assert f(A, B, C, D, E, -1, 256, 256, None) == INVALID
    assert f(A, B, C, D, E, 4, 200, 256, None) == SHAPE
    assert f(A + 2, B, C, D, E, 4, 256, 256, None) == ALIGN
    # a shape whose table variant needs more split-K partials than the
    # scratch array holds is refused on the host, before any device call
    # (M=1024 x N=5120 x K=25600: every column split four ways, 84 MB)
    M, N, K = 1024, 5120, 25600
    assert fq.fp8q_workspace_size(fq.OP_SCALED_MM_BLOCKWISE, M, N, K) > 64 << 20
    assert f(A, B, C, D, E, M, N, K, None) == WS
    # every blockwise shape of the workloads fits
    decode = [(M, N, K) for M in (1, 2, 4, 8, 16, 32)
              for N, K in ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288))]
    prefill = [(M, N, K) for M in (2048, 8192)
               for N, K in ((10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600))]
    for M, N, K in decode + prefill + [(64, 5120, 25600), (4096, 5120, 25600)]:
        assert fq.fp8q_workspace_size(fq.OP_SCALED_MM_BLOCKWISE, M, N, K) <= 64 << 20


def test_gemm_k_limit():
    # the tiled kernels address 256 rows of K bytes with 32-bit offsets
    L = fq.lib()
    for g in (L.fp8q_scaled_mm_blockwise, L.fp8q_scaled_mm_blockwise_ue8m0):
        assert g(A, B, C, D, E, 4, 256, 2**22 + 128, None, 0, None) == SHAPE
    assert L.fp8q_scaled_mm(A, B, C, D, E, 4, 256, 2**22 + 128, None, 0, None) == SHAPE


def test_int8_argument_checks():
    L = fq.lib()
    assert L.fp8q_quant_int8(A, B, C, 4, 128, 1, None) == MODE        # group: not for int8
    assert L.fp8q_quant_int8(A, B, C, 4, 128, 3, None) == MODE        # UE8M0: not for int8
    assert L.fp8q_rmsnorm_quant_int8(A, B, C, D, 4, 100, 1e-6, 0, None) == SHAPE
    assert L.fp8q_rmsnorm_quant_int8(A, B, C, D, 4, 256, 0.0, 0, None) == INVALID
    assert L.fp8q_silu_mul_quant_int8(A, B, C + 2, 4, 128, 0, None) == ALIGN
    mm8 = L.fp8q_scaled_mm_int8
    assert mm8(A, B, C, D, E, 0, 256, 256, None, 0, None) == OK
    assert mm8(A, B, C, D, E, 4, 256, 100, None, 0, None) == SHAPE
    assert mm8(A, B, C, D, E, 4, 256, 131072 + 128, None, 0, None) == SHAPE  # int32 bound
    # engines serve only their own op
    n = L.fp8q_gemm_num_configs()
    i8 = next(i for i in range(n) if fq.fp8q_gemm_config_name(i).startswith("i8_tiled"))
    f16 = next(i for i in range(n) if fq.fp8q_gemm_config_name(i).startswith("f16_tiled"))
    assert L.fp8q_scaled_mm_int8_cfg(A, B, C, D, E, 4, 256, 256, None, 0, f16, None) == CFG
    assert L.fp8q_scaled_mm_cfg(A, B, C, D, E, 4, 256, 256, None, 0, i8, None) == CFG
    assert L.fp8q_scaled_mm_blockwise_cfg(A, B, C, D, E, 4, 256, 256, None, 0, i8, None) == CFG
    for M in (1, 16, 128, 512, 2048):
        cfg = fq.fp8q_gemm_config_for(fq.OP_SCALED_MM_INT8, M, 4096, 2048)
        assert fq.fp8q_gemm_config_name(cfg).startswith("i8_")


def test_elementwise_argument_checks():
    L = fq.lib()
    assert L.fp8q_cvt_e4m3(A, B, 0, None) == OK
    assert L.fp8q_cvt_e4m3(A, B, -1, None) == INVALID
    assert L.fp8q_cvt_e4m3(0, B, 5, None) == INVALID
    assert L.fp8q_silu(A, B + 2, 5, None) == ALIGN


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device path; a GPU is present")
def test_valid_calls_report_no_device_without_gpu():
    L = fq.lib()
    assert L.fp8q_rmsnorm_quant(A, B, C, D, 4, 256, 1e-6, 1, None) == NODEV
    assert L.fp8q_silu_mul_quant(A, B, C, 4, 128, 0, None) == NODEV
    assert L.fp8q_quant(A, B, C, 4, 128, 1, None) == NODEV
    assert L.fp8q_scaled_mm(A, B, C, D, E, 4, 256, 256, None, 0, None) == NODEV
    assert L.fp8q_scaled_mm_blockwise(A, B, C, D, E, 4, 256, 256, None, 0, None) == NODEV
    assert L.fp8q_scaled_mm_blockwise_noalloc(A, B, C, D, E, 4, 256, 256, None) == NODEV
    assert L.fp8q_cvt_e4m3(A, B, 16, None) == NODEV
    assert L.fp8q_silu(A, B, 16, None) == NODEV
    assert L.fp8q_quant_int8(A, B, C, 4, 128, 0, None) == NODEV
    assert L.fp8q_scaled_mm_int8(A, B, C, D, E, 4, 256, 256, None, 0, None) == NODEV


def test_dispatch_table_covers_every_workload_shape():
    """Every GEMM shape of the Qwen3 workloads resolves to a variant that can
    run it, and the workspace query agrees with that variant."""
    shapes = []
    for M in (1, 16, 128, 512, 2048):
        for N, K in ((4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144)):
            shapes.append((0, M, N, K))
    for M in (1, 2, 4, 8, 16, 32):
        for N, K in ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)):
            shapes.append((1, M, N, K))
    for M in (2048, 8192):
        for N, K in ((10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)):
            shapes.append((1, M, N, K))
    for M in (64, 4096):
        shapes.append((1, M, 5120, 25600))
    shapes.append((1, 16, 512, 256))
    for op, M, N, K in shapes:
        cfg = fq.fp8q_gemm_config_for(op, M, N, K)
        assert cfg >= 0, (op, M, N, K)
        assert fq.fp8q_workspace_size(op, M, N, K) == fq.fp8q_workspace_size(op, M, N, K, cfg)
        name = fq.fp8q_gemm_config_name(cfg)
        assert name.startswith("f16_"), name  # the default is the exact engine
        if "_skinny_t" in name:
            assert M <= 16 * int(name.split("_skinny_t")[1].split("_")[0])
