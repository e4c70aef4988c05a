"""CPU checks of the Python binding's own validation: the C interface only
sees pointers, so the binding must refuse tensors whose shapes or devices do
not match the sizes it passes (no library call is made in these cases)."""
import pytest
import torch

import fp8_block_scaled_rms_amd as fq


def _t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_quantizer_shapes_are_checked():
    x = _t((4, 256), torch.bfloat16)
    w = _t((256,), torch.bfloat16)
    with pytest.raises(ValueError, match="q"):
        fq.fp8q_rmsnorm_quant(_t((4, 128), torch.uint8), _t((4,), torch.float32), x, w, 1e-6,
                              fq.PER_TOKEN)
    with pytest.raises(ValueError, match="scale"):
        fq.fp8q_rmsnorm_quant(_t((4, 256), torch.uint8), _t((4,), torch.float32), x, w, 1e-6,
                              fq.GROUP128)  # needs 4 * 2 scales
    with pytest.raises(ValueError, match="w"):
        fq.fp8q_rmsnorm_quant(_t((4, 256), torch.uint8), _t((4,), torch.float32), x,
                              _t((128,), torch.bfloat16), 1e-6, fq.PER_TOKEN)
    with pytest.raises(ValueError, match="even"):
        fq.fp8q_silu_mul_quant(_t((4, 128), torch.uint8), _t((4,), torch.float32),
                               _t((4, 257), torch.bfloat16), fq.PER_TOKEN)
    with pytest.raises(ValueError, match="scale"):
        fq.fp8q_quant(_t((4, 256), torch.uint8), _t((4,), torch.float32), x,
                      fq.PER_TENSOR_STATIC)  # static: exactly one scale
    with pytest.raises(TypeError):
        fq.fp8q_quant_int8(_t((4, 256), torch.uint8), _t((4,), torch.float32), x, fq.PER_TOKEN)


def test_gemm_shapes_are_checked():
    a = _t((8, 256), torch.uint8)
    b = _t((128, 256), torch.uint8)
    y = _t((8, 128), torch.bfloat16)
    with pytest.raises(ValueError, match="b"):
        fq.fp8q_scaled_mm(y, a, _t((128, 128), torch.uint8), _t((8,), torch.float32),
                          _t((128,), torch.float32))
    with pytest.raises(ValueError, match="y"):
        fq.fp8q_scaled_mm(_t((8, 64), torch.bfloat16), a, b, _t((8,), torch.float32),
                          _t((128,), torch.float32))
    with pytest.raises(ValueError, match="sa"):
        fq.fp8q_scaled_mm_blockwise(y, a, b, _t((8,), torch.float32), _t((1, 2), torch.float32))
    with pytest.raises(ValueError, match="sb"):
        fq.fp8q_scaled_mm_blockwise(y, a, b, _t((8, 2), torch.float32), _t((3,), torch.float32))


def test_cpu_tensors_are_refused():
    x = _t((4, 256), torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8q_quant(_t((4, 256), torch.uint8), _t((4,), torch.float32), x, fq.PER_TOKEN)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8q_scaled_mm_int8(_t((8, 128), torch.bfloat16), _t((8, 256), torch.int8),
                               _t((128, 256), torch.int8), _t((8,), torch.float32),
                               _t((128,), torch.float32))
