"""The Python binding's extent checks.  The C ABI receives pointers and row
pitches only, so it cannot see how long a tensor is: an output or scale tensor
shorter than the call implies would be written or read past its end.  The
binding checks every operand's shape and device first and raises ValueError
before anything is launched.  These tests allocate device tensors (hence the
gpu mark) but launch no kernel."""
import pytest
import torch

from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def z(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def u8(*shape):
    return z(*shape, dtype=torch.uint8)


def f32(*shape):
    return z(*shape, dtype=torch.float32)


def test_out_shape_and_device(bg):
    A, B = z(256, 64), z(64, 32)
    with pytest.raises(ValueError, match="out"):
        bg.gemm_bf16(A, B, out=z(1, 32))            # one row where 256 are written
    with pytest.raises(ValueError, match="out"):
        bg.gemm_bf16(A, B, out=z(256, 16))
    with pytest.raises(ValueError, match="out"):
        bg.gemm_bf16(A, B, out=torch.zeros((256, 32), dtype=torch.bfloat16))   # host tensor
    with pytest.raises(ValueError, match="out"):
        bg.gemm_bf16_bt(A, z(32, 64), out=z(255, 32))
    Bp = bg.pack_b_bf16(B)
    with pytest.raises(ValueError, match="out"):
        bg.gemm_bf16_packed(A, Bp, out=z(8, 32))


def test_fp8_scale_shapes(bg):
    M, N, K = 16, 256, 256
    A, B = u8(M, K), u8(K, N)
    with pytest.raises(ValueError, match="sA"):
        bg.gemm_fp8_blockscaled(A, f32(1, K // 128), B, f32(K // 128, 2))
    with pytest.raises(ValueError, match="sB"):
        bg.gemm_fp8_blockscaled(A, f32(M, K // 128), B, f32(1, 2))
    with pytest.raises(ValueError, match="multiple of 128"):
        bg.gemm_fp8_blockscaled(u8(M, 200), f32(M, 2), u8(200, N), f32(2, 2))
    Bp = bg.pack_b_fp8(B)
    with pytest.raises(ValueError, match="sA"):
        bg.gemm_fp8_blockscaled_packed(A, f32(M - 1, K // 128), Bp, f32(K // 128, 2))
    with pytest.raises(ValueError, match="sB"):
        bg.gemm_fp8_blockscaled_packed(A, f32(M, K // 128), Bp, f32(K // 128, 1))


def test_fp4_code_and_scale_shapes(bg):
    M, N, K = 8, 64, 128
    A = z(M, K)
    with pytest.raises(ValueError, match="sB"):
        bg.gemm_fp4_w(A, u8(K, N // 2), u8(1, N), N)
    with pytest.raises(ValueError, match="Bq"):
        bg.gemm_fp4_w(A, u8(K, N // 4), u8(K // 32, N), N)
    with pytest.raises(ValueError, match="sB"):
        bg.pack_b_fp4(u8(K, N // 2), u8(K // 32 - 1, N), N)
    with pytest.raises(ValueError, match="sE"):
        bg.pack_b_mxfp4(u8(K, N // 2), u8(K // 32, N - 2), N)
    Bp = bg.pack_b_mxfp4(u8(K, N // 2), u8(K // 32, N), N)
    with pytest.raises(ValueError, match="sA"):
        bg.gemm_w4a8_packed(u8(M, K), f32(1, 1), Bp)


def test_splitk_and_attention_shapes(bg):
    with pytest.raises(ValueError, match="inner"):
        bg.gemm_bf16_splitk(z(4, 64), z(32, 16), f32(64))
    Q = z(2, 8, 128)
    Kc = z(2, 2, 64, 128)
    with pytest.raises(ValueError, match="seq_lens"):
        bg.decode_attention(Q, Kc, Kc, torch.zeros(1, dtype=torch.int32, device="cuda"), 0.1)
    with pytest.raises(ValueError, match="out"):
        bg.decode_attention(Q, Kc, Kc, torch.zeros(2, dtype=torch.int32, device="cuda"), 0.1,
                            out=z(1, 8, 128))
