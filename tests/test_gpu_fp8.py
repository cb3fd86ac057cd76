"""GPU parity and batch-invariance tests of bi_gemm_fp8_blockscaled (C ABI).

Formats: OCP e4m3fn codes, fp32 scales per 1x128 block of A and per 128x128
block of B (the block-scaled FP8 GEMM that section 3.2 of the lshu.cn article
describes as dequantised inside the K loop).
"""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests import full_size
from tests.gpu_util import check_parity, dev_f32, dev_u8, host_codes, require_gpu, rows_equal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def run(bg, qA, sA, qB, sB, ldb=None):
    N = qB.shape[1]
    if ldb is None:
        ldb = (N + 15) // 16 * 16
    C = bg.gemm_fp8_blockscaled(dev_u8(qA), dev_f32(sA), dev_u8(qB, ldb), dev_f32(sB))
    torch.cuda.synchronize()
    return host_codes(C)


def small_codes(shape, seed):
    """e4m3 codes of +-{1, 1.125, ..., 3.75} * 2^{-1..1}: 4-bit significands in a
    narrow exponent range, so every block sum of 128 products is exact in fp32."""
    g = inputs.rng(seed)
    e = g.integers(6, 9, size=shape)          # biased exponent 6..8 -> 2^-1 .. 2^1
    m = g.integers(0, 8, size=shape)
    s = g.integers(0, 2, size=shape)
    return ((s << 7) | (e << 3) | m).astype(np.uint8)


def pow2(shape, seed, lo=-3, hi=3):
    return np.ldexp(1.0, inputs.rng(seed).integers(lo, hi + 1, size=shape)).astype(np.float32)


# ------------------------------------------------------------------ exact pins


def test_identity_pins_unit_scale_encoding(bg):
    """B = identity (code 0x38 = 1.0) with power-of-two scales: C = A * sA * sB
    exactly.  This also pins the MFMA's unit E8M0 scale (127 -> 2^0)."""
    M, K = 20, 256
    qA = small_codes((M, K), 1)
    sA = pow2((M, K // 128), 2)
    qB = np.zeros((K, K), np.uint8)
    qB[np.arange(K), np.arange(K)] = 0x38
    sB = pow2((K // 128, K // 128), 3)
    C64, _ = oracle.gemm_fp8bs(qA, sA, qB, sB)
    assert np.array_equal(run(bg, qA, sA, qB, sB), oracle.round_bf16(C64))


@pytest.mark.parametrize("M,N,K", [(17, 256, 512), (65, 144, 384), (1, 16, 128), (130, 2048, 1024)])
def test_exact_small_codes_bitwise(bg, M, N, K):
    qA = small_codes((M, K), 10 + M)
    qB = small_codes((K, N), 20 + N)
    # scales in {1, 2}: keeps the cross-block fp32 accumulation exact too
    sA = pow2((M, K // 128), 30 + M, 0, 1)
    sB = pow2((K // 128, (N + 127) // 128), 40 + N, 0, 1)
    C64, _ = oracle.gemm_fp8bs(qA, sA, qB, sB)
    assert np.array_equal(run(bg, qA, sA, qB, sB), oracle.round_bf16(C64))


# ------------------------------------------------------------------ tolerance parity


@pytest.mark.parametrize("M,N,K", [(1, 2048, 7168), (37, 2048, 7168), (129, 300, 1024), (8, 16, 128),
                                   (64, 512, 2048)])
def test_parity_random(bg, M, N, K):
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 301 + M))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, 302 + N))
    C64, S = oracle.gemm_fp8bs(qA, sA, qB, sB)
    check_parity(run(bg, qA, sA, qB, sB), C64, S, K, f"fp8 M{M} N{N} K{K}")


def test_strided_scales_and_operands(bg):
    M, N, K = 33, 160, 512
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 51))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, 52))
    base = run(bg, qA, sA, qB, sB)
    # padded pitches for every operand
    A = dev_u8(qA, K + 64)
    B = dev_u8(qB, 256)
    sAp = torch.zeros((M, 7), dtype=torch.float32, device="cuda")
    sAp[:, :4] = torch.from_numpy(sA).cuda()
    sBp = torch.zeros((4, 5), dtype=torch.float32, device="cuda")
    sBp[:, :2] = torch.from_numpy(sB).cuda()
    C = bg.gemm_fp8_blockscaled(A, sAp[:, :4], B, sBp[:, :2])
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(C), base)


# ------------------------------------------------------------------ invariance (C3)


@pytest.fixture(scope="module")
def c3(bg):
    # fp8 e4m3 K=7168, N=2048; activations 1x128 fp32 scales, weights 128x128
    qA, sA, qB, sB, _, _ = full_size.c3()
    return qA, sA, qB, sB, dev_u8(qA), dev_f32(sA), dev_u8(qB), dev_f32(sB)


def test_c3_invariance_every_m(bg, c3):
    qA, sA, qB, sB, A, sAd, B, sBd = c3
    ref = torch.cat([bg.gemm_fp8_blockscaled(A[i:i + 1], sAd[i:i + 1], B, sBd) for i in range(512)])
    for m in range(1, 513):
        out = bg.gemm_fp8_blockscaled(A[:m], sAd[:m], B, sBd)
        ok = rows_equal(out, ref[:m])
        assert bool(ok.all()), f"M={m}: rows {torch.nonzero(~ok).flatten()[:8].tolist()} differ"
    for m, seed in ((37, 303), (129, 304), (512, 305)):
        p = torch.as_tensor(inputs.rng(seed).choice(512, size=m, replace=False), device="cuda")
        ok = rows_equal(bg.gemm_fp8_blockscaled(A.index_select(0, p), sAd.index_select(0, p), B, sBd),
                        ref.index_select(0, p))
        assert bool(ok.all()), f"shuffle M={m}"


def test_c3_parity_every_row(bg, c3):
    qA, sA, qB, sB, A, sAd, B, sBd = c3
    *_, C64, S = full_size.c3()
    C = host_codes(bg.gemm_fp8_blockscaled(A, sAd, B, sBd))     # M = 512, every row
    check_parity(full_size.all_rows(C, C64), C64, S, 7168, "C3 M=512 every row")
