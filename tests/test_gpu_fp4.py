"""GPU parity and batch-invariance tests of bi_gemm_fp4_w (C ABI).

bf16 activations times e2m1 weights with one e4m3fn scale per 32 K per column,
dequantised inside the K loop (section 3.2 of the lshu.cn article).
"""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests import full_size
from tests.gpu_util import (check_parity, dev_bf16, dev_u8, host_codes, require_gpu, rows_equal)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def run(bg, A, Bq, sB, N, lda=None):
    C = bg.gemm_fp4_w(dev_bf16(A, lda), dev_u8(Bq, (Bq.shape[1] + 15) // 16 * 16),
                      dev_u8(sB, (sB.shape[1] + 15) // 16 * 16), N)
    torch.cuda.synchronize()
    return host_codes(C)


def pack(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_every_code_scale_pair_exact(bg):
    """All 16 e2m1 codes x all 254 finite e4m3fn scale codes: A one-hot selects
    one 32-K block per row, so C[m, n] = e2m1(n) * e4m3(scale m) exactly (bf16
    holds every such product)."""
    scodes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    M, N, K = len(scodes), 16, len(scodes) * 32
    codes = np.tile(np.arange(16, dtype=np.uint8), (K, 1))
    Bq = pack(codes)
    sB = np.repeat(scodes[:, None], N, axis=1)          # block m has scale code scodes[m]
    A = np.zeros((M, K), np.float32)
    A[np.arange(M), 32 * np.arange(M)] = 1.0
    got = run(bg, inputs.f32_to_bf16_codes(A), Bq, sB, N)
    C64, _ = oracle.gemm_fp4w(inputs.f32_to_bf16_codes(A), Bq, sB, N)
    assert np.array_equal(got, oracle.round_bf16(C64))


def test_nan_scale_propagates(bg):
    # a NaN scale (S.1111.111) poisons its block, as in the oracle
    M, N, K = 2, 32, 64
    Bq = np.full((K, N // 2), 0x22, np.uint8)           # every weight code 2 (1.0)
    sB = np.full((K // 32, N), 0x38, np.uint8)
    sB[1, 5] = 0x7F
    A = inputs.f32_to_bf16_codes(np.ones((M, K), np.float32))
    got = inputs.bf16_codes_to_f32(run(bg, A, Bq, sB, N))
    C64, _ = oracle.gemm_fp4w(A, Bq, sB, N)
    assert np.array_equal(np.isnan(got), np.isnan(C64))
    assert np.isnan(got[:, 5]).all() and not np.isnan(np.delete(got, 5, axis=1)).any()


def dyadic_bf16(shape, seed):
    g = inputs.rng(seed)
    m = g.integers(-15, 16, size=shape).astype(np.float64)
    e = g.integers(-2, 2, size=shape)
    return inputs.f32_to_bf16_codes(np.ldexp(m, e).astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(17, 256, 512), (33, 96, 288), (1, 32, 32), (70, 1024, 512)])
def test_exact_dyadic_bitwise(bg, M, N, K):
    # power-of-two scales (mantissa 0) and dyadic activations: every block sum
    # and every scaled accumulation is exact in fp32
    A = dyadic_bf16((M, K), 60 + M)
    g = inputs.rng(70 + N)
    Bq = g.integers(0, 256, size=(K, N // 2)).astype(np.uint8)
    sB = ((g.integers(5, 10, size=(K // 32, N)) << 3)).astype(np.uint8)   # 2^-2 .. 2^2
    C64, _ = oracle.gemm_fp4w(A, Bq, sB, N)
    assert np.array_equal(run(bg, A, Bq, sB, N), oracle.round_bf16(C64))


@pytest.mark.parametrize("M,N,K", [(1, 14336, 4096), (8, 1024, 4096), (64, 512, 1024), (130, 96, 320)])
def test_parity_random(bg, M, N, K):
    A = inputs.normal_bf16((M, K), 1.0, 401 + M)
    Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, 402 + N))
    C64, S = oracle.gemm_fp4w(A, Bq, sB, N)
    check_parity(run(bg, A, Bq, sB, N), C64, S, K, f"fp4 M{M} N{N} K{K}")


@pytest.fixture(scope="module")
def c4(bg):
    # fp4 e2m1 weight-only K=4096, N=14336; weights N(0,0.02) before quantisation
    A, Bq, sB, _, _ = full_size.c4()
    return A, Bq, sB, dev_bf16(A), dev_u8(Bq), dev_u8(sB)


def test_c4_invariance(bg, c4):
    A, Bq, sB, Ad, Bd, sBd = c4
    N = 14336
    ref = torch.cat([bg.gemm_fp4_w(Ad[i:i + 1], Bd, sBd, N) for i in range(512)])
    for m in (1, 8, 64, 512, 3, 100, 257):
        ok = rows_equal(bg.gemm_fp4_w(Ad[:m], Bd, sBd, N), ref[:m])
        assert bool(ok.all()), f"M={m}"
    for s in range(2):
        p = torch.as_tensor(inputs.permutation(512, 403 + s), device="cuda")
        ok = rows_equal(bg.gemm_fp4_w(Ad.index_select(0, p), Bd, sBd, N), ref.index_select(0, p))
        assert bool(ok.all()), f"shuffle {s}"


def test_c4_parity_every_row(bg, c4):
    A, Bq, sB, Ad, Bd, sBd = c4
    *_, C64, S = full_size.c4()
    C = host_codes(bg.gemm_fp4_w(Ad, Bd, sBd, 14336))          # M = 512, every row
    check_parity(full_size.all_rows(C, C64), C64, S, 4096, "C4 M=512 every row")
