"""Seeded random shapes through every GEMM entry point.

Each case draws (M, N, K) -- ragged in every dimension the format allows,
from one row up to sizes whose launch geometries differ -- and checks every
storage form of the weights against the fp64 oracle (tolerance) and against
each other (bitwise: the forms run the same arithmetic per element).  The
grouped GEMM draws a random routing over a random number of experts."""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests.gpu_util import check_parity, dev_bf16, dev_f32, dev_u8, host_codes, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def up(n, a):
    return (n + a - 1) // a * a


def shapes(seed, count, k_step, n_step, big):
    """`count` small shapes and `big` ones with wide N (the larger tiles)."""
    g = inputs.rng(seed)
    out = []
    for i in range(count + big):
        if i < count:
            M = int(g.integers(1, 9 if i % 3 == 0 else 97))   # a third in the few-row range
            N = int(g.integers(1, 601 // n_step + 1)) * n_step
            K = int(g.integers(1, 1153 // k_step + 1)) * k_step
        else:
            M = int(g.integers(60, 301))
            N = int(g.integers(4000 // n_step, 8200 // n_step + 1)) * n_step
            K = int(g.integers(1, 321 // k_step + 1)) * k_step
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", shapes(3001, 24, 1, 1, 6))
def test_bf16_three_layouts(bg, M, N, K):
    A = inputs.normal_bf16((M, K), 1.0, 3002 + M)
    B = inputs.normal_bf16((K, N), 0.5, 3003 + N)
    Ad = dev_bf16(A, up(K, 8))
    Bd = dev_bf16(B, up(N, 8))
    Btd = dev_bf16(np.ascontiguousarray(B.T), up(K, 8))
    rm = host_codes(bg.gemm_bf16(Ad, Bd))
    bt = host_codes(bg.gemm_bf16_bt(Ad, Btd))
    pk = host_codes(bg.gemm_bf16_packed(Ad, bg.pack_b_bf16(Bd)))
    torch.cuda.synchronize()
    C64, S = oracle.gemm_bf16(A, B)
    check_parity(rm, C64, S, K, f"bf16 M{M} N{N} K{K}")
    assert np.array_equal(bt, rm), f"transposed != row-major M{M} N{N} K{K}"
    assert np.array_equal(pk, rm), f"packed != row-major M{M} N{N} K{K}"


@pytest.mark.parametrize("M,N,K", shapes(3101, 20, 128, 1, 5))
def test_fp8_both_layouts(bg, M, N, K):
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 3102 + M))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, 3103 + N))
    A, sAd, sBd = dev_u8(qA), dev_f32(sA), dev_f32(sB)
    B = dev_u8(qB, up(N, 16))
    rm = host_codes(bg.gemm_fp8_blockscaled(A, sAd, B, sBd))
    pk = host_codes(bg.gemm_fp8_blockscaled_packed(A, sAd, bg.pack_b_fp8(B), sBd))
    torch.cuda.synchronize()
    C64, S = oracle.gemm_fp8bs(qA, sA, qB, sB)
    check_parity(rm, C64, S, K, f"fp8 M{M} N{N} K{K}")
    assert np.array_equal(pk, rm), f"packed != row-major M{M} N{N} K{K}"


@pytest.mark.parametrize("M,N,K", shapes(3201, 20, 32, 2, 5))
def test_fp4_both_layouts(bg, M, N, K):
    A = inputs.normal_bf16((M, K), 1.0, 3202 + M)
    Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, 3203 + N))
    Ad = dev_bf16(A, up(K, 8))
    Bqd, sBd = dev_u8(Bq, up(N // 2, 16)), dev_u8(sB, up(N, 16))
    rm = host_codes(bg.gemm_fp4_w(Ad, Bqd, sBd, N))
    pk = host_codes(bg.gemm_fp4_w_packed(Ad, bg.pack_b_fp4(Bqd, sBd, N)))
    torch.cuda.synchronize()
    C64, S = oracle.gemm_fp4w(A, Bq, sB, N)
    check_parity(rm, C64, S, K, f"fp4 M{M} N{N} K{K}")
    assert np.array_equal(pk, rm), f"packed != row-major M{M} N{N} K{K}"


@pytest.mark.parametrize("M,N,K", shapes(3301, 14, 128, 2, 4))
def test_w4a8(bg, M, N, K):
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 3302 + M))
    Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, 3303 + N))
    Bp = bg.pack_b_mxfp4(dev_u8(Bq, up(N // 2, 16)), dev_u8(sE, up(N, 16)), N)
    got = host_codes(bg.gemm_w4a8_packed(dev_u8(qA), dev_f32(sA), Bp))
    torch.cuda.synchronize()
    C64, S = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    check_parity(got, C64, S, K, f"w4a8 M{M} N{N} K{K}")


@pytest.mark.parametrize("case", range(20))
def test_grouped_random_routing(bg, case):
    g = inputs.rng(3400 + case)
    E = int(g.integers(1, 9))
    T = int(g.integers(1, 700))
    N = int(g.integers(1, 1200)) if case % 3 else int(g.integers(2000, 4200))
    K = int(g.integers(1, 400))
    skew = float(g.choice([0.0, 1.0, 3.0]))
    A = inputs.normal_bf16((T, K), 1.0, 3410 + case)
    Bs = [inputs.normal_bf16((K, N), 0.05, 3420 + 10 * case + e) for e in range(E)]
    order, offsets = inputs.group_by_expert(inputs.route_tokens(T, E, 3430 + case, skew), E)
    A = np.ascontiguousarray(A[order])
    Bp = bg.pack_b_bf16_grouped([dev_bf16(b, up(N, 8)) for b in Bs])
    off = torch.as_tensor(offsets, device="cuda")
    got = host_codes(bg.gemm_bf16_grouped_packed(dev_bf16(A, up(K, 8)), off, Bp))
    torch.cuda.synchronize()
    C64, S = oracle.gemm_bf16_grouped(A, offsets, Bs)
    check_parity(got, C64, S, K, f"grouped E{E} T{T} N{N} K{K} skew{skew}")
