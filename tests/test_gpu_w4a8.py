"""GPU tests of the W4A8 GEMM (fp8 e4m3fn activations x OCP MXFP4 weights),
bi_gemm_w4a8_packed, against the fp64 oracle.

The weights' E8M0 block scale is applied by the MFMA itself (one scale per
lane = per 32 K of a column); the exhaustive test below pins that lane
layout, the nibble order and the unit activation scale bit for bit."""
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


def pack4(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def pad16(n):
    return (n + 15) // 16 * 16


def run(bg, qA, sA, Bq, sE, N, A=None, sAd=None):
    A = dev_u8(qA) if A is None else A
    sAd = dev_f32(sA) if sAd is None else sAd
    Bp = bg.pack_b_mxfp4(dev_u8(Bq, pad16(Bq.shape[1])), dev_u8(sE, pad16(sE.shape[1])), N)
    C = bg.gemm_w4a8_packed(A, sAd, Bp)
    torch.cuda.synchronize()
    return host_codes(C)


def onehot_case(e_lo, e_hi, K=1024, N=16):
    """Row m of A is 1.0 at k = m only; weight codes random per (k, n), each
    column holding every code; block scales cycle through E8M0 exponents
    e_lo..e_hi.  C[m, n] is then one product, e2m1(code(m, n)) *
    2^(sE[m/32, n] - 127), so any mix-up of K positions -- in the operands or
    in the scale lanes -- changes some output."""
    M = K
    qA = np.zeros((M, K), np.uint8)
    qA[np.arange(M), np.arange(M)] = 0x38
    sA = np.ones((M, K // 128), np.float32)
    g = inputs.rng(1650 + e_lo)
    codes = np.stack([g.permutation(np.arange(K) % 16) for _ in range(N)], axis=1).astype(np.uint8)
    span = e_hi - e_lo + 1
    sE = (e_lo + (np.arange(K // 32)[:, None] * N + np.arange(N)[None, :]) % span).astype(np.uint8)
    return qA, sA, pack4(codes), sE


def test_every_code_and_normal_scale_exact(bg):
    # exponents 2..252 keep every nonzero product a normal fp32 and bf16 number
    qA, sA, Bq, sE = onehot_case(2, 252)
    N = 16
    got = run(bg, qA, sA, Bq, sE, N)
    C64, _ = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    assert np.array_equal(got, oracle.round_bf16(C64))


def test_extreme_scales_and_nan(bg):
    # 0, 1: products below the fp32 normal range (the MFMA may flush them,
    # inside the tolerance's absolute term); 253, 254: overflow to infinity;
    # 255: NaN
    N = 16
    qA, sA, Bq, sE = onehot_case(0, 1)
    got = run(bg, qA, sA, Bq, sE, N)
    C64, S = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    check_parity(got, C64, S, qA.shape[1], "tiny scales")
    qA, sA, Bq, sE = onehot_case(253, 254)
    got = inputs.bf16_codes_to_f32(run(bg, qA, sA, Bq, sE, N))
    C64, _ = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    ref = inputs.bf16_codes_to_f32(oracle.round_bf16(C64))
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(got[np.isfinite(ref)], ref[np.isfinite(ref)])
    qA, sA, Bq, sE = onehot_case(120, 130, K=256)
    sE[3, 5] = 255
    got = inputs.bf16_codes_to_f32(run(bg, qA, sA, Bq, sE, N))
    C64, _ = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    # the NaN scale poisons its whole column: rows whose one-hot lies in
    # another block still multiply it by zero (0 * NaN = NaN), as in the oracle
    assert np.array_equal(np.isnan(got), np.isnan(C64))
    assert np.isnan(got[:, 5]).all() and not np.isnan(np.delete(got, 5, axis=1)).any()


@pytest.mark.parametrize("M,N,K", [(1, 14336, 4096), (8, 1024, 4096), (9, 1024, 4096), (37, 512, 1024),
                                   (130, 96, 384), (512, 2048, 512)])
def test_parity_random(bg, M, N, K):
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 1601 + M))
    Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, 1602 + N))
    got = run(bg, qA, sA, Bq, sE, N)
    C64, S = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    check_parity(got, C64, S, K, f"w4a8 M{M} N{N} K{K}")


def test_k_tail_ignores_pitch_padding(bg):
    # K = 384: a partial last stage at every geometry; NaN codes / scales in
    # A's and sA's row-pitch padding must not reach the result
    for M, N, K in ((3, 272, 384), (8, 144, 640), (70, 144, 640), (300, 2048, 384), (300, 8192, 384)):
        qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 1701 + M))
        Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, 1702 + N))
        Ap = np.full((M, K + 128), 0x7F, np.uint8)
        Ap[:, :K] = qA
        sAp = np.full((M, K // 128 + 3), np.nan, np.float32)
        sAp[:, :K // 128] = sA
        A = torch.from_numpy(Ap).cuda()[:, :K]
        sAd = torch.from_numpy(sAp).cuda()[:, :K // 128]
        got = run(bg, qA, sA, Bq, sE, N, A=A, sAd=sAd)
        C64, S = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
        check_parity(got, C64, S, K, f"w4a8 tail M{M} N{N} K{K}")


def test_invariance_c4_shape(bg):
    # the fp4 weight shape (K=4096, N=14336) with fp8 activations
    K, N = 4096, 14336
    qA, sA, Bq, sE, C64, S = full_size.w4a8()
    A, sAd = dev_u8(qA), dev_f32(sA)
    Bp = bg.pack_b_mxfp4(dev_u8(Bq), dev_u8(sE), N)
    ref = torch.cat([bg.gemm_w4a8_packed(A[i:i + 1], sAd[i:i + 1], Bp) for i in range(512)])
    for m in (1, 8, 16, 17, 64, 65, 129, 300, 512):
        ok = rows_equal(bg.gemm_w4a8_packed(A[:m], sAd[:m], Bp), ref[:m])
        assert bool(ok.all()), f"M={m}"
    for s in range(2):
        p = torch.as_tensor(inputs.permutation(512, 1803 + s), device="cuda")
        ok = rows_equal(bg.gemm_w4a8_packed(A.index_select(0, p), sAd.index_select(0, p), Bp),
                        ref.index_select(0, p))
        assert bool(ok.all()), f"shuffle {s}"
    # every row, computed alone (M = 1) and in the M = 512 batch
    check_parity(full_size.all_rows(host_codes(ref), C64), C64, S, K, "w4a8 C4 shape rows at M=1")
    full = host_codes(bg.gemm_w4a8_packed(A, sAd, Bp))
    check_parity(full_size.all_rows(full, C64), C64, S, K, "w4a8 C4 shape M=512 every row")
