"""GPU tests of the unstaged small-M kernels of the packed fp8, W4A8 and fp4
GEMMs over several rounds of K blocks.

Those kernels take the 128-K blocks in rounds of 56 (8 waves x 7 blocks):
each round's operands go straight to registers, the block products to LDS,
and four waves fold them in K order, with the next round's loads issued
during the fold.  K past 7168 makes several rounds, the last one partial.
Every row must match the oracle within the tolerance, and be bit-identical
to the same row from a batch large enough to select a staged geometry (and,
for fp8, to the row-major entry point, which never runs unstaged)."""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests.gpu_util import check_parity, dev_bf16, dev_f32, dev_u8, host_codes, require_gpu

pytestmark = pytest.mark.gpu

UNSTAGED_FP8 = {8, 9, 10}    # packed fp8 table: unstaged 8 (half), 16 and 32 columns
UNSTAGED_W4A8 = {7, 8, 9}    # packed W4A8 table: unstaged 16, 8 (half) and 32 columns
UNSTAGED_FP4 = {5}           # packed fp4 table: unstaged 16 columns (narrow weights)


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def pad16(n):
    return (n + 15) // 16 * 16


# (M, N, K): 57 blocks (one round and one block), 113 (two and one), 168
# (exactly three); N below and past 256 column blocks (half blocks, and the
# 32-column tiles whose rounds hold 32 blocks: K = 4096 one round, 7296 two,
# 21504 six); the big batch of 300 rows runs the staged tiles
FP8_CASES = [(1, 272, 7296), (8, 2048, 14464), (5, 4112, 21504), (3, 1000, 7296),
             (16, 4112, 4096), (2, 8192, 7296)]


@pytest.mark.parametrize("M,N,K", FP8_CASES)
def test_fp8_rounds(bg, M, N, K):
    big = 300
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((big, K), 1.0, 5100 + K + M))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, 5200 + N))
    A, sAd, sBd = dev_u8(qA), dev_f32(sA), dev_f32(sB)
    Bd = dev_u8(qB, pad16(N))
    Bp = bg.pack_b_fp8(Bd)
    assert bg.geometry("fp8_packed", M, N, K)["id"] in UNSTAGED_FP8
    assert bg.geometry("fp8_packed", big, N, K)["id"] not in UNSTAGED_FP8
    got = host_codes(bg.gemm_fp8_blockscaled_packed(A[:M], sAd[:M], Bp, sBd))
    C64, S = oracle.gemm_fp8bs(qA[:M], sA[:M], qB, sB)
    check_parity(got, C64, S, K, f"fp8 packed unstaged M{M} N{N} K{K}")
    staged = host_codes(bg.gemm_fp8_blockscaled_packed(A, sAd, Bp, sBd))
    assert np.array_equal(got, staged[:M])
    rowmajor = host_codes(bg.gemm_fp8_blockscaled(A[:M], sAd[:M], Bd, sBd))
    assert np.array_equal(got, rowmajor)


# the unstaged kernel on half blocks, whole blocks (two 16-row slots among
# them) and 32-column tiles (32 K blocks a round; a few rows over wide
# weights, and two slots)
W4A8_CASES = [(1, 1024, 7296), (16, 2048, 14464), (32, 2048, 7296), (7, 4096, 21504),
              (4, 14336, 7296), (24, 4096, 7296)]


@pytest.mark.parametrize("M,N,K", W4A8_CASES)
def test_w4a8_rounds(bg, M, N, K):
    big = 300
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((big, K), 1.0, 5300 + K + M))
    Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, 5400 + N))
    A, sAd = dev_u8(qA), dev_f32(sA)
    Bp = bg.pack_b_mxfp4(dev_u8(Bq, pad16(Bq.shape[1])), dev_u8(sE, pad16(sE.shape[1])), N)
    assert bg.geometry("w4a8_packed", M, N, K)["id"] in UNSTAGED_W4A8
    assert bg.geometry("w4a8_packed", big, N, K)["id"] not in UNSTAGED_W4A8
    got = host_codes(bg.gemm_w4a8_packed(A[:M], sAd[:M], Bp))
    C64, S = oracle.gemm_w4a8(qA[:M], sA[:M], Bq, sE, N)
    check_parity(got, C64, S, K, f"W4A8 unstaged M{M} N{N} K{K}")
    staged = host_codes(bg.gemm_w4a8_packed(A, sAd, Bp))
    assert np.array_equal(got, staged[:M])


def test_grouped_rounds(bg):
    # one token per call through the grouped fp8 and W4A8 entry points at
    # K = 14464 (three rounds): the same bits as the ungrouped call with its
    # expert's weights
    E, N, K = 3, 1024, 14464
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((1, K), 1.0, 5501))
    A, sAd = dev_u8(qA), dev_f32(sA)
    off = torch.as_tensor(np.array([0, 0, 1, 1], np.int32), device="cuda")   # the token -> expert 1
    qBs = [inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, 5510 + e)) for e in range(E)]
    Bd = [dev_u8(q, pad16(N)) for q, _ in qBs]
    sB = dev_f32(np.concatenate([s for _, s in qBs], axis=0))       # [E*K/128, ceil(N/128)]
    assert bg.geometry("fp8_grouped_packed", 1, N, K, groups=E)["id"] in UNSTAGED_FP8
    g8 = host_codes(bg.gemm_fp8_blockscaled_grouped_packed(A, sAd, off, bg.pack_b_fp8_grouped(Bd), sB))
    assert np.array_equal(g8, host_codes(bg.gemm_fp8_blockscaled(A, sAd, Bd[1], dev_f32(qBs[1][1]))))
    mx = [inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, 5520 + e)) for e in range(E)]
    dq = [dev_u8(q, pad16(q.shape[1])) for q, _ in mx]
    ds = [dev_u8(s, pad16(s.shape[1])) for _, s in mx]
    assert bg.geometry("w4a8_grouped_packed", 1, N, K, groups=E)["id"] in UNSTAGED_W4A8
    g4 = host_codes(bg.gemm_w4a8_grouped_packed(A, sAd, off, bg.pack_b_mxfp4_grouped(dq, ds, N)))
    assert np.array_equal(g4, host_codes(bg.gemm_w4a8_packed(A, sAd, bg.pack_b_mxfp4(dq[1], ds[1], N))))


# fp4 takes its 32-K steps in rounds of 16 128-K groups with two rounds in
# flight: K = 7168 is four rounds, 14336 seven (an odd count), 4096 two; 96 is
# one group of three steps
FP4_CASES = [(1, 2048, 7168), (16, 1000, 4096), (5, 272, 14336), (3, 64, 96)]


@pytest.mark.parametrize("M,N,K", FP4_CASES)
def test_fp4_rounds(bg, M, N, K):
    big = 300
    A = inputs.normal_bf16((big, K), 1.0, 5600 + K + M)
    Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, 5700 + N))
    Ad = dev_bf16(A)
    Bd, sBd = dev_u8(Bq, pad16(Bq.shape[1])), dev_u8(sB, pad16(sB.shape[1]))
    Bp = bg.pack_b_fp4(dev_u8(Bq), dev_u8(sB), N)
    assert bg.geometry("fp4_packed", M, N, K)["id"] in UNSTAGED_FP4
    got = host_codes(bg.gemm_fp4_w_packed(Ad[:M], Bp))
    C64, S = oracle.gemm_fp4w(np.ascontiguousarray(A[:M]), Bq, sB, N)
    check_parity(got, C64, S, K, f"fp4 packed unstaged M{M} N{N} K{K}")
    # the same rows in a 300-row batch (another geometry, unstaged with more
    # row slots for the narrowest weights), and through the row-major entry
    # point, whose kernel is always staged
    batch = host_codes(bg.gemm_fp4_w_packed(Ad, Bp))
    assert np.array_equal(got, batch[:M])
    rowmajor = host_codes(bg.gemm_fp4_w(Ad[:M], Bd, sBd, N))
    assert np.array_equal(got, rowmajor)
