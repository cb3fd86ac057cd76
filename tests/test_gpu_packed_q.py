"""GPU tests of the packed-weight fp8 and fp4 entry points (C ABI).

The packed layouts only reorder the weights (and, for fp4, their scales) into
MFMA operand order; each output element must come out bit-identical to the
unpacked entry point, at every launch geometry, and within the parity
tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests import full_size
from tests.gpu_util import check_parity, dev_bf16, dev_f32, dev_u8, host_codes, require_gpu, rows_equal

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


# ------------------------------------------------------------------ fp8


def fp8_case(M, N, K, seed):
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, seed))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, seed + 1))
    return qA, sA, qB, sB


# M values cover every launch geometry: 16 rows x 8 columns (N < 4096) or
# x 16 columns, then 64 x 16, 64 x 32 and 64 x 64 tiles once they still fill
# the compute units.
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (5, 300, 384), (3, 4112, 256), (16, 4096, 128),
                                   (8, 2048, 1152), (7, 144, 896), (9, 272, 1152),
                                   (17, 144, 1024), (40, 272, 512),
                                   (64, 2048, 896), (200, 2048, 1024), (512, 2048, 512),
                                   (129, 4112, 256)])
def test_fp8_packed_bitwise_equal_to_unpacked(bg, M, N, K):
    qA, sA, qB, sB = fp8_case(M, N, K, 700 + M)
    A, sAd, sBd = dev_u8(qA), dev_f32(sA), dev_f32(sB)
    ref = host_codes(bg.gemm_fp8_blockscaled(A, sAd, dev_u8(qB, pad16(N)), sBd))
    Bp = bg.pack_b_fp8(dev_u8(qB, pad16(N)))
    got = host_codes(bg.gemm_fp8_blockscaled_packed(A, sAd, Bp, sBd))
    assert np.array_equal(got, ref)
    if M * N * K <= 64 * 2048 * 1024:
        C64, S = oracle.gemm_fp8bs(qA, sA, qB, sB)
        check_parity(got, C64, S, K, f"fp8 packed M{M} N{N} K{K}")


def test_fp8_packed_empty_and_k0(bg):
    qB = np.zeros((0, 32), np.uint8)
    Bp = bg.pack_b_fp8(dev_u8(np.zeros((1, 32), np.uint8))[:0])
    A = torch.zeros((3, 0), dtype=torch.uint8, device="cuda")
    sA = torch.zeros((3, 0), dtype=torch.float32, device="cuda")
    sB = torch.zeros((0, 1), dtype=torch.float32, device="cuda")
    C = torch.full((3, 32), 7.0, dtype=torch.bfloat16, device="cuda")
    bg.gemm_fp8_blockscaled_packed(A, sA, Bp, sB, out=C)
    torch.cuda.synchronize()
    assert not bool(C.float().abs().sum()) and qB.size == 0


@pytest.fixture(scope="module")
def c3p(bg):
    # fp8 e4m3 K=7168, N=2048 (the same seeded workload as the unpacked tests)
    qA, sA, qB, sB, _, _ = full_size.c3()
    A, sAd, B, sBd = dev_u8(qA), dev_f32(sA), dev_u8(qB), dev_f32(sB)
    return qA, sA, qB, sB, A, sAd, bg.pack_b_fp8(B), sBd, B


def test_fp8_packed_c3_invariance_every_m(bg, c3p):
    qA, sA, qB, sB, A, sAd, Bp, sBd, B = c3p
    ref = torch.cat([bg.gemm_fp8_blockscaled_packed(A[i:i + 1], sAd[i:i + 1], Bp, sBd)
                     for i in range(512)])
    full = bg.gemm_fp8_blockscaled(A, sAd, B, sBd)
    assert bool(rows_equal(full, ref).all()), "packed rows differ from the unpacked path"
    for m in range(1, 513):
        ok = rows_equal(bg.gemm_fp8_blockscaled_packed(A[:m], sAd[:m], Bp, sBd), ref[:m])
        assert bool(ok.all()), f"M={m}: rows {torch.nonzero(~ok).flatten()[:8].tolist()} differ"
    for m, seed in ((37, 303), (129, 304), (512, 305)):
        p = torch.as_tensor(inputs.rng(seed).choice(512, size=m, replace=False), device="cuda")
        ok = rows_equal(bg.gemm_fp8_blockscaled_packed(A.index_select(0, p), sAd.index_select(0, p),
                                                       Bp, sBd), ref.index_select(0, p))
        assert bool(ok.all()), f"shuffle M={m}"
    # every row computed alone (M = 1), which all the comparisons above use
    *_, C64, S = full_size.c3()
    check_parity(full_size.all_rows(host_codes(ref), C64), C64, S, 7168, "C3 packed rows at M=1")


# ------------------------------------------------------------------ fp4


def fp4_run(bg, A, Bq, sB, N):
    Ad = dev_bf16(A)
    ref = host_codes(bg.gemm_fp4_w(Ad, dev_u8(Bq, pad16(Bq.shape[1])), dev_u8(sB, pad16(sB.shape[1])), N))
    Bp = bg.pack_b_fp4(dev_u8(Bq), dev_u8(sB), N)
    got = host_codes(bg.gemm_fp4_w_packed(Ad, Bp))
    return got, ref


@pytest.mark.parametrize("M,N,K", [(1, 32, 32), (3, 130, 288), (6, 4096, 384), (8, 272, 160),
                                   (17, 256, 512), (33, 96, 320),
                                   (65, 1024, 640), (130, 14336, 256), (512, 2048, 384)])
def test_fp4_packed_bitwise_equal_to_unpacked(bg, M, N, K):
    A = inputs.normal_bf16((M, K), 1.0, 800 + M)
    Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, 801 + N))
    got, ref = fp4_run(bg, A, Bq, sB, N)
    assert np.array_equal(got, ref)
    if M * N * K <= 64 * 2048 * 1024:
        C64, S = oracle.gemm_fp4w(A, Bq, sB, N)
        check_parity(got, C64, S, K, f"fp4 packed M{M} N{N} K{K}")


def test_fp4_packed_every_code_scale_pair_exact(bg):
    # all 16 e2m1 codes x all finite e4m3fn scale codes, one-hot A (exact products)
    scodes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    M, N, K = len(scodes), 16, len(scodes) * 32
    Bq = pack4(np.tile(np.arange(16, dtype=np.uint8), (K, 1)))
    sB = np.repeat(scodes[:, None], N, axis=1)
    A = np.zeros((M, K), np.float32)
    A[np.arange(M), 32 * np.arange(M)] = 1.0
    A = inputs.f32_to_bf16_codes(A)
    got, ref = fp4_run(bg, A, Bq, sB, N)
    C64, _ = oracle.gemm_fp4w(A, Bq, sB, N)
    assert np.array_equal(got, oracle.round_bf16(C64)) and np.array_equal(got, ref)


def test_fp4_packed_nan_scale_propagates(bg):
    M, N, K = 2, 32, 64
    Bq = np.full((K, N // 2), 0x22, np.uint8)
    sB = np.full((K // 32, N), 0x38, np.uint8)
    sB[1, 5] = 0x7F
    A = inputs.f32_to_bf16_codes(np.ones((M, K), np.float32))
    got, _ = fp4_run(bg, A, Bq, sB, N)
    got = inputs.bf16_codes_to_f32(got)
    assert np.isnan(got[:, 5]).all() and not np.isnan(np.delete(got, 5, axis=1)).any()


@pytest.fixture(scope="module")
def c4p(bg):
    # fp4 e2m1 weight-only K=4096, N=14336 (same seeded workload as the unpacked tests)
    A, Bq, sB, _, _ = full_size.c4()
    Bd, sBd = dev_u8(Bq), dev_u8(sB)
    return A, Bq, sB, dev_bf16(A), Bd, sBd, bg.pack_b_fp4(Bd, sBd, 14336)


def test_fp4_packed_c4_invariance(bg, c4p):
    A, Bq, sB, Ad, Bd, sBd, Bp = c4p
    N = 14336
    ref = torch.cat([bg.gemm_fp4_w_packed(Ad[i:i + 1], Bp) for i in range(512)])
    assert bool(rows_equal(bg.gemm_fp4_w(Ad, Bd, sBd, N), ref).all()), "packed differs from unpacked"
    for m in (1, 8, 17, 33, 64, 65, 129, 512, 3, 100, 257):
        ok = rows_equal(bg.gemm_fp4_w_packed(Ad[:m], Bp), ref[:m])
        assert bool(ok.all()), f"M={m}"
    for s in range(2):
        p = torch.as_tensor(inputs.permutation(512, 403 + s), device="cuda")
        ok = rows_equal(bg.gemm_fp4_w_packed(Ad.index_select(0, p), Bp), ref.index_select(0, p))
        assert bool(ok.all()), f"shuffle {s}"
    *_, C64, S = full_size.c4()
    check_parity(full_size.all_rows(host_codes(ref), C64), C64, S, 4096, "C4 packed rows at M=1")


# ------------------------------------------------------------------ K tails with poisoned pitch padding


def test_fp8_k_tail_ignores_pitch_padding(bg):
    """K = 384 leaves the last pipeline stage partly past K at every geometry.
    The row pitches of A and sA are padded with NaN codes / NaN scales, which
    must never reach the result (blocks past K contribute exact zeros)."""
    for M, N, K in ((5, 272, 384), (8, 144, 1152), (70, 144, 640), (300, 2048, 384)):
        qA, sA, qB, sB = fp8_case(M, N, K, 950 + M)
        Ap = np.full((M, K + 128), 0x7F, np.uint8)          # e4m3fn NaN past K
        Ap[:, :K] = qA
        sAp = np.full((M, K // 128 + 3), np.nan, np.float32)
        sAp[:, :K // 128] = sA
        A = torch.from_numpy(Ap).cuda()[:, :K]
        sAd = torch.from_numpy(sAp).cuda()[:, :K // 128]
        B, sBd = dev_u8(qB, pad16(N)), dev_f32(sB)
        C64, S = oracle.gemm_fp8bs(qA, sA, qB, sB)
        got = host_codes(bg.gemm_fp8_blockscaled(A, sAd, B, sBd))
        check_parity(got, C64, S, K, f"fp8 tail M{M} N{N} K{K}")
        got_p = host_codes(bg.gemm_fp8_blockscaled_packed(A, sAd, bg.pack_b_fp8(B), sBd))
        assert np.array_equal(got_p, got)


def test_fp4_k_tail_ignores_pitch_padding(bg):
    """K = 288 (not a multiple of either kernel's stage) with A's row pitch
    padded with bf16 NaN."""
    for M, N, K in ((3, 130, 288), (7, 130, 288), (40, 1024, 160), (513, 256, 96)):
        Ah = inputs.normal_bf16((M, K), 1.0, 960 + M)
        Ap = np.full((M, K + 64), 0x7FC0, np.uint16)
        Ap[:, :K] = Ah
        A = torch.from_numpy(Ap.view(np.int16)).view(torch.bfloat16).cuda()[:, :K]
        Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, 961 + N))
        Bd, sBd = dev_u8(Bq, pad16(N // 2)), dev_u8(sB, pad16(N))
        C64, S = oracle.gemm_fp4w(Ah, Bq, sB, N)
        got = host_codes(bg.gemm_fp4_w(A, Bd, sBd, N))
        check_parity(got, C64, S, K, f"fp4 tail M{M} N{N} K{K}")
        got_p = host_codes(bg.gemm_fp4_w_packed(A, bg.pack_b_fp4(Bd, sBd, N)))
        assert np.array_equal(got_p, got)


@pytest.mark.parametrize("M,N", [(19, 272), (3, 272), (6, 272), (130, 8192)])
def test_bf16_k_tail_ignores_pitch_padding(bg, M, N):
    # the same property for the three bf16 layouts (K = 200: a partial 32-step),
    # on small tiles and on the large-M tiles of each layout
    K = 200
    Ah = inputs.normal_bf16((M, K), 1.0, 971)
    Bh = inputs.normal_bf16((K, N), 0.02, 972)
    Ap = np.full((M, K + 56), 0x7FC0, np.uint16)
    Ap[:, :K] = Ah
    Btp = np.full((N, K + 56), 0x7FC0, np.uint16)
    Btp[:, :K] = Bh.T
    A = torch.from_numpy(Ap.view(np.int16)).view(torch.bfloat16).cuda()[:, :K]
    Bt = torch.from_numpy(Btp.view(np.int16)).view(torch.bfloat16).cuda()[:, :K]
    B = dev_bf16(Bh)
    C64, S = oracle.gemm_bf16(Ah, Bh)
    got = host_codes(bg.gemm_bf16(A, B))
    check_parity(got, C64, S, K, "bf16 tail")
    assert np.array_equal(host_codes(bg.gemm_bf16_bt(A, Bt)), got)
    assert np.array_equal(host_codes(bg.gemm_bf16_packed(A, bg.pack_b_bf16(B))), got)
