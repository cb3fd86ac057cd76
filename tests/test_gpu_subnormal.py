"""GPU pins of the rounding rule at the bottom of the range: round to nearest
even with subnormals kept, no flush to zero (the wmrh.cn V4 engineering blog,
section 3.1, on the GEMM's rounding), and the sign of zero.

Every input here is dyadic and chosen so that each partial sum, in any order,
is exactly representable in fp32 -- subnormals included -- so a kernel that
keeps subnormals returns exactly the oracle's direct fp64 -> bf16 RNE of the
exact sum, bit for bit.  A flush to zero anywhere (MFMA products or sums, the
scale FMA, the epilogue) changes some of these bits.

The sign of zero: a negative sum that underflows fp32 leaves the accumulator
at -0 until a +0 product is added, and the number of all-zero K steps after
the last real one follows the launch geometry (so M).  The library writes
every zero result as +0; the exact sum there lies below fp32's range
(|C64| < 2^-149), where the oracle's RNE gives -0.  Those rows are checked to
be +0 in every geometry and bitwise equal across M.
"""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests.gpu_util import dev_bf16, dev_f32, dev_u8, host_codes, require_gpu, rows_equal

pytestmark = pytest.mark.gpu

BF16_MIN_NORMAL = 2.0**-126


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def pad(n, q):
    return (n + q - 1) // q * q


def bf16(x):
    x = np.asarray(x, np.float64)
    codes = inputs.f32_to_bf16_codes(x.astype(np.float32))
    assert np.array_equal(inputs.bf16_codes_to_f32(codes).astype(np.float64), x), "not a bf16 value"
    return codes


def sparse_dyadic(shape, seed, e_lo, e_hi, nnz):
    """nnz nonzeros per row, values +-m * 2^e with m in 1..7, e in [e_lo, e_hi]."""
    g = inputs.rng(seed)
    R, Cn = shape
    x = np.zeros(shape)
    for r in range(R):
        cols = g.choice(Cn, size=min(nnz, Cn), replace=False)
        m = g.integers(1, 8, size=cols.size) * np.where(g.integers(0, 2, size=cols.size) == 1, -1, 1)
        x[r, cols] = np.ldexp(m.astype(np.float64), g.integers(e_lo, e_hi + 1, size=cols.size))
    return x


def dense_dyadic(shape, seed, e_lo, e_hi):
    g = inputs.rng(seed)
    m = g.integers(-7, 8, size=shape).astype(np.float64)
    return np.ldexp(m, g.integers(e_lo, e_hi + 1, size=shape))


def expected(C64):
    """The oracle's bf16 RNE of the exact sum; results whose exact value lies
    below fp32's subnormal range cannot reach the fp32 accumulator and are +0."""
    R = oracle.round_bf16(C64)
    R[np.abs(C64) < 2.0**-150] = 0
    return R


def assert_bits(got, want, what):
    bad = got != want
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs differ, first at {i}: "
                             f"got 0x{int(got[i]):04x}, want 0x{int(want[i]):04x}")


def subnormal_share(C64):
    nz = C64 != 0
    return float(np.mean((np.abs(C64) < BF16_MIN_NORMAL) & nz))


def bf16_all_layouts(bg, A, B, Ms):
    """Row-major, transposed and packed weights at each M: the row blocks of A."""
    M, K = A.shape
    N = B.shape[1]
    Ad = dev_bf16(A, pad(K, 8))
    Bd = dev_bf16(B, pad(N, 8))
    Bt = dev_bf16(np.ascontiguousarray(B.T), pad(K, 8))
    Bp = bg.pack_b_bf16(Bd)
    outs = {}
    for m in Ms:
        outs[("rowmajor", m)] = host_codes(bg.gemm_bf16(Ad[:m], Bd))
        outs[("transposed", m)] = host_codes(bg.gemm_bf16_bt(Ad[:m], Bt))
        outs[("packed", m)] = host_codes(bg.gemm_bf16_packed(Ad[:m], Bp))
    torch.cuda.synchronize()
    return outs


# Geometry switch points of the bf16 kernels at these widths (16-row one-wave,
# 32-row, 64-row streaming, 32x64, 64x64, 64x128 tiles).
MS_SMALL_N = (1, 4, 8, 16, 17, 33, 65, 129, 300)
MS_WIDE_N = (1, 8, 16, 17, 33, 64, 65, 129, 256)


@pytest.mark.parametrize("N,K", [(256, 512), (8192, 300)])
def test_bf16_subnormal_products_no_ftz(bg, N, K):
    """Normal bf16 inputs whose products are fp32 subnormals (2^-130 .. 2^-140):
    sums land on both sides of the bf16 normal boundary, and the bf16 RNE in
    the subnormal range rounds (spacing 2^-133 against products on 2^-140)."""
    M = max(MS_SMALL_N if N == 256 else MS_WIDE_N)
    A = sparse_dyadic((M, K), 31 + N, -75, -70, nnz=3)
    B = dense_dyadic((K, N), 32 + N, -65, -60)
    Ac, Bc = bf16(A), bf16(B)
    C64, _ = oracle.gemm_bf16(Ac, Bc)
    assert subnormal_share(C64) > 0.3, "the inputs must reach the subnormal range"
    want = expected(C64)
    for (layout, m), got in bf16_all_layouts(bg, Ac, Bc, MS_SMALL_N if N == 256 else MS_WIDE_N).items():
        assert_bits(got, want[:m], f"bf16 {layout} M={m} N={N} K={K}")


def test_bf16_subnormal_inputs(bg):
    """bf16 subnormal inputs (m * 2^-133 .. 2^-128) times small integers."""
    M, N, K = 17, 256, 512
    A = sparse_dyadic((M, K), 41, -133, -128, nnz=4)
    B = dense_dyadic((K, N), 42, 0, 1)
    Ac, Bc = bf16(A), bf16(B)
    assert np.mean(np.abs(A[A != 0]) < BF16_MIN_NORMAL) > 0.5
    C64, _ = oracle.gemm_bf16(Ac, Bc)
    want = expected(C64)
    for (layout, m), got in bf16_all_layouts(bg, Ac, Bc, (1, 8, 17)).items():
        assert_bits(got, want[:m], f"bf16 subnormal inputs, {layout} M={m}")


def small_e4m3(shape, seed):
    """e4m3fn codes of +-(1 + m/8) * 2^{-1..1}."""
    g = inputs.rng(seed)
    e = g.integers(6, 9, size=shape)
    return ((g.integers(0, 2, size=shape) << 7) | (e << 3) | g.integers(0, 8, size=shape)).astype(np.uint8)


def fp8_both(bg, qA, sA, qB, sB, Ms):
    N = qB.shape[1]
    A, sAd, sBd = dev_u8(qA), dev_f32(sA), dev_f32(sB)
    B = dev_u8(qB, pad(N, 16))
    Bp = bg.pack_b_fp8(B)
    outs = {}
    for m in Ms:
        outs[("rowmajor", m)] = host_codes(bg.gemm_fp8_blockscaled(A[:m], sAd[:m], B, sBd))
        outs[("packed", m)] = host_codes(bg.gemm_fp8_blockscaled_packed(A[:m], sAd[:m], Bp, sBd))
    torch.cuda.synchronize()
    return outs


def test_fp8_scale_fma_subnormal(bg):
    """The block scale product fl32(sA * sB) and the scaled block sums are fp32
    subnormals (sA * sB = 2^-140 .. 2^-136)."""
    M, N, K = 129, 2048, 512
    qA = small_e4m3((M, K), 51)
    keep = inputs.rng(52).random((M, K)) < 0.03      # sparse rows keep the sums small
    qA[~keep] = 0
    qB = small_e4m3((K, N), 53)
    sA = np.ldexp(1.0, inputs.rng(54).integers(-72, -69, size=(M, K // 128))).astype(np.float32)
    sB = np.ldexp(1.0, inputs.rng(55).integers(-68, -66, size=(K // 128, N // 128))).astype(np.float32)
    C64, _ = oracle.gemm_fp8bs(qA, sA, qB, sB)
    assert subnormal_share(C64) > 0.3
    want = expected(C64)
    for (layout, m), got in fp8_both(bg, qA, sA, qB, sB, (1, 8, 16, 17, 64, 129)).items():
        assert_bits(got, want[:m], f"fp8 {layout} M={m}")


def test_fp8_subnormal_codes(bg):
    """e4m3fn subnormal codes (exponent field 0: m * 2^-9) through the MFMA:
    B = identity (0x38 = 1.0), unit scales, so C = dec(qA) exactly."""
    M, K = 24, 256
    g = inputs.rng(56)
    qA = ((g.integers(0, 2, size=(M, K)) << 7) | g.integers(0, 8, size=(M, K))).astype(np.uint8)
    qB = np.zeros((K, K), np.uint8)
    qB[np.arange(K), np.arange(K)] = 0x38
    sA = np.ones((M, K // 128), np.float32)
    sB = np.ones((K // 128, K // 128), np.float32)
    C64, _ = oracle.gemm_fp8bs(qA, sA, qB, sB)
    want = expected(C64)
    for (layout, m), got in fp8_both(bg, qA, sA, qB, sB, (1, M)).items():
        assert_bits(got, want[:m], f"fp8 subnormal codes {layout} M={m}")


def pack_nibbles(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_fp4_subnormal_results(bg):
    """bf16 activations m * 2^-126 .. 2^-122 times e2m1 weights with e4m3fn
    block scales (subnormal and small normal scale codes): products between
    about 2^-137 and 2^-119."""
    M, N, K = 65, 512, 256
    A = sparse_dyadic((M, K), 61, -126, -122, nnz=4)
    g = inputs.rng(62)
    codes = g.integers(0, 16, size=(K, N)).astype(np.uint8)
    # scale codes: subnormal (exponent 0) and small normal (exponent 1..3)
    s_exp = g.integers(0, 4, size=(K // 32, N))
    sB = ((s_exp << 3) | g.integers(0, 8, size=(K // 32, N))).astype(np.uint8)
    sB[sB == 0] = 0x08
    Ac, Bq = bf16(A), pack_nibbles(codes)
    C64, _ = oracle.gemm_fp4w(Ac, Bq, sB, N)
    assert subnormal_share(C64) > 0.1
    want = expected(C64)
    Ad = dev_bf16(Ac)
    Bd, sBd = dev_u8(Bq), dev_u8(sB)
    Bp = bg.pack_b_fp4(Bd, sBd, N)
    for m in (1, 8, 17, 64, 65):
        got = host_codes(bg.gemm_fp4_w(Ad[:m], Bd, sBd, N))
        assert_bits(got, want[:m], f"fp4 row-major M={m}")
        got = host_codes(bg.gemm_fp4_w_packed(Ad[:m], Bp))
        assert_bits(got, want[:m], f"fp4 packed M={m}")


def test_w4a8_subnormal_results(bg):
    """e4m3fn activations, MXFP4 weights with E8M0 scale 2^-60, activation
    scales 2^-72 .. 2^-70: the MFMA's block sums are normal, the scale FMA
    makes them fp32 subnormals."""
    M, N, K = 65, 256, 512
    qA = small_e4m3((M, K), 71)
    qA[inputs.rng(72).random((M, K)) >= 0.03] = 0
    codes = inputs.rng(73).integers(0, 16, size=(K, N)).astype(np.uint8)
    sE = np.full((K // 32, N), 127 - 60, np.uint8)
    sA = np.ldexp(1.0, inputs.rng(74).integers(-72, -69, size=(M, K // 128))).astype(np.float32)
    Bq = pack_nibbles(codes)
    C64, _ = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    assert subnormal_share(C64) > 0.3
    want = expected(C64)
    A, sAd = dev_u8(qA), dev_f32(sA)
    Bp = bg.pack_b_mxfp4(dev_u8(Bq), dev_u8(sE), N)
    for m in (1, 8, 16, 17, 64, 65):
        got = host_codes(bg.gemm_w4a8_packed(A[:m], sAd[:m], Bp))
        assert_bits(got, want[:m], f"w4a8 M={m}")


# ------------------------------------------------------------------ sign of zero


def tiny_negative_rows(M, K, N, seed):
    """Rows whose every output is an exact sum below fp32's range: one nonzero
    per A row (2^-80) against B entries of +-2^-80 or 0, so each output is
    -2^-160, +2^-160 or an exact zero; plus ordinary rows mixed in."""
    g = inputs.rng(seed)
    A = np.zeros((M, K))
    A[np.arange(M), g.integers(0, K, size=M)] = 2.0**-80
    B = np.ldexp(g.integers(-1, 2, size=(K, N)).astype(np.float64), -80)
    ordinary = np.arange(M) % 5 == 4
    A[ordinary] = dense_dyadic((int(ordinary.sum()), K), seed + 1, -3, 0)
    return bf16(A), bf16(B), ordinary


@pytest.mark.parametrize("N,K,Ms", [(256, 512, MS_SMALL_N), (8192, 300, MS_WIDE_N)])
def test_negative_underflow_is_plus_zero_in_every_geometry(bg, N, K, Ms):
    M = max(Ms)
    A, B, ordinary = tiny_negative_rows(M, K, N, 81 + N)
    C64, _ = oracle.gemm_bf16(A, B)
    assert (C64[~ordinary] < 0).any(), "some sums must be negative"
    want = expected(C64)
    assert not (want[~ordinary] != 0).any()
    outs = bf16_all_layouts(bg, A, B, Ms)
    for (layout, m), got in outs.items():
        assert_bits(got, want[:m], f"bf16 {layout} M={m}")


def test_fp8_negative_underflow_is_plus_zero(bg):
    """fma(P, s, acc) with P * s negative below fp32's range leaves acc = -0;
    the fp8 geometries pad different numbers of zero blocks after it."""
    M, N, K = 300, 2048, 7168
    g = inputs.rng(91)
    qA = np.zeros((M, K), np.uint8)
    qA[np.arange(M), g.integers(0, K, size=M)] = 0x01          # 2^-9
    qB = np.where(g.random((K, N)) < 0.5, 0x81, 0x01).astype(np.uint8)   # +-2^-9
    sA = np.full((M, K // 128), 2.0**-70, np.float32)
    sB = np.full((K // 128, N // 128), 2.0**-70, np.float32)
    C64, _ = oracle.gemm_fp8bs(qA, sA, qB, sB)
    assert (C64 < 0).any() and (np.abs(C64) < 2.0**-150).all()
    want = expected(C64)
    for (layout, m), got in fp8_both(bg, qA, sA, qB, sB, (1, 8, 16, 17, 33, 65, 129, 300)).items():
        assert_bits(got, want[:m], f"fp8 {layout} M={m}")


def test_zero_rows_bitwise_across_m(bg):
    """The same rows computed alone and in batches of every size are bitwise
    equal when their results underflow (the invariance property itself)."""
    N, K = 8192, 300
    A, B, _ = tiny_negative_rows(256, K, N, 95)
    Ad, Bd = dev_bf16(A, pad(K, 8)), dev_bf16(B)
    Bp = bg.pack_b_bf16(Bd)
    alone = torch.cat([bg.gemm_bf16_packed(Ad[i:i + 1], Bp) for i in range(256)])
    for m in MS_WIDE_N:
        assert bool(rows_equal(bg.gemm_bf16_packed(Ad[:m], Bp), alone[:m]).all()), f"M={m}"
        assert bool(rows_equal(bg.gemm_bf16(Ad[:m], Bd), alone[:m]).all()), f"row-major M={m}"
