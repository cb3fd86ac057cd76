"""Pins for the fp64 oracle, independent of the oracle itself (CPU only).

Each test checks the oracle against something fixed outside it: the format
specifications (golden tables), torch's own format conversions, exact
rational arithmetic (fractions.Fraction) on small inputs, closed forms
(identity, permutation, all-ones, one-hot), and numpy's float64 matmul.
They are chosen so that a dropped term, a wrong sign, a wrong index or a
transposed operand in the oracle fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


# ------------------------------------------------------------------ decoders


def test_e4m3fn_spec_spots():
    for code, val in _golden_rows("e4m3fn_spot.txt"):
        assert _same(oracle.dec_e4m3fn(int(code, 16)), float(val)), code


def test_e4m3fn_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    for c in range(256):
        assert _same(oracle.dec_e4m3fn(c), ref[c]), hex(c)


def test_e2m1_spec_table():
    rows = list(_golden_rows("e2m1_values.txt"))
    assert len(rows) == 16
    for code, val in rows:
        assert _same(oracle.dec_e2m1(int(code)), float(val)), code


def test_bf16_decode_exhaustive_vs_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    lib = oracle._load()
    for c in range(0, 65536, 1):
        v = lib.ora_dec_bf16(c)
        r = ref[c]
        if not _same(v, float(r)):
            raise AssertionError(hex(c))


# ------------------------------------------------------------------ rounding


def test_bf16_rounding_fixture():
    for x, code, *_ in _golden_rows("bf16_rounding.txt"):
        assert oracle.rne_bf16(float.fromhex(x)) == int(code, 16), x


def test_bf16_round_trip_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    finite = np.isfinite(vals)
    back = oracle.round_bf16(vals[finite])
    assert np.array_equal(back, codes[finite])
    assert oracle.rne_bf16(float("inf")) == 0x7F80
    assert oracle.rne_bf16(float("-inf")) == 0xFF80
    assert (oracle.rne_bf16(float("nan")) & 0x7FC0) == 0x7FC0


def test_bf16_rounding_matches_torch_on_fp32_values():
    g = np.random.Generator(np.random.PCG64(7))
    bits = g.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_midpoints_tie_to_even():
    # every midpoint between adjacent positive finite bf16 codes
    lo = np.arange(0x0000, 0x7F7F, dtype=np.uint32)
    a = (lo << 16).view(np.float32).astype(np.float64)
    b = ((lo + 1) << 16).view(np.float32).astype(np.float64)
    mid = (a + b) / 2          # exact in fp64
    got = oracle.round_bf16(mid)
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, expect)
    # a hair above / below every midpoint
    up = oracle.round_bf16(np.nextafter(mid, np.inf))
    dn = oracle.round_bf16(np.nextafter(mid, -np.inf))
    assert np.array_equal(up, (lo + 1).astype(np.uint16))
    assert np.array_equal(dn, lo.astype(np.uint16))


# ------------------------------------------------------------------ helpers

def _dyadic_bf16(shape, seed, emin=-4, emax=4):
    """bf16 codes of values m * 2^e with small odd/even integers m: products and
    sums of these are exact in fp64, so fp64 results must equal Fraction sums."""
    g = np.random.Generator(np.random.PCG64(seed))
    m = g.integers(-15, 16, size=shape).astype(np.float64)
    e = g.integers(emin, emax + 1, size=shape)
    v = np.ldexp(m, e).astype(np.float32)
    return inputs.f32_to_bf16_codes(v)


def _frac_bf16(code):
    return Fraction(float(inputs.bf16_codes_to_f32(np.array([code], np.uint16))[0]))


def _brute(Avals, Bvals):
    M, K = len(Avals), len(Avals[0])
    N = len(Bvals[0])
    C = [[sum((Avals[i][k] * Bvals[k][j] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    S = [[sum((abs(Avals[i][k] * Bvals[k][j]) for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    return C, S


# ------------------------------------------------------------------ bf16 GEMM


def test_hand_worked_example():
    rows = list(_golden_rows("hand_gemm.txt"))
    A = np.array([[float(x) for x in r] for r in rows[0:2]], np.float32)
    B = np.array([[float(x) for x in r] for r in rows[2:5]], np.float32)
    C_exp = np.array([float(x) for x in rows[5][1:]]).reshape(2, 2)
    S_exp = np.array([float(x) for x in rows[6][1:]]).reshape(2, 2)
    C, S = oracle.gemm_bf16(inputs.f32_to_bf16_codes(A), inputs.f32_to_bf16_codes(B))
    assert np.array_equal(C, C_exp)
    assert np.array_equal(S, S_exp)


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 1), (3, 5, 7, 2), (6, 4, 8, 3), (4, 3, 40, 4), (2, 9, 33, 5)])
def test_bf16_exact_vs_fraction(M, N, K, seed):
    A = _dyadic_bf16((M, K), seed)
    B = _dyadic_bf16((K, N), seed + 100)
    C, S = oracle.gemm_bf16(A, B)
    Af = [[_frac_bf16(A[i, k]) for k in range(K)] for i in range(M)]
    Bf = [[_frac_bf16(B[k, j]) for j in range(N)] for k in range(K)]
    Ce, Se = _brute(Af, Bf)
    for i in range(M):
        for j in range(N):
            assert Fraction(C[i, j]) == Ce[i][j]
            assert Fraction(S[i, j]) == Se[i][j]


def test_bf16_random_normal_vs_fraction_within_fp64_bound():
    M, N, K = 3, 4, 64
    A = inputs.normal_bf16((M, K), 1.0, 11)
    B = inputs.normal_bf16((K, N), 1.0, 12)
    C, S = oracle.gemm_bf16(A, B)
    Af = [[_frac_bf16(A[i, k]) for k in range(K)] for i in range(M)]
    Bf = [[_frac_bf16(B[k, j]) for j in range(N)] for k in range(K)]
    Ce, Se = _brute(Af, Bf)
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(C[i, j]) - Ce[i][j]) <= Fraction(K * 2.0**-52) * Se[i][j]
            assert abs(Fraction(S[i, j]) - Se[i][j]) <= Fraction(K * 2.0**-52) * Se[i][j]


def test_bf16_sums_in_k_ascending_order():
    # a*b terms 2^60, 1, -2^60 in k order: fp64 sequential sum gives 0; other
    # orders (e.g. pairing the large terms first) would give 1.
    A = inputs.f32_to_bf16_codes(np.array([[2.0**30, 1.0, -(2.0**30)]], np.float32))
    B = inputs.f32_to_bf16_codes(np.array([[2.0**30], [1.0], [2.0**30]], np.float32))
    C, S = oracle.gemm_bf16(A, B)
    assert C[0, 0] == 0.0
    assert S[0, 0] == 2.0**61 + 1 or S[0, 0] == 2.0**61  # fp64 rounding of the |.| sum


def test_bf16_closed_forms():
    g = np.random.Generator(np.random.PCG64(21))
    M, K = 17, 96
    A = inputs.normal_bf16((M, K), 1.0, 22)
    Av = inputs.bf16_codes_to_f32(A).astype(np.float64)
    # identity
    I = inputs.f32_to_bf16_codes(np.eye(K, dtype=np.float32))
    C, _ = oracle.gemm_bf16(A, I)
    assert np.array_equal(C, Av)
    # permutation: column j of B = e_{p[j]}  ->  C[:, j] = A[:, p[j]]
    p = g.permutation(K)
    P = np.zeros((K, K), np.float32)
    P[p, np.arange(K)] = 1
    C, _ = oracle.gemm_bf16(A, inputs.f32_to_bf16_codes(P))
    assert np.array_equal(C, Av[:, p])
    # all-ones B with A in {-1,0,1}: row sums (exact integers)
    T = g.integers(-1, 2, size=(M, K)).astype(np.float32)
    N = 40
    C, S = oracle.gemm_bf16(inputs.f32_to_bf16_codes(T), inputs.f32_to_bf16_codes(np.ones((K, N), np.float32)))
    assert np.array_equal(C, np.repeat(T.sum(1, keepdims=True), N, 1).astype(np.float64))
    assert np.array_equal(S, np.repeat(np.abs(T).sum(1, keepdims=True), N, 1).astype(np.float64))
    # one-hot A rows pick rows of B
    Bc = inputs.normal_bf16((K, N), 1.0, 23)
    rows = g.integers(0, K, size=M)
    H = np.zeros((M, K), np.float32)
    H[np.arange(M), rows] = 1
    C, _ = oracle.gemm_bf16(inputs.f32_to_bf16_codes(H), Bc)
    assert np.array_equal(C, inputs.bf16_codes_to_f32(Bc).astype(np.float64)[rows])


def test_bf16_vs_numpy_matmul():
    A = inputs.normal_bf16((17, 512), 1.0, 101)
    B = inputs.normal_bf16((512, 256), 1.0, 102)
    C, S = oracle.gemm_bf16(A, B)
    ref = inputs.bf16_codes_to_f32(A).astype(np.float64) @ inputs.bf16_codes_to_f32(B).astype(np.float64)
    assert np.all(np.abs(C - ref) <= 1e-12 * S)
    refS = np.abs(inputs.bf16_codes_to_f32(A).astype(np.float64)) @ np.abs(inputs.bf16_codes_to_f32(B).astype(np.float64))
    assert np.all(np.abs(S - refS) <= 1e-12 * S)


def test_bf16_strided_operands():
    A = inputs.normal_bf16((5, 72), 1.0, 31)
    B = inputs.normal_bf16((64, 48), 1.0, 32)
    C1, S1 = oracle.gemm_bf16(np.ascontiguousarray(A[:, :64]), np.ascontiguousarray(B[:, :40]))
    C2, S2 = oracle.gemm_bf16(A[:, :64], B[:, :40])
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2)


def test_bf16_empty_k_gives_zero():
    A = np.zeros((3, 0), np.uint16)
    B = np.zeros((0, 5), np.uint16)
    C, S = oracle.gemm_bf16(A, B)
    assert np.array_equal(C, np.zeros((3, 5))) and np.array_equal(S, np.zeros((3, 5)))


# ------------------------------------------------------------------ fp8 block-scaled


def _e4m3_f64(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_vs_dequantised_numpy():
    M, K, N = 9, 384, 300                        # ragged last column block
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 41))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, 42))
    C, S = oracle.gemm_fp8bs(qA, sA, qB, sB)
    Ad = _e4m3_f64(qA) * np.repeat(sA.astype(np.float64), 128, axis=1)
    Bd = _e4m3_f64(qB) * np.repeat(np.repeat(sB.astype(np.float64), 128, axis=0), 128, axis=1)[:, :N]
    ref = Ad @ Bd
    assert np.all(np.abs(C - ref) <= 1e-12 * S)
    assert np.allclose(S, np.abs(Ad) @ np.abs(Bd), rtol=1e-12, atol=0)


def test_fp8_block_indexing_exact():
    # power-of-two scales that differ per block make every index mistake visible,
    # and keep every product and sum exact in fp64
    M, K, N = 2, 256, 260
    g = np.random.Generator(np.random.PCG64(43))
    qA = g.integers(0, 0x60, size=(M, K)).astype(np.uint8) | (g.integers(0, 2, size=(M, K)).astype(np.uint8) << 7)
    qB = g.integers(0, 0x60, size=(K, N)).astype(np.uint8) | (g.integers(0, 2, size=(K, N)).astype(np.uint8) << 7)
    sA = np.ldexp(1.0, g.integers(-3, 4, size=(M, K // 128))).astype(np.float32)
    sB = np.ldexp(1.0, g.integers(-3, 4, size=(K // 128, 3))).astype(np.float32)
    C, S = oracle.gemm_fp8bs(qA, sA, qB, sB)
    for i in range(M):
        for j in (0, 1, 127, 128, 200, 255, 256, 259):
            exp = Fraction(0)
            for k in range(K):
                a = Fraction(float(_e4m3_f64(qA[i:i + 1, k:k + 1])[0, 0])) * Fraction(float(sA[i, k // 128]))
                b = Fraction(float(_e4m3_f64(qB[k:k + 1, j:j + 1])[0, 0])) * Fraction(float(sB[k // 128, j // 128]))
                exp += a * b
            assert Fraction(C[i, j]) == exp, (i, j)


# ------------------------------------------------------------------ fp4 weight-only

E2M1 = {int(c): float(v) for c, v in _golden_rows("e2m1_values.txt")}


def test_fp4_vs_dequantised_numpy():
    M, K, N = 5, 128, 70
    A = inputs.normal_bf16((M, K), 1.0, 51)
    Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, 52))
    C, S = oracle.gemm_fp4w(A, Bq, sB, N)
    codes = inputs.unpack_fp4(Bq)
    vals = np.vectorize(E2M1.get)(codes).astype(np.float64)
    Bd = vals * np.repeat(_e4m3_f64(sB), 32, axis=0)
    Ad = inputs.bf16_codes_to_f32(A).astype(np.float64)
    assert np.all(np.abs(C - Ad @ Bd) <= 1e-12 * S)


def test_fp4_nibble_order_and_scale_index():
    K, N = 64, 6
    Bq = np.zeros((K, N // 2), np.uint8)
    Bq[40, 1] = 0x72          # column 2 <- code 2 (1.0), column 3 <- code 7 (6.0)
    sB = np.full((K // 32, N), 0x38, np.uint8)   # all scales 1.0
    sB[1, 3] = 0x30           # scale 0.5 for column 3, k-block 1 (k = 32..63)
    A = np.zeros((1, K), np.float32)
    A[0, 40] = 2.0
    C, _ = oracle.gemm_fp4w(inputs.f32_to_bf16_codes(A), Bq, sB, N)
    assert C.tolist() == [[0.0, 0.0, 2.0, 6.0, 0.0, 0.0]]


def test_fp4_exact_vs_fraction():
    M, K, N = 2, 64, 8
    g = np.random.Generator(np.random.PCG64(53))
    Bq = g.integers(0, 256, size=(K, N // 2)).astype(np.uint8)
    sB = g.integers(0, 0x7F, size=(K // 32, N)).astype(np.uint8)
    A = _dyadic_bf16((M, K), 54)
    C, S = oracle.gemm_fp4w(A, Bq, sB, N)
    codes = inputs.unpack_fp4(Bq)
    for i in range(M):
        for j in range(N):
            exp = Fraction(0)
            for k in range(K):
                b = Fraction(E2M1[int(codes[k, j])]) * Fraction(float(_e4m3_f64(sB[k // 32:k // 32 + 1, j:j + 1])[0, 0]))
                exp += _frac_bf16(A[i, k]) * b
            assert abs(Fraction(C[i, j]) - exp) <= Fraction(K * 2.0**-52) * Fraction(S[i, j]), (i, j)


def test_grouped_exact_vs_fraction():
    # grouped GEMM = one GEMM per group of rows, including an empty group
    from fractions import Fraction
    g = np.random.default_rng(11)
    K, N = 6, 3
    A = inputs.f32_to_bf16_codes(g.integers(-4, 5, size=(7, K)).astype(np.float32) / 4)
    Bs = [inputs.f32_to_bf16_codes(g.integers(-4, 5, size=(K, N)).astype(np.float32) / 8)
          for _ in range(3)]
    offsets = [0, 2, 2, 7]
    C, S = oracle.gemm_bf16_grouped(A, offsets, Bs)
    Af = inputs.bf16_codes_to_f32(A)
    for gi, B in enumerate(Bs):
        Bf = inputs.bf16_codes_to_f32(B)
        for m in range(offsets[gi], offsets[gi + 1]):
            for n in range(N):
                exact = sum(Fraction(float(Af[m, k])) * Fraction(float(Bf[k, n])) for k in range(K))
                assert C[m, n] == float(exact)
                assert S[m, n] == float(sum(abs(Fraction(float(Af[m, k])) * Fraction(float(Bf[k, n])))
                                            for k in range(K)))
    with pytest.raises(ValueError):
        oracle.gemm_bf16_grouped(A, [0, 3, 2, 7], Bs)


def test_grouped_fp8_exact_vs_fraction():
    """The grouped fp8 block-scaled GEMM is one block-scaled GEMM per group of
    rows (including an empty group), each value sum_k (e4m3(qa) sA)(e4m3(qb) sB)
    over the 128-long blocks; checked against exact rational arithmetic with
    the e4m3fn values written out from the format definition."""
    from fractions import Fraction

    def e4m3(c):
        s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
        v = Fraction(m, 8) * Fraction(1, 2**6) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2)**(e - 7)
        return -v if s else v

    g = np.random.default_rng(31)
    M, N, K, E = 7, 132, 256, 3                       # N: a ragged second 128-column block
    qA = g.integers(0, 256, size=(M, K)).astype(np.uint8)
    qA[(qA & 0x7F) == 0x7F] = 0x38                    # no NaN codes
    sA = np.ldexp(1.0, g.integers(-4, 4, size=(M, K // 128))).astype(np.float32) * \
        np.float32(1.5)
    qBs, sBs = [], []
    for _ in range(E):
        qB = g.integers(0, 256, size=(K, N)).astype(np.uint8)
        qB[(qB & 0x7F) == 0x7F] = 0x30
        qBs.append(qB)
        sBs.append(np.ldexp(1.0, g.integers(-4, 4, size=(K // 128, 2))).astype(np.float32))
    offsets = [0, 3, 3, 7]                            # group 1 is empty
    C, S = oracle.gemm_fp8bs_grouped(qA, sA, offsets, qBs, sBs)
    for e in range(E):
        for m in range(offsets[e], offsets[e + 1]):
            for n in (0, 5, 127, 128, 131):
                terms = [e4m3(int(qA[m, k])) * Fraction(float(sA[m, k // 128])) *
                         e4m3(int(qBs[e][k, n])) * Fraction(float(sBs[e][k // 128, n // 128]))
                         for k in range(K)]
                exact = sum(terms)
                assert abs(C[m, n] - float(exact)) <= 2.0**-52 * K * float(sum(abs(t) for t in terms))
                assert abs(S[m, n] - float(sum(abs(t) for t in terms))) <= \
                    2.0**-52 * K * float(sum(abs(t) for t in terms))
    # each group's rows are exactly its expert's plain GEMM
    C2, _ = oracle.gemm_fp8bs(np.ascontiguousarray(qA[3:]), np.ascontiguousarray(sA[3:]), qBs[2], sBs[2])
    assert np.array_equal(C[3:], C2)
    with pytest.raises(ValueError):
        oracle.gemm_fp8bs_grouped(qA, sA, [0, 4, 3, 7], qBs, sBs)


# ------------------------------------------------------------------ W4A8 (fp8 x OCP MXFP4)


def test_e8m0_exhaustive_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.dec_e8m0(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_w4a8_exact_vs_fraction():
    g = np.random.default_rng(21)
    M, N, K = 3, 6, 128
    qA = g.integers(0, 256, size=(M, K)).astype(np.uint8)
    qA[(qA & 0x7F) == 0x7F] = 0x38                      # no NaN codes
    sA = np.ldexp(1.0, g.integers(-3, 4, size=(M, 1))).astype(np.float32)
    codes = g.integers(0, 16, size=(K, N)).astype(np.uint8)
    Bq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sE = g.integers(120, 135, size=(K // 32, N)).astype(np.uint8)
    C, S = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    e4 = torch.from_numpy(qA).view(torch.float8_e4m3fn).double().numpy()
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            total = Fraction(0)
            for k in range(K):
                a = Fraction(float(e4[m, k])) * Fraction(float(sA[m, 0]))
                b = Fraction(E2M1[int(codes[k, n])]) * Fraction(2) ** (int(sE[k // 32, n]) - 127)
                exact += a * b
                total += abs(a * b)
            assert C[m, n] == float(exact) and S[m, n] == float(total)


def test_w4a8_vs_dequantised_numpy():
    M, N, K = 5, 34, 256
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 31))
    Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, 32))
    C, S = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    a = torch.from_numpy(qA).view(torch.float8_e4m3fn).double().numpy() * np.repeat(sA, 128, axis=1)
    codes = inputs.unpack_fp4(Bq)
    e2m1 = np.array([E2M1[c] for c in range(16)])
    b = e2m1[codes] * np.repeat(torch.from_numpy(sE).view(torch.float8_e8m0fnu).double().numpy(), 32, axis=0)
    ref = a @ b
    assert np.all(np.abs(C - ref) <= 1e-12 * (np.abs(a) @ np.abs(b)) + 1e-300)
    assert np.allclose(S, np.abs(a) @ np.abs(b), rtol=1e-12, atol=0)


def test_grouped_w4a8_exact_vs_fraction():
    """The grouped W4A8 GEMM is one W4A8 GEMM per group of rows (including an
    empty group), each value sum_k (e4m3(qa) sA)(e2m1(c) 2^(sE - 127)) with
    the 1x128 activation scales and the per-32 E8M0 weight scales; checked
    against exact rational arithmetic on sampled elements."""
    g = np.random.default_rng(41)
    M, N, K, E = 6, 132, 256, 3                       # N: a ragged second 128-column block
    qA = g.integers(0, 256, size=(M, K)).astype(np.uint8)
    qA[(qA & 0x7F) == 0x7F] = 0x38                    # no NaN codes
    sA = np.ldexp(1.0, g.integers(-3, 4, size=(M, K // 128))).astype(np.float32) * np.float32(1.25)
    codes, Bqs, sEs = [], [], []
    for _ in range(E):
        c = g.integers(0, 16, size=(K, N)).astype(np.uint8)
        codes.append(c)
        Bqs.append((c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8))
        sEs.append(g.integers(118, 137, size=(K // 32, N)).astype(np.uint8))
    offsets = [0, 2, 2, 6]                            # group 1 is empty
    C, S = oracle.gemm_w4a8_grouped(qA, sA, offsets, Bqs, sEs, N)
    e4 = torch.from_numpy(qA).view(torch.float8_e4m3fn).double().numpy()
    for e in range(E):
        for m in range(offsets[e], offsets[e + 1]):
            for n in (0, 7, 127, 128, 131):
                terms = [Fraction(float(e4[m, k])) * Fraction(float(sA[m, k // 128])) *
                         Fraction(E2M1[int(codes[e][k, n])]) * Fraction(2) ** (int(sEs[e][k // 32, n]) - 127)
                         for k in range(K)]
                exact = sum(terms)
                total = sum(abs(t) for t in terms)
                assert abs(C[m, n] - float(exact)) <= 2.0**-52 * K * float(total)
                assert abs(S[m, n] - float(total)) <= 2.0**-52 * K * float(total)
    # each group's rows are exactly its expert's plain W4A8 GEMM
    C2, _ = oracle.gemm_w4a8(np.ascontiguousarray(qA[2:]), np.ascontiguousarray(sA[2:]), Bqs[2], sEs[2], N)
    assert np.array_equal(C[2:], C2)
    with pytest.raises(ValueError):
        oracle.gemm_w4a8_grouped(qA, sA, [0, 4, 3, 6], Bqs, sEs, N)


def test_w4a8_scale_block_indexing():
    # one weight block carries a huge scale: it must show up exactly in
    # columns n and rows k of that block only
    M, N, K = 2, 4, 256
    qA = np.full((M, K), 0x38, np.uint8)                  # all 1.0
    sA = np.ones((M, K // 128), np.float32)
    Bq = np.full((K, N // 2), 0x22, np.uint8)             # every weight code 2 (= 1.0)
    sE = np.full((K // 32, N), 127, np.uint8)
    sE[5, 3] = 137                                        # block k in [160, 192), column 3: x 2^10
    C, _ = oracle.gemm_w4a8(qA, sA, Bq, sE, N)
    assert np.array_equal(C[:, :3], np.full((M, 3), 256.0))
    assert np.array_equal(C[:, 3], np.full(M, 224.0 + 32 * 1024.0))


def test_thread_count_does_not_change_results():
    # the host thread count is a timing knob only: each element is summed by
    # one thread in ascending k whatever the count
    A = inputs.normal_bf16((9, 300), 1.0, 71)
    B = inputs.normal_bf16((300, 40), 1.0, 72)
    n = oracle.num_threads()
    try:
        C_all, S_all = oracle.gemm_bf16(A, B)
        oracle.set_num_threads(1)
        assert oracle.num_threads() == 1
        C_one, S_one = oracle.gemm_bf16(A, B)
    finally:
        oracle.set_num_threads(n)
    assert np.array_equal(C_all, C_one) and np.array_equal(S_all, S_one)
