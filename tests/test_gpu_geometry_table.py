"""Every entry of every launch-geometry table runs the same arithmetic.

For each plain (ungrouped) entry point the geometry query is searched over a
grid of (M, N) -- and for the packed fp8 kernel two K, one of them past a
single round of its unstaged entries -- for the smallest call that selects
each table entry; that call is run with a K whose last pipeline stage lies
partly past K, and three of its rows are checked (1) against the fp64 oracle
within the tolerance and (2) bit for bit against the same rows computed alone
(M = 1, which selects another entry).  The grouped entry points have their
own every-geometry tests."""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests.gpu_util import check_parity, dev_bf16, dev_f32, dev_u8, host_codes, require_gpu

pytestmark = pytest.mark.gpu

M_GRID = list(range(1, 65)) + list(range(65, 601, 7)) + [128, 129, 192, 193, 256, 257, 512]
N_GRID = [16, 64, 144, 272, 1024, 2048, 3072, 4096, 4112, 8192, 14336, 16400]


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def pad16(n):
    return (n + 15) // 16 * 16


def cases(bg, entry, Ks):
    """{geometry id: (M, N, K)} -- the smallest M*N*K on the grid that selects it."""
    found = {}
    for K in Ks:
        for N in N_GRID:
            for M in M_GRID:
                gid = bg.geometry(entry, M, N, K)["id"]
                if gid not in found or M * N * K < np.prod(found[gid]):
                    found[gid] = (M, N, K)
    return found


def sample_rows(M):
    return sorted({0, M // 2, M - 1})


def check(bg, entry, gid, M, N, K, batch, alone, ref_rows):
    """batch: [M, N] codes; alone(r): row r computed at M = 1; ref_rows(rows) -> (C64, S)."""
    assert bg.geometry(entry, M, N, K)["id"] == gid
    rows = sample_rows(M)
    C64, S = ref_rows(rows)
    check_parity(batch[rows], C64, S, K, f"{entry} geometry {gid} M{M} N{N} K{K}")
    for i, r in enumerate(rows):
        assert np.array_equal(batch[r], alone(r)), f"{entry} geometry {gid} M{M} N{N}: row {r}"


@pytest.mark.parametrize("entry", ["bf16", "bf16_bt", "bf16_packed"])
def test_bf16_tables(bg, entry):
    for gid, (M, N, K) in sorted(cases(bg, entry, [360]).items()):
        A = inputs.normal_bf16((M, K), 1.0, 9100 + gid)
        B = inputs.normal_bf16((K, N), 0.02, 9200 + gid)
        Ad = dev_bf16(A)
        if entry == "bf16":
            Bd = dev_bf16(B)
            f = lambda X: bg.gemm_bf16(X, Bd)
        elif entry == "bf16_bt":
            Btd = dev_bf16(np.ascontiguousarray(B.T))
            f = lambda X: bg.gemm_bf16_bt(X, Btd)
        else:
            Bp = bg.pack_b_bf16(dev_bf16(B))
            f = lambda X: bg.gemm_bf16_packed(X, Bp)
        batch = host_codes(f(Ad))
        check(bg, entry, gid, M, N, K, batch, lambda r: host_codes(f(Ad[r:r + 1]))[0],
              lambda rows: oracle.gemm_bf16(np.ascontiguousarray(A[rows]), B))


# 384: three K blocks; 7296: 57, one more than a round of the packed kernel's
# unstaged entries, which sends 9..16-row calls to its staged half blocks
FP8_KS = {"fp8": [384], "fp8_packed": [384, 7296]}


@pytest.mark.parametrize("entry", ["fp8", "fp8_packed"])
def test_fp8_tables(bg, entry):
    for gid, (M, N, K) in sorted(cases(bg, entry, FP8_KS[entry]).items()):
        qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 9300 + gid))
        qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, 9400 + gid))
        Ad, sAd, sBd = dev_u8(qA), dev_f32(sA), dev_f32(sB)
        Bd = dev_u8(qB, pad16(N))
        if entry == "fp8":
            f = lambda X, s: bg.gemm_fp8_blockscaled(X, s, Bd, sBd)
        else:
            Bp = bg.pack_b_fp8(Bd)
            f = lambda X, s: bg.gemm_fp8_blockscaled_packed(X, s, Bp, sBd)
        batch = host_codes(f(Ad, sAd))
        check(bg, entry, gid, M, N, K, batch, lambda r: host_codes(f(Ad[r:r + 1], sAd[r:r + 1]))[0],
              lambda rows: oracle.gemm_fp8bs(np.ascontiguousarray(qA[rows]), np.ascontiguousarray(sA[rows]),
                                             qB, sB))


@pytest.mark.parametrize("entry", ["fp4", "fp4_packed"])
def test_fp4_tables(bg, entry):
    for gid, (M, N, K) in sorted(cases(bg, entry, [288]).items()):
        A = inputs.normal_bf16((M, K), 1.0, 9500 + gid)
        Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, 9600 + gid))
        Ad = dev_bf16(A)
        if entry == "fp4":
            Bd, sBd = dev_u8(Bq, pad16(Bq.shape[1])), dev_u8(sB, pad16(sB.shape[1]))
            f = lambda X: bg.gemm_fp4_w(X, Bd, sBd, N)
        else:
            Bp = bg.pack_b_fp4(dev_u8(Bq), dev_u8(sB), N)
            f = lambda X: bg.gemm_fp4_w_packed(X, Bp)
        batch = host_codes(f(Ad))
        check(bg, entry, gid, M, N, K, batch, lambda r: host_codes(f(Ad[r:r + 1]))[0],
              lambda rows: oracle.gemm_fp4w(np.ascontiguousarray(A[rows]), Bq, sB, N))


def test_w4a8_table(bg):
    entry = "w4a8_packed"
    for gid, (M, N, K) in sorted(cases(bg, entry, [384]).items()):
        qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 9700 + gid))
        Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, 9800 + gid))
        Ad, sAd = dev_u8(qA), dev_f32(sA)
        Bp = bg.pack_b_mxfp4(dev_u8(Bq, pad16(Bq.shape[1])), dev_u8(sE, pad16(sE.shape[1])), N)
        f = lambda X, s: bg.gemm_w4a8_packed(X, s, Bp)
        batch = host_codes(f(Ad, sAd))
        check(bg, entry, gid, M, N, K, batch, lambda r: host_codes(f(Ad[r:r + 1], sAd[r:r + 1]))[0],
              lambda rows: oracle.gemm_w4a8(np.ascontiguousarray(qA[rows]), np.ascontiguousarray(sA[rows]),
                                            Bq, sE, N))


def test_tables_fully_reached(bg):
    # the search reaches every plain-call table entry (entry 8 of the packed
    # bf16 table and entries 6 and 7 of the packed fp8 table serve grouped
    # calls only)
    want = {"bf16": 2, "bf16_bt": 5, "bf16_packed": 14, "fp8": 4, "fp8_packed": 9, "fp4": 1,
            "fp4_packed": 6, "w4a8_packed": 10}
    for entry, n in want.items():
        assert len(cases(bg, entry, FP8_KS.get(entry, [384]))) == n, entry
