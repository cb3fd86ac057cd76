"""GPU tests at the size extremes of every plain GEMM entry point: a batch of
4096 rows (many row tiles and several rounds of workgroups per compute unit),
a K of 64K (the longest K loop, with a ragged tail where the format allows
one) and an N of 64K + 16 (the widest grid, with a ragged last column block).

Sampled rows of each launch must be bitwise equal to the same rows computed
alone (M = 1) and within the parity tolerance |err| <= 2^-7 S + 1e-6 of the
fp64 oracle (S = sum |a_k b_k|, the tolerance the method is specified with).
Rows are sampled because the oracle is a plain CPU loop; the samples include
the first and last row of the batch and rows on both sides of tile
boundaries."""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests.gpu_util import check_parity, dev_bf16, dev_f32, dev_u8, host_codes, require_gpu

pytestmark = pytest.mark.gpu

ENTRIES = ["bf16", "bf16_bt", "bf16_packed", "fp8", "fp8_packed", "fp4", "fp4_packed", "w4a8"]


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def pad16(n):
    return (n + 15) // 16 * 16


class Case:
    """One entry point on one seeded problem: device operands, a launch over
    any row range, and the oracle for any set of rows."""

    def __init__(self, bg, entry, M, N, K, seed):
        self.entry, self.N, self.K = entry, N, K
        if entry.startswith("bf16"):
            A = inputs.normal_bf16((M, K), 1.0, seed)
            B = inputs.normal_bf16((K, N), 0.02, seed + 1)
            self.Ad = dev_bf16(A)
            if entry == "bf16":
                Bd = dev_bf16(B)
                self.fn = lambda r: bg.gemm_bf16(self.Ad[r], Bd)
            elif entry == "bf16_bt":
                Btd = dev_bf16(np.ascontiguousarray(B.T))
                self.fn = lambda r: bg.gemm_bf16_bt(self.Ad[r], Btd)
            else:
                Bp = bg.pack_b_bf16(dev_bf16(B))
                self.fn = lambda r: bg.gemm_bf16_packed(self.Ad[r], Bp)
            self.ref = lambda rows: oracle.gemm_bf16(A[rows], B)
        elif entry.startswith("fp8"):
            qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, seed))
            qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, seed + 1))
            Ad, sAd, sBd = dev_u8(qA), dev_f32(sA), dev_f32(sB)
            if entry == "fp8":
                Bd = dev_u8(qB)
                self.fn = lambda r: bg.gemm_fp8_blockscaled(Ad[r], sAd[r], Bd, sBd)
            else:
                Bp = bg.pack_b_fp8(dev_u8(qB))
                self.fn = lambda r: bg.gemm_fp8_blockscaled_packed(Ad[r], sAd[r], Bp, sBd)
            self.ref = lambda rows: oracle.gemm_fp8bs(qA[rows], sA[rows], qB, sB)
        elif entry.startswith("fp4"):
            A = inputs.normal_bf16((M, K), 1.0, seed)
            Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, seed + 1))
            Ad = dev_bf16(A)
            if entry == "fp4":
                Bqd, sBd = dev_u8(Bq, pad16(Bq.shape[1])), dev_u8(sB, pad16(N))
                self.fn = lambda r: bg.gemm_fp4_w(Ad[r], Bqd, sBd, N)
            else:
                Bp = bg.pack_b_fp4(dev_u8(Bq), dev_u8(sB), N)
                self.fn = lambda r: bg.gemm_fp4_w_packed(Ad[r], Bp)
            self.ref = lambda rows: oracle.gemm_fp4w(A[rows], Bq, sB, N)
        else:
            qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, seed))
            Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, seed + 1))
            Ad, sAd = dev_u8(qA), dev_f32(sA)
            Bp = bg.pack_b_mxfp4(dev_u8(Bq, pad16(Bq.shape[1])), dev_u8(sE, pad16(N)), N)
            self.fn = lambda r: bg.gemm_w4a8_packed(Ad[r], sAd[r], Bp)
            self.ref = lambda rows: oracle.gemm_w4a8(qA[rows], sA[rows], Bq, sE, N)

    def check(self, M, rows, what):
        batch = host_codes(self.fn(slice(0, M)))
        alone = np.concatenate([host_codes(self.fn(slice(r, r + 1))) for r in rows])
        torch.cuda.synchronize()
        got = batch[rows]
        bad = [r for r, a, b in zip(rows, got, alone) if not np.array_equal(a, b)]
        assert not bad, f"{what}: rows {bad[:8]} differ from the same rows computed alone"
        C64, S = self.ref(np.asarray(rows))
        check_parity(got, C64, S, self.K, what)


def sample_rows(M, tile_edges, seed, extra=4):
    rows = {0, M - 1}
    for e in tile_edges:
        rows.update(r for r in (e - 1, e) if 0 <= r < M)
    rows.update(int(r) for r in inputs.rng(seed).choice(M, size=extra, replace=False))
    return sorted(rows)


# 4096 rows: the largest tiles (64 rows) give 64 row tiles, and every
# geometry runs several rounds of workgroups on the 256 compute units.
@pytest.mark.parametrize("entry", ENTRIES)
def test_many_rows(bg, entry):
    M, N, K = 4096, 528, 512
    case = Case(bg, entry, M, N, K, 9100 + ENTRIES.index(entry))
    case.check(M, sample_rows(M, (64, 128, 2048, 4032), 9200), f"{entry} M{M} N{N} K{K}")


# K = 64K: the longest K loop of the tests; the bf16 and fp4 cases end in a
# partial K step or stage (K % 32 != 0 is allowed for bf16 only).
@pytest.mark.parametrize("entry", ENTRIES)
def test_long_k(bg, entry):
    K = {"bf16": 65576, "bf16_bt": 65576, "bf16_packed": 65576, "fp4": 65568,
         "fp4_packed": 65568}.get(entry, 65536)
    M, N = 5, 272
    case = Case(bg, entry, M, N, K, 9300 + ENTRIES.index(entry))
    case.check(M, list(range(M)), f"{entry} M{M} N{N} K{K}")


# N = 64K + 16: the widest grid of the tests, ending in a ragged last column
# block for every column tiling (16, 32, 64 and 128 columns).
@pytest.mark.parametrize("entry", ENTRIES)
def test_wide_n(bg, entry):
    N = 65552
    K = 128 if entry in ("fp8", "fp8_packed", "w4a8") else 96
    M = 3
    case = Case(bg, entry, M, N, K, 9500 + ENTRIES.index(entry))
    case.check(M, list(range(M)), f"{entry} M{M} N{N} K{K}")
