"""The full-size seeded workloads and their fp64 oracle results, each computed
once per test session so that every GPU test at that size can check every row
of its largest batch against the oracle.  No GEMM arithmetic lives here: the
inputs come from the seeded generators, the results from the oracle."""
import functools

import numpy as np

import oracle
from invariant_gemm_amd import inputs


@functools.lru_cache(maxsize=None)
def c2():
    """bf16 K = N = 8192: pool A [256, K] ~ N(0,1) (seed 201), B ~ N(0, 0.02) (202);
    returns (A, B, C64, S) with the oracle over all 256 pool rows."""
    A = inputs.normal_bf16((256, 8192), 1.0, 201)
    B = inputs.normal_bf16((8192, 8192), 0.02, 202)
    C64, S = oracle.gemm_bf16(A, B)
    return A, B, C64, S


@functools.lru_cache(maxsize=None)
def c3():
    """fp8 e4m3fn K = 7168, N = 2048: A [512, K] ~ N(0,1) with 1x128 fp32 scales
    (seed 301), B ~ N(0,1) with 128x128 scales (302); oracle over all 512 rows."""
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((512, 7168), 1.0, 301))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((7168, 2048), 1.0, 302))
    C64, S = oracle.gemm_fp8bs(qA, sA, qB, sB)
    return qA, sA, qB, sB, C64, S


@functools.lru_cache(maxsize=None)
def c4():
    """fp4 e2m1 weight-only K = 4096, N = 14336: A [512, K] bf16 ~ N(0,1) (401),
    W ~ N(0, 0.02) quantised per 32 K with e4m3fn scales (402); oracle over all
    512 rows."""
    A = inputs.normal_bf16((512, 4096), 1.0, 401)
    Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((4096, 14336), 0.02, 402))
    C64, S = oracle.gemm_fp4w(A, Bq, sB, 14336)
    return A, Bq, sB, C64, S


@functools.lru_cache(maxsize=None)
def w4a8():
    """W4A8 at the fp4 weight shape K = 4096, N = 14336: A [512, K] ~ N(0,1) as
    e4m3fn with 1x128 scales (1801), W ~ N(0, 0.02) as MXFP4 (1802); oracle over
    all 512 rows."""
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((512, 4096), 1.0, 1801))
    Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((4096, 14336), 0.02, 1802))
    C64, S = oracle.gemm_w4a8(qA, sA, Bq, sE, 14336)
    return qA, sA, Bq, sE, C64, S


def all_rows(C_codes: np.ndarray, C64: np.ndarray) -> np.ndarray:
    """Guard against comparing a partial batch: the GPU result must hold every row."""
    assert C_codes.shape == C64.shape, (C_codes.shape, C64.shape)
    return C_codes
