"""fp64 CPU oracle for the batch-invariant GEMM and decode attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product library never loads it,
and it shares no code with the HIP path: the two meet only through the seeded
inputs that both consume.

The arithmetic lives in ``oracle.c`` (plain C, binary64, k ascending); this
module only builds/loads it and marshals numpy arrays.  What it computes is
the definition C[i][j] = sum_k A[i][k] * B[k][j] (article
"DeepSeek V4的batch invariance：大模型确定性推理的工程基石", section 2.1),
with alpha = 1, beta = 0 (wmrh.cn V4 engineering blog, section 3.1), over the
exact values the input codes encode.  Each call returns

* ``C``  -- the fp64 sum per element,
* ``S``  -- sum_k |a_k * b_k| per element (scale of the tolerance),

and ``round_bf16`` gives the direct fp64 -> bf16 round-to-nearest-even.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: every product and every sum rounds separately, as written.
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
          "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def build() -> str:
    """Compile liboracle.so with gcc (host only, no GPU involved)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.ora_dec_bf16.restype = ctypes.c_double
    lib.ora_dec_bf16.argtypes = [ctypes.c_uint16]
    lib.ora_dec_e4m3fn.restype = ctypes.c_double
    lib.ora_dec_e4m3fn.argtypes = [ctypes.c_uint8]
    lib.ora_dec_e2m1.restype = ctypes.c_double
    lib.ora_dec_e2m1.argtypes = [ctypes.c_uint8]
    lib.ora_rne_bf16.restype = ctypes.c_uint16
    lib.ora_rne_bf16.argtypes = [ctypes.c_double]
    lib.ora_round_bf16.restype = None
    lib.ora_round_bf16.argtypes = [i64, vp, vp]
    lib.ora_num_threads.restype = ctypes.c_int
    lib.ora_num_threads.argtypes = []
    lib.ora_set_num_threads.restype = None
    lib.ora_set_num_threads.argtypes = [ctypes.c_int]
    lib.ora_gemm_bf16.restype = None
    lib.ora_gemm_bf16.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64]
    lib.ora_gemm_fp8bs.restype = None
    lib.ora_gemm_fp8bs.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, i64]
    lib.ora_gemm_fp4w.restype = None
    lib.ora_gemm_fp4w.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, vp, i64]
    lib.ora_dec_e8m0.restype = ctypes.c_double
    lib.ora_dec_e8m0.argtypes = [ctypes.c_uint8]
    lib.ora_gemm_w4a8.restype = None
    lib.ora_gemm_w4a8.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, i64]
    lib.ora_decode_attn.restype = None
    lib.ora_decode_attn.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                    ctypes.c_double, vp, vp, vp]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _rows(a: np.ndarray, dtype, name: str) -> np.ndarray:
    if a.dtype != dtype or a.ndim != 2:
        raise TypeError(f"{name}: expected 2-D {np.dtype(dtype)}, got {a.dtype} {a.shape}")
    if a.size and a.shape[1] > 1 and a.strides[1] != a.itemsize:
        raise ValueError(f"{name}: rows must be contiguous")
    return a


def _ld(a: np.ndarray) -> int:
    return max(a.strides[0] // a.itemsize, a.shape[1], 1)


# ------------------------------------------------------------ decoders

def dec_bf16(code: int) -> float:
    return _load().ora_dec_bf16(int(code))


def dec_e4m3fn(code: int) -> float:
    return _load().ora_dec_e4m3fn(int(code))


def dec_e2m1(code: int) -> float:
    return _load().ora_dec_e2m1(int(code))


def dec_e8m0(code: int) -> float:
    return _load().ora_dec_e8m0(int(code))


def rne_bf16(x: float) -> int:
    return int(_load().ora_rne_bf16(float(x)))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Elementwise direct fp64 -> bf16 (RNE); returns uint16 codes."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().ora_round_bf16(x.size, _p(x), _p(out))
    return out


def num_threads() -> int:
    return int(_load().ora_num_threads())


def set_num_threads(n: int) -> None:
    """Host threads of the parallel loops (timing only; results do not depend on it)."""
    _load().ora_set_num_threads(int(n))


# ------------------------------------------------------------ GEMMs

def gemm_bf16(A: np.ndarray, B: np.ndarray):
    """A uint16 bf16 codes [M,K], B uint16 bf16 codes [K,N] -> (C, S) fp64 [M,N]."""
    A = _rows(A, np.uint16, "A")
    B = _rows(B, np.uint16, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    if M and N:
        _load().ora_gemm_bf16(M, N, K, _p(A), _ld(A), _p(B), _ld(B), _p(C), _p(S), N)
    return C, S


def gemm_bf16_grouped(A: np.ndarray, offsets, Bs):
    """Grouped (mixture-of-experts) GEMM by its definition: rows
    [offsets[g], offsets[g+1]) of A times Bs[g], one plain GEMM per group.
    Returns (C, S) fp64 [M,N]."""
    A = _rows(A, np.uint16, "A")
    offsets = [int(o) for o in offsets]
    if len(offsets) != len(Bs) + 1 or offsets[0] != 0 or offsets[-1] != A.shape[0] \
            or any(b < a for a, b in zip(offsets, offsets[1:])):
        raise ValueError("offsets must run from 0 to M, non-decreasing, one more than groups")
    N = Bs[0].shape[1]
    C = np.zeros((A.shape[0], N), np.float64)
    S = np.zeros((A.shape[0], N), np.float64)
    for g, B in enumerate(Bs):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            C[lo:hi], S[lo:hi] = gemm_bf16(np.ascontiguousarray(A[lo:hi]), B)
    return C, S


def gemm_fp8bs_grouped(qA: np.ndarray, sA: np.ndarray, offsets, qBs, sBs):
    """Grouped (mixture-of-experts) fp8 block-scaled GEMM by its definition:
    rows [offsets[g], offsets[g+1]) of (qA, sA) times expert g's (qBs[g],
    sBs[g]), one plain gemm_fp8bs per group.  Returns (C, S) fp64 [M,N]."""
    qA = _rows(qA, np.uint8, "qA")
    sA = _rows(sA, np.float32, "sA")
    offsets = [int(o) for o in offsets]
    if len(offsets) != len(qBs) + 1 or len(sBs) != len(qBs) or offsets[0] != 0 \
            or offsets[-1] != qA.shape[0] or any(b < a for a, b in zip(offsets, offsets[1:])):
        raise ValueError("offsets must run from 0 to M, non-decreasing, one more than groups")
    N = qBs[0].shape[1]
    C = np.zeros((qA.shape[0], N), np.float64)
    S = np.zeros((qA.shape[0], N), np.float64)
    for g, (qB, sB) in enumerate(zip(qBs, sBs)):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            C[lo:hi], S[lo:hi] = gemm_fp8bs(np.ascontiguousarray(qA[lo:hi]),
                                            np.ascontiguousarray(sA[lo:hi]), qB, sB)
    return C, S


def gemm_w4a8_grouped(qA: np.ndarray, sA: np.ndarray, offsets, Bqs, sEs, N: int):
    """Grouped (mixture-of-experts) W4A8 GEMM by its definition: rows
    [offsets[g], offsets[g+1]) of (qA, sA) times expert g's MXFP4 weights
    (Bqs[g] packed e2m1 [K, N/2], sEs[g] E8M0 [K/32, N]), one plain gemm_w4a8
    per group.  Returns (C, S) fp64 [M,N]."""
    qA = _rows(qA, np.uint8, "qA")
    sA = _rows(sA, np.float32, "sA")
    offsets = [int(o) for o in offsets]
    if len(offsets) != len(Bqs) + 1 or len(sEs) != len(Bqs) or offsets[0] != 0 \
            or offsets[-1] != qA.shape[0] or any(b < a for a, b in zip(offsets, offsets[1:])):
        raise ValueError("offsets must run from 0 to M, non-decreasing, one more than groups")
    C = np.zeros((qA.shape[0], N), np.float64)
    S = np.zeros((qA.shape[0], N), np.float64)
    for g, (Bq, sE) in enumerate(zip(Bqs, sEs)):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            C[lo:hi], S[lo:hi] = gemm_w4a8(np.ascontiguousarray(qA[lo:hi]),
                                           np.ascontiguousarray(sA[lo:hi]), Bq, sE, N)
    return C, S


def gemm_fp8bs(qA: np.ndarray, sA: np.ndarray, qB: np.ndarray, sB: np.ndarray):
    """qA uint8 e4m3fn [M,K], sA fp32 [M,K/128], qB uint8 e4m3fn [K,N],
    sB fp32 [K/128, ceil(N/128)] -> (C, S) fp64 [M,N]."""
    qA = _rows(qA, np.uint8, "qA")
    qB = _rows(qB, np.uint8, "qB")
    sA = _rows(sA, np.float32, "sA")
    sB = _rows(sB, np.float32, "sB")
    M, K = qA.shape
    K2, N = qB.shape
    if K2 != K or K % 128:
        raise ValueError("bad K")
    if sA.shape[0] < M or sA.shape[1] < K // 128:
        raise ValueError("sA too small")
    if sB.shape[0] < K // 128 or sB.shape[1] < (N + 127) // 128:
        raise ValueError("sB too small")
    C = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    if M and N:
        _load().ora_gemm_fp8bs(M, N, K, _p(qA), _ld(qA), _p(sA), _ld(sA),
                               _p(qB), _ld(qB), _p(sB), _ld(sB), _p(C), _p(S), N)
    return C, S


def gemm_fp4w(A: np.ndarray, Bq: np.ndarray, sB: np.ndarray, N: int):
    """A uint16 bf16 [M,K], Bq uint8 packed e2m1 [K, N/2], sB uint8 e4m3fn [K/32, N]
    -> (C, S) fp64 [M,N]."""
    A = _rows(A, np.uint16, "A")
    Bq = _rows(Bq, np.uint8, "Bq")
    sB = _rows(sB, np.uint8, "sB")
    M, K = A.shape
    if Bq.shape[0] != K or Bq.shape[1] * 2 < N or K % 32:
        raise ValueError("bad Bq / K")
    if sB.shape[0] < K // 32 or sB.shape[1] < N:
        raise ValueError("sB too small")
    C = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    if M and N:
        _load().ora_gemm_fp4w(M, N, K, _p(A), _ld(A), _p(Bq), _ld(Bq),
                              _p(sB), _ld(sB), _p(C), _p(S), N)
    return C, S


def gemm_w4a8(qA: np.ndarray, sA: np.ndarray, Bq: np.ndarray, sE: np.ndarray, N: int):
    """fp8 activations x OCP MXFP4 weights.  qA uint8 e4m3fn [M,K], sA fp32
    [M,K/128] (one scale per 1x128 block), Bq uint8 packed e2m1 [K, N/2],
    sE uint8 E8M0 [K/32, N] (one power-of-two scale per 32 K per column)
    -> (C, S) fp64 [M,N]."""
    qA = _rows(qA, np.uint8, "qA")
    sA = _rows(sA, np.float32, "sA")
    Bq = _rows(Bq, np.uint8, "Bq")
    sE = _rows(sE, np.uint8, "sE")
    M, K = qA.shape
    if Bq.shape[0] != K or Bq.shape[1] * 2 < N or K % 128:
        raise ValueError("bad Bq / K")
    if sA.shape[0] < M or sA.shape[1] < K // 128:
        raise ValueError("sA too small")
    if sE.shape[0] < K // 32 or sE.shape[1] < N:
        raise ValueError("sE too small")
    C = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    if M and N:
        _load().ora_gemm_w4a8(M, N, K, _p(qA), _ld(qA), _p(sA), _ld(sA), _p(Bq), _ld(Bq),
                              _p(sE), _ld(sE), _p(C), _p(S), N)
    return C, S


def decode_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, lens, scale: float,
                     weights: bool = False):
    """Decode attention by its definition (scaled dot-product attention,
    Vaswani et al. 2017, equation 1, with grouped-query heads): query head h of
    sequence b attends to keys/values [0, lens[b]) of KV head h // (Hq/Hkv).

    Q uint16 bf16 codes [B,Hq,D]; K, V uint16 bf16 codes [B,Hkv,Lmax,D];
    lens int [B].  Returns O fp64 [B,Hq,D], and with ``weights`` also
    W fp64 [B,Hq,Lmax] (normalised softmax weights, 0 past the length) and
    A fp64 [B,Hq,Lmax] (sum_d |q_d k_jd|, the scale of a score's rounding)."""
    Q = np.ascontiguousarray(Q, np.uint16)
    K = np.ascontiguousarray(K, np.uint16)
    V = np.ascontiguousarray(V, np.uint16)
    B, Hq, D = Q.shape
    B2, Hkv, Lmax, D2 = K.shape
    if V.shape != K.shape or B2 != B or D2 != D or Hkv == 0 or Hq % Hkv:
        raise ValueError("shapes: Q [B,Hq,D], K and V [B,Hkv,Lmax,D], Hq a multiple of Hkv")
    lens = np.ascontiguousarray(lens, np.int32)
    if lens.shape != (B,) or np.any(lens < 0) or np.any(lens > Lmax):
        raise ValueError("lens must be [B] in [0, Lmax]")
    O = np.empty((B, Hq, D), np.float64)
    W = np.empty((B, Hq, Lmax), np.float64) if weights else None
    A = np.empty((B, Hq, Lmax), np.float64) if weights else None
    if B and Hq and D:
        _load().ora_decode_attn(B, Hq, Hkv, D, Lmax, _p(Q), _p(K), _p(V), _p(lens),
                                float(scale), _p(O), _p(W) if weights else None,
                                _p(A) if weights else None)
    return (O, W, A) if weights else O
