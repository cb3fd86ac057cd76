"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects every invalid argument with the documented
status before any HIP call (the pointers below are never dereferenced)."""
import ctypes
import inspect
import os
import re

import pytest

from invariant_gemm_amd import bigemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "bigemm.h")

OK, NULL, SHAPE, STRIDE, ALIGN, UNSUP, LAUNCH, WS = range(8)
P = 0x10000          # fake, 16-byte aligned "device" address; never dereferenced
lib = bigemm.lib


def _declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"bi_gemm_bf16", "bi_gemm_fp8_blockscaled", "bi_gemm_fp4_w", "bi_schedule_query",
            "bi_status_str", "bi_gemm_bf16_splitk"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in bigemm.STATUS.items():
        assert lib.bi_status_str(code).decode() == name
    assert lib.bi_status_str(99).decode() == "BI_ERR_UNKNOWN"
    assert bigemm.version().startswith("libbigemm")


def bf16(M, N, K, A=P, lda=None, B=P, ldb=None, C=P, ldc=None):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return lib.bi_gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, None)


def test_bf16_validation():
    assert bf16(-1, 8, 8) == SHAPE
    assert bf16(8, -1, 8) == SHAPE
    assert bf16(8, 8, -1) == SHAPE
    assert bf16(8, (1 << 24) + 1, 8) == UNSUP
    assert bf16(0, 8, 8, A=None, B=None, C=None) == OK        # empty: no-op
    assert bf16(8, 0, 8, A=None, B=None, C=None) == OK
    assert bf16(8, 8, 8, A=None) == NULL
    assert bf16(8, 8, 8, B=None) == NULL
    assert bf16(8, 8, 8, C=None) == NULL
    assert bf16(8, 8, 16, lda=8) == STRIDE
    assert bf16(8, 16, 8, ldb=8) == STRIDE
    assert bf16(8, 16, 8, ldc=8) == STRIDE
    assert bf16(8, 8, 8, A=P + 2) == ALIGN
    assert bf16(8, 8, 8, B=P + 8) == ALIGN
    assert bf16(8, 8, 8, C=P + 1) == ALIGN
    assert bf16(8, 8, 12) == ALIGN            # lda = 12: row pitch 24 B


def test_bf16_bt_validation():
    f = lambda M, N, K, A=P, lda=None, Bt=P, ldbt=None, C=P, ldc=None: lib.bi_gemm_bf16_bt(
        M, N, K, A, K if lda is None else lda, Bt, K if ldbt is None else ldbt, C,
        N if ldc is None else ldc, None)
    assert f(-1, 8, 8) == SHAPE
    assert f(8, 8, 8, Bt=None) == NULL
    assert f(8, 64, 16, ldbt=8) == STRIDE       # Bt rows hold K elements
    assert f(8, 64, 16, ldbt=20) == ALIGN
    assert f(0, 8, 8, A=None, Bt=None, C=None) == OK


def test_bf16_k0_needs_no_operands():
    # K == 0 with NULL A/B passes validation; it would launch (C = 0), so
    # only the validation order is checked here: a NULL C is still rejected.
    assert bf16(4, 8, 0, A=None, B=None, C=None) == NULL


def fp8(M, N, K, A=P, lda=None, sA=P, ldsa=None, B=P, ldb=None, sB=P, ldsb=None, C=P, ldc=None):
    lda = K if lda is None else lda
    ldsa = K // 128 if ldsa is None else ldsa
    ldb = N if ldb is None else ldb
    ldsb = (N + 127) // 128 if ldsb is None else ldsb
    ldc = N if ldc is None else ldc
    return lib.bi_gemm_fp8_blockscaled(M, N, K, A, lda, sA, ldsa, B, ldb, sB, ldsb, C, ldc, None)


def test_fp8_validation():
    assert fp8(-1, 16, 128) == SHAPE
    assert fp8(4, 16, 100) == SHAPE          # K % 128
    assert fp8(0, 16, 128, A=None) == OK
    assert fp8(4, 16, 128, sA=None) == NULL
    assert fp8(4, 16, 128, sB=None) == NULL
    assert fp8(4, 16, 256, ldsa=1) == STRIDE
    assert fp8(4, 300, 128, ldsb=2) == STRIDE
    assert fp8(4, 16, 128, lda=120) == STRIDE
    assert fp8(4, 16, 128, lda=136) == ALIGN   # 136 B pitch
    assert fp8(4, 24, 128) == ALIGN            # ldb = 24 B pitch
    assert fp8(4, 16, 128, sA=P + 2) == ALIGN  # fp32 scales need 4-byte alignment


def fp4(M, N, K, A=P, lda=None, Bq=P, ldbq=None, sB=P, ldsb=None, C=P, ldc=None):
    lda = K if lda is None else lda
    ldbq = N // 2 if ldbq is None else ldbq
    ldsb = N if ldsb is None else ldsb
    ldc = N if ldc is None else ldc
    return lib.bi_gemm_fp4_w(M, N, K, A, lda, Bq, ldbq, sB, ldsb, C, ldc, None)


def test_fp4_validation():
    assert fp4(4, 64, 48) == SHAPE             # K % 32
    assert fp4(4, 63, 64) == SHAPE             # odd N
    assert fp4(4, 64, 64, Bq=None) == NULL
    assert fp4(4, 64, 64, sB=None) == NULL
    assert fp4(4, 64, 64, ldbq=16) == STRIDE
    assert fp4(4, 64, 64, ldsb=32) == STRIDE
    assert fp4(4, 48, 64) == ALIGN             # ldbq = 24 B
    assert fp4(4, 64, 64, sB=P + 1) == ALIGN
    assert fp4(0, 64, 64, A=None, Bq=None, sB=None, C=None) == OK


def test_splitk_validation():
    f = lib.bi_gemm_bf16_splitk
    assert f(4, 8, 128, P, 128, P, 8, P, 8, None, 1 << 20, 0, None) == WS
    assert f(4, 8, 128, P, 128, P, 8, P, 8, P, 4 * 8 * 4 - 1, 0, None) == WS
    assert f(4, 8, 128, P, 128, P, 8, P, 8, P, 1 << 20, -1, None) == SHAPE
    assert f(4, 8, 128, P + 2, 128, P, 8, P, 8, P, 1 << 20, 0, None) == ALIGN
    # the comparator's split count follows M -- by design, unlike the invariant path
    ks = [bigemm.splitk_choose(m, 8192, 8192) for m in (1, 2, 4, 8, 16, 256)]
    assert len(set(ks)) > 1 and all(1 <= s <= 64 for s in ks)


def test_schedule_has_no_m_argument():
    # the schedule is a function of (dtype, N, K) by construction: the C
    # signature has exactly four parameters and none of them is M
    assert len(lib.bi_schedule_query.argtypes) == 4
    hdr = open(HDR).read()
    decl = re.search(r"bi_status bi_schedule_query\(([^)]*)\)", hdr).group(1)
    params = [p.strip().split()[-1].lstrip("*") for p in decl.split(",")]
    assert params == ["dtype", "N", "K", "out"]
    for dt in (bigemm.BI_BF16, bigemm.BI_FP8_BS, bigemm.BI_FP4_W, bigemm.BI_W4A8):
        s = bigemm.schedule(dt, 8192, 8192)
        assert s["mfma_m"] == 16 and s["mfma_n"] == 16
        # the arithmetic is the same for every N and K the format accepts
        for N, K in ((256, 512), (14336, 4096), (2048, 7168), (130, 1024)):
            assert bigemm.schedule(dt, N, K) == s
    assert bigemm.schedule(bigemm.BI_BF16, 8192, 8192)["order"] == bigemm.ORDER_SEQUENTIAL
    assert bigemm.schedule(bigemm.BI_FP8_BS, 8192, 8192)["order"] == bigemm.ORDER_BLOCK_FMA
    assert lib.bi_schedule_query(7, 8192, 8192, ctypes.byref(bigemm.BiSchedule())) == UNSUP
    assert lib.bi_schedule_query(0, 8192, 8192, None) == NULL
    assert lib.bi_schedule_query(1, 8192, 100, ctypes.byref(bigemm.BiSchedule())) == SHAPE


def test_packed_sizes():
    nb = lambda N: (N + 15) // 16
    assert bigemm.packed_b_bytes(bigemm.BI_BF16, 300, 100) == nb(300) * 4 * 1024
    assert bigemm.packed_b_bytes(bigemm.BI_FP8_BS, 2048, 7168) == 128 * 56 * 2048
    assert bigemm.packed_b_bytes(bigemm.BI_FP8_BS, 2048, 100) == 0          # K % 128
    assert bigemm.packed_b_bytes(bigemm.BI_FP4_W, 14336, 4096) == 896 * 32 * 1088
    assert bigemm.packed_b_bytes(bigemm.BI_FP4_W, 130, 288) == nb(130) * 3 * 1088
    assert bigemm.packed_b_bytes(bigemm.BI_FP4_W, 131, 288) == 0            # odd N
    assert bigemm.packed_b_bytes(bigemm.BI_FP4_W, 130, 48) == 0             # K % 32
    assert bigemm.packed_b_bytes(7, 16, 16) == 0
    assert bigemm.packed_b_bytes(bigemm.BI_BF16, -1, 16) == 0


def test_packed_validation():
    need = lambda dt, N, K: bigemm.packed_b_bytes(dt, N, K)
    # bf16
    f = lambda M, N, K, A=P, lda=None, Bp=P, nb=None, C=P, ldc=None: lib.bi_gemm_bf16_packed(
        M, N, K, A, K if lda is None else lda, Bp, need(0, N, K) if nb is None else nb, C,
        N if ldc is None else ldc, None)
    assert f(8, 64, 64, nb=need(0, 64, 64) - 1) == WS
    assert f(8, 64, 64, Bp=P + 8) == ALIGN
    assert f(8, 64, 64, Bp=None) == NULL
    assert f(0, 64, 64, A=None, Bp=None, C=None) == OK
    # fp8
    g = lambda M, N, K, A=P, lda=None, sA=P, Bp=P, nb=None, sB=P, ldsb=None, C=P: \
        lib.bi_gemm_fp8_blockscaled_packed(M, N, K, A, K if lda is None else lda, sA, max(K // 128, 1),
                                           Bp, need(1, N, K) if nb is None else nb, sB,
                                           (N + 127) // 128 if ldsb is None else ldsb, C, N, None)
    assert g(4, 64, 100) == SHAPE
    assert g(4, 64, 256, nb=need(1, 64, 256) - 16) == WS
    assert g(4, 64, 256, sA=None) == NULL
    assert g(4, 300, 256, ldsb=2) == STRIDE
    assert g(4, 64, 256, lda=264) == ALIGN
    assert g(4, 64, 256, sB=P + 2) == ALIGN
    assert g(0, 64, 256, A=None, sA=None, Bp=None, sB=None, C=None) == OK
    assert lib.bi_pack_b_fp8(64, 100, P, 64, P, 1 << 20, None) == SHAPE
    assert lib.bi_pack_b_fp8(64, 256, P, 32, P, 1 << 20, None) == STRIDE
    assert lib.bi_pack_b_fp8(64, 256, P, 64, P, need(1, 64, 256) - 1, None) == WS
    assert lib.bi_pack_b_fp8(64, 256, None, 64, P, 1 << 20, None) == NULL
    # fp4
    h = lambda M, N, K, A=P, Bp=P, nb=None, C=P: lib.bi_gemm_fp4_w_packed(
        M, N, K, A, K, Bp, need(2, N, K) if nb is None else nb, C, N, None)
    assert h(4, 64, 48) == SHAPE
    assert h(4, 63, 64) == SHAPE
    assert h(4, 64, 64, nb=need(2, 64, 64) - 1) == WS
    assert h(4, 64, 64, Bp=P + 4) == ALIGN
    assert h(4, 64, 64, Bp=None) == NULL
    assert lib.bi_pack_b_fp4(64, 64, P, 32, P, 64, P, need(2, 64, 64) - 1, None) == WS
    assert lib.bi_pack_b_fp4(64, 64, P, 16, P, 64, P, 1 << 20, None) == STRIDE
    assert lib.bi_pack_b_fp4(64, 64, P, 32, None, 64, P, 1 << 20, None) == NULL
    assert lib.bi_pack_b_fp4(64, 48, P, 32, P, 64, P, 1 << 20, None) == SHAPE


def test_grouped_validation():
    need = bigemm.packed_b_bytes(bigemm.BI_BF16, 64, 64)
    f = lambda G, M, N=64, K=64, off=P, A=P, Bp=P, nb=None, C=P: lib.bi_gemm_bf16_grouped_packed(
        G, off, M, N, K, A, K, Bp, need * G if nb is None else nb, C, N, None)
    assert f(-1, 8) == SHAPE
    assert f(0, 8) == SHAPE                    # rows but no group
    assert f(0, 0) == OK
    assert f(3, 0, off=None, A=None, Bp=None, C=None) == OK
    assert f(3, 8, off=None) == NULL
    assert f(3, 8, nb=need * 3 - 1) == WS
    assert f(3, 8, off=P + 2) == ALIGN
    assert f(1 << 20, 8) == UNSUP


def test_grouped_fp8_validation():
    need = bigemm.packed_b_bytes(bigemm.BI_FP8_BS, 64, 256)
    f = lambda G, M, N=64, K=256, off=P, A=P, sA=P, Bp=P, nb=None, sB=P, ldsb=1, C=P: \
        lib.bi_gemm_fp8_blockscaled_grouped_packed(G, off, M, N, K, A, K, sA, K // 128, Bp,
                                                   need * G if nb is None else nb, sB, ldsb, C, N, None)
    assert f(-1, 8) == SHAPE
    assert f(0, 8) == SHAPE                    # rows but no group
    assert f(3, 8, K=200) == SHAPE             # K % 128
    assert f(0, 0) == OK
    assert f(3, 0, off=None, A=None, sA=None, Bp=None, sB=None, C=None) == OK
    assert f(3, 8, off=None) == NULL
    assert f(3, 8, sB=None) == NULL
    assert f(3, 8, ldsb=0) == STRIDE
    assert f(3, 8, nb=need * 3 - 1) == WS
    assert f(3, 8, off=P + 2) == ALIGN
    assert f(3, 8, sB=P + 2) == ALIGN
    assert f(1 << 20, 8) == UNSUP


def test_grouped_w4a8_validation():
    need = bigemm.packed_b_bytes(bigemm.BI_W4A8, 64, 256)
    f = lambda G, M, N=64, K=256, off=P, A=P, lda=None, sA=P, Bp=P, nb=None, C=P: \
        lib.bi_gemm_w4a8_grouped_packed(G, off, M, N, K, A, K if lda is None else lda, sA,
                                        max(K // 128, 1), Bp, need * G if nb is None else nb, C, N, None)
    assert f(-1, 8) == SHAPE
    assert f(0, 8) == SHAPE                    # rows but no group
    assert f(3, 8, K=200) == SHAPE             # K % 128
    assert f(3, 8, N=63) == SHAPE              # N odd
    assert f(0, 0) == OK
    assert f(3, 0, off=None, A=None, sA=None, Bp=None, C=None) == OK
    assert f(3, 8, off=None) == NULL
    assert f(3, 8, sA=None) == NULL
    assert f(3, 8, lda=128) == STRIDE
    assert f(3, 8, nb=need * 3 - 1) == WS
    assert f(3, 8, off=P + 2) == ALIGN
    assert f(3, 8, lda=264) == ALIGN
    assert f(3, 8, sA=P + 2) == ALIGN
    assert f(1 << 20, 8) == UNSUP


def test_w4a8_validation():
    need = lambda N, K: bigemm.packed_b_bytes(bigemm.BI_W4A8, N, K)
    assert need(2048, 7168) == 128 * 56 * 1088 and need(64, 100) == 0 and need(63, 128) == 0
    f = lambda M, N, K, A=P, lda=None, sA=P, Bp=P, nb=None, C=P: lib.bi_gemm_w4a8_packed(
        M, N, K, A, K if lda is None else lda, sA, max(K // 128, 1), Bp,
        need(N, K) if nb is None else nb, C, N, None)
    assert f(4, 64, 100) == SHAPE
    assert f(4, 63, 128) == SHAPE
    assert f(4, 64, 128, sA=None) == NULL
    assert f(4, 64, 128, nb=need(64, 128) - 1) == WS
    assert f(4, 64, 128, lda=136) == ALIGN
    assert f(4, 64, 128, sA=P + 2) == ALIGN
    assert f(0, 64, 128, A=None, sA=None, Bp=None, C=None) == OK
    assert lib.bi_pack_b_mxfp4(64, 100, P, 32, P, 64, P, 1 << 20, None) == SHAPE
    assert lib.bi_pack_b_mxfp4(64, 128, P, 16, P, 64, P, 1 << 20, None) == STRIDE
    assert lib.bi_pack_b_mxfp4(64, 128, P, 32, P, 64, P, need(64, 128) - 1, None) == WS
    s = bigemm.schedule(bigemm.BI_W4A8, 14336, 4096)
    assert s["mfma_k"] == 128


def test_decode_attention_validation():
    need = lambda B, Hq, Hkv, L: lib.bi_decode_attention_workspace_bytes(B, Hq, Hkv, L)
    assert need(1, 64, 8, 4096) == 8 * 16 * (8 * 128 + 16) * 4
    assert need(3, 6, 3, 257) == 3 * 3 * 2 * (2 * 128 + 4) * 4
    assert need(1, 6, 4, 64) == 0 and need(1, 64, 2, 64) == 0   # bad group / G > 16

    def f(B=2, Hq=16, Hkv=2, D=128, L=512, Q=P, K=P, V=P, lens=P, O=P, ws=P, nb=None, kernel=2):
        nb = need(B, Hq, Hkv, L) if nb is None else nb
        return lib.bi_decode_attention_bf16(B, Hq, Hkv, D, L, Q, K, V, lens, 0.1, O, ws, nb,
                                            kernel, None)
    assert f(B=-1) == SHAPE and f(L=-1) == SHAPE and f(D=-1) == SHAPE
    assert f(Hq=15) == SHAPE and f(Hkv=0) == SHAPE
    assert f(D=64) == UNSUP and f(Hq=34) == UNSUP and f(L=(1 << 22) + 1) == UNSUP
    assert f(kernel=3) == UNSUP and f(kernel=-1) == UNSUP
    assert f(B=0, Q=None, K=None, V=None, lens=None, O=None, ws=None) == OK
    assert f(Hq=0, Hkv=0, Q=None, O=None) == OK
    assert f(Q=None) == NULL and f(lens=None) == NULL and f(K=None) == NULL
    assert f(Q=P + 8) == ALIGN and f(V=P + 2) == ALIGN and f(lens=P + 2) == ALIGN
    assert f(ws=None) == WS and f(nb=need(2, 16, 2, 512) - 1) == WS
    assert f(ws=P + 4) == ALIGN
    assert bigemm.decode_attention_choice(1, 64, 8, 4096) == "split"
    assert bigemm.decode_attention_choice(32, 64, 8, 4096) == "single"
    assert bigemm.decode_attention_choice(1, 64, 8, 256) == "single"    # one group: nothing to split


def test_row_pitch_cap():
    # a kernel reads up to 128 rows of an input from one base with 32-bit
    # offsets; pitches past BI_MAX_PITCH_BYTES (16 MiB) are refused up front
    # (every call here must be refused: a call that passed would launch on
    # the fake pointer)
    cap = 1 << 24
    assert bf16(8, 8, 8, lda=cap // 2 + 8) == UNSUP
    assert bf16(8, 8, 8, ldb=cap // 2 + 8) == UNSUP
    assert fp4(8, 8, 32, ldbq=cap + 16) == UNSUP
    assert fp4(8, 8, 32, lda=cap // 2 + 8) == UNSUP
    assert lib.bi_gemm_fp8_blockscaled(8, 8, 128, P, cap + 16, P, 1, P, 16, P, 1, P, 8, None) == UNSUP
    assert lib.bi_gemm_fp8_blockscaled(8, 8, 128, P, 128, P, cap // 4 + 4, P, 16, P, 1, P, 8,
                                       None) == UNSUP
    need = bigemm.packed_b_bytes(bigemm.BI_BF16, 64, 64)
    assert lib.bi_gemm_bf16_packed(8, 64, 64, P, cap // 2 + 8, P, need, P, 64, None) == UNSUP
    need = bigemm.packed_b_bytes(bigemm.BI_W4A8, 64, 128)
    assert lib.bi_gemm_w4a8_packed(8, 64, 128, P, cap + 16, P, 1, P, need, P, 64, None) == UNSUP


# ------------------------------------------------------------------ launch geometry

GEOM_CASES = {
    # entry: (N, K, Ms) -- the configs' shapes and M sweeps
    "bf16": (8192, 8192, [2**i for i in range(9)] + [3, 17, 37, 100, 129, 255]),
    "bf16_bt": (8192, 8192, [2**i for i in range(9)] + [3, 17, 37, 100, 129, 255]),
    "bf16_packed": (8192, 8192, [2**i for i in range(9)] + [3, 17, 37, 100, 129, 160, 255]),
    "fp8": (2048, 7168, list(range(1, 513))),
    "fp8_packed": (2048, 7168, list(range(1, 513))),
    "fp4": (14336, 4096, [1, 8, 64, 512, 3, 100, 257]),
    "fp4_packed": (14336, 4096, [1, 8, 17, 33, 64, 65, 129, 512]),
    "w4a8_packed": (14336, 4096, [1, 8, 16, 17, 64, 65, 129, 300, 512]),
}


@pytest.mark.parametrize("entry", sorted(GEOM_CASES))
def test_geometry_query_covers_the_output(entry):
    """At every M of the sweeps the geometry's tiles cover C exactly once:
    workgroups = ceil(M / bm) * ceil(N / bn), the staged rows fit the tile, and
    the geometry changes only with M (never its arithmetic: bi_schedule_query
    has no M)."""
    N, K, Ms = GEOM_CASES[entry]
    ids = set()
    for M in Ms:
        g = bigemm.geometry(entry, M, N, K)
        assert g["bm"] % 16 == 0 and g["bn"] in (8, 16, 32, 64, 128), g
        assert 1 <= g["a_rows"] <= g["bm"] and 1 <= g["waves"] <= 8, g
        assert g["k_stage"] > 0 and g["stages"] >= 1, g
        assert g["workgroups"] == -(-M // g["bm"]) * -(-N // g["bn"]), (M, g)
        if g["a_rows"] < g["bm"]:
            assert M <= g["a_rows"], (M, g)      # only calls that fit the staged rows
        ids.add(g["id"])
    multi = {"bf16", "bf16_bt", "bf16_packed", "fp8", "fp8_packed", "fp4_packed", "w4a8_packed"}
    assert (len(ids) > 1) == (entry in multi), ids


def test_geometry_query_headline_sweep():
    # the headline sweep K = N = 8192: the packed kernel's tiles grow with M
    # and every one fills the compute units once M allows it
    seen = [bigemm.geometry("bf16_packed", M, 8192, 8192) for M in [2**i for i in range(9)]]
    assert [g["bm"] for g in seen] == [16, 16, 16, 16, 16, 32, 32, 64, 64]
    assert seen[-1]["bn"] == 128 and seen[-1]["workgroups"] == 256
    assert all(g["workgroups"] >= 256 for g in seen)


def test_geometry_query_grouped_and_errors():
    g = bigemm.geometry("bf16_grouped_packed", 512, 2048, 7168, groups=8)
    assert g["bm"] == 64
    # at most one row slot per non-empty group at M = 1
    g1 = bigemm.geometry("bf16_grouped_packed", 1, 2048, 7168, groups=8)
    assert g1["workgroups"] == -(-2048 // g1["bn"])
    for M in (1, 8, 64, 512, 4096):
        g8 = bigemm.geometry("fp8_grouped_packed", M, 2048, 7168, groups=8)
        assert g8["workgroups"] >= -(-M // g8["bm"]) * -(-2048 // g8["bn"])
    assert lib.bi_geometry_query(9, 8, 64, 100, 2, ctypes.byref(bigemm.BiGeometry())) == SHAPE
    out = ctypes.byref(bigemm.BiGeometry())
    assert lib.bi_geometry_query(3, 8, 64, 64, 0, out) == SHAPE          # no groups
    assert lib.bi_geometry_query(99, 8, 64, 64, 0, out) == UNSUP
    assert lib.bi_geometry_query(0, 8, 64, 64, 0, None) == NULL
    assert lib.bi_geometry_query(0, 0, 64, 64, 0, out) == SHAPE          # nothing launched
    assert lib.bi_geometry_query(4, 8, 64, 100, 0, out) == SHAPE         # fp8 K % 128
    assert lib.bi_geometry_query(6, 8, 63, 64, 0, out) == SHAPE          # fp4 odd N
    assert lib.bi_geometry_query(0, -1, 64, 64, 0, out) == SHAPE
