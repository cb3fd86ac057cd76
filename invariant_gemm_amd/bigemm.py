"""Python binding of libbigemm (ctypes): argument marshalling only.

Every function here forwards device pointers, sizes, row pitches and the
current HIP stream of torch to the C ABI declared in ``include/bigemm.h``;
all arithmetic runs in the library's HIP kernels.  Importing this module
raises if ``libbigemm.so`` is missing -- there is no fallback path.

torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbigemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libbigemm.so not found at {LIB_PATH}; build it first with "
        "`python -m invariant_gemm_amd.build` (hipcc, gfx950)")

lib = ctypes.CDLL(LIB_PATH)

_i64, _vp, _i32, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t

STATUS = {0: "BI_OK", 1: "BI_ERR_NULL", 2: "BI_ERR_SHAPE", 3: "BI_ERR_STRIDE",
          4: "BI_ERR_ALIGN", 5: "BI_ERR_UNSUPPORTED", 6: "BI_ERR_LAUNCH", 7: "BI_ERR_WORKSPACE"}
BI_BF16, BI_FP8_BS, BI_FP4_W, BI_W4A8 = 0, 1, 2, 3


class BiSchedule(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("mfma_m", "mfma_n", "mfma_k", "k_block", "order", "id")]


class BiGeometry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("id", "bm", "bn", "waves", "a_rows", "k_stage", "stages", "reserved")] + \
               [("workgroups", ctypes.c_int64)]


ORDER_SEQUENTIAL, ORDER_BLOCK_FMA = 0, 1
ENTRIES = {"bf16": 0, "bf16_bt": 1, "bf16_packed": 2, "bf16_grouped_packed": 3, "fp8": 4,
           "fp8_packed": 5, "fp4": 6, "fp4_packed": 7, "w4a8_packed": 8, "fp8_grouped_packed": 9,
           "w4a8_grouped_packed": 10}


lib.bi_gemm_bf16.restype = _i32
lib.bi_gemm_bf16.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
lib.bi_gemm_bf16_bt.restype = _i32
lib.bi_gemm_bf16_bt.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
lib.bi_packed_b_bytes.restype = _sz
lib.bi_packed_b_bytes.argtypes = [_i32, _i64, _i64]
lib.bi_pack_b_bf16.restype = _i32
lib.bi_pack_b_bf16.argtypes = [_i64, _i64, _vp, _i64, _vp, _sz, _vp]
lib.bi_gemm_bf16_packed.restype = _i32
lib.bi_gemm_bf16_packed.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _sz, _vp, _i64, _vp]
lib.bi_gemm_fp8_blockscaled.restype = _i32
lib.bi_gemm_fp8_blockscaled.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                        _vp, _i64, _vp]
lib.bi_gemm_fp4_w.restype = _i32
lib.bi_gemm_fp4_w.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
lib.bi_gemm_bf16_grouped_packed.restype = _i32
lib.bi_gemm_bf16_grouped_packed.argtypes = [_i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _sz, _vp,
                                            _i64, _vp]
lib.bi_pack_b_mxfp4.restype = _i32
lib.bi_pack_b_mxfp4.argtypes = [_i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]
lib.bi_gemm_w4a8_packed.restype = _i32
lib.bi_gemm_w4a8_packed.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp, _i64, _vp]
lib.bi_gemm_w4a8_grouped_packed.restype = _i32
lib.bi_gemm_w4a8_grouped_packed.argtypes = [_i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp,
                                            _sz, _vp, _i64, _vp]
lib.bi_pack_b_fp8.restype = _i32
lib.bi_pack_b_fp8.argtypes = [_i64, _i64, _vp, _i64, _vp, _sz, _vp]
lib.bi_gemm_fp8_blockscaled_packed.restype = _i32
lib.bi_gemm_fp8_blockscaled_packed.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz,
                                               _vp, _i64, _vp, _i64, _vp]
lib.bi_gemm_fp8_blockscaled_grouped_packed.restype = _i32
lib.bi_gemm_fp8_blockscaled_grouped_packed.argtypes = [_i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp,
                                                       _i64, _vp, _sz, _vp, _i64, _vp, _i64, _vp]
lib.bi_pack_b_fp4.restype = _i32
lib.bi_pack_b_fp4.argtypes = [_i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]
lib.bi_gemm_fp4_w_packed.restype = _i32
lib.bi_gemm_fp4_w_packed.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _sz, _vp, _i64, _vp]
lib.bi_gemm_bf16_splitk.restype = _i32
lib.bi_gemm_bf16_splitk.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz,
                                    _i32, _vp]
lib.bi_splitk_choose.restype = _i32
lib.bi_splitk_choose.argtypes = [_i64, _i64, _i64]
lib.bi_schedule_query.restype = _i32
lib.bi_schedule_query.argtypes = [_i32, _i64, _i64, ctypes.POINTER(BiSchedule)]
lib.bi_decode_attention_bf16_noalloc.restype = _i32
lib.bi_decode_attention_bf16_noalloc.argtypes = [_i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp,
                                                 ctypes.c_float, _vp, _i32, _vp]
lib.bi_probe_stream_read.restype = _i32
lib.bi_probe_stream_read.argtypes = [_vp, _sz, _i32, _i32, _vp, _vp]
lib.bi_probe_empty.restype = _i32
lib.bi_probe_empty.argtypes = [_vp]
lib.bi_geometry_query.restype = _i32
lib.bi_geometry_query.argtypes = [_i32, _i64, _i64, _i64, _i64, ctypes.POINTER(BiGeometry)]
lib.bi_status_str.restype = ctypes.c_char_p
lib.bi_status_str.argtypes = [_i32]
lib.bi_version.restype = ctypes.c_char_p
lib.bi_version.argtypes = []
lib.bi_decode_attention_workspace_bytes.restype = _sz
lib.bi_decode_attention_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
lib.bi_decode_attention_choice.restype = _i32
lib.bi_decode_attention_choice.argtypes = [_i64, _i64, _i64, _i64]
lib.bi_decode_attention_bf16.restype = _i32
lib.bi_decode_attention_bf16.argtypes = [_i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp,
                                         ctypes.c_float, _vp, _vp, _sz, _i32, _vp]


class BigemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.bi_status_str(status).decode()}")


def _check(status: int, what: str):
    if status != 0:
        raise BigemmError(status, what)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _mat(t: torch.Tensor, dtypes, name: str) -> torch.Tensor:
    if t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D tensor, got shape {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.numel() and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: rows must be contiguous (stride(1) == 1)")
    return t


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8, torch.float8_e4m3fn, torch.int8)


def version() -> str:
    return lib.bi_version().decode()


def schedule(dtype: int, N: int, K: int) -> dict:
    s = BiSchedule()
    _check(lib.bi_schedule_query(dtype, N, K, ctypes.byref(s)), "bi_schedule_query")
    return {n: getattr(s, n) for n, _ in BiSchedule._fields_}


def geometry(entry: str, M: int, N: int, K: int, groups: int = 0) -> dict:
    """The launch geometry `entry` uses at M x N x K (informational: no
    geometry changes a result)."""
    g = BiGeometry()
    _check(lib.bi_geometry_query(ENTRIES[entry], M, N, K, groups, ctypes.byref(g)),
           "bi_geometry_query")
    return {n: getattr(g, n) for n, _ in BiGeometry._fields_ if n != "reserved"}


def _out(M, N, device, out):
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device)
    out = _mat(out, _BF16, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out: expected shape {(M, N)}, got {tuple(out.shape)}")
    _same_device(device, out=out)
    return out


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t.device != device:
            raise ValueError(f"{name}: on {t.device}, expected {device}")


def _shape(t: torch.Tensor, shape, name: str):
    """The C ABI sees pointers and pitches only, so every operand's extent is
    checked here: a short tensor would otherwise be read or written past its end."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _blocks(K: int, blk: int, what: str) -> int:
    if K % blk:
        raise ValueError(f"{what}: K = {K} is not a multiple of {blk}")
    return K // blk


def gemm_bf16(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . B (bf16 in/out) via bi_gemm_bf16 on torch's current stream."""
    A = _mat(A, _BF16, "A")
    B = _mat(B, _BF16, "B")
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError("A and B inner dimensions differ")
    N = B.shape[1]
    _same_device(A.device, B=B)
    C = _out(M, N, A.device, out)
    _check(lib.bi_gemm_bf16(M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B),
                            C.data_ptr(), _ld(C), _stream()), "bi_gemm_bf16")
    return C


def gemm_bf16_bt(A: torch.Tensor, Bt: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . Bt^T with the weights stored transposed (Bt [N,K]) via bi_gemm_bf16_bt."""
    A = _mat(A, _BF16, "A")
    Bt = _mat(Bt, _BF16, "Bt")
    M, K = A.shape
    if Bt.shape[1] != K:
        raise ValueError("A and Bt inner dimensions differ")
    N = Bt.shape[0]
    _same_device(A.device, Bt=Bt)
    C = _out(M, N, A.device, out)
    _check(lib.bi_gemm_bf16_bt(M, N, K, A.data_ptr(), _ld(A), Bt.data_ptr(), _ld(Bt),
                               C.data_ptr(), _ld(C), _stream()), "bi_gemm_bf16_bt")
    return C


class PackedWeights:
    """A weight matrix in the library's MFMA-ordered packed layout (device bytes)."""

    def __init__(self, dtype: int, K: int, N: int, data: torch.Tensor, extra=None):
        self.dtype, self.K, self.N, self.data, self.extra = dtype, K, N, data, extra


def packed_b_bytes(dtype: int, N: int, K: int) -> int:
    return int(lib.bi_packed_b_bytes(dtype, N, K))


def pack_b_bf16(B: torch.Tensor) -> PackedWeights:
    """Pack row-major bf16 B [K,N] once (one kernel on the current stream)."""
    B = _mat(B, _BF16, "B")
    K, N = B.shape
    nbytes = packed_b_bytes(BI_BF16, N, K)
    buf = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=B.device)
    _check(lib.bi_pack_b_bf16(N, K, B.data_ptr(), _ld(B), buf.data_ptr(), buf.numel(), _stream()),
           "bi_pack_b_bf16")
    return PackedWeights(BI_BF16, K, N, buf)


def gemm_bf16_packed(A: torch.Tensor, Bp: PackedWeights, out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . B with B packed by pack_b_bf16 (identical bits to gemm_bf16)."""
    A = _mat(A, _BF16, "A")
    M, K = A.shape
    if Bp.dtype != BI_BF16 or Bp.K != K:
        raise ValueError("packed weights do not match A")
    _same_device(A.device, Bp=Bp.data)
    C = _out(M, Bp.N, A.device, out)
    _check(lib.bi_gemm_bf16_packed(M, Bp.N, K, A.data_ptr(), _ld(A), Bp.data.data_ptr(),
                                   Bp.data.numel(), C.data_ptr(), _ld(C), _stream()),
           "bi_gemm_bf16_packed")
    return C


def pack_b_bf16_grouped(Bs) -> PackedWeights:
    """Pack G row-major bf16 matrices [K,N] (one per group) back to back."""
    Bs = [_mat(B, _BF16, "B") for B in Bs]
    K, N = Bs[0].shape
    if any(tuple(B.shape) != (K, N) for B in Bs):
        raise ValueError("all groups' weight matrices must have the same shape")
    one = packed_b_bytes(BI_BF16, N, K)
    buf = torch.empty(max(one * len(Bs), 16), dtype=torch.uint8, device=Bs[0].device)
    for g, B in enumerate(Bs):
        _check(lib.bi_pack_b_bf16(N, K, B.data_ptr(), _ld(B), buf.data_ptr() + g * one, one, _stream()),
               "bi_pack_b_bf16")
    pw = PackedWeights(BI_BF16, K, N, buf)
    pw.groups = len(Bs)
    return pw


def gemm_bf16_grouped_packed(A: torch.Tensor, offsets: torch.Tensor, Bp: PackedWeights,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows [offsets[g], offsets[g+1]) of A times group g's packed weights."""
    A = _mat(A, _BF16, "A")
    M, K = A.shape
    if Bp.dtype != BI_BF16 or Bp.K != K or not hasattr(Bp, "groups"):
        raise ValueError("grouped packed weights do not match A")
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.dim() != 1 \
            or offsets.numel() != Bp.groups + 1 or (offsets.numel() > 1 and offsets.stride(0) != 1):
        raise ValueError("offsets: a contiguous int32 device tensor of G + 1 entries")
    _same_device(A.device, Bp=Bp.data, offsets=offsets)
    C = _out(M, Bp.N, A.device, out)
    _check(lib.bi_gemm_bf16_grouped_packed(Bp.groups, offsets.data_ptr(), M, Bp.N, K, A.data_ptr(),
                                           _ld(A), Bp.data.data_ptr(), Bp.data.numel(),
                                           C.data_ptr(), _ld(C), _stream()),
           "bi_gemm_bf16_grouped_packed")
    return C


def gemm_fp8_blockscaled(A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """C = (A * sA) . (B * sB) with e4m3fn codes and fp32 1x128 / 128x128 scales."""
    A = _mat(A, _U8, "A")
    B = _mat(B, _U8, "B")
    sA = _mat(sA, (torch.float32,), "sA")
    sB = _mat(sB, (torch.float32,), "sB")
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError("A and B inner dimensions differ")
    N = B.shape[1]
    kb = _blocks(K, 128, "gemm_fp8_blockscaled")
    _shape(sA, (M, kb), "sA")
    _shape(sB, (kb, (N + 127) // 128), "sB")
    _same_device(A.device, sA=sA, B=B, sB=sB)
    C = _out(M, N, A.device, out)
    _check(lib.bi_gemm_fp8_blockscaled(M, N, K, A.data_ptr(), _ld(A), sA.data_ptr(), _ld(sA),
                                       B.data_ptr(), _ld(B), sB.data_ptr(), _ld(sB),
                                       C.data_ptr(), _ld(C), _stream()), "bi_gemm_fp8_blockscaled")
    return C


def gemm_fp4_w(A: torch.Tensor, Bq: torch.Tensor, sB: torch.Tensor, N: int,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . dequant(Bq, sB): bf16 activations, packed e2m1 weights, e4m3fn scales per 32 K."""
    A = _mat(A, _BF16, "A")
    Bq = _mat(Bq, _U8, "Bq")
    sB = _mat(sB, _U8, "sB")
    M, K = A.shape
    if Bq.shape[0] != K:
        raise ValueError("A and Bq inner dimensions differ")
    if N % 2:
        raise ValueError(f"gemm_fp4_w: N = {N} must be even")
    _shape(Bq, (K, N // 2), "Bq")
    _shape(sB, (_blocks(K, 32, "gemm_fp4_w"), N), "sB")
    _same_device(A.device, Bq=Bq, sB=sB)
    C = _out(M, N, A.device, out)
    _check(lib.bi_gemm_fp4_w(M, N, K, A.data_ptr(), _ld(A), Bq.data_ptr(), _ld(Bq),
                             sB.data_ptr(), _ld(sB), C.data_ptr(), _ld(C), _stream()),
           "bi_gemm_fp4_w")
    return C


def pack_b_fp8(B: torch.Tensor) -> PackedWeights:
    """Pack row-major e4m3fn B [K,N] once (the scales sB stay as they are)."""
    B = _mat(B, _U8, "B")
    K, N = B.shape
    nbytes = packed_b_bytes(BI_FP8_BS, N, K)
    buf = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=B.device)
    _check(lib.bi_pack_b_fp8(N, K, B.data_ptr(), _ld(B), buf.data_ptr(), buf.numel(), _stream()),
           "bi_pack_b_fp8")
    return PackedWeights(BI_FP8_BS, K, N, buf)


def gemm_fp8_blockscaled_packed(A: torch.Tensor, sA: torch.Tensor, Bp: PackedWeights,
                                sB: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_fp8_blockscaled with B packed by pack_b_fp8 (identical bits)."""
    A = _mat(A, _U8, "A")
    sA = _mat(sA, (torch.float32,), "sA")
    sB = _mat(sB, (torch.float32,), "sB")
    M, K = A.shape
    if Bp.dtype != BI_FP8_BS or Bp.K != K:
        raise ValueError("packed weights do not match A")
    kb = _blocks(K, 128, "gemm_fp8_blockscaled_packed")
    _shape(sA, (M, kb), "sA")
    _shape(sB, (kb, (Bp.N + 127) // 128), "sB")
    _same_device(A.device, sA=sA, Bp=Bp.data, sB=sB)
    C = _out(M, Bp.N, A.device, out)
    _check(lib.bi_gemm_fp8_blockscaled_packed(M, Bp.N, K, A.data_ptr(), _ld(A), sA.data_ptr(),
                                              _ld(sA), Bp.data.data_ptr(), Bp.data.numel(),
                                              sB.data_ptr(), _ld(sB), C.data_ptr(), _ld(C),
                                              _stream()), "bi_gemm_fp8_blockscaled_packed")
    return C


def pack_b_fp8_grouped(Bs) -> PackedWeights:
    """Pack G row-major e4m3fn matrices [K,N] (one per expert) back to back."""
    Bs = [_mat(B, _U8, "B") for B in Bs]
    K, N = Bs[0].shape
    if any(tuple(B.shape) != (K, N) for B in Bs):
        raise ValueError("all experts' weight matrices must have the same shape")
    one = packed_b_bytes(BI_FP8_BS, N, K)
    buf = torch.empty(max(one * len(Bs), 16), dtype=torch.uint8, device=Bs[0].device)
    for g, B in enumerate(Bs):
        _check(lib.bi_pack_b_fp8(N, K, B.data_ptr(), _ld(B), buf.data_ptr() + g * one, one, _stream()),
               "bi_pack_b_fp8")
    pw = PackedWeights(BI_FP8_BS, K, N, buf)
    pw.groups = len(Bs)
    return pw


def gemm_fp8_blockscaled_grouped_packed(A: torch.Tensor, sA: torch.Tensor, offsets: torch.Tensor,
                                        Bp: PackedWeights, sB: torch.Tensor,
                                        out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows [offsets[g], offsets[g+1]) of (A, sA) times expert g's packed fp8
    weights and scales; sB holds the G scale matrices stacked: [G*K/128, ceil(N/128)]."""
    A = _mat(A, _U8, "A")
    sA = _mat(sA, (torch.float32,), "sA")
    sB = _mat(sB, (torch.float32,), "sB")
    M, K = A.shape
    if Bp.dtype != BI_FP8_BS or Bp.K != K or not hasattr(Bp, "groups"):
        raise ValueError("grouped packed fp8 weights do not match A")
    kb = _blocks(K, 128, "gemm_fp8_blockscaled_grouped_packed")
    _shape(sA, (M, kb), "sA")
    _shape(sB, (Bp.groups * kb, (Bp.N + 127) // 128), "sB")
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.dim() != 1 \
            or offsets.numel() != Bp.groups + 1 or (offsets.numel() > 1 and offsets.stride(0) != 1):
        raise ValueError("offsets: a contiguous int32 device tensor of G + 1 entries")
    _same_device(A.device, sA=sA, Bp=Bp.data, sB=sB, offsets=offsets)
    C = _out(M, Bp.N, A.device, out)
    _check(lib.bi_gemm_fp8_blockscaled_grouped_packed(
        Bp.groups, offsets.data_ptr(), M, Bp.N, K, A.data_ptr(), _ld(A), sA.data_ptr(), _ld(sA),
        Bp.data.data_ptr(), Bp.data.numel(), sB.data_ptr(), _ld(sB), C.data_ptr(), _ld(C), _stream()),
        "bi_gemm_fp8_blockscaled_grouped_packed")
    return C


def pack_b_fp4(Bq: torch.Tensor, sB: torch.Tensor, N: int) -> PackedWeights:
    """Pack e2m1 codes Bq [K, N/2] and e4m3fn scales sB [K/32, N] once."""
    Bq = _mat(Bq, _U8, "Bq")
    sB = _mat(sB, _U8, "sB")
    K = Bq.shape[0]
    if N % 2:
        raise ValueError(f"pack_b_fp4: N = {N} must be even")
    _shape(Bq, (K, N // 2), "Bq")
    _shape(sB, (_blocks(K, 32, "pack_b_fp4"), N), "sB")
    _same_device(Bq.device, sB=sB)
    nbytes = packed_b_bytes(BI_FP4_W, N, K)
    buf = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=Bq.device)
    _check(lib.bi_pack_b_fp4(N, K, Bq.data_ptr(), _ld(Bq), sB.data_ptr(), _ld(sB),
                             buf.data_ptr(), buf.numel(), _stream()), "bi_pack_b_fp4")
    return PackedWeights(BI_FP4_W, K, N, buf)


def gemm_fp4_w_packed(A: torch.Tensor, Bp: PackedWeights, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_fp4_w with codes and scales packed by pack_b_fp4 (identical bits)."""
    A = _mat(A, _BF16, "A")
    M, K = A.shape
    if Bp.dtype != BI_FP4_W or Bp.K != K:
        raise ValueError("packed weights do not match A")
    _same_device(A.device, Bp=Bp.data)
    C = _out(M, Bp.N, A.device, out)
    _check(lib.bi_gemm_fp4_w_packed(M, Bp.N, K, A.data_ptr(), _ld(A), Bp.data.data_ptr(),
                                    Bp.data.numel(), C.data_ptr(), _ld(C), _stream()),
           "bi_gemm_fp4_w_packed")
    return C


def pack_b_mxfp4(Bq: torch.Tensor, sE: torch.Tensor, N: int) -> PackedWeights:
    """Pack OCP MXFP4 weights: e2m1 codes Bq [K, N/2] and E8M0 scales sE [K/32, N]."""
    Bq = _mat(Bq, _U8, "Bq")
    sE = _mat(sE, _U8 + (getattr(torch, "float8_e8m0fnu", torch.uint8),), "sE")
    K = Bq.shape[0]
    if N % 2:
        raise ValueError(f"pack_b_mxfp4: N = {N} must be even")
    _shape(Bq, (K, N // 2), "Bq")
    _shape(sE, (_blocks(K, 32, "pack_b_mxfp4"), N), "sE")
    _same_device(Bq.device, sE=sE)
    nbytes = packed_b_bytes(BI_W4A8, N, K)
    buf = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=Bq.device)
    _check(lib.bi_pack_b_mxfp4(N, K, Bq.data_ptr(), _ld(Bq), sE.data_ptr(), _ld(sE),
                               buf.data_ptr(), buf.numel(), _stream()), "bi_pack_b_mxfp4")
    return PackedWeights(BI_W4A8, K, N, buf)


def gemm_w4a8_packed(A: torch.Tensor, sA: torch.Tensor, Bp: PackedWeights,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """C = (A * sA) . MXFP4(B): e4m3fn activations with 1x128 fp32 scales, packed MXFP4 weights."""
    A = _mat(A, _U8, "A")
    sA = _mat(sA, (torch.float32,), "sA")
    M, K = A.shape
    if Bp.dtype != BI_W4A8 or Bp.K != K:
        raise ValueError("packed weights do not match A")
    _shape(sA, (M, _blocks(K, 128, "gemm_w4a8_packed")), "sA")
    _same_device(A.device, sA=sA, Bp=Bp.data)
    C = _out(M, Bp.N, A.device, out)
    _check(lib.bi_gemm_w4a8_packed(M, Bp.N, K, A.data_ptr(), _ld(A), sA.data_ptr(), _ld(sA),
                                   Bp.data.data_ptr(), Bp.data.numel(), C.data_ptr(), _ld(C),
                                   _stream()), "bi_gemm_w4a8_packed")
    return C


def pack_b_mxfp4_grouped(Bqs, sEs, N: int) -> PackedWeights:
    """Pack G experts' OCP MXFP4 weights (codes Bq [K, N/2], E8M0 scales
    sE [K/32, N] each) back to back, one bi_pack_b_mxfp4 layout per expert."""
    if len(Bqs) != len(sEs) or not Bqs:
        raise ValueError("pack_b_mxfp4_grouped: one scale matrix per code matrix, at least one expert")
    parts = [pack_b_mxfp4(Bq, sE, N) for Bq, sE in zip(Bqs, sEs)]
    K = parts[0].K
    if any(p.K != K for p in parts):
        raise ValueError("all experts' weight matrices must have the same shape")
    one = packed_b_bytes(BI_W4A8, N, K)
    buf = torch.empty(max(one * len(parts), 16), dtype=torch.uint8, device=parts[0].data.device)
    for g, p in enumerate(parts):
        buf[g * one:(g + 1) * one].copy_(p.data[:one])
    pw = PackedWeights(BI_W4A8, K, N, buf)
    pw.groups = len(parts)
    return pw


def gemm_w4a8_grouped_packed(A: torch.Tensor, sA: torch.Tensor, offsets: torch.Tensor,
                             Bp: PackedWeights, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows [offsets[g], offsets[g+1]) of (A, sA) times expert g's packed MXFP4 weights
    (pack_b_mxfp4_grouped), via bi_gemm_w4a8_grouped_packed."""
    A = _mat(A, _U8, "A")
    sA = _mat(sA, (torch.float32,), "sA")
    M, K = A.shape
    if Bp.dtype != BI_W4A8 or Bp.K != K or not hasattr(Bp, "groups"):
        raise ValueError("grouped packed MXFP4 weights do not match A")
    _shape(sA, (M, _blocks(K, 128, "gemm_w4a8_grouped_packed")), "sA")
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.dim() != 1 \
            or offsets.numel() != Bp.groups + 1 or (offsets.numel() > 1 and offsets.stride(0) != 1):
        raise ValueError("offsets: a contiguous int32 device tensor of G + 1 entries")
    _same_device(A.device, sA=sA, Bp=Bp.data, offsets=offsets)
    C = _out(M, Bp.N, A.device, out)
    _check(lib.bi_gemm_w4a8_grouped_packed(
        Bp.groups, offsets.data_ptr(), M, Bp.N, K, A.data_ptr(), _ld(A), sA.data_ptr(), _ld(sA),
        Bp.data.data_ptr(), Bp.data.numel(), C.data_ptr(), _ld(C), _stream()),
        "bi_gemm_w4a8_grouped_packed")
    return C


def splitk_choose(M: int, N: int, K: int) -> int:
    return int(lib.bi_splitk_choose(M, N, K))


def gemm_bf16_splitk(A: torch.Tensor, B: torch.Tensor, workspace: torch.Tensor, splits: int = 0,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """NOT batch-invariant: the split-K comparator (fp32 atomics into `workspace`)."""
    A = _mat(A, _BF16, "A")
    B = _mat(B, _BF16, "B")
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError("A and B inner dimensions differ")
    N = B.shape[1]
    if workspace.dtype != torch.float32 or not workspace.is_cuda:
        raise TypeError("workspace must be a float32 device tensor")
    _same_device(A.device, B=B, workspace=workspace)
    C = _out(M, N, A.device, out)
    _check(lib.bi_gemm_bf16_splitk(M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B),
                                   C.data_ptr(), _ld(C), workspace.data_ptr(),
                                   workspace.numel() * 4, splits, _stream()), "bi_gemm_bf16_splitk")
    return C


# ----------------------------------------------------------- decode attention

ATTN_AUTO, ATTN_SINGLE, ATTN_SPLIT = 0, 1, 2
_ATTN_KERNELS = {"auto": ATTN_AUTO, "single": ATTN_SINGLE, "split": ATTN_SPLIT}


def decode_attention_workspace_bytes(B: int, Hq: int, Hkv: int, Lmax: int) -> int:
    return int(lib.bi_decode_attention_workspace_bytes(B, Hq, Hkv, Lmax))


def decode_attention_choice(B: int, Hq: int, Hkv: int, Lmax: int) -> str:
    k = int(lib.bi_decode_attention_choice(B, Hq, Hkv, Lmax))
    return {ATTN_SINGLE: "single", ATTN_SPLIT: "split"}[k]


def decode_attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, seq_lens: torch.Tensor,
                     scale: float, kernel: str = "auto", workspace: torch.Tensor | None = None,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """Batch-invariant decode attention via bi_decode_attention_bf16.

    Q [B,Hq,128] bf16; K, V [B,Hkv,Lmax,128] bf16 (contiguous); seq_lens int32 [B]
    on the device.  kernel: "auto", "single" or "split" (identical results).
    A workspace is allocated here when none is given and the split kernel may run."""
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if t.dtype not in _BF16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name}: expected a contiguous bf16 device tensor")
    if Q.dim() != 3 or K.dim() != 4 or V.shape != K.shape:
        raise ValueError("Q [B,Hq,D], K and V [B,Hkv,Lmax,D]")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_cuda or seq_lens.dim() != 1:
        raise TypeError("seq_lens: int32 device vector")
    B, Hq, D = Q.shape
    Hkv, Lmax = K.shape[1], K.shape[2]
    if K.shape[0] != B or K.shape[3] != D:
        raise ValueError(f"K, V: expected [{B}, Hkv, Lmax, {D}], got {tuple(K.shape)}")
    _shape(seq_lens, (B,), "seq_lens")
    _same_device(Q.device, K=K, V=V, seq_lens=seq_lens)
    k = _ATTN_KERNELS[kernel]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=Q.device)
    elif out.dtype not in _BF16 or not out.is_contiguous() or tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"out: expected a contiguous bf16 tensor of shape {(B, Hq, D)}")
    else:
        _same_device(Q.device, out=out)
    need = decode_attention_workspace_bytes(B, Hq, Hkv, Lmax)
    if workspace is None and k != ATTN_SINGLE and need:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=Q.device)
    if workspace is not None:
        if not workspace.is_contiguous():
            raise ValueError("workspace: must be contiguous")
        _same_device(Q.device, workspace=workspace)
    wp, wb = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) \
        if workspace is not None else (None, 0)
    _check(lib.bi_decode_attention_bf16(B, Hq, Hkv, D, Lmax, Q.data_ptr(), K.data_ptr(),
                                        V.data_ptr(), seq_lens.data_ptr(), float(scale),
                                        out.data_ptr(), wp, wb, k, _stream()),
           "bi_decode_attention_bf16")
    return out


ATTN_SCRATCH_BYTES = 16 << 20      # BI_ATTN_SCRATCH_BYTES


def decode_attention_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                             seq_lens: torch.Tensor, scale: float, out: torch.Tensor,
                             kernel: str = "auto") -> torch.Tensor:
    """bi_decode_attention_bf16_noalloc: the same results as decode_attention,
    with the split-KV states in the library's fixed per-GPU scratch array.
    Nothing is allocated: the caller passes the output tensor."""
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if t.dtype not in _BF16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name}: expected a contiguous bf16 device tensor")
    if Q.dim() != 3 or K.dim() != 4 or V.shape != K.shape:
        raise ValueError("Q [B,Hq,D], K and V [B,Hkv,Lmax,D]")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_cuda or seq_lens.dim() != 1:
        raise TypeError("seq_lens: int32 device vector")
    B, Hq, D = Q.shape
    Hkv, Lmax = K.shape[1], K.shape[2]
    if K.shape[0] != B or K.shape[3] != D:
        raise ValueError(f"K, V: expected [{B}, Hkv, Lmax, {D}], got {tuple(K.shape)}")
    _shape(seq_lens, (B,), "seq_lens")
    if out.dtype not in _BF16 or not out.is_contiguous() or tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"out: expected a contiguous bf16 tensor of shape {(B, Hq, D)}")
    _same_device(Q.device, K=K, V=V, seq_lens=seq_lens, out=out)
    _check(lib.bi_decode_attention_bf16_noalloc(B, Hq, Hkv, D, Lmax, Q.data_ptr(), K.data_ptr(),
                                                V.data_ptr(), seq_lens.data_ptr(), float(scale),
                                                out.data_ptr(), _ATTN_KERNELS[kernel], _stream()),
           "bi_decode_attention_bf16_noalloc")
    return out


PROBE_NONTEMPORAL, PROBE_UNROLL8 = 1, 2


def probe_stream_read(buf: torch.Tensor, workgroups: int, flags: int, out: torch.Tensor) -> None:
    """bi_probe_stream_read: read every byte of `buf` once (measurement only)."""
    if not buf.is_cuda or not buf.is_contiguous() or not out.is_cuda or out.dtype != torch.int32 \
            or out.numel() < workgroups * 256:
        raise ValueError("probe_stream_read: contiguous device buffer, int32 out of workgroups*256")
    _check(lib.bi_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), workgroups,
                                    flags, out.data_ptr(), _stream()), "bi_probe_stream_read")


def probe_empty() -> None:
    """bi_probe_empty: one empty kernel on the current stream."""
    _check(lib.bi_probe_empty(_stream()), "bi_probe_empty")
