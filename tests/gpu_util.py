"""Helpers for the GPU tests: host<->device moves of raw codes, the parity
bounds, and row-bitwise comparison.  No GEMM arithmetic lives here."""
import numpy as np
import torch

from invariant_gemm_amd import inputs


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return torch.device("cuda:0")


def dev_bf16(codes: np.ndarray, ld: int | None = None) -> torch.Tensor:
    """uint16 bf16 codes [R, C] -> device bf16 tensor, optionally with a wider row pitch."""
    R, Cn = codes.shape
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(torch.bfloat16)
    if ld is None or ld == Cn:
        return t.cuda()
    buf = torch.zeros((R, ld), dtype=torch.bfloat16)
    buf[:, :Cn] = t
    return buf.cuda()[:, :Cn]


def dev_u8(codes: np.ndarray, ld: int | None = None) -> torch.Tensor:
    R, Cn = codes.shape
    t = torch.from_numpy(np.ascontiguousarray(codes))
    if ld is None or ld == Cn:
        return t.cuda()
    buf = torch.zeros((R, ld), dtype=torch.uint8)
    buf[:, :Cn] = t
    return buf.cuda()[:, :Cn]


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_codes(t: torch.Tensor) -> np.ndarray:
    """device bf16 tensor -> uint16 codes."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_vals(codes: np.ndarray) -> np.ndarray:
    return inputs.bf16_codes_to_f32(codes).astype(np.float64)


def check_parity(C_codes: np.ndarray, C64: np.ndarray, S: np.ndarray, K: int, what: str = ""):
    """Parity tolerance |err| <= 2^-7 S + 1e-6 and the tight diagnostic bound
    |err| <= 2^-8 |C64| + K 2^-23 S + 1e-6, on every element; finite outputs only."""
    got = bf16_vals(C_codes)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - C64)
    tol = 2.0**-7 * S + 1e-6
    tight = 2.0**-8 * np.abs(C64) + K * 2.0**-23 * S + 1e-6
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond the tolerance, worst at {np.argwhere(bad)[0]}"
    bad = err > tight
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond the tight bound, worst at {np.argwhere(bad)[0]}"
    rms = np.sqrt(np.mean(err**2)) / max(np.sqrt(np.mean(C64**2)), 1e-300)
    return {"max_err_over_tol": float((err / tol).max()), "rel_rms": float(rms)}


def rows_equal(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """Per-row bitwise equality of two bf16 matrices (as int16)."""
    return (a.view(torch.int16) == b.view(torch.int16)).all(dim=1)
