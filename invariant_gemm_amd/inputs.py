"""Seeded synthetic inputs and the quantisers that produce the library's operand formats.

This module holds no GEMM arithmetic.  It draws seeded normal samples
(numpy ``Generator(PCG64(seed))``), rounds them to bf16, and encodes them into
the block-scaled fp8 / fp4 formats the library consumes.  Both the HIP path
and the fp64 oracle consume exactly the codes produced here, so a quantiser
choice never affects parity.

Quantiser rules (the pages fix none; these are the plainest choices):

* fp8 e4m3fn, block of ``(rows x 128)``: ``s = amax / 448`` in fp32 (``s = 1``
  for an all-zero block), ``q = e4m3fn(RNE(clamp(x / s, +-448)))``.
* fp4 e2m1 weight-only, block of 32 along K per column: ``s = e4m3fn(RNE(amax / 6))``
  (raised to the smallest subnormal, code 0x01, if that rounds to zero while
  ``amax > 0``), ``q = e2m1(RNE(clamp(w / dec(s), +-6)))``.  Codes are packed two
  per byte along N: byte ``j`` of row ``k`` holds column ``2j`` in its low nibble
  and column ``2j+1`` in its high nibble.
"""
from __future__ import annotations

import numpy as np
import torch

# ------------------------------------------------------------------ sampling


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(shape, sigma: float, seed: int) -> np.ndarray:
    """fp32 samples of N(0, sigma^2)."""
    x = rng(seed).standard_normal(size=shape, dtype=np.float32)
    return (x * np.float32(sigma)).astype(np.float32)


def f32_to_bf16_codes(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 (RNE, torch CPU) and return the uint16 codes."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_codes_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, sigma: float, seed: int) -> np.ndarray:
    """uint16 bf16 codes of N(0, sigma^2) samples."""
    return f32_to_bf16_codes(normal_f32(shape, sigma, seed))


# ------------------------------------------------------------------ fp8 e4m3fn

E4M3_MAX = 448.0


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> e4m3fn codes, RNE, saturating at +-448 (torch CPU conversion)."""
    x = np.clip(np.asarray(x, np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _e4m3_values(q: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(q, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def quant_fp8_rowblocks(x: np.ndarray, block_k: int = 128):
    """Activations [M,K] -> (q uint8 [M,K], s fp32 [M, K/block_k]), one scale per 1 x block_k."""
    M, K = x.shape
    assert K % block_k == 0
    xb = x.reshape(M, K // block_k, block_k).astype(np.float32)
    amax = np.abs(xb).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = _e4m3_codes(xb / s[:, :, None]).reshape(M, K)
    return q, s


def quant_fp8_tiles(w: np.ndarray, block: int = 128):
    """Weights [K,N] -> (q uint8 [K,N], s fp32 [K/block, ceil(N/block)]), one scale per block x block."""
    K, N = w.shape
    assert K % block == 0
    nb = (N + block - 1) // block
    wp = np.zeros((K, nb * block), np.float32)
    wp[:, :N] = w
    wb = wp.reshape(K // block, block, nb, block)
    amax = np.abs(wb).max(axis=(1, 3))
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = _e4m3_codes(wb / s[:, None, :, None]).reshape(K, nb * block)[:, :N]
    return np.ascontiguousarray(q), s


# ------------------------------------------------------------------ fp4 e2m1

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)


def _e2m1_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> e2m1 codes (0..15), RNE with ties to the even mantissa, saturating at +-6."""
    a = np.abs(x).astype(np.float32)
    idx = np.zeros(a.shape, np.uint8)
    # midpoint between magnitude j and j+1; at an exact tie go to the even code index
    for j in range(7):
        mid = (E2M1_MAG[j] + E2M1_MAG[j + 1]) / 2
        up = (a > mid) | ((a == mid) & (j % 2 == 1))
        idx = np.where(up, np.uint8(j + 1), idx)
    sign = (np.signbit(x) & (idx > 0)).astype(np.uint8)
    return (idx | (sign << 3)).astype(np.uint8)


def quant_fp4_weights(w: np.ndarray, block_k: int = 32):
    """Weights [K,N] -> (Bq uint8 [K, N/2] packed, sB uint8 e4m3fn [K/block_k, N])."""
    K, N = w.shape
    assert K % block_k == 0 and N % 2 == 0
    wb = w.reshape(K // block_k, block_k, N).astype(np.float32)
    amax = np.abs(wb).max(axis=1)                       # [K/32, N]
    sc = _e4m3_codes(amax / np.float32(6.0))
    sc = np.where((sc == 0) & (amax > 0), np.uint8(1), sc).astype(np.uint8)
    sv = _e4m3_values(sc)
    sv_safe = np.where(sv > 0, sv, np.float32(1.0))
    codes = _e2m1_codes(np.clip(wb / sv_safe[:, None, :], -6.0, 6.0)).reshape(K, N)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(sc)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """Packed [K, N/2] -> codes [K, N] (low nibble = even column)."""
    K, H = packed.shape
    out = np.empty((K, 2 * H), np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out


# ------------------------------------------------------------------ batch compositions


def permutation(n: int, seed: int) -> np.ndarray:
    return rng(seed).permutation(n)


def random_subsets(pool: int, size: int, count: int, seed: int):
    g = rng(seed)
    return [g.choice(pool, size=size, replace=False) for _ in range(count)]


def replay_batches(pool: int, steps: int, max_batch: int, seed: int):
    """Dynamic-batching replay: each step draws b ~ U{1..max_batch} distinct rows in random order."""
    g = rng(seed)
    out = []
    for _ in range(steps):
        b = int(g.integers(1, max_batch + 1))
        out.append(g.choice(pool, size=b, replace=False))
    return out


def route_tokens(n_tokens: int, n_experts: int, seed: int, skew: float = 0.0) -> np.ndarray:
    """Expert id per token for a synthetic top-1 routing: probabilities
    proportional to (rank + 1)^-skew over a seeded random expert order
    (skew 0 = uniform; large skew piles most tokens onto a few experts)."""
    g = rng(seed)
    w = (np.arange(n_experts) + 1.0) ** -skew
    p = w[g.permutation(n_experts)]
    return g.choice(n_experts, size=n_tokens, p=p / p.sum())


def group_by_expert(expert: np.ndarray, n_experts: int):
    """Stable order of the tokens by expert and the row offsets per expert."""
    order = np.argsort(expert, kind="stable")
    counts = np.bincount(expert, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return order, offsets


def quant_mxfp4_weights(w: np.ndarray, block_k: int = 32):
    """Weights [K,N] -> (Bq uint8 [K, N/2] packed e2m1, sE uint8 E8M0 [K/block_k, N]),
    the OCP MX scheme: per block of 32 along K and column, the shared scale is
    2^(floor(log2(amax)) - 2) (2 = the largest e2m1 exponent), clamped to the
    E8M0 range (1 for an all-zero block); codes are RNE e2m1 of w / scale,
    saturating at +-6."""
    K, N = w.shape
    wb = w.reshape(K // block_k, block_k, N).astype(np.float32)
    amax = np.abs(wb).max(axis=1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    e = np.clip(e, -127, 127).astype(np.int32)
    scale = np.ldexp(np.float32(1.0), e).astype(np.float32)
    codes = _e2m1_codes((wb / scale[:, None, :]).reshape(K, N))
    Bq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return Bq, (e + 127).astype(np.uint8)


# ------------------------------------------------------------ decode attention

BF16_NAN = 0x7FC0


def seq_lens(batch: int, lmax: int, seed: int, lo: int = 1) -> np.ndarray:
    """Ragged decode lengths: int32 [batch], uniform in [lo, lmax]."""
    return rng(seed).integers(lo, lmax + 1, size=batch).astype(np.int32)


def kv_cache(batch: int, h_kv: int, lmax: int, d: int, seed: int, lens=None,
             sigma: float = 1.0, pad: int = BF16_NAN) -> np.ndarray:
    """One cache tensor, bf16 codes [batch][h_kv][lmax][d] ~ N(0, sigma^2).
    Positions at or past lens[b] hold the code ``pad`` (NaN by default), so a
    kernel that reads past a sequence's length shows it in its output."""
    c = normal_bf16((batch, h_kv, lmax, d), sigma, seed)
    if lens is not None:
        for b, n in enumerate(np.asarray(lens)):
            c[b, :, int(n):, :] = pad
    return c
