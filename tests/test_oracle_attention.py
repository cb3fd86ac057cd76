"""Pins for the decode-attention oracle, independent of the oracle itself (CPU only).

The oracle computes scaled dot-product attention (Vaswani et al. 2017,
equation 1) with grouped-query heads, one query token per sequence, over
each sequence's first ``lens[b]`` cached keys.  These tests pin it to:
torch's own ``scaled_dot_product_attention`` (float64, grouped-query mode),
closed forms (one key, two keys, zero scale), invariances the definition
implies (jointly permuting keys and values, shifting every key's logit by
one constant), and the head mapping and length mask (cache data past a
length and other KV heads must not reach an output).  A dropped
normalisation, a swapped K/V, a wrong head index or an off-by-one length
fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from invariant_gemm_amd import inputs

f32 = inputs.bf16_codes_to_f32


def _case(B, Hq, Hkv, L, D, seed, lens=None, sigma=1.0):
    Q = inputs.normal_bf16((B, Hq, D), sigma, seed)
    K = inputs.kv_cache(B, Hkv, L, D, seed + 1, lens)
    V = inputs.kv_cache(B, Hkv, L, D, seed + 2, lens)
    return Q, K, V


@pytest.mark.parametrize("B,Hq,Hkv,L,D", [(2, 8, 2, 37, 16), (1, 4, 4, 5, 8), (3, 16, 1, 70, 32)])
def test_matches_torch_sdpa(B, Hq, Hkv, L, D):
    lens = np.array([L - 3 * b for b in range(B)], np.int32)
    Q, K, V = _case(B, Hq, Hkv, L, D, 11, lens)
    scale = 1.0 / math.sqrt(D)
    O = oracle.decode_attention(Q, K, V, lens, scale)
    for b in range(B):
        n = int(lens[b])
        q = torch.from_numpy(f32(Q[b]).astype(np.float64))[None, :, None, :]
        k = torch.from_numpy(f32(K[b, :, :n]).astype(np.float64))[None]
        v = torch.from_numpy(f32(V[b, :, :n]).astype(np.float64))[None]
        ref = F.scaled_dot_product_attention(q, k, v, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(O[b], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_single_key_returns_its_value_exactly():
    Q, K, V = _case(2, 4, 2, 9, 16, 21)
    lens = np.array([1, 1], np.int32)
    O = oracle.decode_attention(Q, K, V, lens, 0.7)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(O[b, h], f32(V[b, h // 2, 0]).astype(np.float64))


def test_two_keys_closed_form():
    # o = v1 + (v0 - v1) * sigmoid(z0 - z1), z_j = scale * q.k_j
    Q, K, V = _case(1, 2, 1, 2, 8, 31)
    scale = 0.4
    O = oracle.decode_attention(Q, K, V, np.array([2], np.int32), scale)
    k = f32(K[0, 0]).astype(np.float64)
    v = f32(V[0, 0]).astype(np.float64)
    for h in range(2):
        q = f32(Q[0, h]).astype(np.float64)
        z0, z1 = scale * float(q @ k[0]), scale * float(q @ k[1])
        sig = 1.0 / (1.0 + math.exp(-(z0 - z1)))
        np.testing.assert_allclose(O[0, h], v[1] + (v[0] - v[1]) * sig, rtol=1e-12, atol=1e-14)


def test_zero_scale_is_the_mean_of_the_values():
    lens = np.array([13, 40], np.int32)
    Q, K, V = _case(2, 6, 3, 40, 16, 41, lens)
    O = oracle.decode_attention(Q, K, V, lens, 0.0)
    for b in range(2):
        n = int(lens[b])
        for h in range(6):
            mean = f32(V[b, h // 2, :n]).astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(O[b, h], mean, rtol=1e-12, atol=1e-14)


def test_joint_permutation_of_keys_and_values():
    lens = np.array([50], np.int32)
    Q, K, V = _case(1, 4, 2, 64, 16, 51, lens)
    perm = inputs.permutation(50, 52)
    K2, V2 = K.copy(), V.copy()
    K2[:, :, :50] = K[:, :, perm]
    V2[:, :, :50] = V[:, :, perm]
    O1 = oracle.decode_attention(Q, K, V, lens, 0.25)
    O2 = oracle.decode_attention(Q, K2, V2, lens, 0.25)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-14)
    # permuting only the values must change the result (K and V are paired)
    V3 = V.copy()
    V3[:, :, :50] = V[:, :, perm]
    assert not np.allclose(oracle.decode_attention(Q, K, V3, lens, 0.25), O1, atol=1e-3)


def test_shifting_every_logit_by_a_constant():
    # k_j' = k_j + w for all j adds q.w to every logit of a head: softmax
    # ignores it.  Small integers keep every value exact in bf16 and fp64.
    r = inputs.rng(61)
    D, L = 16, 24
    Q = inputs.f32_to_bf16_codes(r.integers(-3, 4, (1, 4, D)).astype(np.float32))
    K = r.integers(-4, 5, (1, 2, L, D)).astype(np.float32)
    w = r.integers(-8, 9, D).astype(np.float32)
    V = inputs.normal_bf16((1, 2, L, D), 1.0, 62)
    lens = np.array([L], np.int32)
    O1 = oracle.decode_attention(Q, inputs.f32_to_bf16_codes(K), V, lens, 0.125)
    O2 = oracle.decode_attention(Q, inputs.f32_to_bf16_codes(K + w), V, lens, 0.125)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-14)


def test_one_dominant_key_selects_its_value():
    # k_3 = 8 q (the others tiny): w_3 = 1 to within exp(-large)
    D = 16
    Q = inputs.normal_bf16((1, 1, D), 1.0, 71)
    q = f32(Q[0, 0])
    K = np.zeros((1, 1, 8, D), np.float32)
    K[0, 0, 3] = 8 * q
    V = inputs.normal_bf16((1, 1, 8, D), 1.0, 72)
    O = oracle.decode_attention(Q, inputs.f32_to_bf16_codes(K), V, np.array([8], np.int32), 1.0)
    np.testing.assert_allclose(O[0, 0], f32(V[0, 0, 3]), rtol=0, atol=1e-12)


def test_cache_past_length_and_other_heads_are_not_read():
    lens = np.array([17, 1, 33], np.int32)
    Q, K, V = _case(3, 8, 4, 40, 16, 81, lens)          # NaN past every length
    O = oracle.decode_attention(Q, K, V, lens, 0.3)
    assert np.all(np.isfinite(O))
    # changing KV head 1 of sequence 2 changes exactly query heads 2 and 3 of it
    K2 = K.copy()
    K2[2, 1, :33] = inputs.normal_bf16((33, 16), 1.0, 82)
    O2 = oracle.decode_attention(Q, K2, V, lens, 0.3)
    changed = np.any(O2 != O, axis=2)
    expect = np.zeros((3, 8), bool)
    expect[2, 2:4] = True
    assert np.array_equal(changed, expect)


def test_zero_length_gives_zero_and_weights_are_a_distribution():
    lens = np.array([0, 29], np.int32)
    Q, K, V = _case(2, 4, 1, 32, 16, 91, lens)
    O, W, A = oracle.decode_attention(Q, K, V, lens, 0.2, weights=True)
    assert np.all(O[0] == 0) and np.all(W[0] == 0)
    np.testing.assert_allclose(W[1].sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(W[1, :, 29:] == 0) and np.all(W[1, :, :29] > 0)
    q = f32(Q[1]).astype(np.float64)
    k = f32(K[1, 0, :29]).astype(np.float64)
    np.testing.assert_allclose(A[1, :, :29], np.abs(q[:, None, :] * k[None]).sum(-1), rtol=1e-14)
    # O is the W-weighted sum of the values
    v = f32(V[1, 0, :29]).astype(np.float64)
    np.testing.assert_allclose(O[1], W[1, :, :29] @ v, rtol=1e-12, atol=1e-14)
