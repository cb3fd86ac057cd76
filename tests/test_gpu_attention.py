"""Decode attention on the GPU: parity with the fp64 oracle, bit-identity of the
two kernels, batch invariance, edge cases, graph replay.

Tolerance (per output element, derived from the arithmetic): each key's
probability p_j reaches the output with a relative error e_j made of its
bf16 rounding (unit roundoff 2^-9) plus the fp32 score error (at most
D * 2^-24 * scale * sum_d |q_d k_jd| in the exponent); to first order the
output then moves by sum_j w_j e_j (|v_jd| + |o_d|).  The test allows
e_j = 2^-8 + 2^-16 * scale * sum_d |q_d k_jd| (twice each term) plus 2^-8 |o_d|
for the final bf16 rounding and 1e-6 absolute.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import bigemm, inputs

pytestmark = pytest.mark.gpu

D = 128
DEV = "cuda:0"


def _dev(codes):
    return torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(torch.bfloat16).to(DEV)


def _host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _lens(lens):
    return torch.from_numpy(np.ascontiguousarray(lens, np.int32)).to(DEV)


def _case(B, Hq, Hkv, Lmax, seed, lens, qsigma=1.0):
    Q = inputs.normal_bf16((B, Hq, D), qsigma, seed)
    K = inputs.kv_cache(B, Hkv, Lmax, D, seed + 1, lens)
    V = inputs.kv_cache(B, Hkv, Lmax, D, seed + 2, lens)
    return Q, K, V


def _run(Q, K, V, lens, scale, kernel):
    O = bigemm.decode_attention(_dev(Q), _dev(K), _dev(V), _lens(lens), scale, kernel=kernel)
    torch.cuda.synchronize()
    return _host(O)


def _check_parity(Ocodes, Q, K, V, lens, scale, seqs=None):
    seqs = np.arange(Q.shape[0]) if seqs is None else np.asarray(seqs)
    Q, K, V, lens = Q[seqs], K[seqs], V[seqs], np.asarray(lens)[seqs]
    O64, W, A = oracle.decode_attention(Q, K, V, lens, scale, weights=True)
    B, Hq, _ = Q.shape
    Hkv, Lmax = K.shape[1], K.shape[2]
    G = Hq // Hkv
    absv = np.abs(inputs.bf16_codes_to_f32(V).astype(np.float64))
    absv[~np.isfinite(absv)] = 0.0                        # NaN pads: weight 0 there
    e = W * (2.0**-8 + 2.0**-16 * abs(scale) * A)         # [B,Hq,L]
    t1 = np.matmul(e.reshape(B, Hkv, G, Lmax), absv).reshape(B, Hq, D)
    bound = t1 + (e.sum(axis=2)[:, :, None] + 2.0**-8) * np.abs(O64) + 1e-6
    got = inputs.bf16_codes_to_f32(Ocodes[seqs]).astype(np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.abs(got - O64)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} elements out of bound; first {tuple(i)}: "
                             f"got {got[tuple(i)]} want {O64[tuple(i)]} bound {bound[tuple(i)]}")
    return float((err / bound).max())


LEN_MIX = [1, 2, 63, 64, 65, 255, 256, 257, 511, 700, 1000, 1024]


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8), (64, 8), (16, 1), (6, 3)])
@pytest.mark.parametrize("kernel", ["single", "split"])
def test_parity_ragged(Hq, Hkv, kernel):
    lens = np.array(LEN_MIX, np.int32)
    Q, K, V = _case(len(lens), Hq, Hkv, 1024, 1000 + Hq + Hkv, lens)
    scale = 1.0 / math.sqrt(D)
    O = _run(Q, K, V, lens, scale, kernel)
    _check_parity(O, Q, K, V, lens, scale)


@pytest.mark.parametrize("qsigma,scale", [(4.0, 1 / math.sqrt(D)), (1.0, 1.0), (1.0, 0.0), (1.0, -0.05)])
def test_parity_logit_ranges(qsigma, scale):
    lens = np.array([300, 77, 1024, 5], np.int32)
    Q, K, V = _case(4, 16, 2, 1024, 2000, lens, qsigma)
    O = _run(Q, K, V, lens, scale, "split")
    _check_parity(O, Q, K, V, lens, scale)
    assert np.array_equal(O, _run(Q, K, V, lens, scale, "single"))


def test_single_and_split_are_bit_identical():
    r = inputs.rng(3000)
    for trial in range(6):
        Hkv = int(r.choice([1, 2, 4, 8]))
        G = int(r.choice([1, 2, 3, 8, 16]))
        B = int(r.integers(1, 9))
        Lmax = int(r.choice([64, 300, 1024, 2048]))
        lens = inputs.seq_lens(B, Lmax, 3001 + trial, lo=0)
        Q, K, V = _case(B, G * Hkv, Hkv, Lmax, 3100 + 10 * trial, lens)
        a = _run(Q, K, V, lens, 0.09, "single")
        b = _run(Q, K, V, lens, 0.09, "split")
        assert np.array_equal(a, b), f"trial {trial}: B={B} G={G} Hkv={Hkv} Lmax={Lmax}"


def test_split_runs_of_groups_with_ragged_lengths():
    # 16 sequences x 16 KV heads x 16 groups = 4096 groups: the split kernel gives
    # each workgroup a run of 2 consecutive groups (walked with prefetch), so
    # runs end inside and past ragged lengths; bits must not change
    Hq, Hkv, Lmax = 32, 16, 4096
    lens = inputs.seq_lens(16, Lmax, 4500, lo=0)
    lens[:4] = [0, 1, 512, 513]                      # empty, tiny, run boundaries
    Q, K, V = _case(16, Hq, Hkv, Lmax, 4501, lens)
    a = _run(Q, K, V, lens, 0.1, "split")
    assert np.array_equal(a, _run(Q, K, V, lens, 0.1, "single"))
    for b in (1, 2, 3, 9):
        alone = _run(Q[b:b + 1], K[b:b + 1], V[b:b + 1], lens[b:b + 1], 0.1, "split")
        assert np.array_equal(alone[0], a[b]), f"sequence {b}"
    _check_parity(a, Q, K, V, lens, 0.1, seqs=[0, 1, 2, 3, 9])


def test_batch_invariance_across_batch_size_position_and_kernel():
    # a pool of 40 sequences, computed as one batch (the library picks the
    # single-pass kernel: 320 (sequence, KV head) pairs), each alone (it picks
    # the split kernel) and in shuffled sub-batches of either kind
    Hq, Hkv, Lmax = 64, 8, 2048
    lens = inputs.seq_lens(40, Lmax, 4000)
    Q, K, V = _case(40, Hq, Hkv, Lmax, 4001, lens)
    assert bigemm.decode_attention_choice(1, Hq, Hkv, Lmax) == "split"
    assert bigemm.decode_attention_choice(40, Hq, Hkv, Lmax) == "single"
    full = _run(Q, K, V, lens, 0.088, "auto")
    assert np.array_equal(full, _run(Q, K, V, lens, 0.088, "single"))
    for b in (0, 17, 39):
        alone = _run(Q[b:b + 1], K[b:b + 1], V[b:b + 1], lens[b:b + 1], 0.088, "auto")
        assert np.array_equal(alone[0], full[b]), f"sequence {b} alone"
    for s, size in enumerate((5, 13, 32)):
        idx = inputs.permutation(40, 4100 + s)[:size]
        sub = _run(Q[idx], K[idx], V[idx], lens[idx], 0.088, "auto")
        assert np.array_equal(sub, full[idx]), f"sub-batch {size}"
    _check_parity(full, Q, K, V, lens, 0.088, seqs=[0, 17, 39])


def test_cache_capacity_does_not_change_the_result():
    # the same sequences in a cache of larger capacity (Lmax) give the same bits
    lens = np.array([100, 513, 1000], np.int32)
    Q, K, V = _case(3, 16, 4, 1024, 5000, lens)
    K2 = np.full((3, 4, 3000, D), inputs.BF16_NAN, np.uint16)
    V2 = K2.copy()
    K2[:, :, :1024], V2[:, :, :1024] = K, V
    for kernel in ("single", "split"):
        assert np.array_equal(_run(Q, K, V, lens, 0.1, kernel), _run(Q, K2, V2, lens, 0.1, kernel))


def test_zero_lengths_and_empty_cache():
    lens = np.array([0, 5, 0], np.int32)
    Q, K, V = _case(3, 8, 2, 64, 6000, lens)
    for kernel in ("single", "split", "auto"):
        O = _run(Q, K, V, lens, 0.1, kernel)
        assert np.all(O[[0, 2]] == 0)
        _check_parity(O, Q, K, V, lens, 0.1, seqs=[1])
    Q0 = inputs.normal_bf16((2, 8, D), 1.0, 6001)
    empty = torch.empty((2, 2, 0, D), dtype=torch.bfloat16, device=DEV)
    for kernel in ("single", "split"):
        O = bigemm.decode_attention(_dev(Q0), empty, empty, _lens([0, 0]), 0.1, kernel=kernel)
        torch.cuda.synchronize()
        assert torch.all(O.view(torch.int16) == 0)


def test_lengths_are_clamped_to_capacity():
    lens = np.array([64, 64], np.int32)
    Q, K, V = _case(2, 8, 1, 64, 7000, lens)
    want = _run(Q, K, V, lens, 0.1, "single")
    got = _run(Q, K, V, np.array([64, 100000], np.int32), 0.1, "split")
    assert np.array_equal(got, want)
    zero = _run(Q, K, V, np.array([-5, 64], np.int32), 0.1, "single")
    assert np.all(zero[0] == 0) and np.array_equal(zero[1], want[1])


def test_long_sequence():
    lens = np.array([32768, 20001], np.int32)
    Q, K, V = _case(2, 8, 1, 32768, 8000, lens)
    a = _run(Q, K, V, lens, 1 / math.sqrt(D), "split")
    assert np.array_equal(a, _run(Q, K, V, lens, 1 / math.sqrt(D), "single"))
    _check_parity(a, Q, K, V, lens, 1 / math.sqrt(D))


@pytest.fixture(scope="module")
def full_case():
    # the decode workload at full size: B = 64 sequences of 4096 keys,
    # Hq = 64, Hkv = 8, D = 128
    B, Hq, Hkv, L = 64, 64, 8, 4096
    lens = np.full(B, L, np.int32)
    Q = inputs.normal_bf16((B, Hq, D), 1.0, 9000)
    K = inputs.normal_bf16((B, Hkv, L, D), 1.0, 9001)
    V = inputs.normal_bf16((B, Hkv, L, D), 1.0, 9002)
    return Q, K, V, lens


def test_full_size_parity_sampled_and_invariant(full_case):
    Q, K, V, lens = full_case
    scale = 1 / math.sqrt(D)
    Qd, Kd, Vd, ld = _dev(Q), _dev(K), _dev(V), _lens(lens)
    O = {}
    for kernel in ("single", "split"):
        O[kernel] = _host(bigemm.decode_attention(Qd, Kd, Vd, ld, scale, kernel=kernel))
    torch.cuda.synchronize()
    assert np.array_equal(O["single"], O["split"])
    _check_parity(O["single"], Q, K, V, lens, scale, seqs=[0, 31, 63])
    for B in (1, 16):                      # the bench's smaller batches, same sequences
        sub = _host(bigemm.decode_attention(Qd[:B].contiguous(), Kd[:B].contiguous(),
                                            Vd[:B].contiguous(), ld[:B], scale))
        assert np.array_equal(sub, O["single"][:B]), f"B={B}"


@pytest.mark.parametrize("kernel", ["single", "split"])
def test_graph_replay_matches_eager(kernel):
    lens = np.array([1000, 17, 256, 4096], np.int32)
    Q, K, V = _case(4, 64, 8, 4096, 9500, lens)
    Qd, Kd, Vd, ld = _dev(Q), _dev(K), _dev(V), _lens(lens)
    ws = torch.empty(bigemm.decode_attention_workspace_bytes(4, 64, 8, 4096) // 4,
                     dtype=torch.float32, device=DEV)
    out = torch.empty((4, 64, D), dtype=torch.bfloat16, device=DEV)
    eager = _host(bigemm.decode_attention(Qd, Kd, Vd, ld, 0.1, kernel=kernel, workspace=ws))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bigemm.decode_attention(Qd, Kd, Vd, ld, 0.1, kernel=kernel, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bigemm.decode_attention(Qd, Kd, Vd, ld, 0.1, kernel=kernel, workspace=ws, out=out)
    for rep in range(4):
        out.zero_()
        ws.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_host(out), eager), f"replay {rep}"
        _ = torch.randn(1024, device=DEV).sum().item()   # eager work between replays
