"""GPU tests of the grouped (mixture-of-experts) GEMM, bi_gemm_bf16_grouped_packed.

A token's row must come out bit-identical whatever the routing of the other
tokens -- how many tokens share its expert, which ones, and how the other
experts are loaded -- and equal to the plain GEMM of that row with its
expert's weights.  The oracle is the grouped definition (one plain GEMM per
group of rows)."""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests.gpu_util import check_parity, dev_bf16, host_codes, require_gpu, rows_equal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def run(bg, A, offsets, Bp):
    off = torch.as_tensor(np.asarray(offsets, np.int32), device="cuda")
    C = bg.gemm_bf16_grouped_packed(A, off, Bp)
    torch.cuda.synchronize()
    return C


def test_parity_with_empty_and_tiny_groups(bg):
    G, N, K = 5, 272, 520
    sizes = [0, 1, 37, 80, 3]
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    M = int(offsets[-1])
    Ah = inputs.normal_bf16((M, K), 1.0, 1001)
    Bh = [inputs.normal_bf16((K, N), 0.02, 1002 + g) for g in range(G)]
    Bd = [dev_bf16(b) for b in Bh]
    Bp = bg.pack_b_bf16_grouped(Bd)
    got = host_codes(run(bg, dev_bf16(Ah), offsets, Bp))
    C64, S = oracle.gemm_bf16_grouped(Ah, offsets, Bh)
    check_parity(got, C64, S, K, "grouped")
    # each group's rows: the same bits as the ungrouped packed GEMM
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            ref = host_codes(bg.gemm_bf16_packed(dev_bf16(Ah[lo:hi]), bg.pack_b_bf16(Bd[g])))
            assert np.array_equal(got[lo:hi], ref), f"group {g}"


@pytest.fixture(scope="module")
def moe(bg):
    # 64 tokens, 8 experts, K=2048, N=1024; reference: every token through every
    # expert with the ungrouped packed GEMM (whose rows are M-invariant)
    T, E, K, N = 64, 8, 2048, 1024
    Ah = inputs.normal_bf16((T, K), 1.0, 1101)
    Bh = [inputs.normal_bf16((K, N), 0.02, 1102 + e) for e in range(E)]
    A = dev_bf16(Ah)
    Bd = [dev_bf16(b) for b in Bh]
    Bp = bg.pack_b_bf16_grouped(Bd)
    ref = torch.stack([bg.gemm_bf16_packed(A, bg.pack_b_bf16(b)) for b in Bd])   # [E, T, N]
    return Ah, Bh, A, Bp, ref


@pytest.mark.parametrize("skew", [0.0, 1.0, 3.0, 50.0])
def test_routing_invariance(bg, moe, skew):
    Ah, Bh, A, Bp, ref = moe
    T, E = A.shape[0], len(Bh)
    for r in range(6):
        expert = inputs.route_tokens(T, E, 1200 + 10 * r + int(skew), skew)
        order, offsets = inputs.group_by_expert(expert, E)
        perm = torch.as_tensor(order, device="cuda")
        C = run(bg, A.index_select(0, perm), offsets, Bp)
        want = ref[torch.as_tensor(expert[order], device="cuda"), perm]
        ok = rows_equal(C, want)
        assert bool(ok.all()), f"skew {skew} routing {r}: rows {torch.nonzero(~ok).flatten()[:8].tolist()}"


def test_all_tokens_one_expert_and_subsets(bg, moe):
    Ah, Bh, A, Bp, ref = moe
    T, E = A.shape[0], len(Bh)
    for e in (0, 5, 7):
        offsets = [0] * (e + 1) + [T] * (E - e)
        C = run(bg, A, offsets, Bp)
        assert bool(rows_equal(C, ref[e]).all()), f"expert {e}"
    # a subset of tokens, shuffled, spread over the experts
    for seed in range(3):
        pick = inputs.rng(1300 + seed).choice(T, size=17, replace=False)
        expert = inputs.rng(1310 + seed).integers(0, E, size=17)
        order, offsets = inputs.group_by_expert(expert, E)
        rows = torch.as_tensor(pick[order], device="cuda")
        C = run(bg, A.index_select(0, rows), offsets, Bp)
        want = ref[torch.as_tensor(expert[order], device="cuda"), rows]
        assert bool(rows_equal(C, want).all()), f"subset {seed}"


def test_every_geometry(bg):
    # mean rows per group picks the launch geometry; all must give the same bits
    E, K, N = 4, 256, 4096
    Bh = [inputs.normal_bf16((K, N), 0.02, 1400 + e) for e in range(E)]
    Bd = [dev_bf16(b) for b in Bh]
    Bp = bg.pack_b_bf16_grouped(Bd)
    single = [bg.pack_b_bf16(b) for b in Bd]
    for M in (1, 2, 4, 7, 70, 100, 130, 250, 600, 900, 2000):
        Ah = inputs.normal_bf16((M, K), 1.0, 1410 + M)
        expert = inputs.route_tokens(M, E, 1420 + M, 1.0)
        order, offsets = inputs.group_by_expert(expert, E)
        A = dev_bf16(Ah[order])
        C = host_codes(run(bg, A, offsets, Bp))
        for e in range(E):
            lo, hi = offsets[e], offsets[e + 1]
            if hi > lo:
                ref = host_codes(bg.gemm_bf16_packed(A[lo:hi], single[e]))
                assert np.array_equal(C[lo:hi], ref), f"M={M} expert {e}"


def test_narrow_n_few_rows(bg):
    # few rows over a narrow, ragged N (the one-wave geometry with its tight
    # slot count): every expert's rows must equal the row-major kernel's
    # result for that expert, bit for bit
    E, K, N = 3, 256, 1000
    Bh = [inputs.normal_bf16((K, N), 0.02, 1460 + e) for e in range(E)]
    Bd = [dev_bf16(b) for b in Bh]
    Bp = bg.pack_b_bf16_grouped(Bd)
    for M in (1, 3, 9):
        Ah = inputs.normal_bf16((M, K), 1.0, 1470 + M)
        expert = inputs.route_tokens(M, E, 1480 + M, 1.0)
        order, offsets = inputs.group_by_expert(expert, E)
        A = dev_bf16(Ah[order])
        C = host_codes(run(bg, A, offsets, Bp))
        for e in range(E):
            lo, hi = offsets[e], offsets[e + 1]
            if hi > lo:
                ref = host_codes(bg.gemm_bf16(A[lo:hi], Bd[e]))
                assert np.array_equal(C[lo:hi], ref), f"M={M} expert {e}"


def test_malformed_offsets_stay_in_bounds(bg):
    # a decreasing entry is clamped (no access outside A, B or C); the rows of
    # the well-formed groups before it still come out right
    E, K, N, M = 3, 128, 64, 40
    Ah = inputs.normal_bf16((M, K), 1.0, 1501)
    Bd = [dev_bf16(inputs.normal_bf16((K, N), 0.02, 1502 + e)) for e in range(E)]
    Bp = bg.pack_b_bf16_grouped(Bd)
    A = dev_bf16(Ah)
    C = run(bg, A, [0, 30, 10, 999], Bp)
    ref = host_codes(bg.gemm_bf16_packed(A[:30], bg.pack_b_bf16(Bd[0])))
    assert np.array_equal(host_codes(C)[:30], ref)


def test_empty_batch(bg, moe):
    Ah, Bh, A, Bp, ref = moe
    C = run(bg, A[:0], [0] * (len(Bh) + 1), Bp)
    assert C.shape[0] == 0


@pytest.mark.parametrize("G", [63, 64, 127, 200])
def test_many_groups(bg, G):
    # more groups than one 63-entry chunk of the offsets lookup: tokens spread
    # over G experts with many empty ones; each expert's rows equal its
    # ungrouped packed GEMM bit for bit, and the batch matches the oracle
    K, N, T = 256, 64, 300
    Ah = inputs.normal_bf16((T, K), 1.0, 1301 + G)
    Bh = [inputs.normal_bf16((K, N), 0.02, 1400 + g) for g in range(G)]
    Bd = [dev_bf16(b) for b in Bh]
    Bp = bg.pack_b_bf16_grouped(Bd)
    expert = inputs.route_tokens(T, G, 1350 + G, 1.0)
    order, offsets = inputs.group_by_expert(expert, G)
    A = dev_bf16(np.ascontiguousarray(Ah[order]))
    got = host_codes(run(bg, A, offsets, Bp))
    C64, S = oracle.gemm_bf16_grouped(np.ascontiguousarray(Ah[order]), offsets, Bh)
    check_parity(got, C64, S, K, f"grouped, {G} groups")
    assert int(np.count_nonzero(np.diff(offsets) == 0)) > 0      # some experts get no token
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            ref = host_codes(bg.gemm_bf16_packed(A[lo:hi], bg.pack_b_bf16(Bd[g])))
            assert np.array_equal(got[lo:hi], ref), f"group {g} of {G}"
