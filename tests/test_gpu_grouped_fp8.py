"""GPU tests of the grouped (mixture-of-experts) fp8 block-scaled GEMM,
bi_gemm_fp8_blockscaled_grouped_packed.

A token's row must come out bit-identical whatever the routing of the other
tokens -- how many tokens share its expert, which ones, and how the other
experts are loaded -- and equal to the plain fp8 GEMM of that row with its
expert's weights and scales.  The oracle is the grouped definition (one
block-scaled GEMM per group of rows)."""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests.gpu_util import check_parity, dev_f32, dev_u8, host_codes, require_gpu, rows_equal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def experts(E, K, N, seed):
    qBs, sBs = [], []
    for e in range(E):
        qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, seed + e))
        qBs.append(qB)
        sBs.append(sB)
    return qBs, sBs


def upload(bg, qBs, sBs):
    Bd = [dev_u8(q, (q.shape[1] + 15) // 16 * 16) for q in qBs]
    Bp = bg.pack_b_fp8_grouped(Bd)
    sB = dev_f32(np.concatenate(sBs, axis=0))
    return Bd, Bp, sB


def run(bg, A, sA, offsets, Bp, sB):
    off = torch.as_tensor(np.asarray(offsets, np.int32), device="cuda")
    C = bg.gemm_fp8_blockscaled_grouped_packed(A, sA, off, Bp, sB)
    torch.cuda.synchronize()
    return C


def test_parity_with_empty_and_tiny_groups(bg):
    E, N, K = 5, 272, 512
    sizes = [0, 1, 37, 80, 3]
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    M = int(offsets[-1])
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 2001))
    qBs, sBs = experts(E, K, N, 2002)
    Bd, Bp, sB = upload(bg, qBs, sBs)
    A, sAd = dev_u8(qA), dev_f32(sA)
    got = host_codes(run(bg, A, sAd, offsets, Bp, sB))
    C64, S = oracle.gemm_fp8bs_grouped(qA, sA, offsets, qBs, sBs)
    check_parity(got, C64, S, K, "grouped fp8")
    # each group's rows: the same bits as the ungrouped GEMM with its expert
    for g in range(E):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            ref = host_codes(bg.gemm_fp8_blockscaled(A[lo:hi], sAd[lo:hi], Bd[g], dev_f32(sBs[g])))
            assert np.array_equal(got[lo:hi], ref), f"group {g}"


@pytest.fixture(scope="module")
def moe(bg):
    # 64 tokens, 8 experts, K = 7168, N = 2048 (the fp8 weight shape); the
    # reference is every token through every expert with the ungrouped packed
    # GEMM, whose rows are M-invariant
    T, E, K, N = 64, 8, 7168, 2048
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((T, K), 1.0, 2101))
    qBs, sBs = experts(E, K, N, 2102)
    Bd, Bp, sB = upload(bg, qBs, sBs)
    A, sAd = dev_u8(qA), dev_f32(sA)
    ref = torch.stack([bg.gemm_fp8_blockscaled_packed(A, sAd, bg.pack_b_fp8(b), dev_f32(s))
                       for b, s in zip(Bd, sBs)])                          # [E, T, N]
    return qA, sA, qBs, sBs, A, sAd, Bp, sB, ref


@pytest.mark.parametrize("skew", [0.0, 1.0, 3.0, 50.0])
def test_routing_invariance(bg, moe, skew):
    qA, sA, qBs, sBs, A, sAd, Bp, sB, ref = moe
    T, E = A.shape[0], len(qBs)
    for r in range(4):
        expert = inputs.route_tokens(T, E, 2200 + 10 * r + int(skew), skew)
        order, offsets = inputs.group_by_expert(expert, E)
        perm = torch.as_tensor(order, device="cuda")
        C = run(bg, A.index_select(0, perm), sAd.index_select(0, perm), offsets, Bp, sB)
        want = ref[torch.as_tensor(expert[order], device="cuda"), perm]
        ok = rows_equal(C, want)
        assert bool(ok.all()), f"skew {skew} routing {r}: rows {torch.nonzero(~ok).flatten()[:8].tolist()}"


def test_parity_full_shape_routed(bg, moe):
    qA, sA, qBs, sBs, A, sAd, Bp, sB, ref = moe
    T, E = A.shape[0], len(qBs)
    expert = inputs.route_tokens(T, E, 2250, 1.0)
    order, offsets = inputs.group_by_expert(expert, E)
    perm = torch.as_tensor(order, device="cuda")
    got = host_codes(run(bg, A.index_select(0, perm), sAd.index_select(0, perm), offsets, Bp, sB))
    C64, S = oracle.gemm_fp8bs_grouped(np.ascontiguousarray(qA[order]), np.ascontiguousarray(sA[order]),
                                       offsets, qBs, sBs)
    check_parity(got, C64, S, qA.shape[1], "grouped fp8 K=7168 N=2048, every token")


def test_all_tokens_one_expert_and_subsets(bg, moe):
    qA, sA, qBs, sBs, A, sAd, Bp, sB, ref = moe
    T, E = A.shape[0], len(qBs)
    for e in (0, 5, 7):
        offsets = [0] * (e + 1) + [T] * (E - e)
        C = run(bg, A, sAd, offsets, Bp, sB)
        assert bool(rows_equal(C, ref[e]).all()), f"expert {e}"
    for seed in range(3):
        pick = inputs.rng(2300 + seed).choice(T, size=17, replace=False)
        expert = inputs.rng(2310 + seed).integers(0, E, size=17)
        order, offsets = inputs.group_by_expert(expert, E)
        rows = torch.as_tensor(pick[order], device="cuda")
        C = run(bg, A.index_select(0, rows), sAd.index_select(0, rows), offsets, Bp, sB)
        want = ref[torch.as_tensor(expert[order], device="cuda"), rows]
        assert bool(rows_equal(C, want).all()), f"subset {seed}"


def test_every_geometry(bg):
    # the mean rows per group picks the launch geometry; all give the same bits
    E, K = 4, 256
    seen = set()
    for N in (1024, 4096):
        qBs, sBs = experts(E, K, N, 2400 + N)
        Bd, Bp, sB = upload(bg, qBs, sBs)
        single = [bg.pack_b_fp8(b) for b in Bd]
        for M in (1, 2, 7, 9, 70, 100, 130, 250, 600, 1100):
            qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 2410 + M))
            expert = inputs.route_tokens(M, E, 2420 + M, 1.0)
            order, offsets = inputs.group_by_expert(expert, E)
            A, sAd = dev_u8(np.ascontiguousarray(qA[order])), dev_f32(np.ascontiguousarray(sA[order]))
            C = host_codes(run(bg, A, sAd, offsets, Bp, sB))
            geo = bg.geometry("fp8_grouped_packed", M, N, K, groups=E)
            seen.add(geo["id"])
            for e in range(E):
                lo, hi = offsets[e], offsets[e + 1]
                if hi > lo:
                    ref = host_codes(bg.gemm_fp8_blockscaled_packed(A[lo:hi], sAd[lo:hi], single[e],
                                                                    dev_f32(sBs[e])))
                    assert np.array_equal(C[lo:hi], ref), f"N={N} M={M} expert {e} geometry {geo}"
    # unstaged half and whole blocks, 16 x 32 and 16 x 64 tiles, a tiled entry
    assert seen >= {2, 6, 7, 8, 9}, seen


def test_malformed_offsets_stay_in_bounds(bg):
    E, K, N, M = 3, 128, 64, 40
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 2501))
    qBs, sBs = experts(E, K, N, 2502)
    Bd, Bp, sB = upload(bg, qBs, sBs)
    A, sAd = dev_u8(qA), dev_f32(sA)
    C = run(bg, A, sAd, [0, 30, 10, 999], Bp, sB)
    ref = host_codes(bg.gemm_fp8_blockscaled(A[:30], sAd[:30], Bd[0], dev_f32(sBs[0])))
    assert np.array_equal(host_codes(C)[:30], ref)


def test_empty_batch(bg, moe):
    qA, sA, qBs, sBs, A, sAd, Bp, sB, ref = moe
    C = run(bg, A[:0], sAd[:0], [0] * (len(qBs) + 1), Bp, sB)
    assert C.shape[0] == 0


@pytest.mark.parametrize("G", [63, 64, 130])
def test_many_groups(bg, G):
    # more groups than one 63-entry chunk of the offsets lookup (many of them
    # empty): each expert's rows equal its ungrouped GEMM bit for bit, and the
    # batch matches the grouped oracle
    K, N, T = 256, 128, 200
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((T, K), 1.0, 2601 + G))
    qBs, sBs = experts(G, K, N, 2700)
    Bd, Bp, sB = upload(bg, qBs, sBs)
    expert = inputs.route_tokens(T, G, 2650 + G, 1.0)
    order, offsets = inputs.group_by_expert(expert, G)
    qAo, sAo = np.ascontiguousarray(qA[order]), np.ascontiguousarray(sA[order])
    A, sAd = dev_u8(qAo), dev_f32(sAo)
    got = host_codes(run(bg, A, sAd, offsets, Bp, sB))
    C64, S = oracle.gemm_fp8bs_grouped(qAo, sAo, offsets, qBs, sBs)
    check_parity(got, C64, S, K, f"grouped fp8, {G} groups")
    assert int(np.count_nonzero(np.diff(offsets) == 0)) > 0
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            ref = host_codes(bg.gemm_fp8_blockscaled(A[lo:hi], sAd[lo:hi], Bd[g], dev_f32(sBs[g])))
            assert np.array_equal(got[lo:hi], ref), f"group {g} of {G}"
