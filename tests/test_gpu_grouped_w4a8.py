"""GPU tests of the grouped (mixture-of-experts) W4A8 GEMM,
bi_gemm_w4a8_grouped_packed: fp8 activations times each expert's OCP MXFP4
weights.

A token's row must come out bit-identical whatever the routing of the other
tokens -- how many tokens share its expert, which ones, and how the other
experts are loaded -- and equal to the plain W4A8 GEMM of that row with its
expert's weights.  The oracle is the grouped definition (one W4A8 GEMM per
group of rows)."""
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


def pad16(n):
    return (n + 15) // 16 * 16


def experts(E, K, N, seed):
    Bqs, sEs = [], []
    for e in range(E):
        Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((K, N), 0.02, seed + e))
        Bqs.append(Bq)
        sEs.append(sE)
    return Bqs, sEs


def upload(bg, Bqs, sEs, N):
    dq = [dev_u8(q, pad16(q.shape[1])) for q in Bqs]
    ds = [dev_u8(s, pad16(s.shape[1])) for s in sEs]
    single = [bg.pack_b_mxfp4(q, s, N) for q, s in zip(dq, ds)]
    return single, bg.pack_b_mxfp4_grouped(dq, ds, N)


def run(bg, A, sA, offsets, Bp):
    off = torch.as_tensor(np.asarray(offsets, np.int32), device="cuda")
    C = bg.gemm_w4a8_grouped_packed(A, sA, off, Bp)
    torch.cuda.synchronize()
    return C


def test_parity_with_empty_and_tiny_groups(bg):
    E, N, K = 5, 272, 512
    sizes = [0, 1, 37, 80, 3]
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    M = int(offsets[-1])
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 3001))
    Bqs, sEs = experts(E, K, N, 3002)
    single, Bp = upload(bg, Bqs, sEs, N)
    A, sAd = dev_u8(qA), dev_f32(sA)
    got = host_codes(run(bg, A, sAd, offsets, Bp))
    C64, S = oracle.gemm_w4a8_grouped(qA, sA, offsets, Bqs, sEs, N)
    check_parity(got, C64, S, K, "grouped W4A8")
    # each group's rows: the same bits as the ungrouped GEMM with its expert
    for g in range(E):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            ref = host_codes(bg.gemm_w4a8_packed(A[lo:hi], sAd[lo:hi], single[g]))
            assert np.array_equal(got[lo:hi], ref), f"group {g}"


@pytest.fixture(scope="module")
def moe(bg):
    # 64 tokens, 8 experts, K = 7168, N = 2048 (the MoE expert shape of the
    # bench); the reference is every token through every expert with the
    # ungrouped packed GEMM, whose rows are M-invariant
    T, E, K, N = 64, 8, 7168, 2048
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((T, K), 1.0, 3101))
    Bqs, sEs = experts(E, K, N, 3102)
    single, Bp = upload(bg, Bqs, sEs, N)
    A, sAd = dev_u8(qA), dev_f32(sA)
    ref = torch.stack([bg.gemm_w4a8_packed(A, sAd, s) for s in single])       # [E, T, N]
    return qA, sA, Bqs, sEs, A, sAd, Bp, ref


@pytest.mark.parametrize("skew", [0.0, 1.0, 3.0, 50.0])
def test_routing_invariance(bg, moe, skew):
    qA, sA, Bqs, sEs, A, sAd, Bp, ref = moe
    T, E = A.shape[0], len(Bqs)
    for r in range(4):
        expert = inputs.route_tokens(T, E, 3200 + 10 * r + int(skew), skew)
        order, offsets = inputs.group_by_expert(expert, E)
        perm = torch.as_tensor(order, device="cuda")
        C = run(bg, A.index_select(0, perm), sAd.index_select(0, perm), offsets, Bp)
        want = ref[torch.as_tensor(expert[order], device="cuda"), perm]
        ok = rows_equal(C, want)
        assert bool(ok.all()), f"skew {skew} routing {r}: rows {torch.nonzero(~ok).flatten()[:8].tolist()}"


def test_parity_full_shape_routed(bg, moe):
    qA, sA, Bqs, sEs, A, sAd, Bp, ref = moe
    T, E = A.shape[0], len(Bqs)
    N = Bp.N
    expert = inputs.route_tokens(T, E, 3250, 1.0)
    order, offsets = inputs.group_by_expert(expert, E)
    perm = torch.as_tensor(order, device="cuda")
    got = host_codes(run(bg, A.index_select(0, perm), sAd.index_select(0, perm), offsets, Bp))
    C64, S = oracle.gemm_w4a8_grouped(np.ascontiguousarray(qA[order]), np.ascontiguousarray(sA[order]),
                                      offsets, Bqs, sEs, N)
    check_parity(got, C64, S, qA.shape[1], "grouped W4A8 K=7168 N=2048, every token")


def test_all_tokens_one_expert_and_subsets(bg, moe):
    qA, sA, Bqs, sEs, A, sAd, Bp, ref = moe
    T, E = A.shape[0], len(Bqs)
    for e in (0, 5, 7):
        offsets = [0] * (e + 1) + [T] * (E - e)
        C = run(bg, A, sAd, offsets, Bp)
        assert bool(rows_equal(C, ref[e]).all()), f"expert {e}"
    for seed in range(3):
        pick = inputs.rng(3300 + seed).choice(T, size=17, replace=False)
        expert = inputs.rng(3310 + seed).integers(0, E, size=17)
        order, offsets = inputs.group_by_expert(expert, E)
        rows = torch.as_tensor(pick[order], device="cuda")
        C = run(bg, A.index_select(0, rows), sAd.index_select(0, rows), offsets, Bp)
        want = ref[torch.as_tensor(expert[order], device="cuda"), rows]
        assert bool(rows_equal(C, want).all()), f"subset {seed}"


def test_every_geometry(bg):
    # the rows per group pick the launch geometry; all give the same bits
    E, K = 4, 256
    seen = set()
    for N in (512, 2048, 8192):
        Bqs, sEs = experts(E, K, N, 3400 + N)
        single, Bp = upload(bg, Bqs, sEs, N)
        for M in (1, 2, 7, 9, 40, 70, 100, 130, 250, 300, 600, 1100):
            qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 3410 + M))
            expert = inputs.route_tokens(M, E, 3420 + M, 1.0)
            order, offsets = inputs.group_by_expert(expert, E)
            A, sAd = dev_u8(np.ascontiguousarray(qA[order])), dev_f32(np.ascontiguousarray(sA[order]))
            C = host_codes(run(bg, A, sAd, offsets, Bp))
            geo = bg.geometry("w4a8_grouped_packed", M, N, K, groups=E)
            seen.add(geo["id"])
            for e in range(E):
                lo, hi = offsets[e], offsets[e + 1]
                if hi > lo:
                    ref = host_codes(bg.gemm_w4a8_packed(A[lo:hi], sAd[lo:hi], single[e]))
                    assert np.array_equal(C[lo:hi], ref), f"N={N} M={M} expert {e} geometry {geo}"
    # every entry but the 64 x 128 tiles (large M only), unstaged ones included
    assert seen >= {0, 1, 2, 3, 4, 5, 7, 8, 9}, seen


def test_malformed_offsets_stay_in_bounds(bg):
    E, K, N, M = 3, 128, 64, 40
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 3501))
    Bqs, sEs = experts(E, K, N, 3502)
    single, Bp = upload(bg, Bqs, sEs, N)
    A, sAd = dev_u8(qA), dev_f32(sA)
    C = run(bg, A, sAd, [0, 30, 10, 999], Bp)
    ref = host_codes(bg.gemm_w4a8_packed(A[:30], sAd[:30], single[0]))
    assert np.array_equal(host_codes(C)[:30], ref)


def test_empty_batch(bg, moe):
    qA, sA, Bqs, sEs, A, sAd, Bp, ref = moe
    C = run(bg, A[:0], sAd[:0], [0] * (len(Bqs) + 1), Bp)
    assert C.shape[0] == 0


@pytest.mark.parametrize("G", [63, 64, 130])
def test_many_groups(bg, G):
    # more groups than one 63-entry chunk of the offsets lookup (many of them
    # empty): each expert's rows equal its ungrouped GEMM bit for bit, and the
    # batch matches the grouped oracle
    K, N, T = 256, 128, 200
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((T, K), 1.0, 3601 + G))
    Bqs, sEs = experts(G, K, N, 3700)
    single, Bp = upload(bg, Bqs, sEs, N)
    expert = inputs.route_tokens(T, G, 3650 + G, 1.0)
    order, offsets = inputs.group_by_expert(expert, G)
    qAo, sAo = np.ascontiguousarray(qA[order]), np.ascontiguousarray(sA[order])
    A, sAd = dev_u8(qAo), dev_f32(sAo)
    got = host_codes(run(bg, A, sAd, offsets, Bp))
    C64, S = oracle.gemm_w4a8_grouped(qAo, sAo, offsets, Bqs, sEs, N)
    check_parity(got, C64, S, K, f"grouped W4A8, {G} groups")
    assert int(np.count_nonzero(np.diff(offsets) == 0)) > 0
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            ref = host_codes(bg.gemm_w4a8_packed(A[lo:hi], sAd[lo:hi], single[g]))
            assert np.array_equal(got[lo:hi], ref), f"group {g} of {G}"
