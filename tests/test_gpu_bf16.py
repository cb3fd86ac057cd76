"""GPU parity and batch-invariance tests of bi_gemm_bf16 (through the C ABI).

Parity: every element within |err| <= 2^-7 S + 1e-6 of the fp64 oracle and
within the tight diagnostic bound; on exact-input closed forms the GPU must
equal the oracle's correctly rounded result bit for bit.
Invariance: each row computed alone (M = 1) must be bit-identical to the same
row computed at every other M, position and set of batch companions -- the
definition in section "什么是batch invariance" of the QbitAI article, checked
with the same-row-across-batch-sizes recipe of section 5.1 of the lshu.cn
article.
"""
import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests import full_size
from tests.gpu_util import (bf16_vals, check_parity, dev_bf16, host_codes, require_gpu,
                            rows_equal)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def run(bg, A_codes, B_codes, lda=None, ldb=None, ldc=None):
    M, K = A_codes.shape
    N = B_codes.shape[1]
    A = dev_bf16(A_codes, lda)
    B = dev_bf16(B_codes, ldb)
    out = None
    if ldc is not None and ldc != N:
        out = torch.zeros((M, ldc), dtype=torch.bfloat16, device="cuda")[:, :N]
    C = bg.gemm_bf16(A, B, out=out)
    torch.cuda.synchronize()
    return host_codes(C)


def dyadic(shape, seed, emin=-2, emax=1):
    g = inputs.rng(seed)
    m = g.integers(-15, 16, size=shape).astype(np.float64)
    e = g.integers(emin, emax + 1, size=shape)
    return inputs.f32_to_bf16_codes(np.ldexp(m, e).astype(np.float32))


# ------------------------------------------------------------------ exact pins


@pytest.mark.parametrize("M,N,K", [(17, 256, 512), (37, 100, 203), (1, 8, 1), (65, 40, 129)])
def test_exact_dyadic_bitwise(bg, M, N, K):
    # every partial sum of these inputs is exact in fp32, so any correct
    # kernel returns exactly the oracle's rounded sum
    A = dyadic((M, K), 1000 + M)
    B = dyadic((K, N), 2000 + N)
    C64, _ = oracle.gemm_bf16(A, B)
    lda = (K + 7) // 8 * 8
    ldb = (N + 7) // 8 * 8
    got = run(bg, A, B, lda=lda, ldb=ldb, ldc=ldb)
    assert np.array_equal(got, oracle.round_bf16(C64))


def test_identity_permutation_onehot(bg):
    M, K = 17, 512
    A = inputs.normal_bf16((M, K), 1.0, 11)
    I = inputs.f32_to_bf16_codes(np.eye(K, dtype=np.float32))
    assert np.array_equal(run(bg, A, I), A)
    p = inputs.permutation(K, 12)
    P = np.zeros((K, K), np.float32)
    P[p, np.arange(K)] = 1
    assert np.array_equal(run(bg, A, inputs.f32_to_bf16_codes(P)), A[:, p])
    B = inputs.normal_bf16((K, 256), 1.0, 13)
    rows = inputs.rng(14).integers(0, K, size=40)
    H = np.zeros((40, K), np.float32)
    H[np.arange(40), rows] = 1
    assert np.array_equal(run(bg, inputs.f32_to_bf16_codes(H), B), B[rows])


def test_all_ones_row_sums(bg):
    M, K, N = 33, 8192, 64
    T = inputs.rng(15).integers(-1, 2, size=(M, K)).astype(np.float32)
    got = run(bg, inputs.f32_to_bf16_codes(T), inputs.f32_to_bf16_codes(np.ones((K, N), np.float32)))
    exp = oracle.round_bf16(np.repeat(T.sum(1, keepdims=True).astype(np.float64), N, 1))
    assert np.array_equal(got, exp)


def test_k_zero_writes_zeros(bg):
    C = torch.full((5, 24), 7.0, dtype=torch.bfloat16, device="cuda")
    A = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((0, 24), dtype=torch.bfloat16, device="cuda")
    bg.gemm_bf16(A, B, out=C)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), torch.zeros_like(C).view(torch.int16))


def test_empty_m_is_noop(bg):
    A = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda")
    C = bg.gemm_bf16(A, B)
    assert C.shape == (0, 32)


# ------------------------------------------------------------------ tolerance parity


@pytest.mark.parametrize("M,N,K", [(17, 256, 512), (1, 256, 512), (130, 264, 1000), (64, 72, 4096),
                                   (200, 40, 33), (3, 8, 31)])
def test_parity_random(bg, M, N, K):
    A = inputs.normal_bf16((M, K), 1.0, 100 + M)
    B = inputs.normal_bf16((K, N), 1.0, 200 + N)
    C64, S = oracle.gemm_bf16(A, B)
    lda = (K + 7) // 8 * 8
    ldb = (N + 7) // 8 * 8
    got = run(bg, A, B, lda=lda, ldb=ldb, ldc=ldb)
    check_parity(got, C64, S, K, f"M{M} N{N} K{K}")


def test_padded_pitches_same_bits(bg):
    M, N, K = 40, 256, 512
    A = inputs.normal_bf16((M, K), 1.0, 31)
    B = inputs.normal_bf16((K, N), 1.0, 32)
    base = run(bg, A, B)
    assert np.array_equal(run(bg, A, B, lda=K + 64, ldb=N + 8, ldc=N + 40), base)


def test_deterministic_repeat(bg):
    A = dev_bf16(inputs.normal_bf16((100, 1024), 1.0, 41))
    B = dev_bf16(inputs.normal_bf16((1024, 512), 1.0, 42))
    c1 = bg.gemm_bf16(A, B)
    c2 = bg.gemm_bf16(A, B)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


# ------------------------------------------------------------------ invariance, small config


def _alone(bg, A, B):
    """Each row of A computed as its own M = 1 batch."""
    return torch.cat([bg.gemm_bf16(A[i:i + 1], B) for i in range(A.shape[0])])


def test_c1_invariance_and_parity(bg):
    # bf16 K=512, N=256, M in {1,3,8,17}; A,B ~ N(0,1)
    K, N = 512, 256
    pool = inputs.normal_bf16((17, K), 1.0, 101)
    Bc = inputs.normal_bf16((K, N), 1.0, 102)
    A = dev_bf16(pool)
    B = dev_bf16(Bc)
    ref = _alone(bg, A, B)
    C64, S = oracle.gemm_bf16(pool, Bc)
    check_parity(host_codes(ref), C64, S, K, "C1 rows alone")

    def check(idx, what):
        idx_t = torch.as_tensor(np.asarray(idx), device="cuda")
        out = bg.gemm_bf16(A.index_select(0, idx_t), B)
        ok = rows_equal(out, ref.index_select(0, idx_t))
        assert bool(ok.all()), f"{what}: rows {np.asarray(idx)[~ok.cpu().numpy()]} differ"

    check(np.arange(17), "M=17 in order")
    for r in range(17):
        check(np.roll(np.arange(17), r), f"rotation {r}")
    for s in range(8):
        check(inputs.permutation(17, 103 + s), f"permutation {s}")
    for m, seed in ((3, 104), (8, 105)):
        for j, sub in enumerate(inputs.random_subsets(17, m, 32, seed)):
            check(sub, f"M={m} subset {j}")
    # every position 0..63 of a 64-row batch (all residues mod 16 and 32)
    for pos in range(64):
        idx = np.array([(pos + 5 * t) % 17 for t in range(64)])
        idx[pos] = 0
        check(idx, f"row 0 at position {pos}")


# ------------------------------------------------------------------ C2 projection config


@pytest.fixture(scope="module")
def c2(bg):
    pool, Bc, _, _ = full_size.c2()
    return pool, Bc, dev_bf16(pool), dev_bf16(Bc)


def test_c2_invariance_all_m(bg, c2):
    pool, Bc, A, B = c2
    ref = _alone(bg, A, B)                     # 256 launches at M = 1
    for m in [2**i for i in range(9)]:
        out = bg.gemm_bf16(A[:m], B)
        ok = rows_equal(out, ref[:m])
        assert bool(ok.all()), f"M={m}: {int((~ok).sum())} rows differ"
    for s in range(4):
        p = torch.as_tensor(inputs.permutation(256, 203 + s), device="cuda")
        ok = rows_equal(bg.gemm_bf16(A.index_select(0, p), B), ref.index_select(0, p))
        assert bool(ok.all()), f"shuffle {s}"
    # lda = K + 64
    Ap = torch.zeros((256, 8192 + 64), dtype=torch.bfloat16, device="cuda")
    Ap[:, :8192] = A
    ok = rows_equal(bg.gemm_bf16(Ap[:, :8192], B), ref)
    assert bool(ok.all()), "lda = K + 64"
    # ragged M that are not powers of two
    for m in (3, 17, 37, 100, 129, 255):
        assert bool(rows_equal(bg.gemm_bf16(A[:m], B), ref[:m]).all()), f"M={m}"


def test_c2_parity_every_row(bg, c2):
    pool, Bc, A, B = c2
    _, _, C64, S = full_size.c2()
    C = host_codes(bg.gemm_bf16(A, B))       # the M = 256 batch, every row
    check_parity(full_size.all_rows(C, C64), C64, S, 8192, "C2 M=256 every row")


# ------------------------------------------------------------------ negative control


def test_splitk_comparator_is_flagged(bg, c2):
    """The split-K variant, whose split count follows M, must fail the same
    bitwise invariance check (else the checker is blind) while staying inside
    the tolerance."""
    pool, Bc, A, B = c2
    M = 16
    ws = torch.empty(M * 8192, dtype=torch.float32, device="cuda")
    alone = torch.cat([bg.gemm_bf16_splitk(A[i:i + 1], B, ws) for i in range(M)])
    batch = bg.gemm_bf16_splitk(A[:M], B, ws)
    torch.cuda.synchronize()
    assert bg.splitk_choose(1, 8192, 8192) != bg.splitk_choose(M, 8192, 8192)
    ok = rows_equal(alone, batch)
    assert not bool(ok.all()), "split-K with an M-dependent split passed the invariance check"
    C64, S = oracle.gemm_bf16(np.ascontiguousarray(pool[:2]), Bc)
    check_parity(host_codes(batch[:2]), C64, S, 8192, "split-K parity")
    # and the invariant kernel on the same rows is clean
    inv_alone = _alone(bg, A[:M], B)
    assert bool(rows_equal(inv_alone, bg.gemm_bf16(A[:M], B)).all())


# ------------------------------------------------------------------ transposed weight storage


@pytest.mark.parametrize("M,N,K", [(17, 256, 512), (37, 100, 203), (1, 8, 1), (65, 40, 129),
                                   (3, 2048, 7168), (16, 1000, 777), (9, 8200, 300),
                                   (4, 8192, 320), (7, 8192, 200), (6, 1000, 777), (8, 2048, 96),
                                   (40, 8200, 200), (64, 8192, 96), (200, 8200, 300), (130, 8192, 96),
                                   (130, 264, 1000), (1, 8192, 8192), (200, 96, 4096)])
def test_bt_bitwise_equal_to_rowmajor(bg, M, N, K):
    """Storing the weights transposed changes only the data movement: the same
    MFMA sequence per element must give identical bits."""
    A = inputs.normal_bf16((M, K), 1.0, 500 + M)
    B = inputs.normal_bf16((K, N), 1.0, 600 + N)
    lda = (K + 7) // 8 * 8
    ldb = (N + 7) // 8 * 8
    rm = run(bg, A, B, lda=lda, ldb=ldb, ldc=ldb)
    Ad = dev_bf16(A, lda)
    Bt = dev_bf16(np.ascontiguousarray(B.T), lda)
    bt = host_codes(bg.gemm_bf16_bt(Ad, Bt))
    assert np.array_equal(bt, rm)
    C64, S = oracle.gemm_bf16(A, B)
    check_parity(bt, C64, S, K, f"bt M{M} N{N} K{K}")


def test_bt_c2_invariance_all_m(bg, c2):
    pool, Bc, A, B = c2
    Bt = dev_bf16(np.ascontiguousarray(Bc.T))
    ref = torch.cat([bg.gemm_bf16_bt(A[i:i + 1], Bt) for i in range(256)])
    assert bool(rows_equal(ref, bg.gemm_bf16(A, B)).all()), "bt rows differ from row-major rows"
    for m in [2**i for i in range(9)] + [3, 17, 100, 255]:
        assert bool(rows_equal(bg.gemm_bf16_bt(A[:m], Bt), ref[:m]).all()), f"M={m}"
    p = torch.as_tensor(inputs.permutation(256, 207), device="cuda")
    assert bool(rows_equal(bg.gemm_bf16_bt(A.index_select(0, p), Bt), ref.index_select(0, p)).all())


# ------------------------------------------------------------------ packed weights


@pytest.mark.parametrize("M,N,K", [(17, 256, 512), (37, 100, 203), (1, 8, 1), (65, 40, 129),
                                   (3, 2048, 7168), (16, 1000, 777), (9, 8200, 300),
                                   (4, 8192, 320), (7, 8192, 200), (6, 1000, 777), (8, 2048, 96),
                                   (40, 8200, 200), (64, 8192, 96), (200, 8200, 300), (130, 8192, 96),
                                   (130, 264, 1000), (200, 96, 4096), (256, 2048, 512),
                                   (300, 4096, 256)])
def test_packed_bitwise_equal_to_rowmajor(bg, M, N, K):
    A = inputs.normal_bf16((M, K), 1.0, 700 + M)
    B = inputs.normal_bf16((K, N), 1.0, 800 + N)
    lda = (K + 7) // 8 * 8
    ldb = (N + 7) // 8 * 8
    rm = run(bg, A, B, lda=lda, ldb=ldb, ldc=ldb)
    Bp = bg.pack_b_bf16(dev_bf16(B, ldb))
    pk = host_codes(bg.gemm_bf16_packed(dev_bf16(A, lda), Bp))
    assert np.array_equal(pk, rm)


def test_packed_c2_all_geometries_bitwise(bg, c2):
    """Rows computed by the streaming geometry (M = 1), the medium and the large
    geometry (larger M) must be identical: the geometry follows M, the
    arithmetic does not."""
    pool, Bc, A, B = c2
    Bp = bg.pack_b_bf16(B)
    ref = torch.cat([bg.gemm_bf16_packed(A[i:i + 1], Bp) for i in range(256)])
    assert bool(rows_equal(ref, bg.gemm_bf16(A, B)).all())
    for m in [1, 2, 4, 8, 16, 32, 48, 64, 100, 128, 129, 192, 200, 256]:
        assert bool(rows_equal(bg.gemm_bf16_packed(A[:m], Bp), ref[:m]).all()), f"M={m}"
    for s in range(3):
        p = torch.as_tensor(inputs.permutation(256, 208 + s), device="cuda")
        assert bool(rows_equal(bg.gemm_bf16_packed(A.index_select(0, p), Bp),
                               ref.index_select(0, p)).all()), f"shuffle {s}"
    # every row computed alone (M = 1), which all the comparisons above use
    _, _, C64, S = full_size.c2()
    check_parity(full_size.all_rows(host_codes(ref), C64), C64, S, 8192, "packed C2 rows at M=1")
