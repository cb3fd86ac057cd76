"""Library launches captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must reproduce the eager result bit for bit.  The
replays are separated by eager work that overwrites the outputs (and the
split-K workspace), so a replay that skipped or reordered a kernel -- the
split-K zero-fill included -- would show."""
import numpy as np
import pytest
import torch

from invariant_gemm_amd import inputs
from tests.gpu_util import dev_bf16, dev_f32, dev_u8, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    require_gpu()
    from invariant_gemm_amd import bigemm
    return bigemm


def replay_matches_eager(calls, outs, extra=(), inexact=()):
    """`inexact`: indices of outputs whose bits legitimately vary from run to
    run (the split-K comparator's atomics); those are compared within a
    tolerance instead, which still catches a skipped zero-fill (NaN) or a
    doubled accumulation."""
    for f in calls:
        f()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in calls:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    for r in range(4):
        for o in list(outs) + list(extra):
            o.fill_(float("nan") if o.is_floating_point() else 7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            if i in inexact:
                assert torch.allclose(o.float(), e.float(), rtol=2**-7, atol=1e-3), f"replay {r}: output {i}"
            else:
                assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {r}: output {i} differs"


def test_graph_replay_all_entry_points(bg):
    M, N, K = 37, 272, 512
    A = dev_bf16(inputs.normal_bf16((M, K), 1.0, 901))
    B = dev_bf16(inputs.normal_bf16((K, N), 0.02, 902))
    Bt = B.t().contiguous()
    Bp = bg.pack_b_bf16(B)
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((M, K), 1.0, 903))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((K, N), 1.0, 904))
    A8, sA8, B8, sB8 = dev_u8(qA), dev_f32(sA), dev_u8(qB), dev_f32(sB)
    Bp8 = bg.pack_b_fp8(B8)
    Bq, s4 = inputs.quant_fp4_weights(inputs.normal_f32((K, N), 0.02, 905))
    Bq4, s44 = dev_u8(Bq, (N // 2 + 15) // 16 * 16), dev_u8(s4)   # code rows padded to 16 B
    Bp4 = bg.pack_b_fp4(Bq4, s44, N)
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(8)]
    ws = torch.empty(M * N, dtype=torch.float32, device="cuda")
    calls = [
        lambda: bg.gemm_bf16(A, B, out=outs[0]),
        lambda: bg.gemm_bf16_bt(A, Bt, out=outs[1]),
        lambda: bg.gemm_bf16_packed(A, Bp, out=outs[2]),
        lambda: bg.gemm_fp8_blockscaled(A8, sA8, B8, sB8, out=outs[3]),
        lambda: bg.gemm_fp8_blockscaled_packed(A8, sA8, Bp8, sB8, out=outs[4]),
        lambda: bg.gemm_fp4_w(A, Bq4, s44, N, out=outs[5]),
        lambda: bg.gemm_fp4_w_packed(A, Bp4, out=outs[6]),
        lambda: bg.gemm_bf16_splitk(A, B, ws, 4, out=outs[7]),
    ]
    replay_matches_eager(calls, outs, extra=[ws], inexact=(7,))
    # identical bits across the three bf16 layouts and across packed/unpacked
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    assert torch.equal(outs[3].view(torch.int16), outs[4].view(torch.int16))
    assert torch.equal(outs[5].view(torch.int16), outs[6].view(torch.int16))
    assert not np.isnan(outs[7].float().cpu().numpy()).any()
