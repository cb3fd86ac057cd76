#!/usr/bin/env python3
"""Throughput of the batch-invariant GEMMs on one MI355X against its roofline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--quick]

Headline workload (one "step"): the bf16 projection GEMM, K = N = 8192,
weights B ~ N(0, 0.02), activations A ~ N(0, 1), swept over
M = 1, 2, 4, ..., 256 -- nine launches of bi_gemm_bf16_packed, one per M, on
weights packed once (outside the timed region) into the MFMA operand order;
the packed path returns the same bits as bi_gemm_bf16 on the row-major
weights.  Every launch reads a different copy of (A, B) from a rotation of
more than 1 GiB, so B comes from HBM and not from the 256 MB Infinity Cache.
Inputs are resident in HBM before the timed region starts.  `value` is
whole-job TFLOP/s over the timed steps (2MNK per launch).

The same JSON line carries, per M: launch time, TFLOP/s, algorithmic GB/s and
the fractions of the HBM and MFMA roofs and of the attainable roof
(min over both); the fp8 block-scaled (K=7168, N=2048) and fp4 weight-only
(K=4096, N=14336) sweeps; the dynamic-batching replay; the gap against the
non-invariant split-K comparator; and the fp64 oracle timed on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0                      # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # dense, published
ROT_BYTES = 1 << 30                        # rotation footprint (> 2 x (MALL + L2))
ROOT = os.path.dirname(os.path.abspath(__file__))

SWEEP_C2 = [1, 2, 4, 8, 16, 32, 64, 128, 256]
SWEEP_C3 = [1, 2, 4, 8, 16, 32, 37, 64, 128, 129, 256, 512]
SWEEP_C4 = [1, 8, 64, 512]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops(M, N, K):
    return 2.0 * M * N * K


# algorithmic bytes: each operand once, plus the output
def bytes_bf16(M, N, K):
    return 2 * M * K + 2 * K * N + 2 * M * N


def bytes_fp8(M, N, K):
    kb, nb = K // 128, (N + 127) // 128
    return M * K + 4 * M * kb + K * N + 4 * kb * nb + 2 * M * N


def bytes_fp4(M, N, K):
    return 2 * M * K + K * N // 2 + (K // 32) * N + 2 * M * N


def roof(M, N, K, nbytes, t_us, mfma_peak):
    f = flops(M, N, K)
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), f / (mfma_peak * 1e12)) * 1e6
    return {"us": round(t_us, 2), "tflops": round(f / t_us / 1e6, 2),
            "gbs": round(nbytes / t_us / 1e3, 1),
            "frac_hbm": round(nbytes / t_us / 1e3 / HBM_PEAK_GBS, 4),
            "frac_mfma": round(f / t_us / 1e6 / mfma_peak, 4),
            "frac_attainable": round(t_roof / t_us, 4),
            "bound": "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= f / (mfma_peak * 1e12) else "mfma"}


def capture(torch, fn, n):
    """A HIP graph of n calls of fn (each call enqueues library kernels on
    torch's current stream).  Replaying it puts the launches on the GPU
    back-to-back, so a timing measures the kernels and not the host's
    per-call launch rate (several microseconds per ctypes call)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return g


def time_launches(torch, fn, reps, rounds):
    """Median and min per-launch time (us) over `rounds` replays of a graph of
    `reps` back-to-back launches, measured with HIP events on the stream the
    kernels run on."""
    g = capture(torch, fn, reps)
    per = []
    for _ in range(rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / reps)
    del g
    per.sort()
    return per[len(per) // 2], per[0]


def rotation(one_copy_bytes):
    return max(2, -(-ROT_BYTES // one_copy_bytes))


# ------------------------------------------------------------------ workloads

class C2:
    """bf16 projection GEMM K=N=8192, A ~ N(0,1) [256 rows], B ~ N(0,0.02)."""
    K = N = 8192

    def __init__(self, torch, bg, inputs):
        self.torch, self.bg = torch, bg
        pool = inputs.normal_bf16((256, self.K), 1.0, 201)
        Bc = inputs.normal_bf16((self.K, self.N), 0.02, 202)
        A0 = torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).cuda()
        B0 = torch.from_numpy(Bc.view(np.int16)).view(torch.bfloat16).cuda()
        self.nbuf = rotation(self.K * self.N * 2)
        self.A = [A0.clone() for _ in range(self.nbuf)]
        self.B = [B0.clone() for _ in range(self.nbuf)]
        self.C = torch.empty((256, self.N), dtype=torch.bfloat16, device="cuda")
        self.i = 0

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_bf16(self.A[j][:M], self.B[j], out=self.C[:M])

    def launch_splitk(self, M, ws):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_bf16_splitk(self.A[j][:M], self.B[j], ws, 0, out=self.C[:M])

    def step(self):
        for M in SWEEP_C2:
            self.launch(M)


class C2T(C2):
    """The same projection GEMM with the weights stored transposed (Bt [N,K])."""

    def __init__(self, torch, bg, inputs):
        super().__init__(torch, bg, inputs)
        self.B = [b.t().contiguous() for b in self.B]
        torch.cuda.synchronize()

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_bf16_bt(self.A[j][:M], self.B[j], out=self.C[:M])


class C2P(C2):
    """The same projection GEMM on weights packed once into the MFMA order."""

    def __init__(self, torch, bg, inputs):
        super().__init__(torch, bg, inputs)
        t0 = time.perf_counter()
        self.Bp = [bg.pack_b_bf16(b) for b in self.B]
        torch.cuda.synchronize()
        self.pack_ms = (time.perf_counter() - t0) * 1e3 / len(self.B)
        self.B = None

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_bf16_packed(self.A[j][:M], self.Bp[j], out=self.C[:M])


class C3:
    """fp8 e4m3 K=7168, N=2048, 1x128 / 128x128 fp32 scales, values N(0,1)."""
    K, N = 7168, 2048

    def __init__(self, torch, bg, inputs):
        self.bg = bg
        qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((512, self.K), 1.0, 301))
        qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((self.K, self.N), 1.0, 302))
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        self.nbuf = rotation(qB.nbytes)
        self.A = [t(qA) for _ in range(self.nbuf)]
        self.sA = [t(sA) for _ in range(self.nbuf)]
        self.B = [t(qB) for _ in range(self.nbuf)]
        self.sB = [t(sB) for _ in range(self.nbuf)]
        self.C = torch.empty((512, self.N), dtype=torch.bfloat16, device="cuda")
        self.i = 0

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_fp8_blockscaled(self.A[j][:M], self.sA[j][:M], self.B[j], self.sB[j],
                                     out=self.C[:M])


class C3P(C3):
    """The fp8 workload on weights packed once into the MFMA order."""

    def __init__(self, torch, bg, inputs):
        super().__init__(torch, bg, inputs)
        t0 = time.perf_counter()
        self.Bp = [bg.pack_b_fp8(b) for b in self.B]
        torch.cuda.synchronize()
        self.pack_ms = (time.perf_counter() - t0) * 1e3 / len(self.B)
        self.B = None

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_fp8_blockscaled_packed(self.A[j][:M], self.sA[j][:M], self.Bp[j], self.sB[j],
                                            out=self.C[:M])


class C4:
    """fp4 e2m1 weight-only K=4096, N=14336, e4m3 scales per 32 K, W ~ N(0,0.02)."""
    K, N = 4096, 14336

    def __init__(self, torch, bg, inputs):
        self.bg = bg
        A = inputs.normal_bf16((512, self.K), 1.0, 401)
        Bq, sB = inputs.quant_fp4_weights(inputs.normal_f32((self.K, self.N), 0.02, 402))
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        self.nbuf = rotation(Bq.nbytes + sB.nbytes)
        self.A = [t(A.view(np.int16)).view(torch.bfloat16) for _ in range(self.nbuf)]
        self.B = [t(Bq) for _ in range(self.nbuf)]
        self.sB = [t(sB) for _ in range(self.nbuf)]
        self.C = torch.empty((512, self.N), dtype=torch.bfloat16, device="cuda")
        self.i = 0

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_fp4_w(self.A[j][:M], self.B[j], self.sB[j], self.N, out=self.C[:M])


class C4P(C4):
    """The fp4 workload on codes and scales packed once into the MFMA order."""

    def __init__(self, torch, bg, inputs):
        super().__init__(torch, bg, inputs)
        t0 = time.perf_counter()
        self.Bp = [bg.pack_b_fp4(b, s, self.N) for b, s in zip(self.B, self.sB)]
        torch.cuda.synchronize()
        self.pack_ms = (time.perf_counter() - t0) * 1e3 / len(self.B)
        self.B = self.sB = None

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_fp4_w_packed(self.A[j][:M], self.Bp[j], out=self.C[:M])


def bytes_w4a8(M, N, K):
    return M * K + 4 * M * (K // 128) + K * N // 2 + (K // 32) * N + 2 * M * N


class W4A8:
    """fp8 e4m3 activations (1x128 fp32 scales) x OCP MXFP4 weights, the fp4
    weight shape K=4096, N=14336; weights ~ N(0,0.02) before quantisation."""
    K, N = 4096, 14336
    SWEEP = [1, 8, 64, 512]

    def __init__(self, torch, bg, inputs):
        self.bg = bg
        qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((512, self.K), 1.0, 701))
        Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((self.K, self.N), 0.02, 702))
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        one = bg.pack_b_mxfp4(t(Bq), t(sE), self.N)
        self.nbuf = rotation(one.data.numel())
        self.Bp = [one] + [bg.PackedWeights(one.dtype, one.K, one.N, one.data.clone())
                           for _ in range(self.nbuf - 1)]
        self.A, self.sA = t(qA), t(sA)
        self.C = torch.empty((512, self.N), dtype=torch.bfloat16, device="cuda")
        self.i = 0

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_w4a8_packed(self.A[:M], self.sA[:M], self.Bp[j], out=self.C[:M])


class MoE:
    """Grouped (mixture-of-experts) bf16 GEMM: E = 8 experts, K = 7168,
    N = 2048, T tokens routed top-1 uniformly (seeded), rows grouped by
    expert; packed expert weights rotated over HBM copies."""
    E, K, N = 8, 7168, 2048
    SWEEP = [1, 8, 64, 512]

    def __init__(self, torch, bg, inputs):
        self.torch, self.bg = torch, bg
        A = inputs.normal_bf16((max(self.SWEEP), self.K), 1.0, 601)
        self.A = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).cuda()
        Bs = [torch.from_numpy(inputs.normal_bf16((self.K, self.N), 0.02, 602 + e).view(np.int16))
              .view(torch.bfloat16).cuda() for e in range(self.E)]
        one = bg.pack_b_bf16_grouped(Bs)
        del Bs
        self.nbuf = rotation(one.data.numel())
        self.Bp = [one] + [bg.PackedWeights(one.dtype, one.K, one.N, one.data.clone())
                           for _ in range(self.nbuf - 1)]
        for b in self.Bp:
            b.groups = self.E
        self.routes = {}
        for T in self.SWEEP:
            expert = inputs.route_tokens(T, self.E, 603 + T, 0.0)
            order, offsets = inputs.group_by_expert(expert, self.E)
            self.routes[T] = (self.A[:T].index_select(0, torch.as_tensor(order, device="cuda")),
                              torch.as_tensor(offsets, device="cuda"), int(np.count_nonzero(np.diff(offsets))))
        self.C = torch.empty((max(self.SWEEP), self.N), dtype=torch.bfloat16, device="cuda")
        self.i = 0

    def launch(self, T):
        j = self.i % self.nbuf
        self.i += 1
        A, off, _ = self.routes[T]
        self.bg.gemm_bf16_grouped_packed(A, off, self.Bp[j], out=self.C[:T])

    def nbytes(self, T, N, K):
        return self.routes[T][2] * K * N * 2 + 2 * T * K + 2 * T * N


class MoE8:
    """Grouped (mixture-of-experts) fp8 block-scaled GEMM: E = 8 experts,
    K = 7168, N = 2048, e4m3fn activations with 1x128 scales, e4m3fn weights
    with 128x128 scales, T tokens routed top-1 uniformly (seeded); packed
    expert weights rotated over HBM copies."""
    E, K, N = 8, 7168, 2048
    SWEEP = [1, 8, 64, 512]

    def __init__(self, torch, bg, inputs):
        self.torch, self.bg = torch, bg
        T = max(self.SWEEP)
        qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((T, self.K), 1.0, 611))
        self.A = torch.from_numpy(qA).cuda()
        self.sA = torch.from_numpy(sA).cuda()
        Bs, sBs = [], []
        for e in range(self.E):
            qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((self.K, self.N), 1.0, 612 + e))
            Bs.append(torch.from_numpy(qB).cuda())
            sBs.append(sB)
        one = bg.pack_b_fp8_grouped(Bs)
        del Bs
        self.sB = torch.from_numpy(np.concatenate(sBs, axis=0)).cuda()
        self.nbuf = rotation(one.data.numel())
        self.Bp = [one] + [bg.PackedWeights(one.dtype, one.K, one.N, one.data.clone())
                           for _ in range(self.nbuf - 1)]
        for b in self.Bp:
            b.groups = self.E
        self.routes = {}
        for t in self.SWEEP:
            expert = inputs.route_tokens(t, self.E, 613 + t, 0.0)
            order, offsets = inputs.group_by_expert(expert, self.E)
            perm = torch.as_tensor(order, device="cuda")
            self.routes[t] = (self.A[:t].index_select(0, perm), self.sA[:t].index_select(0, perm),
                              torch.as_tensor(offsets, device="cuda"),
                              int(np.count_nonzero(np.diff(offsets))))
        self.C = torch.empty((T, self.N), dtype=torch.bfloat16, device="cuda")
        self.i = 0

    def launch(self, T):
        j = self.i % self.nbuf
        self.i += 1
        A, sA, off, _ = self.routes[T]
        self.bg.gemm_fp8_blockscaled_grouped_packed(A, sA, off, self.Bp[j], self.sB, out=self.C[:T])

    def nbytes(self, T, N, K):
        hit = self.routes[T][3]
        return bytes_fp8(T, N, K) - K * N - 4 * (K // 128) * ((N + 127) // 128) + \
            hit * (K * N + 4 * (K // 128) * ((N + 127) // 128))


class MoEW4A8:
    """Grouped (mixture-of-experts) W4A8 GEMM: E = 8 experts, K = 7168,
    N = 2048, e4m3fn activations with 1x128 scales, OCP MXFP4 expert weights
    (N(0, 0.02) before quantisation), T tokens routed top-1 uniformly (seeded);
    packed expert weights rotated over HBM copies."""
    E, K, N = 8, 7168, 2048
    SWEEP = [1, 8, 64, 512]

    def __init__(self, torch, bg, inputs):
        self.torch, self.bg = torch, bg
        T = max(self.SWEEP)
        qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((T, self.K), 1.0, 621))
        self.A = torch.from_numpy(qA).cuda()
        self.sA = torch.from_numpy(sA).cuda()
        Bqs, sEs = [], []
        for e in range(self.E):
            Bq, sE = inputs.quant_mxfp4_weights(inputs.normal_f32((self.K, self.N), 0.02, 622 + e))
            Bqs.append(torch.from_numpy(Bq).cuda())
            sEs.append(torch.from_numpy(sE).cuda())
        one = bg.pack_b_mxfp4_grouped(Bqs, sEs, self.N)
        del Bqs, sEs
        self.nbuf = rotation(one.data.numel())
        self.Bp = [one] + [bg.PackedWeights(one.dtype, one.K, one.N, one.data.clone())
                           for _ in range(self.nbuf - 1)]
        for b in self.Bp:
            b.groups = self.E
        self.routes = {}
        for t in self.SWEEP:
            expert = inputs.route_tokens(t, self.E, 623 + t, 0.0)
            order, offsets = inputs.group_by_expert(expert, self.E)
            perm = torch.as_tensor(order, device="cuda")
            self.routes[t] = (self.A[:t].index_select(0, perm), self.sA[:t].index_select(0, perm),
                              torch.as_tensor(offsets, device="cuda"),
                              int(np.count_nonzero(np.diff(offsets))))
        self.C = torch.empty((T, self.N), dtype=torch.bfloat16, device="cuda")
        self.i = 0

    def launch(self, T):
        j = self.i % self.nbuf
        self.i += 1
        A, sA, off, _ = self.routes[T]
        self.bg.gemm_w4a8_grouped_packed(A, sA, off, self.Bp[j], out=self.C[:T])

    def nbytes(self, T, N, K):
        hit = self.routes[T][3]
        w = K * N // 2 + (K // 32) * N
        return bytes_w4a8(T, N, K) - w + hit * w


# ------------------------------------------------------------------ cpu baseline

def cpu_baseline(budget_s=12.0):
    """The fp64 oracle as it stands, on the host cores, on a bounded sample of
    the headline workload (rows of the M = 256 batch, full N and K)."""
    import oracle
    from invariant_gemm_amd import inputs
    K, N = C2.K, C2.N
    pool = inputs.normal_bf16((256, K), 1.0, 201)
    Bc = inputs.normal_bf16((K, N), 0.02, 202)
    rows, t_tot, r = 0, 0.0, 0
    while t_tot < budget_s and rows < 256:
        A = np.ascontiguousarray(pool[r:r + 8])
        t0 = time.perf_counter()
        oracle.gemm_bf16(A, Bc)
        t_tot += time.perf_counter() - t0
        rows += A.shape[0]
        r += 8
    fl = flops(rows, N, K)
    out = {"value": round(fl / t_tot / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "kind": "oracle",
           "sample": f"fp64 oracle on {rows} rows of the M=256 bf16 batch (K=N=8192): "
                     f"{fl / 1e9:.1f} GFLOP in {t_tot:.2f} s"}
    # the same oracle on one host thread, on a smaller sample of the same rows
    n_threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        A = np.ascontiguousarray(pool[:4])
        t0 = time.perf_counter()
        oracle.gemm_bf16(A, Bc)
        t1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(n_threads)
    out["value_1core"] = round(flops(4, N, K) / t1 / 1e12, 6)
    out["sample_1core"] = (f"fp64 oracle, one thread, on 4 rows of the same batch: "
                           f"{flops(4, N, K) / 1e9:.2f} GFLOP in {t1:.2f} s")
    out["host"] = host_info()
    out["formats"] = cpu_baseline_formats()
    return out


def cpu_baseline_formats(budget_s=3.0):
    """The same oracle on the quantised configurations, on a few rows each
    (the fp64 work per row is fixed by N and K): fp8 block-scaled K = 7168,
    N = 2048 and fp4 weight-only K = 4096, N = 14336, seeded as the GPU legs."""
    import oracle
    from invariant_gemm_amd import inputs
    res = {}
    qA, sA = inputs.quant_fp8_rowblocks(inputs.normal_f32((16, 7168), 1.0, 301))
    qB, sB = inputs.quant_fp8_tiles(inputs.normal_f32((7168, 2048), 1.0, 302))
    A4 = inputs.normal_bf16((16, 4096), 1.0, 401)
    Bq, s4 = inputs.quant_fp4_weights(inputs.normal_f32((4096, 14336), 0.02, 402))
    for name, N, K, run in (
            ("fp8_blockscaled_K7168_N2048", 2048, 7168,
             lambda a, b: oracle.gemm_fp8bs(np.ascontiguousarray(qA[a:b]), np.ascontiguousarray(sA[a:b]), qB, sB)),
            ("fp4_weight_only_K4096_N14336", 14336, 4096,
             lambda a, b: oracle.gemm_fp4w(np.ascontiguousarray(A4[a:b]), Bq, s4, 14336))):
        rows, t_tot = 0, 0.0
        while t_tot < budget_s and rows < 16:
            t0 = time.perf_counter()
            run(rows, rows + 2)
            t_tot += time.perf_counter() - t0
            rows += 2
        res[name] = {"value": round(flops(rows, N, K) / t_tot / 1e12, 5), "unit": "TFLOP/s",
                     "sample": f"fp64 oracle on {rows} rows: {flops(rows, N, K) / 1e9:.2f} GFLOP "
                               f"in {t_tot:.2f} s"}
    return res


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


# ------------------------------------------------------------------ device and HBM context

def device_info(torch):
    """Name, architecture and compute units of GPU 0, plus the clock levels
    rocm-smi reports (read only; clocks are not locked)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2**30, 1)}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=30)
        card = next(iter(json.loads(r.stdout).values()))
        info["clocks"] = {k: v for k, v in card.items()
                          if any(c in k for c in ("sclk", "mclk", "fclk")) and "speed" in k}
    except Exception as e:          # informational only
        info["clocks"] = f"unavailable ({type(e).__name__})"
    return info


def measured_roof(torch, bg, rounds=5):
    """The measured roofs the kernels are compared with, from the library's
    own probes (bi_probe_stream_read, bi_probe_empty), timed like the GEMM
    legs (graph replay of back-to-back launches, buffers rotated so that no
    launch finds its data in the 256 MB Infinity Cache):

    * read roof: one 128 MiB stream per launch (the size of the K = N = 8192
      bf16 weights) over 8 rotated buffers, for 256..2048 workgroups, 4 or 8
      loads in flight per thread, default or non-temporal loads -- the best
      configuration is the measured roof; the same configuration over one
      1 GiB buffer;
    * small streams: 14.7 MB (the fp8 K = 7168, N = 2048 weights) and 31.2 MB
      (the fp4 K = 4096, N = 14336 codes and scales) read by 256 workgroups,
      rotated over windows of 1 GiB -- the floor a GEMM streaming that many
      bytes cannot beat;
    * launch floor: back-to-back launches of an empty kernel."""
    one, nbuf = 128 << 20, 8
    bufs = [torch.zeros(one, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sink = torch.zeros(2048 * 256, dtype=torch.int32, device="cuda")
    state = {"i": 0}

    def reader(views, wg, flags):
        def fn():
            v = views[state["i"] % len(views)]
            state["i"] += 1
            bg.probe_stream_read(v, wg, flags, sink)
        return fn

    best = None
    table = {}
    for wg in (256, 512, 1024, 2048):
        for flags, name in ((0, "default"), (bg.PROBE_NONTEMPORAL, "nt"),
                            (bg.PROBE_UNROLL8, "default_u8"),
                            (bg.PROBE_NONTEMPORAL | bg.PROBE_UNROLL8, "nt_u8")):
            med, mn = time_launches(torch, reader(bufs, wg, flags), reps=nbuf, rounds=rounds)
            gbs = one / (med * 1e3)
            table[f"wg{wg}_{name}"] = round(gbs, 1)
            if best is None or gbs > best[0]:
                best = (gbs, wg, flags, med)
    del bufs
    big = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    med1g, _ = time_launches(torch, reader([big], best[1], best[2]), reps=2, rounds=rounds)
    small = {}
    for label, nbytes in (("fp8_weights_14.7MB", 7168 * 2048),
                          ("fp4_weights_31.2MB", 4096 * 14336 // 2 + (4096 // 32) * 14336)):
        nb = (nbytes + 4095) // 4096 * 4096
        views = [big[k * nb:(k + 1) * nb] for k in range(min(64, (1 << 30) // nb))]
        med, mn = time_launches(torch, reader(views, 256, best[2]), reps=len(views), rounds=rounds)
        small[label] = {"bytes": nbytes, "us": round(med, 2), "us_min": round(mn, 2),
                        "GBps": round(nbytes / (med * 1e3), 1)}
    del big
    emp, emp_min = time_launches(torch, bg.probe_empty, reps=200, rounds=rounds)
    return {"read_roof_GBps": round(best[0], 1),
            "read_roof_config": {"workgroups": best[1], "flags": best[2],
                                 "us_per_128MiB": round(best[3], 2)},
            "read_1GiB_GBps": round((1 << 30) / (med1g * 1e3), 1),
            "read_128MiB_GBps_by_config": table,
            "small_streams": small,
            "empty_launch_us": round(emp, 3), "empty_launch_us_min": round(emp_min, 3),
            "note": "bi_probe_stream_read / bi_probe_empty, graph replay, HIP events on the "
                    "launch stream; the nominal HBM peak is 8000 GB/s"}


def single_launch_us(torch, fn, n=15):
    """Median time of one eager launch between HIP events on its stream
    (launch overhead included), each launch after a full synchronisation."""
    t = []
    for _ in range(n):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3)
    t.sort()
    return round(t[len(t) // 2], 2)


# ------------------------------------------------------------------ traffic evidence

def kernel_sha256(paths) -> str:
    """SHA-256 over the kernel's source files, in order."""
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def traffic_from_profiles(kernel_src):
    """Measured HBM bytes per launch of the headline sweep, from the committed
    rocprofv3 --pmc summary, if that summary was taken on the current kernel
    source; else None."""
    p = os.path.join(ROOT, "profiles", "gemm_bf16_packed_c2_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    h = kernel_sha256(kernel_src)
    if d.get("kernel_sha256") != h:
        return None
    return d.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20


def pmc_probe(torch, wl):
    """Launch sequence for the HBM-traffic counters: a plain device copy of
    COPY_BYTES (the calibration reference: it must fetch and write exactly
    that many bytes), then three launches per M of the headline sweep, each on
    a different rotated copy of B."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    for M in SWEEP_C2:
        for _ in range(3):
            wl.launch(M)
    torch.cuda.synchronize()
    log("pmc probe done: copy", COPY_BYTES, "bytes x3, then 3 launches per M", SWEEP_C2)


def pmc_summary(fetch_dir: str, write_dir: str):
    """Turn the counter CSVs of the two `rocprofv3 --pmc` runs of
    `--pmc-probe` (FETCH_SIZE, then WRITE_SIZE) into HBM bytes per launch of
    the headline sweep.  Each counter is calibrated on the probe's copy of
    COPY_BYTES (which must read and write exactly that many bytes)."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = int(r["Dispatch_Id"])
                name, v = vals.get(key, (r["Kernel_Name"], 0.0))
                vals[key] = (name, v + float(r["Counter_Value"]))
        return [vals[k] for k in sorted(vals)]

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = per_dispatch(d, counter)
        first = next(i for i, (n, _) in enumerate(rows) if "gemm_bf16_packed_kernel" in n)
        # the probe's three calibration copies are the last copy dispatches
        # before the first GEMM (set-up clones of A and B come earlier)
        copies = [v for n, v in rows[:first] if "copy" in n.lower()][-3:]
        gemms = [v for n, v in rows if "gemm_bf16_packed_kernel" in n]
        if len(copies) != 3 or len(gemms) != 3 * len(SWEEP_C2):
            raise SystemExit(f"{counter}: {len(copies)} copy and {len(gemms)} GEMM dispatches "
                             f"(expected 3 and {3 * len(SWEEP_C2)})")
        copy_kib = sorted(copies)[len(copies) // 2]
        factor = COPY_BYTES / (copy_kib * 1024.0)
        per_m = {}
        for i, M in enumerate(SWEEP_C2):
            v = sorted(gemms[3 * i:3 * i + 3])[1]
            per_m[str(M)] = round(v * 1024.0 * factor)
        out[counter] = {"copy_kib_per_dispatch": copy_kib, "scale_factor": round(factor, 4),
                        "bytes_per_launch": per_m}
    K, N = C2.K, C2.N
    fetch = out["FETCH_SIZE"]["bytes_per_launch"]
    write = out["WRITE_SIZE"]["bytes_per_launch"]
    per_m = {m: {"hbm_bytes": fetch[m] + write[m], "fetch_bytes": fetch[m], "write_bytes": write[m],
                 "algorithmic_bytes": bytes_bf16(int(m), N, K)} for m in fetch}
    total = sum(v["hbm_bytes"] for v in per_m.values())
    src = [os.path.join(ROOT, "invariant_gemm_amd", "csrc", f) for f in ("gemm_bf16_packed.hip", "common.h")]
    return {"kernel": "gemm_bf16_packed_kernel (bi_gemm_bf16_packed)",
            "kernel_sha256": kernel_sha256(src),
            "workload": "bf16 K=N=8192, M = 1,2,4,...,256, B packed, rotated copies",
            "hbm_bytes_per_launch": round(total / len(per_m)),
            "algorithmic_bytes_per_launch": round(sum(v["algorithmic_bytes"] for v in per_m.values())
                                                  / len(per_m)),
            "per_m": per_m, "calibration": {k: {kk: vv for kk, vv in v.items() if kk != "bytes_per_launch"}
                                            for k, v in out.items()}}


def legs_pmc():
    """(name, kernel name prefix, workload class, M sweep, algorithmic bytes)
    of the quantised legs whose HBM traffic the counters check (the prefix
    matches a format's staged and unstaged kernels alike)."""
    return (("fp8_blockscaled_packed_K7168_N2048", "gemm_fp8_packed_", C3P, SWEEP_C3, bytes_fp8),
            ("fp4_weight_only_packed_K4096_N14336", "gemm_fp4_packed_", C4P, SWEEP_C4, bytes_fp4),
            ("w4a8_mxfp4_K4096_N14336", "gemm_w4a8_packed_", W4A8, W4A8.SWEEP, bytes_w4a8))


def pmc_probe_legs(torch, bg, inputs):
    """Launch sequence for the quantised legs' HBM-traffic counters: after the
    first leg's set-up, a device copy of COPY_BYTES (the calibration
    reference), then per leg three launches per M of its sweep, each on a
    different rotated copy of the weights."""
    for i, (name, _, cls, sweep_ms, _) in enumerate(legs_pmc()):
        wl = cls(torch, bg, inputs)
        torch.cuda.synchronize()
        if i == 0:
            src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        for M in sweep_ms:
            for _ in range(3):
                wl.launch(M)
        torch.cuda.synchronize()
        del wl
        log("pmc legs probe:", name, "3 launches per M", sweep_ms)


def pmc_summary_legs(fetch_dir: str, write_dir: str):
    """HBM bytes per launch of the quantised legs from the FETCH_SIZE and
    WRITE_SIZE runs of `--pmc-probe-legs`, calibrated on the probe's copy, beside
    each launch's algorithmic bytes."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = int(r["Dispatch_Id"])
                name, v = vals.get(key, (r["Kernel_Name"], 0.0))
                vals[key] = (name, v + float(r["Counter_Value"]))
        return [vals[k] for k in sorted(vals)]

    legs = legs_pmc()
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = per_dispatch(d, counter)
        first = next(i for i, (n, _) in enumerate(rows) if legs[0][1] in n)
        copies = [v for n, v in rows[:first] if "copy" in n.lower()][-3:]
        if len(copies) != 3:
            raise SystemExit(f"{counter}: {len(copies)} calibration copies before the first launch")
        factor = COPY_BYTES / (sorted(copies)[1] * 1024.0)
        for name, kern, cls, sweep_ms, nbytes in legs:
            vals = [v for n, v in rows if kern in n]
            if len(vals) != 3 * len(sweep_ms):
                raise SystemExit(f"{counter} {name}: {len(vals)} dispatches (expected {3 * len(sweep_ms)})")
            leg = out.setdefault(name, {})
            for i, M in enumerate(sweep_ms):
                v = sorted(vals[3 * i:3 * i + 3])[1] * 1024.0 * factor
                leg.setdefault(str(M), {})[counter] = round(v)
        out.setdefault("calibration", {})[counter] = {"scale_factor": round(factor, 4)}
    for name, kern, cls, sweep_ms, nbytes in legs:
        for M in sweep_ms:
            e = out[name][str(M)]
            alg = nbytes(M, cls.N, cls.K)
            e["hbm_bytes"] = e["FETCH_SIZE"] + e["WRITE_SIZE"]
            e["algorithmic_bytes"] = alg
            e["ratio"] = round(e["hbm_bytes"] / alg, 3)
    return out


SIMDS, CUS, CLOCK_GHZ = 1024, 256, 2.4     # MI355X: 256 compute units x 4 SIMDs, peak clock


def pmc_counters(dirs):
    """Per-M medians of every counter in `rocprofv3 --pmc` runs of
    `--pmc-probe` (three launches per M of the headline sweep), with the
    dispatches' own durations, and the ratios the kernel notes use:
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x duration x 2.4 GHz)
    (the counter sums over all SIMDs); wave time waiting on anything /
    unable to issue its next instruction = SQ_WAIT_ANY / SQ_WAVE_CYCLES and
    SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; LDS bank conflicts per active LDS
    cycle; L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS); texture-address stall
    = TA_ADDR_STALLED_BY_TC_CYCLES / (CUs x duration x 2.4 GHz)."""
    import csv
    import glob
    res = _counters_per_m(dirs, [("gemm_bf16_packed_kernel", SWEEP_C2)], csv, glob)[0]
    # MFMA work actually issued (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts 512 flops)
    # against 2MNK: every 16 x 16 block of a tile runs its whole K chain once,
    # so the ratio is the tile's rows over M (16-row blocks at M < 16)
    for M, row in res["per_m"].items():
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in row:
            fl = row["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
            row["derived"]["mfma_flops"] = fl
            row["derived"]["mfma_flops_over_2mnk"] = round(fl / flops(int(M), C2.N, C2.K), 4)
    return res | {
        "kernel": "gemm_bf16_packed_kernel (bi_gemm_bf16_packed)",
        "kernel_sha256": kernel_sha256([os.path.join(ROOT, "invariant_gemm_amd", "csrc", f)
                                        for f in ("gemm_bf16_packed.hip", "common.h")])}


def pmc_counters_legs(dirs):
    """The same per-M counter summary for the runs of `--pmc-probe-legs`,
    with the MFMA work issued (SQ_INSTS_VALU_MFMA_MOPS_* count 512 flops each:
    bf16 for the fp4 weight-only kernel, whose codes enter the MFMA as bf16;
    fp8 and f6f4 for the scaled f8f6f4 MFMAs) against 2MNK."""
    import csv
    import glob
    legs = legs_pmc()
    res = _counters_per_m(dirs, [(kern, sweep_ms) for _, kern, _, sweep_ms, _ in legs], csv, glob)
    mops = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4")
    for (_, _, cls, _, _), r in zip(legs, res):
        for M, row in r["per_m"].items():
            if any(c in row for c in mops):
                fl = sum(row.get(c, 0.0) for c in mops) * 512.0
                row["derived"]["mfma_flops"] = fl
                row["derived"]["mfma_flops_over_2mnk"] = round(fl / flops(int(M), cls.N, cls.K), 4)
    return {name: r for (name, *_), r in zip(legs, res)}


def _counters_per_m(dirs, kernels, csv, glob):
    out = [{"per_m": {str(M): {} for M in sweep_ms}} for _, sweep_ms in kernels]
    for d in dirs:
        disp = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                e = disp.setdefault(int(r["Dispatch_Id"]), {
                    "name": r["Kernel_Name"], "c": {},
                    "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for (kern, sweep_ms), res in zip(kernels, out):
            gemms = [disp[k] for k in sorted(disp) if kern in disp[k]["name"]]
            if len(gemms) != 3 * len(sweep_ms):
                raise SystemExit(f"{d}: {len(gemms)} {kern} dispatches (expected {3 * len(sweep_ms)})")
            for i, M in enumerate(sweep_ms):
                grp = gemms[3 * i:3 * i + 3]
                row = res["per_m"][str(M)]
                for name in grp[0]["c"]:
                    row[name] = sorted(g["c"][name] for g in grp)[1]
                row.setdefault("duration_ns", sorted(g["ns"] for g in grp)[1])
    for res in out:
        _derive(res["per_m"])
    return out


def _derive(per_m):
    def ratio(row, a, b, scale=1.0):
        return round(row[a] / (row[b] * scale), 4) if a in row and b in row and row[b] else None

    for M, row in per_m.items():
        cyc = row["duration_ns"] * CLOCK_GHZ
        d = {}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in row:
            d["mfma_busy"] = round(row["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cyc), 4)
        if "TA_ADDR_STALLED_BY_TC_CYCLES" in row:
            d["ta_stalled_by_cache"] = round(row["TA_ADDR_STALLED_BY_TC_CYCLES"] / (CUS * cyc), 4)
        d["wave_waiting_any"] = ratio(row, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")
        d["wave_cannot_issue"] = ratio(row, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")
        d["lds_bank_conflicts_per_active_cycle"] = ratio(row, "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")
        if "TCC_HIT" in row and "TCC_MISS" in row:
            d["l2_hit_rate"] = round(row["TCC_HIT"] / max(row["TCC_HIT"] + row["TCC_MISS"], 1.0), 4)
        row["derived"] = d


# ------------------------------------------------------------------ legs

MEASURED_ROOF = {"GBps": None}


def sweep(torch, wl, Ms, nbytes_fn, peak, rounds):
    out = {}
    for M in Ms:
        med, mn = time_launches(torch, lambda: wl.launch(M), reps=wl.nbuf, rounds=rounds)
        r = roof(M, wl.N, wl.K, nbytes_fn(M, wl.N, wl.K), med, peak)
        r["us_min"] = round(mn, 2)
        if MEASURED_ROOF["GBps"]:
            r["frac_hbm_measured"] = round(r["gbs"] / MEASURED_ROOF["GBps"], 4)
        out[str(M)] = r
    return out


def decode_attention(torch, bg, rounds, L=4096, Hq=64, Hkv=8, Bs=(1, 16, 64)):
    """Dual-kernel decode attention, one query token per sequence over a
    4096-key bf16 cache (Hq = 64 query heads, Hkv = 8 KV heads, D = 128): per
    batch size the single-pass kernel, the split-KV kernel (+ merge) and the
    one the library picks.  The cache of the largest batch (1.07 GB of K and
    V) is filled once with seeded N(0,1) values; smaller batches rotate over
    its sequences so every launch reads HBM.  Bytes: K and V of every
    sequence plus Q and O."""
    D = 128
    Bmax = max(Bs)
    g = torch.Generator(device="cuda")
    g.manual_seed(20260)
    Kc = torch.randn((Bmax, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
    Vc = torch.randn((Bmax, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
    Qa = torch.randn((Bmax, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    lens = torch.full((Bmax,), L, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    res = {}
    for B in Bs:
        nrot = Bmax // B
        views = [(Qa[i * B:(i + 1) * B], Kc[i * B:(i + 1) * B], Vc[i * B:(i + 1) * B])
                 for i in range(nrot)]
        ws = torch.empty(bg.decode_attention_workspace_bytes(B, Hq, Hkv, L) // 4,
                         dtype=torch.float32, device="cuda")
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        nbytes = 2 * B * Hkv * L * D * 2 + 2 * B * Hq * D * 2
        row = {"bytes": nbytes, "auto_picks": bg.decode_attention_choice(B, Hq, Hkv, L)}
        for kern in ("single", "split"):
            i = [0]

            def fn():
                q, k, v = views[i[0] % nrot]
                i[0] += 1
                bg.decode_attention(q, k, v, lens[:B], scale, kernel=kern, workspace=ws, out=out)
            med, mn = time_launches(torch, fn, reps=max(nrot, 16), rounds=max(3, rounds // 2))
            gbs = nbytes / (med * 1e-6) / 1e9
            row[kern] = {"us": round(med, 2), "us_min": round(mn, 2), "gbs": round(gbs, 1),
                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        row["auto"] = row[row["auto_picks"]]
        res[str(B)] = row
        del ws, out
    del Kc, Vc, Qa
    torch.cuda.empty_cache()
    return res


def attention_probe(torch, bg, L=4096, Hq=64, Hkv=8):
    """Three eager single-pass launches at B = 64, then three split launches
    at B = 1 (each followed by its merge), on distinct cache slices."""
    D = 128
    g = torch.Generator(device="cuda")
    g.manual_seed(20261)
    Kc = torch.randn((67, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
    Vc = torch.randn((67, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
    Q = torch.randn((64, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    lens = torch.full((64,), L, dtype=torch.int32, device="cuda")
    for i in range(3):
        bg.decode_attention(Q, Kc[i:i + 64], Vc[i:i + 64], lens, 0.088, kernel="single")
    torch.cuda.synchronize()
    log("probe: 3 x single-pass B=64 done")
    ws = torch.empty(bg.decode_attention_workspace_bytes(1, Hq, Hkv, L) // 4, dtype=torch.float32,
                     device="cuda")
    for i in range(3):
        bg.decode_attention(Q[:1], Kc[64 + i:65 + i], Vc[64 + i:65 + i], lens[:1], 0.088,
                            kernel="split", workspace=ws)
    torch.cuda.synchronize()
    log("probe: 3 x split B=1 done")


def replay(torch, bg, inputs, steps=1000):
    """Dynamic-batching replay on the bf16 projection shape: pool of 4096 rows,
    `steps` batches of 1..256 distinct rows; GPU time of the GEMM launches."""
    K = N = 8192
    P = torch.from_numpy(inputs.normal_bf16((4096, K), 1.0, 501).view(np.int16)).view(torch.bfloat16).cuda()
    B = torch.from_numpy(inputs.normal_bf16((K, N), 0.02, 502).view(np.int16)).view(torch.bfloat16).cuda()
    batches = [torch.as_tensor(b, device="cuda") for b in inputs.replay_batches(4096, steps, 256, 503)]
    As = [P.index_select(0, b) for b in batches]
    C = torch.empty((256, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    it = iter(As)

    def one():
        A = next(it)
        bg.gemm_bf16(A, B, out=C[:A.shape[0]])

    # the warm-up call inside capture() consumes the first batch: time the rest
    g = capture(torch, one, steps - 1)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1)
    As = As[1:]
    steps -= 1
    rows = sum(a.shape[0] for a in As)
    return {"steps": steps, "rows": rows, "ms": round(ms, 3),
            "tflops": round(flops(rows, N, K) / (ms * 1e-3) / 1e12, 2),
            "note": "B stays in the Infinity Cache across steps (one weight matrix, as in serving)"}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rounds", type=int, default=10, help="rounds per timed M point")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline only, no extra legs")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="only run a known-size copy plus 3 launches per M (for rocprofv3 --pmc)")
    ap.add_argument("--legs", default=None,
                    help="only these per-M sweeps, comma separated (bf16_packed, bf16, bf16_bt, "
                         "fp8, fp8_packed, fp4, fp4_packed, w4a8, moe, moe_fp8); one JSON object")
    ap.add_argument("--roof", action="store_true",
                    help="only the measured roofs (streaming read, small streams, launch floor)")
    ap.add_argument("--attention", action="store_true",
                    help="only the decode-attention leg (one JSON object)")
    ap.add_argument("--attention-probe", action="store_true",
                    help="eager decode-attention launches for rocprofv3 --pmc: B = 64 single "
                         "pass x3, then B = 1 split x3 (L = 4096, Hq = 64, Hkv = 8)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise the FETCH_SIZE and WRITE_SIZE runs of --pmc-probe (no GPU)")
    ap.add_argument("--pmc-counters", nargs="+", metavar="DIR",
                    help="summarise other counter runs of --pmc-probe per M (no GPU)")
    ap.add_argument("--pmc-probe-legs", action="store_true",
                    help="a known-size copy plus 3 launches per M of the fp8, fp4 and W4A8 packed "
                         "legs (for rocprofv3 --pmc)")
    ap.add_argument("--pmc-summary-legs", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise the FETCH_SIZE and WRITE_SIZE runs of --pmc-probe-legs (no GPU)")
    ap.add_argument("--pmc-counters-legs", nargs="+", metavar="DIR",
                    help="summarise other counter runs of --pmc-probe-legs per leg and M (no GPU)")
    args = ap.parse_args()

    if args.pmc_summary:
        print(json.dumps(pmc_summary(*args.pmc_summary), indent=1))
        return
    if args.pmc_counters:
        print(json.dumps(pmc_counters(args.pmc_counters), indent=1))
        return
    if args.pmc_counters_legs:
        print(json.dumps(pmc_counters_legs(args.pmc_counters_legs), indent=1))
        return
    if args.pmc_summary_legs:
        print(json.dumps(pmc_summary_legs(*args.pmc_summary_legs), indent=1))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the batch-invariant GEMM is timed on a single "
              "MI355X (sharding the rows or the output columns over GPUs needs no exchange "
              "between them; only the one-GPU path is implemented).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from invariant_gemm_amd import bigemm, inputs
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.cuda.get_device_properties(0)
    log(f"device: {dev.name}, CUs {dev.multi_processor_count}")

    if args.attention:
        print(json.dumps(decode_attention(torch, bigemm, args.rounds)), flush=True)
        return
    if args.roof:
        print(json.dumps(measured_roof(torch, bigemm, args.rounds)), flush=True)
        return
    if args.legs:
        legs = {"bf16_packed": (C2P, SWEEP_C2, bytes_bf16, "bf16"), "bf16": (C2, SWEEP_C2, bytes_bf16, "bf16"),
                "bf16_bt": (C2T, SWEEP_C2, bytes_bf16, "bf16"), "fp8": (C3, SWEEP_C3, bytes_fp8, "fp8"),
                "fp8_packed": (C3P, SWEEP_C3, bytes_fp8, "fp8"), "fp4": (C4, SWEEP_C4, bytes_fp4, "bf16"),
                "fp4_packed": (C4P, SWEEP_C4, bytes_fp4, "bf16"),
                "w4a8": (W4A8, W4A8.SWEEP, bytes_w4a8, "fp8"), "moe": (MoE, MoE.SWEEP, None, "bf16"),
                "moe_fp8": (MoE8, MoE8.SWEEP, None, "fp8"), "moe_w4a8": (MoEW4A8, MoEW4A8.SWEEP, None, "fp8")}
        res = {}
        for name in args.legs.split(","):
            cls, Ms, nb, peak = legs[name]
            wl = cls(torch, bigemm, inputs)
            res[name] = sweep(torch, wl, Ms, nb if nb else wl.nbytes, MFMA_PEAK_TFLOPS[peak], args.rounds)
            res[name + "_us"] = {m: v["us"] for m, v in res[name].items()}
            del wl
            torch.cuda.empty_cache()
        print(json.dumps(res), flush=True)
        return
    if args.attention_probe:
        attention_probe(torch, bigemm)
        return
    if args.pmc_probe_legs:
        pmc_probe_legs(torch, bigemm, inputs)
        return
    wl = C2P(torch, bigemm, inputs)
    if args.pmc_probe:
        pmc_probe(torch, wl)
        return
    K, N = C2.K, C2.N
    step_flops = sum(flops(M, N, K) for M in SWEEP_C2)
    step_bytes = sum(bytes_bf16(M, N, K) for M in SWEEP_C2)

    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    # The timed region launches exactly `steps` steps (9 launches each, every
    # launch on the next rotated copy of A and B) eagerly on the stream: the
    # host enqueues a launch in about 12 us and the GPU needs 21-60 us for
    # it, so the queue stays ahead and the events time the GPU.  A graph of
    # the same steps, replayed afterwards, is reported beside it (HIP graph
    # replay adds about 1 us per kernel node on this stack).
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        wl.step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps: {ms:.4f} ms/step (wall {wall:.3f} s)")
    g = capture(torch, wl.step, args.steps)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    ms_graph = e0.elapsed_time(e1) / args.steps

    tflops = step_flops / (ms * 1e-3) / 1e12
    gbs = step_bytes / (ms * 1e-3) / 1e9
    kernel_src = [os.path.join(ROOT, "invariant_gemm_amd", "csrc", f)
                  for f in ("gemm_bf16_packed.hip", "common.h")]
    out = {
        "metric": "TFLOP/s and HBM GB/s vs roofline per M (1..512), bitwise-invariant rows",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_graph_replay": round(ms_graph, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": "bf16 projection GEMM C=A.B, K=N=8192, M sweep 1,2,4,...,256 "
                               "(one launch per M); B packed once into MFMA operand order "
                               f"({wl.pack_ms:.2f} ms per matrix, outside the timed region), "
                               f"rotated over {wl.nbuf} HBM copies",
                   "launches_per_step": len(SWEEP_C2), "K": K, "N": N, "M": SWEEP_C2,
                   "entry_point": "bi_gemm_bf16_packed"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles(kernel_src),
                     "kernel": "gemm_bf16_packed_kernel (bi_gemm_bf16_packed, all launch geometries)",
                     "algorithmic_bytes_per_launch": step_bytes / len(SWEEP_C2)},
    }

    if not args.quick:
        out["measured_roof"] = measured_roof(torch, bigemm)
        MEASURED_ROOF["GBps"] = out["measured_roof"]["read_roof_GBps"]
        out["roofline"]["frac_measured_roof"] = round(gbs / MEASURED_ROOF["GBps"], 4)
        out["per_m"] = sweep(torch, wl, SWEEP_C2, bytes_bf16, MFMA_PEAK_TFLOPS["bf16"], args.rounds)
        for M in SWEEP_C2:
            out["per_m"][str(M)]["us_single_launch"] = single_launch_us(torch, lambda: wl.launch(M))
        packed_us = {m: v["us"] for m, v in out["per_m"].items()}
        del wl
        c2 = C2(torch, bigemm, inputs)
        out["bf16_rowmajor_K8192_N8192"] = sweep(torch, c2, SWEEP_C2, bytes_bf16,
                                                 MFMA_PEAK_TFLOPS["bf16"], args.rounds)
        # the gap against the non-invariant split-K variant of the same
        # (row-major) kernel, and against the packed invariant path
        ws = torch.empty(256 * N, dtype=torch.float32, device="cuda")
        gap = {}
        for M in SWEEP_C2:
            med, _ = time_launches(torch, lambda: c2.launch_splitk(M, ws), reps=c2.nbuf,
                                   rounds=max(3, args.rounds // 2))
            gap[str(M)] = {"splits": bigemm.splitk_choose(M, N, K), "us": round(med, 2),
                           "invariant_over_splitk_time":
                               round(out["bf16_rowmajor_K8192_N8192"][str(M)]["us"] / med, 3),
                           "packed_invariant_over_splitk_time": round(packed_us[str(M)] / med, 3)}
        out["splitk_gap"] = gap
        del ws
        del c2
        c2t = C2T(torch, bigemm, inputs)
        out["bf16_bt_K8192_N8192"] = sweep(torch, c2t, SWEEP_C2, bytes_bf16,
                                           MFMA_PEAK_TFLOPS["bf16"], args.rounds)
        del c2t
        c3 = C3(torch, bigemm, inputs)
        out["fp8_blockscaled_K7168_N2048"] = sweep(torch, c3, SWEEP_C3, bytes_fp8,
                                                   MFMA_PEAK_TFLOPS["fp8"], args.rounds)
        del c3
        c3p = C3P(torch, bigemm, inputs)
        out["fp8_blockscaled_packed_K7168_N2048"] = sweep(torch, c3p, SWEEP_C3, bytes_fp8,
                                                          MFMA_PEAK_TFLOPS["fp8"], args.rounds)
        out["fp8_blockscaled_packed_K7168_N2048"]["pack_ms_once"] = round(c3p.pack_ms, 3)
        del c3p
        c4 = C4(torch, bigemm, inputs)
        out["fp4_weight_only_K4096_N14336"] = sweep(torch, c4, SWEEP_C4, bytes_fp4,
                                                    MFMA_PEAK_TFLOPS["bf16"], args.rounds)
        del c4
        c4p = C4P(torch, bigemm, inputs)
        out["fp4_weight_only_packed_K4096_N14336"] = sweep(torch, c4p, SWEEP_C4, bytes_fp4,
                                                           MFMA_PEAK_TFLOPS["bf16"], args.rounds)
        out["fp4_weight_only_packed_K4096_N14336"]["pack_ms_once"] = round(c4p.pack_ms, 3)
        del c4p
        w48 = W4A8(torch, bigemm, inputs)
        out["w4a8_mxfp4_K4096_N14336"] = sweep(torch, w48, W4A8.SWEEP, bytes_w4a8,
                                               MFMA_PEAK_TFLOPS["fp8"], args.rounds)
        del w48
        moe = MoE(torch, bigemm, inputs)
        out["moe_grouped_bf16_E8_K7168_N2048"] = sweep(torch, moe, MoE.SWEEP, moe.nbytes,
                                                       MFMA_PEAK_TFLOPS["bf16"], args.rounds)
        del moe
        moe8 = MoE8(torch, bigemm, inputs)
        out["moe_grouped_fp8_E8_K7168_N2048"] = sweep(torch, moe8, MoE8.SWEEP, moe8.nbytes,
                                                      MFMA_PEAK_TFLOPS["fp8"], args.rounds)
        del moe8
        moew4 = MoEW4A8(torch, bigemm, inputs)
        out["moe_grouped_w4a8_E8_K7168_N2048"] = sweep(torch, moew4, MoEW4A8.SWEEP, moew4.nbytes,
                                                       MFMA_PEAK_TFLOPS["fp8"], args.rounds)
        del moew4
        out["replay_bf16_K8192_N8192"] = replay(torch, bigemm, inputs)
        out["decode_attention_L4096_Hq64_Hkv8_D128"] = decode_attention(torch, bigemm, args.rounds)
        out["device"] = device_info(torch)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
