#!/usr/bin/env python3
"""Throughput of the batch-invariant GEMMs on one MI355X against its roofline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

Workload (one "step"): the bf16 projection GEMM, K = N = 8192, weights
B ~ N(0, 0.02), activations A ~ N(0, 1), swept over M = 1, 2, 4, ..., 256 --
nine launches of bi_gemm_bf16, one per M.  Every launch reads a different
copy of (A, B) out of a rotation that totals more than 1 GiB, so B is read
from HBM and not from the 256 MB Infinity Cache.  Inputs are resident in HBM
before the timed region starts.

`value` is whole-job TFLOP/s over the timed steps (2MNK per launch).  The
JSON line also carries, per M, the launch time, TFLOP/s, algorithmic GB/s and
roofline fractions; the fp8 block-scaled and fp4 weight-only sweeps; the gap
against the non-invariant split-K comparator; and the fp64 oracle timed on
the host (a bounded sample of the same workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # dense, published
SWEEP_C2 = [1, 2, 4, 8, 16, 32, 64, 128, 256]
K2 = N2 = 8192
ROT_BYTES = 1 << 30             # rotation footprint per operand set (> 2 x (MALL + L2))

ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_bf16(M, N, K):
    return 2 * M * K + 2 * K * N + 2 * M * N


def flops(M, N, K):
    return 2.0 * M * N * K


# ------------------------------------------------------------------ workload

class C2Workload:
    def __init__(self, torch, bigemm, inputs):
        self.torch, self.bg = torch, bigemm
        pool = inputs.normal_bf16((256, K2), 1.0, 201)
        Bc = inputs.normal_bf16((K2, N2), 0.02, 202)
        A0 = torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).cuda()
        B0 = torch.from_numpy(Bc.view(np.int16)).view(torch.bfloat16).cuda()
        self.nbuf = max(2, -(-ROT_BYTES // (K2 * N2 * 2)))
        self.A = [A0.clone() for _ in range(self.nbuf)]
        self.B = [B0.clone() for _ in range(self.nbuf)]
        self.C = torch.empty((256, N2), dtype=torch.bfloat16, device="cuda")
        self.i = 0

    def launch(self, M):
        j = self.i % self.nbuf
        self.i += 1
        self.bg.gemm_bf16(self.A[j][:M], self.B[j], out=self.C[:M])

    def step(self):
        for M in SWEEP_C2:
            self.launch(M)


def time_launches(torch, fn, reps, rounds):
    """Median and min per-launch time (us) over `rounds` rounds of `reps`
    back-to-back launches, measured with HIP events on the launch stream."""
    per = []
    for _ in range(rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / reps)
    per.sort()
    return per[len(per) // 2], per[0]


# ------------------------------------------------------------------ cpu baseline

def cpu_baseline(budget_s=12.0):
    """The fp64 oracle as it stands, on the host cores, on a bounded sample of
    the same workload (rows of the M = 256 batch, full N and K)."""
    import oracle
    from invariant_gemm_amd import inputs
    pool = inputs.normal_bf16((256, K2), 1.0, 201)
    Bc = inputs.normal_bf16((K2, N2), 0.02, 202)
    rows, t_tot, r = 0, 0.0, 0
    chunk = 8
    while t_tot < budget_s and rows < 256:
        A = np.ascontiguousarray(pool[r:r + chunk])
        t0 = time.perf_counter()
        oracle.gemm_bf16(A, Bc)
        t_tot += time.perf_counter() - t0
        rows += A.shape[0]
        r += chunk
    fl = flops(rows, N2, K2)
    return {"value": fl / t_tot / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"fp64 oracle on {rows} rows of the M=256 batch (K=N=8192): "
                      f"{fl / 1e9:.1f} GFLOP in {t_tot:.2f} s"}


# ------------------------------------------------------------------ traffic evidence

def traffic_from_profiles(kernel_src: str, algorithmic_bytes: float):
    """HBM traffic per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "gemm_bf16_c2_pmc.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    h = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if d.get("kernel_sha256") != h:
        return None
    return d.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ counters

COPY_BYTES = 256 << 20


def pmc_probe(torch, wl):
    """Launch sequence for the HBM-traffic counters: a plain device copy of
    COPY_BYTES (the calibration reference: it must fetch and write exactly
    that many bytes), then three launches per M of the swept GEMM, each on a
    different rotated copy of B."""
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


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rounds", type=int, default=20, help="rounds per-M timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the per-M and comparator legs")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="only run a known-size copy plus 3 launches per M (for rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the batch-invariant GEMM is timed on a single "
              "MI355X; multi-GPU sharding is described in DESIGN.md and not run here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from invariant_gemm_amd import bigemm, inputs
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.cuda.get_device_properties(0)
    log(f"device: {dev.name}, CUs {dev.multi_processor_count}")

    wl = C2Workload(torch, bigemm, inputs)
    if args.pmc_probe:
        pmc_probe(torch, wl)
        return
    step_flops = sum(flops(M, N2, K2) for M in SWEEP_C2)
    step_bytes = sum(bytes_bf16(M, N2, K2) for M in SWEEP_C2)

    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
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

    tflops = step_flops / (ms * 1e-3) / 1e12
    gbs = step_bytes / (ms * 1e-3) / 1e9
    kernel_src = os.path.join(ROOT, "invariant_gemm_amd", "csrc", "gemm_bf16.hip")
    traffic = traffic_from_profiles(kernel_src, step_bytes / len(SWEEP_C2))

    out = {
        "metric": "TFLOP/s and HBM GB/s vs roofline per M (1..512), bitwise-invariant rows",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": "bf16 projection GEMM C=A.B, K=N=8192, M sweep "
                               "1,2,4,...,256 (one launch per M); B rotated over "
                               f"{wl.nbuf} HBM copies",
                   "launches_per_step": len(SWEEP_C2), "K": K2, "N": N2, "M": SWEEP_C2},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "gemm_bf16_kernel (bi_gemm_bf16)",
                     "algorithmic_bytes_per_launch": step_bytes / len(SWEEP_C2)},
    }

    if not args.no_extra:
        per_m = {}
        for M in SWEEP_C2:
            med, mn = time_launches(torch, lambda: wl.launch(M), reps=8 * wl.nbuf // 8 or 8,
                                    rounds=args.rounds)
            f, b = flops(M, N2, K2), bytes_bf16(M, N2, K2)
            per_m[str(M)] = {"us": round(med, 2), "us_min": round(mn, 2),
                             "tflops": round(f / med / 1e6, 2), "gbs": round(b / med / 1e3, 1),
                             "frac_hbm": round(b / med / 1e3 / HBM_PEAK_GBS, 4),
                             "frac_mfma": round(f / med / 1e6 / MFMA_PEAK_TFLOPS["bf16"], 4)}
        out["per_m"] = per_m
        # split-K comparator (not invariant): split count chosen from M
        ws = torch.empty(256 * N2, dtype=torch.float32, device="cuda")
        gap = {}
        for M in SWEEP_C2:
            def sk(M=M):
                j = wl.i % wl.nbuf
                wl.i += 1
                bigemm.gemm_bf16_splitk(wl.A[j][:M], wl.B[j], ws, 0, out=wl.C[:M])
            med, _ = time_launches(torch, sk, reps=8, rounds=max(5, args.rounds // 2))
            gap[str(M)] = {"splits": bigemm.splitk_choose(M, N2, K2), "us": round(med, 2),
                           "invariant_over_splitk_time": round(per_m[str(M)]["us"] / med, 3)}
        out["splitk_gap"] = gap

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
