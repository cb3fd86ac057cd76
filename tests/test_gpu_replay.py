"""Dynamic-batching replay (bf16, K = N = 8192): a pool of 4096 fixed token
rows, 1000 steps, each a seeded random batch of 1-256 distinct rows in random
order.  Every token's output row must be bitwise equal across all of its
appearances -- the online-serving scenario of the QbitAI article, section
"什么是batch invariance" (a request batched with A and B today, with C and D
tomorrow).  A per-token SHA-256 digest table (the digest-whitelist idea of the
wmrh.cn V4 engineering blog, section 5.3) is then re-derived in a second
process, which checks determinism across processes.
"""
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from invariant_gemm_amd import inputs
from tests.gpu_util import check_parity, dev_bf16, host_codes, require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POOL, K, N, STEPS, MAXB = 4096, 8192, 8192, 1000, 256


def digests(rows_codes: np.ndarray):
    return [hashlib.sha256(r.tobytes()).hexdigest() for r in rows_codes]


def test_replay_every_appearance_bitwise(tmp_path):
    require_gpu()
    from invariant_gemm_amd import bigemm
    pool = inputs.normal_bf16((POOL, K), 1.0, 501)
    Bc = inputs.normal_bf16((K, N), 0.02, 502)
    P = dev_bf16(pool)
    B = dev_bf16(Bc)
    first = torch.zeros((POOL, N), dtype=torch.bfloat16, device="cuda")
    seen = torch.zeros(POOL, dtype=torch.bool, device="cuda")
    appearances = 0
    mismatched_tokens = set()
    for step, idx in enumerate(inputs.replay_batches(POOL, STEPS, MAXB, 503)):
        it = torch.as_tensor(idx, device="cuda")
        out = bigemm.gemm_bf16(P.index_select(0, it), B)
        was = seen.index_select(0, it)
        ref = first.index_select(0, it)
        eq = (out.view(torch.int16) == ref.view(torch.int16)).all(dim=1)
        bad = was & ~eq
        if bool(bad.any()):
            mismatched_tokens.update(idx[bad.cpu().numpy()].tolist())
        new = ~was
        if bool(new.any()):
            first.index_copy_(0, it[new], out[new])
            seen.index_fill_(0, it[new], True)
        appearances += len(idx)
    torch.cuda.synchronize()
    assert not mismatched_tokens, f"{len(mismatched_tokens)} tokens changed bits across batches"
    assert appearances > 100_000
    toks = torch.nonzero(seen).flatten().cpu().numpy()
    assert len(toks) > 4000

    # parity of the served rows against the fp64 oracle on a sample
    sample = np.sort(inputs.rng(504).choice(toks, size=8, replace=False))
    C64, S = oracle.gemm_bf16(np.ascontiguousarray(pool[sample]), Bc)
    check_parity(host_codes(first[torch.as_tensor(sample, device="cuda")]), C64, S, K, "replay")

    # digest table, then a second process recomputes a subset and compares
    table = dict(zip(map(int, toks), digests(host_codes(first[torch.as_tensor(toks, device="cuda")]))))
    sub = [int(t) for t in inputs.rng(505).choice(toks, size=64, replace=False)]
    path = tmp_path / "digests.json"
    path.write_text(json.dumps({"tokens": sub, "digests": [table[t] for t in sub]}))
    code = (
        "import json, sys, numpy as np, torch\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from invariant_gemm_amd import bigemm, inputs\n"
        "from tests.gpu_util import dev_bf16, host_codes\n"
        "from tests.test_gpu_replay import digests, POOL, K, N\n"
        f"d = json.load(open({str(path)!r}))\n"
        "pool = inputs.normal_bf16((POOL, K), 1.0, 501)\n"
        "B = dev_bf16(inputs.normal_bf16((K, N), 0.02, 502))\n"
        "A = dev_bf16(np.ascontiguousarray(pool[d['tokens']]))\n"
        "batch = digests(host_codes(bigemm.gemm_bf16(A, B)))\n"
        "alone = [digests(host_codes(bigemm.gemm_bf16(A[i:i+1], B)))[0] for i in range(len(d['tokens']))]\n"
        "assert batch == d['digests'], 'batched digests differ across processes'\n"
        "assert alone == d['digests'], 'single-row digests differ across processes'\n"
        "print('second process digests match')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stdout + r.stderr
