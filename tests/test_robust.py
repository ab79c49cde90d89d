"""Robustness of the verify step against stale workspace contents and the split count.

Every run below first fills the whole workspace past its header (the partial outputs, code
scales, per-split scalars and the per-row placement table) with 0xFF bytes: NaN as fp32, -1 as
int16/int32, a negative placement. A kernel that read a partial it did not write in the same
run would change the output or make it non-finite; the runs must instead equal an unpoisoned
run bit for bit. (The header, the status words and the row of zeros that unusable keys read, is
set once at create and is not the caller's to write.)"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.conftest import gpu_available
from tests.gpu_helpers import compare, run_gpu, run_oracle, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

HEADER_BYTES = 1536   # status words + zero row, 256-byte aligned


def poisoned_context(w, kernel, num_splits=0):
    from mla_tree_verify_paged_amd import VerifyAttn
    va = VerifyAttn(w.num_heads, in_dtype=w.in_dtype, max_batch=max(1, w.bs),
                    max_q_per_req=max(1, w.max_q_per_req), max_q_tokens=max(1, w.num_tokens),
                    num_splits=num_splits, kernel=kernel, workspace="torch")
    base = va.cfg.workspace - va.workspace.data_ptr()
    body = va.workspace[base + HEADER_BYTES: base + va.cfg.workspace_bytes]
    return va, body


CASES = {
    "rows1024": lambda: wl.build_workload("p1", np.random.default_rng(50), 64, [3000], [16],
                                          8192),
    "rows32": lambda: wl.build_workload("p2", np.random.default_rng(51), 8, [5000], [4], 8192),
    "rows3072": lambda: wl.build_workload("p3", np.random.default_rng(52), 64,
                                          [700, 2100, 40, 1500], [16, 8, 12, 12], 8192),
    "more_splits_than_keys": lambda: wl.build_workload("p4", np.random.default_rng(53), 16,
                                                       [3, 40], [2, 5], 128),
}


@pytest.mark.parametrize("kernel", ["simple", "mfma"])
@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("splits", [0, 3])
def test_poisoned_workspace_changes_nothing(kernel, case, splits):
    w = CASES[case]()
    say(f"poison: {case}, {kernel}, splits={splits}")
    clean = run_gpu(w, kernel=kernel, num_splits=splits)
    va, body = poisoned_context(w, kernel, splits)
    for rep in range(2):
        body.fill_(0xFF)
        torch.cuda.synchronize()
        got = run_gpu(w, kernel=kernel, va=va)
        assert got[3] == 0, f"status {got[3]}"
        for k in range(3):
            assert np.array_equal(got[k], clean[k]), f"output {k} differs after poisoning"
    ref = run_oracle(w)
    compare(w, got, ref, exact_argmax=kernel == "simple" and w.in_dtype == "fp32")
    va.close()
