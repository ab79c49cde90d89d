"""The allocation-free entry point (verify_attn_run_static) through the C ABI against the
context entry point (verify_attn_run) on the same inputs: two calls in a row on one GPU, the
second with a smaller input, so that the second runs on the scratch the first left behind.
Both calls must equal the context path bit for bit (the same kernels and plan) and meet the
oracle bar."""
import numpy as np
import pytest

import workloads as wl
from tests.conftest import gpu_available
from tests.gpu_helpers import compare, run_gpu, run_oracle, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run_static(w, cfg):
    import torch
    from mla_tree_verify_paged_amd import binding as B
    from mla_tree_verify_paged_amd.device_inputs import to_device
    dev = to_device(w)
    n, h = w.num_tokens, w.num_heads
    out = torch.full((n, h, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((n, h), float("nan"), dtype=torch.float32, device="cuda")
    am = torch.full((n, h), -7, dtype=torch.int32, device="cuda")
    B.validate_run(h, "bf16", "fp32", dev["q"], dev["kv_buffer"], dev["kv_indices"],
                   dev["kv_indptr"], dev["qo_indptr"], dev["custom_mask"], dev["mask_indptr"],
                   out, lse, am, w.bs, n)
    B.verify_attn_run_static(
        cfg, dev["q"].data_ptr(), dev["kv_buffer"].data_ptr(), dev["kv_buffer"].shape[0],
        dev["kv_indices"].data_ptr(), dev["kv_indices"].numel(), dev["kv_indptr"].data_ptr(),
        dev["qo_indptr"].data_ptr(), dev["custom_mask"].data_ptr(), dev["custom_mask"].numel(),
        dev["mask_indptr"].data_ptr(), None, w.bs, n, w.scale, out.data_ptr(), lse.data_ptr(),
        am.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return (out.cpu().numpy().astype(np.float64).reshape(n * h, 512),
            lse.cpu().numpy().astype(np.float64).ravel(),
            am.cpu().numpy().astype(np.int64).ravel())


@pytest.mark.parametrize("kernel", ["mfma", "simple"])
def test_static_entry_matches_the_context_entry(kernel):
    from mla_tree_verify_paged_amd import binding as B
    kern = {"mfma": B.VA_KERNEL_MFMA, "simple": B.VA_KERNEL_SIMPLE}[kernel]
    big = wl.build_workload("na_big", np.random.default_rng(60), 64, [6000, 2500], [16, 9],
                            1 << 16)
    small = wl.build_workload("na_small", np.random.default_rng(61), 64, [900], [5], 1 << 14)
    # one config for both calls, sized for the larger
    cfg = B.make_config(64, max_batch=2, max_q_per_req=16, max_q_tokens=25, kernel=kern)
    for w in (big, small):
        say(f"static entry, {kernel}: {w.name} bs={w.bs} P={w.prefix_lens.tolist()} "
            f"T={w.tree_lens.tolist()}")
        got = run_static(w, cfg)
        ctx = run_gpu(w, kernel=kernel, max_batch=2, max_q_per_req=16, max_q_tokens=25)
        assert ctx[3] == 0
        for k in range(3):
            assert np.array_equal(got[k], ctx[k]), f"output {k} differs from verify_attn_run"
        compare(w, (*got, 0), run_oracle(w))
