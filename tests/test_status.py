"""Bad device-side data never faults: the offending key or request is ignored, the rows it
touches are written as documented, and the sticky status word reports it."""
import numpy as np
import pytest

import workloads as wl
from mla_tree_verify_paged_amd import binding as B
from tests.conftest import gpu_available
from tests.gpu_helpers import compare, run_gpu, run_oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KERNELS = ["simple", "mfma"]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("h", [8, 64])  # the 4- and the 8-wavefront partial kernel
def test_out_of_range_slot_is_ignored_and_flagged(kernel, h):
    w = wl.build_workload("slot", np.random.default_rng(20), h, [40], [4], 128)
    p = 40
    # reference: tree key 3 hidden from every query
    ref_w = wl.build_workload("slot", np.random.default_rng(20), h, [40], [4], 128)
    ref_w.custom_mask.reshape(4, 44)[:, p + 3] = 0
    ref = run_oracle(ref_w)
    w.kv_indices[p + 3] = w.num_slots + 5
    from mla_tree_verify_paged_amd.device_inputs import to_device
    dev = to_device(ref_w)
    dev["kv_indices"][p + 3] = w.num_slots + 5
    o, l, a, st = run_gpu(w, kernel=kernel, dev=dev)
    assert st & B.VA_DEV_SLOT_RANGE
    # the run must equal the oracle on the same inputs with that key hidden
    compare(ref_w, (o, l, a, 0), ref)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("h", [8, 64])
def test_too_many_tree_tokens_for_the_context(kernel, h):
    w = wl.build_workload("tq", np.random.default_rng(21), h, [30, 30], [3, 9], 128)
    o, l, a, st = run_gpu(w, kernel=kernel, max_q_per_req=4, max_q_tokens=12)
    assert st & B.VA_DEV_Q_PER_REQ
    ref = run_oracle(w)
    first = 3 * h
    compare(w, (o, l, a, 0), (ref[0][:first], ref[1][:first], ref[2][:first]),
            rows=np.arange(first))
    assert np.all(o[first:] == 0) and np.all(l[first:] == -np.inf) and np.all(a[first:] == -1)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("h", [4, 64])
def test_prefix_shorter_than_tree_is_flagged(kernel, h):
    w = wl.build_workload("seg", np.random.default_rng(22), h, [10, 20], [4, 4], 128)
    from mla_tree_verify_paged_amd.device_inputs import to_device
    dev = to_device(w)
    dev["kv_indptr"][1] = 2          # request 0: L=2 < T=4; request 1: L=32
    o, l, a, st = run_gpu(w, kernel=kernel, dev=dev)
    assert st & B.VA_DEV_SEGMENT
    assert np.all(o[:4 * h] == 0) and np.all(l[:4 * h] == -np.inf)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("h,t", [(4, 5), (64, 16), (64, 40)])
def test_tokens_not_covered_by_qo_indptr(kernel, h, t):
    """num_tokens = T + 2 but qo_indptr covers T tokens: the rows of the last two tokens are
    empty. H*(T+2) = 28, 1152 and 2688 rows: the three launch shapes of the combine."""
    import torch
    from mla_tree_verify_paged_amd import VerifyAttn
    from mla_tree_verify_paged_amd.device_inputs import to_device
    w = wl.build_workload("tok", np.random.default_rng(23), h, [300], [t], 512)
    dev = to_device(w)
    n = t + 2
    q = torch.cat([dev["q"], dev["q"][:2]])
    va = VerifyAttn(h, max_batch=1, max_q_per_req=t, max_q_tokens=n, kernel=kernel)
    out = torch.full((n, h, 512), float("nan"), device="cuda")
    lse = torch.zeros((n, h), device="cuda")
    am = torch.full((n, h), 7, dtype=torch.int32, device="cuda")
    va.run(q, dev["kv_buffer"], dev["kv_indices"], dev["kv_indptr"], dev["qo_indptr"],
           dev["custom_mask"], dev["mask_indptr"], w.scale, out, lse, am, bs=1, num_tokens=n)
    st = va.read_device_status()
    assert st & B.VA_DEV_TOKENS
    o = out.cpu().numpy()
    assert np.all(o[t:] == 0) and np.all(np.isfinite(o))
    assert np.all(lse.cpu().numpy()[t:] == -np.inf)
    assert np.all(am.cpu().numpy()[t:] == -1)
    ref = run_oracle(w)
    compare(w, (o[:t].reshape(-1, 512).astype(np.float64), lse.cpu().numpy()[:t].ravel(), None,
                0), ref)


@pytest.mark.parametrize("kernel", KERNELS)
def test_non_positive_scale_is_rejected(kernel):
    from mla_tree_verify_paged_amd.device_inputs import to_device
    w = wl.build_workload("scale", np.random.default_rng(24), 4, [8], [2], 32)
    dev = to_device(w)
    for bad in (0.0, -0.5, float("inf"), float("nan")):
        w.scale = bad
        with pytest.raises(B.VerifyAttnError) as e:
            run_gpu(w, kernel=kernel, dev=dev)
        assert e.value.status == B.VA_ERR_INVALID


@pytest.mark.parametrize("kernel", KERNELS)
def test_mask_offset_near_int64_max_is_flagged(kernel):
    """A corrupt mask_indptr entry next to INT64_MAX: the bounds check must not overflow, so
    request 0 is rejected (rows empty, status flagged) and request 1 is untouched."""
    from mla_tree_verify_paged_amd.device_inputs import to_device
    w = wl.build_workload("m64", np.random.default_rng(24), 8, [50, 70], [5, 6], 256)
    dev = to_device(w)
    dev["mask_indptr"][0] = 2**63 - 2
    o, l, a, st = run_gpu(w, kernel=kernel, dev=dev)
    assert st & B.VA_DEV_SEGMENT
    first = 5 * 8
    assert np.all(o[:first] == 0) and np.all(l[:first] == -np.inf) and np.all(a[:first] == -1)
    ref = run_oracle(w)
    rows = np.arange(first, w.num_tokens * w.num_heads)
    compare(w, (o, l, a, 0), (ref[0][first:], ref[1][first:], ref[2][first:]), rows=rows)
