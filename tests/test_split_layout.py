"""GPU parity for the split slot layout: prefix slots in kv_indices, the tree tokens' slots in
out_cache_loc ("The Final Solder Joint", section "The Three-Edits Sequence"). Each case is
checked against the oracle run on the same split buffers, and against the GPU's own result on
the combined layout, which must be bit-identical: the same keys in the same order."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_helpers import compare, run_gpu, run_oracle, sample_rows, say, stress_depth8_rows

pytestmark = pytest.mark.gpu

BF16_KERNELS = ["simple", "mfma"]


def both_layouts(w, kernel, **kw):
    from mla_tree_verify_paged_amd.device_inputs import to_device
    dev = to_device(w)
    a = run_gpu(w, kernel=kernel, dev=dev, split=True, **kw)
    b = run_gpu(w, kernel=kernel, dev=dev, split=False, **kw)
    assert np.array_equal(a[0], b[0]), "split and combined layouts differ"
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    return a


def test_tiny_fp32_split_exact_argmax():
    w = wl.tiny()
    say("tiny fp32, split layout")
    got = both_layouts(w, "simple")
    ref = run_oracle(w, split=True)
    compare(w, got, ref, exact_argmax=True, tol=1e-4)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_short_split(kernel):
    w = wl.short()
    say(f"short, split layout, {kernel}")
    got = both_layouts(w, kernel)
    rows = sample_rows(w, 256, seed=3)
    ref = run_oracle(w, rows=rows, split=True)
    compare(w, got, ref, rows=rows, split=True)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_segmented_split(kernel):
    w = wl.segmented()
    say(f"segmented, split layout, {kernel}")
    got = both_layouts(w, kernel)
    rows = sample_rows(w, 256, seed=4)
    ref = run_oracle(w, rows=rows, split=True)
    compare(w, got, ref, rows=rows, split=True)


def test_stress_split_mfma():
    w = wl.stress()
    say("stress, split layout, mfma")
    got = both_layouts(w, "mfma")
    rows = sample_rows(w, 64, seed=5, must=stress_depth8_rows(w)[:16])
    ref = run_oracle(w, rows=rows, split=True)
    compare(w, got, ref, rows=rows, split=True)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_split_tree_slot_out_of_range_is_flagged(kernel):
    """A tree slot outside the pool makes that key invisible and sets the slot-range bit."""
    import torch
    from mla_tree_verify_paged_amd.device_inputs import to_device
    w = wl.short()
    dev = to_device(w)
    bad = dev["out_cache_loc"].clone()
    bad[5] = w.num_slots + 3
    dev["out_cache_loc"] = bad
    o, l, a, status = run_gpu(w, kernel=kernel, dev=dev, split=True)
    assert status & 1, f"slot-range bit not set: {status}"
    assert np.all(np.isfinite(o))
