"""The seeded generators: determinism, the documented draw order, the bf16 encoding and
the buffer layout (CPU only)."""
import os

import numpy as np
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_fp32_oracle.txt")


def test_bf16_encoding_is_round_to_nearest_even():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 10
    x[:4] = [np.inf, -np.inf, 0.0, -0.0]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.to_bf16_bits(x), ref)
    assert np.array_equal(wl.bf16_bits_to_f32(ref),
                          torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())
    assert wl.to_bf16_bits(np.array([np.nan], np.float32))[0] == wl.BF16_NAN_BITS


def test_segmented_draws():
    w = wl.segmented(0)
    assert w.prefix_lens.tolist() == [9311, 2608, 1180, 1084, 17155, 24217, 8382, 12832]
    assert w.tree_lens.tolist() == [16, 16, 16, 32, 8, 32, 32, 8]
    assert int(w.kv_indptr[-1]) == 76_929


def test_generators_are_deterministic():
    a, b = wl.short(0), wl.short(0)
    for f in ("q", "kv_rows", "kv_indices", "custom_mask", "kv_indptr", "qo_indptr"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_layout_invariants():
    for w in (wl.tiny(), wl.short()):
        assert w.kv_indptr.dtype == np.int32 and w.qo_indptr.dtype == np.int64
        assert w.kv_indices.dtype == np.int64 and w.custom_mask.dtype == np.uint8
        assert len(np.unique(w.kv_indices)) == len(w.kv_indices)
        assert w.kv_indices.min() >= 0 and w.kv_indices.max() < w.num_slots
        for r in range(w.bs):
            t, p = int(w.tree_lens[r]), int(w.prefix_lens[r])
            m = w.custom_mask[w.mask_indptr[r]:w.mask_indptr[r + 1]].reshape(t, t + p)
            assert np.all(m[:, :p] == 1)
            tail = m[:, p:]
            assert np.all(np.diag(tail) == 1) and np.all(np.triu(tail, 1) == 0)


def test_tiny_is_a_chain_over_a_permutation():
    w = wl.tiny()
    assert w.in_dtype == "fp32" and w.q.shape == (4, 8, 576) and w.kv_rows.shape == (68, 576)
    tail = w.custom_mask.reshape(4, 68)[:, 64:]
    assert np.array_equal(tail, np.tril(np.ones((4, 4), np.uint8)))
    assert np.array_equal(w.kv_indices, np.random.default_rng(0).permutation(128)[:68])


def test_stress_tree_depth_bound():
    rng = np.random.default_rng(0)
    for _ in range(20):
        d = wl.tree_depths(wl.random_tree(64, rng, max_depth=8))
        assert d.max() <= 8


def test_unreferenced_pool_rows_are_nan():
    w = wl.tiny()
    pool = w.pool_np()
    unused = np.setdiff1d(np.arange(w.num_slots), w.kv_indices)
    assert np.all(np.isnan(pool[unused]))


def test_tiny_golden_regression():
    """The oracle still reproduces the stored tiny-workload fixture."""
    rows = np.loadtxt(GOLDEN, comments="#")
    out, lse, am = oracle.run_workload(wl.tiny())
    assert np.array_equal(am, rows[:, 3].astype(np.int64))
    assert np.allclose(lse, rows[:, 4], rtol=1e-15, atol=0)
    assert np.allclose(out.sum(axis=1), rows[:, 5], rtol=1e-13, atol=1e-13)
    assert np.allclose(out[:, [0, 1, 511]], rows[:, 6:9], rtol=1e-15, atol=0)


def test_tiny_argmax_is_well_posed():
    """The top-2 score gap of every tiny row is far above fp32 rounding."""
    w = wl.tiny()
    k = w.pool_np()[w.kv_indices].astype(np.float64)
    q = w.q.astype(np.float64).reshape(32, 576)
    s = w.scale * q @ k.T
    vis = np.repeat(w.custom_mask.reshape(4, 68) != 0, 8, axis=0)
    s[~vis] = -np.inf
    top2 = np.sort(s, axis=1)[:, -2:]
    assert np.min(top2[:, 1] - top2[:, 0]) > 1e-3
