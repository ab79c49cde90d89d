"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded inputs.

Bar: max |out - oracle| <= 1e-2 (fp32 out); lse within 2^-10 + 1e-5 |lse| (the fp16 rounding of
each softmax weight moves the denominator by up to 2^-11 relative); the argmax equal on every
row of the tiny fp32 workload and, for bf16 inputs, a visible key within the fp32 score-rounding
bound of the exact maximum (equal to the oracle's wherever the exact top-2 gap exceeds that
bound); device status clean."""
import numpy as np
import pytest

import workloads as wl
from tests.conftest import gpu_available
from tests.gpu_helpers import (check_argmax, compare, run_gpu, run_oracle, sample_rows, say,
                               stress_depth8_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

BF16_KERNELS = ["simple", "mfma"]


def test_tiny_fp32_exact_argmax():
    w = wl.tiny()
    say("tiny fp32, simple kernel")
    ref = run_oracle(w)
    for splits in (0, 1, 3, 64):
        gpu = run_gpu(w, kernel="simple", num_splits=splits)
        err = compare(w, gpu, ref, exact_argmax=True)
        assert err <= 1e-4  # fp32 inputs and arithmetic


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_short(kernel):
    w = wl.short()
    say(f"short, {kernel}")
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_long_full(kernel):
    w = wl.long()
    say(f"long, {kernel}")
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)
    # the launch bench.py times: out and lse, no argmax (the kernels' other instantiation)
    compare(w, run_gpu(w, kernel=kernel, want_argmax=False), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_segmented_full(kernel):
    """All 10,240 rows of the 8-request batch."""
    w = wl.segmented()
    say(f"segmented, {kernel}, all rows")
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)
    compare(w, run_gpu(w, kernel=kernel, want_argmax=False), ref)


def stress_rows(w, n_random=800):
    """Every head of every depth-8 tree node, plus a seeded sample of other rows."""
    must = []
    for row in stress_depth8_rows(w):
        must.extend(range(row, row + w.num_heads))
    return sample_rows(w, n_random, seed=2, must=must)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_stress_sampled(kernel):
    w = wl.stress()
    rows = stress_rows(w)
    assert len(rows) >= 1024
    say(f"stress, {kernel}, {len(rows)} rows (every head of each depth-8 node)")
    ref = run_oracle(w, rows=rows)
    compare(w, run_gpu(w, kernel=kernel), ref, rows=rows)
    compare(w, run_gpu(w, kernel=kernel, want_argmax=False), ref, rows=rows)


# ----------------------------------------------------------------------------- seeded fuzz
@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("seed", range(6))
def test_fuzz_small_shapes(kernel, seed):
    rng = np.random.default_rng(500 + seed)
    bs = int(rng.integers(1, 5))
    h = int(rng.choice([1, 3, 8, 64]))
    t = rng.integers(1, 34, bs)
    p = rng.integers(0, 3001, bs)
    w = wl.build_workload(f"fuzz{seed}", rng, h, p, t, int((p + t).sum()) * 2 + 7)
    splits = int(rng.choice([0, 1, 5, 17]))
    say(f"fuzz seed={seed} {kernel}: bs={bs} H={h} T={t.tolist()} P={p.tolist()} S={splits}")
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel, num_splits=splits), ref)


# ----------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("h", [8, 64])  # the 4- and the 8-wavefront partial kernel
def test_zero_prefix_and_single_token(kernel, h):
    rng = np.random.default_rng(7)
    w = wl.build_workload("p0", rng, h, [0, 0, 5], [1, 7, 1], 64)
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("h", [16, 64])
def test_more_splits_than_keys(kernel, h):
    rng = np.random.default_rng(8)
    w = wl.build_workload("split", rng, h, [3, 40], [2, 5], 128)
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel, num_splits=64), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("h", [4, 64])
def test_fully_masked_rows_are_empty(kernel, h):
    rng = np.random.default_rng(9)
    w = wl.build_workload("masked", rng, h, [0], [6], 32)
    m = w.custom_mask.reshape(6, 6)
    m[2, :] = 0
    m[4, :] = 0
    ref = run_oracle(w)
    o, l, a, st = run_gpu(w, kernel=kernel)
    for tok in (2, 4):
        rows = slice(tok * h, tok * h + h)
        assert np.all(o[rows] == 0) and np.all(l[rows] == -np.inf) and np.all(a[rows] == -1)
    compare(w, (o, l, a, st), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("h", [8, 64])
def test_request_without_tree_tokens(kernel, h):
    rng = np.random.default_rng(10)
    w = wl.build_workload("t0", rng, h, [50, 30, 70], [3, 0, 4], 256)
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("h", [8, 64])
def test_empty_batches_write_nothing(kernel, h):
    """bs = 0, and a batch whose requests all have T_r = 0 (num_tokens = 0): the call succeeds,
    enqueues nothing that writes, and leaves the output buffers as they were."""
    import torch
    from mla_tree_verify_paged_amd import VerifyAttn
    from mla_tree_verify_paged_amd.device_inputs import to_device
    rng = np.random.default_rng(11)
    w = wl.build_workload("t0all", rng, h, [40, 0, 25], [0, 0, 0], 128)
    assert w.num_tokens == 0
    dev = to_device(w)
    va = VerifyAttn(h, max_batch=4, max_q_per_req=4, max_q_tokens=8, kernel=kernel)
    q = torch.zeros((8, h, 576), dtype=torch.bfloat16, device="cuda")
    out = torch.full((8, h, 512), 3.0, device="cuda")
    lse = torch.full((8, h), 5.0, device="cuda")
    am = torch.full((8, h), 7, dtype=torch.int32, device="cuda")
    for bs in (0, w.bs):
        va.run(q, dev["kv_buffer"], dev["kv_indices"], dev["kv_indptr"], dev["qo_indptr"],
               dev["custom_mask"], dev["mask_indptr"], w.scale, out, lse, am, bs=bs,
               num_tokens=0)
        torch.cuda.synchronize()
        assert va.read_device_status() == 0
        assert bool((out == 3.0).all()) and bool((lse == 5.0).all()) and bool((am == 7).all())


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_many_heads(kernel):
    """H = 128: a 128-row tile is one token's heads; 5 tokens give 5 row tiles."""
    rng = np.random.default_rng(12)
    w = wl.build_workload("h128", rng, 128, [900], [5], 4096)
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)


def test_partial_variant_follows_num_heads():
    """The MFMA partial workgroup runs 8 wavefronts (two per SIMD) exactly when H is a multiple
    of 64, so that no work item has 32 rows or fewer; otherwise 4. The fp32 kernel runs 4."""
    from mla_tree_verify_paged_amd import VerifyAttn
    for h, waves in ((64, 8), (128, 8), (192, 8), (8, 4), (16, 4), (48, 4), (96, 4)):
        va = VerifyAttn(h, max_batch=2, max_q_per_req=4, max_q_tokens=8, kernel="mfma")
        assert va.info.partial_waves == waves, (h, va.info.partial_waves)
    va = VerifyAttn(64, in_dtype="fp32", max_batch=1, max_q_per_req=4, max_q_tokens=4)
    assert va.info.partial_waves == 4


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_eight_wave_half_tiles(kernel):
    """H = 64 with odd tree sizes: requests of 1, 3 and 5 tokens end in a 64-row tile whose last
    two row groups lie past the request (their wavefronts stage and compute but never store),
    with empty, one-tile and many-tile prefixes."""
    rng = np.random.default_rng(21)
    w = wl.build_workload("half64", rng, 64, [0, 33, 1500, 95], [1, 3, 5, 2], 4096)
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_large_tree(kernel):
    """A 384-node draft tree at H = 8 (3072 rows: the wavefront-per-row combine) over a short
    prefix, so most keys of most rows are tree keys under the mask."""
    rng = np.random.default_rng(13)
    w = wl.build_workload("bigtree", rng, 8, [200], [384], 4096)
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("shape", ["short", "rows2560", "rows48"])
def test_bf16_output(kernel, shape):
    """bf16 output in each combine launch shape: 1024 rows (a workgroup per row), 2560 rows
    (a wavefront per row) and 48 rows (a quarter row per workgroup)."""
    if shape == "short":
        w = wl.short()
    elif shape == "rows2560":
        w = wl.build_workload("bf16out", np.random.default_rng(15), 64, [900, 2500], [24, 16],
                              8192)
    else:
        w = wl.build_workload("bf16out", np.random.default_rng(16), 8, [3000, 1200], [4, 2],
                              8192)
    ref = run_oracle(w)
    o, l, a, st = run_gpu(w, kernel=kernel, out_dtype="bf16")
    err = np.abs(o - ref[0])
    bound = 1e-2 + np.abs(ref[0]) * 2.0 ** -8
    assert np.all(err <= bound), float((err - bound).max())
    assert st == 0
    check_argmax(w, a, ref[2])


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_optional_outputs_may_be_null(kernel):
    w = wl.build_workload("null", np.random.default_rng(11), 8, [100], [5], 256)
    ref = run_oracle(w)
    o, _, _, st = run_gpu(w, kernel=kernel, want_lse=False, want_argmax=False)
    compare(w, (o, None, None, st), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_oversized_bounds(kernel):
    """A context sized for more requests and tokens than the call uses."""
    rng = np.random.default_rng(12)
    w = wl.build_workload("big", rng, 64, [700, 20], [9, 16], 2048)
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel, max_batch=5, max_q_per_req=40, max_q_tokens=200), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_bitwise_deterministic(kernel):
    w = wl.build_workload("det", np.random.default_rng(13), 64, [1500], [16], 4096)
    a = run_gpu(w, kernel=kernel)
    b = run_gpu(w, kernel=kernel)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.skipif("mfma" not in BF16_KERNELS, reason="MFMA kernel not built yet")
def test_mfma_matches_simple_closely():
    """Both kernels agree far inside the oracle tolerance."""
    w = wl.build_workload("xk", np.random.default_rng(14), 64, [2000, 900], [16, 8], 8192)
    a = run_gpu(w, kernel="simple")
    b = run_gpu(w, kernel="mfma")
    assert np.max(np.abs(a[0] - b[0])) <= 5e-3


# ----------------------------------------------------------------------------- few rows per request
@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_tp8_full(kernel):
    """H=8, T=4: 32 rows against 23,004 keys (three of the four wavefronts have no rows)."""
    w = wl.tp8()
    say(f"tp8, {kernel}")
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel=kernel), ref)
    compare(w, run_gpu(w, kernel=kernel, want_argmax=False), ref)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_tp8_batch_sampled(kernel):
    w = wl.tp8_batch()
    rows = sample_rows(w, 256, seed=3)
    say(f"tp8_batch, {kernel}, {len(rows)} sampled rows")
    ref = run_oracle(w, rows=rows)
    compare(w, run_gpu(w, kernel=kernel), ref, rows=rows)
    compare(w, run_gpu(w, kernel=kernel, want_argmax=False), ref, rows=rows)


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_small_trees_sampled(kernel):
    """H=64, T_r in 1..4: requests of 64 rows (a 128-row item with two of its four wavefronts
    idle), 128, 192 (a full row tile plus 64 rows) and 256."""
    w = wl.small_trees()
    rows = sample_rows(w, 384, seed=6)
    say(f"small_trees, {kernel}, {len(rows)} sampled rows, T={w.tree_lens.tolist()}")
    ref = run_oracle(w, rows=rows)
    compare(w, run_gpu(w, kernel=kernel), ref, rows=rows)
    compare(w, run_gpu(w, kernel=kernel, want_argmax=False), ref, rows=rows)


# ----------------------------------------------------------------------------- the device work list
def test_work_list_more_requests_than_a_wavefront():
    """70 requests of mixed length: the plan scans the request tables in chunks of 64, and the
    long requests get several splits while the short ones get one."""
    rng = np.random.default_rng(15)
    p = np.where(rng.random(70) < 0.1, rng.integers(3000, 9000, 70), rng.integers(0, 400, 70))
    t = rng.integers(1, 5, 70)
    w = wl.build_workload("wl70", rng, 8, p, t, int((p + t).sum()) * 2)
    say(f"work list: bs=70 H=8 sum P={int(p.sum())}")
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel="mfma"), ref)
    # a context sized for more requests than the call has
    compare(w, run_gpu(w, kernel="mfma", max_batch=130, max_q_per_req=9), ref)


def test_work_list_more_row_tiles_than_workgroups():
    """300 requests x 2 row tiles: more row tiles than compute units, so each row tile is one
    item covering all of its request's keys."""
    rng = np.random.default_rng(16)
    p = rng.integers(0, 200, 300)
    t = rng.integers(3, 5, 300)
    w = wl.build_workload("wl300", rng, 64, p, t, int((p + t).sum()) * 2)
    rows = sample_rows(w, 2048, seed=4)
    say(f"work list: bs=300 H=64, {len(rows)} sampled rows")
    ref = run_oracle(w, rows=rows)
    compare(w, run_gpu(w, kernel="mfma"), ref, rows=rows)


def test_work_list_one_long_request_among_short_ones():
    rng = np.random.default_rng(17)
    w = wl.build_workload("wl_skew", rng, 64, [40000, 100, 0, 2500], [16, 3, 7, 1], 1 << 17)
    rows = sample_rows(w, 512, seed=5)
    say(f"work list: skewed batch, {len(rows)} sampled rows")
    ref = run_oracle(w, rows=rows)
    compare(w, run_gpu(w, kernel="mfma"), ref, rows=rows)
    compare(w, run_gpu(w, kernel="mfma", num_splits=7), ref, rows=rows)


def test_row_tile_boundaries():
    """Requests whose row counts straddle the two item shapes: 1..32 rows (all four
    wavefronts share the rows), 33..128 (one 32-row group per wavefront, some idle), and more
    than 128 (several row tiles, the last one possibly of at most 32 rows)."""
    rng = np.random.default_rng(18)
    t = np.array([1, 31, 32, 33, 64, 96, 127, 128, 129, 160])
    p = rng.integers(0, 700, len(t))
    w = wl.build_workload("tiles", rng, 1, p, t, int((p + t).sum()) * 2)
    say(f"row tiles: H=1 T={t.tolist()}")
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel="mfma"), ref)
    compare(w, run_gpu(w, kernel="mfma", num_splits=3), ref)


# ----------------------------------------------------------------------------- value ranges
# Latent dims in four 128-dim groups at very different magnitudes: keys scaled by 2^6, 1,
# 2^-6, 2^-12 per group and queries by the inverse powers of two, so every product q_d k_d, and
# hence every score, is exactly that of the unscaled draw, while the values (the latent dims of
# the keys) span 18 binary orders. The absolute 1e-2 bar cannot see an error in the small
# groups, so each group is held to a bound relative to its own largest reference value:
# 2^-8 covers the fp16 rounding of P (2^-11 of each weight) and of V, and the 16-bit partial
# codes (one step = 2^-15 of the group's largest partial value) with room to spare; the
# smallest group also absorbs fp16 subnormal rounding of V (at most 2^-25 absolute).
GROUP_EXP = (6, 0, -6, -12)


def _group_scaled(w):
    import dataclasses
    k = w.kv_rows_f32().copy()
    q = w.q_f32().copy()
    for g, e in enumerate(GROUP_EXP):
        k[:, 128 * g:128 * (g + 1)] *= np.float32(2.0 ** e)
        q[:, :, 128 * g:128 * (g + 1)] *= np.float32(2.0 ** -e)
    return dataclasses.replace(w, name=w.name + "_groups", kv_rows=wl.to_bf16_bits(k),
                               q=wl.to_bf16_bits(q))


@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("shape", ["rows1344", "rows24"])
def test_value_groups_at_different_scales(kernel, shape):
    rng = np.random.default_rng(77)
    if shape == "rows1344":   # the 128-row path and the whole-row combine
        base = wl.build_workload("groups", rng, 64, [3000, 700], [16, 5], 16384)
    else:                     # the few-rows path and the quarter-row combine
        base = wl.build_workload("groups", rng, 8, [5000], [3], 16384)
    w = _group_scaled(base)
    say(f"value groups {GROUP_EXP}, {shape}, {kernel}")
    ref_o, ref_l, _ = run_oracle(w)
    o, l, _, status = run_gpu(w, kernel=kernel)
    assert status == 0
    assert np.all(np.isfinite(o))
    for g, e in enumerate(GROUP_EXP):
        sl = slice(128 * g, 128 * (g + 1))
        ref_max = float(np.max(np.abs(ref_o[:, sl])))
        err = float(np.max(np.abs(o[:, sl] - ref_o[:, sl])))
        say(f"  group {g} (x2^{e}): max|ref| {ref_max:.3e}, max err {err:.3e}")
        assert err <= 2.0 ** -8 * ref_max + 2.0 ** -24, (g, err, ref_max)
    # the scores did not change, so the lse matches the oracle's as in every other test
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(l), fin)


# ----------------------------------------------------------------------------- argmax tie rule
@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("splits", [0, 8])
@pytest.mark.parametrize("h", [4, 64])
def test_argmax_tie_across_splits_goes_to_the_lower_key(kernel, splits, h):
    """One slot appears at key positions 300 and 2800 (in different key splits) and holds a
    row aligned with every query, so both positions attain the maximum with bit-identical
    scores: the argmax must be the lower position, 300 (the oracle's rule, pinned there by
    brute force)."""
    rng = np.random.default_rng(40)
    p, t = 3000, 2
    w = wl.build_workload("tie", rng, h, [p], [t], 8192)
    q = wl.bf16_bits_to_f32(w.q)
    q[:, :, :] = q[0, 0]                       # every row has the same query
    w.q = wl.to_bf16_bits(q)
    rows = wl.bf16_bits_to_f32(w.kv_rows)
    rows[300] = np.clip(q[0, 0] * 4.0, -30, 30)   # score ~ 4 |q|^2 scale: far above the rest
    w.kv_rows = wl.to_bf16_bits(rows)
    w.kv_indices[2800] = w.kv_indices[300]
    w.kv_rows[2800] = w.kv_rows[300]
    ref = run_oracle(w)
    assert np.all(ref[2] == 300)
    gpu = run_gpu(w, kernel=kernel, num_splits=splits)
    assert np.all(gpu[2] == 300), np.unique(gpu[2])
    compare(w, gpu, ref)


# ----------------------------------------------------------------------------- split counts
@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_split_counts_agree(kernel):
    """One split, the device-chosen count and 256 splits: each run meets the oracle bar, and
    the runs agree with each other within twice the per-run rounding scale (fp16 weights,
    2^-11 of the largest value, and the 16-bit partial codes)."""
    w = wl.build_workload("nsplit", np.random.default_rng(41), 64, [9000, 2500], [16, 8], 16384)
    ref = run_oracle(w)
    runs = {}
    for s in (1, 0, 256):
        runs[s] = run_gpu(w, kernel=kernel, num_splits=s)
        compare(w, runs[s], ref)
    vmax = float(np.abs(wl.bf16_bits_to_f32(w.kv_rows)[:, :512]).max())
    tol = 2 * (2.0 ** -11 + 2.0 ** -15) * vmax
    for s in (0, 256):
        d = float(np.max(np.abs(runs[s][0] - runs[1][0])))
        say(f"  splits {s} vs 1: max diff {d:.3e} (bound {tol:.3e})")
        assert d <= tol


@pytest.mark.parametrize("shape,splits", [
    ("few_rows", 1), ("few_rows", 5), ("few_rows", 13), ("few_rows", 64), ("few_rows", 65),
    ("few_rows", 256), ("rows1024", 3), ("rows1024", 13), ("rows1024", 33), ("rows3072", 3),
    ("rows3072", 7)])
def test_combine_shapes_over_split_counts(shape, splits):
    """Each merge kernel over fixed split counts against the oracle: the few-rows merge (32
    rows, H = 8; split counts that leave lane groups partly empty, more than 64 splits so lanes
    hold several splits' scalars, and 256 capped at the 188 key tiles), the one-workgroup-per-row
    merge (1024 rows) and the one-wavefront-per-row merge (3072 rows)."""
    if shape == "few_rows":
        w = wl.build_workload("cs", np.random.default_rng(60 + splits), 8, [6000], [4], 16384)
    elif shape == "rows1024":
        w = wl.build_workload("cs", np.random.default_rng(70 + splits), 64, [3000], [16], 16384)
    else:
        w = wl.build_workload("cs", np.random.default_rng(80 + splits), 64, [2000, 1500],
                              [32, 16], 16384)
    say(f"{shape}, {splits} splits")
    ref = run_oracle(w)
    compare(w, run_gpu(w, kernel="mfma", num_splits=splits), ref)

# ----------------------------------------------------------------------------- value range
@pytest.mark.parametrize("shape", ["rows1024", "rows24"])
def test_latent_values_beyond_fp16_saturate_as_documented(shape):
    """The bf16 path converts value dims to fp16 with round-toward-zero, so a latent value of
    magnitude 65536 or more saturates to +-65504 (include/verify_attn.h, "Value range"). Plant
    +-131072 (exact in bf16) in three visible keys, all in the first 128-dim group, with the
    queries zero on those dims (scores unchanged), and compare with the oracle on the same
    inputs with those values saturated (fp32 inputs, since 65504 is not a bf16 value):
      * dims 128..511 meet the usual 1e-2 bar;
      * the planted group meets its own bound: a 16-bit code step of the group's largest
        partial value (at most 65504 / 32767 per split, so 2.5 after the merge) plus 2^-10 of
        the value for the fp16 rounding of the weights;
      * on a planted dim where saturating matters (the unsaturated result differs from the
        saturated one by more than 50), the result is within a tenth of that difference of
        the saturated one."""
    import dataclasses
    rng = np.random.default_rng(90)
    if shape == "rows1024":
        w = wl.build_workload("sat", rng, 64, [1500], [16], 4096)
    else:
        w = wl.build_workload("sat", rng, 8, [2000], [3], 4096)
    rows = wl.bf16_bits_to_f32(w.kv_rows)
    q = wl.bf16_bits_to_f32(w.q)
    keys, dims = [11, 700, 1234], [5, 40, 100]
    for k, d in zip(keys, dims):
        rows[k, d] = 131072.0 if k % 2 else -131072.0
        q[:, :, d] = 0.0
    w.kv_rows = wl.to_bf16_bits(rows)
    w.q = wl.to_bf16_bits(q)
    o, l, a, st = run_gpu(w, kernel="mfma")
    assert st == 0 and np.all(np.isfinite(o))
    sat = rows.copy()
    for k, d in zip(keys, dims):
        sat[k, d] = np.sign(rows[k, d]) * 65504.0
    as_fp32 = dict(in_dtype="fp32", q=wl.bf16_bits_to_f32(w.q))
    ref = run_oracle(dataclasses.replace(w, kv_rows=sat.astype(np.float32), **as_fp32))
    unsat = run_oracle(dataclasses.replace(w, kv_rows=rows.astype(np.float32), **as_fp32))
    # the scores are the unplanted ones: lse and argmax as in every other comparison
    compare(w, (o[:, 128:], l, a, st), (ref[0][:, 128:], ref[1], ref[2]))
    g0 = slice(0, 128)
    bound = 2.0 ** -10 * np.abs(ref[0][:, g0]) + 2.5
    excess = np.abs(o[:, g0] - ref[0][:, g0]) - bound
    say(f"  planted group: max err {np.abs(o[:, g0] - ref[0][:, g0]).max():.3e}")
    assert excess.max() <= 0, float(excess.max())
    gap = np.abs(unsat[0][:, dims] - ref[0][:, dims])
    sel = gap > 50
    assert sel.sum() >= 10, int(sel.sum())
    err = np.abs(o[:, dims] - ref[0][:, dims])
    assert np.all(err[sel] < 0.1 * gap[sel])
    say(f"  {int(sel.sum())} (row, dim) pairs where saturating moves the result by > 50: "
        f"worst err / gap {float((err[sel] / gap[sel]).max()):.2e}")
