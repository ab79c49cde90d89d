"""Shared helpers for the GPU tests: run a workload through the C ABI, run the oracle on the
same inputs, compare."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
import workloads as wl

OUT_TOL = 1e-2      # max-abs on out, bf16 inputs with fp32 accumulation (and fp32 inputs)
# lse: the MFMA path rounds each softmax weight to fp16 (relative error <= 2^-11) and sums the
# rounded weights, so the denominator, hence lse, may move by up to 2^-11 in natural-log units;
# twice that plus fp32 score rounding is the bound.
LSE_ATOL = 2.0 ** -10
LSE_RTOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(w, kernel="auto", num_splits=0, out_dtype="fp32", want_lse=True, want_argmax=True,
            max_batch=None, max_q_per_req=None, max_q_tokens=None, dev=None, va=None,
            split=False):
    """Runs workload `w` through the C ABI. Returns (out f64 [rows,512], lse, argmax, status).
    With `split`, the key slots go in the prefix-only kv_indices plus out_cache_loc layout."""
    import torch
    from mla_tree_verify_paged_amd import VerifyAttn
    from mla_tree_verify_paged_amd.device_inputs import to_device
    if dev is None:
        dev = to_device(w)
    if va is None:
        va = VerifyAttn(w.num_heads, in_dtype=w.in_dtype, out_dtype=out_dtype,
                        max_batch=max_batch or max(1, w.bs),
                        max_q_per_req=max_q_per_req or max(1, w.max_q_per_req),
                        max_q_tokens=max_q_tokens or max(1, w.num_tokens),
                        num_splits=num_splits, kernel=kernel)
    n = w.num_tokens
    odt = torch.float32 if out_dtype == "fp32" else torch.bfloat16
    out = torch.full((n, w.num_heads, 512), float("nan"), dtype=odt, device="cuda")
    lse = torch.full((n, w.num_heads), float("nan"), dtype=torch.float32, device="cuda") \
        if want_lse else None
    am = torch.full((n, w.num_heads), -7, dtype=torch.int32, device="cuda") \
        if want_argmax else None
    if split:
        va.run(dev["q"], dev["kv_buffer"], dev["kv_indices_prefix"], dev["kv_indptr_prefix"],
               dev["qo_indptr"], dev["custom_mask"], dev["mask_indptr"], w.scale, out, lse, am,
               bs=w.bs, num_tokens=n, out_cache_loc=dev["out_cache_loc"])
    else:
        va.run(dev["q"], dev["kv_buffer"], dev["kv_indices"], dev["kv_indptr"], dev["qo_indptr"],
               dev["custom_mask"], dev["mask_indptr"], w.scale, out, lse, am, bs=w.bs,
               num_tokens=n)
    torch.cuda.synchronize()
    status = va.read_device_status()
    o = out.float().cpu().numpy().astype(np.float64).reshape(n * w.num_heads, 512)
    l = lse.cpu().numpy().astype(np.float64).ravel() if want_lse else None
    a = am.cpu().numpy().astype(np.int64).ravel() if want_argmax else None
    return o, l, a, status


def sample_rows(w, n, seed=0, must=()):
    rows_total = w.num_tokens * w.num_heads
    rng = np.random.default_rng(seed)
    rows = rng.choice(rows_total, size=min(n, rows_total), replace=False)
    rows = np.unique(np.concatenate([rows, np.asarray(must, dtype=np.int64)]))
    return rows.astype(np.int64)


def run_oracle(w, rows=None, pool=None, split=False):
    t0 = time.time()
    res = oracle.run_workload(w, rows=rows, pool=pool, split=split)
    say(f"  oracle {w.name}: {0 if rows is None else len(rows)} rows in {time.time() - t0:.1f}s")
    return res


# Score rounding bound for the argmax check. A GPU score is an fp32 sum, in some order, of
# the 576 products q_d k_d (exact in fp32 for bf16 inputs, rounded once for fp32 inputs), so
# |s_gpu - s| <= GAMMA * sum_d |q_d k_d| with GAMMA = (576 + 1) u / (1 - 577 u), u = 2^-24
# (the classical bound for recursive summation, which covers every order). The kernels compare
# raw scores, and the split merge compares per-split maxima after a scaling that is monotone
# but may round two distinct maxima to one value (a tie, resolved to the lower key): that adds
# at most a few ulps of the score itself, covered by SCALED_ULPS * |s|.
_U = 2.0 ** -24
GAMMA = 577 * _U / (1 - 577 * _U)
SCALED_ULPS = 8 * _U


def check_argmax(w, a, ref_am, rows=None, split=False):
    """Validates the argmax of a run that is not bit-exact (bf16 inputs): on every compared
    row the returned key is -1 exactly when the row sees no key, else a visible key whose exact
    score is within the rounding bound of the exact maximum; where the exact top-2 gap exceeds
    twice that bound the key equals the oracle's."""
    n_rows = w.num_tokens * w.num_heads
    sel = np.arange(n_rows) if rows is None else np.asarray(rows, dtype=np.int64)
    assert a.shape == sel.shape
    empty = ref_am < 0
    assert np.array_equal(a[empty], ref_am[empty]), "argmax of an empty row is not -1"
    assert np.all(a[~empty] >= 0), "a row with visible keys returned no argmax"
    live = ~empty
    top = oracle.workload_top2(w, rows=sel[live], pair_rows=sel[live], pair_keys=a[live],
                               split=split)
    assert np.array_equal(top["arg1"], ref_am[live])
    assert np.all(top["pair_vis"] == 1), "argmax is not a visible key"
    m1, m2, amax = top["top1"], top["top2"], top["absmax"]
    tol = GAMMA * (top["pair_abs"] + amax) + SCALED_ULPS * np.abs(m1)
    short = m1 - top["pair_s"] - tol
    assert short.size == 0 or short.max() <= 0, \
        f"argmax score below the max by more than the bound ({short.max():.3e})"
    sure = (m1 - m2) > 2 * GAMMA * amax + SCALED_ULPS * np.abs(m1)
    wrong = sure & (a[live] != ref_am[live])
    assert not wrong.any(), f"{int(wrong.sum())} rows with a clear top-2 gap differ"
    say(f"  argmax: {int(live.sum())} rows checked, {int(sure.sum())} with a clear gap "
        f"(exact), {int((a[live] == ref_am[live]).sum())} equal to the oracle")


def compare(w, gpu, ref, rows=None, exact_argmax=False, tol=OUT_TOL, split=False):
    o, l, a, status = gpu
    ro, rl, ra = ref
    if rows is not None:
        o = o[rows]
        l = None if l is None else l[rows]
        a = None if a is None else a[rows]
    err = float(np.max(np.abs(o - ro))) if o.size else 0.0
    say(f"  {w.name}: max|out-ref| = {err:.3e} over {o.shape[0]} rows, status={status}")
    assert status == 0, f"device status {status}"
    assert np.all(np.isfinite(o)), "non-finite output"
    assert err <= tol, f"max abs err {err} > {tol}"
    if l is not None:
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(l), fin)
        excess = np.abs(l[fin] - rl[fin]) - (LSE_ATOL + LSE_RTOL * np.abs(rl[fin]))
        assert excess.size == 0 or excess.max() <= 0, f"lse error exceeds bound by {excess.max()}"
    if a is not None and exact_argmax:
        assert np.array_equal(a, ra), "argmax differs"
    elif a is not None:
        check_argmax(w, a, ra, rows=rows, split=split)
    return err


def stress_depth8_rows(w):
    """Flat rows (t*H + h, head 0) of every depth-8 tree node of the stress workload."""
    rows = []
    for r in range(w.bs):
        d = wl.tree_depths(w.parents[r])
        for i in np.nonzero(d == d.max())[0]:
            rows.append((int(w.qo_indptr[r]) + int(i)) * w.num_heads)
    return rows
