"""Capture safety: verify_attn_run recorded into a HIP graph and replayed after the contents
of the static buffers change (new queries, new KV rows, a different prefix length and tree)
gives the eager result bit for bit and matches the oracle on every replay."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.conftest import gpu_available
from tests.gpu_helpers import compare, run_oracle, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KERNELS = ["simple", "mfma"]


def make(seed, p, t, h=64):
    return wl.build_workload(f"g{seed}", np.random.default_rng(seed), h, [p], [t], 65536)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("h,max_t", [(64, 16), (64, 40), (8, 4)])
def test_graph_replay_with_new_buffer_contents(kernel, h, max_t):
    """H*T = 1024, 2560 and 32 rows: the three launch shapes of the combine (and, at H=8, the
    partial kernel's few-rows path)."""
    from mla_tree_verify_paged_amd import VerifyAttn
    from mla_tree_verify_paged_amd.device_inputs import to_device
    max_l = 4000
    va = VerifyAttn(h, max_batch=1, max_q_per_req=max_t, max_q_tokens=max_t, kernel=kernel)
    # static buffers sized for the largest step
    q = torch.zeros((max_t, h, 576), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((65536, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(max_l, dtype=torch.int64, device="cuda")
    kv_indptr = torch.zeros(2, dtype=torch.int32, device="cuda")
    qo_indptr = torch.zeros(2, dtype=torch.int64, device="cuda")
    mask = torch.zeros(max_t * max_l, dtype=torch.uint8, device="cuda")
    mask_indptr = torch.zeros(2, dtype=torch.int64, device="cuda")
    out = torch.zeros((max_t, h, 512), dtype=torch.float32, device="cuda")
    lse = torch.zeros((max_t, h), dtype=torch.float32, device="cuda")

    def load(w):
        d = to_device(w)
        n = w.num_tokens
        q.zero_()
        q[:n].copy_(d["q"])
        pool.copy_(d["kv_buffer"])
        idx[:d["kv_indices"].numel()].copy_(d["kv_indices"])
        kv_indptr.copy_(d["kv_indptr"])
        qo_indptr.copy_(d["qo_indptr"])
        mask[:d["custom_mask"].numel()].copy_(d["custom_mask"])
        mask_indptr.copy_(d["mask_indptr"])

    def step():
        va.run(q, pool, idx, kv_indptr, qo_indptr, mask, mask_indptr, wl.DEFAULT_SCALE, out,
               lse, None, bs=1, num_tokens=max_t)

    # the graph is recorded once with num_tokens = max_t; steps with fewer tokens leave the
    # extra rows empty (qo_indptr covers fewer tokens), which the C ABI reports in its status
    w0 = make(100, 3000, max_t, h)
    load(w0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for seed, p in ((101, 3000), (102, 1200), (103, 4000 - max_t), (104, 2500)):
        t = max_t
        w = make(seed, p, t, h)
        load(w)
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64).reshape(-1, 512)
        got_lse = lse.cpu().numpy().astype(np.float64).ravel()
        # eager on the same buffers
        step()
        torch.cuda.synchronize()
        eager = out.cpu().numpy().astype(np.float64).reshape(-1, 512)
        assert np.array_equal(got, eager), "replay differs from eager"
        st = va.read_device_status()
        say(f"replay seed={seed} P={p}")
        ref = run_oracle(w)
        compare(w, (got, got_lse, None, st), ref)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("h", [16, 64])
def test_graph_replay_of_a_changing_batch(kernel, h):
    """A graph captured once for six requests and 96 token slots, replayed on batches whose
    prefix lengths, tree sizes (empty requests included) and tree shapes change from replay to
    replay; the static buffers are rewritten in place between replays and token slots past the
    batch's tokens stay padding. Every replay equals eager bit for bit and matches the oracle
    (out, lse and argmax); the padding rows are empty."""
    from mla_tree_verify_paged_amd import VerifyAttn
    from mla_tree_verify_paged_amd.device_inputs import to_device
    bs, max_t, pool_slots = 6, 16, 1 << 17
    n_tok = bs * max_t
    max_keys = bs * (4000 + max_t)
    va = VerifyAttn(h, max_batch=bs, max_q_per_req=max_t, max_q_tokens=n_tok, kernel=kernel)
    q = torch.zeros((n_tok, h, 576), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((pool_slots, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(max_keys, dtype=torch.int64, device="cuda")
    kv_indptr = torch.zeros(bs + 1, dtype=torch.int32, device="cuda")
    qo_indptr = torch.zeros(bs + 1, dtype=torch.int64, device="cuda")
    mask = torch.zeros(max_t * max_keys, dtype=torch.uint8, device="cuda")
    mask_indptr = torch.zeros(bs + 1, dtype=torch.int64, device="cuda")
    out = torch.zeros((n_tok, h, 512), dtype=torch.float32, device="cuda")
    lse = torch.zeros((n_tok, h), dtype=torch.float32, device="cuda")
    am = torch.zeros((n_tok, h), dtype=torch.int32, device="cuda")

    def make_batch(seed):
        rng = np.random.default_rng(seed)
        p = rng.integers(0, 4000, bs)
        t = rng.integers(0, max_t + 1, bs)
        t[rng.integers(0, bs)] = 0          # at least one request without tree tokens
        t[rng.integers(0, bs)] = max_t      # and one full tree
        return wl.build_workload(f"gb{seed}", rng, h, p, t, pool_slots)

    def load(w):
        d = to_device(w)
        n = w.num_tokens
        q.zero_()
        q[:n].copy_(d["q"])
        pool.copy_(d["kv_buffer"])
        idx.zero_()
        idx[:d["kv_indices"].numel()].copy_(d["kv_indices"])
        kv_indptr.copy_(d["kv_indptr"])
        qo_indptr.copy_(d["qo_indptr"])
        mask.zero_()
        mask[:d["custom_mask"].numel()].copy_(d["custom_mask"])
        mask_indptr.copy_(d["mask_indptr"])

    def step():
        va.run(q, pool, idx, kv_indptr, qo_indptr, mask, mask_indptr, wl.DEFAULT_SCALE, out,
               lse, am, bs=bs, num_tokens=n_tok)

    load(make_batch(200))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    va.read_device_status()

    for seed in (201, 202, 203, 204):
        w = make_batch(seed)
        n = w.num_tokens
        load(w)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64).reshape(-1, 512)
        got_lse = lse.cpu().numpy().astype(np.float64).ravel()
        got_am = am.cpu().numpy().astype(np.int64).ravel()
        st = va.read_device_status()
        # token slots past the batch's tokens are padding: empty rows, reported as such
        assert (st & ~8) == 0 and (n == n_tok or st & 8), st
        pad = slice(n * h, n_tok * h)
        assert np.all(got[pad] == 0) and np.all(got_lse[pad] == -np.inf)
        assert np.all(got_am[pad] == -1)
        step()
        torch.cuda.synchronize()
        va.read_device_status()
        assert np.array_equal(got, out.cpu().numpy().astype(np.float64).reshape(-1, 512))
        assert np.array_equal(got_am, am.cpu().numpy().astype(np.int64).ravel())
        say(f"replay seed={seed} T={w.tree_lens.tolist()} P={w.prefix_lens.tolist()}")
        ref = run_oracle(w)
        rows = slice(0, n * h)
        compare(w, (got[rows], got_lse[rows], got_am[rows], 0), ref)
