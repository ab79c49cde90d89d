"""GPU checks of the two tree kernels through the C ABI, against the tree oracle: the verify
mask built from parent arrays (byte-exact), and greedy acceptance (exact)."""
import numpy as np
import pytest

import workloads as wl
from oracle import tree_oracle as to
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def ctx_for(w):
    from mla_tree_verify_paged_amd import VerifyAttn
    return VerifyAttn(w.num_heads, in_dtype=w.in_dtype, max_batch=max(1, w.bs),
                      max_q_per_req=max(1, w.max_q_per_req), max_q_tokens=max(1, w.num_tokens),
                      kernel="simple" if w.in_dtype == "fp32" else "auto")


def gpu_mask(w, split, indptr=None):
    import torch
    va = ctx_for(w)
    parents = torch.from_numpy(np.concatenate(w.parents).astype(np.int64)).cuda()
    qo = torch.from_numpy(w.qo_indptr).cuda()
    kv = torch.from_numpy(w.split_buffers()[1] if split else w.kv_indptr).cuda()
    size = int(indptr[-1]) if indptr is not None else int(w.mask_indptr[-1])
    mask = torch.full((max(size, 1),), 7, dtype=torch.uint8, device="cuda")
    if indptr is None:
        ind = torch.full((w.bs + 1,), -5, dtype=torch.int64, device="cuda")
        va.build_mask(parents, qo, kv, mask, ind, split_layout=split, write_mask_indptr=True)
    else:
        ind = torch.from_numpy(indptr).cuda()
        va.build_mask(parents, qo, kv, mask, ind, split_layout=split, write_mask_indptr=False)
    torch.cuda.synchronize()
    return mask.cpu().numpy()[:size], ind.cpu().numpy(), va.read_device_status()


@pytest.mark.parametrize("name", ["tiny", "short", "segmented", "stress"])
@pytest.mark.parametrize("split", [False, True])
def test_build_mask_matches_oracle(name, split):
    w = wl.make(name)
    say(f"mask build {name} split={split}")
    parents = np.concatenate(w.parents)
    kv = w.split_buffers()[1] if split else w.kv_indptr
    ref_mask, ref_ind = to.build_mask(parents, w.qo_indptr, kv, split=split)
    mask, ind, status = gpu_mask(w, split)
    assert status == 0
    assert np.array_equal(ind, ref_ind)
    assert np.array_equal(mask, ref_mask)
    assert np.array_equal(mask, w.custom_mask)  # the generator's own mask, built on the host


@pytest.mark.parametrize("split", [False, True])
def test_build_mask_many_requests(split):
    """300 requests, some without tree tokens: the single-launch build reduces and scans the
    segment lengths over more requests than one workgroup pass covers."""
    rng = np.random.default_rng(70)
    t = rng.integers(0, 6, 300)
    p = rng.integers(0, 400, 300)
    w = wl.build_workload("mask300", rng, 2, p, t, int((p + t).sum()) + 64)
    parents = np.concatenate(w.parents) if w.num_tokens else np.zeros(0, np.int64)
    kv = w.split_buffers()[1] if split else w.kv_indptr
    ref_mask, ref_ind = to.build_mask(parents, w.qo_indptr, kv, split=split)
    mask, ind, status = gpu_mask(w, split)
    assert status == 0
    assert np.array_equal(ind, ref_ind)
    assert np.array_equal(mask, ref_mask)
    # and with the offsets given instead of written
    mask2, ind2, status2 = gpu_mask(w, split, indptr=ref_ind)
    assert status2 == 0 and np.array_equal(mask2, ref_mask)


def test_build_mask_reads_given_indptr():
    """Segments at caller-chosen offsets (with gaps): only the segments are written."""
    w = wl.segmented()
    gaps = np.arange(w.bs + 1, dtype=np.int64) * 37
    indptr = w.mask_indptr + gaps
    mask, ind, status = gpu_mask(w, False, indptr=indptr)
    assert status == 0 and np.array_equal(ind, indptr)
    for r in range(w.bs):
        seg = mask[indptr[r]:indptr[r] + (w.mask_indptr[r + 1] - w.mask_indptr[r])]
        assert np.array_equal(seg, w.custom_mask[w.mask_indptr[r]:w.mask_indptr[r + 1]])
        if r + 1 < w.bs:
            assert np.all(mask[indptr[r] + len(seg):indptr[r + 1]] == 7)  # gap untouched


def test_mask_built_on_gpu_drives_verify_bitwise():
    import torch
    from mla_tree_verify_paged_amd.device_inputs import to_device
    from tests.gpu_helpers import run_gpu
    w = wl.short()
    dev = to_device(w)
    ref = run_gpu(w, dev=dev)
    mask, ind, status = gpu_mask(w, False)
    dev["custom_mask"] = torch.from_numpy(mask).cuda()
    dev["mask_indptr"] = torch.from_numpy(ind).cuda()
    got = run_gpu(w, dev=dev)
    assert status == 0 and got[3] == 0
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_bad_parent_is_flagged():
    import torch
    w = wl.tiny()
    va = ctx_for(w)
    parents = np.concatenate(w.parents).astype(np.int64)
    parents[2] = 3  # a parent that does not precede its child
    mask = torch.zeros(int(w.mask_indptr[-1]), dtype=torch.uint8, device="cuda")
    ind = torch.zeros(w.bs + 1, dtype=torch.int64, device="cuda")
    va.build_mask(torch.from_numpy(parents).cuda(), torch.from_numpy(w.qo_indptr).cuda(),
                  torch.from_numpy(w.kv_indptr).cuda(), mask, ind)
    torch.cuda.synchronize()
    assert va.read_device_status() & 16


def random_accept_case(seed, bs, max_t):
    rng = np.random.default_rng(seed)
    t = rng.integers(0, max_t + 1, bs)
    t[0] = max(t[0], 1)
    parents, draft, target = [], [], []
    for r in range(bs):
        par = wl.random_tree(int(t[r]), rng, max_depth=6) if t[r] else np.zeros(0, np.int64)
        d = rng.integers(0, 5, int(t[r]))          # small vocabulary: ties among siblings
        g = rng.integers(0, 5, int(t[r]))
        for c in range(1, int(t[r])):
            if rng.random() < 0.5:
                g[par[c]] = d[c]
        parents.append(par); draft.append(d); target.append(g)
    qo = np.zeros(bs + 1, np.int64)
    qo[1:] = np.cumsum(t)
    cat = lambda xs: np.concatenate(xs).astype(np.int64) if sum(len(x) for x in xs) else \
        np.zeros(1, np.int64)
    return qo, cat(parents), cat(draft), cat(target), int(t.max())


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("max_path", [3, 64])
def test_accept_matches_oracle(seed, max_path):
    import torch
    from mla_tree_verify_paged_amd import VerifyAttn
    bs = 9
    qo, par, drf, tgt, tmax = random_accept_case(900 + seed, bs, 40)
    n = int(qo[-1])
    va = VerifyAttn(8, max_batch=bs, max_q_per_req=max(1, tmax), max_q_tokens=max(1, n))
    acc = torch.full((bs,), -9, dtype=torch.int32, device="cuda")
    path = torch.full((bs, max_path), -9, dtype=torch.int64, device="cuda")
    nxt = torch.full((bs,), -9, dtype=torch.int64, device="cuda")
    d = lambda a: torch.from_numpy(a).cuda()
    va.accept(d(par), d(drf), d(tgt), d(qo), acc, path, nxt, num_tokens=n)
    torch.cuda.synchronize()
    ra, rp, rn = to.accept(par, drf, tgt, qo, max_path)
    say(f"accept seed {seed}: lengths {ra.tolist()}")
    assert va.read_device_status() == 0
    assert np.array_equal(acc.cpu().numpy(), ra)
    assert np.array_equal(path.cpu().numpy(), rp)
    assert np.array_equal(nxt.cpu().numpy(), rn)


def test_build_mask_offset_near_int64_max_is_flagged():
    """A given mask_indptr entry next to INT64_MAX: the overflow-free bounds check rejects that
    request (its rows unwritten, status flagged) and still writes the other one."""
    rng = np.random.default_rng(71)
    w = wl.build_workload("m64", rng, 2, [30, 40], [4, 5], 128)
    indptr = w.mask_indptr.copy()
    indptr[0] = 2**63 - 2
    import torch
    va = ctx_for(w)
    parents = torch.from_numpy(np.concatenate(w.parents).astype(np.int64)).cuda()
    size = int(w.mask_indptr[-1])
    mask = torch.full((size,), 7, dtype=torch.uint8, device="cuda")
    ind = torch.from_numpy(indptr).cuda()
    va.build_mask(parents, torch.from_numpy(w.qo_indptr).cuda(),
                  torch.from_numpy(w.kv_indptr).cuda(), mask, ind, write_mask_indptr=False)
    torch.cuda.synchronize()
    got = mask.cpu().numpy()
    assert va.read_device_status() & 2
    s1 = int(w.mask_indptr[1])
    assert np.all(got[:s1] == 7)
    assert np.array_equal(got[s1:], w.custom_mask[s1:])


def test_tree_kernels_at_the_node_limit():
    """A 2048-node tree (the largest max_q_per_req the tree kernels take) next to a 1-node one:
    the mask byte-exact against the tree oracle, and acceptance along a 2047-step chain whose
    draft tokens all match (one wavefront walks the whole path)."""
    import torch
    from mla_tree_verify_paged_amd import VerifyAttn
    rng = np.random.default_rng(72)
    w = wl.build_workload("t2048", rng, 1, [100, 50], [2048, 1], 4096)
    parents = np.concatenate(w.parents)
    ref_mask, ref_ind = to.build_mask(parents, w.qo_indptr, w.kv_indptr)
    mask, ind, status = gpu_mask(w, False)
    assert status == 0
    assert np.array_equal(ind, ref_ind) and np.array_equal(mask, ref_mask)

    t = 2048
    chain = np.arange(-1, t - 1, dtype=np.int64)        # node k's parent is k - 1
    draft = rng.integers(0, 1000, t).astype(np.int64)
    target = np.roll(draft, -1)                          # node k's target is node k+1's draft
    target[-1] = 5
    qo = np.array([0, t], np.int64)
    va = VerifyAttn(8, max_batch=1, max_q_per_req=t, max_q_tokens=t)
    acc = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    path = torch.full((1, t), -9, dtype=torch.int64, device="cuda")
    nxt = torch.full((1,), -9, dtype=torch.int64, device="cuda")
    d = lambda a: torch.from_numpy(a).cuda()
    va.accept(d(chain), d(draft), d(target), d(qo), acc, path, nxt, num_tokens=t)
    torch.cuda.synchronize()
    ra, rp, rn = to.accept(chain, draft, target, qo, t)
    assert va.read_device_status() == 0
    assert int(ra[0]) == t - 1
    assert np.array_equal(acc.cpu().numpy(), ra)
    assert np.array_equal(path.cpu().numpy(), rp)
    assert np.array_equal(nxt.cpu().numpy(), rn)
