"""Pins for the tree-mask and acceptance oracle (CPU only): closed forms, a transitive
closure computed a different way, and brute force over root paths."""
import itertools

import numpy as np
import pytest

import workloads as wl
from oracle import tree_oracle as to


def closure(parents_r):
    """Ancestor-or-self by boolean matrix powers of the parent relation (independent of the
    oracle's walk)."""
    t = len(parents_r)
    a = np.eye(t, dtype=np.int64)
    e = np.zeros((t, t), dtype=np.int64)
    for i, p in enumerate(parents_r):
        if p >= 0:
            e[i, p] = 1
    step = a.copy()
    for _ in range(t):
        step = (step @ e > 0).astype(np.int64)
        a |= step
    return a.astype(bool)


def test_chain_is_lower_triangular():
    t = 7
    anc = to.ancestors_or_self(np.arange(-1, t - 1))
    assert np.array_equal(anc, np.tril(np.ones((t, t), dtype=bool)))


def test_star_is_identity_plus_root_column():
    t = 6
    par = np.array([-1] + [0] * (t - 1))
    anc = to.ancestors_or_self(par)
    ref = np.eye(t, dtype=bool)
    ref[:, 0] = True
    assert np.array_equal(anc, ref)


@pytest.mark.parametrize("seed", range(6))
def test_random_trees_match_matrix_closure(seed):
    rng = np.random.default_rng(300 + seed)
    t = int(rng.integers(1, 40))
    par = wl.random_tree(t, rng, max_depth=int(rng.integers(1, 9)))
    assert np.array_equal(to.ancestors_or_self(par), closure(par))


def test_parent_must_precede_child():
    with pytest.raises(to.TreeError):
        to.ancestors_or_self(np.array([-1, 2, 0]))


@pytest.mark.parametrize("split", [False, True])
def test_build_mask_layout(split):
    """Prefix columns are all ones, the tail is the closure, rows are L_r long, segments
    follow each other from offset 0."""
    rng = np.random.default_rng(11)
    w = wl.build_workload("m", rng, 2, [5, 0, 9], [3, 4, 1], 64)
    parents = np.concatenate(w.parents)
    kvi, kvp, ocl = w.split_buffers()
    kv = kvp if split else w.kv_indptr
    mask, ind = to.build_mask(parents, w.qo_indptr, kv, split=split)
    t = w.tree_lens
    l = w.prefix_lens + t
    assert ind[0] == 0 and np.array_equal(np.diff(ind), t * l)
    for r in range(w.bs):
        m = mask[ind[r]:ind[r + 1]].reshape(int(t[r]), int(l[r]))
        p = int(w.prefix_lens[r])
        assert np.all(m[:, :p] == 1)
        assert np.array_equal(m[:, p:].astype(bool), closure(w.parents[r]))


def brute_force_accept(par, draft, target):
    """The longest root path whose every step matches (child's draft token == the target's
    token at its parent), by enumerating every node's root path."""
    t = len(par)
    best = [0]
    for n in range(t):
        walk = [n]
        while walk[-1] != 0:
            walk.append(par[walk[-1]])
        walk = walk[::-1]
        if walk[0] != 0:
            continue
        if all(draft[walk[k + 1]] == target[walk[k]] for k in range(len(walk) - 1)):
            if len(walk) > len(best):
                best = walk
    return best


@pytest.mark.parametrize("seed", range(8))
def test_accept_matches_brute_force_with_distinct_sibling_tokens(seed):
    """With distinct tokens among siblings at most one child can match, so the greedy walk
    is the unique longest matching root path."""
    rng = np.random.default_rng(500 + seed)
    t = int(rng.integers(1, 30))
    par = wl.random_tree(t, rng, max_depth=6)
    draft = np.zeros(t, dtype=np.int64)
    for p in range(t):
        kids = [c for c in range(t) if par[c] == p]
        draft[kids] = rng.permutation(8)[:len(kids)]
    target = rng.integers(0, 8, t)
    # make a few long matches likely
    for c in range(1, t):
        if rng.random() < 0.6:
            target[par[c]] = draft[c]
    acc, path, nxt = to.accept(par, draft, target, [0, t], t)
    ref = brute_force_accept(list(par), list(draft), list(target))
    assert acc[0] == len(ref) - 1
    assert list(path[0, :len(ref)]) == ref and np.all(path[0, len(ref):] == -1)
    assert nxt[0] == target[ref[-1]]


def test_accept_chain_closed_forms():
    par = np.arange(-1, 5)                 # chain of 6 nodes
    draft = np.array([0, 10, 11, 12, 13, 14])
    target = np.array([10, 11, 12, 99, 14, 15])  # the 4th step mismatches
    acc, path, nxt = to.accept(par, draft, target, [0, 6], 6)
    assert acc[0] == 3 and list(path[0]) == [0, 1, 2, 3, -1, -1] and nxt[0] == 99


def test_accept_tie_takes_lowest_index_and_empty_request():
    par = np.array([-1, 0, 0, 1, 2])
    draft = np.array([0, 7, 7, 5, 6])
    target = np.array([7, 5, 6, 1, 2])
    acc, path, nxt = to.accept(np.concatenate([par, par]), np.concatenate([draft, draft]),
                               np.concatenate([target, target]), [0, 5, 5, 10], 5)
    assert list(acc) == [2, 0, 2]
    assert list(path[0, :3]) == [0, 1, 3] and nxt[0] == 1
    assert np.all(path[1] == -1) and nxt[1] == -1
