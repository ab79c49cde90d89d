"""Oracle for the two steps around verify attention: building the verify mask from the draft
trees, and greedy acceptance of a verified tree.

TEST INFRASTRUCTURE ONLY: plain loops over small trees, for the tests, the smoke check and the
benchmark's CPU baseline. It shares no code with the GPU library.

The mask ("The Glue That Binds: Wiring a Custom CUDA Kernel into Production via C-ABI",
section "The Thinking Process": the mask is rebuilt from the tree structure rather than
decoded from a packed format; its layout, indexed by the global key position, is the
mask[b][i][j] of "The Glue That Connects", section "Design Decisions and Trade-Offs"):
request r's mask is a [T_r, L_r] row-major byte matrix at mask_indptr[r]; row i holds 1 in
every prefix column j < P_r and, in tail column P_r + k, 1 iff tree node k is node i or one of
its ancestors. mask_indptr is the running sum of T_r * L_r from 0.

Acceptance (the same C-ABI library exposes tree acceptance and tree building next to
verification attention: "The Glue That Connects", section "What the Edit Actually Does"; no
algorithm is given, so this is the plain greedy reading): node 0
of each request is the root, the last accepted token. Walking from the root, the next node is
the lowest-indexed child whose draft token equals the target model's token at the current
node; the walk stops when no child matches. Returned: the number of accepted draft nodes (the
path length minus the root), the path (root first) and the bonus token, the target's token at
the last node of the path.
"""
from __future__ import annotations

import numpy as np


class TreeError(ValueError):
    pass


def request_shapes(qo_indptr, kv_indptr, split=False):
    """(T_r, P_r, L_r) per request, for either slot layout."""
    qo = np.asarray(qo_indptr, dtype=np.int64)
    kv = np.asarray(kv_indptr, dtype=np.int64)
    t = np.diff(qo)
    n = np.diff(kv)
    l = n + t if split else n
    p = l - t
    if np.any(t < 0) or np.any(p < 0):
        raise TreeError("negative tree or prefix length")
    return t, p, l


def ancestors_or_self(parents_r):
    """Boolean [T, T] matrix: anc[i, k] is True iff node k is node i or an ancestor of it.
    Parents must precede their children (-1 for a root)."""
    t = len(parents_r)
    anc = np.zeros((t, t), dtype=bool)
    for i in range(t):
        node = i
        while node >= 0:
            anc[i, node] = True
            p = int(parents_r[node])
            if p >= node:
                raise TreeError(f"node {node} has parent {p}, which does not precede it")
            node = p
    return anc


def mask_indptr(qo_indptr, kv_indptr, split=False):
    t, _, l = request_shapes(qo_indptr, kv_indptr, split)
    out = np.zeros(len(t) + 1, dtype=np.int64)
    out[1:] = np.cumsum(t * l)
    return out


def build_mask(parents, qo_indptr, kv_indptr, split=False):
    """(custom_mask uint8 [sum T_r L_r], mask_indptr int64 [bs+1]) for the trees in
    `parents` (int64 [num_tokens], node indices within each request)."""
    t, p, l = request_shapes(qo_indptr, kv_indptr, split)
    ind = mask_indptr(qo_indptr, kv_indptr, split)
    mask = np.zeros(int(ind[-1]), dtype=np.uint8)
    qo = np.asarray(qo_indptr, dtype=np.int64)
    for r in range(len(t)):
        tr, pr, lr = int(t[r]), int(p[r]), int(l[r])
        if tr == 0:
            continue
        anc = ancestors_or_self(np.asarray(parents[qo[r]:qo[r] + tr], dtype=np.int64))
        m = mask[ind[r]:ind[r + 1]].reshape(tr, lr)
        m[:, :pr] = 1
        m[:, pr:] = anc
    return mask, ind


def accept(parents, draft_tokens, target_tokens, qo_indptr, max_path):
    """Greedy acceptance per request. Returns (accept_len int32 [bs], path int64
    [bs, max_path] with -1 padding, next_token int64 [bs]); a request without tree tokens gets
    accept_len 0, an all -1 path and next_token -1."""
    qo = np.asarray(qo_indptr, dtype=np.int64)
    bs = len(qo) - 1
    acc = np.zeros(bs, dtype=np.int32)
    path = np.full((bs, max_path), -1, dtype=np.int64)
    nxt = np.full(bs, -1, dtype=np.int64)
    for r in range(bs):
        q0, t = int(qo[r]), int(qo[r + 1] - qo[r])
        if t == 0:
            continue
        par = [int(x) for x in parents[q0:q0 + t]]
        cur, walk = 0, [0]
        while True:
            want = int(target_tokens[q0 + cur])
            nxt_node = -1
            for c in range(t):  # lowest index first
                if par[c] == cur and int(draft_tokens[q0 + c]) == want:
                    nxt_node = c
                    break
            if nxt_node < 0:
                break
            cur = nxt_node
            walk.append(cur)
        acc[r] = len(walk) - 1
        path[r, :min(len(walk), max_path)] = walk[:max_path]
        nxt[r] = int(target_tokens[q0 + cur])
    return acc, path, nxt
