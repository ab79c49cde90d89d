"""Seeded synthetic inputs for MLA tree-verify attention over a paged latent KV cache.

This module is shared by the tests, the benchmark and the oracle's callers. It holds
none of the attention arithmetic: only random draws, the bf16 encoding of those draws,
draft-tree construction, the ancestor-or-self visibility mask, and the buffer layout that
the verify call consumes.

Buffer layout (the problem statement of "The Glue That Binds: Wiring a Custom CUDA Kernel
into Production via C-ABI", section "The Broader Engineering Effort", and the dtypes listed
in "The Final Solder Joint", section "The Investigation"):

* ``q``            [num_tokens, H, 576]  absorbed queries (bf16 bits as uint16, or float32)
* ``kv_rows``      [sum_L, 576]          one latent row (512 latent + 64 rope) per key position
* ``kv_indices``   int64 [sum_L]         the pool slot of each key position
* ``kv_indptr``    int32 [bs+1]          per-request key offsets
* ``qo_indptr``    int64 [bs+1]          per-request query-token offsets
* ``custom_mask``  uint8                 per request a [T_r, L_r] row-major byte matrix
* ``mask_indptr``  int64 [bs+1]          element offset of each request's matrix

Per request the last T_r key positions are the draft-tree tokens, in query order, so key
position P_r + k is query token k itself. Prefix columns of the mask are filled with 1;
tree columns hold ancestor-or-self visibility.

Draw order for every workload (numpy ``default_rng(seed)``):
  1. batched workloads only: prefix lengths, then tree sizes;
  2. per request, the tree parents;
  3. the pool slots (distinct);
  4. q ~ N(0,1) float32 [num_tokens, H, 576];
  5. kv ~ N(0,1) float32 [sum_L, 576];
  6. peaked-softmax workload only: the x8 key-row selection.
Then the power-of-two scalings, then rounding to bf16 (round-to-nearest-even).
Unreferenced pool rows hold NaN so that any stray read shows up in the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

LATENT_DIM = 512
ROPE_DIM = 64
KV_DIM = LATENT_DIM + ROPE_DIM
BF16_NAN_BITS = 0x7FC0
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)


# ----------------------------------------------------------------------------- bf16 encoding
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round-to-nearest-even; NaN -> 0x7FC0."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    nan = np.isnan(f)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    r = r.astype(np.uint16)
    r[nan] = BF16_NAN_BITS
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32, exact."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------- draft trees
def chain_tree(t: int) -> np.ndarray:
    """Parents of a linear chain: node i's parent is i-1 (node 0 is the root)."""
    p = np.arange(-1, t - 1, dtype=np.int64)
    return p


def random_tree(t: int, rng: np.random.Generator, max_depth: int | None = None) -> np.ndarray:
    """Node 0 is the root; node i's parent is uniform over earlier nodes (of depth < max_depth)."""
    parents = np.full(t, -1, dtype=np.int64)
    depth = np.zeros(t, dtype=np.int64)
    for i in range(1, t):
        if max_depth is None:
            cand = np.arange(i)
        else:
            cand = np.nonzero(depth[:i] <= max_depth - 1)[0]
        p = int(cand[rng.integers(0, len(cand))])
        parents[i] = p
        depth[i] = depth[p] + 1
    return parents


def tree_depths(parents: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parents), dtype=np.int64)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def ancestor_or_self(parents: np.ndarray) -> np.ndarray:
    """vis[i, k] = 1 iff node k is node i or one of its ancestors."""
    t = len(parents)
    vis = np.zeros((t, t), dtype=np.uint8)
    for i in range(t):
        k = i
        while k >= 0:
            vis[i, k] = 1
            k = int(parents[k])
    return vis


# ----------------------------------------------------------------------------- workload
@dataclass
class Workload:
    name: str
    in_dtype: str                  # "bf16" or "fp32"
    num_heads: int
    scale: float
    num_slots: int
    prefix_lens: np.ndarray        # int64 [bs]
    tree_lens: np.ndarray          # int64 [bs]
    parents: list                  # per request int64 [T_r]
    q: np.ndarray                  # [num_tokens, H, 576] uint16 bits or float32
    kv_rows: np.ndarray            # [sum_L, 576] uint16 bits or float32
    kv_indices: np.ndarray         # int64 [sum_L]
    kv_indptr: np.ndarray          # int32 [bs+1]
    qo_indptr: np.ndarray          # int64 [bs+1]
    custom_mask: np.ndarray        # uint8 [sum_r T_r*L_r]
    mask_indptr: np.ndarray        # int64 [bs+1]
    meta: dict = field(default_factory=dict)

    @property
    def bs(self) -> int:
        return int(len(self.prefix_lens))

    @property
    def num_tokens(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def max_q_per_req(self) -> int:
        return int(self.tree_lens.max()) if self.bs else 0

    @property
    def max_kv_per_req(self) -> int:
        return int((self.prefix_lens + self.tree_lens).max()) if self.bs else 0

    def pool_np(self) -> np.ndarray:
        """The paged KV buffer [num_slots, 576]; unreferenced rows hold NaN."""
        if self.in_dtype == "bf16":
            pool = np.full((self.num_slots, KV_DIM), BF16_NAN_BITS, dtype=np.uint16)
        else:
            pool = np.full((self.num_slots, KV_DIM), np.nan, dtype=np.float32)
        pool[self.kv_indices] = self.kv_rows
        return pool

    def split_buffers(self):
        """The same key slots in the prefix / out_cache_loc layout: (kv_indices holding each
        request's prefix slots only, its int32 indptr, out_cache_loc [num_tokens] holding the
        tree tokens' slots in token order)."""
        kvi, kvp, ocl = [], [0], []
        for r in range(self.bs):
            a, b = int(self.kv_indptr[r]), int(self.kv_indptr[r + 1])
            p = int(self.prefix_lens[r])
            kvi.append(self.kv_indices[a:a + p])
            ocl.append(self.kv_indices[a + p:b])
            kvp.append(kvp[-1] + p)
        cat = lambda xs: (np.concatenate(xs) if xs else np.zeros(0)).astype(np.int64)
        return cat(kvi), np.asarray(kvp, dtype=np.int32), cat(ocl)

    def q_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.q) if self.in_dtype == "bf16" else self.q

    def kv_rows_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.kv_rows) if self.in_dtype == "bf16" else self.kv_rows


def _encode(x: np.ndarray, in_dtype: str) -> np.ndarray:
    if in_dtype == "bf16":
        return to_bf16_bits(x)
    if in_dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(in_dtype)


def build_workload(
    name: str,
    rng: np.random.Generator,
    num_heads: int,
    prefix_lens,
    tree_lens,
    num_slots: int,
    in_dtype: str = "bf16",
    tree: str = "random",
    max_depth: int | None = None,
    rope_scale: float = 1.0,
    spike_frac: float = 0.0,
    spike_scale: float = 8.0,
    scale: float = DEFAULT_SCALE,
    slots: str = "choice",
) -> Workload:
    """Draws steps 2-6 of the documented order from ``rng`` and lays out the buffers."""
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    tree_lens = np.asarray(tree_lens, dtype=np.int64)
    bs = len(prefix_lens)
    kv_lens = prefix_lens + tree_lens
    # 2. trees
    parents = []
    for r in range(bs):
        t = int(tree_lens[r])
        if tree == "chain":
            parents.append(chain_tree(t))
        elif tree == "random":
            parents.append(random_tree(t, rng, max_depth) if t > 0 else np.zeros(0, np.int64))
        else:
            raise ValueError(tree)
    # 3. slots
    sum_l = int(kv_lens.sum())
    if sum_l > num_slots:
        raise ValueError("pool too small")
    if slots == "permutation":
        kv_indices = rng.permutation(num_slots)[:sum_l].astype(np.int64)
    else:
        kv_indices = rng.choice(num_slots, sum_l, replace=False).astype(np.int64)
    # 4./5. q and kv draws
    num_tokens = int(tree_lens.sum())
    q = rng.standard_normal((num_tokens, num_heads, KV_DIM), dtype=np.float32)
    kv = rng.standard_normal((sum_l, KV_DIM), dtype=np.float32)
    # 6. spikes
    if spike_frac > 0.0:
        spike = rng.random(sum_l) < spike_frac
        kv[spike] *= np.float32(spike_scale)
    if rope_scale != 1.0:
        q[:, :, LATENT_DIM:] *= np.float32(rope_scale)
        kv[:, LATENT_DIM:] *= np.float32(rope_scale)
    # layout
    kv_indptr = np.zeros(bs + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(kv_lens)
    qo_indptr = np.zeros(bs + 1, dtype=np.int64)
    qo_indptr[1:] = np.cumsum(tree_lens)
    mask_indptr = np.zeros(bs + 1, dtype=np.int64)
    mask_indptr[1:] = np.cumsum(tree_lens * kv_lens)
    custom_mask = np.zeros(int(mask_indptr[-1]), dtype=np.uint8)
    for r in range(bs):
        t, p, l = int(tree_lens[r]), int(prefix_lens[r]), int(kv_lens[r])
        m = custom_mask[mask_indptr[r]:mask_indptr[r + 1]].reshape(t, l)
        m[:, :p] = 1
        m[:, p:] = ancestor_or_self(parents[r])
    return Workload(
        name=name, in_dtype=in_dtype, num_heads=num_heads, scale=float(scale),
        num_slots=int(num_slots), prefix_lens=prefix_lens, tree_lens=tree_lens,
        parents=parents, q=_encode(q, in_dtype), kv_rows=_encode(kv, in_dtype),
        kv_indices=kv_indices, kv_indptr=kv_indptr, qo_indptr=qo_indptr,
        custom_mask=custom_mask, mask_indptr=mask_indptr,
    )


# ----------------------------------------------------------------------------- the five workloads
def tiny(seed: int = 0) -> Workload:
    """1 request, H=8, P=64, T=4 linear chain, fp32 N(0,1), 68 of 128 slots."""
    rng = np.random.default_rng(seed)
    return build_workload("tiny", rng, 8, [64], [4], 128, in_dtype="fp32", tree="chain",
                          slots="permutation")


def short(seed: int = 0) -> Workload:
    """1 request, H=64, P=5,700, T=16 random tree, bf16, 262,144-slot pool."""
    rng = np.random.default_rng(seed)
    return build_workload("short", rng, 64, [5700], [16], 262_144)


def long(seed: int = 0) -> Workload:
    """1 request, H=64, P=23,000, T=16 random tree, bf16, rope dims x0.5, 1,048,576-slot pool."""
    rng = np.random.default_rng(seed)
    return build_workload("long", rng, 64, [23_000], [16], 1_048_576, rope_scale=0.5)


def segmented(seed: int = 0) -> Workload:
    """8 requests, H=64, P_r log-uniform in [1024, 32768], T_r in {8,16,32}, bf16."""
    rng = np.random.default_rng(seed)
    p = np.floor(np.exp(rng.uniform(math.log(1024), math.log(32768), 8))).astype(np.int64)
    t = rng.choice([8, 16, 32], 8).astype(np.int64)
    return build_workload("segmented", rng, 64, p, t, 1_048_576)


def stress(seed: int = 0) -> Workload:
    """2 requests, H=64, P=131,072, T=64 trees of depth <= 8, 1% of key rows x8, bf16."""
    rng = np.random.default_rng(seed)
    return build_workload("stress", rng, 64, [131_072, 131_072], [64, 64], 2_097_152,
                          max_depth=8, spike_frac=0.01)


# ----------------------------------------------------------------------------- few rows per request
# One GPU's share of the heads under 8-way tensor parallelism (H = 64 / 8) with small draft trees:
# few query rows per request, so the key rows' bytes decide the time rather than the matrix work.
def tp8(seed: int = 0) -> Workload:
    """1 request, H=8, P=23,000, T=4 random tree, bf16, rope dims x0.5, 1,048,576-slot pool."""
    rng = np.random.default_rng(seed)
    return build_workload("tp8", rng, 8, [23_000], [4], 1_048_576, rope_scale=0.5)


def tp8_batch(seed: int = 0) -> Workload:
    """32 requests, H=8, P_r log-uniform in [1024, 32768], T_r uniform in {1, 2, 3, 4}, bf16."""
    rng = np.random.default_rng(seed)
    p = np.floor(np.exp(rng.uniform(math.log(1024), math.log(32768), 32))).astype(np.int64)
    t = rng.integers(1, 5, 32).astype(np.int64)
    return build_workload("tp8_batch", rng, 8, p, t, 1_048_576)


def small_trees(seed: int = 0) -> Workload:
    """16 requests, H=64, P_r log-uniform in [1024, 32768], T_r uniform in {1, 2, 3, 4}, bf16:
    small draft trees with all heads on one GPU (64 to 256 rows per request)."""
    rng = np.random.default_rng(seed)
    p = np.floor(np.exp(rng.uniform(math.log(1024), math.log(32768), 16))).astype(np.int64)
    t = rng.integers(1, 5, 16).astype(np.int64)
    return build_workload("small_trees", rng, 64, p, t, 1_048_576)


CONFIGS = {"tiny": tiny, "short": short, "long": long, "segmented": segmented, "stress": stress,
           "tp8": tp8, "tp8_batch": tp8_batch, "small_trees": small_trees}


def make(name: str, seed: int = 0) -> Workload:
    return CONFIGS[name](seed)
