"""Uploads a seeded workload (numpy buffers) into device tensors laid out as the C ABI
expects. Data movement only: the paged pool is filled with NaN and the key rows are scattered
into their slots on the device."""
from __future__ import annotations

import numpy as np
import torch

BF16_NAN_BITS = 0x7FC0


def pool_on_device(w, device="cuda"):
    """The paged KV buffer [num_slots, 576] on `device`; unreferenced rows hold NaN."""
    idx = torch.from_numpy(w.kv_indices).to(device)
    if w.in_dtype == "bf16":
        pool = torch.full((w.num_slots, w.kv_rows.shape[1]), BF16_NAN_BITS, dtype=torch.int16,
                          device=device)
        pool[idx] = torch.from_numpy(w.kv_rows.view(np.int16)).to(device)
        return pool.view(torch.bfloat16)
    pool = torch.full((w.num_slots, w.kv_rows.shape[1]), float("nan"), dtype=torch.float32,
                      device=device)
    pool[idx] = torch.from_numpy(w.kv_rows).to(device)
    return pool


def to_device(w, device="cuda", pool=True):
    """Returns a dict of device tensors for `w` (a workloads.Workload): the buffers of both
    slot layouts (tree slots at the tail of each kv_indices segment, and the prefix-only
    kv_indices with the tree slots in out_cache_loc)."""
    if w.in_dtype == "bf16":
        q = torch.from_numpy(w.q.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        q = torch.from_numpy(w.q).to(device)
    mask = w.custom_mask if w.custom_mask.size else np.zeros(1, np.uint8)
    d = dict(
        q=q,
        kv_indices=torch.from_numpy(w.kv_indices).to(device),
        kv_indptr=torch.from_numpy(w.kv_indptr).to(device),
        qo_indptr=torch.from_numpy(w.qo_indptr).to(device),
        custom_mask=torch.from_numpy(mask).to(device),
        mask_indptr=torch.from_numpy(w.mask_indptr).to(device),
    )
    kvi_p, kvp_p, ocl = w.split_buffers()
    d["kv_indices_prefix"] = torch.from_numpy(kvi_p if kvi_p.size else np.zeros(1, np.int64)).to(
        device)
    d["kv_indptr_prefix"] = torch.from_numpy(kvp_p).to(device)
    d["out_cache_loc"] = torch.from_numpy(ocl if ocl.size else np.zeros(1, np.int64)).to(device)
    if pool:
        d["kv_buffer"] = pool_on_device(w, device)
    return d
