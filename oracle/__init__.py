"""Python access to the fp64 CPU oracle for MLA tree-verify attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the GPU library or its binding. The oracle itself is plain C
(``verify_attn_oracle.c``); this wrapper compiles it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "verify_attn_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_verify_attn.so")
_CFLAGS = ["-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c99", "-Wall", "-Wextra"]

_lib = None


def build(src: str = _SRC, out: str = LIB_PATH, extra=()) -> str:
    """Compile the oracle into a shared library (gcc, no fast-math)."""
    tmp = out + ".tmp"
    cmd = ["gcc", *_CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


def load(path: str = LIB_PATH):
    global _lib
    if path == LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path) or (
            path == LIB_PATH and os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build(out=path)
    lib = ctypes.CDLL(path)
    f = lib.oracle_verify_attn_f64
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int64, vp, vp, vp, vp, vp, vp,
                  ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_double, vp, ctypes.c_int64, vp, vp, vp, ctypes.c_int32]
    g = lib.oracle_score_top2_f64
    g.restype = ctypes.c_int
    g.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int64, vp, vp, vp, vp, vp, vp,
                  ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_double, vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                  vp, vp, vp, ctypes.c_int32]
    if path == LIB_PATH:
        _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def verify_attn(q, kv_buffer, kv_indices, kv_indptr, qo_indptr, custom_mask, mask_indptr,
                num_heads, scale, latent_dim=512, rope_dim=64, rows=None, nthreads=0,
                lib=None, out_cache_loc=None):
    """Runs the oracle. ``q`` and ``kv_buffer`` are bf16 bits (uint16) or float32.

    With ``out_cache_loc`` (int64 [num_tokens]) the kv_indices segments hold the prefix slots
    only and the tree tokens' slots are taken from ``out_cache_loc``.

    Returns (out [n, Dl] float64, lse [n] float64, argmax [n] int64) where n runs over
    ``rows`` (flat t*H + h ids) or over every (token, head) row.
    """
    lib = lib or load()
    if q.dtype == np.uint16:
        in_dtype = 0
    elif q.dtype == np.float32:
        in_dtype = 1
    else:
        raise TypeError(q.dtype)
    if kv_buffer.dtype != q.dtype:
        raise TypeError("q and kv_buffer dtypes differ")
    d = latent_dim + rope_dim
    q = np.ascontiguousarray(q)
    kv_buffer = np.ascontiguousarray(kv_buffer)
    if q.size % (num_heads * d) or kv_buffer.size % d:
        raise ValueError("shape")
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int64)
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    qo_indptr = np.ascontiguousarray(qo_indptr, dtype=np.int64)
    custom_mask = np.ascontiguousarray(custom_mask, dtype=np.uint8)
    mask_indptr = np.ascontiguousarray(mask_indptr, dtype=np.int64)
    if out_cache_loc is not None:
        out_cache_loc = np.ascontiguousarray(out_cache_loc, dtype=np.int64)
    bs = len(kv_indptr) - 1
    num_tokens = int(qo_indptr[-1]) if bs > 0 else 0
    if q.size != num_tokens * num_heads * d:
        raise ValueError("q does not match qo_indptr")
    if out_cache_loc is not None and out_cache_loc.size < num_tokens:
        raise ValueError("out_cache_loc shorter than the token count")
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = len(rows)
    else:
        n = num_tokens * num_heads
    out = np.zeros((n, latent_dim), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    am = np.zeros(n, dtype=np.int64)
    mask_arg = custom_mask if custom_mask.size else np.zeros(1, np.uint8)
    rc = lib.oracle_verify_attn_f64(
        _ptr(q), _ptr(kv_buffer), in_dtype, kv_buffer.size // d, _ptr(kv_indices),
        _ptr(kv_indptr), _ptr(qo_indptr), _ptr(out_cache_loc), _ptr(mask_arg), _ptr(mask_indptr),
        custom_mask.size, bs, num_heads, latent_dim, rope_dim, float(scale), _ptr(rows), n,
        _ptr(out), _ptr(lse), _ptr(am), int(nthreads))
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")
    return out, lse, am


def run_workload(w, rows=None, nthreads=0, pool=None, lib=None, split=False):
    """The oracle on a ``workloads.Workload`` (with ``split``, given in the prefix /
    out_cache_loc layout)."""
    if pool is None:
        pool = w.pool_np()
    if split:
        kvi, kvp, ocl = w.split_buffers()
        return verify_attn(w.q, pool, kvi, kvp, w.qo_indptr, w.custom_mask, w.mask_indptr,
                           w.num_heads, w.scale, rows=rows, nthreads=nthreads, lib=lib,
                           out_cache_loc=ocl)
    return verify_attn(w.q, pool, w.kv_indices, w.kv_indptr, w.qo_indptr, w.custom_mask,
                       w.mask_indptr, w.num_heads, w.scale, rows=rows, nthreads=nthreads,
                       lib=lib)


def score_top2(q, kv_buffer, kv_indices, kv_indptr, qo_indptr, custom_mask, mask_indptr,
               num_heads, scale, rows=None, pair_rows=None, pair_keys=None, latent_dim=512,
               rope_dim=64, nthreads=0, lib=None, out_cache_loc=None):
    """Exact score diagnostics (see ``oracle_score_top2_f64``): per listed row the largest
    visible score, its lowest key position, the runner-up score and the largest
    ``|scale| * sum_d |q_d k_d|``; per (row, key) pair the score, that magnitude and
    visibility. Returns a dict of numpy arrays."""
    lib = lib or load()
    in_dtype = {np.dtype(np.uint16): 0, np.dtype(np.float32): 1}[np.dtype(q.dtype)]
    q = np.ascontiguousarray(q)
    kv_buffer = np.ascontiguousarray(kv_buffer)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int64)
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    qo_indptr = np.ascontiguousarray(qo_indptr, dtype=np.int64)
    custom_mask = np.ascontiguousarray(custom_mask, dtype=np.uint8)
    mask_indptr = np.ascontiguousarray(mask_indptr, dtype=np.int64)
    if out_cache_loc is not None:
        out_cache_loc = np.ascontiguousarray(out_cache_loc, dtype=np.int64)
    d = latent_dim + rope_dim
    bs = len(kv_indptr) - 1
    num_tokens = int(qo_indptr[-1]) if bs > 0 else 0
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = len(rows)
    else:
        n = num_tokens * num_heads
    if pair_rows is None:
        pair_rows = np.zeros(0, np.int64)
        pair_keys = np.zeros(0, np.int64)
    pair_rows = np.ascontiguousarray(pair_rows, dtype=np.int64)
    pair_keys = np.ascontiguousarray(pair_keys, dtype=np.int64)
    if pair_rows.shape != pair_keys.shape:
        raise ValueError("pair_rows and pair_keys differ in length")
    npair = len(pair_rows)
    res = {"top1": np.zeros(n), "arg1": np.zeros(n, np.int64), "top2": np.zeros(n),
           "absmax": np.zeros(n), "pair_s": np.zeros(npair), "pair_abs": np.zeros(npair),
           "pair_vis": np.zeros(npair, np.int32)}
    mask_arg = custom_mask if custom_mask.size else np.zeros(1, np.uint8)
    rc = lib.oracle_score_top2_f64(
        _ptr(q), _ptr(kv_buffer), in_dtype, kv_buffer.size // d, _ptr(kv_indices),
        _ptr(kv_indptr), _ptr(qo_indptr), _ptr(out_cache_loc), _ptr(mask_arg), _ptr(mask_indptr),
        custom_mask.size, bs, num_heads, latent_dim, rope_dim, float(scale), _ptr(rows), n,
        _ptr(res["top1"]), _ptr(res["arg1"]), _ptr(res["top2"]), _ptr(res["absmax"]),
        _ptr(pair_rows), _ptr(pair_keys), npair, _ptr(res["pair_s"]), _ptr(res["pair_abs"]),
        _ptr(res["pair_vis"]), int(nthreads))
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")
    return res


def workload_top2(w, rows=None, pair_rows=None, pair_keys=None, pool=None, split=False,
                  nthreads=0):
    """``score_top2`` on a ``workloads.Workload``."""
    if pool is None:
        pool = w.pool_np()
    if split:
        kvi, kvp, ocl = w.split_buffers()
        return score_top2(w.q, pool, kvi, kvp, w.qo_indptr, w.custom_mask, w.mask_indptr,
                          w.num_heads, w.scale, rows=rows, pair_rows=pair_rows,
                          pair_keys=pair_keys, nthreads=nthreads, out_cache_loc=ocl)
    return score_top2(w.q, pool, w.kv_indices, w.kv_indptr, w.qo_indptr, w.custom_mask,
                      w.mask_indptr, w.num_heads, w.scale, rows=rows, pair_rows=pair_rows,
                      pair_keys=pair_keys, nthreads=nthreads)
