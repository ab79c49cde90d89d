"""Thin ctypes binding of libverify_attn.so (the C ABI in include/verify_attn.h).

Every step of the verify path runs in the library's HIP kernels; this module only marshals
arguments. PyTorch supplies device memory and the current stream. If the library is not
built, importing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

# torch first: its bundled HIP runtime (soname libamdhip64.so.7) must be the one the library
# binds to, so that streams and device pointers from torch are valid in the library.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("VERIFY_ATTN_LIB", os.path.join(_HERE, "libverify_attn.so"))

VA_OK, VA_ERR_NULL, VA_ERR_INVALID, VA_ERR_UNSUPPORTED, VA_ERR_WORKSPACE, VA_ERR_HIP = range(6)
VA_BF16, VA_FP32 = 0, 1
VA_KERNEL_AUTO, VA_KERNEL_SIMPLE, VA_KERNEL_MFMA = 0, 1, 2
VA_DEV_SLOT_RANGE, VA_DEV_SEGMENT, VA_DEV_Q_PER_REQ, VA_DEV_TOKENS, VA_DEV_TREE = 1, 2, 4, 8, 16

EXPORTED = (
    "verify_attn_workspace_bytes", "verify_attn_create", "verify_attn_run",
    "verify_attn_read_device_status", "verify_attn_set_profiling_events",
    "verify_attn_get_info", "verify_attn_destroy", "verify_attn_last_error",
    "verify_attn_build_mask", "verify_attn_accept", "verify_attn_run_static",
)


class verify_attn_config(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32), ("latent_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("max_batch", ctypes.c_int32),
        ("max_q_per_req", ctypes.c_int32), ("max_q_tokens", ctypes.c_int64),
        ("num_splits", ctypes.c_int32), ("kernel", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class verify_attn_info(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32), ("row_tiles_per_req", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t), ("partial_waves", ctypes.c_int32),
    ]


class VerifyAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"verify_attn status {status}: {msg}")
        self.status = status


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() or "
                          f"python mla_tree_verify_paged_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    cfgp = ctypes.POINTER(verify_attn_config)
    lib.verify_attn_workspace_bytes.argtypes = [cfgp]
    lib.verify_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.verify_attn_create.argtypes = [cfgp, ctypes.POINTER(vp)]
    lib.verify_attn_create.restype = ctypes.c_int
    lib.verify_attn_run.argtypes = [vp, vp, vp, i64, vp, i64, vp, vp, vp, i64, vp, vp, i32,
                                    i64, f32, vp, vp, vp, vp]
    lib.verify_attn_run.restype = ctypes.c_int
    lib.verify_attn_run_static.argtypes = [cfgp, vp, vp, i64, vp, i64, vp, vp, vp, i64, vp, vp,
                                           i32, i64, f32, vp, vp, vp, vp]
    lib.verify_attn_run_static.restype = ctypes.c_int
    lib.verify_attn_read_device_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.verify_attn_read_device_status.restype = ctypes.c_int
    lib.verify_attn_set_profiling_events.argtypes = [vp, vp, vp, vp]
    lib.verify_attn_set_profiling_events.restype = ctypes.c_int
    lib.verify_attn_get_info.argtypes = [vp, ctypes.POINTER(verify_attn_info)]
    lib.verify_attn_get_info.restype = ctypes.c_int
    lib.verify_attn_build_mask.argtypes = [vp, vp, vp, vp, i32, i32, i64, vp, i64, vp, i32, vp]
    lib.verify_attn_build_mask.restype = ctypes.c_int
    lib.verify_attn_accept.argtypes = [vp, vp, vp, vp, vp, i32, i64, vp, vp, i32, vp, vp]
    lib.verify_attn_accept.restype = ctypes.c_int
    lib.verify_attn_destroy.argtypes = [vp]
    lib.verify_attn_destroy.restype = None
    lib.verify_attn_last_error.argtypes = []
    lib.verify_attn_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def verify_attn_last_error() -> str:
    return lib.verify_attn_last_error().decode()


def _check(st: int):
    if st != VA_OK:
        raise VerifyAttnError(st, verify_attn_last_error())


def make_config(num_heads, in_dtype=VA_BF16, out_dtype=VA_FP32, max_batch=1, max_q_per_req=16,
                max_q_tokens=None, num_splits=0, kernel=VA_KERNEL_AUTO, workspace=None,
                workspace_bytes=0, latent_dim=512, rope_dim=64) -> verify_attn_config:
    if max_q_tokens is None:
        max_q_tokens = max_batch * max_q_per_req
    return verify_attn_config(num_heads, latent_dim, rope_dim, in_dtype, out_dtype, max_batch,
                              max_q_per_req, max_q_tokens, num_splits, kernel, workspace,
                              workspace_bytes)


def verify_attn_workspace_bytes(cfg: verify_attn_config) -> int:
    return int(lib.verify_attn_workspace_bytes(ctypes.byref(cfg)))


def verify_attn_create(cfg: verify_attn_config) -> int:
    ctx = ctypes.c_void_p()
    _check(lib.verify_attn_create(ctypes.byref(cfg), ctypes.byref(ctx)))
    return ctx.value


def verify_attn_run(ctx, q, kv_buffer, num_slots, kv_indices, num_kv_indices, kv_indptr,
                    qo_indptr, custom_mask, mask_len, mask_indptr, out_cache_loc, bs, num_tokens,
                    sm_scale, out, out_lse, out_argmax, stream) -> None:
    """Pointer-level call: every buffer argument is a device address (int) or None."""
    _check(lib.verify_attn_run(ctx, q, kv_buffer, num_slots, kv_indices, num_kv_indices,
                               kv_indptr, qo_indptr, custom_mask, mask_len, mask_indptr,
                               out_cache_loc, bs, num_tokens, sm_scale, out, out_lse,
                               out_argmax, stream))


def verify_attn_run_static(cfg, q, kv_buffer, num_slots, kv_indices, num_kv_indices, kv_indptr,
                           qo_indptr, custom_mask, mask_len, mask_indptr, out_cache_loc, bs,
                           num_tokens, sm_scale, out, out_lse, out_argmax, stream) -> None:
    """Pointer-level call of the allocation-free entry point (a config, no context)."""
    _check(lib.verify_attn_run_static(ctypes.byref(cfg), q, kv_buffer, num_slots, kv_indices,
                                      num_kv_indices, kv_indptr, qo_indptr, custom_mask,
                                      mask_len, mask_indptr, out_cache_loc, bs, num_tokens,
                                      sm_scale, out, out_lse, out_argmax, stream))


def verify_attn_build_mask(ctx, parents, qo_indptr, kv_indptr, split_layout, bs, num_tokens,
                           custom_mask, mask_len, mask_indptr, write_mask_indptr,
                           stream) -> None:
    """Pointer-level call: every buffer argument is a device address (int) or None."""
    _check(lib.verify_attn_build_mask(ctx, parents, qo_indptr, kv_indptr, split_layout, bs,
                                      num_tokens, custom_mask, mask_len, mask_indptr,
                                      write_mask_indptr, stream))


def verify_attn_accept(ctx, parents, draft_tokens, target_tokens, qo_indptr, bs, num_tokens,
                       accept_len, accept_path, max_path, next_token, stream) -> None:
    """Pointer-level call: every buffer argument is a device address (int) or None."""
    _check(lib.verify_attn_accept(ctx, parents, draft_tokens, target_tokens, qo_indptr, bs,
                                  num_tokens, accept_len, accept_path, max_path, next_token,
                                  stream))


def verify_attn_read_device_status(ctx, stream=None) -> int:
    flags = ctypes.c_uint32()
    _check(lib.verify_attn_read_device_status(ctx, stream, ctypes.byref(flags)))
    return int(flags.value)


def verify_attn_set_profiling_events(ctx, before, between, after) -> None:
    _check(lib.verify_attn_set_profiling_events(ctx, before, between, after))


def verify_attn_get_info(ctx) -> verify_attn_info:
    info = verify_attn_info()
    _check(lib.verify_attn_get_info(ctx, ctypes.byref(info)))
    return info


def verify_attn_destroy(ctx) -> None:
    lib.verify_attn_destroy(ctx)


# ----------------------------------------------------------------------------- torch marshalling
def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_tensor(name, t, dtypes, min_numel=0, shape=None, device_check=True):
    """Raises ValueError unless `t` has one of `dtypes`, at least `min_numel` elements, the
    given trailing shape (None entries match anything), is contiguous and (with
    device_check) lives on a GPU. Shape and dtype are checked first."""
    import torch
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
    if shape is not None:
        _need(t.dim() == len(shape), f"{name} must have {len(shape)} dims, got {tuple(t.shape)}")
        for i, (got, want) in enumerate(zip(t.shape, shape)):
            _need(want is None or got == want,
                  f"{name} dim {i} is {got}, expected {want} (shape {tuple(t.shape)})")
    _need(t.numel() >= min_numel, f"{name} holds {t.numel()} elements, needs >= {min_numel}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if device_check:
        _need(t.is_cuda, f"{name} must be a GPU tensor")


def validate_run(num_heads, in_dtype, out_dtype, q, kv_buffer, kv_indices, kv_indptr,
                 qo_indptr, custom_mask, mask_indptr, out, out_lse, out_argmax, bs, num_tokens,
                 out_cache_loc=None, device_check=True):
    """Checks the tensors of one verify step against the layouts include/verify_attn.h
    states (dtype, shape, contiguity, device), so that no pointer reaches the C ABI with a
    layout the kernels would misread. Raises ValueError."""
    import torch
    fdt = {"bf16": torch.bfloat16, "fp32": torch.float32}
    _need(bs >= 0 and num_tokens >= 0, "bs and num_tokens must be >= 0")
    dc = device_check
    _check_tensor("q", q, (fdt[in_dtype],), num_tokens * num_heads * 576,
                  (None, num_heads, 576), dc)
    _check_tensor("kv_buffer", kv_buffer, (fdt[in_dtype],), 576, (None, 576), dc)
    _check_tensor("kv_indices", kv_indices, (torch.int64,), 0, None, dc)
    _check_tensor("kv_indptr", kv_indptr, (torch.int32,), bs + 1, None, dc)
    _check_tensor("qo_indptr", qo_indptr, (torch.int64,), bs + 1, None, dc)
    _check_tensor("custom_mask", custom_mask, (torch.uint8, torch.bool), 0, None, dc)
    _check_tensor("mask_indptr", mask_indptr, (torch.int64,), bs + 1, None, dc)
    if out_cache_loc is not None:
        _check_tensor("out_cache_loc", out_cache_loc, (torch.int64,), num_tokens, None, dc)
    _check_tensor("out", out, (fdt[out_dtype],), num_tokens * num_heads * 512,
                  (None, num_heads, 512), dc)
    if out_lse is not None:
        _check_tensor("out_lse", out_lse, (torch.float32,), num_tokens * num_heads, None, dc)
    if out_argmax is not None:
        _check_tensor("out_argmax", out_argmax, (torch.int32,), num_tokens * num_heads, None,
                      dc)


def validate_tree_args(parents, qo_indptr, kv_indptr, bs, num_tokens, custom_mask=None,
                       mask_indptr=None, draft_tokens=None, target_tokens=None, accept_len=None,
                       accept_path=None, next_token=None, device_check=True):
    """The same checks for the mask build and the acceptance calls."""
    import torch
    dc = device_check
    _need(bs >= 0 and num_tokens >= 0, "bs and num_tokens must be >= 0")
    _check_tensor("parents", parents, (torch.int64,), num_tokens, None, dc)
    _check_tensor("qo_indptr", qo_indptr, (torch.int64,), bs + 1, None, dc)
    if kv_indptr is not None:
        _check_tensor("kv_indptr", kv_indptr, (torch.int32,), bs + 1, None, dc)
    if custom_mask is not None:
        _check_tensor("custom_mask", custom_mask, (torch.uint8, torch.bool), 0, None, dc)
    if mask_indptr is not None:
        _check_tensor("mask_indptr", mask_indptr, (torch.int64,), bs + 1, None, dc)
    for name, t in (("draft_tokens", draft_tokens), ("target_tokens", target_tokens)):
        if t is not None:
            _check_tensor(name, t, (torch.int64,), num_tokens, None, dc)
    if accept_len is not None:
        _check_tensor("accept_len", accept_len, (torch.int32,), bs, None, dc)
    if accept_path is not None:
        _check_tensor("accept_path", accept_path, (torch.int64,), bs, (None, None), dc)
        _need(accept_path.shape[0] >= bs, "accept_path needs bs rows")
    if next_token is not None:
        _check_tensor("next_token", next_token, (torch.int64,), bs, None, dc)


class VerifyAttn:
    """Owns one context; ``run`` marshals torch tensors into ``verify_attn_run``."""

    def __init__(self, num_heads, in_dtype="bf16", out_dtype="fp32", max_batch=1,
                 max_q_per_req=16, max_q_tokens=None, num_splits=0, kernel="auto",
                 workspace=None):
        import torch
        dt = {"bf16": VA_BF16, "fp32": VA_FP32}
        kern = {"auto": VA_KERNEL_AUTO, "simple": VA_KERNEL_SIMPLE, "mfma": VA_KERNEL_MFMA}
        self.cfg = make_config(num_heads, dt[in_dtype], dt[out_dtype], max_batch, max_q_per_req,
                               max_q_tokens, num_splits, kern[kernel])
        self.workspace = workspace
        if workspace == "torch":
            nbytes = verify_attn_workspace_bytes(self.cfg)
            if nbytes == 0:
                self.ctx = None
                _check(VA_ERR_INVALID)
            self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
            base = self.workspace.data_ptr()
            self.cfg.workspace = (base + 255) & ~255
            self.cfg.workspace_bytes = nbytes
        self.ctx = verify_attn_create(self.cfg)
        self.info = verify_attn_get_info(self.ctx)
        self.num_heads = num_heads
        self.in_dtype = in_dtype
        self.out_dtype = out_dtype

    def run(self, q, kv_buffer, kv_indices, kv_indptr, qo_indptr, custom_mask, mask_indptr,
            sm_scale, out, out_lse=None, out_argmax=None, bs=None, num_tokens=None, stream=None,
            out_cache_loc=None, check=True):
        """One verify step. With check=False the tensor layout checks (validate_run) are
        skipped: for callers that reuse buffers already checked once, since the checks cost
        tens of microseconds of host time per call."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        if bs is None:
            bs = kv_indptr.numel() - 1
        if num_tokens is None:
            num_tokens = q.shape[0]
        if check:
            validate_run(self.num_heads, self.in_dtype, self.out_dtype, q, kv_buffer, kv_indices,
                         kv_indptr, qo_indptr, custom_mask, mask_indptr, out, out_lse,
                         out_argmax, int(bs), int(num_tokens), out_cache_loc)
        verify_attn_run(self.ctx, _ptr(q), _ptr(kv_buffer), kv_buffer.shape[0], _ptr(kv_indices),
                        kv_indices.numel(), _ptr(kv_indptr), _ptr(qo_indptr), _ptr(custom_mask),
                        custom_mask.numel(), _ptr(mask_indptr), _ptr(out_cache_loc), int(bs),
                        int(num_tokens),
                        float(sm_scale), _ptr(out), _ptr(out_lse), _ptr(out_argmax), stream)
        return out

    def build_mask(self, parents, qo_indptr, kv_indptr, custom_mask, mask_indptr,
                   split_layout=False, write_mask_indptr=True, bs=None, num_tokens=None,
                   stream=None, check=True):
        """Builds the verify mask from the tree parents into `custom_mask` (and, by default,
        writes `mask_indptr`)."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        if bs is None:
            bs = qo_indptr.numel() - 1
        if num_tokens is None:
            num_tokens = parents.numel()
        if check:
            validate_tree_args(parents, qo_indptr, kv_indptr, int(bs), int(num_tokens),
                               custom_mask=custom_mask, mask_indptr=mask_indptr)
        verify_attn_build_mask(self.ctx, _ptr(parents), _ptr(qo_indptr), _ptr(kv_indptr),
                               int(bool(split_layout)), int(bs), int(num_tokens),
                               _ptr(custom_mask), custom_mask.numel(), _ptr(mask_indptr),
                               int(bool(write_mask_indptr)), stream)
        return custom_mask

    def accept(self, parents, draft_tokens, target_tokens, qo_indptr, accept_len, accept_path,
               next_token, bs=None, num_tokens=None, stream=None, check=True):
        """Greedy acceptance: fills accept_len [bs], accept_path [bs, max_path] and
        next_token [bs]."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        if bs is None:
            bs = qo_indptr.numel() - 1
        if num_tokens is None:
            num_tokens = parents.numel()
        if check:
            validate_tree_args(parents, qo_indptr, None, int(bs), int(num_tokens),
                               draft_tokens=draft_tokens, target_tokens=target_tokens,
                               accept_len=accept_len, accept_path=accept_path,
                               next_token=next_token)
        verify_attn_accept(self.ctx, _ptr(parents), _ptr(draft_tokens), _ptr(target_tokens),
                           _ptr(qo_indptr), int(bs), int(num_tokens), _ptr(accept_len),
                           _ptr(accept_path), int(accept_path.shape[1]), _ptr(next_token),
                           stream)

    def read_device_status(self, stream=None) -> int:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return verify_attn_read_device_status(self.ctx, stream)

    def close(self):
        if getattr(self, "ctx", None):
            verify_attn_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
