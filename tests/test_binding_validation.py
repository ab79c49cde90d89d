"""The Python binding refuses tensors whose layout include/verify_attn.h does not allow,
before any pointer reaches the C ABI (CPU tensors here: shape and dtype are checked before
the device, so each case reports its own error)."""
import pytest
import torch

from mla_tree_verify_paged_amd.binding import validate_run, validate_tree_args

H, T, P = 8, 4, 30


def good(**over):
    n = T
    a = dict(
        q=torch.zeros((n, H, 576), dtype=torch.bfloat16),
        kv_buffer=torch.zeros((100, 576), dtype=torch.bfloat16),
        kv_indices=torch.zeros(P + T, dtype=torch.int64),
        kv_indptr=torch.tensor([0, P + T], dtype=torch.int32),
        qo_indptr=torch.tensor([0, T], dtype=torch.int64),
        custom_mask=torch.ones(T * (P + T), dtype=torch.uint8),
        mask_indptr=torch.tensor([0, T * (P + T)], dtype=torch.int64),
        out=torch.zeros((n, H, 512), dtype=torch.float32),
        out_lse=torch.zeros((n, H), dtype=torch.float32),
        out_argmax=torch.zeros((n, H), dtype=torch.int32),
    )
    a.update(over)
    return a


def call(device_check=False, in_dtype="bf16", out_dtype="fp32", bs=1, num_tokens=T, **kw):
    a = good(**kw)
    validate_run(H, in_dtype, out_dtype, a["q"], a["kv_buffer"], a["kv_indices"], a["kv_indptr"],
                 a["qo_indptr"], a["custom_mask"], a["mask_indptr"], a["out"], a["out_lse"],
                 a["out_argmax"], bs, num_tokens, device_check=device_check)


def test_good_layout_passes_shape_checks():
    call()
    call(out_lse=None, out_argmax=None)
    call(custom_mask=torch.ones(T * (P + T), dtype=torch.bool))


def test_cpu_tensors_are_refused():
    with pytest.raises(ValueError, match="GPU"):
        call(device_check=True)


@pytest.mark.parametrize("over,msg", [
    (dict(q=torch.zeros((T, H, 576), dtype=torch.float32)), "q has dtype"),
    (dict(q=torch.zeros((T, H + 1, 576), dtype=torch.bfloat16)), "q dim 1"),
    (dict(q=torch.zeros((T - 1, H, 576), dtype=torch.bfloat16)), "q holds"),
    (dict(kv_buffer=torch.zeros((100, 512), dtype=torch.bfloat16)), "kv_buffer dim 1"),
    (dict(kv_buffer=torch.zeros((100, 576), dtype=torch.float32)), "kv_buffer has dtype"),
    (dict(kv_indices=torch.zeros(P + T, dtype=torch.int32)), "kv_indices has dtype"),
    (dict(kv_indptr=torch.tensor([0, P + T], dtype=torch.int64)), "kv_indptr has dtype"),
    (dict(qo_indptr=torch.tensor([0, T], dtype=torch.int32)), "qo_indptr has dtype"),
    (dict(mask_indptr=torch.tensor([0], dtype=torch.int64)), "mask_indptr holds"),
    (dict(custom_mask=torch.ones(4, dtype=torch.int32)), "custom_mask has dtype"),
    (dict(out=torch.zeros((T, H, 512), dtype=torch.bfloat16)), "out has dtype"),
    (dict(out=torch.zeros((T, H, 576), dtype=torch.float32)), "out dim 2"),
    (dict(out_lse=torch.zeros((T, H), dtype=torch.float64)), "out_lse has dtype"),
    (dict(out_argmax=torch.zeros((T, H), dtype=torch.int64)), "out_argmax has dtype"),
    (dict(out_argmax=torch.zeros((T, H - 1), dtype=torch.int32)), "out_argmax holds"),
    (dict(q=torch.zeros((H, T, 576), dtype=torch.bfloat16).transpose(0, 1)), "contiguous"),
])
def test_bad_layouts_are_refused(over, msg):
    with pytest.raises(ValueError, match=msg):
        call(**over)


def test_out_dtype_follows_the_context():
    call(out_dtype="bf16", out=torch.zeros((T, H, 512), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out has dtype"):
        call(out_dtype="bf16")


def test_fp32_inputs_need_fp32_tensors():
    call(in_dtype="fp32", q=torch.zeros((T, H, 576)), kv_buffer=torch.zeros((100, 576)))
    with pytest.raises(ValueError, match="q has dtype"):
        call(in_dtype="fp32")


def test_tree_argument_checks():
    par = torch.tensor([-1, 0, 0, 1], dtype=torch.int64)
    qo = torch.tensor([0, 4], dtype=torch.int64)
    kv = torch.tensor([0, 34], dtype=torch.int32)
    validate_tree_args(par, qo, kv, 1, 4, custom_mask=torch.zeros(136, dtype=torch.uint8),
                       mask_indptr=torch.zeros(2, dtype=torch.int64), device_check=False)
    with pytest.raises(ValueError, match="parents has dtype"):
        validate_tree_args(par.int(), qo, kv, 1, 4, device_check=False)
    with pytest.raises(ValueError, match="accept_path"):
        validate_tree_args(par, qo, None, 1, 4, accept_path=torch.zeros(4, dtype=torch.int64),
                           device_check=False)
