"""The C-ABI library on the host: it loads, exports every function include/verify_attn.h
declares, its structs match the binding, and host-side validation returns the documented
status codes (no GPU work is launched here)."""
import ctypes
import os
import re
import subprocess

import pytest

from mla_tree_verify_paged_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verify_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(verify_attn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing


def test_struct_layout_matches_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "verify_attn.h"\n'
        "int main(void){\n"
        'printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(verify_attn_config),'
        " offsetof(verify_attn_config, max_q_tokens), offsetof(verify_attn_config, num_splits),"
        " offsetof(verify_attn_config, workspace), offsetof(verify_attn_config, workspace_bytes),"
        " sizeof(verify_attn_info));\nreturn 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(prog), "-o",
                    str(exe)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                       check=True).stdout.split()))
    C = B.verify_attn_config
    assert got == [ctypes.sizeof(C), C.max_q_tokens.offset, C.num_splits.offset,
                   C.workspace.offset, C.workspace_bytes.offset,
                   ctypes.sizeof(B.verify_attn_info)]


def test_header_compiles_as_c_and_cxx(tmp_path):
    for comp, ext in (("gcc", "c"), ("g++", "cpp")):
        src = tmp_path / f"inc.{ext}"
        src.write_text('#include "verify_attn.h"\nint main(void){return VA_OK;}\n')
        subprocess.run([comp, "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                        "-o", str(tmp_path / f"inc_{ext}")], check=True)


def cfg(**kw):
    base = dict(num_heads=64, max_batch=1, max_q_per_req=16)
    base.update(kw)
    return B.make_config(**base)


def test_workspace_bytes_positive_and_monotone_in_splits():
    a = B.verify_attn_workspace_bytes(cfg(num_splits=4))
    b = B.verify_attn_workspace_bytes(cfg(num_splits=8))
    assert 0 < a < b
    # S * R partial rows of 512 int16 codes, 4 scales and 3 scalars, R = 16 * 64 rows
    assert b >= 8 * 1024 * (512 * 2 + 7 * 4)


def _align256(x):
    return (x + 255) // 256 * 256


def _layout_bytes(part_rows, rows, elem_bytes):
    """The workspace layout the header documents: header, part_o (elem_bytes per dim),
    part_scale (4 floats per partial row), lse, max, arg, row_info."""
    o = _align256(256 + 1152)
    o = _align256(o + part_rows * 512 * elem_bytes)
    o = _align256(o + part_rows * 4 * 4)
    for _ in range(3):
        o = _align256(o + part_rows * 4)
    return _align256(o + rows * 16)


def test_workspace_size_follows_the_documented_layout():
    rows = 16 * 64
    # MFMA kernel, splits chosen on the device: 128 rows per item, one item per compute unit
    # (256 when no device answers, as in this container), plus one row per output row
    auto = B.verify_attn_workspace_bytes(cfg(kernel=B.VA_KERNEL_MFMA))
    assert auto == _layout_bytes(128 * 256 + rows, rows, 2)
    # a fixed split count: that many partial rows per output row
    assert B.verify_attn_workspace_bytes(cfg(kernel=B.VA_KERNEL_MFMA, num_splits=5)) == \
        _layout_bytes(5 * rows, rows, 2)
    assert B.verify_attn_workspace_bytes(cfg(kernel=B.VA_KERNEL_SIMPLE, num_splits=3)) == \
        _layout_bytes(3 * rows, rows, 4)


@pytest.mark.parametrize("bad", [
    dict(num_heads=0), dict(latent_dim=256), dict(rope_dim=0), dict(in_dtype=7),
    dict(out_dtype=3), dict(max_batch=0), dict(max_q_per_req=0), dict(num_splits=-1),
    dict(num_splits=100000), dict(kernel=9), dict(in_dtype=B.VA_FP32, kernel=B.VA_KERNEL_MFMA),
])
def test_invalid_configs_are_rejected(bad):
    c = cfg(**bad)
    assert B.verify_attn_workspace_bytes(c) == 0
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_create(c)
    assert e.value.status in (B.VA_ERR_INVALID, B.VA_ERR_UNSUPPORTED)
    assert B.verify_attn_last_error()


def test_unsupported_dims_report_unsupported():
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_create(cfg(latent_dim=256))
    assert e.value.status == B.VA_ERR_UNSUPPORTED


def test_small_caller_workspace_is_rejected_before_any_device_call():
    c = cfg(num_splits=4)
    need = B.verify_attn_workspace_bytes(c)
    c.workspace = 1 << 20
    c.workspace_bytes = need - 1
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_create(c)
    assert e.value.status == B.VA_ERR_WORKSPACE
    c.workspace = (1 << 20) + 8
    c.workspace_bytes = need
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_create(c)
    assert e.value.status == B.VA_ERR_WORKSPACE


def test_null_arguments():
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_run(None, None, None, 1, None, 0, None, None, None, 0, None, None, 1, 1,
                          1.0, None, None, None, None)
    assert e.value.status == B.VA_ERR_NULL
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_get_info(None)
    assert e.value.status == B.VA_ERR_NULL
    B.verify_attn_destroy(None)  # no-op
    assert B.lib.verify_attn_create(None, None) == B.VA_ERR_NULL


def test_static_entry_rejects_configs_beyond_its_scratch():
    """The allocation-free entry point refuses, before any device work, a config whose
    workspace exceeds its 64 MiB static scratch, and a config that brings a workspace."""
    args = (None, None, 1, None, 0, None, None, None, 0, None, None, 1, 1, 1.0, None, None,
            None, None)
    big = B.make_config(64, max_batch=1, max_q_per_req=16, max_q_tokens=478)
    assert B.verify_attn_workspace_bytes(big) > 64 << 20
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_run_static(big, *args)
    assert e.value.status == B.VA_ERR_WORKSPACE and "static scratch" in B.verify_attn_last_error()
    fits = B.make_config(64, max_batch=1, max_q_per_req=16, max_q_tokens=477)
    assert B.verify_attn_workspace_bytes(fits) <= 64 << 20
    fits.workspace = 1 << 20
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_run_static(fits, *args)
    assert e.value.status == B.VA_ERR_INVALID
    with pytest.raises(B.VerifyAttnError) as e:
        B.verify_attn_run_static(B.make_config(0), *args)
    assert e.value.status == B.VA_ERR_INVALID
