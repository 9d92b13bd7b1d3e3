"""The C-ABI library on a machine without a GPU: it loads, exports what the header declares, and rejects bad
arguments on the host before touching the device (no compute call is made here)."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def _lib():
    import paged_kv_cache_300_amd as pkv
    if not os.path.exists(pkv.library_path()):
        pytest.skip("libpagedkv.so not built (run __graft_entry__.build())")
    return pkv, pkv.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for fn in ("kv_slot_mapping", "kv_store", "kv_store_qk_norm_rope", "attn_prefill_varlen",
               "attn_prefill_workspace_bytes",
               "attn_decode_paged", "attn_decode_paged_store", "attn_decode_workspace_bytes", "pkv_last_error"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    _, L = _lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def _err(L):
    return L.pkv_last_error().decode()


def test_store_rejects_bad_arguments_on_host():
    pkv, L = _lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
    # num_kv_heads = 0
    assert L.kv_store(fake, 8, fake, 8, fake, fake, 16, fake, 4, 0, 8, pkv.PKV_BF16, None) == -1
    assert "num_kv_heads" in _err(L)
    # key stride shorter than a row
    assert L.kv_store(fake, 4, fake, 8, fake, fake, 16, fake, 4, 1, 8, pkv.PKV_BF16, None) == -1
    assert "stride" in _err(L)
    # unknown dtype
    assert L.kv_store(fake, 8, fake, 8, fake, fake, 16, fake, 4, 1, 8, 7, None) == -1
    # null pointers with tokens to copy
    assert L.kv_store(None, 8, fake, 8, fake, fake, 16, fake, 4, 1, 8, pkv.PKV_F32, None) == -1
    # nothing to do is fine and launches nothing
    assert L.kv_store(None, 8, None, 8, None, None, 0, None, 0, 1, 8, pkv.PKV_F32, None) == 0
    assert _err(L) == ""


def test_qk_norm_rope_store_rejects_bad_arguments_on_host():
    pkv, L = _lib()
    fake = ctypes.c_void_p(0x1000)
    args = lambda hd, eps, theta, qs: (fake, qs, fake, 8 * hd, fake, 8 * hd, fake, fake, fake, eps, theta, fake, fake,
                                       fake, 4096, fake, 4, 16, 8, hd, pkv.PKV_BF16, None)
    assert L.kv_store_qk_norm_rope(*args(96, 1e-6, 1e6, 16 * 96)) == -2          # head_dim not a power of two
    assert L.kv_store_qk_norm_rope(*args(128, -1.0, 1e6, 16 * 128)) == -1        # negative eps
    assert L.kv_store_qk_norm_rope(*args(128, 1e-6, 0.0, 16 * 128)) == -1        # theta must be > 0
    assert L.kv_store_qk_norm_rope(*args(128, 1e-6, 1e6, 15 * 128)) == -1        # q stride shorter than a row
    assert "stride" in _err(L)


def test_fused_decode_store_rejects_bad_arguments_on_host():
    pkv, L = _lib()
    fake = ctypes.c_void_p(0x1000)
    need = L.attn_decode_workspace_bytes(64, 16, 8, 128, 16, 256, pkv.PKV_BF16)

    def call(ks=1024, vs=1024, knew=fake, ws=need, num_blocks=4096):
        return L.attn_decode_paged_store(fake, 2048, knew, ks, fake, vs, fake, fake, num_blocks, fake, fake, 64, 16,
                                         256, 16, 8, 128, 0.088, fake, None, fake, ws, pkv.PKV_BF16, None)
    assert call(ks=1000) == -1 and "k_new_stride" in _err(L)       # new-row stride shorter than a row
    assert call(vs=0) == -1
    assert call(knew=None) == -1 and "k_new" in _err(L)            # no new rows
    assert call(ws=need - 1) == -3 and "workspace" in _err(L)      # same workspace rule as attn_decode_paged
    assert call(num_blocks=2 ** 23 + 1) == -2                      # slots past int32


def test_slot_mapping_rejects_bad_arguments_on_host():
    pkv, L = _lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.kv_slot_mapping(fake, None, fake, fake, 2, 4, 4, 2, fake, None) == -1  # both modes at once
    assert L.kv_slot_mapping(fake, None, None, fake, 2, 4, 0, 2, fake, None) == -1  # block_size 0
    assert L.kv_slot_mapping(None, None, None, fake, 2, 4, 4, 2, fake, None) == -1  # prefill without cu_q
    assert L.kv_slot_mapping(fake, None, None, fake, 2, 4, 4, 0, None, None) == 0    # zero tokens


def test_attention_rejects_bad_arguments_on_host():
    pkv, L = _lib()
    fake = ctypes.c_void_p(0x1000)
    # Hq not a multiple of Hkv
    rc = L.attn_prefill_varlen(fake, 48, fake, 32, fake, 32, fake, fake, 4, 4, 1, 4, 4, 3, 2, 16, 0.25, 1, None, 0, 0,
                               fake, None, 0, pkv.PKV_F32, None)
    assert rc == -1 and "multiple" in _err(L)
    # head_dim beyond what is implemented
    rc = L.attn_prefill_varlen(fake, 4 * 512, fake, 2 * 512, fake, 2 * 512, fake, fake, 4, 4, 1, 4, 4, 4, 2, 512, 0.25,
                               1, None, 0, 0, fake, None, 0, pkv.PKV_F32, None)
    assert rc == -2
    # causal must be 0/1
    rc = L.attn_prefill_varlen(fake, 64, fake, 32, fake, 32, fake, fake, 4, 4, 1, 4, 4, 4, 2, 16, 0.25, 5, None, 0, 0,
                               fake, None, 0, pkv.PKV_F32, None)
    assert rc == -1
    # paged cache whose slot count is not a multiple of block_size
    rc = L.attn_prefill_varlen(fake, 64, fake, 0, fake, 0, fake, fake, 4, 4, 1, 4, 10, 4, 2, 16, 0.25, 1, fake, 2, 4,
                               fake, None, 0, pkv.PKV_F32, None)
    assert rc == -1
    # prefill: a workspace smaller than the longest-first planner needs
    need_p = L.attn_prefill_workspace_bytes(4, 4, 4, 16, 8, 128, pkv.PKV_BF16)
    assert need_p > 0
    rc = L.attn_prefill_varlen(fake, 2048, fake, 1024, fake, 1024, fake, fake, 4, 4, 4, 4, 4, 16, 8, 128, 0.088, 1,
                               None, 0, 0, fake, fake, need_p - 1, pkv.PKV_BF16, None)
    assert rc == -3 and "workspace" in _err(L)
    # decode: undersized workspace for the split-KV path
    need = L.attn_decode_workspace_bytes(64, 16, 8, 128, 16, 256, pkv.PKV_BF16)
    assert need > 0
    rc = L.attn_decode_paged(fake, 2048, fake, fake, 4096, fake, fake, 64, 16, 256, 16, 8, 128, 0.088, fake, fake,
                             need - 1, pkv.PKV_BF16, None)
    assert rc == -3 and "workspace" in _err(L)
    # non-finite scale
    rc = L.attn_decode_paged(fake, 2048, fake, fake, 4096, fake, fake, 64, 16, 256, 16, 8, 128, float("nan"), fake,
                             fake, need, pkv.PKV_BF16, None)
    assert rc == -1


def test_workspace_size_formula_is_monotone():
    pkv, L = _lib()
    small = L.attn_decode_workspace_bytes(8, 16, 8, 128, 16, 256, pkv.PKV_BF16)
    big = L.attn_decode_workspace_bytes(256, 16, 8, 128, 128, 256, pkv.PKV_BF16)
    assert 0 <= small <= big
    assert L.attn_decode_workspace_bytes(8, 4, 2, 16, 4, 4, pkv.PKV_F32) == 0  # generic path: no workspace
    assert L.attn_prefill_workspace_bytes(8, 100, 50, 4, 2, 16, pkv.PKV_F32) == 0  # generic path: no workspace
    assert L.attn_prefill_workspace_bytes(5000, 9000, 64, 16, 8, 128, pkv.PKV_BF16) == 0  # batch past the planner
    # one count plus one entry per possible query tile: grows with the tokens, bounded by batch * tiles
    a = L.attn_prefill_workspace_bytes(16, 5000, 512, 16, 8, 128, pkv.PKV_BF16)
    b = L.attn_prefill_workspace_bytes(16, 9000, 512, 16, 8, 128, pkv.PKV_BF16)
    assert 0 < a <= b


def test_row_tensor_checks_on_host():
    """Token-row tensors: head_dim contiguous and heads packed; an empty batch passes whatever strides its view
    reports (a zero-row view of a NumPy array reports zeros)."""
    import numpy as np
    import torch
    from paged_kv_cache_300_amd import _lib as L
    empty = torch.from_numpy(np.zeros((0, 8, 128), np.int16)).view(torch.bfloat16)
    assert L._rows(empty, "k", heads=8) == 8 * 128
    with pytest.raises(ValueError):
        L._rows(empty, "k", heads=4)
    full = torch.zeros(5, 8, 128, dtype=torch.bfloat16)
    assert L._rows(full, "k") == 8 * 128
    assert L._rows(torch.zeros(5, 24, 128)[:, 8:16], "k") == 24 * 128  # a view into a merged projection
    with pytest.raises(ValueError):
        L._rows(full.transpose(1, 2), "k")


def test_c_program_uses_the_abi(tmp_path):
    """The header compiles as C11 and a plain C program links the library and gets the documented host-side
    results (workspace sizes, rejected arguments with a message); nothing is enqueued on a GPU."""
    _lib()  # skips when the library is not built
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    here = os.path.dirname(os.path.abspath(__file__))
    pkg = os.path.join(os.path.dirname(here), "paged_kv_cache_300_amd")
    exe = str(tmp_path / "abi_from_c")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [gcc, "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.dirname(HEADER)}", f"-I{rocm}/include",
           os.path.join(here, "c_abi", "abi_from_c.c"), f"-L{pkg}", "-lpagedkv", f"-Wl,-rpath,{pkg}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr


def test_noalloc_decode_refuses_oversized_workspace_on_host():
    """The allocation-free fused decode takes its workspace from a fixed 32 MiB static array: a batch whose
    workspace would not fit is refused with the workspace code before any device call."""
    pkv, L = _lib()
    fake = ctypes.c_void_p(0x1000)  # 16-byte aligned, never dereferenced: the size check comes first
    need = L.attn_decode_workspace_bytes(20000, 16, 8, 128, 16, 256, pkv.PKV_BF16)
    assert need > 32 << 20
    rc = L.attn_decode_paged_store_noalloc(fake, 2048, fake, 1024, fake, 1024, fake, fake, 4096, fake, fake, 20000,
                                           16, 256, 16, 8, 128, ctypes.c_float(0.088), fake, None, pkv.PKV_BF16, None)
    assert rc == -3
    assert "static scratch" in _err(L)
