"""The C ABI library loads and exports every function include/spkv.h declares
(no compute calls: runs without a GPU)."""
import ctypes
import os
import re

import pytest

from learned_kv_cache_sp_amd import spkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "spkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spkv_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(spkv.LIB_PATH):
        from learned_kv_cache_sp_amd import build
        build.build()
    return spkv.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(spkv.EXPORTS)


def test_pure_host_helpers(lib):
    assert lib.spkv_version() == 2
    assert lib.spkv_status_str(0) == b"ok"
    assert b"capacity" in lib.spkv_status_str(-4)
    c = spkv.CacheDesc()
    c.batch, c.n_kv, c.head_dim, c.window, c.page_size, c.n_pages, c.max_pages_per_head = 2, 8, 128, 128, 64, 10, 5
    c.dtype = spkv.SPKV_BF16
    sizes = (ctypes.c_size_t * 7)()
    tot = lib.spkv_cache_bytes(ctypes.byref(c), sizes)
    assert sizes[0] == 10 * 64 * 128 * 2 and sizes[3] == 2 * 8 * 5 * 4 and tot == sum(sizes)


def test_argument_errors_before_any_launch(lib):
    # a null cache / descriptor is rejected on the host, with a message
    assert lib.spkv_decode_attn(None, 32, None, 0, None, 1.0, None, None, None, 0, None) == spkv.SPKV_E_INVALID
    assert b"NULL" in lib.spkv_last_error()
    g = spkv.GateDesc()
    g.d_model, g.d_hidden, g.n_kv, g.dtype = 100, 128, 8, spkv.SPKV_BF16
    assert lib.spkv_gate(ctypes.byref(g), None, 1, 100, 0.5, None, None, None, 0, None) == spkv.SPKV_E_UNSUPPORTED
    c = spkv.CacheDesc()
    c.batch, c.n_kv, c.head_dim, c.window, c.page_size = 1, 8, 128, 100, 64
    assert lib.spkv_cache_reset(ctypes.byref(c), None) in (spkv.SPKV_E_UNSUPPORTED, spkv.SPKV_E_INVALID)


def test_build_flags_kernels_with_scratch():
    # the build refuses kernels that spill register arrays to scratch memory
    from learned_kv_cache_sp_amd import build
    remarks = ("x.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 144 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build.scratch_kernels(remarks) == [("kern_b", 144)]
