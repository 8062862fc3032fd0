"""The binding refuses mis-shaped tensors before anything reaches the library.

The decode and prefill kernels read and write every sequence of the cache
(decode) or every row of the chunk (prefill); a tensor with fewer rows or a
wrong inner shape would make them read or write past its end.  These checks
run on the host (CPU tensors), so no GPU is needed."""
import os

import pytest
import torch

from learned_kv_cache_sp_amd import spkv


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(spkv.LIB_PATH):
        from learned_kv_cache_sp_amd import build
        build.build()
    return spkv.load_library()


B, NKV, HD, NQ, D = 3, 2, 64, 8, 128


def cache():
    return spkv.Cache(B, NKV, HD, 64, 32, 16, 4, torch.bfloat16, device="cpu")


def gate():
    return spkv.GateWeights(torch.zeros(32, D, dtype=torch.bfloat16), torch.zeros(32), torch.zeros(NKV, 32),
                            torch.zeros(NKV))


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


@pytest.mark.parametrize("q, t, msg", [
    (bf(B - 1, NQ, HD), i32(B), "q has shape"),          # fewer sequences than the cache
    (bf(B, NQ, HD // 2), i32(B), "q has shape"),         # wrong head_dim
    (bf(B, NQ + 1, HD), i32(B), "not a multiple"),       # n_q not a multiple of n_kv
    (bf(B, NQ, HD), i32(B - 1), "t has shape"),          # short t
    (torch.zeros(B, NQ, HD), i32(B), "dtype"),           # q in f32 for a bf16 cache
    (bf(B, NQ, HD), torch.zeros(B, dtype=torch.int64), "dtype"),
])
def test_decode_attn_rejects(q, t, msg):
    with pytest.raises(ValueError, match=msg):
        spkv.spkv_decode_attn(cache(), q, t, 0.125)


def test_decode_attn_rejects_small_outputs():
    q, t = bf(B, NQ, HD), i32(B)
    with pytest.raises(ValueError, match="out has shape"):
        spkv.spkv_decode_attn(cache(), q, t, 0.125, out=torch.zeros(B - 1, NQ, HD))
    with pytest.raises(ValueError, match="lse has shape"):
        spkv.spkv_decode_attn(cache(), q, t, 0.125, lse=torch.zeros(B, NQ - 1))
    with pytest.raises(ValueError, match="out must be contiguous"):
        spkv.spkv_decode_attn(cache(), q, t, 0.125, out=torch.zeros(B, HD, NQ).transpose(1, 2))


def test_decode_step_rejects():
    c, g = cache(), gate()
    q, t = bf(B, NQ, HD), i32(B)
    k, v, h = bf(B, NKV, HD), bf(B, NKV, HD), bf(B, D)
    with pytest.raises(ValueError, match="k has shape"):
        spkv.spkv_decode_step(c, g, h, 0.5, bf(B - 1, NKV, HD), v, q, t, 0.125)
    with pytest.raises(ValueError, match="v has shape"):
        spkv.spkv_decode_step(c, g, h, 0.5, k, bf(B, NKV, HD // 2), q, t, 0.125)
    with pytest.raises(ValueError, match="hidden has shape"):
        spkv.spkv_decode_step(c, g, bf(B - 1, D), 0.5, k, v, q, t, 0.125)
    with pytest.raises(ValueError, match="keep has shape"):
        spkv.spkv_decode_step(c, g, h, 0.5, k, v, q, t, 0.125, keep=torch.zeros(B, 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="utility has shape"):
        spkv.spkv_decode_step(c, g, h, 0.5, k, v, q, t, 0.125, utility=torch.zeros(B - 1, NKV))
    with pytest.raises(ValueError, match="q has shape"):
        spkv.spkv_decode_step(c, None, None, 0.5, k, v, bf(B + 1, NQ, HD), t, 0.125)
    g3 = spkv.GateWeights(g.w1, g.b1, torch.zeros(NKV + 1, 32), torch.zeros(NKV + 1))
    with pytest.raises(ValueError, match="outputs"):
        spkv.spkv_decode_step(c, g3, h, 0.5, k, v, q, t, 0.125)


def test_prefill_rejects():
    c = cache()
    n = 40
    q, k, v = bf(n, NQ, HD), bf(n, NKV, HD), bf(n, NKV, HD)
    with pytest.raises(ValueError, match="k has shape"):
        spkv.spkv_prefill_attn(c, 0, q, bf(n - 1, NKV, HD), v, 0, 0.125)
    with pytest.raises(ValueError, match="v has shape"):
        spkv.spkv_prefill_attn(c, 0, q, k, bf(n, NKV + 1, HD), 0, 0.125)
    with pytest.raises(ValueError, match="outside"):
        spkv.spkv_prefill_attn(c, B, q, k, v, 0, 0.125)
    with pytest.raises(ValueError, match="out has shape"):
        spkv.spkv_prefill_attn(c, 0, q, k, v, 0, 0.125, out=torch.zeros(n - 1, NQ, HD))
    with pytest.raises(ValueError, match="lse has shape"):
        spkv.spkv_prefill_attn(c, 0, q, k, v, 0, 0.125, lse=torch.zeros(n))


def test_well_shaped_cpu_tensors_reach_the_device_check():
    # with every shape right, the only complaint left is that the tensors are not on the GPU
    with pytest.raises(ValueError, match="device tensors"):
        spkv.spkv_decode_attn(cache(), bf(B, NQ, HD), i32(B), 0.125)


def test_hbm_read_refuses_bad_arguments():
    # argument checks happen on the host before any launch
    lib = spkv.load_library()
    fake = 1 << 40
    assert lib.spkv_hbm_read(fake, 1000, 0, 256, fake, None) == spkv.SPKV_E_INVALID      # not 16 KB multiple
    assert lib.spkv_hbm_read(fake + 8, 16384, 0, 256, fake, None) == spkv.SPKV_E_INVALID  # misaligned
    assert lib.spkv_hbm_read(fake, 16384, 4, 256, fake, None) == spkv.SPKV_E_INVALID      # unknown flag
    assert lib.spkv_hbm_read(fake, 16384, 0, 0, fake, None) == spkv.SPKV_E_INVALID        # empty grid
    assert lib.spkv_hbm_read(None, 16384, 0, 256, fake, None) == spkv.SPKV_E_INVALID
    assert lib.spkv_hbm_read(fake, 0, 0, 256, fake, None) == spkv.SPKV_OK                 # nothing to read


def test_guard_canaries_detect_a_stray_write():
    # host-side check of the canary mechanism on a CPU cache: a byte written
    # just past a buffer (into its padding or its trailing guard) is reported
    c = spkv.Cache(1, 2, 64, 32, 32, 4, 2, torch.bfloat16, device="cpu", guard=256)
    assert c.check_guards() == []
    name, raw, g, n = c._guards[3]          # the page table
    assert name == "page_table"
    raw[g + n] = 0
    assert c.check_guards() == ["page_table"]
    raw[g + n] = spkv.Cache.GUARD_BYTE
    raw[g - 1] = 1                           # the byte just before the buffer
    assert c.check_guards() == ["page_table"]
    raw[g - 1] = spkv.Cache.GUARD_BYTE
    c.k_pages.fill_(3.0)                     # writes inside the buffer are fine
    assert c.check_guards() == []
    assert bool((c.page_table == -1).all())
