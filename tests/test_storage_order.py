"""Storage order of cached keys and values (CPU only).

The header documents where the key and value of slot r, dimension d, sit
inside a 32-slot block; the binding's read-back (Cache.read_head /
read_ring) undoes that order.  These tests build the stored order element by
element from the header's formula and check that the read-back recovers the
logical [slots, head_dim] arrays, and that the formula is a permutation.
"""
import numpy as np
import pytest
import torch

from learned_kv_cache_sp_amd import spkv


def header_row(r: int) -> int:
    # row(r) = 16 * ((r / 4) % 2) + 4 * (r / 8) + r % 4   (integer division)
    return 16 * ((r // 4) % 2) + 4 * (r // 8) + r % 4


def header_key_offset(slot: int, d: int, hd: int) -> int:
    blk, r = divmod(slot, 32)
    return blk * 32 * hd + (d // 32) * 1024 + header_row(r) * 32 + d % 32


def header_value_offset(slot: int, d: int, hd: int) -> int:
    blk, r = divmod(slot, 32)
    return blk * 32 * hd + d * 32 + r


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("n", [32, 64, 256])
def test_formula_is_a_permutation(hd, n):
    ko = sorted(header_key_offset(s, d, hd) for s in range(n) for d in range(hd))
    vo = sorted(header_value_offset(s, d, hd) for s in range(n) for d in range(hd))
    assert ko == list(range(n * hd)) and vo == list(range(n * hd))


def test_decode_tiles_are_contiguous_runs():
    # rows 16t .. 16t+15 of dims 32cc .. 32cc+31 (one MFMA operand tile of the
    # decode step) are one contiguous 1 KB run at bf16
    hd = 128
    for t in range(2):
        for cc in range(hd // 32):
            offs = sorted(header_key_offset(s, d, hd) for s in range(32) for d in range(32 * cc, 32 * cc + 32)
                          if 16 * t <= header_row(s) < 16 * t + 16)
            assert offs == list(range(offs[0], offs[0] + 512)) and offs[0] % 512 == 0
    # a value tile: 16 dimensions x 32 slots
    for nt in range(hd // 16):
        offs = sorted(header_value_offset(s, d, hd) for s in range(32) for d in range(16 * nt, 16 * nt + 16))
        assert offs == list(range(offs[0], offs[0] + 512))


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_read_back_inverts_the_header_order(hd, dtype):
    rng = np.random.default_rng(7 + hd)
    n = 96
    logical_k = torch.from_numpy(rng.standard_normal((n, hd)).astype(np.float32)).to(dtype)
    logical_v = torch.from_numpy(rng.standard_normal((n, hd)).astype(np.float32)).to(dtype)
    ko = torch.tensor([[header_key_offset(s, d, hd) for d in range(hd)] for s in range(n)]).reshape(-1)
    vo = torch.tensor([[header_value_offset(s, d, hd) for d in range(hd)] for s in range(n)]).reshape(-1)
    stored_k = torch.empty(n * hd, dtype=dtype)
    stored_v = torch.empty(n * hd, dtype=dtype)
    stored_k[ko] = logical_k.reshape(-1)
    stored_v[vo] = logical_v.reshape(-1)
    # the read-back takes the stored elements as an [n, hd] view
    assert torch.equal(spkv.unblock_keys(stored_k.reshape(n, hd)), logical_k)
    assert torch.equal(spkv.unblock_values(stored_v.reshape(n, hd)), logical_v)
