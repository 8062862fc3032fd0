"""spkv_decode_attn_noalloc (built-in scratch, no workspace argument) against
spkv_decode_attn on the same inputs: two calls in a row, the second on a
smaller cache, both bit-identical to the workspace entry point (the same
kernel and split run on both); a cache too large for the scratch is refused
before any launch."""
import numpy as np
import pytest
import torch

from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW


def _cache_and_query(wl, prefix, rates, seed):
    B = len(prefix)
    data = []
    for b in range(B):
        tok = inputs.tokens(wl, prefix[b] + 1, seed, b)
        z = inputs.bernoulli_mask(prefix[b] + 1, rates, seed, b)
        data.append((tok["Q"], tok["K"], tok["V"], z))
    cache = tl.new_cache(wl, B, max(prefix) + 1)
    t = list(prefix)
    rows = lambda i: [d[i][:t[b] + 1] for b, d in enumerate(data)]  # noqa: E731
    tl.append(cache, rows(3), rows(1), rows(2), [0] * B, G_ | W_)
    q = tl.dev(np.stack([data[b][0][t[b]] for b in range(B)]), cache.dtype)
    return cache, q, tl.dev(np.array(t, np.int32))


def _compare(cache, q, t, scale):
    ws = spkv.workspace(spkv.spkv_decode_ws_bytes(cache, q.shape[1]))
    o_ref, l_ref = spkv.spkv_decode_attn(cache, q, t, scale, ws=ws)
    o, l = spkv.spkv_decode_attn_noalloc(cache, q, t, scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(l, l_ref)
    assert spkv.spkv_cache_check(cache) == 0
    return o


def test_noalloc_matches_workspace_entry_point_twice():
    wl = tl.small_workload("decode_32k", batch=6)
    cache, q, t = _cache_and_query(wl, [3000, 2100, 4500, 700, 3900, 2600], wl.keep, 3101)
    o1 = _compare(cache, q, t, tl.scale_for(wl.head_dim))
    # second call, smaller input: fewer sequences, shorter contexts, another head size
    wl2 = tl.small_workload("decode_32k", batch=2, head_dim=64, n_q=16)
    cache2, q2, t2 = _cache_and_query(wl2, [900, 300], wl2.keep, 3102)
    o2 = _compare(cache2, q2, t2, tl.scale_for(64))
    assert o1.shape != o2.shape
    # and the first cache again after the smaller one (the scratch keeps no stale state)
    _compare(cache, q, t, tl.scale_for(wl.head_dim))


def test_noalloc_refuses_a_cache_beyond_the_scratch():
    # batch * n_kv = 2048 with G = 16: the partials alone need > 4 MiB
    cache = spkv.Cache(256, 8, 128, 32, 32, 8, 1, torch.bfloat16)
    q = torch.zeros((256, 128, 128), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(spkv.SpkvError) as e:
        spkv.spkv_decode_attn_noalloc(cache, q, t, 0.1)
    assert e.value.code == spkv.SPKV_E_WORKSPACE
