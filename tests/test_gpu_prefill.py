"""GPU parity of spkv_prefill_attn (chunked prefill, Eq. 3-4) against the oracle.

Schedule per chunk: gate -> append(GLOBAL) -> prefill_attn -> append(WINDOW).
Chunked prefill must give the rows of one-shot prefill (Eq. 4 is per token).
"""
import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW


def prefill_chunks(wl, Q, K, V, z, chunk, page=64):
    T = Q.shape[0]
    cache = tl.new_cache(wl, 1, T, page_size=page)
    dt = cache.dtype
    outs, lses = [], []
    scale = tl.scale_for(wl.head_dim)
    for p0 in range(0, T, chunk):
        sl = slice(p0, min(T, p0 + chunk))
        tl.append(cache, [z[sl]], [K[sl]], [V[sl]], [p0], G_)
        o, l = spkv.spkv_prefill_attn(cache, 0, tl.dev(Q[sl], dt), tl.dev(K[sl], dt), tl.dev(V[sl], dt), p0, scale)
        tl.append(cache, None, [K[sl]], [V[sl]], [p0], W_)
        outs.append(o.cpu().numpy())
        lses.append(l.cpu().numpy())
    assert spkv.spkv_cache_check(cache) == 0
    return np.concatenate(outs), np.concatenate(lses), cache


@pytest.mark.parametrize("chunk", [1024, 256, 300])
def test_prefill_tiny_f32(chunk):
    wl = inputs.WORKLOADS["tiny"]
    T = 1024
    tok = inputs.tokens(wl, T, 50, 0)
    z = inputs.bernoulli_mask(T, [0.25, 0.25], 50, 0)
    out, lse, _ = prefill_chunks(wl, tok["Q"], tok["K"], tok["V"], z, chunk)
    ro, rl = oracle.attention(tok["Q"], np.arange(T), tok["K"], tok["V"], z, wl.window, threads=tl.oracle_threads())
    print(f"[prefill tiny chunk={chunk}] max|dout|={tl.max_abs(out, ro):.2e} max|dlse|={tl.max_abs(lse, rl):.2e}")
    assert tl.max_abs(out, ro) <= tl.TOL_F32 and tl.max_abs(lse, rl) <= tl.TOL_F32


@pytest.mark.parametrize("T,chunk,rates", [(700, 300, [0.3] * 8), (1000, 1000, [0.0, 1.0, 0.1, 0.3, 0.3, 0.3, 0.5, 0.9]),
                                           (600, 129, [0.3] * 8)])
def test_prefill_bf16_8b_shape(T, chunk, rates):
    wl = inputs.WORKLOADS["prefill_64k"]
    tok = inputs.tokens(wl, T, 51, 0)
    z = inputs.bernoulli_mask(T, rates, 51, 0)
    out, lse, _ = prefill_chunks(wl, tok["Q"], tok["K"], tok["V"], z, chunk)
    rows = np.arange(T)
    ro, rl = oracle.attention(tok["Q"], rows, tok["K"], tok["V"], z, wl.window, threads=tl.oracle_threads())
    print(f"[prefill bf16 T={T} chunk={chunk}] max|dout|={tl.max_abs(out, ro):.2e} max|dlse|={tl.max_abs(lse, rl):.2e}")
    assert tl.max_abs(out, ro) <= tl.TOL_PREFILL and tl.max_abs(lse, rl) <= tl.TOL_REGRESS


@pytest.mark.parametrize("window,hd,n_q,page", [(32, 128, 32, 64), (96, 128, 32, 32), (256, 64, 16, 128)])
def test_prefill_bf16_windows(window, hd, n_q, page):
    # the ring (s < pos0) and the chunk's own rows as window keys for rings of
    # one, three and eight 32-slot blocks, chunks shorter and longer than w
    import dataclasses
    wl = dataclasses.replace(inputs.WORKLOADS["prefill_64k"], window=window, head_dim=hd, n_q=n_q)
    T = 900
    tok = inputs.tokens(wl, T, 55, 0)
    z = inputs.bernoulli_mask(T, [0.5, 0.3, 0.9, 0.3, 0.1, 0.3, 0.7, 1.0], 55, 0)
    out, lse, _ = prefill_chunks(wl, tok["Q"], tok["K"], tok["V"], z, 70 if window >= 96 else 300, page=page)
    ro, rl = oracle.attention(tok["Q"], np.arange(T), tok["K"], tok["V"], z, wl.window, threads=tl.oracle_threads())
    print(f"[prefill w={window} hd={hd}] max|dout|={tl.max_abs(out, ro):.2e} max|dlse|={tl.max_abs(lse, rl):.2e}")
    assert tl.max_abs(out, ro) <= tl.TOL_PREFILL and tl.max_abs(lse, rl) <= tl.TOL_REGRESS


@pytest.mark.parametrize("page", [32, 128, 256])
def test_prefill_bf16_page_sizes(page):
    # pages smaller than a 64-key block take the per-lane address path of the
    # direct loads, larger ones the page-based one with blocks inside a page
    wl = inputs.WORKLOADS["prefill_64k"]
    T = 1100
    tok = inputs.tokens(wl, T, 54, 0)
    z = inputs.bernoulli_mask(T, [0.5, 0.3, 0.9, 0.3, 0.1, 0.3, 0.7, 1.0], 54, 0)
    out, lse, _ = prefill_chunks(wl, tok["Q"], tok["K"], tok["V"], z, 500, page=page)
    ro, rl = oracle.attention(tok["Q"], np.arange(T), tok["K"], tok["V"], z, wl.window, threads=tl.oracle_threads())
    print(f"[prefill bf16 page={page}] max|dout|={tl.max_abs(out, ro):.2e} max|dlse|={tl.max_abs(lse, rl):.2e}")
    assert tl.max_abs(out, ro) <= tl.TOL_PREFILL and tl.max_abs(lse, rl) <= tl.TOL_REGRESS


def test_prefill_chunked_equals_one_shot():
    wl = inputs.WORKLOADS["prefill_64k"]
    T = 900
    tok = inputs.tokens(wl, T, 52, 0)
    z = inputs.bernoulli_mask(T, [0.3] * 8, 52, 0)
    o1, l1, c1 = prefill_chunks(wl, tok["Q"], tok["K"], tok["V"], z, T)
    o2, l2, c2 = prefill_chunks(wl, tok["Q"], tok["K"], tok["V"], z, 200)
    assert tl.max_abs(o1, o2) <= 1e-5 and tl.max_abs(l1, l2) <= 1e-5
    for g in range(wl.n_kv):
        for x, y in zip(c1.read_head(0, g), c2.read_head(0, g)):
            assert torch.equal(x, y)


def test_prefill_zero_keys_counts_visible_set():
    wl = inputs.WORKLOADS["prefill_64k"]
    T = 800
    tok = inputs.tokens(wl, T, 53, 0)
    tok["K"][:] = 0
    z = inputs.bernoulli_mask(T, [0.05, 0.1, 0.2, 0.3, 0.4, 0.5, 0.7, 1.0], 53, 0)
    out, lse, _ = prefill_chunks(wl, tok["Q"], tok["K"], tok["V"], z, 300)
    for g in range(wl.n_kv):
        n = oracle.visible_count(z[:, g], np.arange(T), wl.window)
        for h in range(g * wl.group, (g + 1) * wl.group):
            assert np.all(np.abs(lse[:, h] - np.log(n)) <= 2e-6 * np.maximum(1.0, np.log(n)))


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("n_q, n_kv", [(8, 8), (16, 1), (32, 2), (48, 3), (64, 16), (256, 16)])
def test_prefill_bf16_head_shapes(n_q, n_kv, hd):
    # group sizes 1, 4 and 16, a key-head count (3) that does not divide 8,
    # the widest query count, both head sizes; two chunks with a ragged tail
    wl = tl.small_workload("prefill_64k", n_q=n_q, n_kv=n_kv, head_dim=hd, window=64)
    T = 333 if n_q >= 64 else 530
    seed = 55 + n_q + n_kv + hd
    tok = inputs.tokens(wl, T, seed, 0)
    rates = [0.1 + 0.8 * g / max(1, n_kv - 1) for g in range(n_kv)]
    z = inputs.bernoulli_mask(T, rates, seed, 0)
    out, lse, _ = prefill_chunks(wl, tok["Q"], tok["K"], tok["V"], z, 200)
    ro, rl = oracle.attention(tok["Q"], np.arange(T), tok["K"], tok["V"], z, wl.window, threads=tl.oracle_threads())
    print(f"[prefill bf16 n_q={n_q} n_kv={n_kv} hd={hd}] max|dout|={tl.max_abs(out, ro):.2e} "
          f"max|dlse|={tl.max_abs(lse, rl):.2e}")
    assert tl.max_abs(out, ro) <= tl.TOL_PREFILL and tl.max_abs(lse, rl) <= tl.TOL_REGRESS
