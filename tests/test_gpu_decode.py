"""GPU parity of spkv_decode_attn (Eq. 3-4) against the fp64 oracle.

The cache is built through spkv_compact_append from keep masks given to both
sides; the oracle evaluates Eq. (3)-(4) directly on the full sequence.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW


def _decode_case(wl, prefix, steps, rates, seed, zero_keys=False, page=64, tol=None):
    """Prefix appended in one call, then `steps` decode steps of one token per sequence."""
    B = len(prefix)
    T = [p + steps for p in prefix]
    data = []
    for b in range(B):
        tok = inputs.tokens(wl, T[b], seed, b)
        if zero_keys:
            tok["K"][:] = 0.0
        z = inputs.bernoulli_mask(T[b], rates, seed, b)
        data.append((tok["Q"], tok["K"], tok["V"], z))
    cache = tl.new_cache(wl, B, max(T), page_size=page)
    dt = cache.dtype
    tl.append(cache, [d[3][:prefix[b]] for b, d in enumerate(data)], [d[1][:prefix[b]] for b, d in enumerate(data)],
              [d[2][:prefix[b]] for b, d in enumerate(data)], [0] * B, G_ | W_)
    ws = spkv.workspace(spkv.spkv_decode_ws_bytes(cache, wl.n_q))
    scale = tl.scale_for(wl.head_dim)
    worst, worst_lse = 0.0, 0.0
    th = tl.oracle_threads()
    for s in range(steps):
        t = [prefix[b] + s for b in range(B)]
        tl.append(cache, [data[b][3][t[b]:t[b] + 1] for b in range(B)], [data[b][1][t[b]:t[b] + 1] for b in range(B)],
                  [data[b][2][t[b]:t[b] + 1] for b in range(B)], t, G_ | W_)
        q = np.stack([data[b][0][t[b]] for b in range(B)])
        out, lse = spkv.spkv_decode_attn(cache, tl.dev(q, dt), tl.dev(np.array(t, np.int32)), scale, ws=ws)
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        for b in range(B):
            Q, K, V, z = data[b]
            ro, rl = oracle.attention(Q[t[b]:t[b] + 1], [t[b]], K, V, z, wl.window, scale, threads=th)
            worst = max(worst, tl.max_abs(out[b], ro[0]))
            worst_lse = max(worst_lse, tl.max_abs(lse[b], rl[0]))
            if zero_keys:
                # K = 0: lse = log |visible(t)| exactly, per key head
                for g in range(wl.n_kv):
                    n = oracle.visible_count(z[:, g], [t[b]], wl.window)[0]
                    assert np.all(np.abs(lse[b, g * wl.group:(g + 1) * wl.group] - np.log(n)) < 2e-6 * max(1.0, np.log(n))), \
                        (b, g, n, lse[b, g * wl.group:(g + 1) * wl.group])
    assert spkv.spkv_cache_check(cache) == 0
    return worst, worst_lse


def test_decode_tiny_f32():
    wl = inputs.WORKLOADS["tiny"]
    worst, wl_lse = _decode_case(wl, [1024], 16, [0.25, 0.25], 31)
    print(f"[decode tiny f32] max|dout|={worst:.2e} max|dlse|={wl_lse:.2e}")
    assert worst <= tl.TOL_F32 and wl_lse <= tl.TOL_F32


@pytest.mark.parametrize("prefix,rates,page", [
    ([3000, 1200], [0.2] * 8, 64),
    ([700, 5000, 129], [0.0, 1.0, 0.02, 0.05, 0.1, 0.2, 0.4, 0.6], 64),   # skewed per-head lengths
    ([2000], [0.3] * 8, 32),
    ([2000, 300], [0.3] * 8, 256),
])
def test_decode_bf16_8b_shape(prefix, rates, page):
    wl = inputs.WORKLOADS["decode_32k"]
    worst, worst_lse = _decode_case(wl, prefix, 3, rates, 32, page=page)
    print(f"[decode bf16 {prefix} p={page}] max|dout|={worst:.2e} max|dlse|={worst_lse:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_lse <= tl.TOL_REGRESS


@pytest.mark.parametrize("prefix", [[0], [5], [126], [127], [128], [129]])
def test_decode_short_context(prefix):
    # rows whose window is not yet full (t < w) and the first rows past it
    wl = inputs.WORKLOADS["decode_32k"]
    worst, worst_lse = _decode_case(wl, prefix, 2, [0.5] * 8, 33)
    assert worst <= tl.TOL_REGRESS and worst_lse <= tl.TOL_REGRESS


@pytest.mark.parametrize("n_q,n_kv,hd", [(8, 8, 128), (16, 8, 128), (64, 8, 128), (32, 2, 128),
                                         (32, 8, 64), (16, 1, 64)])
def test_decode_group_sizes_and_head_dims(n_q, n_kv, hd):
    wl = dataclasses.replace(inputs.WORKLOADS["decode_32k"], n_q=n_q, n_kv=n_kv, head_dim=hd,
                             keep=(0.25,) * n_kv)
    worst, worst_lse = _decode_case(wl, [1000, 2500], 2, [0.25] * n_kv, 34)
    print(f"[decode G={n_q // n_kv} hd={hd}] max|dout|={worst:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_lse <= tl.TOL_REGRESS


@pytest.mark.parametrize("window,hd,n_q", [(32, 128, 32), (96, 128, 32), (256, 128, 32), (96, 64, 16), (32, 64, 16)])
@pytest.mark.parametrize("zero_keys", [False, True])
def test_decode_windows(window, hd, n_q, zero_keys):
    # rings of one, three and eight 32-slot blocks; contexts shorter than the
    # window, within one step of it and far past it; K = 0 pins the visible
    # set exactly (lse = log |visible|)
    wl = dataclasses.replace(inputs.WORKLOADS["decode_32k"], window=window, head_dim=hd, n_q=n_q)
    prefix = [window - 2, window + 1, 3 * window + 17, 1500]
    worst, worst_lse = _decode_case(wl, prefix, 3, [0.0, 1.0, 0.05, 0.2, 0.3, 0.5, 0.7, 0.9], 37,
                                    zero_keys=zero_keys, page=32 if hd == 64 else 64)
    print(f"[decode w={window} hd={hd} zero_keys={zero_keys}] max|dout|={worst:.2e} max|dlse|={worst_lse:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_lse <= tl.TOL_REGRESS


def test_decode_f32_window_96():
    wl = dataclasses.replace(inputs.WORKLOADS["tiny"], window=96)
    worst, wl_lse = _decode_case(wl, [94, 300], 4, [0.25, 0.6], 38)
    assert worst <= tl.TOL_F32 and wl_lse <= tl.TOL_F32


def test_decode_zero_keys_counts_visible_set():
    # K = 0 (exact in bf16): softmax is uniform over the visible set, so
    # lse = log |visible| pins key-set membership exactly
    wl = inputs.WORKLOADS["decode_32k"]
    worst, _ = _decode_case(wl, [4000, 333], 3, [0.02, 0.05, 0.1, 0.2, 0.3, 0.5, 0.8, 1.0], 35, zero_keys=True)
    assert worst <= tl.TOL_REGRESS


def test_decode_f32_zero_keys():
    wl = inputs.WORKLOADS["tiny"]
    worst, _ = _decode_case(wl, [1024], 4, [0.25, 0.6], 36, zero_keys=True)
    assert worst <= tl.TOL_F32


def test_decode_is_deterministic():
    wl = inputs.WORKLOADS["decode_32k"]
    B = 2
    data = [(inputs.tokens(wl, 3000, 40, b), inputs.bernoulli_mask(3000, [0.3] * 8, 40, b)) for b in range(B)]
    cache = tl.new_cache(wl, B, 3000)
    tl.append(cache, [d[1] for d in data], [d[0]["K"] for d in data], [d[0]["V"] for d in data], [0] * B, G_ | W_)
    ws = spkv.workspace(spkv.spkv_decode_ws_bytes(cache, wl.n_q))
    q = tl.dev(np.stack([d[0]["Q"][-1] for d in data]), torch.bfloat16)
    t = tl.dev(np.array([2999, 2999], np.int32))
    o1, l1 = spkv.spkv_decode_attn(cache, q, t, tl.scale_for(128), ws=ws)
    o2, l2 = spkv.spkv_decode_attn(cache, q, t, tl.scale_for(128), ws=ws)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
