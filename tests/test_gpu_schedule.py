"""Buffered gating (the decode-time hidden-state buffer of Fast KVzip's method
section, applied to SP-KV's gate): every step appends the new token to the
window ring and runs decode attention; every `buffer` steps the buffered rows
of all sequences are gated at once and their kept pairs appended.  Because the
buffer is no longer than the window, every token is gated before it leaves the
window, so the attention outputs equal those of per-token gating (SP-KV Eq. 4
holds at every step).  Both schedules run on the GPU and are compared with the
fp64 oracle, which gates every token on its own.
"""
import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW


def _i32(x):
    return torch.tensor(np.asarray(x, np.int32), device="cuda")


def run_schedule(wl, ctxs, steps, buffer, li):
    """Decode `steps` tokens of every sequence after its prefix; gate per token
    (buffer = 0) or in buffers of `buffer` rows.  Returns outputs, lse, the GPU
    keep bits of every gated row and the cache."""
    B = len(ctxs)
    dt = tl.torch_dtype(wl)
    gw = tl.gate_weights(li, dt)
    cache = tl.new_cache(wl, B, max(ctxs) + steps, spare_pages=2)
    scale = tl.scale_for(wl.head_dim)
    # prefix: one gate call over all sequences' rows, one append
    Hp = np.concatenate([li.H[b][:ctxs[b]] for b in range(B)])
    _, zp = spkv.spkv_gate(gw, tl.dev(Hp, dt), wl.tau)
    offs = np.concatenate([[0], np.cumsum(ctxs)])
    zpre = zp.cpu().numpy()
    tl.append(cache, [zpre[offs[b]:offs[b + 1]] for b in range(B)], [li.K[b][:ctxs[b]] for b in range(B)],
              [li.V[b][:ctxs[b]] for b in range(B)], [0] * B, G_ | W_)
    z_gpu = [[zpre[offs[b]:offs[b + 1]]] for b in range(B)]
    ws = spkv.workspace(spkv.spkv_decode_ws_bytes(cache, wl.n_q))
    ro1 = _i32(np.arange(B + 1))
    outs, lses = [], []
    for s in range(steps):
        t = [ctxs[b] + s for b in range(B)]
        td = _i32(t)
        K = tl.dev(np.stack([li.K[b][t[b]] for b in range(B)]), dt)
        V = tl.dev(np.stack([li.V[b][t[b]] for b in range(B)]), dt)
        if buffer == 0:
            _, z = spkv.spkv_gate(gw, tl.dev(np.stack([li.H[b][t[b]] for b in range(B)]), dt), wl.tau)
            spkv.spkv_compact_append(cache, z, K, V, ro1, td, 1, G_ | W_)
            zh = z.cpu().numpy()
            for b in range(B):
                z_gpu[b].append(zh[b:b + 1])
        else:
            spkv.spkv_compact_append(cache, None, K, V, ro1, td, 1, W_)
        q = tl.dev(np.stack([li.Q[b][t[b]] for b in range(B)]), dt)
        o, l = spkv.spkv_decode_attn(cache, q, td, scale, ws=ws)
        outs.append(o.cpu().numpy())
        lses.append(l.cpu().numpy())
        if buffer and (s + 1) % buffer == 0:
            lo = s + 1 - buffer
            rows = [slice(ctxs[b] + lo, ctxs[b] + s + 1) for b in range(B)]
            Hb = np.concatenate([li.H[b][rows[b]] for b in range(B)])
            _, z = spkv.spkv_gate(gw, tl.dev(Hb, dt), wl.tau)
            zh = z.cpu().numpy()
            zb = [zh[b * buffer:(b + 1) * buffer] for b in range(B)]
            tl.append(cache, zb, [li.K[b][rows[b]] for b in range(B)], [li.V[b][rows[b]] for b in range(B)],
                      [ctxs[b] + lo for b in range(B)], G_)
            for b in range(B):
                z_gpu[b].append(zb[b])
    assert spkv.spkv_cache_check(cache) == 0
    return np.stack(outs), np.stack(lses), [np.concatenate(zz) for zz in z_gpu], cache


@pytest.mark.parametrize("buffer", [128, 64])
def test_buffered_gating_equals_per_token_gating(buffer):
    wl = tl.small_workload("ragged_32", batch=4)
    ctxs = [700, 129, 333, 40]          # ragged, one shorter than the window
    steps = 2 * buffer + 44             # two flushes and a partial buffer
    li = tl.layer_inputs(wl, [c + steps for c in ctxs], seed=911)
    o_buf, l_buf, z_buf, cache_buf = run_schedule(wl, ctxs, steps, buffer, li)
    o_tok, l_tok, z_tok, _ = run_schedule(wl, ctxs, steps, 0, li)
    B = len(ctxs)
    scale = tl.scale_for(wl.head_dim)
    worst = worst_l = 0.0
    for b in range(B):
        rows = np.arange(ctxs[b], ctxs[b] + steps)
        ro, rl = oracle.attention(li.Q[b][rows], rows, li.K[b], li.V[b], li.z[b], wl.window, scale,
                                  threads=tl.oracle_threads())
        for o, l in ((o_buf, l_buf), (o_tok, l_tok)):
            worst = max(worst, tl.max_abs(o[:, b], ro))
            worst_l = max(worst_l, tl.max_abs(l[:, b], rl))
        # every gated row's keep bits equal the oracle's (per-token) decisions
        n_buf = z_buf[b].shape[0]
        np.testing.assert_array_equal(z_buf[b], li.z[b][:n_buf])
        np.testing.assert_array_equal(z_tok[b], li.z[b][:ctxs[b] + steps])
        # the buffered cache holds exactly the kept rows gated so far, in order
        lists = oracle.compact(li.z[b][:n_buf], 0)
        for g in range(wl.n_kv):
            k, v, pos = cache_buf.read_head(b, g)
            np.testing.assert_array_equal(pos.cpu().numpy(), lists[g])
            np.testing.assert_array_equal(v.float().cpu().numpy(), li.V[b][lists[g], g])
    print(f"[buffered gating {buffer}] max|dout|={worst:.2e} max|dlse|={worst_l:.2e} "
          f"max|buffered - per-token|={tl.max_abs(o_buf, o_tok):.2e}")
    assert worst <= tl.TOL_REGRESS and worst_l <= tl.TOL_REGRESS
    assert tl.max_abs(o_buf, o_tok) <= tl.TOL_REGRESS
