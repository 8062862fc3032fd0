"""End to end on the tiny layer (f32) and a reduced 8B-shaped layer (bf16):
gate -> compaction -> chunked prefill -> decode steps, every stage checked
against the fp64 oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW


def run_pipeline(wl, T_prefix, steps, chunk, seed):
    li = tl.layer_inputs(wl, [T_prefix + steps], seed)
    H, Q, K, V, z_ref = li.H[0], li.Q[0], li.K[0], li.V[0], li.z[0]
    dt = tl.torch_dtype(wl)
    gw = tl.gate_weights(li, dt)
    cache = tl.new_cache(wl, 1, T_prefix + steps)
    scale = tl.scale_for(wl.head_dim)
    outs, lses, zs = [], [], []
    for p0 in range(0, T_prefix, chunk):
        sl = slice(p0, min(T_prefix, p0 + chunk))
        _, z = spkv.spkv_gate(gw, tl.dev(H[sl], dt), wl.tau)
        zs.append(z.cpu().numpy())
        kd, vd = tl.dev(K[sl], dt), tl.dev(V[sl], dt)
        n = kd.shape[0]
        ro = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        p0d = torch.tensor([p0], dtype=torch.int32, device="cuda")
        spkv.spkv_compact_append(cache, z, kd, vd, ro, p0d, n, G_)
        o, l = spkv.spkv_prefill_attn(cache, 0, tl.dev(Q[sl], dt), kd, vd, p0, scale)
        spkv.spkv_compact_append(cache, None, kd, vd, ro, p0d, n, W_)
        outs.append(o.cpu().numpy())
        lses.append(l.cpu().numpy())
    ws = spkv.workspace(spkv.spkv_decode_ws_bytes(cache, wl.n_q))
    dec_o, dec_l = [], []
    for t in range(T_prefix, T_prefix + steps):
        _, z = spkv.spkv_gate(gw, tl.dev(H[t:t + 1], dt), wl.tau)
        zs.append(z.cpu().numpy())
        kd, vd = tl.dev(K[t:t + 1], dt), tl.dev(V[t:t + 1], dt)
        ro = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
        td = torch.tensor([t], dtype=torch.int32, device="cuda")
        spkv.spkv_compact_append(cache, z, kd, vd, ro, td, 1, G_ | W_)
        o, l = spkv.spkv_decode_attn(cache, tl.dev(Q[t:t + 1], dt), td, scale, ws=ws)
        dec_o.append(o.cpu().numpy()[0])
        dec_l.append(l.cpu().numpy()[0])
    assert spkv.spkv_cache_check(cache) == 0
    z_gpu = np.concatenate(zs)
    np.testing.assert_array_equal(z_gpu, z_ref)
    rows = np.arange(T_prefix + steps)
    ro_, rl_ = oracle.attention(Q, rows, K, V, z_ref, wl.window, scale, threads=tl.oracle_threads())
    out = np.concatenate(outs + [np.stack(dec_o)])
    lse = np.concatenate(lses + [np.stack(dec_l)])
    # the cache holds exactly the oracle's kept list
    lists = oracle.compact(z_ref, 0)
    for g in range(wl.n_kv):
        k, v, pos = cache.read_head(0, g)
        np.testing.assert_array_equal(pos.cpu().numpy(), lists[g])
        np.testing.assert_array_equal(k.float().cpu().numpy(), K[lists[g], g])
    return tl.max_abs(out, ro_), tl.max_abs(lse, rl_), z_ref.mean(0)


def test_pipeline_tiny_f32():
    wl = inputs.WORKLOADS["tiny"]
    e_o, e_l, keep = run_pipeline(wl, 1024, 16, 1024, wl.seed)
    print(f"[pipeline tiny] max|dout|={e_o:.2e} max|dlse|={e_l:.2e} keep={keep}")
    assert e_o <= tl.TOL_F32 and e_l <= tl.TOL_F32
    assert np.all(np.abs(keep - 0.25) < 0.08)


def test_pipeline_bf16_reduced_8b_layer():
    wl = inputs.WORKLOADS["prefill_64k"]
    e_o, e_l, keep = run_pipeline(wl, 1500, 6, 512, wl.seed)
    print(f"[pipeline bf16] max|dout|={e_o:.2e} max|dlse|={e_l:.2e} keep={keep}")
    assert e_o <= tl.TOL_PREFILL and e_l <= tl.TOL_REGRESS
