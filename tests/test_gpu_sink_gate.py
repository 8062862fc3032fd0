"""GPU parity of spkv_gate_sink (the sink-attention gate of the Fast KVzip
page) against the oracle's O8, on seeded inputs.  Hidden rows whose oracle
utility lies within 1e-3 of tau for some head are redrawn, so that the keep
bits are decided the same way on both sides and compared exactly.

Tolerance on the utility: the projections are bf16 x bf16 products summed in
f32 over d_model terms (relative error a few 1e-7 for the O(1) values drawn
here), the scores, softmax and maximum are f32; the utility moves by at most
a quarter of a score's error, so 5e-5 holds with a wide margin."""
import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

U_TOL = 5e-5
BAND = 1e-3


def _weights(n_kv, G, S, d, seed):
    r = np.random.default_rng(seed)
    # entries ~ N(0, 1/d): projections of N(0, 1) hidden rows are O(1), scores O(1)
    W = inputs.normal((n_kv, (G + 1) * 16, d), seed, 1) / np.float32(np.sqrt(d))
    W = torch.from_numpy(W).to(torch.bfloat16).float().numpy()     # bf16-exact values
    sinks = r.standard_normal((n_kv, S, 16)).astype(np.float32)
    return W, sinks


def _rows(n, d, W, sinks, G, tau, seed):
    """Hidden rows, their oracle utilities and keep bits at tau (None: the 70th
    percentile of the rows' utilities, so that both decisions are common)."""
    H = inputs.normal((n, d), seed, 2, dtype="bf16")
    u, z = oracle.sink_gate(H, W, sinks, G, 0.5, threads=tl.oracle_threads())
    if tau is None:
        tau = float(np.quantile(u, 0.7))
    z = (u >= tau).astype(np.uint8)
    for attempt in range(50):
        bad = np.flatnonzero(np.any(np.abs(u - tau) < BAND, axis=1))
        if bad.size == 0:
            return H, u, z, tau
        H[bad] = inputs.normal((bad.size, d), seed, 3, attempt, dtype="bf16")
        u[bad], z[bad] = oracle.sink_gate(H[bad], W, sinks, G, tau, threads=tl.oracle_threads())
    raise RuntimeError("band redraw did not converge")


@pytest.mark.parametrize("n_kv, G, S, d, n", [
    (8, 4, 16, 4096, 200),    # the 8B-shaped layer, the page's S and d_key; a ragged row tile
    (8, 4, 16, 256, 64),
    (3, 1, 1, 320, 63),
    (2, 2, 0, 128, 130),      # no sinks: every pair is kept
    (1, 8, 64, 512, 1),
    (16, 8, 5, 192, 77),
    (8, 1, 16, 4096, 300),    # 4 heads per workgroup (8 projection tiles), d_model 4096: 2 iterations in flight
    (6, 2, 5, 4096, 257),     # 2 heads per workgroup (6 tiles), two 256-row tiles, the second of one row
    (4, 8, 16, 4096, 100),    # one head per workgroup (9 tiles), d_model 4096
    (5, 2, 3, 640, 513),      # n_kv odd: one head per workgroup, three row tiles
    (12, 1, 64, 1024, 1030),  # 4 heads per workgroup, 64 sinks (four 16-sink tiles)
])
def test_sink_gate_matches_oracle(n_kv, G, S, d, n):
    W, sinks = _weights(n_kv, G, S, d, 40 + n_kv + G + S)
    H, u_ref, z_ref, tau = _rows(n, d, W, sinks, G, None if S else 0.9, 50 + d)
    g = spkv.SinkGateWeights(tl.dev(W, torch.bfloat16), tl.dev(sinks), G)
    u, z = spkv.spkv_gate_sink(g, tl.dev(H, torch.bfloat16), tau)
    torch.cuda.synchronize()
    err = tl.max_abs(u.cpu().numpy(), u_ref)
    print(f"[sink gate n_kv={n_kv} G={G} S={S} d={d} n={n}] tau={tau:.4f} max|du|={err:.2e} keep={z_ref.mean():.3f}")
    assert err <= U_TOL
    np.testing.assert_array_equal(z.cpu().numpy(), z_ref)


def test_sink_gate_zero_rows_and_nan():
    W, sinks = _weights(2, 4, 16, 256, 7)
    g = spkv.SinkGateWeights(tl.dev(W, torch.bfloat16), tl.dev(sinks), 4)
    H = np.zeros((3, 256), np.float32)
    H[1, 5] = np.nan
    u, z = spkv.spkv_gate_sink(g, tl.dev(H, torch.bfloat16), 1.0 / 17)
    torch.cuda.synchronize()
    u, z = u.cpu().numpy(), z.cpu().numpy()
    np.testing.assert_allclose(u[[0, 2]], 1.0 / 17, rtol=0, atol=1e-7)   # q = k = 0: 1 / (1 + S)
    assert np.all(np.isnan(u[1])) and np.all(z[1] == 0)
    empty = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    u0, z0 = spkv.spkv_gate_sink(g, empty, 0.5)
    assert u0.shape == (0, 2) and z0.shape == (0, 2)


def test_sink_gate_full_size_sampled_rows():
    # 16384 rows of the 8B-shaped layer (d_model 4096, 8 key heads, G 4, S 16,
    # d_key 16) in one launch, checked on 256 sampled rows; tau at the 70th
    # percentile of the sampled rows' utilities
    n_kv, G, S, d, n = 8, 4, 16, 4096, 16384
    W, sinks = _weights(n_kv, G, S, d, 91)
    g = spkv.SinkGateWeights(tl.dev(W, torch.bfloat16), tl.dev(sinks), G)
    Hd = inputs.device_normal((n, d), 91, inputs.STREAM_H, torch.bfloat16)
    rows = np.sort(np.random.default_rng(3).choice(n, 256, replace=False))
    Hs = Hd[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    u_ref, _ = oracle.sink_gate(Hs, W, sinks, G, 0.5, threads=tl.oracle_threads())
    tau = float(np.quantile(u_ref, 0.7))
    z_ref = (u_ref >= tau).astype(np.uint8)
    u, z = spkv.spkv_gate_sink(g, Hd, tau)
    torch.cuda.synchronize()
    ug, zg = u.cpu().numpy()[rows], z.cpu().numpy()[rows]
    err = tl.max_abs(ug, u_ref)
    clear = np.abs(u_ref - tau) >= BAND
    print(f"[sink gate full] tau={tau:.4f} max|du|={err:.2e} clear={clear.mean():.4f} keep={z_ref.mean():.3f}")
    assert err <= U_TOL
    np.testing.assert_array_equal(zg[clear], z_ref[clear])
