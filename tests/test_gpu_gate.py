"""GPU parity of spkv_gate (Eq. 1-2) against the fp64 oracle.

Masks must match bit for bit (inputs whose oracle utility lies within 1e-3 of
tau are redrawn first); utilities within 2e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu


def _run(wl, n_rows, seed=7, tau=None, d_hidden=None, d_model=None):
    import dataclasses
    if d_hidden is not None:
        wl = dataclasses.replace(wl, d_hidden=d_hidden)
    if d_model is not None:
        wl = dataclasses.replace(wl, d_model=d_model)
    w = tl.calibrated_weights(wl)
    H = inputs.normal((n_rows, wl.d_model), seed, 99, dtype=wl.dtype)
    H, u_ref, z_ref = tl.resample_band(wl, w, H, seed, 99)
    dt = tl.torch_dtype(wl)
    gw = tl.gate_weights(w, dt)
    u, z = spkv.spkv_gate(gw, tl.dev(H, dt), wl.tau if tau is None else tau)
    torch.cuda.synchronize()
    return u.cpu().numpy(), z.cpu().numpy(), u_ref, z_ref


@pytest.mark.parametrize("name,n_rows,d_hidden", [
    ("tiny", 1024, None),          # f32, VALU
    ("tiny", 37, None),
    ("tiny", 1, None),             # few rows: one workgroup per hidden unit
    ("tiny", 16, None),
    ("decode_32k", 1, None),
    ("decode_32k", 8, None),       # bf16 decode step (few-row MFMA tiles)
    ("decode_32k", 16, None),      # largest few-row batch
    ("decode_32k", 3, 256),
    ("decode_32k", 12, 48),
    ("decode_32k", 17, None),      # bf16, d_model split over workgroups
    ("decode_32k", 64, None),      # largest split batch
    ("decode_32k", 65, None),      # first full-tile batch, ragged tail (pipelined kernel, d_model 4096)
    ("decode_32k", 1500, None),    # several 64-row tiles, ragged last tile
    ("decode_32k", 1024, 64),      # 64-row kernel, d_hidden 64 (16 iterations in flight)
    ("decode_32k", 2000, 256),     # 64-row kernel, d_hidden 256 (4 in flight)
    ("decode_32k", 40, 32),        # d_hidden 32 on the split path
    ("decode_32k", 300, 256),
    ("decode_32k", 200, 32),       # pipelined kernel, every unit width
    ("decode_32k", 129, 64),
    ("decode_32k", 50, 48),        # d_hidden without an MFMA tiling: VALU kernel
])
def test_gate_matches_oracle(name, n_rows, d_hidden):
    u, z, u_ref, z_ref = _run(inputs.WORKLOADS[name], n_rows, d_hidden=d_hidden)
    print(f"[gate {name} n={n_rows} hg={d_hidden}] max|du|={tl.max_abs(u, u_ref):.3e} kept={z.mean():.3f}")
    np.testing.assert_array_equal(z, z_ref)
    assert tl.max_abs(u, u_ref) <= tl.U_TOL


@pytest.mark.parametrize("d_model,n_rows,d_hidden", [
    (1088, 300, 128),   # pipelined kernel, run-time trip count not a multiple of its depth
    (128, 100, 256),    # two iterations: fewer than the pipeline depth
    (640, 70, 64),
    (96, 130, 128),     # d_model not a multiple of 64: the plain MFMA kernel
    (1152, 1300, 128),  # 18 iterations at a run-time trip count
    (640, 1100, 64),    # 10 iterations, fewer than the depth (16)
])
def test_gate_other_model_widths(d_model, n_rows, d_hidden):
    u, z, u_ref, z_ref = _run(inputs.WORKLOADS["decode_32k"], n_rows, d_hidden=d_hidden, d_model=d_model)
    print(f"[gate d_model={d_model} n={n_rows} hg={d_hidden}] max|du|={tl.max_abs(u, u_ref):.3e} kept={z.mean():.3f}")
    np.testing.assert_array_equal(z, z_ref)
    assert tl.max_abs(u, u_ref) <= tl.U_TOL


def test_gate_threshold_edges_and_nan():
    wl = inputs.WORKLOADS["decode_32k"]
    w = tl.calibrated_weights(wl)
    H = inputs.normal((70, wl.d_model), 3, 1, dtype=wl.dtype)
    H[5, 100] = np.nan
    gw = tl.gate_weights(w, torch.bfloat16)
    hd = tl.dev(H, torch.bfloat16)
    _, z0 = spkv.spkv_gate(gw, hd, 0.0)
    _, z1 = spkv.spkv_gate(gw, hd, 1.5)
    u, zh = spkv.spkv_gate(gw, hd, 0.5)
    z0, z1, zh, u = z0.cpu().numpy(), z1.cpu().numpy(), zh.cpu().numpy(), u.cpu().numpy()
    good = np.ones(70, bool)
    good[5] = False
    assert np.all(z0[good] == 1) and np.all(z1 == 0)
    assert np.all(np.isnan(u[5])) and np.all(zh[5] == 0) and np.all(z0[5] == 0)


def test_gate_is_deterministic():
    wl = inputs.WORKLOADS["decode_32k"]
    w = tl.calibrated_weights(wl)
    H = tl.dev(inputs.normal((8, wl.d_model), 4, 1, dtype=wl.dtype), torch.bfloat16)
    gw = tl.gate_weights(w, torch.bfloat16)
    u1, _ = spkv.spkv_gate(gw, H, 0.5)
    u2, _ = spkv.spkv_gate(gw, H, 0.5)
    assert torch.equal(u1, u2)


def test_gate_workspace_reuse_across_batch_sizes():
    # one workspace shared by consecutive calls of every launch shape; each
    # call leaves it ready for the next
    wl = inputs.WORKLOADS["decode_32k"]
    w = tl.calibrated_weights(wl)
    gw = tl.gate_weights(w, torch.bfloat16)
    sizes = [16, 5, 40, 3, 1, 64, 8, 3000, 20, 1500, 64]   # few-row and many-row kernels
    ws = spkv.workspace(max(spkv.spkv_gate_ws_bytes(gw, n) for n in sizes))
    for i, n in enumerate(sizes):
        H = tl.dev(inputs.normal((n, wl.d_model), 6, i, dtype=wl.dtype), torch.bfloat16)
        u1, z1 = spkv.spkv_gate(gw, H, 0.5, ws=ws)
        u2, z2 = spkv.spkv_gate(gw, H, 0.5)
        assert torch.equal(u1, u2) and torch.equal(z1, z2)
