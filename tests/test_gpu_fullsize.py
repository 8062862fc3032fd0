"""Parity at the full workload sizes, in the launch configuration the
benchmark uses, on outputs the fp64 oracle computes one by one.

Inputs are drawn with torch's seeded device generator (learned_kv_cache_sp_amd
.inputs.device_normal / device_bernoulli_mask) and copied to the host for the
oracle; keep masks given to both sides come from the generator, so nothing
the HIP path computes is fed to the oracle.  The gate is checked at full size
on sampled rows (masks exactly, wherever the oracle's utility is at least
1e-3 away from tau; utilities within 2e-5 everywhere).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def build_decode_cache(wl, contexts, steps, seed, page=64):
    """Prefix of every sequence appended in one call (as the benchmark does),
    then `steps` decode steps of one token per sequence."""
    B = len(contexts)
    T = [int(cx) + steps for cx in contexts]
    K = [inputs.device_normal((T[b], wl.n_kv, wl.head_dim), seed, 10 + b, torch.bfloat16) for b in range(B)]
    V = [inputs.device_normal((T[b], wl.n_kv, wl.head_dim), seed, 100 + b, torch.bfloat16) for b in range(B)]
    Q = [inputs.device_normal((steps, wl.n_q, wl.head_dim), seed, 200 + b, torch.bfloat16) for b in range(B)]
    Z = [inputs.device_bernoulli_mask(T[b], wl.keep, seed, 300 + b) for b in range(B)]
    max_pages = max(T) // page + 2
    need = sum(spkv.Cache.pages_needed([int(Z[b][:, g].sum()) for g in range(wl.n_kv)], page) for b in range(B))
    cache = spkv.Cache(B, wl.n_kv, wl.head_dim, wl.window, page, need + B * wl.n_kv + 8, max_pages, torch.bfloat16)
    ctx = [int(cx) for cx in contexts]
    offs = torch.tensor(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32), device="cuda")
    spkv.spkv_compact_append(cache, torch.cat([Z[b][:ctx[b]] for b in range(B)]),
                             torch.cat([K[b][:ctx[b]] for b in range(B)]),
                             torch.cat([V[b][:ctx[b]] for b in range(B)]), offs,
                             torch.zeros(B, dtype=torch.int32, device="cuda"), max(ctx), G_ | W_)
    return cache, K, V, Q, Z, ctx


def run_decode_parity(name, contexts, steps, check_steps, seed, zero_keys_heads=None):
    wl = inputs.WORKLOADS[name]
    B = len(contexts)
    cache, K, V, Q, Z, ctx = build_decode_cache(wl, contexts, steps, seed)
    ws = spkv.workspace(spkv.spkv_decode_ws_bytes(cache, wl.n_q))
    scale = 1.0 / math.sqrt(wl.head_dim)
    ro1 = torch.arange(0, B + 1, dtype=torch.int32, device="cuda")
    outs = {}
    for s in range(steps):
        t = torch.tensor([ctx[b] + s for b in range(B)], dtype=torch.int32, device="cuda")
        zs = torch.stack([Z[b][ctx[b] + s] for b in range(B)])
        ks = torch.stack([K[b][ctx[b] + s] for b in range(B)])
        vs = torch.stack([V[b][ctx[b] + s] for b in range(B)])
        spkv.spkv_compact_append(cache, zs, ks, vs, ro1, t, 1, G_ | W_)
        q = torch.stack([Q[b][s] for b in range(B)])
        o, l = spkv.spkv_decode_attn(cache, q, t, scale, ws=ws)
        if s in check_steps:
            outs[s] = (o.cpu().numpy(), l.cpu().numpy())
    assert spkv.spkv_cache_check(cache) == 0
    worst = worst_l = 0.0
    th = tl.oracle_threads()
    for b in range(B):
        Kh, Vh, Zh, Qh = host_f32(K[b]), host_f32(V[b]), Z[b].cpu().numpy(), host_f32(Q[b])
        for s, (o, l) in outs.items():
            t = ctx[b] + s
            ro, rl = oracle.attention(Qh[s:s + 1], [t], Kh, Vh, Zh, wl.window, scale, threads=th)
            worst = max(worst, tl.max_abs(o[b], ro[0]))
            worst_l = max(worst_l, tl.max_abs(l[b], rl[0]))
        # the cache of every head holds exactly the oracle's kept list
        lists = oracle.compact(Zh, 0)
        for g in range(wl.n_kv):
            kk, vv, pos = cache.read_head(b, g)
            np.testing.assert_array_equal(pos.cpu().numpy(), lists[g])
            sel = np.linspace(0, len(lists[g]) - 1, 64).astype(int) if len(lists[g]) else []
            np.testing.assert_array_equal(kk[sel].float().cpu().numpy(), Kh[lists[g][sel], g])
            np.testing.assert_array_equal(vv[sel].float().cpu().numpy(), Vh[lists[g][sel], g])
    return worst, worst_l


def test_decode_32k_full_size():
    wl = inputs.WORKLOADS["decode_32k"]
    worst, worst_l = run_decode_parity("decode_32k", [wl.context] * wl.batch, 3, {0, 2}, 71)
    print(f"[decode_32k full] max|dout|={worst:.2e} max|dlse|={worst_l:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_l <= tl.TOL_REGRESS


def test_decode_131k_skewed_full_size():
    wl = inputs.WORKLOADS["decode_131k"]
    worst, worst_l = run_decode_parity("decode_131k", [wl.context] * wl.batch, 2, {1}, 72)
    print(f"[decode_131k full] max|dout|={worst:.2e} max|dlse|={worst_l:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_l <= tl.TOL_REGRESS


def test_decode_ragged_32_full_size():
    wl = inputs.WORKLOADS["ragged_32"]
    ctx = inputs.ragged_contexts(wl)
    worst, worst_l = run_decode_parity("ragged_32", list(ctx), 2, {1}, 73)
    print(f"[ragged_32 full] max|dout|={worst:.2e} max|dlse|={worst_l:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_l <= tl.TOL_REGRESS


def run_decode_step_parity(name, steps, seed):
    """spkv_decode_step (gate + kept/window append + attention in one launch)
    for `steps` consecutive tokens of every sequence, on the benchmark's
    configuration.  The step tokens' hidden rows are drawn on the host and
    redrawn where the oracle's utility lies within 1e-3 of tau, so that the
    keep bits are decided the same way on both sides; the prefix's keep bits
    come from the seeded generator."""
    wl = inputs.WORKLOADS[name]
    B, nkv, nq, hd = wl.batch, wl.n_kv, wl.n_q, wl.head_dim
    contexts = [wl.context] * B
    w = tl.calibrated_weights(wl, seed)
    gw = tl.gate_weights(w, torch.bfloat16)
    cache, K, V, Q, Z, ctx = build_decode_cache(wl, contexts, steps, seed)
    ws = spkv.workspace(spkv.spkv_decode_step_ws_bytes(cache, gw, nq))
    scale = 1.0 / math.sqrt(hd)
    Zfull = [Z[b].cpu().numpy().copy() for b in range(B)]
    outs = {}
    worst_u = 0.0
    for s in range(steps):
        H = inputs.normal((B, wl.d_model), seed, 400, s, dtype=wl.dtype)
        H, u_ref, z_ref = tl.resample_band(wl, w, H, seed, 500 + s)
        for b in range(B):
            Zfull[b][ctx[b] + s] = z_ref[b]
        t = torch.tensor([ctx[b] + s for b in range(B)], dtype=torch.int32, device="cuda")
        ks = torch.stack([K[b][ctx[b] + s] for b in range(B)])
        vs = torch.stack([V[b][ctx[b] + s] for b in range(B)])
        q = torch.stack([Q[b][s] for b in range(B)])
        u, z, o, l = spkv.spkv_decode_step(cache, gw, tl.dev(H, torch.bfloat16), wl.tau, ks, vs, q, t, scale, ws=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(z.cpu().numpy(), z_ref.astype(np.uint8))
        worst_u = max(worst_u, tl.max_abs(u.cpu().numpy(), u_ref))
        assert tl.step_counters_settled(ws, B, nkv), "arrival counters not settled"
        outs[s] = (o.cpu().numpy(), l.cpu().numpy())
    assert spkv.spkv_cache_check(cache) == 0
    assert worst_u <= tl.U_TOL
    worst = worst_l = 0.0
    th = tl.oracle_threads()
    lengths = cache.lengths.cpu().numpy()
    for b in range(B):
        Kh, Vh, Qh = host_f32(K[b]), host_f32(V[b]), host_f32(Q[b])
        for s, (o, l) in outs.items():
            ro, rl = oracle.attention(Qh[s:s + 1], [ctx[b] + s], Kh, Vh, Zfull[b], wl.window, scale, threads=th)
            worst = max(worst, tl.max_abs(o[b], ro[0]))
            worst_l = max(worst_l, tl.max_abs(l[b], rl[0]))
        lists = oracle.compact(Zfull[b], 0)
        for g in range(nkv):
            assert lengths[b, g] == len(lists[g])
            kk, vv, pos = cache.read_head(b, g)
            np.testing.assert_array_equal(pos.cpu().numpy(), lists[g])
            # the step rows that were kept, and a spread of the prefix's
            sel = np.unique(np.concatenate([np.linspace(0, len(lists[g]) - 1, 64).astype(int),
                                            np.flatnonzero(lists[g] >= ctx[b])])) if len(lists[g]) else []
            np.testing.assert_array_equal(kk[sel].float().cpu().numpy(), Kh[lists[g][sel], g])
            np.testing.assert_array_equal(vv[sel].float().cpu().numpy(), Vh[lists[g][sel], g])
    return worst, worst_l, worst_u


def test_decode_step_32k_full_size():
    worst, worst_l, worst_u = run_decode_step_parity("decode_32k", 3, 81)
    print(f"[decode_step 32k full] max|dout|={worst:.2e} max|dlse|={worst_l:.2e} max|du|={worst_u:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_l <= tl.TOL_REGRESS


def test_decode_step_131k_full_size():
    worst, worst_l, worst_u = run_decode_step_parity("decode_131k", 2, 82)
    print(f"[decode_step 131k full] max|dout|={worst:.2e} max|dlse|={worst_l:.2e} max|du|={worst_u:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_l <= tl.TOL_REGRESS


def test_gate_full_size_sampled_rows():
    # the benchmark's prefix gate: 262,144 rows of the 8B-shaped layer
    wl = inputs.WORKLOADS["decode_32k"]
    w = tl.calibrated_weights(wl)
    gw = tl.gate_weights(w, torch.bfloat16)
    n = wl.batch * wl.context
    H = inputs.device_normal((n, wl.d_model), wl.seed, 77, torch.bfloat16)
    u, z = spkv.spkv_gate(gw, H, wl.tau)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                     np.random.default_rng(0).integers(0, n, 1500)]))
    Hs = H[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    u_ref, _, z_ref = oracle.gate(Hs, w["W1"], w["b1"], w["W2"], w["b2"], wl.tau, threads=tl.oracle_threads())
    ug, zg = u[torch.from_numpy(rows).cuda()].cpu().numpy(), z[torch.from_numpy(rows).cuda()].cpu().numpy()
    clear = np.abs(u_ref - wl.tau) >= tl.BAND
    print(f"[gate full] rows={len(rows)} max|du|={tl.max_abs(ug, u_ref):.2e} clear={clear.mean():.4f} "
          f"keep={zg.mean():.3f}")
    assert tl.max_abs(ug, u_ref) <= tl.U_TOL
    np.testing.assert_array_equal(zg[clear], z_ref[clear])
    # the keep rate the benchmark's output bias targets
    assert abs(float(z.float().mean()) - 0.20) < 0.02


def test_prefill_64k_full_size_sampled_rows():
    wl = inputs.WORKLOADS["prefill_64k"]
    T, CH = wl.context, wl.chunk
    seed = 74
    K = inputs.device_normal((T, wl.n_kv, wl.head_dim), seed, 1, torch.bfloat16)
    V = inputs.device_normal((T, wl.n_kv, wl.head_dim), seed, 2, torch.bfloat16)
    Q = inputs.device_normal((T, wl.n_q, wl.head_dim), seed, 3, torch.bfloat16)
    Z = inputs.device_bernoulli_mask(T, wl.keep, seed, 4)
    per = T // 64 + 2
    cache = spkv.Cache(1, wl.n_kv, wl.head_dim, wl.window, 64, wl.n_kv * per, per, torch.bfloat16)
    scale = 1.0 / math.sqrt(wl.head_dim)
    rng = np.random.default_rng(5)
    sample = []
    for c0 in range(0, T, CH):
        sample += list(range(c0, c0 + 6)) + list(range(c0 + 125, c0 + 131)) + list(c0 + rng.integers(131, CH, 8))
    sample = np.array(sorted(set(sample)))
    got_o, got_l = {}, {}
    for c0 in range(0, T, CH):
        n = min(CH, T - c0)
        ro = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        p0 = torch.tensor([c0], dtype=torch.int32, device="cuda")
        spkv.spkv_compact_append(cache, Z[c0:c0 + n], K[c0:c0 + n], V[c0:c0 + n], ro, p0, n, G_)
        o, l = spkv.spkv_prefill_attn(cache, 0, Q[c0:c0 + n], K[c0:c0 + n], V[c0:c0 + n], c0, scale)
        spkv.spkv_compact_append(cache, None, K[c0:c0 + n], V[c0:c0 + n], ro, p0, n, W_)
        rows = sample[(sample >= c0) & (sample < c0 + n)]
        oc, lc = o.cpu().numpy(), l.cpu().numpy()
        for r in rows:
            got_o[r], got_l[r] = oc[r - c0], lc[r - c0]
    assert spkv.spkv_cache_check(cache) == 0
    ro_, rl_ = oracle.attention(host_f32(Q[torch.from_numpy(sample).cuda()]), sample, host_f32(K), host_f32(V),
                                Z.cpu().numpy(), wl.window, scale, threads=tl.oracle_threads())
    out = np.stack([got_o[r] for r in sample])
    lse = np.stack([got_l[r] for r in sample])
    print(f"[prefill_64k full] rows={len(sample)} max|dout|={tl.max_abs(out, ro_):.2e} "
          f"max|dlse|={tl.max_abs(lse, rl_):.2e}")
    assert tl.max_abs(out, ro_) <= tl.TOL_PREFILL and tl.max_abs(lse, rl_) <= tl.TOL_REGRESS


def test_rethreshold_decode_32k_full_size():
    # the decode_32k cache (8 x 32768 tokens, 8 key heads, 20 % kept) with
    # generator utilities, rebuilt at a threshold keeping about half; every
    # list's positions exact against the oracle (O2 at tau, then O5 at tau2),
    # keys, values and utilities of sampled lists exact
    wl = inputs.WORKLOADS["decode_32k"]
    B, T, nkv, hd, P = wl.batch, wl.context, wl.n_kv, wl.head_dim, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    tau = 0.8  # 20 % of uniform utilities pass
    u = torch.rand((B * T, nkv), generator=gen, device="cuda", dtype=torch.float32)
    z = (u >= tau).to(torch.uint8)
    K = inputs.device_normal((B * T, nkv, hd), 17, inputs.STREAM_K, torch.bfloat16)
    V = inputs.device_normal((B * T, nkv, hd), 17, inputs.STREAM_V, torch.bfloat16)
    per_head = int(T * 0.25 / P) + 4
    src = spkv.Cache(B, nkv, hd, wl.window, P, B * nkv * per_head, per_head, torch.bfloat16, utilities=True)
    dst = spkv.Cache(B, nkv, hd, wl.window, P, B * nkv * per_head, per_head, torch.bfloat16, utilities=True)
    ro = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
    spkv.spkv_compact_append(src, z, K, V, ro, torch.zeros(B, dtype=torch.int32, device="cuda"), T, G_ | W_,
                             utility=u)
    tau2 = 0.9
    spkv.spkv_cache_rethreshold(src, dst, tau2)
    torch.cuda.synchronize()
    assert spkv.spkv_cache_check(src) == 0 and spkv.spkv_cache_check(dst) == 0
    uh = u.cpu().numpy()
    for b in range(B):
        ub = uh[b * T:(b + 1) * T]
        for g in range(nkv):
            kept = oracle.compact((ub[:, g:g + 1] >= np.float32(tau)).astype(np.uint8))[0]
            rows = kept[oracle.rethreshold(ub[kept, g], float(np.float32(tau2)))]
            pos = dst.read_head(b, g)[2].cpu().numpy()
            np.testing.assert_array_equal(pos, rows, err_msg=f"b={b} g={g}")
            if (b * nkv + g) % 13 == 0:
                k, v, _ = dst.read_head(b, g)
                sel = torch.from_numpy(b * T + rows).cuda()
                assert torch.equal(k, K[sel, g]) and torch.equal(v, V[sel, g])
                assert torch.equal(dst.read_head_u(b, g), u[sel, g])


def test_head_stats_full_size():
    # 1,048,576 rows x 8 heads, the benchmark's shape and generator
    n, nkv = 1 << 20, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    u = torch.rand((n, nkv), generator=gen, device="cuda", dtype=torch.float32)
    z = (torch.rand((n, nkv), generator=gen, device="cuda") < 0.2).to(torch.uint8)
    us, kp = spkv.spkv_head_stats(u, z)
    ru, rk = oracle.head_stats(u.cpu().numpy(), z.cpu().numpy())
    np.testing.assert_array_equal(kp.cpu().numpy(), rk)
    np.testing.assert_allclose(us.cpu().numpy(), ru, rtol=1e-12)


def test_soft_prefill_16k_full_size_sampled_rows():
    # the soft_prefill_16k workload (16384 tokens, 8B layer, beta 0.01,
    # c 1e6, every token cached), checked on sampled rows against O7
    wl = inputs.WORKLOADS["prefill_64k"]
    T, nq, nkv, hd, w, P = 16384, wl.n_q, wl.n_kv, wl.head_dim, wl.window, 64
    per_head = T // P + 2
    cache = spkv.Cache(1, nkv, hd, w, P, nkv * per_head, per_head, torch.bfloat16, utilities=True)
    Q = inputs.device_normal((T, nq, hd), 23, inputs.STREAM_Q, torch.bfloat16)
    K = inputs.device_normal((T, nkv, hd), 23, inputs.STREAM_K, torch.bfloat16)
    V = inputs.device_normal((T, nkv, hd), 23, inputs.STREAM_V, torch.bfloat16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(23)
    u = torch.rand((T, nkv), generator=gen, device="cuda", dtype=torch.float32)
    ro = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    p0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    spkv.spkv_compact_append(cache, torch.ones((T, nkv), dtype=torch.uint8, device="cuda"), K, V, ro, p0, T, G_,
                             utility=u)
    scale = 1.0 / math.sqrt(hd)
    out, lse = spkv.spkv_prefill_attn(cache, 0, Q, K, V, 0, scale, soft=(wl.tau, 0.01, 1e6))
    torch.cuda.synchronize()
    rows = np.concatenate([[0, 1, w - 1, w, w + 1, T - 1], np.random.default_rng(3).integers(0, T, 10)])
    Qh, Kh, Vh, uh = host_f32(Q), host_f32(K), host_f32(V), u.cpu().numpy()
    ro_, rl = oracle.soft_attention(Qh[rows], rows, Kh, Vh, uh, w, wl.tau, 0.01, 1e6, scale,
                                    threads=tl.oracle_threads())
    o = out.cpu().numpy()[rows]
    l = lse.cpu().numpy()[rows]
    print(f"[soft_prefill_16k full] max|dout|={tl.max_abs(o, ro_):.2e} max|dlse|={tl.max_abs(l, rl):.2e}")
    assert tl.max_abs(o, ro_) < tl.TOL_PREFILL
    assert tl.max_abs(l, rl) < tl.TOL_REGRESS
