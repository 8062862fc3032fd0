"""GPU parity of spkv_decode_step (gate + append + decode attention in one
launch) against the three separate calls and the fp64 oracle.

Per step: utilities and keep bits equal those of spkv_gate bit for bit; the
lengths equal those of spkv_compact_append(GLOBAL | WINDOW); outputs and lse
agree with spkv_decode_attn up to the rounding of the split-K merge and with
the oracle within the bf16 bound.  At the end the logical content of every
(sequence, key head) and the window ring are equal to the separate calls'
and to the oracle's stable filter of the keep bits.
"""
import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW
TOL_SPLIT = 2e-5  # fused vs separate: only the split-K merge order differs


def _i32(x):
    return torch.tensor(np.asarray(x, np.int32), device="cuda")


def _run(wl, ctxs, steps, tau, page, seed, shared_ws=False):
    B = len(ctxs)
    dt = tl.torch_dtype(wl)
    li = tl.layer_inputs(wl, [c + steps for c in ctxs], seed=seed)
    if tau != wl.tau:
        # the oracle's decisions at this threshold (band resampling is for wl.tau;
        # tau = 0 keeps every pair and tau > 1 none, whatever the utilities)
        assert tau <= 0.0 or tau > 1.0
        li.z = [np.full_like(z, 1 if tau <= 0.0 else 0) for z in li.z]
    gw = tl.gate_weights(li, dt)
    caches = [tl.new_cache(wl, B, max(ctxs) + steps, page_size=page, spare_pages=2) for _ in range(2)]
    # prefix through the separate calls on both caches
    Hp = np.concatenate([li.H[b][:ctxs[b]] for b in range(B)])
    _, zp = spkv.spkv_gate(gw, tl.dev(Hp, dt), tau)
    zpre = zp.cpu().numpy()
    offs = np.concatenate([[0], np.cumsum(ctxs)])
    for cache in caches:
        tl.append(cache, [zpre[offs[b]:offs[b + 1]] for b in range(B)], [li.K[b][:ctxs[b]] for b in range(B)],
                  [li.V[b][:ctxs[b]] for b in range(B)], [0] * B, G_ | W_)
    fused, sep = caches
    ws_step = spkv.workspace(spkv.spkv_decode_step_ws_bytes(fused, gw, wl.n_q))
    ws_attn = ws_step if shared_ws else spkv.workspace(spkv.spkv_decode_ws_bytes(sep, wl.n_q))
    ro1 = _i32(np.arange(B + 1))
    scale = tl.scale_for(wl.head_dim)
    th = tl.oracle_threads()
    worst = worst_l = split = 0.0
    for s in range(steps):
        t = [ctxs[b] + s for b in range(B)]
        td = _i32(t)
        h = tl.dev(np.stack([li.H[b][t[b]] for b in range(B)]), dt)
        k = tl.dev(np.stack([li.K[b][t[b]] for b in range(B)]), dt)
        v = tl.dev(np.stack([li.V[b][t[b]] for b in range(B)]), dt)
        q = tl.dev(np.stack([li.Q[b][t[b]] for b in range(B)]), dt)
        uf, zf, of, lf = spkv.spkv_decode_step(fused, gw, h, tau, k, v, q, td, scale, ws=ws_step)
        us, zs = spkv.spkv_gate(gw, h, tau)
        spkv.spkv_compact_append(sep, zs, k, v, ro1, td, 1, G_ | W_)
        os_, ls = spkv.spkv_decode_attn(sep, q, td, scale, ws=ws_attn)
        assert torch.equal(uf, us), f"step {s}: utilities differ from spkv_gate"
        assert torch.equal(zf, zs), f"step {s}: keep bits differ from spkv_gate"
        assert torch.equal(fused.lengths, sep.lengths), f"step {s}: lengths differ"
        of, lf, os_, ls = (x.cpu().numpy() for x in (of, lf, os_, ls))
        assert np.all(np.isfinite(of)) and np.all(np.isfinite(lf))
        split = max(split, tl.max_abs(of, os_), tl.max_abs(lf, ls))
        zh = zf.cpu().numpy()
        for b in range(B):
            np.testing.assert_array_equal(zh[b], li.z[b][t[b]], err_msg=f"keep b={b} t={t[b]}")
            ro, rl = oracle.attention(li.Q[b][t[b]:t[b] + 1], [t[b]], li.K[b], li.V[b], li.z[b], wl.window,
                                      scale, threads=th)
            worst = max(worst, tl.max_abs(of[b], ro[0]))
            worst_l = max(worst_l, tl.max_abs(lf[b], rl[0]))
    torch.cuda.synchronize()
    assert spkv.spkv_cache_check(fused) == 0 and spkv.spkv_cache_check(sep) == 0
    for b in range(B):
        lists = oracle.compact(li.z[b][:ctxs[b] + steps], 0)
        for g in range(wl.n_kv):
            kf, vf, pf = fused.read_head(b, g)
            ks, vs, ps = sep.read_head(b, g)
            np.testing.assert_array_equal(pf.cpu().numpy(), lists[g], err_msg=f"pos b={b} g={g}")
            assert torch.equal(pf, ps) and torch.equal(kf, ks) and torch.equal(vf, vs), (b, g)
            np.testing.assert_array_equal(vf.float().cpu().numpy(), li.V[b][lists[g], g])
            rkf, rvf = fused.read_ring(b, g)
            rks, rvs = sep.read_ring(b, g)
            assert torch.equal(rkf, rks) and torch.equal(rvf, rvs), f"ring b={b} g={g}"
    # the workspace counters are settled (the next call relies on it)
    assert tl.step_counters_settled(ws_step, B, wl.n_kv)
    return worst, worst_l, split


@pytest.mark.parametrize("name,over,ctxs,steps,tau,page", [
    ("decode_32k", dict(batch=4), [700, 129, 333, 40], 40, None, 64),     # ragged, one shorter than w
    ("decode_32k", dict(batch=3, head_dim=64, n_q=16), [300, 1000, 90], 24, None, 32),  # hd 64, G 2
    ("decode_32k", dict(batch=2), [95, 31], 70, 0.0, 32),                  # keep all: page after page
    ("decode_32k", dict(batch=2), [200, 5], 20, 2.0, 32),                  # keep none
    ("decode_32k", dict(batch=16), [64 + 37 * i for i in range(16)], 6, None, 64),  # 16 sequences
    ("decode_32k", dict(batch=3, n_q=8, d_hidden=256), [400, 150, 260], 12, None, 64),  # G 1, d_hidden 256
    ("decode_32k", dict(batch=2, d_hidden=16), [300, 41], 12, None, 64),   # d_hidden 16
    ("decode_32k", dict(batch=3, window=32), [300, 20, 1000], 40, None, 64),  # one ring block
    ("decode_32k", dict(batch=2, window=96, head_dim=64, n_q=16), [500, 90], 30, None, 32),  # three
    ("decode_32k", dict(batch=2, window=256), [600, 250], 20, None, 64),   # eight
])
def test_decode_step_equals_separate_calls(name, over, ctxs, steps, tau, page):
    wl = tl.small_workload(name, **over)
    tau = wl.tau if tau is None else tau
    worst, worst_l, split = _run(wl, ctxs, steps, tau, page, seed=1201)
    print(f"[decode step {over} tau={tau} p={page}] max|dout|={worst:.2e} max|dlse|={worst_l:.2e} "
          f"max|fused - separate|={split:.2e}")
    assert worst <= tl.TOL_REGRESS and worst_l <= tl.TOL_REGRESS
    assert split <= TOL_SPLIT


def test_decode_step_shares_workspace_with_decode_attn():
    wl = tl.small_workload("decode_32k", batch=3)
    worst, worst_l, split = _run(wl, [500, 260, 77], 8, wl.tau, 64, seed=1202, shared_ws=True)
    assert worst <= tl.TOL_REGRESS and worst_l <= tl.TOL_REGRESS and split <= TOL_SPLIT


def test_decode_step_is_deterministic():
    wl = tl.small_workload("decode_32k", batch=4)
    ctxs = [900, 400, 130, 2000]
    dt = tl.torch_dtype(wl)
    li = tl.layer_inputs(wl, [c + 1 for c in ctxs], seed=1203)
    gw = tl.gate_weights(li, dt)
    B = len(ctxs)
    cache = tl.new_cache(wl, B, max(ctxs) + 1)
    tl.append(cache, [li.z[b][:ctxs[b]] for b in range(B)], [li.K[b][:ctxs[b]] for b in range(B)],
              [li.V[b][:ctxs[b]] for b in range(B)], [0] * B, G_ | W_)
    snap = cache.snapshot()
    ws = spkv.workspace(spkv.spkv_decode_step_ws_bytes(cache, gw, wl.n_q))
    td = _i32(ctxs)
    args = [tl.dev(np.stack([x[b][ctxs[b]] for b in range(B)]), dt) for x in (li.H, li.K, li.V, li.Q)]
    res = []
    for _ in range(3):
        cache.restore(snap)
        u, z, o, l = spkv.spkv_decode_step(cache, gw, args[0], wl.tau, args[1], args[2], args[3], td,
                                           tl.scale_for(wl.head_dim), ws=ws)
        res.append([x.clone() for x in (u, z, o, l, cache.lengths)])
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert torch.equal(a, b)


def test_decode_step_rejects_unsupported_shapes():
    wl = tl.small_workload("decode_32k", batch=17)
    dt = tl.torch_dtype(wl)
    li = tl.layer_inputs(wl, [10] * 17, seed=1204)
    gw = tl.gate_weights(li, dt)
    cache = tl.new_cache(wl, 17, 64)
    z = lambda *s: torch.zeros(s, dtype=dt, device="cuda")  # noqa: E731
    with pytest.raises(spkv.SpkvError) as e:
        spkv.spkv_decode_step(cache, gw, z(17, wl.d_model), wl.tau, z(17, wl.n_kv, wl.head_dim),
                              z(17, wl.n_kv, wl.head_dim), z(17, wl.n_q, wl.head_dim), _i32([9] * 17), 0.1,
                              ws=spkv.workspace(1 << 20))
    assert e.value.code == spkv.SPKV_E_UNSUPPORTED
    # too small a workspace is refused before any launch
    wl2 = tl.small_workload("decode_32k", batch=2)
    cache2 = tl.new_cache(wl2, 2, 64)
    need = spkv.spkv_decode_step_ws_bytes(cache2, gw, wl2.n_q)
    with pytest.raises(spkv.SpkvError) as e:
        spkv.spkv_decode_step(cache2, gw, z(2, wl.d_model), wl.tau, z(2, wl.n_kv, wl.head_dim),
                              z(2, wl.n_kv, wl.head_dim), z(2, wl.n_q, wl.head_dim), _i32([9, 9]), 0.1,
                              ws=spkv.workspace(need - 256))
    assert e.value.code == spkv.SPKV_E_WORKSPACE


def test_decode_step_capacity_overflow_matches_separate_calls():
    """A pool too small for the kept rows: both paths drop the same rows and flag it."""
    wl = tl.small_workload("decode_32k", batch=2)
    B, ctxs, steps = 2, [40, 60], 40
    dt = tl.torch_dtype(wl)
    li = tl.layer_inputs(wl, [c + steps for c in ctxs], seed=1205)
    gw = tl.gate_weights(li, dt)
    P = 32
    # every pair kept (tau = 0): each head needs 3 pages by the end; give the
    # pool 2 per head, so the pool runs out part-way
    mk = lambda: spkv.Cache(B, wl.n_kv, wl.head_dim, wl.window, P, 2 * B * wl.n_kv, 4, dt)  # noqa: E731
    fused, sep = mk(), mk()
    ws = spkv.workspace(spkv.spkv_decode_step_ws_bytes(fused, gw, wl.n_q))
    ro1 = _i32(np.arange(B + 1))
    for cache in (fused, sep):
        tl.append(cache, [np.ones((ctxs[b], wl.n_kv), np.uint8) for b in range(B)],
                  [li.K[b][:ctxs[b]] for b in range(B)], [li.V[b][:ctxs[b]] for b in range(B)], [0] * B, G_ | W_)
    for s in range(steps):
        t = [ctxs[b] + s for b in range(B)]
        td = _i32(t)
        h, k, v, q = (tl.dev(np.stack([x[b][t[b]] for b in range(B)]), dt) for x in (li.H, li.K, li.V, li.Q))
        spkv.spkv_decode_step(fused, gw, h, 0.0, k, v, q, td, 0.125, ws=ws)
        _, zs = spkv.spkv_gate(gw, h, 0.0)
        spkv.spkv_compact_append(sep, zs, k, v, ro1, td, 1, G_ | W_)
    torch.cuda.synchronize()
    assert int(fused.status.item()) & spkv.STATUS_POOL_FULL
    assert int(sep.status.item()) & spkv.STATUS_POOL_FULL
    # the total kept is bounded by the pool; each head's content is a prefix
    # of its keep-all list (dropped rows never leave a hole)
    assert torch.equal(fused.lengths, sep.lengths)
    assert int(fused.lengths.sum()) <= 2 * B * wl.n_kv * P
    for b in range(B):
        for g in range(wl.n_kv):
            _, _, pos = fused.read_head(b, g)
            n = pos.numel()
            np.testing.assert_array_equal(pos.cpu().numpy(), np.arange(n))


@pytest.mark.parametrize("B,hd,nq,w", [(32, 128, 32, 128), (3, 64, 16, 128), (4, 128, 32, 32), (3, 64, 16, 96)])
def test_ring_only_step_equals_window_append_plus_attn(B, hd, nq, w):
    """spkv_decode_step without a gate: the ring write and the attention of
    the separate calls, bit for bit (same kernel plan), any batch size."""
    wl = tl.small_workload("decode_32k", batch=B, head_dim=hd, n_q=nq, window=w)
    ctxs = [100 + 53 * b for b in range(B)]
    steps = 5
    dt = tl.torch_dtype(wl)
    li = tl.layer_inputs(wl, [c + steps for c in ctxs], seed=1206)
    caches = [tl.new_cache(wl, B, max(ctxs) + steps) for _ in range(2)]
    for cache in caches:
        tl.append(cache, [li.z[b][:ctxs[b]] for b in range(B)], [li.K[b][:ctxs[b]] for b in range(B)],
                  [li.V[b][:ctxs[b]] for b in range(B)], [0] * B, G_ | W_)
    one, sep = caches
    ws1 = spkv.workspace(spkv.spkv_decode_step_ws_bytes(one, None, wl.n_q))
    ws2 = spkv.workspace(spkv.spkv_decode_ws_bytes(sep, wl.n_q))
    ro1 = _i32(np.arange(B + 1))
    scale = tl.scale_for(wl.head_dim)
    for s in range(steps):
        t = [ctxs[b] + s for b in range(B)]
        td = _i32(t)
        k, v, q = (tl.dev(np.stack([x[b][t[b]] for b in range(B)]), dt) for x in (li.K, li.V, li.Q))
        u1, z1, o1, l1 = spkv.spkv_decode_step(one, None, None, 0.0, k, v, q, td, scale, ws=ws1)
        assert u1 is None and z1 is None
        spkv.spkv_compact_append(sep, None, k, v, ro1, td, 1, W_)
        o2, l2 = spkv.spkv_decode_attn(sep, q, td, scale, ws=ws2)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"step {s}"
        # every sequence's output against the oracle (window + kept before the window)
        oh = o1.cpu().numpy()
        for b in (0, B - 1):
            ro, _ = oracle.attention(li.Q[b][t[b]:t[b] + 1], [t[b]], li.K[b], li.V[b], li.z[b], wl.window, scale,
                                     threads=tl.oracle_threads())
            assert tl.max_abs(oh[b], ro[0]) <= tl.TOL_REGRESS
    torch.cuda.synchronize()
    assert torch.equal(one.lengths, sep.lengths)
    assert torch.equal(one.ring_k, sep.ring_k) and torch.equal(one.ring_v, sep.ring_v)
    assert spkv.spkv_cache_check(one) == 0


def test_decode_step_recovers_after_timeout():
    """A step whose finisher's waits give up at once (wait limit 0) sets the
    timeout bit and stores no append and no lengths; the same workspace then
    serves the next steps without a new zero fill, with results equal bit for
    bit to those of a fresh workspace."""
    wl = tl.small_workload("decode_32k", batch=3)
    ctxs = [700, 260, 1500]
    steps = 3
    dt = tl.torch_dtype(wl)
    li = tl.layer_inputs(wl, [c + steps for c in ctxs], seed=1205)
    gw = tl.gate_weights(li, dt)
    B = len(ctxs)
    cache = tl.new_cache(wl, B, max(ctxs) + steps)
    tl.append(cache, [li.z[b][:ctxs[b]] for b in range(B)], [li.K[b][:ctxs[b]] for b in range(B)],
              [li.V[b][:ctxs[b]] for b in range(B)], [0] * B, G_ | W_)
    snap = cache.snapshot()
    scale = tl.scale_for(wl.head_dim)
    nbytes = spkv.spkv_decode_step_ws_bytes(cache, gw, wl.n_q)

    def step_args(s):
        t = [c + s for c in ctxs]
        return [tl.dev(np.stack([x[b][t[b]] for b in range(B)]), dt) for x in (li.H, li.K, li.V, li.Q)], _i32(t)

    def run_steps(ws):
        res = []
        for s in range(steps):
            (h, k, v, q), td = step_args(s)
            u, z, o, l = spkv.spkv_decode_step(cache, gw, h, wl.tau, k, v, q, td, scale, ws=ws)
            torch.cuda.synchronize()
            assert int(cache.status.item()) == 0
            res.append([x.clone() for x in (u, z, o, l, cache.lengths)])
        return res

    ref = run_steps(spkv.workspace(nbytes))
    cache.restore(snap)
    ws = spkv.workspace(nbytes)
    lengths0 = cache.lengths.clone()
    (h, k, v, q), td = step_args(0)
    spkv.spkv_set_wait_limit(0)
    try:
        spkv.spkv_decode_step(cache, gw, h, wl.tau, k, v, q, td, scale, ws=ws)
        torch.cuda.synchronize()
    finally:
        spkv.spkv_set_wait_limit(-1)
    assert int(cache.status.item()) & spkv.STATUS_STEP_TIMEOUT
    assert torch.equal(cache.lengths, lengths0), "a timed-out step stored lengths"
    assert tl.step_counters_settled(ws, B, wl.n_kv)
    cache.restore(snap)
    got = run_steps(ws)
    for s in range(steps):
        for name, a, b in zip(("utility", "keep", "out", "lse", "lengths"), ref[s], got[s]):
            assert torch.equal(a, b), f"step {s}: {name} differs after the timeout"
    assert tl.step_counters_settled(ws, B, wl.n_kv)
