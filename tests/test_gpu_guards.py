"""Guard canaries: no call writes outside the buffers it is given.

Every buffer of the caches (key, value, position and utility pages, page
table, lengths, pool counter, status, rings), the workspaces and the outputs
sit between runs of canary bytes.  The pool and the page tables are sized to
exactly what the appends need, so that the last page of the pool and the last
slot of a page table are written -- where an overrun would land first.  After
chunked prefill (kept append, prefill attention, window append), decode steps
through both entry points and a re-threshold into a second guarded cache,
every canary must be intact and the status clean.
"""
import math

import numpy as np
import pytest
import torch

from learned_kv_cache_sp_amd import inputs, spkv

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW
GUARD = 4096
CANARY = spkv.Cache.GUARD_BYTE


def guarded(shape, dtype, fill=0):
    """A device tensor between two GUARD-byte canary runs; returns (tensor, checker)."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    body = (n + 255) // 256 * 256
    raw = torch.full((GUARD + body + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
    t = raw[GUARD:GUARD + n].view(dtype).view(shape)
    t.fill_(fill)

    def intact():
        return not bool((torch.cat([raw[:GUARD], raw[GUARD + n:]]) != CANARY).any())
    return t, intact


@pytest.mark.parametrize("hd, page", [(128, 32), (64, 64)])
def test_guards_intact(hd, page):
    B, nkv, nq, w, d, dh = 3, 2, 8, 32, 256, 32
    tau = 0.5
    ctx = [300, 517, 64]          # prefill lengths (two chunks each)
    steps = 5                     # decode steps after the prefill
    T = [c + steps for c in ctx]
    seed = 31
    K = [inputs.device_normal((T[b], nkv, hd), seed, 10 + b, torch.bfloat16) for b in range(B)]
    V = [inputs.device_normal((T[b], nkv, hd), seed, 20 + b, torch.bfloat16) for b in range(B)]
    Q = [inputs.device_normal((T[b], nq, hd), seed, 30 + b, torch.bfloat16) for b in range(B)]
    Z = [inputs.device_bernoulli_mask(T[b], (0.4, 0.7), seed, 40 + b) for b in range(B)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    U = [torch.rand((T[b], nkv), generator=gen, device="cuda") for b in range(B)]
    # decode steps 0..2 go through spkv_compact_append + spkv_decode_attn with
    # the drawn bits; steps 3..4 through spkv_decode_step with a gate that
    # keeps every pair (output bias +40), so every kept count is known
    for b in range(B):
        Z[b][ctx[b] + 3:] = 1
    counts = [[int(Z[b][:, g].sum()) for g in range(nkv)] for b in range(B)]
    per_head = [[-(-c // page) for c in cb] for cb in counts]
    n_pages = sum(sum(p) for p in per_head)
    max_pages = max(max(p) for p in per_head)
    cache = spkv.Cache(B, nkv, hd, w, page, n_pages, max_pages, torch.bfloat16, utilities=True, guard=GUARD)
    scale = 1.0 / math.sqrt(hd)
    checks = []

    # ---- chunked prefill, sequence by sequence ----------------------------
    for b in range(B):
        c0 = 0
        for n in (ctx[b] // 2, ctx[b] - ctx[b] // 2):
            sl = slice(c0, c0 + n)
            ro = torch.tensor([0] * b + [0, n] + [n] * (B - 1 - b), dtype=torch.int32, device="cuda")
            p0 = torch.full((B,), c0, dtype=torch.int32, device="cuda")
            cws, cws_ok = guarded((spkv.spkv_compact_ws_bytes(cache, n, n) // 4 + 1,), torch.int32)
            spkv.spkv_compact_append(cache, Z[b][sl], K[b][sl], V[b][sl], ro, p0, n, G_, ws=cws, utility=U[b][sl])
            out, out_ok = guarded((n, nq, hd), torch.float32)
            lse, lse_ok = guarded((n, nq), torch.float32)
            pws, pws_ok = guarded((max(1, spkv.spkv_prefill_ws_bytes(cache, nq, n) // 4 + 1),), torch.int32)
            spkv.spkv_prefill_attn(cache, b, Q[b][sl], K[b][sl], V[b][sl], c0, scale, out=out, lse=lse, ws=pws)
            spkv.spkv_compact_append(cache, None, K[b][sl], V[b][sl], ro, p0, n, W_, ws=cws)
            checks += [("compact ws", cws_ok), ("prefill out", out_ok), ("prefill lse", lse_ok),
                       ("prefill ws", pws_ok)]
            c0 += n
    torch.cuda.synchronize()
    assert cache.check_guards() == []

    # ---- decode: three separate steps, then two fused steps ----------------
    ro1 = torch.arange(0, B + 1, dtype=torch.int32, device="cuda")
    dws, dws_ok = guarded((spkv.spkv_decode_ws_bytes(cache, nq) // 4 + 1,), torch.int32)
    gen_w = np.random.default_rng(seed)
    W1 = torch.from_numpy((gen_w.standard_normal((dh, d)) * 0.05).astype(np.float32)).cuda().to(torch.bfloat16)
    gw = spkv.GateWeights(W1, torch.zeros(dh, device="cuda"), torch.zeros(nkv, dh, device="cuda"),
                          torch.full((nkv,), 40.0, device="cuda"))
    fws, fws_ok = guarded((spkv.spkv_decode_step_ws_bytes(cache, gw, nq) // 4 + 1,), torch.int32)
    H = inputs.device_normal((steps, B, d), seed, 50, torch.bfloat16)
    for s in range(steps):
        t = torch.tensor([ctx[b] + s for b in range(B)], dtype=torch.int32, device="cuda")
        ks = torch.stack([K[b][ctx[b] + s] for b in range(B)])
        vs = torch.stack([V[b][ctx[b] + s] for b in range(B)])
        qs = torch.stack([Q[b][ctx[b] + s] for b in range(B)])
        out, out_ok = guarded((B, nq, hd), torch.float32)
        lse, lse_ok = guarded((B, nq), torch.float32)
        if s < 3:
            zs = torch.stack([Z[b][ctx[b] + s] for b in range(B)])
            us = torch.stack([U[b][ctx[b] + s] for b in range(B)])
            spkv.spkv_compact_append(cache, zs, ks, vs, ro1, t, 1, G_ | W_, utility=us)
            spkv.spkv_decode_attn(cache, qs, t, scale, out=out, lse=lse, ws=dws)
        else:
            keep, keep_ok = guarded((B, nkv), torch.uint8)
            util, util_ok = guarded((B, nkv), torch.float32)
            spkv.spkv_decode_step(cache, gw, H[s], tau, ks, vs, qs, t, scale, utility=util, keep=keep, out=out,
                                  lse=lse, ws=fws)
            checks += [("step keep", keep_ok), ("step utility", util_ok)]
            torch.cuda.synchronize()
            assert bool((keep == 1).all())
        checks += [("decode out", out_ok), ("decode lse", lse_ok)]
    torch.cuda.synchronize()
    assert spkv.spkv_cache_check(cache) == 0
    assert cache.check_guards() == []
    np.testing.assert_array_equal(cache.lengths.cpu().numpy(), np.array(counts))
    assert int(cache.pool_next.item()) == n_pages      # the pool is used to its last page

    # ---- re-threshold into a second guarded cache of the same exact size ---
    dst = spkv.Cache(B, nkv, hd, w, page, n_pages, max_pages, torch.bfloat16, utilities=True, guard=GUARD)
    dst.share_ring(cache)
    rws, rws_ok = guarded((spkv.spkv_rethreshold_ws_bytes(cache) // 4 + 1,), torch.int32)
    spkv.spkv_cache_rethreshold(cache, dst, 0.3, ws=rws)
    torch.cuda.synchronize()
    checks.append(("rethreshold ws", rws_ok))
    assert spkv.spkv_cache_check(dst) == 0
    assert dst.check_guards() == []
    assert cache.check_guards() == []
    spkv.spkv_cache_reset(dst)
    torch.cuda.synchronize()
    assert dst.check_guards() == []
    bad = [name for name, ok in checks if not ok()]
    assert bad == [], f"canaries overwritten around: {bad}"
