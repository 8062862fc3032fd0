"""GPU parity of spkv_prefill_attn_soft (the soft relaxation of SP-KV
section 2.1, Eq. 5-6) against the oracle's direct evaluation (O7).

Every token of the sequence enters the cache (keep = 1) with its utility, so
the kernel's cached keys are all causal keys outside the window and each
carries the additive score c (alpha - 1); window keys carry none.  Chunked
as spkv_prefill_attn is: GLOBAL append, attention, WINDOW append.  The
tolerance is the prefill one (attention weights rounded to bf16 before the
value product); utilities come from the seeded generator (NaN replaced: the
soft mask is defined for finite utilities).
"""
import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW


def _i32(x):
    return torch.tensor(np.asarray(x, np.int32), device="cuda")


def _run(T, hd, P, chunk, w, tau, beta, c, nkv=2, G=4, seed=4):
    nq = nkv * G
    Q = inputs.normal((T, nq, hd), seed, 1, dtype="bf16")
    K = inputs.normal((T, nkv, hd), seed, 2, dtype="bf16")
    V = inputs.normal((T, nkv, hd), seed, 3, dtype="bf16")
    u = inputs.utilities(T, nkv, seed, 4)
    u[np.isnan(u)] = np.float32(0.3)
    per_head = (T + P - 1) // P + 1
    cache = spkv.Cache(1, nkv, hd, w, P, nkv * per_head, per_head, torch.bfloat16, utilities=True)
    scale = tl.scale_for(hd)
    out = np.zeros((T, nq, hd), np.float32)
    lse = np.zeros((T, nq), np.float32)
    for p0 in range(0, T, chunk):
        n = min(chunk, T - p0)
        kd = tl.dev(K[p0:p0 + n], torch.bfloat16)
        vd = tl.dev(V[p0:p0 + n], torch.bfloat16)
        ro, pz = _i32([0, n]), _i32([p0])
        keep = torch.ones((n, nkv), dtype=torch.uint8, device="cuda")
        spkv.spkv_compact_append(cache, keep, kd, vd, ro, pz, n, G_, utility=tl.dev(u[p0:p0 + n]))
        o, l = spkv.spkv_prefill_attn(cache, 0, tl.dev(Q[p0:p0 + n], torch.bfloat16), kd, vd, p0, scale,
                                      soft=(tau, beta, c))
        spkv.spkv_compact_append(cache, None, kd, vd, ro, pz, n, W_)
        out[p0:p0 + n], lse[p0:p0 + n] = o.cpu().numpy(), l.cpu().numpy()
    torch.cuda.synchronize()
    assert spkv.spkv_cache_check(cache) == 0
    ro_, rl = oracle.soft_attention(Q, np.arange(T), K, V, u, w, tau, beta, c, scale, threads=tl.oracle_threads())
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    return tl.max_abs(out, ro_), tl.max_abs(lse, rl)


@pytest.mark.parametrize("hd,P,chunk,w,beta,c", [
    (128, 64, 500, 128, 0.01, 1e6),    # the pages' constants
    (64, 32, 1100, 64, 0.01, 1e6),
    (128, 256, 700, 128, 0.1, 10.0),   # a mild mask: every cached key weighs in
    (128, 64, 333, 32, 0.05, 4.0),
])
def test_soft_prefill_matches_oracle(hd, P, chunk, w, beta, c):
    err_o, err_l = _run(1100, hd, P, chunk, w, 0.5, beta, c)
    print(f"[soft hd={hd} P={P} chunk={chunk} w={w} beta={beta} c={c}] max|dout|={err_o:.2e} max|dlse|={err_l:.2e}")
    assert err_o < tl.TOL_PREFILL, err_o
    # the normaliser is summed in f32 from f32 weights, as on the hard path
    assert err_l < tl.TOL_REGRESS, err_l


def test_soft_prefill_arguments():
    cache = spkv.Cache(1, 2, 128, 128, 64, 8, 4, torch.bfloat16, utilities=False)
    q = torch.zeros((4, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(spkv.SpkvError):  # no stored utilities
        spkv.spkv_prefill_attn(cache, 0, q, k, k, 0, 0.1, soft=(0.5, 0.01, 1e6))
    cache = spkv.Cache(1, 2, 128, 128, 64, 8, 4, torch.bfloat16, utilities=True)
    for bad in ((0.5, 0.0, 1e6), (0.5, 0.01, -1.0), (float("nan"), 0.01, 1.0), (0.5, float("inf"), 1.0),
                (0.5, 1e-45, 1.0), (0.5, 0.01, 3e38)):
        with pytest.raises(spkv.SpkvError):
            spkv.spkv_prefill_attn(cache, 0, q, k, k, 0, 0.1, soft=bad)


@pytest.mark.parametrize("nkv, G", [(3, 16), (5, 2)])
def test_soft_prefill_key_heads_not_dividing_8(nkv, G):
    # key-head counts that do not divide 8, with the widest and a small group
    err_o, err_l = _run(700, 128, 64, 300, 64, 0.5, 0.01, 1e6, nkv=nkv, G=G, seed=9)
    print(f"[soft nkv={nkv} G={G}] max|dout|={err_o:.2e} max|dlse|={err_l:.2e}")
    assert err_o < tl.TOL_PREFILL, err_o
    assert err_l < tl.TOL_REGRESS, err_l
