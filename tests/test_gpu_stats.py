"""GPU parity of spkv_head_stats against the oracle's per-head sums (O6).

SP-KV (arXiv 2605.14037) reports density as the share of pairs outside the
window that are kept (Table 1 caption) and ranks heads by mean utility to
choose global heads (section 4).  Kept counts must be exact; utility sums are
fp64 sums of f32 values taken in another order than the oracle's, so they
agree to rounding (relative 1e-12 here, far below any use of the figure) and
are bit-identical from run to run.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv

pytestmark = pytest.mark.gpu


def _inputs(n, nkv, seed):
    u = inputs.utilities(n, nkv, seed, 0)
    u[np.isnan(u)] = np.float32(0.125)  # NaN is covered separately
    z = inputs.bernoulli_mask(n, [0.05 + 0.1 * g for g in range(nkv)], seed, 1)
    return u, z


@pytest.mark.parametrize("n,nkv", [(0, 8), (1, 1), (300, 3), (4097, 8), (100003, 16), (262144, 8)])
def test_head_stats_parity(n, nkv):
    u, z = _inputs(n, nkv, 7 + n)
    us, kp = spkv.spkv_head_stats(torch.from_numpy(u).cuda(), torch.from_numpy(z).cuda())
    ru, rk = oracle.head_stats(u, z)
    np.testing.assert_array_equal(kp.cpu().numpy(), rk)
    np.testing.assert_allclose(us.cpu().numpy(), ru, rtol=1e-12, atol=0)
    # deterministic: a second call gives the same bits
    us2, kp2 = spkv.spkv_head_stats(torch.from_numpy(u).cuda(), torch.from_numpy(z).cuda())
    assert torch.equal(us, us2) and torch.equal(kp, kp2)


def test_head_stats_accumulates_and_halves():
    n, nkv = 50000, 8
    u, z = _inputs(n, nkv, 3)
    ud, zd = torch.from_numpy(u).cuda(), torch.from_numpy(z).cuda()
    us = torch.zeros(nkv, dtype=torch.float64, device="cuda")
    kp = torch.zeros(nkv, dtype=torch.int64, device="cuda")
    ru, rk = None, None
    for lo, hi in ((0, 16384), (16384, 16385), (16385, 40000), (40000, n)):
        spkv.spkv_head_stats(ud[lo:hi], zd[lo:hi], us, kp)
        ru, rk = oracle.head_stats(u[lo:hi], z[lo:hi], ru, rk)
    np.testing.assert_array_equal(kp.cpu().numpy(), rk)
    np.testing.assert_allclose(us.cpu().numpy(), ru, rtol=1e-12)
    # only one half given: the other accumulator is left alone
    only_u, none_k = spkv.spkv_head_stats(ud, None)
    assert none_k is None
    np.testing.assert_allclose(only_u.cpu().numpy(), oracle.head_stats(u, None)[0], rtol=1e-12)
    none_u, only_k = spkv.spkv_head_stats(None, zd)
    assert none_u is None
    np.testing.assert_array_equal(only_k.cpu().numpy(), np.count_nonzero(z, axis=0))


def test_head_stats_nan_and_errors():
    u = np.full((1000, 2), 0.5, np.float32)
    u[777, 1] = np.nan
    us, _ = spkv.spkv_head_stats(torch.from_numpy(u).cuda(), None)
    us = us.cpu().numpy()
    assert us[0] == 500.0 and math.isnan(us[1])
    with pytest.raises(spkv.SpkvError):
        spkv.spkv_head_stats(torch.zeros((4, 17), device="cuda"), None)  # n_kv > 16
    lib = spkv.load_library()
    assert lib.spkv_head_stats(None, None, 4, 2, None, None, None, 0, None) == spkv.SPKV_E_INVALID
    assert lib.spkv_head_stats(None, None, 0, 2, None, None, None, 0, None) == spkv.SPKV_OK
    x = torch.zeros((4, 2), device="cuda")
    assert lib.spkv_head_stats(x.data_ptr(), None, 4, 2, None, None, None, 0, None) == spkv.SPKV_E_INVALID


def test_head_stats_unaligned_rows_take_the_row_path():
    # a view starting one row in (8 bytes for two heads) is not 16-byte
    # aligned: the row-per-thread path runs; it must agree as well
    n, nkv = 5001, 2
    u, z = _inputs(n, nkv, 11)
    ud, zd = torch.from_numpy(u).cuda(), torch.from_numpy(z).cuda()
    us, kp = spkv.spkv_head_stats(ud[1:], zd[1:])
    ru, rk = oracle.head_stats(u[1:], z[1:])
    np.testing.assert_array_equal(kp.cpu().numpy(), rk)
    np.testing.assert_allclose(us.cpu().numpy(), ru, rtol=1e-12)


def test_head_stats_one_workspace_across_calls():
    # one workspace shared by calls of both paths and many sizes: each call
    # leaves its arrival counter at zero for the next, and every result equals
    # that of a fresh workspace bit for bit
    sizes = [(262144, 8), (300, 3), (4097, 8), (1, 1), (100003, 16), (5000, 2)]
    ws = spkv.workspace(max(spkv.spkv_head_stats_ws_bytes(n, k) for n, k in sizes))
    for i, (n, nkv) in enumerate(sizes):
        u, z = _inputs(n, nkv, 40 + i)
        ud, zd = torch.from_numpy(u).cuda(), torch.from_numpy(z).cuda()
        if i == 5:  # a view one row in: the row path
            ud, zd = ud[1:], zd[1:]
        a = spkv.spkv_head_stats(ud, zd, ws=ws)
        b = spkv.spkv_head_stats(ud, zd)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (n, nkv)
    assert not ws[:4352 // 4].any()  # the counter header is back at zero
