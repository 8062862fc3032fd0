"""GPU parity of spkv_compact_append against the oracle's stable filter.

The logical content of every (sequence, key head) -- positions, key rows and
value rows in order -- must equal the oracle's list exactly; physical page
ids are not compared.  Also: the window ring, append offsets, capacity and
row-offset errors.
"""
import numpy as np
import pytest
import torch

import oracle
from learned_kv_cache_sp_amd import inputs, spkv
import spkv_testlib as tl

pytestmark = pytest.mark.gpu

G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW


def _seq_data(wl, T, b, seed, rates):
    tok = inputs.tokens(wl, T, seed, b)
    z = inputs.bernoulli_mask(T, rates, seed, b)
    return tok["K"], tok["V"], z


def _check_cache(cache, wl, K, V, Z, lengths_done):
    for b, T in enumerate(lengths_done):
        lists = oracle.compact(Z[b][:T], 0)
        for g in range(wl.n_kv):
            k, v, pos = cache.read_head(b, g)
            ref = lists[g]
            np.testing.assert_array_equal(pos.cpu().numpy(), ref, err_msg=f"pos b={b} g={g}")
            np.testing.assert_array_equal(k.float().cpu().numpy(), K[b][ref, g], err_msg=f"K b={b} g={g}")
            np.testing.assert_array_equal(v.float().cpu().numpy(), V[b][ref, g], err_msg=f"V b={b} g={g}")


@pytest.mark.parametrize("name,page", [("decode_32k", 64), ("tiny", 32), ("decode_32k", 256)])
def test_compaction_incremental_and_chunked(name, page):
    wl = inputs.WORKLOADS[name]
    B = 3
    rates = np.linspace(0.0, 1.0, wl.n_kv)  # includes never-kept and always-kept heads
    T = [1500, 777, 2100]
    K, V, Z = zip(*[_seq_data(wl, T[b], b, 21, rates) for b in range(B)])
    cache = tl.new_cache(wl, B, max(T), page_size=page)
    done = [0] * B
    # appends of mixed sizes: large (several tiles), small, single rows, empty
    schedule = [[600, 0, 1000], [1, 1, 1], [255, 300, 0], [0, 1, 1], [644, 475, 1098]]
    for step in schedule:
        rz, rk, rv, p0 = [], [], [], []
        for b in range(B):
            n = min(step[b], T[b] - done[b])
            sl = slice(done[b], done[b] + n)
            rz.append(Z[b][sl] if n else None)
            rk.append(K[b][sl] if n else None)
            rv.append(V[b][sl] if n else None)
            p0.append(done[b])
            done[b] += n
        ao = torch.full((B, wl.n_kv), -7, dtype=torch.int32, device="cuda")
        before = cache.lengths.clone()
        tl.append(cache, rz, rk, rv, p0, G_ | W_, append_offsets=ao)
        torch.cuda.synchronize()
        assert torch.equal(ao, before)
    assert done == T
    assert spkv.spkv_cache_check(cache) == 0
    _check_cache(cache, wl, K, V, Z, T)
    # lengths = popcounts
    for b in range(B):
        np.testing.assert_array_equal(cache.lengths[b].cpu().numpy(), Z[b].sum(0))
    # ring: slot p % w holds position p for the last w positions
    w = wl.window
    for b in range(B):
        rk, rv = cache.read_ring(b, 0)
        for p in range(T[b] - w, T[b]):
            for g in range(wl.n_kv):
                rk_, rv_ = cache.read_ring(b, g)
                np.testing.assert_array_equal(rk_[p % w].float().cpu().numpy(), K[b][p, g])
                np.testing.assert_array_equal(rv_[p % w].float().cpu().numpy(), V[b][p, g])


def test_compaction_window_only_and_global_only():
    wl = inputs.WORKLOADS["decode_32k"]
    K, V, Z = _seq_data(wl, 700, 0, 5, [0.3] * 8)
    cache = tl.new_cache(wl, 1, 700)
    tl.append(cache, None, [K[:400]], [V[:400]], [0], W_)
    torch.cuda.synchronize()
    assert int(cache.lengths.sum()) == 0
    tl.append(cache, [Z], [K], [V], [0], G_)
    tl.append(cache, None, [K[400:]], [V[400:]], [400], W_)
    torch.cuda.synchronize()
    _check_cache(cache, wl, [K], [V], [Z], [700])
    rk, rv = cache.read_ring(0, 3)
    for p in range(700 - 128, 700):
        np.testing.assert_array_equal(rk[p % 128].float().cpu().numpy(), K[p, 3])


def test_compaction_is_deterministic_in_logical_content():
    wl = inputs.WORKLOADS["decode_32k"]
    B = 4
    data = [_seq_data(wl, 3000, b, 9, [0.5] * 8) for b in range(B)]
    caches = []
    for _ in range(2):
        c = tl.new_cache(wl, B, 3000)
        tl.append(c, [d[2] for d in data], [d[0] for d in data], [d[1] for d in data], [0] * B, G_ | W_)
        caches.append(c)
    torch.cuda.synchronize()
    for b in range(B):
        for g in range(wl.n_kv):
            a = caches[0].read_head(b, g)
            c = caches[1].read_head(b, g)
            for x, y in zip(a, c):
                assert torch.equal(x, y)


def test_capacity_overflow_is_flagged():
    wl = inputs.WORKLOADS["decode_32k"]
    K, V, Z = _seq_data(wl, 2000, 0, 11, [1.0] * 8)
    from learned_kv_cache_sp_amd.spkv import Cache
    cache = Cache(1, wl.n_kv, wl.head_dim, wl.window, 64, n_pages=40, max_pages_per_head=32,
                  dtype=torch.bfloat16)
    tl.append(cache, [Z], [K], [V], [0], G_)
    torch.cuda.synchronize()
    with pytest.raises(spkv.SpkvError) as ei:
        spkv.spkv_cache_check(cache)
    assert ei.value.code == spkv.SPKV_E_CAPACITY
    lens = cache.lengths[0].cpu().numpy()
    assert lens.sum() <= 40 * 64 and np.all(lens <= 32 * 64)
    # what was kept is still an exact prefix of the oracle list
    for g in range(wl.n_kv):
        k, v, pos = cache.read_head(0, g)
        ref = oracle.compact(Z, 0)[g][: len(pos)]
        np.testing.assert_array_equal(pos.cpu().numpy(), ref)
        np.testing.assert_array_equal(k.float().cpu().numpy(), K[ref, g])


@pytest.mark.parametrize("window,rows", [(128, 3000), (512, 2000), (1024, 1500), (1024, 700)])
def test_window_only_appends_of_long_chunks(window, rows):
    # window-only appends of more rows than one tile, windows longer than a
    # tile: the ring holds exactly the last `window` positions of each sequence
    import dataclasses
    wl = dataclasses.replace(inputs.WORKLOADS["decode_32k"], window=window)
    B = 2
    data = [_seq_data(wl, rows + 37 * b, b, 13, [0.3] * 8) for b in range(B)]
    cache = tl.new_cache(wl, B, rows + 37 * B)
    n = [rows + 37 * b for b in range(B)]
    tl.append(cache, None, [data[b][0][:n[b]] for b in range(B)], [data[b][1][:n[b]] for b in range(B)],
              [0] * B, W_)
    torch.cuda.synchronize()
    assert spkv.spkv_cache_check(cache) == 0
    assert int(cache.lengths.sum()) == 0
    for b in range(B):
        K, V, _ = data[b]
        for g in (0, 5):
            rk, rv = cache.read_ring(b, g)
            rk, rv = rk.float().cpu().numpy(), rv.float().cpu().numpy()
            for p in range(max(0, n[b] - window), n[b]):
                np.testing.assert_array_equal(rk[p % window], K[p, g])
                np.testing.assert_array_equal(rv[p % window], V[p, g])


def test_negative_positions_are_flagged():
    wl = inputs.WORKLOADS["decode_32k"]
    K, V, Z = _seq_data(wl, 300, 0, 14, [0.5] * 8)
    cache = tl.new_cache(wl, 2, 300)
    kd, vd, keep = tl.dev(K, torch.bfloat16), tl.dev(V, torch.bfloat16), tl.dev(Z)
    for ro_, p0_, mr in (([0, 1, 2], [-5, 7], 1), ([0, 120, 300], [-1, 0], 180), ([0, 150, 300], [0, -3], 150),
                         ([0, 290, 300], [-2, 0], 290)):
        cache = tl.new_cache(wl, 2, 300)
        spkv.spkv_compact_append(cache, keep, kd, vd, tl.dev(np.array(ro_, np.int32)),
                                 tl.dev(np.array(p0_, np.int32)), mr, G_ | W_)
        torch.cuda.synchronize()
        with pytest.raises(spkv.SpkvError) as ei:
            spkv.spkv_cache_check(cache)
        assert ei.value.code == spkv.SPKV_E_ROWS
        bad = 0 if p0_[0] < 0 else 1
        assert int(cache.lengths[bad].sum()) == 0  # the sequence with a negative position was skipped


def test_bad_row_offsets_are_flagged():
    wl = inputs.WORKLOADS["decode_32k"]
    K, V, Z = _seq_data(wl, 300, 0, 12, [0.5] * 8)
    cache = tl.new_cache(wl, 2, 300)
    kd, vd = tl.dev(K, torch.bfloat16), tl.dev(V, torch.bfloat16)
    keep = tl.dev(Z)
    ro = tl.dev(np.array([0, 200, 300], np.int32))
    p0 = tl.dev(np.array([0, 0], np.int32))
    # max_rows_per_seq = 150 < 200 rows of sequence 0
    spkv.spkv_compact_append(cache, keep, kd, vd, ro, p0, 150, G_)
    torch.cuda.synchronize()
    with pytest.raises(spkv.SpkvError) as ei:
        spkv.spkv_cache_check(cache)
    assert ei.value.code == spkv.SPKV_E_ROWS
    assert int(cache.lengths[0].sum()) == 0  # the bad sequence was skipped
    ref = oracle.compact(Z[200:], 0)
    for g in range(wl.n_kv):
        assert int(cache.lengths[1, g]) == len(ref[g])


def test_host_side_argument_errors():
    wl = inputs.WORKLOADS["decode_32k"]
    cache = tl.new_cache(wl, 1, 100)
    k = torch.zeros((10, 8, 128), dtype=torch.bfloat16, device="cuda")
    ro = torch.tensor([0, 10], dtype=torch.int32, device="cuda")
    p0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(spkv.SpkvError) as ei:
        spkv.spkv_compact_append(cache, None, k, k, ro, p0, 10, G_)  # keep missing
    assert ei.value.code == spkv.SPKV_E_INVALID
    with pytest.raises(spkv.SpkvError) as ei:
        spkv.spkv_compact_append(cache, None, k, k, ro, p0, 10, 8)  # unknown flag
    assert ei.value.code == spkv.SPKV_E_INVALID
    bad = spkv.Cache(1, 8, 96, 128, 64, 4, 4, torch.bfloat16)
    with pytest.raises(spkv.SpkvError) as ei:
        spkv.spkv_compact_append(bad, None, k, k, ro, p0, 10, W_)
    assert ei.value.code in (spkv.SPKV_E_UNSUPPORTED, spkv.SPKV_E_INVALID)


@pytest.mark.parametrize("name,page", [("decode_32k", 64), ("tiny", 32)])
def test_one_row_appends(name, page):
    # decode-style appends: at most one row per sequence per call, with page
    # boundaries crossed many times and sequences that sit out some calls
    wl = inputs.WORKLOADS[name]
    B = 3
    rates = [0.0, 1.0] + [0.4] * (wl.n_kv - 2)
    T = [300, 70, 200]
    K, V, Z = zip(*[_seq_data(wl, T[b], b, 31, rates) for b in range(B)])
    cache = tl.new_cache(wl, B, max(T), page_size=page)
    done = [0] * B
    step = 0
    while any(done[b] < T[b] for b in range(B)):
        rz, rk, rv, p0 = [], [], [], []
        for b in range(B):
            take = done[b] < T[b] and not (b == 2 and step % 3 == 1)
            sl = slice(done[b], done[b] + 1)
            rz.append(Z[b][sl] if take else None)
            rk.append(K[b][sl] if take else None)
            rv.append(V[b][sl] if take else None)
            p0.append(done[b])
            done[b] += int(take)
        ao = torch.full((B, wl.n_kv), -7, dtype=torch.int32, device="cuda")
        before = cache.lengths.clone()
        tl.append(cache, rz, rk, rv, p0, G_ | W_, append_offsets=ao)
        torch.cuda.synchronize()
        assert torch.equal(ao, before)
        step += 1
    assert spkv.spkv_cache_check(cache) == 0
    _check_cache(cache, wl, K, V, Z, T)
    w = wl.window
    for b in range(B):
        for g in range(wl.n_kv):
            rk_, rv_ = cache.read_ring(b, g)
            for p in range(max(0, T[b] - w), T[b]):
                np.testing.assert_array_equal(rk_[p % w].float().cpu().numpy(), K[b][p, g])
                np.testing.assert_array_equal(rv_[p % w].float().cpu().numpy(), V[b][p, g])


def test_one_row_appends_capacity_and_bad_rows():
    wl = inputs.WORKLOADS["decode_32k"]
    K, V, Z = _seq_data(wl, 200, 0, 13, [1.0] * 8)
    from learned_kv_cache_sp_amd.spkv import Cache
    cache = Cache(1, wl.n_kv, wl.head_dim, wl.window, 32, n_pages=20, max_pages_per_head=3,
                  dtype=torch.bfloat16)
    for t in range(200):
        tl.append(cache, [Z[t:t + 1]], [K[t:t + 1]], [V[t:t + 1]], [t], G_ | W_)
    torch.cuda.synchronize()
    with pytest.raises(spkv.SpkvError) as ei:
        spkv.spkv_cache_check(cache)
    assert ei.value.code == spkv.SPKV_E_CAPACITY
    lens = cache.lengths[0].cpu().numpy()
    assert lens.sum() <= 20 * 32 and np.all(lens <= 3 * 32)
    for g in range(wl.n_kv):
        k, v, pos = cache.read_head(0, g)
        np.testing.assert_array_equal(pos.cpu().numpy(), np.arange(len(pos)))
        np.testing.assert_array_equal(v.float().cpu().numpy(), V[: len(pos), g])
    # two rows for a sequence while max_rows_per_seq = 1
    cache2 = tl.new_cache(wl, 2, 10)
    kd, vd = tl.dev(K[:3], torch.bfloat16), tl.dev(V[:3], torch.bfloat16)
    spkv.spkv_compact_append(cache2, tl.dev(Z[:3]), kd, vd, tl.dev(np.array([0, 2, 3], np.int32)),
                             tl.dev(np.array([0, 0], np.int32)), 1, G_)
    torch.cuda.synchronize()
    with pytest.raises(spkv.SpkvError) as ei:
        spkv.spkv_cache_check(cache2)
    assert ei.value.code == spkv.SPKV_E_ROWS
    assert int(cache2.lengths[0].sum()) == 0 and int(cache2.lengths[1].sum()) == wl.n_kv


@pytest.mark.parametrize("name, n_kv, hd, misalign", [
    ("decode_32k", 8, 128, False),   # packed keep rows (one 8-byte load per row)
    ("decode_32k", 8, 128, True),    # keep rows not 8-byte aligned: per-byte count
    ("decode_32k", 3, 64, False),    # a head count that does not divide 16
    ("decode_32k", 16, 64, False),
    ("decode_32k", 1, 128, False),
    ("tiny", 2, 64, False),          # f32 cache
])
def test_large_appends_share_one_workspace(name, n_kv, hd, misalign):
    # appends of more than 256 rows per sequence run as one launch whose
    # workgroups coordinate through the workspace; one workspace serves many
    # calls of different sizes, including one that overflows the pool, and
    # is back at zero after each
    wl = tl.small_workload(name, n_kv=n_kv, head_dim=hd, n_q=n_kv)
    B = 3
    T = [2600, 1900, 3100]
    rates = [0.3, 0.05, 0.2, 0.5, 0.7, 0.9, 1.0, 0.0] * 2
    K, V, Z = zip(*[_seq_data(wl, T[b], b, 33, rates[:n_kv]) for b in range(B)])
    cache = tl.new_cache(wl, B, max(T))
    dt = tl.torch_dtype(wl)
    ws = spkv.workspace(spkv.spkv_compact_ws_bytes(cache, sum(T), 1400))
    done = [0] * B

    def keep_dev(z):
        z = z.astype(np.uint8)
        if not misalign:
            return tl.dev(z)
        flat = torch.zeros(z.size + 1, dtype=torch.uint8, device="cuda")
        flat[1:] = tl.dev(z.reshape(-1))
        return flat[1:].view(z.shape)

    for step in ([1400, 300, 1000], [257, 1400, 1100], [943, 200, 1000], [0, 0, 0]):
        counts = [min(step[b], T[b] - done[b]) for b in range(B)]
        offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        zz = np.concatenate([Z[b][done[b]:done[b] + counts[b]] for b in range(B)])
        kk = np.concatenate([K[b][done[b]:done[b] + counts[b]] for b in range(B)])
        vv = np.concatenate([V[b][done[b]:done[b] + counts[b]] for b in range(B)])
        if offs[-1]:
            spkv.spkv_compact_append(cache, keep_dev(zz), tl.dev(kk, dt), tl.dev(vv, dt), tl.dev(offs),
                                     tl.dev(np.array(done, np.int32)), 1400, G_ | W_, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.abs().sum().item()) == 0, "workspace not back at zero"
        done = [done[b] + counts[b] for b in range(B)]
        if step == [943, 200, 1000]:
            # an overflowing append on another cache, through the same workspace
            need = sum(-(-int(Z[2][:1400, g].sum()) // 64) for g in range(n_kv))
            assert need >= 2
            n_small = need // 2              # half the pages the append needs
            small = spkv.Cache(1, wl.n_kv, wl.head_dim, wl.window, 64, n_pages=n_small, max_pages_per_head=12,
                               dtype=dt)
            spkv.spkv_compact_append(small, keep_dev(Z[2][:1400]), tl.dev(K[2][:1400], dt), tl.dev(V[2][:1400], dt),
                                     tl.dev(np.array([0, 1400], np.int32)), tl.dev(np.array([0], np.int32)), 1400, G_,
                                     ws=ws)
            torch.cuda.synchronize()
            assert int(ws.abs().sum().item()) == 0
            with pytest.raises(spkv.SpkvError) as ei:
                spkv.spkv_cache_check(small)
            assert ei.value.code == spkv.SPKV_E_CAPACITY
            lists = oracle.compact(Z[2][:1400], 0)
            for g in range(wl.n_kv):
                k, v, pos = small.read_head(0, g)
                assert len(pos) <= min(12 * 64, len(lists[g]))
                np.testing.assert_array_equal(pos.cpu().numpy(), lists[g][:len(pos)])
                np.testing.assert_array_equal(v.float().cpu().numpy(), V[2][lists[g][:len(pos)], g])
            assert int(small.lengths.sum()) <= n_small * 64
    assert done == T
    assert spkv.spkv_cache_check(cache) == 0
    _check_cache(cache, wl, K, V, Z, T)
