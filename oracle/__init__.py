"""fp64 CPU oracle for SP-KV (test infrastructure only).

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this package.  It wraps ``spkv_oracle.c`` (plain C, fp64) through
ctypes and shares no code with the HIP library or its Python binding.

Citations are to "Self-Pruned Key-Value Attention" (arXiv 2605.14037),
section 2.1, equations (1)-(4).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spkv_oracle.c")
# SPKV_ORACLE_LIB names another build of the same source (the sanitizer
# build that the test suite makes and loads in a child process)
_LIB = os.environ.get("SPKV_ORACLE_LIB") or os.path.join(_HERE, "libspkv_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c99", "-fopenmp", "-Wall", "-Wextra",
            "-shared", "-fPIC", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i64, f64, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    lib.spkv_oracle_gate.argtypes = [i64, i64, i64, i64, vp, i64, vp, vp, vp, vp,
                                     f64, vp, vp, vp, ci]
    lib.spkv_oracle_gate.restype = ci
    lib.spkv_oracle_compact.argtypes = [i64, i64, vp, i64, vp, vp]
    lib.spkv_oracle_compact.restype = ci
    lib.spkv_oracle_rethreshold.argtypes = [i64, vp, f64, vp, vp]
    lib.spkv_oracle_rethreshold.restype = ci
    lib.spkv_oracle_head_stats.argtypes = [i64, i64, vp, vp, vp, vp]
    lib.spkv_oracle_head_stats.restype = ci
    lib.spkv_oracle_soft_attention.argtypes = [i64, i64, i64, i64, i64, vp, vp, i64, vp, vp,
                                               i64, vp, f64, f64, f64, f64, vp, vp, ci]
    lib.spkv_oracle_soft_attention.restype = ci
    lib.spkv_oracle_attention.argtypes = [i64, i64, i64, i64, i64, vp, vp, i64, vp, vp,
                                          i64, vp, f64, vp, vp, ci]
    lib.spkv_oracle_attention.restype = ci
    lib.spkv_oracle_visible_count.argtypes = [i64, i64, i64, vp, vp, i64, i64, vp]
    lib.spkv_oracle_visible_count.restype = ci
    lib.spkv_oracle_sink_gate.argtypes = [i64, i64, i64, i64, i64, i64, vp, i64, vp, vp, f64, vp, vp, ci]
    lib.spkv_oracle_sink_gate.restype = ci
    lib.spkv_oracle_max_threads.restype = ci
    lib.spkv_oracle_version.restype = ci
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        a = a.astype(np.float32)
    return np.ascontiguousarray(a)


def max_threads() -> int:
    return int(_load().spkv_oracle_max_threads())


def gate(H, W1, b1, W2, b2, tau: float, threads: int = 1):
    """O1, Eq. (1)-(2).  Returns (u [n, n_kv] f64, logit [n, n_kv] f64, z [n, n_kv] u8).

    H [n, d_model], W1 [d_hidden, d_model], b1 [d_hidden], W2 [n_kv, d_hidden],
    b2 [n_kv]; every value must be exactly representable in float32.
    """
    lib = _load()
    H = _f32(H)
    W1, b1, W2, b2 = _f32(W1), _f32(b1), _f32(W2), _f32(b2)
    n, d = H.shape
    hg = W1.shape[0]
    nkv = W2.shape[0]
    assert W1.shape == (hg, d) and b1.shape == (hg,) and W2.shape == (nkv, hg) and b2.shape == (nkv,)
    u = np.empty((n, nkv), np.float64)
    logit = np.empty((n, nkv), np.float64)
    z = np.empty((n, nkv), np.uint8)
    rc = lib.spkv_oracle_gate(n, d, hg, nkv, _p(H), d, _p(W1), _p(b1), _p(W2), _p(b2),
                              float(tau), _p(u), _p(logit), _p(z), int(threads))
    if rc != 0:
        raise ValueError(f"spkv_oracle_gate rejected its arguments ({rc})")
    return u, logit, z


def sink_gate(H, W, sinks, group: int, tau: float, threads: int = 1):
    """O8, the sink-attention gate (Fast KVzip page, core method).  Returns
    (u [n, n_kv] f64, z [n, n_kv] u8).

    H [n, d_model]; W [n_kv, (group + 1) * d_key, d_model] (per head the
    group query blocks, then the key block); sinks [n_kv, n_sinks, d_key]."""
    lib = _load()
    H, W, sinks = _f32(H), _f32(W), _f32(sinks)
    n, d = H.shape
    nkv, ns, dk = sinks.shape
    assert W.shape == (nkv, (group + 1) * dk, d)
    u = np.empty((n, nkv), np.float64)
    z = np.empty((n, nkv), np.uint8)
    rc = lib.spkv_oracle_sink_gate(n, d, nkv, int(group), dk, ns, _p(H), d, _p(W), _p(sinks), float(tau),
                                   _p(u), _p(z), int(threads))
    if rc != 0:
        raise ValueError(f"spkv_oracle_sink_gate rejected its arguments ({rc})")
    return u, z


def compact(z, pos0: int = 0):
    """O2: per key head, the positions of the kept rows in token order.

    Returns a list of int64 arrays (one per head)."""
    lib = _load()
    z = np.ascontiguousarray(np.asarray(z, dtype=np.uint8))
    n, nkv = z.shape
    pos = np.zeros((nkv, max(n, 1)), np.int64)
    ln = np.zeros((nkv,), np.int64)
    rc = lib.spkv_oracle_compact(n, nkv, _p(z), int(pos0), _p(pos), _p(ln))
    if rc != 0:
        raise ValueError("spkv_oracle_compact rejected its arguments")
    return [pos[g, : ln[g]].copy() for g in range(nkv)]


def rethreshold(u, tau2: float):
    """O5: indices of the entries of one cache list whose stored utility
    passes the new threshold (u >= tau2), in logical order.

    u is one (sequence, key head) list's stored utilities (float32)."""
    lib = _load()
    u = np.ascontiguousarray(np.asarray(u, dtype=np.float32).reshape(-1))
    n = u.shape[0]
    idx = np.zeros((max(n, 1),), np.int64)
    ln = np.zeros((1,), np.int64)
    rc = lib.spkv_oracle_rethreshold(n, _p(u), float(tau2), _p(idx), _p(ln))
    if rc != 0:
        raise ValueError("spkv_oracle_rethreshold rejected its arguments")
    return idx[: ln[0]].copy()


def head_stats(u, z, u_sum=None, kept=None):
    """O6: per key head, the sum of the utilities (fp64, row order) and the
    count of kept pairs over the rows of u / z ([n_rows, n_kv]; either may be
    None), added to u_sum / kept (fresh zeros when None).  Returns both."""
    lib = _load()
    ref = u if u is not None else z
    n, nkv = np.asarray(ref).shape
    u_c = None if u is None else np.ascontiguousarray(np.asarray(u, dtype=np.float32))
    z_c = None if z is None else np.ascontiguousarray(np.asarray(z, dtype=np.uint8))
    us = np.zeros(nkv, np.float64) if u_sum is None else np.array(u_sum, np.float64)
    kp = np.zeros(nkv, np.int64) if kept is None else np.array(kept, np.int64)
    rc = lib.spkv_oracle_head_stats(n, nkv, None if u_c is None else _p(u_c), None if z_c is None else _p(z_c),
                                    _p(us), _p(kp))
    if rc != 0:
        raise ValueError("spkv_oracle_head_stats rejected its arguments")
    return us, kp


def attention(Q, t_rows, K, V, z, w: int, scale: float | None = None, threads: int = 1):
    """O3, Eq. (3)-(4) on the full sequence.

    Q [n_rows, n_q, hd]; t_rows [n_rows]; K, V [T, n_kv, hd]; z [T, n_kv].
    Returns (out [n_rows, n_q, hd] f64, lse [n_rows, n_q] f64)."""
    lib = _load()
    Q = _f32(Q)
    K = _f32(K)
    V = _f32(V)
    z = np.ascontiguousarray(np.asarray(z, dtype=np.uint8))
    t_rows = np.ascontiguousarray(np.asarray(t_rows, dtype=np.int64))
    n_rows, nq, hd = Q.shape
    T, nkv, hd2 = K.shape
    assert hd2 == hd and V.shape == K.shape and z.shape == (T, nkv) and t_rows.shape == (n_rows,)
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    out = np.empty((n_rows, nq, hd), np.float64)
    lse = np.empty((n_rows, nq), np.float64)
    rc = lib.spkv_oracle_attention(T, nq, nkv, hd, int(w), _p(Q), _p(t_rows), n_rows,
                                   _p(K), _p(V), nkv * hd, _p(z), float(scale),
                                   _p(out), _p(lse), int(threads))
    if rc != 0:
        raise ValueError("spkv_oracle_attention rejected its arguments")
    return out, lse


def soft_attention(Q, t_rows, K, V, u, w: int, tau: float, beta: float = 0.01, c: float = 1e6,
                   scale: float | None = None, threads: int = 1):
    """O7, Eq. (5)-(6): every causal key, with the additive soft mask outside
    the window.  Shapes as attention(); u [T, n_kv] float32 utilities."""
    lib = _load()
    Q = _f32(Q)
    K = _f32(K)
    V = _f32(V)
    u = np.ascontiguousarray(np.asarray(u, dtype=np.float32))
    t_rows = np.ascontiguousarray(np.asarray(t_rows, dtype=np.int64))
    n_rows, nq, hd = Q.shape
    T, nkv, hd2 = K.shape
    assert hd2 == hd and V.shape == K.shape and u.shape == (T, nkv) and t_rows.shape == (n_rows,)
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    out = np.empty((n_rows, nq, hd), np.float64)
    lse = np.empty((n_rows, nq), np.float64)
    rc = lib.spkv_oracle_soft_attention(T, nq, nkv, hd, int(w), _p(Q), _p(t_rows), n_rows, _p(K), _p(V),
                                        nkv * hd, _p(u), float(tau), float(beta), float(c), float(scale),
                                        _p(out), _p(lse), int(threads))
    if rc != 0:
        raise ValueError("spkv_oracle_soft_attention rejected its arguments")
    return out, lse


def attention_head(q_rows, t_rows, K_g, V_g, z_g, group: int, w: int,
                   scale: float | None = None, threads: int = 1):
    """O3 for the query heads of ONE key head g.

    q_rows [n_rows, group, hd]; K_g, V_g [T, hd] (any row stride, float32);
    z_g [T].  Returns (out [n_rows, group, hd], lse [n_rows, group])."""
    lib = _load()
    q_rows = _f32(q_rows)
    K_g = np.asarray(K_g)
    V_g = np.asarray(V_g)
    assert K_g.dtype == np.float32 and V_g.dtype == np.float32
    assert K_g.strides == V_g.strides and K_g.strides[1] == 4
    ld = K_g.strides[0] // 4
    T, hd = K_g.shape
    z_g = np.ascontiguousarray(np.asarray(z_g, dtype=np.uint8).reshape(T))
    t_rows = np.ascontiguousarray(np.asarray(t_rows, dtype=np.int64))
    n_rows = q_rows.shape[0]
    assert q_rows.shape == (n_rows, group, hd)
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    out = np.empty((n_rows, group, hd), np.float64)
    lse = np.empty((n_rows, group), np.float64)
    rc = lib.spkv_oracle_attention(T, group, 1, hd, int(w), _p(q_rows), _p(t_rows), n_rows,
                                   K_g.ctypes.data_as(ctypes.c_void_p),
                                   V_g.ctypes.data_as(ctypes.c_void_p), ld, _p(z_g),
                                   float(scale), _p(out), _p(lse), int(threads))
    if rc != 0:
        raise ValueError("spkv_oracle_attention rejected its arguments")
    return out, lse


def visible_count(z_g, t_rows, w: int):
    """|visible(t)| of Eq. (4) for one key head (z_g [T])."""
    lib = _load()
    z_g = np.ascontiguousarray(np.asarray(z_g, dtype=np.uint8))
    T = z_g.shape[0]
    t_rows = np.ascontiguousarray(np.asarray(t_rows, dtype=np.int64))
    cnt = np.empty(t_rows.shape, np.int64)
    rc = lib.spkv_oracle_visible_count(T, 1, int(w), _p(z_g), _p(t_rows), t_rows.shape[0], 0, _p(cnt))
    if rc != 0:
        raise ValueError("spkv_oracle_visible_count rejected its arguments")
    return cnt
