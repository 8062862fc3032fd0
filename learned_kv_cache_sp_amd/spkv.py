"""Python binding of libspkv (the SP-KV hot path on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libspkv.so.  torch supplies device memory and the stream.  The functions
``spkv_gate``, ``spkv_compact_append``, ``spkv_decode_attn``,
``spkv_prefill_attn`` (``soft=`` for ``spkv_prefill_attn_soft``),
``spkv_decode_step``, ``spkv_cache_rethreshold`` and ``spkv_head_stats`` mirror the C calls of include/spkv.h one to one and take
torch tensors in place of pointers.  ``Cache`` and ``GateWeights``
allocate the buffers the C structs point to.

There is no fallback: if libspkv.so is missing or no GPU is visible, the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspkv.so")

SPKV_OK = 0
SPKV_E_INVALID = -1
SPKV_E_UNSUPPORTED = -2
SPKV_E_HIP = -3
SPKV_E_CAPACITY = -4
SPKV_E_WORKSPACE = -5
SPKV_E_ROWS = -6
SPKV_E_TIMEOUT = -7

SPKV_F32 = 0
SPKV_BF16 = 1
SPKV_APPEND_GLOBAL = 1
SPKV_APPEND_WINDOW = 2

STATUS_POOL_FULL = 1
STATUS_TABLE_FULL = 2
STATUS_BAD_ROWS = 4
STATUS_STEP_TIMEOUT = 8


class SpkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


class GateDesc(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("d_hidden", ctypes.c_int32), ("n_kv", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("b2", ctypes.c_void_p),
    ]


class SinkGateDesc(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("group", ctypes.c_int32),
        ("d_key", ctypes.c_int32), ("n_sinks", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("w", ctypes.c_void_p), ("sinks", ctypes.c_void_p),
    ]


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32), ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32),
        ("max_pages_per_head", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p), ("pos_pages", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("lengths", ctypes.c_void_p), ("pool_next", ctypes.c_void_p),
        ("status", ctypes.c_void_p), ("ring_k", ctypes.c_void_p), ("ring_v", ctypes.c_void_p),
        ("u_pages", ctypes.c_void_p),
    ]


EXPORTS = [
    "spkv_gate", "spkv_gate_ws_bytes", "spkv_compact_append", "spkv_compact_ws_bytes",
    "spkv_decode_attn", "spkv_decode_ws_bytes", "spkv_decode_attn_noalloc", "spkv_decode_step", "spkv_decode_step_ws_bytes",
    "spkv_prefill_attn", "spkv_prefill_ws_bytes", "spkv_cache_rethreshold", "spkv_rethreshold_ws_bytes",
    "spkv_head_stats", "spkv_head_stats_ws_bytes", "spkv_prefill_attn_soft",
    "spkv_cache_bytes", "spkv_cache_reset", "spkv_cache_check", "spkv_status_str",
    "spkv_last_error", "spkv_version", "spkv_hbm_read", "spkv_gate_sink", "spkv_set_wait_limit",
]

# ---- storage order of cached keys and values ---------------------------------
# Pages (and the ring of each (b, g)) hold blocks of 32 slots.  A key block is
# [head_dim / 32][32 rows][32 dims] with row p holding slot _SLOT_OF_ROW[p]
# (the rows of the decode kernel's two 16 x 16 x 32 MFMA operand tiles), a
# value block is [head_dim][32 slots].  The tensors keep their declared
# shapes; these helpers give the logical [slots, head_dim] views.
_SLOT_OF_ROW = [8 * ((p & 15) >> 2) + 4 * (p >> 4) + (p & 3) for p in range(32)]
_ROW_OF_SLOT = [_SLOT_OF_ROW.index(r) for r in range(32)]


def unblock_keys(x: torch.Tensor) -> torch.Tensor:
    """Stored keys of n slots (n a multiple of 32), given as an [n, hd] view of
    the stored elements -> logical keys [n, hd]."""
    n, hd = x.numel() // x.shape[-1], x.shape[-1]
    blk = x.reshape(n // 32, hd // 32, 32, 32).permute(0, 2, 1, 3)        # [blk][row][cc][dd]
    idx = torch.tensor(_ROW_OF_SLOT, device=x.device)
    return blk.index_select(1, idx).reshape(n, hd)


def unblock_values(x: torch.Tensor) -> torch.Tensor:
    """Stored values of n slots (n a multiple of 32), given as an [n, hd] view
    of the stored elements -> logical values [n, hd]."""
    n, hd = x.numel() // x.shape[-1], x.shape[-1]
    return x.reshape(n // 32, hd, 32).permute(0, 2, 1).reshape(n, hd)


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libspkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with learned_kv_cache_sp_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    G, C = ctypes.POINTER(GateDesc), ctypes.POINTER(CacheDesc)
    sig = {
        "spkv_gate": ([G, vp, i64, i64, f32, vp, vp, vp, sz, vp], ctypes.c_int),
        "spkv_gate_ws_bytes": ([G, i64], sz),
        "spkv_compact_append": ([C, vp, vp, vp, vp, i64, vp, vp, i32, i32, i32, vp, vp, sz, vp], ctypes.c_int),
        "spkv_compact_ws_bytes": ([C, i32, i32], sz),
        "spkv_decode_attn": ([C, i32, vp, i64, vp, f32, vp, vp, vp, sz, vp], ctypes.c_int),
        "spkv_decode_ws_bytes": ([C, i32], sz),
        "spkv_decode_attn_noalloc": ([C, i32, vp, i64, vp, f32, vp, vp, vp], ctypes.c_int),
        "spkv_decode_step": ([C, G, i32, vp, i64, f32, vp, vp, i64, vp, i64, vp, f32, vp, vp, vp, vp, vp, sz, vp],
                             ctypes.c_int),
        "spkv_decode_step_ws_bytes": ([C, G, i32], sz),
        "spkv_prefill_attn": ([C, i32, i32, vp, i64, vp, vp, i64, i32, i32, f32, vp, vp, vp, sz, vp],
                              ctypes.c_int),
        "spkv_prefill_ws_bytes": ([C, i32, i32], sz),
        "spkv_cache_rethreshold": ([C, C, f32, vp, sz, vp], ctypes.c_int),
        "spkv_rethreshold_ws_bytes": ([C], sz),
        "spkv_head_stats": ([vp, vp, i64, i32, vp, vp, vp, sz, vp], ctypes.c_int),
        "spkv_head_stats_ws_bytes": ([i64, i32], sz),
        "spkv_prefill_attn_soft": ([C, i32, i32, vp, i64, vp, vp, i64, i32, i32, f32, f32, f32, f32, vp, vp, vp, sz,
                                    vp], ctypes.c_int),
        "spkv_cache_bytes": ([C, vp], sz),
        "spkv_cache_reset": ([C, vp], ctypes.c_int),
        "spkv_cache_check": ([C, vp, vp], ctypes.c_int),
        "spkv_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "spkv_last_error": ([], ctypes.c_char_p),
        "spkv_version": ([], ctypes.c_int),
        "spkv_hbm_read": ([vp, sz, i32, i32, vp, vp], ctypes.c_int),
        "spkv_gate_sink": ([ctypes.POINTER(SinkGateDesc), vp, i64, i64, f32, vp, vp, vp], ctypes.c_int),
        "spkv_set_wait_limit": ([i32], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int):
    if rc != SPKV_OK:
        lib = load_library()
        raise SpkvError(rc, lib.spkv_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not isinstance(t, int) and not t.is_cuda:
            raise ValueError("libspkv works on device tensors only")


def _expect(name: str, t, shape, dtype=None, packed: bool = True):
    """Raise ValueError unless t has `shape` (and `dtype`).  packed: the whole
    tensor is contiguous; otherwise only its rows (dim 0 may be strided, as
    for arguments passed with a row stride)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if packed and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not packed and t.shape[0] > 0 and t.dim() > 1 and not t[0].is_contiguous():
        raise ValueError(f"{name} rows must be contiguous")


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return SPKV_BF16
    if dt == torch.float32:
        return SPKV_F32
    raise ValueError(f"unsupported dtype {dt}")


def _torch_dtype(code: int):
    return torch.bfloat16 if code == SPKV_BF16 else torch.float32


def _row_stride(t: torch.Tensor) -> int:
    """Elements between consecutive rows (dim 0) of a tensor whose other dims are packed."""
    if t.dim() == 1:
        return t.shape[0]
    if t.shape[0] == 0:
        return max(1, int(np.prod(t.shape[1:])))
    inner = t[0]
    if not inner.is_contiguous():
        raise ValueError("rows must be contiguous")
    return t.stride(0)


# ----------------------------------------------------------------------------
# buffers
# ----------------------------------------------------------------------------

@dataclass
class GateWeights:
    """W1 [d_hidden, d_model] (dtype), b1 [d_hidden], W2 [n_kv, d_hidden], b2 [n_kv] (f32)."""
    w1: torch.Tensor
    b1: torch.Tensor
    w2: torch.Tensor
    b2: torch.Tensor

    def desc(self) -> GateDesc:
        _need_gpu(self.w1, self.b1, self.w2, self.b2)
        for t in (self.b1, self.w2, self.b2):
            if t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError("b1, w2, b2 must be contiguous float32")
        if not self.w1.is_contiguous():
            raise ValueError("w1 must be contiguous")
        d = GateDesc()
        d.d_hidden, d.d_model = self.w1.shape
        d.n_kv = self.w2.shape[0]
        d.dtype = _dtype_code(self.w1.dtype)
        d.w1, d.b1, d.w2, d.b2 = (_ptr(self.w1), _ptr(self.b1), _ptr(self.w2), _ptr(self.b2))
        self._desc = d  # keep alive
        return d


@dataclass
class SinkGateWeights:
    """Sink-attention gate: w [n_kv, (group + 1) * d_key, d_model] (bf16; per head
    the group query blocks, then the key block), sinks [n_kv, n_sinks, d_key] f32."""
    w: torch.Tensor
    sinks: torch.Tensor
    group: int

    def desc(self) -> SinkGateDesc:
        _need_gpu(self.w, self.sinks)
        if self.w.dim() != 3 or self.sinks.dim() != 3:
            raise ValueError("w must be [n_kv, (group + 1) * d_key, d_model], sinks [n_kv, n_sinks, d_key]")
        nkv, per, d_model = self.w.shape
        ns, dk = self.sinks.shape[1], self.sinks.shape[2]
        if self.sinks.shape[0] != nkv or per != (self.group + 1) * dk:
            raise ValueError(f"w {tuple(self.w.shape)} and sinks {tuple(self.sinks.shape)} do not match group "
                             f"{self.group}")
        if not self.w.is_contiguous() or not self.sinks.is_contiguous() or self.sinks.dtype != torch.float32:
            raise ValueError("w must be contiguous, sinks contiguous float32")
        d = SinkGateDesc()
        d.d_model, d.n_kv, d.group, d.d_key, d.n_sinks = d_model, nkv, int(self.group), dk, ns
        d.dtype = _dtype_code(self.w.dtype)
        d.w, d.sinks = _ptr(self.w), _ptr(self.sinks)
        self._desc = d
        return d


class Cache:
    """Device buffers of one layer's SP-KV cache (see include/spkv.h, spkv_cache)."""

    GUARD_BYTE = 0xA5

    def __init__(self, batch: int, n_kv: int, head_dim: int, window: int, page_size: int,
                 n_pages: int, max_pages_per_head: int, dtype=torch.bfloat16, device="cuda",
                 utilities: bool = False, guard: int = 0):
        """guard > 0 (a multiple of 256): every buffer sits between two runs of
        `guard` canary bytes (GUARD_BYTE), which check_guards() inspects --
        a test aid for catching writes outside the buffers."""
        dt = dtype
        self.batch, self.n_kv, self.head_dim, self.window = batch, n_kv, head_dim, window
        self.page_size, self.n_pages, self.max_pages_per_head = page_size, n_pages, max_pages_per_head
        self.dtype = dt
        if guard % 256:
            raise ValueError("guard must be a multiple of 256 bytes")
        self._guards = []

        def z(shape, d=dt, fill=0, name=""):
            if not guard:
                return torch.full(shape, fill, dtype=d, device=device)
            n = int(np.prod(shape)) * torch.empty((), dtype=d).element_size()
            body = (n + 255) // 256 * 256
            raw = torch.full((guard + body + guard,), self.GUARD_BYTE, dtype=torch.uint8, device=device)
            t = raw[guard:guard + n].view(d).view(shape)
            t.fill_(fill)
            self._guards.append((name, raw, guard, n))
            return t

        self.k_pages = z((n_pages, page_size, head_dim), name="k_pages")
        self.v_pages = z((n_pages, head_dim, page_size), name="v_pages")
        self.pos_pages = z((n_pages, page_size), torch.int32, name="pos_pages")
        self.page_table = z((batch, n_kv, max_pages_per_head), torch.int32, -1, name="page_table")
        self.lengths = z((batch, n_kv), torch.int32, name="lengths")
        self.pool_next = z((1,), torch.int32, name="pool_next")
        self.status = z((1,), torch.int32, name="status")
        self.ring_k = z((batch, n_kv, window, head_dim), name="ring_k")
        self.ring_v = z((batch, n_kv, head_dim, window), name="ring_v")
        # utility of each entry (kept for spkv_cache_rethreshold)
        self.u_pages = z((n_pages, page_size), torch.float32, name="u_pages") if utilities else None
        self._desc = None

    def check_guards(self) -> list:
        """Names of the buffers whose canary bytes (before, after or in the
        padding after the buffer) are no longer intact."""
        bad = []
        for name, raw, g, n in self._guards:
            outside = torch.cat([raw[:g], raw[g + n:]])
            if bool((outside != self.GUARD_BYTE).any()):
                bad.append(name)
        return bad

    @staticmethod
    def pages_needed(lengths_per_head, page_size: int) -> int:
        return int(sum((int(n) + page_size - 1) // page_size for n in lengths_per_head))

    def desc(self) -> CacheDesc:
        if self._desc is None:
            d = CacheDesc()
            d.batch, d.n_kv, d.head_dim, d.window = self.batch, self.n_kv, self.head_dim, self.window
            d.page_size, d.n_pages, d.max_pages_per_head = self.page_size, self.n_pages, self.max_pages_per_head
            d.dtype = _dtype_code(self.dtype)
            for name in ("k_pages", "v_pages", "pos_pages", "page_table", "lengths", "pool_next",
                         "status", "ring_k", "ring_v", "u_pages"):
                setattr(d, name, _ptr(getattr(self, name)))
            self._desc = d
        return self._desc

    def nbytes(self) -> int:
        return int(load_library().spkv_cache_bytes(ctypes.byref(self.desc()), None))

    # ---- logical read-back (host side; for checks and tools) ---------------
    def read_head(self, b: int, g: int):
        """Cached entries of (b, g) in logical order: (K [n, hd], V [n, hd], pos [n])."""
        n = int(self.lengths[b, g].item())
        P = self.page_size
        npg = (n + P - 1) // P
        pages = self.page_table[b, g, :npg].long()
        k = unblock_keys(self.k_pages[pages].reshape(npg * P, self.head_dim))[:n]
        v = unblock_values(self.v_pages[pages].reshape(npg * P, self.head_dim))[:n]
        pos = self.pos_pages[pages].reshape(npg * P)[:n]
        return k, v, pos

    def read_head_u(self, b: int, g: int):
        """Stored utilities of the entries of (b, g) in logical order (f32 [n])."""
        if self.u_pages is None:
            raise ValueError("this cache does not store utilities")
        n = int(self.lengths[b, g].item())
        P = self.page_size
        npg = (n + P - 1) // P
        pages = self.page_table[b, g, :npg].long()
        return self.u_pages[pages].reshape(npg * P)[:n]

    def share_ring(self, other: "Cache"):
        """Point this cache's ring at other's (for a cache rebuilt from other)."""
        self.ring_k, self.ring_v = other.ring_k, other.ring_v
        self._desc = None

    def read_ring(self, b: int, g: int):
        """Ring of (b, g): K [w, hd], V [w, hd] indexed by slot = position % w."""
        return unblock_keys(self.ring_k[b, g]), unblock_values(self.ring_v[b, g].reshape(self.window, self.head_dim))

    def snapshot(self) -> dict:
        names = ("k_pages", "v_pages", "pos_pages", "page_table", "lengths", "pool_next", "status",
                 "ring_k", "ring_v", "u_pages")
        return {n: getattr(self, n).clone() for n in names if getattr(self, n) is not None}

    def restore(self, snap: dict):
        for n, t in snap.items():
            getattr(self, n).copy_(t)


def workspace(nbytes: int, device="cuda") -> torch.Tensor | None:
    """Zero-filled device workspace (16-byte aligned)."""
    if nbytes == 0:
        return None
    return torch.zeros(((nbytes + 15) // 16) * 4, dtype=torch.int32, device=device)


# ----------------------------------------------------------------------------
# the four calls
# ----------------------------------------------------------------------------

def spkv_gate_ws_bytes(weights: GateWeights, n_rows: int) -> int:
    return int(load_library().spkv_gate_ws_bytes(ctypes.byref(weights.desc()), n_rows))


def spkv_gate(weights: GateWeights, hidden: torch.Tensor, tau: float, utility=None, keep=None,
              ws=None, stream=None):
    """Eq. (1)-(2) for every row of hidden [n_rows, d_model].  Returns (utility, keep)."""
    lib = load_library()
    desc = weights.desc()
    n = hidden.shape[0]
    dev = hidden.device
    if keep is None:
        keep = torch.empty((n, desc.n_kv), dtype=torch.uint8, device=dev)
    if utility is None:
        utility = torch.empty((n, desc.n_kv), dtype=torch.float32, device=dev)
    _need_gpu(hidden, keep, utility)
    if hidden.dtype != weights.w1.dtype:
        raise ValueError("hidden and w1 dtypes differ")
    need = spkv_gate_ws_bytes(weights, n)
    if ws is None and need:
        ws = workspace(need, dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.spkv_gate(ctypes.byref(desc), _ptr(hidden), n, _row_stride(hidden), float(tau),
                         _ptr(utility), _ptr(keep), _ptr(ws), ws_bytes, _stream(stream)))
    return utility, keep


def spkv_gate_sink(weights: SinkGateWeights, hidden: torch.Tensor, tau: float, utility=None, keep=None,
                   stream=None):
    """The sink-attention gate for every row of hidden [n_rows, d_model].  Returns (utility, keep)."""
    lib = load_library()
    desc = weights.desc()
    if hidden.dim() != 2 or hidden.shape[1] != desc.d_model:
        raise ValueError(f"hidden has shape {tuple(hidden.shape)}, expected [n_rows, {desc.d_model}]")
    n = hidden.shape[0]
    dev = hidden.device
    if keep is None:
        keep = torch.empty((n, desc.n_kv), dtype=torch.uint8, device=dev)
    if utility is None:
        utility = torch.empty((n, desc.n_kv), dtype=torch.float32, device=dev)
    _expect("keep", keep, (n, desc.n_kv), torch.uint8)
    _expect("utility", utility, (n, desc.n_kv), torch.float32)
    _need_gpu(hidden, keep, utility)
    if hidden.dtype != weights.w.dtype:
        raise ValueError("hidden and w dtypes differ")
    _check(lib.spkv_gate_sink(ctypes.byref(desc), _ptr(hidden), n, _row_stride(hidden), float(tau), _ptr(utility),
                              _ptr(keep), _stream(stream)))
    return utility, keep


def spkv_compact_ws_bytes(cache: Cache, n_rows: int, max_rows_per_seq: int) -> int:
    return int(load_library().spkv_compact_ws_bytes(ctypes.byref(cache.desc()), n_rows, max_rows_per_seq))


def spkv_compact_append(cache: Cache, keep, k: torch.Tensor, v: torch.Tensor, row_offsets: torch.Tensor,
                        pos0: torch.Tensor, max_rows_per_seq: int, flags: int, append_offsets=None,
                        ws=None, stream=None, utility=None):
    """Append rows [n_rows, n_kv, hd] (CSR by row_offsets) to the cache; see spkv.h."""
    lib = load_library()
    _need_gpu(keep, k, v, row_offsets, pos0, append_offsets, utility)
    if utility is not None and utility.dtype != torch.float32:
        raise ValueError("utility must be float32")
    if k.dtype != cache.dtype or v.dtype != cache.dtype:
        raise ValueError("k / v dtype differs from the cache")
    if row_offsets.dtype != torch.int32 or pos0.dtype != torch.int32:
        raise ValueError("row_offsets and pos0 must be int32")
    if keep is not None and keep.dtype != torch.uint8:
        raise ValueError("keep must be uint8")
    n = k.shape[0]
    ld = _row_stride(k)
    if _row_stride(v) != ld:
        raise ValueError("k and v must share a row stride")
    for name, t in (("keep", keep), ("utility", utility)):
        if t is not None and (tuple(t.shape) != (n, cache.n_kv) or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [{n}, {cache.n_kv}] tensor")
    need = spkv_compact_ws_bytes(cache, n, max_rows_per_seq)
    if ws is None and need:
        ws = workspace(need, k.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.spkv_compact_append(ctypes.byref(cache.desc()), _ptr(keep), _ptr(utility), _ptr(k), _ptr(v), ld,
                                   _ptr(row_offsets), _ptr(pos0), n, int(max_rows_per_seq), int(flags),
                                   _ptr(append_offsets), _ptr(ws), ws_bytes, _stream(stream)))


def spkv_decode_ws_bytes(cache: Cache, n_q_heads: int) -> int:
    return int(load_library().spkv_decode_ws_bytes(ctypes.byref(cache.desc()), n_q_heads))


def spkv_decode_attn(cache: Cache, q: torch.Tensor, t: torch.Tensor, scale: float, out=None, lse=None,
                     ws=None, stream=None):
    """One query per sequence: q [batch, n_q, hd], t [batch] int32.  Returns (out, lse)."""
    lib = load_library()
    B, nq, hd = _decode_shapes(cache, q, t)
    if out is None:
        out = torch.empty((B, nq, hd), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, nq), dtype=torch.float32, device=q.device)
    _expect("out", out, (B, nq, hd), torch.float32)
    _expect("lse", lse, (B, nq), torch.float32)
    _need_gpu(q, t, out, lse)
    need = spkv_decode_ws_bytes(cache, nq)
    if ws is None and need:
        ws = workspace(need, q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.spkv_decode_attn(ctypes.byref(cache.desc()), nq, _ptr(q), _row_stride(q), _ptr(t),
                                float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))
    return out, lse


def spkv_decode_attn_noalloc(cache: Cache, q: torch.Tensor, t: torch.Tensor, scale: float, out=None, lse=None,
                             stream=None):
    """spkv_decode_attn with the library's built-in scratch in place of a workspace
    (the C call allocates nothing; calls on one GPU must not overlap).  Returns (out, lse)."""
    lib = load_library()
    B, nq, hd = _decode_shapes(cache, q, t)
    if out is None:
        out = torch.empty((B, nq, hd), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, nq), dtype=torch.float32, device=q.device)
    _expect("out", out, (B, nq, hd), torch.float32)
    _expect("lse", lse, (B, nq), torch.float32)
    _need_gpu(q, t, out, lse)
    _check(lib.spkv_decode_attn_noalloc(ctypes.byref(cache.desc()), nq, _ptr(q), _row_stride(q), _ptr(t),
                                        float(scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def _decode_shapes(cache: Cache, q: torch.Tensor, t: torch.Tensor):
    """q [cache.batch, n_q, head_dim] in the cache dtype with packed rows, t [cache.batch] int32;
    returns (batch, n_q, head_dim).  The kernels read and write every sequence of the cache."""
    if q.dim() != 3:
        raise ValueError(f"q must be [batch, n_q, head_dim], got shape {tuple(q.shape)}")
    B, nq = cache.batch, q.shape[1]
    if nq < 1 or nq % cache.n_kv:
        raise ValueError(f"n_q = {nq} is not a multiple of n_kv = {cache.n_kv}")
    _expect("q", q, (B, nq, cache.head_dim), cache.dtype, packed=False)
    _expect("t", t, (B,), torch.int32)
    return B, nq, cache.head_dim


def spkv_decode_step_ws_bytes(cache: Cache, weights: GateWeights | None, n_q_heads: int) -> int:
    g = None if weights is None else ctypes.byref(weights.desc())
    return int(load_library().spkv_decode_step_ws_bytes(ctypes.byref(cache.desc()), g, n_q_heads))


def spkv_decode_step(cache: Cache, weights: GateWeights | None, hidden, tau: float, k: torch.Tensor,
                     v: torch.Tensor, q: torch.Tensor, t: torch.Tensor, scale: float, utility=None, keep=None,
                     out=None, lse=None, ws=None, stream=None):
    """Gate + append (GLOBAL | WINDOW) + decode attention of one step in one launch; with weights
    None, only the ring write (WINDOW) + attention (hidden, tau ignored).
    hidden [batch, d_model], k / v [batch, n_kv, hd], q [batch, n_q, hd], t [batch] int32.
    Returns (utility, keep, out, lse) (utility and keep None without a gate)."""
    lib = load_library()
    B, nq, hd = _decode_shapes(cache, q, t)
    dev = q.device
    gated = weights is not None
    nkv = cache.n_kv
    if gated:
        if weights.w2.shape[0] != nkv:
            raise ValueError(f"the gate has {weights.w2.shape[0]} outputs, the cache {nkv} key heads")
        if keep is None:
            keep = torch.empty((B, nkv), dtype=torch.uint8, device=dev)
        if utility is None:
            utility = torch.empty((B, nkv), dtype=torch.float32, device=dev)
        _expect("hidden", hidden, (B, weights.w1.shape[1]), weights.w1.dtype, packed=False)
        _expect("keep", keep, (B, nkv), torch.uint8)
        _expect("utility", utility, (B, nkv), torch.float32)
    else:
        utility = keep = hidden = None
    if out is None:
        out = torch.empty((B, nq, hd), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, nq), dtype=torch.float32, device=dev)
    _expect("k", k, (B, nkv, hd), cache.dtype, packed=False)
    _expect("v", v, (B, nkv, hd), cache.dtype, packed=False)
    _expect("out", out, (B, nq, hd), torch.float32)
    _expect("lse", lse, (B, nq), torch.float32)
    _need_gpu(hidden, k, v, q, t, keep, utility, out, lse)
    ld = _row_stride(k)
    if _row_stride(v) != ld:
        raise ValueError("k and v must share a row stride")
    need = spkv_decode_step_ws_bytes(cache, weights, nq)
    if ws is None and need:
        ws = workspace(need, dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.spkv_decode_step(ctypes.byref(cache.desc()), ctypes.byref(weights.desc()) if gated else None, nq,
                                _ptr(hidden), _row_stride(hidden) if gated else 0, float(tau), _ptr(k), _ptr(v), ld,
                                _ptr(q), _row_stride(q), _ptr(t), float(scale), _ptr(utility), _ptr(keep), _ptr(out),
                                _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))
    return utility, keep, out, lse


def spkv_prefill_ws_bytes(cache: Cache, n_q_heads: int, n_rows: int) -> int:
    return int(load_library().spkv_prefill_ws_bytes(ctypes.byref(cache.desc()), n_q_heads, n_rows))


def spkv_prefill_attn(cache: Cache, b: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos0: int,
                      scale: float, out=None, lse=None, ws=None, stream=None, soft=None):
    """Rows pos0 .. pos0+n-1 of sequence b: q [n, n_q, hd], k/v [n, n_kv, hd].  Returns (out, lse).

    soft = (tau, beta, c) calls spkv_prefill_attn_soft (the mask of Eq. 5-6
    on the cached keys, from their stored utilities)."""
    lib = load_library()
    if q.dim() != 3:
        raise ValueError(f"q must be [n_rows, n_q, head_dim], got shape {tuple(q.shape)}")
    n, nq, hd = q.shape
    if not 0 <= int(b) < cache.batch:
        raise ValueError(f"sequence {b} is outside the cache's batch of {cache.batch}")
    if nq < 1 or nq % cache.n_kv:
        raise ValueError(f"n_q = {nq} is not a multiple of n_kv = {cache.n_kv}")
    _expect("q", q, (n, nq, cache.head_dim), cache.dtype, packed=False)
    _expect("k", k, (n, cache.n_kv, cache.head_dim), cache.dtype, packed=False)
    _expect("v", v, (n, cache.n_kv, cache.head_dim), cache.dtype, packed=False)
    if out is None:
        out = torch.empty((n, nq, hd), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((n, nq), dtype=torch.float32, device=q.device)
    _expect("out", out, (n, nq, hd), torch.float32)
    _expect("lse", lse, (n, nq), torch.float32)
    _need_gpu(q, k, v, out, lse)
    need = spkv_prefill_ws_bytes(cache, nq, n)
    if ws is None and need:
        ws = workspace(need, q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    ld_kv = _row_stride(k)
    if _row_stride(v) != ld_kv:
        raise ValueError("k and v must share a row stride")
    if soft is not None:
        tau, beta, c_mask = soft
        _check(lib.spkv_prefill_attn_soft(ctypes.byref(cache.desc()), nq, int(b), _ptr(q), _row_stride(q), _ptr(k),
                                          _ptr(v), ld_kv, int(pos0), n, float(scale), float(tau), float(beta),
                                          float(c_mask), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))
    else:
        _check(lib.spkv_prefill_attn(ctypes.byref(cache.desc()), nq, int(b), _ptr(q), _row_stride(q), _ptr(k),
                                     _ptr(v), ld_kv, int(pos0), n, float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                     ws_bytes, _stream(stream)))
    return out, lse


def spkv_rethreshold_ws_bytes(src: Cache) -> int:
    return int(load_library().spkv_rethreshold_ws_bytes(ctypes.byref(src.desc())))


def spkv_cache_rethreshold(src: Cache, dst: Cache, tau: float, ws=None, stream=None):
    """Rebuild dst from the entries of src whose stored utility is >= tau; see spkv.h."""
    lib = load_library()
    need = spkv_rethreshold_ws_bytes(src)
    if ws is None and need:
        ws = workspace(need, src.k_pages.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.spkv_cache_rethreshold(ctypes.byref(src.desc()), ctypes.byref(dst.desc()), float(tau),
                                      _ptr(ws), ws_bytes, _stream(stream)))


def spkv_head_stats_ws_bytes(n_rows: int, n_kv: int) -> int:
    return int(load_library().spkv_head_stats_ws_bytes(int(n_rows), int(n_kv)))


def spkv_head_stats(utility, keep, u_sum=None, n_kept=None, ws=None, stream=None):
    """Add per-head utility sums (f64) and kept counts (int64) of the rows of
    utility / keep [n_rows, n_kv] (either may be None) to u_sum / n_kept
    (fresh zeros when None).  Returns (u_sum, n_kept)."""
    lib = load_library()
    ref = utility if utility is not None else keep
    if ref is None:
        raise ValueError("utility and keep are both None")
    n, nkv = ref.shape
    dev = ref.device
    _need_gpu(utility, keep, u_sum, n_kept)
    if utility is not None and (utility.dtype != torch.float32 or not utility.is_contiguous()):
        raise ValueError("utility must be contiguous float32")
    if keep is not None and (keep.dtype != torch.uint8 or not keep.is_contiguous()):
        raise ValueError("keep must be contiguous uint8")
    if u_sum is None and utility is not None:
        u_sum = torch.zeros(nkv, dtype=torch.float64, device=dev)
    if n_kept is None and keep is not None:
        n_kept = torch.zeros(nkv, dtype=torch.int64, device=dev)
    need = spkv_head_stats_ws_bytes(n, nkv)
    if ws is None and need:
        ws = workspace(need, dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.spkv_head_stats(_ptr(utility), _ptr(keep), n, nkv, _ptr(u_sum), _ptr(n_kept), _ptr(ws),
                               ws_bytes, _stream(stream)))
    return u_sum, n_kept


def spkv_cache_reset(cache: Cache, stream=None):
    _check(load_library().spkv_cache_reset(ctypes.byref(cache.desc()), _stream(stream)))


def spkv_cache_check(cache: Cache, stream=None) -> int:
    """Synchronise and return the sticky status bits; raises on capacity / row errors."""
    bits = ctypes.c_int32(0)
    rc = load_library().spkv_cache_check(ctypes.byref(cache.desc()), _stream(stream), ctypes.byref(bits))
    if rc != SPKV_OK:
        raise SpkvError(rc, load_library().spkv_last_error().decode() + f" bits={bits.value}")
    return bits.value


def spkv_set_wait_limit(polls: int):
    """Polls after which the fused decode step's bounded waits give up
    (0: at once; negative: the default)."""
    _check(load_library().spkv_set_wait_limit(int(polls)))


def spkv_hbm_read(src, sink, nontemporal: bool = False, runs: bool = False, grid: int = 0, stream=None):
    """Stream every byte of the device tensor ``src`` once (the measured read ceiling).

    ``src`` is contiguous with a byte size that is a multiple of 16384;
    ``sink`` is a device tensor with at least one 4-byte element.  ``runs``:
    every wave reads its own contiguous run of 16 KB blocks, else a
    grid-stride sweep.  ``grid`` 0 takes 8 workgroups per compute unit."""
    if not (src.is_cuda and sink.is_cuda):
        raise ValueError("spkv_hbm_read needs device tensors")
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    if sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("sink needs one 4-byte element")
    nbytes = src.numel() * src.element_size()
    if grid <= 0:
        grid = 8 * torch.cuda.get_device_properties(src.device).multi_processor_count
    flags = (1 if nontemporal else 0) | (2 if runs else 0)
    _check(load_library().spkv_hbm_read(_ptr(src), nbytes, flags, int(grid), _ptr(sink), _stream(stream)))
