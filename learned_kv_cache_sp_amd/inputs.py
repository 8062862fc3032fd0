"""Seeded synthetic inputs for the SP-KV hot path.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no gate, no compaction, no attention), so both the HIP
path and the fp64 oracle can be fed from it.

Workloads (the five layer shapes the library is exercised on):

* ``tiny``        fp32, batch 1, d_model 256, 4 query / 2 key heads, head_dim
                  64, T = 1024, window 128, gate 256 -> 32 -> 2, ~25 % kept;
                  prefill over T, then 16 decode steps.
* ``decode_32k``  bf16 Llama-3-8B-shaped layer (d_model 4096, 32/8 heads,
                  head_dim 128, gate 4096 -> 128 -> 8), batch 8, 32768-token
                  context, ~20 % kept on every head, 256 decode steps.
* ``decode_131k`` same layer, batch 4, 131072-token context, per-key-head keep
                  rates {2, 2, 5, 5, 10, 20, 40, 60} %, 256 decode steps.
* ``prefill_64k`` same layer, batch 1, a 65536-token sequence prefilled in
                  16384-token chunks, ~30 % kept.
* ``ragged_32``   same layer, batch 32, per-sequence contexts uniform in
                  [4096, 65536], ~15 % kept, 1024 decode steps, hidden states
                  gated in 128-row buffers.

The keep rates stand in for the densities reported for trained SP-KV models
(about 30 % of keys kept on validation data, 17-50 % by task, 5-7 % on
needle retrieval); the 16K chunk and the 128-row buffer follow the schedules
of Fast KVzip (chunked prefill; decode hidden-state buffer).  No dataset item
is used anywhere: every tensor is drawn here.

Distributions: hidden states, queries, keys and values are i.i.d. N(0, 1);
W1 ~ N(0, 1/d_model), W2 ~ N(0, 1/d_hidden), b1 = 0.  The output bias b2 is
placed from a sample of pre-bias logits (``place_output_bias``) so that each
key head keeps the requested fraction of tokens.  bf16 workloads round every
bf16 tensor to nearest-even in bf16 here, so the float32 arrays handed to the
oracle hold exactly the values the device sees.

CPU arrays come from numpy's PCG64 (``SeedSequence([seed, *stream])``);
device tensors for the large workloads come from torch's seeded device
generator.  The two generators give different (but equally distributed)
numbers; every test feeds the same drawn values to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                    # "f32" or "bf16"
    batch: int
    d_model: int
    n_q: int
    n_kv: int
    head_dim: int
    window: int
    d_hidden: int
    tau: float
    keep: tuple                   # target keep fraction per key head
    context: int                  # prefix length (decode) or sequence length (prefill)
    decode_steps: int = 0
    chunk: int = 0                # prefill chunk (0 = whole sequence)
    buffer: int = 0               # hidden-state buffer for buffered gating (0 = per token)
    ragged: tuple = field(default=())  # (lo, hi) for per-sequence contexts
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


WORKLOADS = {
    "tiny": Workload("tiny", "f32", 1, 256, 4, 2, 64, 128, 32, 0.5, (0.25, 0.25),
                     1024, decode_steps=16, seed=1001),
    "decode_32k": Workload("decode_32k", "bf16", 8, 4096, 32, 8, 128, 128, 128, 0.5,
                           (0.20,) * 8, 32768, decode_steps=256, seed=1002),
    "decode_131k": Workload("decode_131k", "bf16", 4, 4096, 32, 8, 128, 128, 128, 0.5,
                            (0.02, 0.02, 0.05, 0.05, 0.10, 0.20, 0.40, 0.60), 131072,
                            decode_steps=256, seed=1003),
    "prefill_64k": Workload("prefill_64k", "bf16", 1, 4096, 32, 8, 128, 128, 128, 0.5,
                            (0.30,) * 8, 65536, chunk=16384, seed=1004),
    "ragged_32": Workload("ragged_32", "bf16", 32, 4096, 32, 8, 128, 128, 128, 0.5,
                          (0.15,) * 8, 65536, decode_steps=1024, buffer=128,
                          ragged=(4096, 65536), seed=1005),
}


# ----------------------------------------------------------------------------
# numpy generators
# ----------------------------------------------------------------------------

def rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); NaN stays NaN.

    A data-type conversion: the result is a float32 array holding bf16 values."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = x[nan]
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that already hold bf16 values."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


STREAM_W1, STREAM_W2, STREAM_H, STREAM_Q, STREAM_K, STREAM_V, STREAM_CAL, STREAM_RESAMPLE, \
    STREAM_MASK, STREAM_CTX, STREAM_UTIL = range(11)


def layer_weights(wl: Workload, seed: int | None = None) -> dict:
    """W1 [d_hidden, d_model], b1 [d_hidden], W2 [n_kv, d_hidden], b2 [n_kv] (zeros)."""
    s = wl.seed if seed is None else seed
    w1 = rng(s, STREAM_W1).standard_normal((wl.d_hidden, wl.d_model), dtype=np.float32)
    w1 *= np.float32(1.0 / math.sqrt(wl.d_model))
    w2 = rng(s, STREAM_W2).standard_normal((wl.n_kv, wl.d_hidden), dtype=np.float32)
    w2 *= np.float32(1.0 / math.sqrt(wl.d_hidden))
    return {
        "W1": _cast(w1, wl.dtype),
        "b1": np.zeros((wl.d_hidden,), np.float32),
        "W2": w2.astype(np.float32),          # second layer stays float32
        "b2": np.zeros((wl.n_kv,), np.float32),
    }


def normal(shape, seed: int, *stream: int, dtype: str = "f32") -> np.ndarray:
    """i.i.d. N(0, 1) in float32 (bf16-rounded when dtype == 'bf16')."""
    x = rng(seed, *stream).standard_normal(shape, dtype=np.float32)
    return _cast(x, dtype)


def tokens(wl: Workload, n: int, seed: int, *stream: int) -> dict:
    """Hidden states H [n, d_model], Q [n, n_q, hd], K/V [n, n_kv, hd]."""
    hd = wl.head_dim
    return {
        "H": normal((n, wl.d_model), seed, STREAM_H, *stream, dtype=wl.dtype),
        "Q": normal((n, wl.n_q, hd), seed, STREAM_Q, *stream, dtype=wl.dtype),
        "K": normal((n, wl.n_kv, hd), seed, STREAM_K, *stream, dtype=wl.dtype),
        "V": normal((n, wl.n_kv, hd), seed, STREAM_V, *stream, dtype=wl.dtype),
    }


def bernoulli_mask(n: int, rates, seed: int, *stream: int) -> np.ndarray:
    """Keep bits [n, len(rates)] drawn independently with the given rates."""
    r = rng(seed, STREAM_MASK, *stream).random((n, len(rates)))
    return (r < np.asarray(rates)[None, :]).astype(np.uint8)


def utilities(n: int, n_kv: int, seed: int, *stream: int) -> np.ndarray:
    """Stored utilities [n, n_kv] float32: uniform in [0, 1), with exact ties
    at 0.5 and 0.75 on about 1/8 and 1/16 of the entries and NaN on about
    1/64 (a utility the threshold comparison must drop)."""
    r = rng(seed, STREAM_UTIL, *stream)
    u = r.random((n, n_kv)).astype(np.float32)
    pick = r.random((n, n_kv))
    u[pick < 1 / 8] = np.float32(0.5)
    u[(pick >= 1 / 8) & (pick < 3 / 16)] = np.float32(0.75)
    u[(pick >= 3 / 16) & (pick < 3 / 16 + 1 / 64)] = np.float32(np.nan)
    return u


def ragged_contexts(wl: Workload, seed: int | None = None) -> np.ndarray:
    """Per-sequence context lengths, uniform integers in [lo, hi]."""
    s = wl.seed if seed is None else seed
    if not wl.ragged:
        return np.full((wl.batch,), wl.context, np.int64)
    lo, hi = wl.ragged
    return rng(s, STREAM_CTX).integers(lo, hi + 1, size=wl.batch).astype(np.int64)


def place_output_bias(prebias_logits: np.ndarray, keep, tau: float) -> np.ndarray:
    """Output bias b2 so that a fraction keep[k] of the sample clears the threshold.

    prebias_logits [n, n_kv] are the second-layer outputs without b2 on a
    calibration sample (computed by the caller).  The threshold tau on the
    sigmoid output is the threshold log(tau / (1 - tau)) on the logit, so
    b2[k] = log(tau/(1-tau)) - quantile(prebias_logits[:, k], 1 - keep[k])."""
    z = np.asarray(prebias_logits, dtype=np.float64)
    t_logit = math.log(tau / (1.0 - tau))
    b2 = np.array([t_logit - np.quantile(z[:, k], 1.0 - keep[k]) for k in range(z.shape[1])])
    return b2.astype(np.float32)


# ----------------------------------------------------------------------------
# torch device generators (large workloads; values differ from numpy's)
# ----------------------------------------------------------------------------

def device_normal(shape, seed: int, stream: int, torch_dtype, device="cuda"):
    """i.i.d. N(0, 1) drawn with torch's seeded generator on `device`, cast to torch_dtype
    (round-to-nearest-even for bfloat16)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(stream))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch_dtype)


def device_bernoulli_mask(n: int, rates, seed: int, stream: int, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + 7919 * int(stream) + 17)
    r = torch.rand((n, len(rates)), generator=g, device=device)
    return (r < torch.tensor(list(rates), device=device)[None, :]).to(torch.uint8)
