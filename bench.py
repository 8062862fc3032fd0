#!/usr/bin/env python3
"""Benchmark of the SP-KV hot path on one MI355X.

Default workload ``decode_32k``: one Llama-3-8B-shaped attention layer
(d_model 4096, 32 query / 8 key heads, head_dim 128, gate 4096 -> 128 -> 8),
bf16, batch 8, 32768-token context, ~20 % of tokens kept per key head,
window 128.  One step = the whole decode path for one new token of every
sequence:

    spkv_gate           hidden rows -> utilities and keep bits (Eq. 1-2)
    spkv_compact_append keep bits + K/V -> persistent cache and window ring
    spkv_decode_attn    every query head of every sequence over window + kept keys

run as one spkv_decode_step launch that does all three (``--step-mode
separate`` times the three calls instead).

Other workloads (``--workload``): ``decode_131k`` (batch 4, 131072 tokens,
per-head keep 2-60 %), ``ragged_32`` (batch 32, contexts 4096-65536, 15 %,
hidden states buffered: window append + attention every step -- one
spkv_decode_step launch without gate -- and gate + kept append of all
32 x 128 buffered rows every 128 steps), ``prefill_64k``
(one step = chunked prefill of a 65536-token sequence in 16384-token chunks:
gate, kept append, prefill attention, window append per chunk),
``rethreshold_32k`` (one step = rebuild of the decode_32k cache at a higher
threshold that keeps half of its entries) and ``head_stats_1m`` (one step =
per-head utility sums and kept counts of 1,048,576 gate rows x 8 heads)
and ``soft_prefill_16k`` (one step = forward of the soft relaxation of
Eq. 5-6 over a 16384-token sequence).

Inputs are synthetic (seeded) and resident in HBM before timing starts.
Decode prefixes are gated and compacted through the same calls during set-up.
Several independent layer caches are used in rotation so that one step's
working set cannot stay in the 256 MB Infinity Cache between its visits: the
figures are HBM figures, as for a model whose every layer owns its cache.

Prints ONE JSON line.  ``roofline`` is for the dominant kernel: decode
attention (algorithmic bytes = visible kept + window entries x 512 B per
launch, plus the gate's and the appends' bytes in the fused step) or prefill
attention (4 hd flops per visible (row, key) pair and query head).  Decode
workloads with one launch per step take the launch time from the timed pass
(its time per step, an upper bound of the launch); prefill takes it from a
second pass with HIP events around each launch on the launch stream.
``traffic`` is read from the committed rocprofv3 counter summary for that
kernel and workload when its recorded source hash matches the kernel source
in this tree, else null.  ``hbm_ceiling`` is the library's streaming-read
kernel (spkv_hbm_read) at the decode launch's byte count and at 2 GiB, and
the decode roofline also gives its fraction of that measured ceiling.
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on every host core this process may use (nproc, affinity, cgroup
quota and CPU model recorded).  The default decode_32k run also carries a
``secondary`` list: decode_131k, ragged_32, prefill_64k and the batch-16
pair decode_32k_b16 / decode_32k_b16_tau0 (keep rates against every pair
kept, with their per-step ratio in ``sparse_vs_full_batch16``), each measured
the same way with its own default steps.

Profile summaries (no GPU needed):
    python bench.py --summarize-stats DIR
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --kernel NAME --workload W
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "gated-KV decode tokens/s + achieved HBM GB/s (% of peak), 8B shape 32K ctx"
KERNEL_SOURCES = {
    "decode_bf16_kernel": "learned_kv_cache_sp_amd/csrc/spkv_decode.hip",
    "prefill_bf16_kernel": "learned_kv_cache_sp_amd/csrc/spkv_prefill.hip",
    "gate_bf16_kernel": "learned_kv_cache_sp_amd/csrc/spkv_gate.hip",
    "compact_onepass_kernel": "learned_kv_cache_sp_amd/csrc/spkv_compact.hip",
    "compact_small_kernel": "learned_kv_cache_sp_amd/csrc/spkv_compact.hip",
    "rethresh_scatter_kernel": "learned_kv_cache_sp_amd/csrc/spkv_compact.hip",
    "stats_kernel": "learned_kv_cache_sp_amd/csrc/spkv_stats.hip",
}
CALIBRATION_BYTES = 1 << 30  # the plain copy: 1 GiB read + 1 GiB written


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps of --workload (decode 256, prefill 4; secondary lines take their defaults)")
    p.add_argument("--warmup", type=int, default=None, help="untimed steps (decode 16, prefill 1)")
    p.add_argument("--workload", default="decode_32k",
                   choices=["decode_32k", "decode_131k", "ragged_32", "prefill_64k", "rethreshold_32k",
                            "head_stats_1m", "soft_prefill_16k", "sink_gate_16k", "decode_32k_b16",
                            "decode_32k_b16_tau0"])
    p.add_argument("--layers", type=int, default=4, help="decode: layer caches used in rotation")
    p.add_argument("--page-size", type=int, default=64)
    p.add_argument("--step-mode", choices=("auto", "fused", "separate"), default="auto",
                   help="decode without a gate buffer: one spkv_decode_step launch per step (fused; auto "
                        "where the batch allows) or spkv_gate + spkv_compact_append + spkv_decode_attn")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB elementwise copy (for scaling HBM counters)")
    p.add_argument("--summarize-stats", metavar="DIR")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--summarize-mfma", metavar="DIR",
                   help="matrix-core counters (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, "
                        "SQ_INSTS_VALU_MFMA_MOPS_BF16) per kernel")
    p.add_argument("--no-ceiling", action="store_true", help="skip the measured HBM read ceiling")
    p.add_argument("--no-secondary", action="store_true",
                   help="decode_32k: skip the decode_131k, ragged_32 and prefill_64k lines")
    p.add_argument("--kernel", default="decode_bf16_kernel")
    return p.parse_args()


# ----------------------------------------------------------------------------
# profile summaries and the stored traffic figure
# ----------------------------------------------------------------------------

def _short(name: str) -> str:
    if name.startswith("_Z"):
        # a name the profiler left mangled: keep the kernel identifier
        import re
        m = re.search(r"_GLOBAL__N_1(\d+)", name) or re.search(r"N4spkv(\d+)", name)
        if m:
            k = int(m.group(1))
            return name[m.end():m.end() + k] + "<...>"
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    n = n.replace("spkv::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            n = n[:i]
            break
    return n if len(n) <= 72 else n[:69] + "..."


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def summarize_stats(d: str) -> str:
    rows = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"{'kernel':72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows[:16]:
        out.append(f"{_short(r['Name']):72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    return "\n".join(out)


def _source_hash(kernel: str) -> str:
    path = os.path.join(ROOT, KERNEL_SOURCES[kernel])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def _pmc_means(d: str, counter: str):
    """Per kernel: (dispatches, mean counter value), and the calibration copy's value."""
    per, calib = {}, []
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        if "neg_kernel" in r["Kernel_Name"]:
            calib.append(v)
            continue
        per.setdefault(_short(r["Kernel_Name"]), []).append(v)
    return {k: (len(v), float(np.mean(v))) for k, v in per.items()}, (max(calib) if calib else None)


def summarize_pmc(fetch_dir: str, write_dir: str, kernel: str, workload: str) -> str:
    f_per, f_cal = _pmc_means(fetch_dir, "FETCH_SIZE")
    w_per, w_cal = _pmc_means(write_dir, "WRITE_SIZE")
    if f_cal is None or w_cal is None:
        raise SystemExit("the calibration copy (run with --copy-calibration) is missing")
    f_fac = CALIBRATION_BYTES / (f_cal * 1024.0)
    w_fac = CALIBRATION_BYTES / (w_cal * 1024.0)
    out = [f"calibration copy of {CALIBRATION_BYTES} B: FETCH_SIZE {f_cal:.0f} KiB -> factor {f_fac:.4f}; "
           f"WRITE_SIZE {w_cal:.0f} KiB -> factor {w_fac:.4f}",
           f"{'kernel':72s} {'n':>4s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'scaled_MB':>10s}"]
    for k in sorted(set(f_per) | set(w_per)):
        if not any(x in k for x in ("gate", "compact", "decode", "prefill", "cache_reset", "rethresh", "stats")):
            continue
        nf, fv = f_per.get(k, (0, 0.0))
        _, wv = w_per.get(k, (0, 0.0))
        out.append(f"{k:72s} {nf:4d} {fv:12.1f} {wv:12.1f} {(fv * f_fac + wv * w_fac) * 1024 / 1e6:10.2f}")
    hits = [k for k in f_per if k.startswith(kernel)]
    if hits:
        k = max(hits, key=lambda x: f_per[x][0])
        wv = w_per.get(k, (0, 0.0))[1]
        rec = {"kernel": k, "workload": workload,
               "fetch_kib": round(f_per[k][1], 1), "write_kib": round(wv, 1),
               "fetch_factor": round(f_fac, 5), "write_factor": round(w_fac, 5),
               "bytes_per_launch": round((f_per[k][1] * f_fac + wv * w_fac) * 1024),
               "source": KERNEL_SOURCES[kernel], "source_sha256": _source_hash(kernel)}
        out.append("traffic_json: " + json.dumps(rec))
    return "\n".join(out)


SIMD_NUM = 256 * 4  # MI355X: 256 compute units x 4 SIMDs
XCD_NUM = 8         # GRBM_GUI_ACTIVE comes summed over the XCDs' GRBM instances


def summarize_mfma(d: str) -> str:
    """Matrix-core utilisation per kernel from one counter pass: busy = summed
    MFMA-busy cycles / (GPU-active cycles x SIMDs), the rocprof MfmaUtil
    definition, with the active cycles of one XCD (the counter arrives summed
    over the 8 XCDs: 8x the kernel's duration in cycles); and the bf16 MFMA
    work the counters saw (MOPS x 512 FLOP)."""
    names = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    per = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] in names:
            key = (_short(r["Kernel_Name"]), r.get("Dispatch_Id", ""))
            per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    agg = {}
    for (k, _), v in per.items():
        if all(n in v for n in names):
            agg.setdefault(k, []).append(v)
    out = [f"{'kernel':60s} {'n':>4s} {'MFMA_busy_%':>12s} {'active_cycles':>15s} {'MFMA_TFLOP/disp':>16s}"]
    for k in sorted(agg):
        if not any(x in k for x in ("gate", "compact", "decode", "prefill")):
            continue
        vs = agg[k]
        busy = np.mean([v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / XCD_NUM * SIMD_NUM) for v in vs]) * 100
        gui = np.mean([v["GRBM_GUI_ACTIVE"] / XCD_NUM for v in vs])
        fl = np.mean([v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 for v in vs]) / 1e12
        out.append(f"{k:60s} {len(vs):4d} {busy:12.1f} {gui:15.0f} {fl:16.3f}")
    return "\n".join(out)


def stored_traffic(kernel: str, workload: str, variant: str | None = None):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the kernel source in this tree (and on this instantiation); else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.pmc_traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic_json: "):
            rec = json.loads(line[len("traffic_json: "):])
            if variant is not None and rec.get("kernel") != variant:
                return None
            if rec.get("workload") == workload and rec.get("source_sha256") == _source_hash(kernel):
                return float(rec["bytes_per_launch"])
    return None


# ----------------------------------------------------------------------------
# shared set-up
# ----------------------------------------------------------------------------

def gate_weights(wl, torch, inputs, spkv, dev):
    """Gate weights with the output bias placed for the workload's keep rates on
    65536 device-drawn calibration rows (evaluated by the gate itself)."""
    wts = inputs.layer_weights(wl)
    gw = spkv.GateWeights(torch.from_numpy(wts["W1"]).to(dev).to(torch.bfloat16),
                          torch.from_numpy(wts["b1"]).to(dev), torch.from_numpy(wts["W2"]).to(dev),
                          torch.zeros(wl.n_kv, dtype=torch.float32, device=dev))
    if wl.tau <= 0.0:
        return gw  # tau = 0 keeps every pair whatever the bias
    Hc = inputs.device_normal((65536, wl.d_model), wl.seed, inputs.STREAM_CAL, torch.bfloat16)
    u_cal, _ = spkv.spkv_gate(gw, Hc, wl.tau)
    u64 = u_cal.double().clamp(1e-300, 1 - 1e-16)
    logit = (torch.log(u64) - torch.log1p(-u64)).cpu().numpy()
    gw.b2.copy_(torch.from_numpy(inputs.place_output_bias(logit, wl.keep, wl.tau)).to(dev))
    return gw


def _stats_us(ms):
    ms = np.asarray(ms)
    return {"mean": round(float(ms.mean() * 1e3), 2),
            "p10_p90": [round(float(np.percentile(ms, 10) * 1e3), 2),
                        round(float(np.percentile(ms, 90) * 1e3), 2)]}


# ----------------------------------------------------------------------------
# decode workloads
# ----------------------------------------------------------------------------

def bench_decode(args, wl):
    import torch
    from learned_kv_cache_sp_amd import inputs, spkv

    dev = "cuda"
    B, d, nq, nkv, hd, w = wl.batch, wl.d_model, wl.n_q, wl.n_kv, wl.head_dim, wl.window
    ctxs = [int(c) for c in inputs.ragged_contexts(wl)]
    P, L = args.page_size, max(1, args.layers)
    steps = 256 if args.steps is None else args.steps
    warm = 16 if args.warmup is None else args.warmup
    buf = wl.buffer if wl.buffer > 0 else 1
    if buf > 1:
        # whole buffer periods, so the timed pass holds its share of gate + append flushes
        steps = -(-steps // (buf * L)) * buf * L
    S = warm + 2 * steps                 # warm-up, the timed pass, the per-launch timing pass
    n_loc = -(-S // L)                   # steps per layer cache
    n_fl = -(-n_loc // buf)              # gate groups per layer cache
    scale = 1.0 / math.sqrt(hd)
    G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW
    seed = wl.seed

    gw = gate_weights(wl, torch, inputs, spkv, dev)

    # ---- prefix: gate + compaction of every sequence's context ---------------
    offs = np.concatenate([[0], np.cumsum(ctxs)]).astype(np.int64)
    n_pre = int(offs[-1])
    grow = n_fl * buf
    max_pages = int(math.ceil((max(ctxs) + grow) / P)) + 2
    n_pages = sum(min(max_pages, int(math.ceil((c + grow) * r / P * 1.25)) + 8) for c in ctxs for r in wl.keep)
    caches = [spkv.Cache(B, nkv, hd, w, P, n_pages, max_pages, torch.bfloat16) for _ in range(L)]
    zpre = torch.empty((n_pre, nkv), dtype=torch.uint8, device=dev)
    ro_pre = torch.tensor(offs, dtype=torch.int32, device=dev)
    pos0 = torch.zeros(B, dtype=torch.int32, device=dev)
    CH = 65536
    for r0 in range(0, n_pre, CH):
        Hp = inputs.device_normal((min(CH, n_pre - r0), d), seed, 1000 + r0 // CH, torch.bfloat16)
        spkv.spkv_gate(gw, Hp, wl.tau, keep=zpre[r0:r0 + Hp.shape[0]])
        del Hp
    Kp = inputs.device_normal((n_pre, nkv, hd), seed, inputs.STREAM_K, torch.bfloat16)
    Vp = inputs.device_normal((n_pre, nkv, hd), seed, inputs.STREAM_V, torch.bfloat16)
    for c in caches:
        spkv.spkv_compact_append(c, zpre, Kp, Vp, ro_pre, pos0, max(ctxs), G_ | W_)
    torch.cuda.synchronize()
    for c in caches:
        spkv.spkv_cache_check(c)
    del Kp, Vp
    kept_frac = zpre.float().mean(0).cpu().numpy()

    # ---- per-step inputs, laid out per layer cache and gate group -------------
    # a gate group holds `buf` consecutive tokens of every sequence, sequence-major
    Hl = inputs.device_normal((L, n_fl, B, buf, d), seed, 2001, torch.bfloat16)
    Ql = inputs.device_normal((L, n_loc, B, nq, hd), seed, 2002, torch.bfloat16)
    Kl = inputs.device_normal((L, n_fl, B, buf, nkv, hd), seed, 2003, torch.bfloat16)
    Vl = inputs.device_normal((L, n_fl, B, buf, nkv, hd), seed, 2004, torch.bfloat16)
    ctx_t = torch.tensor(ctxs, dtype=torch.int32, device=dev)
    tpos = (ctx_t[None, :] + torch.arange(n_loc, dtype=torch.int32, device=dev)[:, None]).contiguous()
    gpos = (ctx_t[None, :] + buf * torch.arange(n_fl, dtype=torch.int32, device=dev)[:, None]).contiguous()
    zl = torch.zeros((L, n_fl, B, buf, nkv), dtype=torch.uint8, device=dev)
    ul = torch.zeros((L, n_fl, B, buf, nkv), dtype=torch.float32, device=dev)
    ro1 = torch.arange(0, B + 1, dtype=torch.int32, device=dev)
    robuf = (ro1 * buf).contiguous()
    out = torch.empty((B, nq, hd), dtype=torch.float32, device=dev)
    lse = torch.empty((B, nq), dtype=torch.float32, device=dev)
    gate_ws = spkv.workspace(spkv.spkv_gate_ws_bytes(gw, B * buf))
    comp_ws = spkv.workspace(spkv.spkv_compact_ws_bytes(caches[0], B * buf, buf))
    # fused: one spkv_decode_step launch per step -- with the gate (no buffer,
    # up to 16 sequences) or, with a gate buffer, the window append only
    fused = buf == 1 and args.step_mode != "separate" and B <= 16
    ring = buf > 1 and args.step_mode != "separate"
    if args.step_mode == "fused" and not (fused or ring):
        raise SystemExit("the fused step with a gate takes up to 16 sequences")
    if fused:
        dec_ws = [spkv.workspace(spkv.spkv_decode_step_ws_bytes(c, gw, nq)) for c in caches]
    else:
        dec_ws = [spkv.workspace(spkv.spkv_decode_ws_bytes(c, nq)) for c in caches]

    # pre-marshalled raw calls (keeps host overhead far below the GPU time)
    lib = spkv.load_library()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    gdesc = gw.desc()
    cdescs = [c.desc() for c in caches]

    def pn(t):
        return (None, 0) if t is None else (t.data_ptr(), t.numel() * t.element_size())

    gws, cws = pn(gate_ws), pn(comp_ws)
    dws = [pn(x) for x in dec_ws]
    ld_step = buf * nkv * hd
    ev = {}

    def record(key):
        if key is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            ev.setdefault(key, []).append(e)

    def pre(s):
        """work of step s before its decode: gate + append (or window append)"""
        if fused or ring:
            return
        l, i = s % L, s // L
        f, j = i // buf, i % buf
        cd = ctypes.byref(cdescs[l])
        rc = 0
        if buf == 1:
            rc |= lib.spkv_gate(ctypes.byref(gdesc), Hl[l, f].data_ptr(), B, d, wl.tau, ul[l, f].data_ptr(),
                                zl[l, f].data_ptr(), gws[0], gws[1], sp)
            rc |= lib.spkv_compact_append(cd, zl[l, f].data_ptr(), None, Kl[l, f].data_ptr(), Vl[l, f].data_ptr(),
                                          nkv * hd, ro1.data_ptr(), tpos[i].data_ptr(), B, 1, G_ | W_, None,
                                          cws[0], cws[1], sp)
        else:
            rc |= lib.spkv_compact_append(cd, None, None, Kl[l, f, 0, j].data_ptr(), Vl[l, f, 0, j].data_ptr(),
                                          ld_step, ro1.data_ptr(), tpos[i].data_ptr(), B, 1, W_, None,
                                          cws[0], cws[1], sp)
        if rc:
            raise RuntimeError(lib.spkv_last_error().decode())

    def dec(s):
        l, i = s % L, s // L
        if fused:
            rc = lib.spkv_decode_step(ctypes.byref(cdescs[l]), ctypes.byref(gdesc), nq, Hl[l, i].data_ptr(), d,
                                      wl.tau, Kl[l, i].data_ptr(), Vl[l, i].data_ptr(), nkv * hd,
                                      Ql[l, i].data_ptr(), nq * hd, tpos[i].data_ptr(), scale, ul[l, i].data_ptr(),
                                      zl[l, i].data_ptr(), out.data_ptr(), lse.data_ptr(), dws[l][0], dws[l][1],
                                      sp)
            if rc:
                raise RuntimeError(lib.spkv_last_error().decode())
            return
        if ring:
            f, j = i // buf, i % buf
            rc = lib.spkv_decode_step(ctypes.byref(cdescs[l]), None, nq, None, 0, wl.tau, Kl[l, f, 0, j].data_ptr(),
                                      Vl[l, f, 0, j].data_ptr(), ld_step, Ql[l, i].data_ptr(), nq * hd,
                                      tpos[i].data_ptr(), scale, None, None, out.data_ptr(), lse.data_ptr(),
                                      dws[l][0], dws[l][1], sp)
            if rc:
                raise RuntimeError(lib.spkv_last_error().decode())
            return
        rc = lib.spkv_decode_attn(ctypes.byref(cdescs[l]), nq, Ql[l, i].data_ptr(), nq * hd, tpos[i].data_ptr(),
                                  scale, out.data_ptr(), lse.data_ptr(), dws[l][0], dws[l][1], sp)
        if rc:
            raise RuntimeError(lib.spkv_last_error().decode())

    def post(s, timing=False):
        """after the decode: a full buffer of this layer cache is gated and its kept rows appended"""
        l, i = s % L, s // L
        f, j = i // buf, i % buf
        if buf > 1 and j == buf - 1:
            cd = ctypes.byref(cdescs[l])
            record("f0" if timing else None)
            rc = lib.spkv_gate(ctypes.byref(gdesc), Hl[l, f].data_ptr(), B * buf, d, wl.tau,
                               ul[l, f].data_ptr(), zl[l, f].data_ptr(), gws[0], gws[1], sp)
            rc |= lib.spkv_compact_append(cd, zl[l, f].data_ptr(), None, Kl[l, f].data_ptr(), Vl[l, f].data_ptr(),
                                          nkv * hd, robuf.data_ptr(), gpos[f].data_ptr(), B * buf, buf, G_,
                                          None, cws[0], cws[1], sp)
            record("f1" if timing else None)
            if rc:
                raise RuntimeError(lib.spkv_last_error().decode())

    def step(s):
        pre(s)
        dec(s)
        post(s)

    for s in range(warm):
        step(s)
    torch.cuda.synchronize()
    # pass 1 (the figure of merit): K whole steps, bracketed by two events
    t0 = time.perf_counter()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_start.record(stream)
    for s in range(warm, warm + steps):
        step(s)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e_start.elapsed_time(e_end)
    # pass 2: the same number of steps again, L at a time (one per layer
    # cache, independent of each other): the pre-decode work of the L steps,
    # then their L decode launches back to back between two events, then the
    # post-decode work.  The per-launch time is the bracket over L, so the
    # event overhead is spread over L launches and stays out of pass 1.
    for s0 in range(warm + steps, S, L):
        group = list(range(s0, min(S, s0 + L)))
        for s in group:
            pre(s)
        record("d0")
        for s in group:
            dec(s)
        record("d1")
        ev.setdefault("n", []).append(len(group))
        for s in group:
            post(s, timing=True)
    torch.cuda.synchronize()
    for c in caches:
        spkv.spkv_cache_check(c)

    # ---- bytes each decode launch had to read --------------------------------
    # visible entries of (b, g) at position t: window min(t+1, w) + kept positions <= t - w
    zpre_h = zpre.cpu().numpy().astype(np.int64)
    Epre = np.vstack([np.zeros((1, nkv), np.int64), np.cumsum(zpre_h, 0)])
    zl_h = zl.cpu().numpy().astype(np.int64)              # [L, n_fl, B, buf, nkv]
    Estep = np.zeros((L, B, n_fl * buf + 1, nkv), np.int64)
    for l in range(L):
        for b in range(B):
            Estep[l, b, 1:] = np.cumsum(zl_h[l, :, b].reshape(n_fl * buf, nkv), 0)
    # one decode launch per step (fused / ring): the launch time is taken from
    # the timed pass itself -- its time per step, an upper bound of the launch
    # duration -- and the bytes from the same steps; the separate mode has
    # other launches in its steps and takes the second pass's brackets
    one_launch = fused or ring
    byte_steps = range(warm, warm + steps) if one_launch else range(warm + steps, S)
    bytes_per = []
    for s in byte_steps:
        l, i = s % L, s // L
        tot = 0
        for b in range(B):
            t = ctxs[b] + i
            p = t - w
            if p >= 0:
                q = min(p, ctxs[b] - 1)
                vis = Epre[offs[b] + q + 1] - Epre[offs[b]]
                if p >= ctxs[b]:
                    vis = vis + Estep[l, b, p - ctxs[b] + 1]
                tot += int(vis.sum())
            tot += nkv * min(t + 1, w)
        extra = 0
        if ring:
            extra = 2 * B * nkv * hd * 2 * 2  # new K/V rows read and written to the ring
        if fused:
            # the launch also reads W1 and the hidden rows (gate), reads the new
            # K/V rows and writes them to the ring, and writes the kept ones
            # (K, V, position) to the pages
            kept_now = int(zl_h[l, i].sum())
            extra = (wl.d_hidden * d * 2 + B * d * 2 + 2 * B * nkv * hd * 2 * 2
                     + kept_now * (2 * hd * 2 + 4))
        bytes_per.append(float(tot * 2 * hd * 2 + extra))
    bytes_per = np.array(bytes_per)
    grp_ms = np.array([a.elapsed_time(b) for a, b in zip(ev["d0"], ev["d1"])])
    dec_ms = grp_ms / np.array(ev["n"])          # mean launch time within each bracket
    launch_ms = gpu_ms / steps if one_launch else float(grp_ms.sum() / sum(ev["n"]))
    achieved = float(bytes_per.mean() / (launch_ms * 1e-3) / 1e9)

    res = {
        "metric": METRIC,
        "value": round(B * steps / (gpu_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(gpu_ms / steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B,
                   "context": ctxs[0] if not wl.ragged else {"min": min(ctxs), "max": max(ctxs),
                                                             "mean": round(float(np.mean(ctxs)), 1)},
                   "d_model": d, "n_q_heads": nq, "n_kv_heads": nkv, "head_dim": hd, "window": w,
                   "gate": f"{d}->{wl.d_hidden}->{nkv}", "keep_target": list(wl.keep),
                   "keep_measured": [round(float(x), 4) for x in kept_frac],
                   "page_size": P, "layer_caches_rotated": L, "gate_buffer": buf,
                   "step": ("spkv_decode_step: gate, kept-row + window append and decode attention in "
                            "one launch (one token per sequence)" if fused else
                            "spkv_gate + spkv_compact_append + spkv_decode_attn (one token per sequence)"
                            if buf == 1 else
                            f"spkv_decode_step without gate (window append + attention) every step; spkv_gate + "
                            f"spkv_compact_append(kept) of {B}x{buf} buffered rows when a buffer fills" if ring else
                            f"spkv_compact_append(window) + spkv_decode_attn every step; spkv_gate + "
                            f"spkv_compact_append(kept) of {B}x{buf} buffered rows when a buffer fills")},
        "roofline": {"bound": "hbm", "kernel": "decode_bf16_kernel (%s)" % (
                         "spkv_decode_step" if fused else "spkv_decode_step, no gate" if ring else "spkv_decode_attn"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic("decode_bf16_kernel", wl.name,
                                               f"decode_bf16_kernel<{hd}, {1 if fused else 2 if ring else 0}>"),
                     "bytes_per_launch": float(bytes_per.mean()),
                     "launch_us": round(launch_ms * 1e3, 2),
                     "launch_us_from": ("the timed pass: its time per step (one launch per step), an upper "
                                        "bound of the launch duration" if one_launch else
                                        f"a second pass: brackets of {L} back-to-back launches"),
                     "bracketed_launch_us": _stats_us(dec_ms), "launches_per_bracket": L},
        "host_wall_s": round(wall, 4),
    }
    if "f0" in ev:
        fl_ms = np.array([a.elapsed_time(b) for a, b in zip(ev["f0"], ev["f1"])])
        res["buffer_flush"] = {"rows": B * buf, "every_n_steps_per_layer": buf, "us": _stats_us(fl_ms),
                               "in_timed_pass": sum(1 for s in range(warm, warm + steps)
                                                    if (s // L) % buf == buf - 1)}
    return res


# ----------------------------------------------------------------------------
# chunked prefill
# ----------------------------------------------------------------------------

def bench_prefill(args, wl):
    import torch
    from learned_kv_cache_sp_amd import inputs, spkv

    dev = "cuda"
    d, nq, nkv, hd, w = wl.d_model, wl.n_q, wl.n_kv, wl.head_dim, wl.window
    T, CH, G = wl.context, wl.chunk, wl.group
    P = args.page_size
    steps = 4 if args.steps is None else args.steps
    warm = 1 if args.warmup is None else args.warmup
    scale = 1.0 / math.sqrt(hd)
    G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW
    seed = wl.seed

    gw = gate_weights(wl, torch, inputs, spkv, dev)
    H = inputs.device_normal((T, d), seed, inputs.STREAM_H, torch.bfloat16)
    Q = inputs.device_normal((T, nq, hd), seed, inputs.STREAM_Q, torch.bfloat16)
    K = inputs.device_normal((T, nkv, hd), seed, inputs.STREAM_K, torch.bfloat16)
    V = inputs.device_normal((T, nkv, hd), seed, inputs.STREAM_V, torch.bfloat16)
    per = -(-T // P) + 2
    cache = spkv.Cache(1, nkv, hd, w, P, nkv * per, per, torch.bfloat16)
    z = torch.zeros((T, nkv), dtype=torch.uint8, device=dev)
    u = torch.zeros((T, nkv), dtype=torch.float32, device=dev)
    out = torch.empty((CH, nq, hd), dtype=torch.float32, device=dev)
    lse = torch.empty((CH, nq), dtype=torch.float32, device=dev)
    chunks = [(c0, min(CH, T - c0)) for c0 in range(0, T, CH)]
    ro = [torch.tensor([0, n], dtype=torch.int32, device=dev) for _, n in chunks]
    p0 = [torch.tensor([c0], dtype=torch.int32, device=dev) for c0, _ in chunks]
    gate_ws = spkv.workspace(spkv.spkv_gate_ws_bytes(gw, CH))
    comp_ws = spkv.workspace(spkv.spkv_compact_ws_bytes(cache, CH, CH))
    pre_ws = spkv.workspace(spkv.spkv_prefill_ws_bytes(cache, nq, CH))
    stream = torch.cuda.current_stream()
    ev = {}

    def record(key):
        if key is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            ev.setdefault(key, []).append(e)

    def step(timing=False):
        spkv.spkv_cache_reset(cache)
        for k, (c0, n) in enumerate(chunks):
            record("g0" if timing else None)
            spkv.spkv_gate(gw, H[c0:c0 + n], wl.tau, utility=u[c0:c0 + n], keep=z[c0:c0 + n], ws=gate_ws)
            record("c0" if timing else None)
            spkv.spkv_compact_append(cache, z[c0:c0 + n], K[c0:c0 + n], V[c0:c0 + n], ro[k], p0[k], n, G_,
                                     ws=comp_ws)
            record("a0" if timing else None)
            spkv.spkv_prefill_attn(cache, 0, Q[c0:c0 + n], K[c0:c0 + n], V[c0:c0 + n], c0, scale,
                                   out=out[:n], lse=lse[:n], ws=pre_ws)
            record("a1" if timing else None)
            spkv.spkv_compact_append(cache, None, K[c0:c0 + n], V[c0:c0 + n], ro[k], p0[k], n, W_, ws=comp_ws)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_start.record(stream)
    for _ in range(steps):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e_start.elapsed_time(e_end)
    for _ in range(steps):
        step(timing=True)
    torch.cuda.synchronize()
    spkv.spkv_cache_check(cache)

    # flops of each prefill launch: 4 hd per visible (row, key) pair and query head
    zh = z.cpu().numpy().astype(np.int64)
    E = np.vstack([np.zeros((1, nkv), np.int64), np.cumsum(zh, 0)])
    t = np.arange(T)
    win = np.minimum(t + 1, w).astype(np.int64)
    kept = np.where((t - w)[:, None] >= 0, E[np.clip(t - w + 1, 0, T)], 0)      # [T, nkv]
    vis = win[:, None] + kept
    flops = np.array([4.0 * hd * G * float(vis[c0:c0 + n].sum()) for c0, n in chunks])
    nc = len(chunks)
    a_ms = np.array([a.elapsed_time(b) for a, b in zip(ev["a0"], ev["a1"])])
    g_ms = np.array([a.elapsed_time(b) for a, b in zip(ev["g0"], ev["c0"])])
    c_ms = np.array([a.elapsed_time(b) for a, b in zip(ev["c0"], ev["a0"])])
    fl = np.tile(flops, steps)
    achieved = float((fl / (a_ms * 1e-3)).mean() / 1e12)
    kept_rows = zh.sum(0)
    res = {
        "metric": "chunked-prefill tokens/s (gate + compaction + masked attention), 8B shape 64K",
        "value": round(T * steps / (gpu_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(gpu_ms / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": 1, "tokens": T, "chunk": CH, "d_model": d, "n_q_heads": nq,
                   "n_kv_heads": nkv, "head_dim": hd, "window": w, "gate": f"{d}->{wl.d_hidden}->{nkv}",
                   "keep_target": list(wl.keep),
                   "keep_measured": [round(float(x), 4) for x in kept_rows / T], "page_size": P,
                   "step": "per chunk: spkv_gate, spkv_compact_append(kept), spkv_prefill_attn, "
                           "spkv_compact_append(window)"},
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel (spkv_prefill_attn)",
                     "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic("prefill_bf16_kernel", wl.name),
                     "flops_per_launch": float(flops.mean()), "launch_us": _stats_us(a_ms)},
        "components_per_chunk": {
            "gate": {"us": _stats_us(g_ms), "hbm_GBs": round(float((CH * d * 2 + wl.d_hidden * d * 2)
                                                                   / (g_ms.mean() * 1e-3) / 1e9), 1),
                     "TFLOPs": round(float(2.0 * CH * d * wl.d_hidden / (g_ms.mean() * 1e-3) / 1e12), 1)},
            "compaction": {"us": _stats_us(c_ms),
                           "hbm_GBs": round(float((2 * kept_rows.sum() / nc * 2 * hd * 2 + CH * nkv)
                                                  / (c_ms.mean() * 1e-3) / 1e9), 1),
                           "launches": "one (spkv_compact_append, GLOBAL, 16384 rows)"},
            "fraction_of_step": {k: round(float(v.mean() * nc / (gpu_ms / steps)), 4)
                                 for k, v in (("gate", g_ms), ("compaction", c_ms), ("attention", a_ms))},
        },
        "host_wall_s": round(wall, 4),
    }
    return res


# ----------------------------------------------------------------------------
# the oracle on the host cores
# ----------------------------------------------------------------------------

def bench_rethreshold(args, wl):
    """Rebuild of the decode_32k cache (8 sequences x 32768 tokens, 20 % of the
    pairs kept at tau) at a higher threshold that keeps about half of its
    entries (SP-KV section 2.1, deployment paragraph: periodic rebuild;
    section 3.3: threshold moved after training).  One step = reset of the
    destination cache + spkv_cache_rethreshold."""
    import torch
    from learned_kv_cache_sp_amd import inputs, spkv
    dev = "cuda"
    B, T, nkv, hd, w, P, d = wl.batch, wl.context, wl.n_kv, wl.head_dim, wl.window, 64, wl.d_model
    G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW
    gw = gate_weights(wl, torch, inputs, spkv, dev)
    n = B * T
    max_pages = T // P + 2
    n_pages = int(B * nkv * (T * max(wl.keep) / P * 1.25 + 8))
    src = spkv.Cache(B, nkv, hd, w, P, n_pages, max_pages, torch.bfloat16, utilities=True)
    dst = spkv.Cache(B, nkv, hd, w, P, n_pages, max_pages, torch.bfloat16, utilities=True)
    dst.share_ring(src)
    z = torch.empty((n, nkv), dtype=torch.uint8, device=dev)
    u = torch.empty((n, nkv), dtype=torch.float32, device=dev)
    CH = 65536
    for r0 in range(0, n, CH):
        Hp = inputs.device_normal((min(CH, n - r0), d), wl.seed, 1000 + r0 // CH, torch.bfloat16)
        spkv.spkv_gate(gw, Hp, wl.tau, utility=u[r0:r0 + Hp.shape[0]], keep=z[r0:r0 + Hp.shape[0]])
        del Hp
    K = inputs.device_normal((n, nkv, hd), wl.seed, inputs.STREAM_K, torch.bfloat16)
    V = inputs.device_normal((n, nkv, hd), wl.seed, inputs.STREAM_V, torch.bfloat16)
    ro = torch.arange(0, n + 1, T, dtype=torch.int32, device=dev)
    spkv.spkv_compact_append(src, z, K, V, ro, torch.zeros(B, dtype=torch.int32, device=dev), T, G_ | W_,
                             utility=u)
    torch.cuda.synchronize()
    spkv.spkv_cache_check(src)
    del K, V
    kept_u = u[z.bool()]
    tau2 = float(torch.quantile(kept_u[:: max(1, kept_u.numel() // (1 << 24))].double(), 0.5))
    ws = spkv.workspace(spkv.spkv_rethreshold_ws_bytes(src))
    stream = torch.cuda.current_stream()

    def step(ev=None):
        spkv.spkv_cache_reset(dst)
        if ev is not None:
            ev[0].record(stream)
        spkv.spkv_cache_rethreshold(src, dst, tau2, ws=ws)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    spkv.spkv_cache_check(dst)
    ms = e0.elapsed_time(e1) / args.steps
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    L_src = int(src.lengths.sum().item())
    L_dst = int(dst.lengths.sum().item())
    # algorithmic bytes of one rebuild: every stored utility read once; each
    # surviving entry's key and value rows (2 * hd bf16), position and
    # utility read and written
    ent = 2 * hd * 2
    alg = 4 * L_src + L_dst * ((ent + 4) + (ent + 8))
    call_s = float(np.mean(call_ms)) * 1e-3
    achieved = alg / call_s / 1e9
    return {
        "metric": "cache entries re-thresholded per second", "value": L_src / (ms * 1e-3),
        "unit": "entries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rethreshold_32k", "batch": B, "context": T, "n_kv": nkv, "head_dim": hd,
                   "page_size": P, "tau": wl.tau, "tau2": tau2, "entries_src": L_src, "entries_dst": L_dst,
                   "step": "spkv_cache_reset(dst) + spkv_cache_rethreshold(src, dst, tau2)"},
        "roofline": {"bound": "hbm", "kernel": "spkv_cache_rethreshold (count + plan + scatter kernels)",
                     "achieved": achieved, "peak": 8000.0, "unit": "GB/s", "frac": achieved / 8000.0,
                     "traffic": stored_traffic("rethresh_scatter_kernel", "rethreshold_32k"),
                     "algorithmic_bytes_per_launch": alg, "avg_call_us": call_s * 1e6,
                     "call_us": _stats_us(call_ms)},
        "wall_s": wall,
    }


def bench_soft_prefill(args, wl):
    """Forward of the soft relaxation (SP-KV section 2.1, Eq. 5-6) over one
    16384-token sequence of the 8B-shaped layer: every token enters the cache
    with its utility, then spkv_prefill_attn_soft attends over all causal keys
    (window keys unmasked, the others with c (alpha - 1), beta = 0.01,
    c = 1e6).  One step = cache reset + GLOBAL append of the 16384 rows +
    soft prefill attention + WINDOW append."""
    import torch
    from learned_kv_cache_sp_amd import inputs, spkv
    T, nq, nkv, hd, w, P = 16384, wl.n_q, wl.n_kv, wl.head_dim, wl.window, 64
    G_, W_ = spkv.SPKV_APPEND_GLOBAL, spkv.SPKV_APPEND_WINDOW
    beta, cmask = 0.01, 1e6
    per_head = T // P + 2
    cache = spkv.Cache(1, nkv, hd, w, P, nkv * per_head, per_head, torch.bfloat16, utilities=True)
    Q = inputs.device_normal((T, nq, hd), wl.seed, inputs.STREAM_Q, torch.bfloat16)
    K = inputs.device_normal((T, nkv, hd), wl.seed, inputs.STREAM_K, torch.bfloat16)
    V = inputs.device_normal((T, nkv, hd), wl.seed, inputs.STREAM_V, torch.bfloat16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    u = torch.rand((T, nkv), generator=gen, device="cuda", dtype=torch.float32)
    keep = torch.ones((T, nkv), dtype=torch.uint8, device="cuda")
    ro = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    p0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((T, nq, hd), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, nq), dtype=torch.float32, device="cuda")
    cws = spkv.workspace(spkv.spkv_compact_ws_bytes(cache, T, T))
    scale = 1.0 / math.sqrt(hd)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        spkv.spkv_cache_reset(cache)
        spkv.spkv_compact_append(cache, keep, K, V, ro, p0, T, G_, ws=cws, utility=u)
        if ev is not None:
            ev[0].record(stream)
        spkv.spkv_prefill_attn(cache, 0, Q, K, V, 0, scale, out=out, lse=lse, soft=(wl.tau, beta, cmask))
        if ev is not None:
            ev[1].record(stream)
        spkv.spkv_compact_append(cache, None, K, V, ro, p0, T, W_, ws=cws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    e1.record(stream)
    torch.cuda.synchronize()
    spkv.spkv_cache_check(cache)
    ms = e0.elapsed_time(e1) / args.steps
    a_ms = np.array([a.elapsed_time(b) for a, b in evs])
    pairs = T * (T + 1) // 2          # every causal (row, key) pair, per query head
    flops = pairs * nq * 4 * hd        # q.k and p.v, 2 flops per multiply-add
    a_s = float(np.mean(a_ms)) * 1e-3
    achieved = flops / a_s / 1e12
    return {
        "metric": "soft-mask forward tokens/s (Eq. 5-6, 8B shape, 16K tokens)", "value": T / (ms * 1e-3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "soft_prefill_16k", "tokens": T, "n_q_heads": nq, "n_kv_heads": nkv,
                   "head_dim": hd, "window": w, "tau": wl.tau, "beta": beta, "c": cmask,
                   "step": "spkv_cache_reset + spkv_compact_append(GLOBAL, keep all, utilities) + "
                           "spkv_prefill_attn_soft + spkv_compact_append(WINDOW)"},
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel<128, true> (spkv_prefill_attn_soft)",
                     "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s", "frac": achieved / 2500.0,
                     "traffic": None, "flops_per_launch": flops, "launch_us": _stats_us(a_ms)},
    }


def cpu_baseline_soft(wl, budget_s: float) -> dict:
    """The oracle's soft-mask attention for sampled rows of a 16384-token
    sequence (all 32 query heads per row), timed for about budget_s."""
    import oracle
    from learned_kv_cache_sp_amd import inputs
    oracle.build(force=False)
    T, nq, nkv, hd = 16384, wl.n_q, wl.n_kv, wl.head_dim
    th = _threads()
    K = inputs.normal((T, nkv, hd), 1, 2, dtype="bf16")
    V = inputs.normal((T, nkv, hd), 1, 3, dtype="bf16")
    u = np.random.default_rng(1).random((T, nkv)).astype(np.float32)
    rows = done_pairs = 0
    t0 = time.perf_counter()
    r = np.random.default_rng(2)
    while time.perf_counter() - t0 < budget_s:
        t = int(r.integers(0, T))
        q = inputs.normal((1, nq, hd), 1, 10 + rows, dtype="bf16")
        oracle.soft_attention(q, [t], K, V, u, wl.window, wl.tau, 0.01, 1e6, threads=th)
        rows += 1
        done_pairs += t + 1
    el = time.perf_counter() - t0
    # tokens/s of the whole forward at the sampled rate of (row, key) pairs
    pairs_seq = T * (T + 1) / 2
    return {"value": done_pairs / el / pairs_seq * T, "unit": "tokens/s", "cores": th, "kind": "oracle",
            "sample": f"{rows} random rows of a {T}-token sequence, all {nq} heads, {el:.1f} s "
                      f"(scaled by the pairs of the whole forward)"}


SINK_ROWS, SINK_G, SINK_S = 16384, 4, 16


def bench_sink_gate(args, wl):
    """The sink-attention gate of the Fast KVzip page (spkv_gate_sink) over one
    16384-row prefill chunk of the 8B-shaped layer: d_model 4096, 8 key heads,
    4 query heads per key head, the page's S = 16 sinks and d_key = 16;
    weights N(0, 1/d_model) in bf16, sinks N(0, 1).  One step = one call."""
    import torch
    from learned_kv_cache_sp_amd import inputs, spkv
    n, d, nkv, G, S = SINK_ROWS, wl.d_model, wl.n_kv, SINK_G, SINK_S
    W = torch.from_numpy(inputs.normal((nkv, (G + 1) * 16, d), wl.seed, 1) / np.float32(np.sqrt(d)))
    W = W.to(torch.bfloat16).cuda()
    sinks = torch.from_numpy(np.random.default_rng(wl.seed).standard_normal((nkv, S, 16)).astype(np.float32)).cuda()
    g = spkv.SinkGateWeights(W, sinks, G)
    Hs = [inputs.device_normal((n, d), wl.seed, 4000 + i, torch.bfloat16) for i in range(4)]
    u = torch.empty((n, nkv), dtype=torch.float32, device="cuda")
    z = torch.empty((n, nkv), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        spkv.spkv_gate_sink(g, Hs[i % 4], wl.tau, utility=u, keep=z)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        spkv.spkv_gate_sink(g, Hs[i % 4], wl.tau, utility=u, keep=z)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 2.0 * n * d * (G + 1) * 16 * nkv
    achieved = flops / (ms * 1e-3) / 1e12
    return {
        "metric": "sink-attention gate rows/s (Fast KVzip gate, 8B shape)", "value": n / (ms * 1e-3),
        "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "sink_gate_16k", "rows": n, "d_model": d, "n_kv": nkv, "group": G, "n_sinks": S,
                   "d_key": 16, "step": "spkv_gate_sink (one launch; the time per step is the launch's)"},
        "roofline": {"bound": "mfma", "kernel": "gate_sink_tall_kernel<4, 2, 64> (spkv_gate_sink)",
                     "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": flops, "hidden_GBs": round(n * d * 2 / (ms * 1e-3) / 1e9, 1),
                     "launch_us": round(ms * 1e3, 2)},
    }


def cpu_baseline_sink_gate(wl, budget_s: float) -> dict:
    """The oracle's sink gate on 64-row samples of the same shapes until about budget_s."""
    import oracle
    from learned_kv_cache_sp_amd import inputs
    oracle.build(force=False)
    th = _threads()
    d, nkv, G, S = wl.d_model, wl.n_kv, SINK_G, SINK_S
    W = inputs.normal((nkv, (G + 1) * 16, d), wl.seed, 1) / np.float32(np.sqrt(d))
    sinks = np.random.default_rng(wl.seed).standard_normal((nkv, S, 16)).astype(np.float32)
    rows = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        H = inputs.normal((64, d), wl.seed, 4100 + rows, dtype="bf16")
        oracle.sink_gate(H, W, sinks, G, wl.tau, threads=th)
        rows += 64
    el = time.perf_counter() - t0
    return {"value": rows / el, "unit": "rows/s", "cores": th, "kind": "oracle",
            "sample": f"{rows} rows in 64-row calls of oracle.sink_gate, {el:.1f} s"}


HEAD_STATS_ROWS, HEAD_STATS_KV = 1 << 20, 8


HEAD_STATS_COPIES = 8  # input sets rotated so that the 8 x 42 MB exceed the 256 MB Infinity Cache


def bench_head_stats(args):
    """Per-head utility sums and kept counts (SP-KV Table 1 density, section 4
    mean utility) over 1,048,576 gate output rows x 8 key heads (the gate
    outputs of 8 sequences of 131,072 tokens), f32 utilities and u8 keep bits
    from a seeded generator.  One step = one spkv_head_stats call, on one of
    HEAD_STATS_COPIES input sets in turn (so every call reads from HBM); the
    C entry point is called with its arguments marshalled once, so that the
    host keeps ahead of the GPU and the timed pass measures the launches."""
    import ctypes
    import torch
    from learned_kv_cache_sp_amd import spkv
    n, nkv = HEAD_STATS_ROWS, HEAD_STATS_KV
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    sets = []
    for _ in range(HEAD_STATS_COPIES):
        u = torch.rand((n, nkv), generator=gen, device="cuda", dtype=torch.float32)
        z = (torch.rand((n, nkv), generator=gen, device="cuda") < 0.2).to(torch.uint8)
        sets.append((u, z))
    us = torch.zeros(nkv, dtype=torch.float64, device="cuda")
    kp = torch.zeros(nkv, dtype=torch.int64, device="cuda")
    nbytes = spkv.spkv_head_stats_ws_bytes(n, nkv)
    ws = spkv.workspace(nbytes)
    stream = torch.cuda.current_stream()
    lib = spkv.load_library()
    calls = [(ctypes.c_void_p(u.data_ptr()), ctypes.c_void_p(z.data_ptr()), ctypes.c_int64(n), ctypes.c_int32(nkv),
              ctypes.c_void_p(us.data_ptr()), ctypes.c_void_p(kp.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
              ctypes.c_size_t(nbytes), ctypes.c_void_p(stream.cuda_stream)) for u, z in sets]
    fn = lib.spkv_head_stats

    def step(i):
        rc = fn(*calls[i % len(calls)])
        if rc != spkv.SPKV_OK:
            raise spkv.SpkvError(rc, lib.spkv_last_error().decode())
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    alg = 5 * n * nkv  # each utility (4 B) and keep byte read once
    call_s = ms * 1e-3
    achieved = alg / call_s / 1e9
    return {
        "metric": "gate output rows summarised per second", "value": n / (ms * 1e-3), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "head_stats_1m", "rows": n, "n_kv": nkv, "step": "spkv_head_stats",
                   "input_sets_rotated": HEAD_STATS_COPIES},
        "roofline": {"bound": "hbm", "kernel": "spkv_head_stats (stats_kernel<true>, one launch)",
                     "achieved": achieved, "peak": 8000.0, "unit": "GB/s", "frac": achieved / 8000.0,
                     "traffic": stored_traffic("stats_kernel", "head_stats_1m"),
                     "algorithmic_bytes_per_launch": alg, "launch_us": call_s * 1e6,
                     "launch_us_from": "the timed pass: its time per call (one launch per call), an upper bound "
                                       "of the launch duration"},
    }


def cpu_baseline_head_stats(budget_s: float) -> dict:
    """The oracle's per-head sums over repeated 131,072-row x 8-head samples."""
    import oracle
    oracle.build(force=False)
    r = np.random.default_rng(5)
    n = 131072
    u = r.random((n, HEAD_STATS_KV)).astype(np.float32)
    z = (r.random((n, HEAD_STATS_KV)) < 0.2).astype(np.uint8)
    done = calls = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.head_stats(u, z)
        done += n
        calls += 1
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} calls of oracle.head_stats on {n} rows x {HEAD_STATS_KV} heads, {el:.1f} s"}


def cpu_baseline_rethreshold(wl, budget_s: float) -> dict:
    """The oracle's re-threshold over a bounded sample of lists shaped like the
    decode_32k cache (about 6.5k stored utilities per list, from the seeded
    generator, kept at tau), timed alone."""
    import oracle
    from learned_kv_cache_sp_amd import inputs
    oracle.build(force=False)
    n_rows = int(wl.context * max(wl.keep) / 0.5)
    pool = [u[u >= np.float32(wl.tau)] for u in (inputs.utilities(n_rows, 1, wl.seed, i)[:, 0] for i in range(16))]
    done = lists = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        u = pool[lists % len(pool)]
        oracle.rethreshold(u, 0.75)
        done += u.size
        lists += 1
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "entries/s", "cores": 1, "kind": "oracle",
            "sample": f"{lists} lists of {pool[0].size}-{max(p.size for p in pool)} stored utilities "
                      f"({done} entries), oracle.rethreshold only, {el:.1f} s"}


def _threads():
    return host_cpu()[0]


def cpu_baseline_decode(wl, budget_s: float) -> dict:
    """fp64 oracle on a bounded sample of the same decode steps, on the host cores.

    Sample: decode steps of 2 of the sequences at their contexts: the oracle
    gate of each new token and the oracle attention of all query heads over a
    seeded keep mask with the workload's keep rates.  Steps are taken until
    about `budget_s` seconds have passed (at least 2)."""
    import oracle
    from learned_kv_cache_sp_amd import inputs

    threads = _threads()
    ctxs = [int(c) for c in inputs.ragged_contexts(wl)][:2]
    max_steps = 256
    w = inputs.layer_weights(wl)
    work = []
    for b, ctx in enumerate(ctxs):
        T = ctx + max_steps
        tok = {
            "Q": inputs.normal((max_steps, wl.n_q, wl.head_dim), wl.seed, 3001, b, dtype=wl.dtype),
            "K": inputs.normal((T, wl.n_kv, wl.head_dim), wl.seed, 3002, b, dtype=wl.dtype),
            "V": inputs.normal((T, wl.n_kv, wl.head_dim), wl.seed, 3003, b, dtype=wl.dtype),
            "H": inputs.normal((max_steps, wl.d_model), wl.seed, 3004, b, dtype=wl.dtype),
        }
        z = inputs.bernoulli_mask(T, wl.keep, wl.seed, 3005, b)
        work.append((ctx, tok, z))
    n_tok = 0
    t0 = time.perf_counter()
    for i in range(max_steps):
        for ctx, tok, z in work:
            oracle.gate(tok["H"][i:i + 1], w["W1"], w["b1"], w["W2"], w["b2"], wl.tau, threads=threads)
            oracle.attention(tok["Q"][i:i + 1], [ctx + i], tok["K"], tok["V"], z, wl.window, threads=threads)
            n_tok += 1
        if time.perf_counter() - t0 > budget_s and i >= 1:
            break
    dt = time.perf_counter() - t0
    return {"value": round(n_tok / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_tok} sequence-steps of {wl.name} decode at contexts {ctxs}: oracle gate of "
                      f"the new token + oracle attention of all {wl.n_q} query heads over a seeded mask "
                      f"with the workload's keep rates; {dt:.1f} s"}


def cpu_baseline_prefill(wl, budget_s: float) -> dict:
    """fp64 oracle on rows drawn uniformly from the 65536-token sequence: the
    gate of the row and the attention of all its query heads (the mean cost per
    token of the whole prefill), until about `budget_s` seconds have passed."""
    import oracle
    from learned_kv_cache_sp_amd import inputs

    threads = _threads()
    T = wl.context
    w = inputs.layer_weights(wl)
    K = inputs.normal((T, wl.n_kv, wl.head_dim), wl.seed, 3102, dtype=wl.dtype)
    V = inputs.normal((T, wl.n_kv, wl.head_dim), wl.seed, 3103, dtype=wl.dtype)
    z = inputs.bernoulli_mask(T, wl.keep, wl.seed, 3105)
    rows = inputs.rng(wl.seed, 3106).integers(0, T, 4096)
    Q = inputs.normal((len(rows), wl.n_q, wl.head_dim), wl.seed, 3101, dtype=wl.dtype)
    H = inputs.normal((len(rows), wl.d_model), wl.seed, 3104, dtype=wl.dtype)
    n, t0 = 0, time.perf_counter()
    while n < len(rows):
        r = slice(n, n + 8)
        oracle.gate(H[r], w["W1"], w["b1"], w["W2"], w["b2"], wl.tau, threads=threads)
        oracle.attention(Q[r], rows[r], K, V, z, wl.window, threads=threads)
        n += len(rows[r])
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} rows drawn uniformly from the {T}-token sequence: oracle gate + oracle attention "
                      f"of all {wl.n_q} query heads over a seeded mask with keep {wl.keep[0]}; {dt:.1f} s"}


def hbm_ceiling(torch, decode_bytes: float | None) -> dict:
    """The measured read ceiling: spkv_hbm_read, the library's streaming-read
    kernel (16-byte loads, nothing computed), over every access order, hint
    and grid it offers.  Two sizes: the bytes of one decode launch, read from
    regions rotated over 1.5 GB so that none is still in the 256 MB Infinity
    Cache when it is read again (as the decode launches' layer caches are),
    and a 2 GiB buffer.  Launches are timed back to back, 16 between two
    events, as the decode steps are; the median of 5 brackets is kept."""
    from learned_kv_cache_sp_amd import spkv
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def sweep(regions, nbytes):
        rows = []
        for runs in (False, True):
            for nt in (False, True):
                for per_cu in (1, 2, 4, 8):
                    grid = per_cu * cu
                    ts = []
                    for rep in range(6):
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for k in range(16):
                            spkv.spkv_hbm_read(regions[(rep * 16 + k) % len(regions)], sink, nontemporal=nt,
                                               runs=runs, grid=grid, stream=stream)
                        e1.record(stream)
                        torch.cuda.synchronize()
                        if rep:
                            ts.append(e0.elapsed_time(e1) / 16)
                    us = float(np.median(ts)) * 1e3
                    rows.append({"order": "runs" if runs else "stride", "nontemporal": nt, "grid": grid,
                                 "us": round(us, 2), "GBs": round(nbytes / (us * 1e-6) / 1e9, 1)})
        best = max(rows, key=lambda r: r["GBs"])
        return {"bytes": int(nbytes), "best": best,
                "table": [[r["order"], int(r["nontemporal"]), r["grid"], r["GBs"]] for r in rows]}

    res = {"kernel": "spkv_hbm_read (16-byte loads, one read of every byte)", "unit": "GB/s",
           "table_columns": ["order", "nontemporal", "grid", "GB/s"]}
    if decode_bytes:
        nb = int(math.ceil(decode_bytes / 16384.0)) * 16384
        n_reg = max(2, int(math.ceil(1.5e9 / nb)))
        big = torch.ones(n_reg * nb // 4, dtype=torch.int32, device="cuda")
        regions = [big[k * nb // 4:(k + 1) * nb // 4] for k in range(n_reg)]
        res["decode_sized"] = sweep(regions, nb)
        del regions, big
    x = torch.ones((2 << 30) // 4, dtype=torch.int32, device="cuda")
    res["read_2GiB"] = sweep([x], x.numel() * 4)
    del x
    torch.cuda.empty_cache()
    return res


def host_cpu() -> tuple[int, dict]:
    """The host cores this process may use (affinity, capped by a cgroup CPU
    quota if one is set) and what identifies them."""
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    quota = None
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = int(q) / int(per)
    except (OSError, ValueError):
        pass
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = aff if quota is None else max(1, min(aff, int(quota)))
    return threads, {"nproc": os.cpu_count(), "affinity_cpus": aff, "cgroup_cpu_quota": quota,
                     "cpu_model": model, "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(name: str, wl, budget_s: float) -> dict:
    if name == "soft_prefill_16k":
        r = cpu_baseline_soft(wl, budget_s)
    elif name == "sink_gate_16k":
        r = cpu_baseline_sink_gate(wl, budget_s)
    elif name == "head_stats_1m":
        r = cpu_baseline_head_stats(budget_s)
    elif name == "rethreshold_32k":
        r = cpu_baseline_rethreshold(wl, budget_s)
    else:
        r = (cpu_baseline_prefill if wl.chunk else cpu_baseline_decode)(wl, budget_s)
    r["host"] = host_cpu()[1]
    return r


DEFAULT_STEPS = {"decode": (256, 16), "prefill": (4, 1), "rethreshold_32k": (20, 3), "head_stats_1m": (50, 5),
                 "soft_prefill_16k": (5, 1), "sink_gate_16k": (50, 5)}
SECONDARY = ["decode_131k", "ragged_32", "prefill_64k", "decode_32k_b16", "decode_32k_b16_tau0"]
# secondary lines without a CPU baseline (the same oracle work as decode_32k's)
SECONDARY_NO_CPU = {"decode_32k_b16", "decode_32k_b16_tau0"}


def workload(name: str):
    """The named workload; decode_32k_b16 is decode_32k at batch 16 (the batch
    of SP-KV's decode-kernel comparison, section 3.4), decode_32k_b16_tau0 the
    same with tau = 0 (every pair kept: full attention through the same
    kernels), so that their ratio is the speed-up of the configured keep
    rates over full attention."""
    import dataclasses
    from learned_kv_cache_sp_amd import inputs
    if name == "decode_32k_b16":
        return dataclasses.replace(inputs.WORKLOADS["decode_32k"], name=name, batch=16)
    if name == "decode_32k_b16_tau0":
        return dataclasses.replace(inputs.WORKLOADS["decode_32k"], name=name, batch=16, tau=0.0, keep=(1.0,) * 8)
    return inputs.WORKLOADS[name]


def run_workload(args, name: str, steps=None, warmup=None) -> dict:
    import torch
    from learned_kv_cache_sp_amd import inputs
    a = argparse.Namespace(**vars(args))
    kind = name if name in DEFAULT_STEPS else ("prefill" if workload(name).chunk else "decode")
    a.steps = DEFAULT_STEPS[kind][0] if steps is None else steps
    a.warmup = DEFAULT_STEPS[kind][1] if warmup is None else warmup
    if name == "soft_prefill_16k":
        wl = inputs.WORKLOADS["prefill_64k"]
        res = bench_soft_prefill(a, wl)
    elif name == "sink_gate_16k":
        wl = inputs.WORKLOADS["prefill_64k"]
        res = bench_sink_gate(a, wl)
    elif name == "head_stats_1m":
        wl = None
        res = bench_head_stats(a)
    elif name == "rethreshold_32k":
        wl = inputs.WORKLOADS["decode_32k"]
        res = bench_rethreshold(a, wl)
    else:
        wl = workload(name)
        res = bench_prefill(a, wl) if wl.chunk else bench_decode(a, wl)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, wl


# ----------------------------------------------------------------------------

def main():
    args = parse()
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.kernel, args.workload))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: this benchmark measures the path on one MI355X; "
                                   "more than one GPU is not supported", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    res, wl = run_workload(args, args.workload, args.steps, args.warmup)
    print(f"[bench] {args.workload}: {res['value']:.1f} {res['unit']}, roofline frac {res['roofline']['frac']}",
          file=sys.stderr, flush=True)

    if args.copy_calibration:
        a = torch.zeros(CALIBRATION_BYTES // 2, dtype=torch.int16, device="cuda")
        b_ = torch.empty_like(a)
        torch.neg(a, out=b_)
        torch.cuda.synchronize()
        del a, b_
        res["copy_calibration_bytes"] = CALIBRATION_BYTES

    if not args.no_ceiling:
        dec_bytes = res["roofline"].get("bytes_per_launch") if res["roofline"]["bound"] == "hbm" else None
        res["hbm_ceiling"] = hbm_ceiling(torch, dec_bytes)
        if dec_bytes:
            ceil_gbs = res["hbm_ceiling"]["decode_sized"]["best"]["GBs"]
            res["roofline"]["measured_ceiling_GBs"] = ceil_gbs
            res["roofline"]["frac_of_measured_ceiling"] = round(res["roofline"]["achieved"] / ceil_gbs, 4)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.workload, wl, args.cpu_budget)

    # the other single-GPU workloads, each with its own default steps, its
    # roofline and its CPU baseline, in the same JSON line
    if args.workload == "decode_32k" and not args.no_secondary:
        res["secondary"] = []
        for name in SECONDARY:
            t0 = time.perf_counter()
            r2, wl2 = run_workload(args, name)
            if not args.no_cpu_baseline and name not in SECONDARY_NO_CPU:
                r2["cpu_baseline"] = cpu_baseline(name, wl2, args.cpu_budget)
            r2["wall_s"] = round(time.perf_counter() - t0, 1)
            res["secondary"].append(r2)
            print(f"[bench] {name}: {r2['value']:.1f} {r2['unit']}, roofline frac {r2['roofline']['frac']}",
                  file=sys.stderr, flush=True)
        # SP-KV's own comparison (section 3.4, Fig. 3 right: its sparse decode
        # kernel against full attention at batch 16) through these kernels:
        # the configured keep rates against tau = 0 (every pair kept)
        by = {r["config"]["workload"]: r for r in res["secondary"]}
        sp, full = by.get("decode_32k_b16"), by.get("decode_32k_b16_tau0")
        if sp and full:
            res["sparse_vs_full_batch16"] = {
                "speedup_per_step": round(full["ms_per_step"] / sp["ms_per_step"], 3),
                "bytes_ratio": round(full["roofline"]["bytes_per_launch"] / sp["roofline"]["bytes_per_launch"], 3),
                "sparse_ms_per_step": sp["ms_per_step"], "full_ms_per_step": full["ms_per_step"]}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
