#!/usr/bin/env python3
"""Throughput of the whole quantisation pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload stack8b]

A step is one pass of the whole path over the resident weights: EWQ entropy
of every matrix and block tiering, the tier read-back, then per tier SINQ
Sinkhorn balancing + group RTN int4 packing, int8 per-row, or nothing.
Inputs are seeded synthetic bf16 weights with the shapes of 32 Llama-3.1-8B
transformer blocks (6.98e9 weights, 13.96 GB), resident in HBM before the
timed region; outputs are preallocated.  The value is bf16 input bytes per
second of wall time (GB/s, 1e9 bytes).

Printed as one JSON line.  ``roofline`` describes the dominant call (the
Sinkhorn sweep on this workload), timed with HIP events on the stream it is
launched on, against its algorithmic bytes (one read of every weight per
iteration); ``traffic`` is the measured HBM traffic per call from the
rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/, valid while the
kernel source it was taken on is unchanged.  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload, and ``parity`` compares the
timed steps' own outputs on that sample with the oracle's (entropies, s and
t, and the codes both stage-isolated and end to end).

Outside the timed steps the line also carries ``dequant`` (the tier's codes
decoded back to bf16), ``df11`` (the lossless code of the kept blocks) and
``codebook`` (the same tier coded on the normal-quantile book and decoded),
each timed with HIP events.

Two "% of HBM peak" figures are given: input bytes / time, and compulsory
traffic / time, where compulsory traffic is the entropy read of every
weight, a second read of every weight that is quantised (the tiers need the
global entropy statistics first) and every output written.

``ceilings`` gives what plain kernels with no arithmetic reach on the same
GPU in the same run (libwoq_probe.so): an 8 GiB read from HBM, a 1 GiB copy,
128 MiB re-read from the Infinity Cache, 16 MiB from the L2 caches, and the
fp32 FMA issue rate; the dominant call's rate is also given against the HBM
read ceiling.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s bf16 weights quantised (+% HBM peak), Llama-8B-shaped stack, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sinq_sweep_stack8b_traffic.md")
TRAFFIC_WORKLOAD = "stack8b"   # the workload the counter summary was taken on
SINQ_SOURCES = [os.path.join(ROOT, "weight_only_quantization_softmax_amd", "csrc", f)
                for f in ("sinq.hip", "api.hip", "woq_internal.h")]


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _host_f32(t):
    """A device matrix as host fp32 (bf16 widened exactly, in numpy)."""
    import numpy as np
    import torch
    if t.dtype == torch.bfloat16:
        u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return (u.astype(np.uint32) << 16).view(np.float32)
    return t.contiguous().cpu().numpy()


def cpu_workers() -> int:
    """Host cores this process may use, at most 16 (one GPU's share of the machine)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(wl, specs, mats, qp, tiers, blocks_per_action=2):
    """The oracle (numpy fp64; fp32 where the decisions are fp32) on the host
    cores, over a bounded sample of the workload, and the parity of the timed
    steps' own GPU outputs on that sample.

    Sample: the first ``blocks_per_action`` blocks of every action the tiers
    chose, each matrix taken through exactly what the pass does for it
    (entropy, then Sinkhorn + group RTN + pack, int8 per-row + pack, ternary +
    pack, or nothing).  The matrices of one action run concurrently on a
    thread pool of ``cpu_workers()`` threads: the oracle is numpy array
    kernels, which release the GIL, so the threads use that many cores.
    Each action's seconds per byte (wall clock of its pool) are applied to
    the workload's own tier mix.  Returns (baseline, parity); the parity
    comparisons run after the timed oracle work.
    """
    import concurrent.futures as cf
    import numpy as np
    import oracle

    acts = qp.action_of_block(tiers)
    nw = cpu_workers()
    by_act = {}
    for b, a in enumerate(acts):
        if len(by_act.setdefault(a, [])) < blocks_per_action:
            by_act[a].append(b)
    sample = {a: [i for i, sp in enumerate(specs) if sp.block in bl] for a, bl in by_act.items()}
    host = {i: _host_f32(mats[i]) for idx in sample.values() for i in idx}   # untimed copies

    def run(i, a):
        w = host[i]
        r = {"h": oracle.matrix_entropy(w)}
        if a == "sinq":
            s, t = oracle.sinkhorn_std(w, wl.iters)
            q = oracle.quantize_groupwise_f32(w, s.astype(np.float32), t.astype(np.float32),
                                              wl.bits, wl.group)[0]
            oracle.pack_codes(q, wl.bits)
            r.update(s=s, t=t, q=q)
        elif a == "int8row":
            q = oracle.quantize_groupwise_f32(w, None, None, 8, w.shape[1])[0]
            oracle.pack_codes(q, 8)
            r.update(q=q)
        elif a == "ternary":
            q, _ = oracle.ternary_quantize(w)
            oracle.pack_codes((q + 1).astype(np.uint8), 2)
            r.update(q=q)
        return r

    secs, nbytes, res = {}, {}, {}
    with cf.ThreadPoolExecutor(nw) as ex:
        for a, idx in sample.items():
            t0 = time.perf_counter()
            out = list(ex.map(lambda i: run(i, a), idx))
            secs[a] = time.perf_counter() - t0
            nbytes[a] = sum(mats[i].numel() * mats[i].element_size() for i in idx)
            res.update(zip(idx, out))
    total = 0.0
    for m, sp in zip(mats, specs):
        a = acts[sp.block]
        total += m.numel() * m.element_size() * secs[a] / nbytes[a]
    base = {"value": round(qp.bytes_in / total / 1e9, 6), "unit": "GB/s", "cores": nw,
            "kind": "oracle",
            "sample": ("; ".join(f"{a}: blocks {by_act[a]} ({nbytes[a] / 1e9:.3f} GB, {secs[a]:.1f} s)"
                                 for a in sample)
                       + f"; each matrix through entropy and its action's steps (Sinkhorn K={wl.iters} "
                       f"+ int{wl.bits} g{wl.group}, int8 per-row, ternary or none), the matrices of "
                       f"an action on {nw} threads (numpy array kernels release the GIL); per-action "
                       "seconds per byte applied to the workload's tier mix")}

    # parity of the timed steps' own outputs on the sample (untimed)
    h_gpu = qp.h_mat.cpu().numpy()
    par = {"matrices": len(res), "blocks": {a: by_act[a] for a in by_act},
           "entropy_max_rel_err": max(abs(h_gpu[i] / r["h"] - 1.0) for i, r in res.items())}

    def codes(i):
        o, r, w = qp.outputs[i], res[i], host[i]
        a = o["action"]
        if a == "sinq":
            sg, tg = o["s"].cpu().numpy(), o["t"].cpu().numpy()
            cg = oracle.unpack_codes(o["codes"].cpu().numpy().reshape(w.shape[0], -1), wl.bits, w.shape[1])
            qi = oracle.quantize_groupwise_f32(w, sg, tg, wl.bits, wl.group)[0]
            q64 = oracle.quantize_groupwise_f64(w, sg, tg, wl.bits, wl.group)[0]
            diff = cg != q64
            tie_ok = bool(np.all(~diff | oracle.near_tie_mask(w, sg, tg, wl.bits, wl.group))) if diff.any() else True
            e2e = cg != r["q"]
            return {"n": cg.size, "iso": int(np.count_nonzero(cg != qi)), "def": int(diff.sum()),
                    "tie_ok": tie_ok, "e2e": int(e2e.sum()),
                    "e2e_step": int(np.max(np.abs(cg.astype(np.int16) - r["q"].astype(np.int16)))),
                    "s": float(np.max(np.abs(sg / r["s"] - 1))), "t": float(np.max(np.abs(tg / r["t"] - 1)))}
        if a == "int8row":
            cg = o["codes"].cpu().numpy().reshape(w.shape)
            q64 = oracle.quantize_groupwise_f64(w, None, None, 8, w.shape[1])[0]
            return {"n": cg.size, "iso": int(np.count_nonzero(cg != r["q"])),
                    "def": int(np.count_nonzero(cg != q64)), "tie_ok": True, "e2e": 0, "e2e_step": 0}
        return None

    with cf.ThreadPoolExecutor(nw) as ex:
        cres = [c for c in ex.map(codes, sorted(res)) if c is not None]
    if cres:
        sq = [c for c in cres if "s" in c]
        par.update({"codes": sum(c["n"] for c in cres),
                    "codes_mismatch_stage_isolated": sum(c["iso"] for c in cres),
                    "codes_vs_fp64_definition": sum(c["def"] for c in cres),
                    "definition_mismatches_all_near_ties": all(c["tie_ok"] for c in cres),
                    "codes_mismatch_end_to_end": sum(c["e2e"] for c in cres),
                    "end_to_end_max_code_step": max(c["e2e_step"] for c in cres)})
        if sq:
            par.update({"s_max_rel_err": max(c["s"] for c in sq), "t_max_rel_err": max(c["t"] for c in sq)})
    return base, par


def _sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SINQ_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per Sinkhorn call from the committed counter summary, or None
    if the summary is missing or the kernel sources changed since."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            vals[k.strip("`")] = v.strip().strip("`")
    if vals.get("source_sha256") != _sources_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def compulsory_bytes(mats, specs, acts, bits, group):
    """Entropy read of every weight, plus a second read of each quantised
    weight and its outputs (codes, fp32 delta + uint8 zero per group, fp32
    per-row / per-column scales)."""
    total = 0
    for m, sp in zip(mats, specs):
        r, c = m.shape
        nb = m.numel() * m.element_size()
        total += nb
        a = acts[sp.block]
        if a == "sinq":
            total += nb + r * c * bits // 8 + r * (c // group) * 5 + 4 * (r + c)
        elif a == "int8row":
            total += nb + r * c + r * 5
        elif a == "ternary":
            total += nb + r * c // 4 + 4 * r
    return total


def gpu_call_ms(f, stream, reps):
    """Median GPU time of one call of f (HIP events on ``stream``).  Each call
    is enqueued behind a sleep kernel longer than twice the host's own time
    for the call (checks and descriptor tables for thousands of matrices
    take milliseconds), so that the host's work overlaps GPU work instead
    of showing as idle time between the events."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    f()
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    cycles = int(3e9 * (2 * host_s + 0.005))   # at most ~3 GHz shader clock
    ts = []
    for _ in range(reps):
        with torch.cuda.stream(stream):
            torch.cuda._sleep(cycles)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        f()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return sorted(ts)[len(ts) // 2]


def dequant_rate(qp, mats, wl, stream, reps=5):
    """Decode the Sinkhorn tier's packed outputs back to bf16 with
    dequant_unpack (outside the timed region) and time it with HIP events:
    bytes = codes + deltas + zero-points + s + t read, 2 B per weight written."""
    import torch
    import weight_only_quantization_softmax_amd as woq

    sel = [i for i, o in sorted(qp.outputs.items()) if o["action"] == "sinq"]
    if not sel:
        return None
    o = [qp.outputs[i] for i in sel]
    shapes = [tuple(mats[i].shape) for i in sel]
    outs = [torch.empty_like(mats[i]) for i in sel]
    args = dict(zeros=[x["zeros"] for x in o], row_scale=[x["s"] for x in o],
                col_scale=[x["t"] for x in o], out_dtype=mats[sel[0]].dtype, out=outs,
                stream=stream)
    codes, scales = [x["codes"] for x in o], [x["scales"] for x in o]
    woq.dequant_unpack(shapes, codes, scales, wl.bits, wl.group, **args)
    ms = gpu_call_ms(lambda: woq.dequant_unpack(shapes, codes, scales, wl.bits, wl.group, **args),
                     stream, reps)
    nbytes = sum(x["codes"].numel() + 5 * x["scales"].numel() + 4 * (x["s"].numel() + x["t"].numel())
                 + 2 * m.numel() for x, m in zip(o, (mats[i] for i in sel)))
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"call": "dequant_unpack", "matrices": len(sel), "ms": round(ms, 4), "bytes": int(nbytes),
            "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def codebook_rate(qp, mats, wl, stream, reps=5):
    """The non-uniform grid on the Sinkhorn tier: the same matrices, balancing
    scales and width as the step, coded with the normal-quantile book
    (quant_pack_codebook) and decoded back to bf16 (dequant_codebook), each
    timed with HIP events.  Bytes: quantise reads 2 B per weight + s + t and
    writes the codes + 4 B per group; dequantise the reverse."""
    import torch
    import weight_only_quantization_softmax_amd as woq

    sel = [i for i, o in sorted(qp.outputs.items()) if o["action"] == "sinq"]
    if not sel or wl.bits > 4:
        return None
    # the matrices whose codes, scales and decoded copy fit in 90% of the free
    # memory (all of them except on the 70B stack)
    torch.cuda.synchronize()
    free = 0.9 * torch.cuda.mem_get_info()[0]
    need, fit = 0, []
    for i in sel:
        m = mats[i]
        need += m.numel() * (m.element_size() + wl.bits / 8) + 4 * m.numel() / wl.group
        if need > free:
            break
        fit.append(i)
    if not fit:
        return None
    sel = fit
    o = [qp.outputs[i] for i in sel]
    ms_ = [mats[i] for i in sel]
    rs, ct = [x["s"] for x in o], [x["t"] for x in o]
    codes, scales = woq.quant_pack_codebook(ms_, wl.bits, wl.group, row_scale=rs, col_scale=ct,
                                            stream=stream)
    outs = [torch.empty_like(m) for m in ms_]
    shapes = [tuple(m.shape) for m in ms_]

    def quant():
        woq.quant_pack_codebook(ms_, wl.bits, wl.group, row_scale=rs, col_scale=ct, codes=codes,
                                scales=scales, stream=stream)

    def dequant():
        woq.dequant_codebook(shapes, codes, scales, wl.bits, wl.group, row_scale=rs, col_scale=ct,
                             out_dtype=ms_[0].dtype, out=outs, stream=stream)

    res = {"call": "quant_pack_codebook / dequant_codebook", "book": f"normal {wl.bits}-bit",
           "matrices": len(sel), "of": sum(1 for o_ in qp.outputs.values() if o_["action"] == "sinq")}
    n = sum(m.numel() for m in ms_)
    nbytes = (2 * n + sum(c.numel() + 4 * a.numel() for c, a in zip(codes, scales))
              + 4 * sum(x.numel() + y.numel() for x, y in zip(rs, ct)))
    for name, f in (("quant", quant), ("dequant", dequant)):
        f()
        ms = gpu_call_ms(f, stream, reps)
        gbs = nbytes / (ms / 1e3) / 1e9
        res[name] = {"ms": round(ms, 4), "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    res["bytes"] = int(nbytes)
    return res


def df11_rate(qp, mats, specs, acts, stream, reps=3):
    """Lossless code of the blocks the tiers keep in bf16: encode them (one
    df11_compress over all of them from the exponent histograms the timed
    pass's entropy call already counted, outside the timed region, after one
    untimed call; wall clock including the host-side code construction and
    its one synchronisation), then time decoding with one batched
    df11_decode per transformer block (HIP events).  Bytes = encoded
    exponents + sign/mantissa bytes + gaps + block positions read, 2 B per
    weight written.  One block is checked bit for bit after decoding."""
    import torch
    import weight_only_quantization_softmax_amd as woq

    keep = sorted(b for b, a in enumerate(acts) if a == "keep")
    if not keep:
        return None
    per_idx = [[i for i, sp in enumerate(specs) if sp.block == b] for b in keep]
    per = [[mats[i] for i in ix] for ix in per_idx]
    allm = [m for ms in per for m in ms]
    hist = qp.exp_hist[[i for ix in per_idx for i in ix]]
    woq.df11_compress(allm, hist=hist, stream=stream)   # untimed: the allocator's first growth
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    flat = woq.df11_compress(allm, hist=hist, stream=stream)
    torch.cuda.synchronize()
    t_enc = time.perf_counter() - t0
    enc, i = [], 0
    for ms in per:
        enc.append(flat[i:i + len(ms)])
        i += len(ms)
    outs = [torch.empty_like(m) for m in per[0]]
    woq.df11_decode(enc[0], out=outs, stream=stream)
    torch.cuda.synchronize()
    exact = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(per[0], outs))
    def decode_all():
        for e in enc:
            woq.df11_decode(e, out=outs, stream=stream)
    ms = gpu_call_ms(decode_all, stream, reps)
    n = sum(m.numel() for ms_ in per for m in ms_)
    stored = sum(x["enc"].numel() + x["sm"].numel() + x["gaps"].numel() + 4 * x["block_pos"].numel()
                 for e in enc for x in e)
    gbs = (stored + 2 * n) / (ms / 1e3) / 1e9
    return {"call": "df11_decode", "blocks": len(keep), "weights": int(n), "exact": bool(exact),
            "bits_per_weight": round(8 * stored / n, 3), "encode_s": round(t_enc, 4),
            "decode_ms": round(ms, 4), "decode_ms_per_block": round(ms / len(keep), 4),
            "bf16_GBps": round(2 * n / (ms / 1e3) / 1e9, 1), "GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


PROBE_LIB = os.path.join(ROOT, "weight_only_quantization_softmax_amd", "libwoq_probe.so")


def _probe():
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build it with "
                           "python -m weight_only_quantization_softmax_amd.build")
    lib = ctypes.CDLL(PROBE_LIB)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.probe_read.argtypes = [vp, sz, i32, i32, i32, vp, vp]
    lib.probe_copy.argtypes = [vp, vp, sz, i32, vp]
    lib.probe_fma.argtypes = [vp, i32, i32, vp]
    lib.probe_barrier.argtypes = [vp, vp, i32, i32, i32, ctypes.c_uint, i32, vp]
    for f in (lib.probe_read, lib.probe_copy, lib.probe_fma, lib.probe_barrier):
        f.restype = i32
    return lib


def barrier_us(lib, grid, team, mode=0, n_bar=2000, spin_limit=1 << 22):
    """Microseconds per barrier among teams of `team` workgroups in one
    cooperative launch of `grid` workgroups (n_bar barriers minus one,
    HIP events); None if a wait gave up.  mode 0: every poll an acquire
    load; 1: relaxed polls and one acquire fence; 2: as 1, arrivals on eight
    sub-counters first; 3: as 1, with a release and an acquire by every
    wave (the form that publishes data written by all waves)."""
    import torch
    stream = torch.cuda.current_stream()
    sh = ctypes_stream(stream)
    cnt = torch.zeros((grid // team) * 9 * 64, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(n):
        cnt.zero_()
        err.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = lib.probe_barrier(cnt.data_ptr(), err.data_ptr(), n, grid, team, spin_limit, mode, sh)
        e1.record(stream)
        e1.synchronize()
        if rc != 0:
            raise RuntimeError(f"probe_barrier failed: {rc}")
        return e0.elapsed_time(e1), int(err.item())
    run(8)
    t1, e_1 = run(1)
    tn, e_n = run(n_bar)
    if e_1 or e_n:
        return None
    return round((tn - t1) * 1e3 / (n_bar - 1), 3)


def probe_rate(lib, kind, nbytes, passes=1, grid=2048, chunked=0, reps=5, bufs=None):
    """GB/s of one probe kernel (median of `reps` launches, HIP events on the
    stream the probe is launched on).  kind: "read", "copy" or "fma" (for
    "fma", nbytes is the iteration count and the result is T lane-ops/s)."""
    import torch
    stream = torch.cuda.current_stream()
    sh = ctypes_stream(stream)
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    src, dst = bufs if bufs else (None, None)

    def launch():
        if kind == "read":
            rc = lib.probe_read(src.data_ptr(), nbytes, passes, grid, chunked, sink.data_ptr(), sh)
        elif kind == "copy":
            rc = lib.probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, grid, sh)
        else:
            rc = lib.probe_fma(sink.data_ptr(), nbytes, grid, sh)
        if rc != 0:
            raise RuntimeError(f"probe_{kind} failed: {rc}")

    launch()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    if kind == "fma":
        ops = 8 * nbytes * grid * 256
        return {"ms": round(ms, 4), "T_lane_ops_per_s": round(ops / (ms / 1e3) / 1e12, 2)}
    moved = nbytes * passes * (2 if kind == "copy" else 1)
    return {"ms": round(ms, 4), "GBps": round(moved / (ms / 1e3) / 1e9, 1)}


def ctypes_stream(stream):
    import ctypes
    return ctypes.c_void_p(stream.cuda_stream)


def ceilings():
    """What plain kernels with no arithmetic reach on this GPU (the library's
    streaming kernels are compared with these, not only with the
    8 TB/s spec): a grid-stride read of 8 GiB from HBM, a 1 GiB copy (read +
    write), re-reads of a 128 MiB buffer that stays in the 256 MB Infinity
    Cache (32 passes in one launch; grid-stride and per-workgroup contiguous
    order), a 16 MiB buffer re-read from the L2 caches, and the fp32 FMA issue
    rate without packed instructions."""
    import torch
    lib = _probe()
    big = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    res = {"hbm_read_8GiB": probe_rate(lib, "read", 8 << 30, bufs=(big, None))}
    a = big[: 1 << 30]
    b = big[1 << 30: 2 << 30]
    res["hbm_copy_1GiB"] = probe_rate(lib, "copy", 1 << 30, bufs=(a, b))
    res["mall_reread_128MiB_x32"] = probe_rate(lib, "read", 128 << 20, passes=32, bufs=(a, None))
    res["mall_reread_128MiB_x32_chunked"] = probe_rate(lib, "read", 128 << 20, passes=32, chunked=1,
                                                      bufs=(a, None))
    res["l2_reread_16MiB_x64"] = probe_rate(lib, "read", 16 << 20, passes=64, bufs=(a, None))
    res["fp32_fma"] = probe_rate(lib, "fma", 4096, grid=4096)
    res["grid_barrier_us_512wg"] = barrier_us(lib, 512, 512)
    res["grid_barrier_us_512wg_relaxed_polls"] = barrier_us(lib, 512, 512, mode=1)
    res["grid_barrier_us_512wg_two_level"] = barrier_us(lib, 512, 512, mode=2)
    res["grid_barrier_us_512wg_every_wave"] = barrier_us(lib, 512, 512, mode=3)
    del big
    torch.cuda.synchronize()
    return res


def ceilings_sweep():
    """The probes over buffer sizes, grids and access orders (re-reads of
    8 MiB .. 1 GiB: L2-resident up to 32 MiB, Infinity-Cache-resident up to
    256 MiB), the 1 GiB copy per grid, the fp32 FMA rate, and barriers among
    teams of workgroups of one cooperative launch.  One JSON line each."""
    import torch
    lib = _probe()
    big = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    out = {f"hbm_read_8GiB_g{g}": probe_rate(lib, "read", 8 << 30, grid=g, bufs=(big, None))["GBps"]
           for g in (1024, 2048, 4096)}
    out["hbm_read_4GiB_chunked_g2048"] = probe_rate(lib, "read", 4 << 30, chunked=1,
                                                    bufs=(big, None))["GBps"]
    print(json.dumps(out), flush=True)
    for mb in (8, 16, 32, 48, 64, 96, 128, 160, 192, 224, 256, 320, 384, 512, 1024):
        passes = max(2, min(64, 4096 // mb))
        r = {"MiB": mb, "passes": passes}
        for g in (1024, 2048, 4096):
            for ch in (0, 1):
                r[f"g{g}{'_chunked' if ch else ''}"] = probe_rate(
                    lib, "read", mb << 20, passes=passes, grid=g, chunked=ch, bufs=(big, None))["GBps"]
        print(json.dumps(r), flush=True)
    for g in (1024, 2048, 4096):
        print(json.dumps({"copy_1GiB_grid": g, **probe_rate(lib, "copy", 1 << 30, grid=g,
                                                            bufs=(big[:1 << 30], big[1 << 30:2 << 30]))}),
              flush=True)
    print(json.dumps({"fp32_fma": probe_rate(lib, "fma", 8192, grid=8192)}), flush=True)
    for grid, team in ((16, 16), (32, 32), (64, 64), (256, 256), (512, 512), (1024, 1024),
                       (2048, 2048), (512, 128), (512, 64), (512, 32), (512, 8)):
        r = {"barrier_grid": grid, "team": team}
        for mode in (0, 1, 2, 3):
            if mode == 2 and team % 8:
                continue
            r[f"us_mode{mode}"] = barrier_us(lib, grid, team, mode=mode)
        print(json.dumps(r), flush=True)
    return 0


def torch_reference(reps=20):
    """Streaming rates of torch's stock kernels on this GPU (not the
    library's), for comparison with the library's kernels: a 1 GiB device
    copy (read + write), 1 GiB read-only reductions, and the same reduction
    over a 128 MiB buffer that stays in the 256 MB Infinity Cache across
    reps.  HIP events on the current stream, after one untimed run each."""
    import torch
    torch.cuda.set_device(0)
    n = 1 << 30
    a = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    small = a[: (128 << 20) // 2]
    out = torch.empty((), dtype=torch.float32, device="cuda")
    outb = torch.empty((), dtype=torch.bfloat16, device="cuda")

    def rate(f, nbytes, r):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(r):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / r
        return {"ms": round(ms, 4), "GBps": round(nbytes / (ms / 1e3) / 1e9, 1)}

    res = {
        "copy_1GiB (read + write)": rate(lambda: b.copy_(a), 2 * n, reps),
        "sum_1GiB (read)": rate(lambda: torch.sum(a, dim=0, dtype=torch.float32, out=out), n, reps),
        "amax_1GiB (read)": rate(lambda: torch.amax(a, dim=0, out=outb), n, reps),
        "sum_128MiB_cache_resident (read)": rate(lambda: torch.sum(small, dim=0, dtype=torch.float32, out=out),
                                                 128 << 20, 10 * reps),
    }
    print(json.dumps({"torch_reference": res, "torch": torch.__version__}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="stack8b")
    ap.add_argument("--sinq-batch-mb", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time an untiered workload eagerly instead of as graph replays")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming-ceiling probes (libwoq_probe.so)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    ap.add_argument("--torch-reference", action="store_true",
                    help="only measure torch's stock streaming kernels on this GPU")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="only measure the streaming ceilings (libwoq_probe.so)")
    ap.add_argument("--ceilings-sweep", action="store_true",
                    help="only sweep the probes over sizes, grids and barrier teams")
    args = ap.parse_args()
    if args.ceilings_sweep:
        import torch
        torch.cuda.set_device(0)
        return ceilings_sweep()
    if args.torch_reference:
        return torch_reference()
    if args.ceilings_only:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps({"ceilings": ceilings()}), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py: this pass runs on one GPU; --gpus {args.gpus} is not supported "
              "(blocks are independent after tiering; see the sharding design)", file=sys.stderr)
        return 2

    import torch
    import woqdata
    from weight_only_quantization_softmax_amd.pipeline import QuantPass

    torch.cuda.set_device(0)
    if args.copy_probe_mb:
        # an elementwise kernel that reads N bytes and writes N bytes
        src = torch.zeros((args.copy_probe_mb << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    _log(f"[bench] generating workload {args.workload}")
    wl, specs, mats = woqdata.generate(args.workload, device="cuda")
    torch.cuda.synchronize()
    qp = QuantPass(mats, [m.block for m in specs], wl.n_blocks, iters=wl.iters, bits=wl.bits,
                   group=wl.group, x=wl.x, tiered=wl.tiered,
                   actions=(wl.low_tier, wl.mid_tier, wl.high_tier),
                   sinq_batch_bytes=args.sinq_batch_mb << 20)
    _log(f"[bench] {len(mats)} matrices, {qp.bytes_in / 1e9:.3f} GB; warmup {args.warmup}")
    for _ in range(args.warmup):
        tiers = qp.run()
        _log(f"[bench] tiers {tiers}")
    torch.cuda.synchronize()
    timers = {}
    stream = torch.cuda.current_stream()
    # an untiered pass (the tiers decide nothing) is captured into a graph
    # and timed as graph replays; a tiered pass reads its tiers back on the
    # host mid-pass and runs eagerly
    graph = qp.graph(stream) if (not wl.tiered and not args.no_graph) else None
    _log(f"[bench] timing {args.steps} steps" + (" (graph replays)" if graph else ""))
    if graph is not None:
        graph.replay()
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_ev[i][0].record(stream)
        if graph is None:
            tiers = qp.run(stream=stream, timers=timers)
        else:
            graph.replay()
        step_ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    value = qp.bytes_in / (ms / 1e3) / 1e9
    step_ms = sorted(a.elapsed_time(b) for a, b in step_ev)
    timed_steps = args.steps
    if graph is not None:
        # the per-call times come from eager passes after the timed replays
        tiers = qp.tier.cpu().tolist()
        timed_steps = max(1, min(args.steps, 3))
        for _ in range(timed_steps):
            qp.run(stream=stream, timers=timers)
        torch.cuda.synchronize()

    per_kind = {}
    for kind, evs in timers.items():
        tot = sum(a.elapsed_time(b) for a, b, _ in evs)
        per_kind[kind] = {"ms_per_step": tot / timed_steps, "calls": len(evs) // timed_steps,
                          "bytes": evs[0][2]}
    dominant = max(per_kind, key=lambda k: per_kind[k]["ms_per_step"])
    d = per_kind[dominant]
    launch_ms = d["ms_per_step"] / max(d["calls"], 1)
    traffic = None
    if dominant == "sinq":
        # one read of every weight per iteration (row scales, column partials
        # and the column reduction are not counted)
        alg = d["bytes"] * wl.iters
        kernel = ("sinq_balance (K fused row/column sweeps + column reductions; the tier's "
                  "wave-form and wider matrices as two concurrent calls)")
        traffic = measured_traffic() if args.workload == TRAFFIC_WORKLOAD else None
    else:
        alg = d["bytes"]
        kernel = {"entropy": "ewq_block_entropy"}.get(dominant, dominant)
    achieved = alg / (launch_ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
            "algorithmic_bytes_per_launch": int(alg), "launch_ms": round(launch_ms, 4)}
    acts = qp.action_of_block(tiers)
    comp = compulsory_bytes(mats, specs, acts, wl.bits, wl.group)
    deq = dequant_rate(qp, mats, wl, stream)
    df11 = df11_rate(qp, mats, specs, acts, stream)
    book = codebook_rate(qp, mats, wl, stream)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "matrices": len(mats), "blocks": wl.n_blocks,
                   "bf16_bytes": qp.bytes_in, "iters": wl.iters, "bits": wl.bits, "group": wl.group,
                   "tiers": {str(k): tiers.count(k) for k in (1, 2, 3)},
                   "hbm_frac_input_bytes": round(value / HBM_PEAK_GBS, 4),
                   "compulsory_bytes": comp,
                   "hbm_frac_compulsory": round(comp / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 3), "min": round(step_ms[0], 3),
                    "max": round(step_ms[-1], 3)},
        "timing": ("graph replays of the whole pass; per-call times from eager passes"
                   if graph is not None else "eager passes (one tier read-back each)"),
        "roofline": roof,
        "dequant": deq,
        "df11": df11,
        "codebook": book,
        "calls": {k: {"ms_per_step": round(v["ms_per_step"], 3), "calls": v["calls"]}
                  for k, v in per_kind.items()},
    }
    if not args.no_ceilings:
        _log("[bench] streaming ceilings")
        ceil = ceilings()
        ceil["dominant_vs_hbm_read_ceiling"] = round(achieved / ceil["hbm_read_8GiB"]["GBps"], 4)
        out["ceilings"] = ceil
    if not args.no_cpu_baseline:
        _log("[bench] cpu baseline (oracle on a sample)")
        out["cpu_baseline"], out["parity"] = cpu_baseline(wl, specs, mats, qp, tiers)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
