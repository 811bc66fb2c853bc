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


def cpu_baseline(wl, specs, mats, qp, tiers):
    """The oracle (numpy fp64, fp32 where the decisions are fp32) on host
    cores over a bounded sample of the workload, and the parity of the
    timed steps' own GPU outputs on that sample.

    Sample: the matrices of the first block of the Sinkhorn tier (else the
    first block), in order, until at least 60 M weights (Llama-8B shapes: q,
    k, v, o and gate, 92.3 M weights), each taken through every stage the
    workload uses (entropy; Sinkhorn + group RTN + pack; int8 per-row +
    pack; ternary + pack).  Each stage's seconds per byte on the sample are
    applied to the workload's own tier mix.  Returns (baseline, parity); the
    parity comparisons run outside the timed oracle work.
    """
    import numpy as np
    import oracle

    acts = qp.action_of_block(tiers)
    sinq_blocks = [sp.block for sp in specs if acts[sp.block] == "sinq"]
    first = sinq_blocks[0] if sinq_blocks else specs[0].block
    pick, n = [], 0
    for i, m in enumerate(specs):
        if m.block == first and n < 60_000_000:
            pick.append(i)
            n += mats[i].numel()
    t_ent = t_sinq = t_i8 = t_ter = 0.0
    nbytes = 0
    h_gpu = qp.h_mat.cpu().numpy()
    par = {"matrices": len(pick), "block": first, "entropy_max_rel_err": 0.0}
    s_err = t_err = 0.0
    n_codes = iso_bad = e2e_bad = 0
    for i in pick:
        w = mats[i].float().cpu().numpy()
        nbytes += mats[i].numel() * mats[i].element_size()
        t0 = time.perf_counter()
        h = oracle.matrix_entropy(w)
        t1 = time.perf_counter()
        s, t = oracle.sinkhorn_std(w, wl.iters)
        q = oracle.quantize_groupwise_f32(w, s.astype(np.float32), t.astype(np.float32), wl.bits,
                                          wl.group)
        oracle.pack_codes(q[0], wl.bits)
        t2 = time.perf_counter()
        q8 = oracle.quantize_groupwise_f32(w, None, None, 8, w.shape[1])
        oracle.pack_codes(q8[0], 8)
        t3 = time.perf_counter()
        qt, _ = oracle.ternary_quantize(w)
        oracle.pack_codes((qt + 1).astype(np.uint8), 2)
        t4 = time.perf_counter()
        t_ent += t1 - t0
        t_sinq += t2 - t1
        t_i8 += t3 - t2
        t_ter += t4 - t3
        # parity of the step's outputs (untimed)
        if h != 0.0:
            par["entropy_max_rel_err"] = max(par["entropy_max_rel_err"], abs(h_gpu[i] / h - 1.0))
        o = qp.outputs.get(i)
        if o is not None and o["action"] == "sinq":
            sg, tg = o["s"].cpu().numpy(), o["t"].cpu().numpy()
            s_err = max(s_err, float(np.max(np.abs(sg / s - 1.0))))
            t_err = max(t_err, float(np.max(np.abs(tg / t - 1.0))))
            cg = oracle.unpack_codes(o["codes"].cpu().numpy(), wl.bits, w.shape[1])
            qi = oracle.quantize_groupwise_f32(w, sg, tg, wl.bits, wl.group)[0]
            n_codes += cg.size
            iso_bad += int(np.count_nonzero(cg != qi))
            e2e_bad += int(np.count_nonzero(cg != q[0]))
    if n_codes:
        par.update({"s_max_rel_err": s_err, "t_max_rel_err": t_err, "codes": n_codes,
                    "codes_mismatch_stage_isolated": iso_bad,
                    "codes_mismatch_end_to_end": e2e_bad})
    per_byte = {"sinq": t_sinq / nbytes, "int8row": t_i8 / nbytes, "ternary": t_ter / nbytes,
                "keep": 0.0}
    total = qp.bytes_in * (t_ent / nbytes)
    for m, sp in zip(mats, specs):
        total += m.numel() * m.element_size() * per_byte[acts[sp.block]]
    base = {"value": round(qp.bytes_in / total / 1e9, 6), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"{len(pick)} matrices of block {first} ({nbytes / 1e9:.3f} GB) through "
                       f"entropy ({t_ent:.1f}s), Sinkhorn K={wl.iters} + int{wl.bits} g{wl.group} "
                       f"({t_sinq:.1f}s), int8 per-row ({t_i8:.1f}s), ternary ({t_ter:.1f}s); "
                       "per-byte costs applied to the workload's tier mix; numpy, one thread")}
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        woq.dequant_unpack(shapes, codes, scales, wl.bits, wl.group, **args)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = nbytes / (ms / 1e3) / 1e9
        res[name] = {"ms": round(ms, 4), "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    res["bytes"] = int(nbytes)
    return res


def df11_rate(mats, specs, acts, stream, reps=3):
    """Lossless code of the blocks the tiers keep in bf16: encode them (one
    df11_compress over all of them, outside the timed region, after one
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
    per = [[m for m, sp in zip(mats, specs) if sp.block == b] for b in keep]
    allm = [m for ms in per for m in ms]
    woq.df11_compress(allm, stream=stream)       # untimed: the allocator's first growth
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    flat = woq.df11_compress(allm, stream=stream)
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        for e in enc:
            woq.df11_decode(e, out=outs, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n = sum(m.numel() for ms_ in per for m in ms_)
    stored = sum(x["enc"].numel() + x["sm"].numel() + x["gaps"].numel() + 4 * x["block_pos"].numel()
                 for e in enc for x in e)
    gbs = (stored + 2 * n) / (ms / 1e3) / 1e9
    return {"call": "df11_decode", "blocks": len(keep), "weights": int(n), "exact": bool(exact),
            "bits_per_weight": round(8 * stored / n, 3), "encode_s": round(t_enc, 4),
            "decode_ms": round(ms, 4), "decode_ms_per_block": round(ms / len(keep), 4),
            "bf16_GBps": round(2 * n / (ms / 1e3) / 1e9, 1), "GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def torch_reference(reps=20):
    """Streaming rates of torch's stock kernels on the box (not the
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
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    ap.add_argument("--torch-reference", action="store_true",
                    help="only measure torch's stock streaming kernels on the box")
    args = ap.parse_args()
    if args.torch_reference:
        return torch_reference()
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
    _log(f"[bench] timing {args.steps} steps")
    stream = torch.cuda.current_stream()
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_ev[i][0].record(stream)
        tiers = qp.run(stream=stream, timers=timers)
        step_ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    value = qp.bytes_in / (ms / 1e3) / 1e9
    step_ms = sorted(a.elapsed_time(b) for a, b in step_ev)

    per_kind = {}
    for kind, evs in timers.items():
        tot = sum(a.elapsed_time(b) for a, b, _ in evs)
        per_kind[kind] = {"ms_per_step": tot / args.steps, "calls": len(evs) // args.steps,
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
    df11 = df11_rate(mats, specs, acts, stream)
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
        "roofline": roof,
        "dequant": deq,
        "df11": df11,
        "codebook": book,
        "calls": {k: {"ms_per_step": round(v["ms_per_step"], 3), "calls": v["calls"]}
                  for k, v in per_kind.items()},
    }
    if not args.no_cpu_baseline:
        _log("[bench] cpu baseline (oracle on a sample)")
        out["cpu_baseline"], out["parity"] = cpu_baseline(wl, specs, mats, qp, tiers)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
