#!/usr/bin/env python3
"""Throughput of one rank's share of an Ulysses attention layer on one GPU.

One step is the whole rank-share path over one batch of synthetic input,
inputs already resident in HBM:

  forward : seq_to_head of Q, K and V in one batched launch   (8 chunks each)
            attention forward (O, LSE)
            head_to_seq(O)
  backward: seq_to_head(dO)
            attention backward (dQ, dK, dV)
            head_to_seq of dQ, dK and dV in one batched launch

Workload: the Llama-8B-shaped rank share at P=8 and N=131072 (32 query /
8 key-value heads globally, so 4 query heads and 1 key/value head per rank,
head size 128, bf16, causal).  Prints one JSON line.

Besides the step, `breakdown.configs` holds the other workloads of the
measurement plan, each timed alone (HIP events around every call, median
over the iterations): the same share at N=32768, the 262144-token forward
and the packed-document 65536-token forward and backward (block-diagonal
causal mask).  `--oracle-plan` instead times the CPU oracle on the whole
plan (full passes where they take minutes, sampled rows with a labelled
extrapolation where they would take hours) and prints that as JSON.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 matrix-core peak
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E peak
WORKLOAD = "llama8b-share-128k"

# Memory-side bytes per call of each attention entry point at this workload,
# from rocprofv3 FETCH_SIZE and WRITE_SIZE (one counter per run), scaled by
# what the same counters read for a plain 512 MiB device copy (FETCH x2.0,
# WRITE x1.0); the table is in profiles/attn_step_llama8b-share-128k_hbm_traffic.md.
# A figure is only reported while the kernel sources hash to what was
# measured; after any change to them the roofline's traffic is null.
MEASURED_TRAFFIC = {
    "attn_bwd": {"bytes": 5.40929e10, "sources": ("attn_bwd.hip", "attn_f32.hip", "device_common.h"),
                 "sha256_16": "5614bebb6b465c74"},
    "attn_fwd": {"bytes": 9.15775e9, "sources": ("attn_fwd.hip", "device_common.h"),
                 "sha256_16": "c8a660809813ee5b"},
}


def traffic_if_current(unit):
    import hashlib
    rec = MEASURED_TRAFFIC.get(unit)
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, "ulysses_sp_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return rec["bytes"] if h.hexdigest()[:16] == rec["sha256_16"] else None


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload records of the other configurations")
    ap.add_argument("--oracle-plan", action="store_true",
                    help="time the CPU oracle on the measurement plan instead (no GPU use)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--loss-shard-rows", type=int, default=4096,
                    help="rows of logits per shard in the language-model loss record")
    ap.add_argument("--no-logits-loss", action="store_true",
                    help="skip the language-model loss and tiled MLP records (outside the "
                         "attention step)")
    ap.add_argument("--cpu-rows", type=int, default=2560,
                    help="query rows of the oracle's timed sample (about 10-15 s on 16 cores)")
    ap.add_argument("--pack-sets", type=int, default=4,
                    help="distinct buffer sets the rotated exchange measurement cycles through")
    ap.add_argument("--pack-reps", type=int, default=24,
                    help="back-to-back launches per exchange in the rotated measurement")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before timing, run one plain device-to-device copy of MIB MiB "
                         "(a known-size reference for hardware byte counters)")
    return ap.parse_args()


def git_sha():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except Exception:
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def median_ms(events):
    """Median of the elapsed times of consecutive event pairs."""
    import numpy as np
    return float(np.median([a.elapsed_time(b) for a, b in events]))


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the path; --gpus {args.gpus} is not supported "
              "(libulysses runs on a single GPU, with no collectives between GPUs)", file=sys.stderr)
        return 2
    if args.oracle_plan:
        print(json.dumps(oracle_plan()))
        return 0

    import numpy as np
    import torch

    import synth
    import ulysses_sp_attention_amd as uly

    if not os.path.exists(uly.LIB_PATH):
        from ulysses_sp_attention_amd import _build
        _build.build_lib()
    uly.load_library()
    torch.cuda.set_device(0)

    w = synth.WORKLOADS[WORKLOAD]
    N, P, n, r = w.seqlen, w.P, w.n_local, w.rank
    hl, kl, hd = w.hq_local, w.hkv_local, w.head_dim

    def dev_seq(stream, heads, scale=1.0):
        host = w.seq_tensor(stream, heads, scale=scale)
        t = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).cuda()
        del host
        return t

    t0 = time.time()
    q_full = dev_seq(synth.STREAM_Q, w.hq, w.q_prescale)
    k_full = dev_seq(synth.STREAM_K, w.hkv)
    v_full = dev_seq(synth.STREAM_V, w.hkv)
    do_full = dev_seq(synth.STREAM_DO, w.hq)
    gen_s = time.time() - t0

    def chunks(t):
        return [t[c * n:(c + 1) * n] for c in range(P)]

    bf = torch.bfloat16
    cq, ck, cv, cdo = chunks(q_full), chunks(k_full), chunks(v_full), chunks(do_full)
    o_full = torch.zeros_like(q_full)
    dq_full, dk_full, dv_full = torch.zeros_like(q_full), torch.zeros_like(k_full), torch.zeros_like(v_full)
    co, cdq, cdk, cdv = chunks(o_full), chunks(dq_full), chunks(dk_full), chunks(dv_full)
    q = torch.empty((N, 1, hl, hd), dtype=bf, device="cuda")
    k = torch.empty((N, 1, kl, hd), dtype=bf, device="cuda")
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    do = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    lse = torch.empty((1, hl, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(uly.ulysses_attn_bwd_workspace_size(N, 1, hl, kl, hd, uly.BF16),
                     dtype=torch.uint8, device="cuda")
    scale = w.softmax_scale

    stream = torch.cuda.current_stream()
    names = ["pack_qkv", "attn_fwd", "unpack_o", "pack_do", "attn_bwd", "unpack_dqkv"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        uly.ulysses_seq_to_head_batch([(cq, q), (ck, k), (cv, v)], r)
        mark(1)
        uly.ulysses_attn_fwd(q, k, v, o, lse, scale, True)
        mark(2)
        uly.ulysses_head_to_seq(o, r, co)
        mark(3)
        uly.ulysses_seq_to_head(cdo, r, do)
        mark(4)
        uly.ulysses_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, True)
        mark(5)
        uly.ulysses_head_to_seq_batch([(dq, cdq), (dk, cdk), (dv, cdv)], r)
        mark(6)

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / args.steps

    seg_ms = {nm: [] for nm in names}
    for ev in events:
        for i, nm in enumerate(names):
            seg_ms[nm].append(ev[i].elapsed_time(ev[i + 1]))
    # per-segment median over the timed steps (HIP events on the launch stream)
    avg = {nm: float(np.median(v_)) for nm, v_ in seg_ms.items()}

    # Algorithmic work (causal pairs per query head; recompute not counted).
    pairs = w.causal_pairs()
    fwd_flop = 4.0 * hd * hl * pairs
    bwd_flop = 10.0 * hd * hl * pairs
    e = 2
    pack_qkv_bytes = 2.0 * N * (hl + 2 * kl) * hd * e   # read + write
    unpack_o_bytes = 2.0 * N * hl * hd * e
    pack_do_bytes = 2.0 * N * hl * hd * e
    unpack_dqkv_bytes = pack_qkv_bytes

    def tflops(flop, ms):
        return flop / (ms * 1e-3) / 1e12

    def gbps(b, ms):
        return b / (ms * 1e-3) / 1e9

    fwd_tf = tflops(fwd_flop, avg["attn_fwd"])
    bwd_tf = tflops(bwd_flop, avg["attn_bwd"])
    value = tflops(fwd_flop + bwd_flop, ms_step)
    breakdown = {
        "attn_fwd": {"ms": avg["attn_fwd"], "TFLOP/s": fwd_tf, "frac_of_mfma_peak": fwd_tf / MFMA_BF16_PEAK_TFLOPS},
        "attn_bwd": {"ms": avg["attn_bwd"], "TFLOP/s": bwd_tf, "frac_of_mfma_peak": bwd_tf / MFMA_BF16_PEAK_TFLOPS},
        "pack_qkv": {"ms": avg["pack_qkv"], "GB/s": gbps(pack_qkv_bytes, avg["pack_qkv"])},
        "unpack_o": {"ms": avg["unpack_o"], "GB/s": gbps(unpack_o_bytes, avg["unpack_o"])},
        "pack_do": {"ms": avg["pack_do"], "GB/s": gbps(pack_do_bytes, avg["pack_do"])},
        "unpack_dqkv": {"ms": avg["unpack_dqkv"], "GB/s": gbps(unpack_dqkv_bytes, avg["unpack_dqkv"])},
    }
    pack_ms = avg["pack_qkv"] + avg["unpack_o"] + avg["pack_do"] + avg["unpack_dqkv"]
    pack_bytes = pack_qkv_bytes + unpack_o_bytes + pack_do_bytes + unpack_dqkv_bytes
    breakdown["pack_all"] = {"ms": pack_ms, "GB/s": gbps(pack_bytes, pack_ms),
                             "frac_of_hbm_peak": gbps(pack_bytes, pack_ms) / HBM_PEAK_GBPS}

    breakdown["fused_step"] = measure_fused(uly, torch, np, stream, args, r, scale, lse, ws,
                                            (cq, ck, cv, co, cdo, cdq, cdk, cdv),
                                            fwd_flop, bwd_flop, ms_step)

    rotated = measure_exchanges(w, uly, torch, stream, args.pack_sets, args.pack_reps)
    breakdown["pack_rotated"] = rotated
    breakdown["attn_merge"] = measure_merge(w, uly, torch, stream, args.pack_sets, args.pack_reps)
    if not args.no_logits_loss:
        breakdown["logits_loss"] = measure_logits_loss(uly, torch, np, stream, args)
        breakdown["tiled_mlp"] = measure_tiled_mlp(uly, torch, np, stream, args)
    if not args.no_configs:
        del q_full, k_full, v_full, do_full, o_full, dq_full, dk_full, dv_full
        del q, k, v, o, do, dq, dk, dv, ws
        torch.cuda.empty_cache()
        breakdown["configs"] = {name: measure_config(synth.WORKLOADS[name], uly, torch, np, stream,
                                                     args)
                                for name in ("llama8b-share-32k", "long-256k", "packed-docs-64k")}

    # Roofline of the dominant unit of the step, timed with events on the
    # stream its kernels run on.  The attention backward is one entry point
    # (ulysses_attn_bwd) that enqueues three kernels back to back: the D
    # row-dot, the dQ kernel and the dK/dV kernel; its algorithmic work is the
    # five products of the backward (10 * hd flop per visible pair and head).
    # The forward is one kernel (2 products, 4 * hd flop per pair and head).
    units = {"attn_fwd": (fwd_flop, ["attn_fwd_bf16_kernel"]),
             "attn_bwd": (bwd_flop, ["bwd_stats_kernel", "attn_bwd_dq_kernel", "attn_bwd_dkv_kernel"])}
    dominant = max(units, key=lambda k_: avg[k_])
    flop, kernels = units[dominant]
    achieved = tflops(flop, avg[dominant])
    roofline = {
        "kernel": dominant,
        "launches": kernels,
        "bound": "mfma",
        "achieved": achieved,
        "peak": MFMA_BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
        "traffic": traffic_if_current(dominant),
        "traffic_unit": "bytes per call (memory side of L2)",
        "per_launch_flop": flop,
        "avg_ms": avg[dominant],
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_rows)

    line = {
        "metric": "causal attn fwd/bwd TFLOP/s at N=128K (4q/1kv heads, d=128); pack GB/s",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "seqlen": N, "P": P, "rank": r, "bs": 1,
                   "hq_local": hl, "hkv_local": kl, "head_dim": hd, "causal": True,
                   "step": "pack QKV + attn fwd + unpack O + pack dO + attn bwd + unpack dQ/dK/dV"},
        "timing": "per-segment figures are medians over the timed steps; value and ms_per_step "
                  "are the wall clock of all timed steps",
        "breakdown": breakdown,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "input_gen_s": gen_s,
        "git": git_sha(),
    }
    print(json.dumps(line))
    return 0


def measure_config(w, uly, torch, np, stream, args):
    """One workload of the measurement plan on its own: the rank-share path
    (exchange of Q, K, V from the P chunks, attention forward, exchange of O;
    with a backward, exchange of dO, attention backward, exchange of dQ, dK,
    dV), or the forward alone on head-sharded inputs.  Each call is bracketed
    by HIP events on the launch stream; figures are medians over the
    iterations.  Work is algorithmic: 4 hd flop per visible (query, key) pair
    and query head forward, 10 hd backward; exchanges move each byte of the
    rank's slice once each way."""
    import synth
    N, hl, kl, hd = w.seqlen, w.hq_local, w.hkv_local, w.head_dim
    bf = torch.bfloat16
    # The measurement plan's counts: at least 20 timed iterations (5 for the
    # 256K forward, 55 ms each) after 3 warm-up calls.
    reps = max(args.steps, 5 if N >= 262144 else 20)
    warm = max(3, args.warmup)
    cu = w.cu_seqlens()
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    pairs = w.causal_pairs()
    fwd_flop = 4.0 * hd * hl * pairs
    bwd_flop = 10.0 * hd * hl * pairs

    def dev(host):
        return torch.from_numpy(host.view(np.int16)).view(bf).cuda()

    out = {"seqlen": N, "hq_local": hl, "hkv_local": kl, "head_dim": hd, "causal": True,
           "documents": None if cu is None else len(cu) - 1, "visible_pairs_per_head": pairs,
           "iterations": reps, "warmup": warm}
    lse = torch.empty((1, hl, N), dtype=torch.float32, device="cuda")
    segs = {}
    if w.head_sharded_inputs:
        q = dev(w.head_tensor(synth.STREAM_Q, hl, scale=w.q_prescale))
        k = dev(w.head_tensor(synth.STREAM_K, kl))
        v = dev(w.head_tensor(synth.STREAM_V, kl))
        o = torch.empty_like(q)
        segs["attn_fwd"] = lambda: uly.ulysses_attn_fwd(q, k, v, o, lse, w.softmax_scale, True, cu_t)
        order = ["attn_fwd"]
    else:
        P, n, r = w.P, w.n_local, w.rank
        full = {s_: dev(w.seq_tensor(s_, h_, scale=w.q_prescale if s_ == synth.STREAM_Q else 1.0))
                for s_, h_ in ((synth.STREAM_Q, w.hq), (synth.STREAM_K, w.hkv),
                               (synth.STREAM_V, w.hkv), (synth.STREAM_DO, w.hq))}
        ch = {s_: [t[c * n:(c + 1) * n] for c in range(P)] for s_, t in full.items()}
        outs = {nm: torch.zeros_like(full[s_]) for nm, s_ in (("o", 1), ("dq", 1), ("dk", 2), ("dv", 3))}
        och = {nm: [t[c * n:(c + 1) * n] for c in range(P)] for nm, t in outs.items()}
        q = torch.empty((N, 1, hl, hd), dtype=bf, device="cuda")
        k = torch.empty((N, 1, kl, hd), dtype=bf, device="cuda")
        v, o, do = torch.empty_like(k), torch.empty_like(q), torch.empty_like(q)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
        ws = torch.empty(uly.ulysses_attn_bwd_workspace_size(N, 1, hl, kl, hd, uly.BF16),
                         dtype=torch.uint8, device="cuda")
        segs["pack_qkv"] = lambda: uly.ulysses_seq_to_head_batch(
            [(ch[1], q), (ch[2], k), (ch[3], v)], r)
        segs["attn_fwd"] = lambda: uly.ulysses_attn_fwd(q, k, v, o, lse, w.softmax_scale, True, cu_t)
        segs["unpack_o"] = lambda: uly.ulysses_head_to_seq(o, r, och["o"])
        segs["pack_do"] = lambda: uly.ulysses_seq_to_head(ch[4], r, do)
        segs["attn_bwd"] = lambda: uly.ulysses_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws,
                                                        w.softmax_scale, True, cu_t)
        segs["unpack_dqkv"] = lambda: uly.ulysses_head_to_seq_batch(
            [(dq, och["dq"]), (dk, och["dk"]), (dv, och["dv"])], r)
        order = ["pack_qkv", "attn_fwd", "unpack_o", "pack_do", "attn_bwd", "unpack_dqkv"]
    for _ in range(warm):
        for nm in order:
            segs[nm]()
    torch.cuda.synchronize()
    ev = {nm: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)] for nm in order}
    for i in range(reps):
        for nm in order:
            ev[nm][i][0].record(stream)
            segs[nm]()
            ev[nm][i][1].record(stream)
    torch.cuda.synchronize()
    e = 2
    xbytes = {"pack_qkv": 2.0 * N * (hl + 2 * kl) * hd * e, "unpack_o": 2.0 * N * hl * hd * e,
              "pack_do": 2.0 * N * hl * hd * e, "unpack_dqkv": 2.0 * N * (hl + 2 * kl) * hd * e}
    for nm in order:
        ms = median_ms(ev[nm])
        if nm.startswith("attn"):
            flop = fwd_flop if nm == "attn_fwd" else bwd_flop
            tf = flop / (ms * 1e-3) / 1e12
            out[nm] = {"ms": ms, "TFLOP/s": tf, "frac_of_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                       "flop": flop}
        else:
            gb = xbytes[nm] / (ms * 1e-3) / 1e9
            out[nm] = {"ms": ms, "GB/s": gb, "frac_of_hbm_peak": gb / HBM_PEAK_GBPS}
    out["method"] = (f"{reps} iterations after {warm} warm-up, each call bracketed by HIP events on "
                     "the launch stream, median")
    del segs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def oracle_plan():
    """The CPU oracle (fp64, OpenMP over output rows) timed on this host over
    the measurement plan: the forward of the tiny P=2 share (both ranks) and
    of the 32K share in full, the packed-document 64K share forward and
    backward in full, and sampled query rows (first 256, last 256, 1024
    seeded random; all heads) of the 128K and 256K forwards, each with the
    full-pass time extrapolated from the sample's algorithmic flop (labelled
    as such).  A reported baseline, not a target."""
    import numpy as np

    import oracle
    import synth

    def f64(w, s_, heads, scale=1.0):
        return synth.to_f64(w.head_tensor(s_, heads, scale=scale), w.dtype)

    res = {"cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle", "runs": {}}

    def record(name, flop, dt, **extra):
        res["runs"][name] = dict({"seconds": dt, "flop": flop, "TFLOP/s": flop / dt / 1e12}, **extra)
        print(f"oracle plan: {name} {dt:.1f} s", file=sys.stderr, flush=True)

    # tiny P=2 share: both ranks' forward (fp32 inputs)
    w = synth.WORKLOADS["tiny-p2"]
    t0 = time.perf_counter()
    flop = 0.0
    for r in range(w.P):
        q, k, v = (synth.to_f64(synth.normal(w.seed, s_, (w.seqlen, 1, w.hq, w.head_dim), "f32"), "f32")
                   [:, :, r * w.hq_local:(r + 1) * w.hq_local] for s_ in (1, 2, 3))
        oracle.attn_fwd(np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v),
                        w.softmax_scale, True)
        flop += 4.0 * w.head_dim * w.hq_local * w.causal_pairs()
    record("tiny-p2 forward (both ranks, full)", flop, time.perf_counter() - t0)

    for name, bwd in (("llama8b-share-32k", False), ("packed-docs-64k", True)):
        w = synth.WORKLOADS[name]
        q = f64(w, synth.STREAM_Q, w.hq_local, w.q_prescale)
        k, v = f64(w, synth.STREAM_K, w.hkv_local), f64(w, synth.STREAM_V, w.hkv_local)
        cu = w.cu_seqlens()
        flop = 4.0 * w.head_dim * w.hq_local * w.causal_pairs()
        t0 = time.perf_counter()
        oracle.attn_fwd(q, k, v, w.softmax_scale, True, cu)
        record(f"{name} forward (full)", flop, time.perf_counter() - t0)
        if bwd:
            # Documents are independent (block-diagonal mask), so the full
            # backward is each document's backward in turn; one progress line
            # per document.
            do = f64(w, synth.STREAM_DO, w.hq_local)
            t0 = time.perf_counter()
            for d0, d1 in zip(cu[:-1], cu[1:]):
                sl = slice(int(d0), int(d1))
                oracle.attn_bwd(np.ascontiguousarray(q[sl]), np.ascontiguousarray(k[sl]),
                                np.ascontiguousarray(v[sl]), np.ascontiguousarray(do[sl]),
                                w.softmax_scale, True)
                print(f"oracle plan: {name} backward, document of {d1 - d0} tokens done "
                      f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
            record(f"{name} backward (full, document by document)", 2.5 * flop,
                   time.perf_counter() - t0)

    for name in ("llama8b-share-128k", "long-256k"):
        w = synth.WORKLOADS[name]
        N = w.seqlen
        rng = np.random.default_rng(w.seed)
        rows = np.unique(np.concatenate([np.arange(256), np.arange(N - 256, N),
                                         rng.integers(0, N, size=1024)])).astype(np.int64)
        q = f64(w, synth.STREAM_Q, w.hq_local, w.q_prescale)
        k, v = f64(w, synth.STREAM_K, w.hkv_local), f64(w, synth.STREAM_V, w.hkv_local)
        flop = 4.0 * w.head_dim * w.hq_local * float(np.sum(rows + 1))
        t0 = time.perf_counter()
        oracle.attn_fwd(q, k, v, w.softmax_scale, True, None, rows=rows)
        dt = time.perf_counter() - t0
        full = 4.0 * w.head_dim * w.hq_local * w.causal_pairs()
        record(f"{name} forward ({len(rows)} sampled rows)", flop, dt,
               extrapolated_full_seconds=dt * full / flop,
               extrapolation="sample time x (full algorithmic flop / sample flop); not measured")
    return res


def measure_fused(uly, torch, np, stream, args, rank, scale, lse, ws, tables, fwd_flop,
                  bwd_flop, unfused_ms):
    """The same step with the exchange fused into the attention kernels
    (ulysses_attn_fwd_fused + ulysses_attn_bwd_fused: no head-sharded copies,
    no exchange launches), timed like the main step."""
    cq, ck, cv, co, cdo, cdq, cdk, cdv = tables

    def fstep(ev=None):
        if ev is not None:
            ev[0].record(stream)
        uly.ulysses_attn_fwd_fused(cq, ck, cv, co, lse, rank, scale, True)
        if ev is not None:
            ev[1].record(stream)
        uly.ulysses_attn_bwd_fused(cq, ck, cv, co, lse, cdo, cdq, cdk, cdv, ws, rank, scale, True)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        fstep()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        fstep(events[s_])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in events]))
    bwd_ms = float(np.mean([ev[1].elapsed_time(ev[2]) for ev in events]))
    tf = (fwd_flop + bwd_flop) / (ms * 1e-3) / 1e12
    return {"ms_per_step": ms, "TFLOP/s": tf, "speedup_vs_unfused_step": unfused_ms / ms,
            "attn_fwd_fused": {"ms": fwd_ms, "TFLOP/s": fwd_flop / (fwd_ms * 1e-3) / 1e12},
            "attn_bwd_fused": {"ms": bwd_ms, "TFLOP/s": bwd_flop / (bwd_ms * 1e-3) / 1e12},
            "method": "ulysses_attn_fwd_fused + ulysses_attn_bwd_fused on the sequence chunks, "
                      "same inputs, steps and warmup as the main step"}


def measure_logits_loss(uly, torch, np, stream, args):
    """The language-model loss of one rank's tokens at the Llama-8B lm_head
    (d = 4096, vocab = 128256) over the 128K share's 16384 tokens,
    --loss-shard-rows rows of logits at a time: three GEMMs per shard (6 T V d
    flop in all) and the
    row kernel.  Outside the attention step; timed with HIP events on the
    launch stream around each call."""
    import synth
    T, d, V, shard = 16384, 4096, 128256, args.loss_shard_rows
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    h = torch.randn((T, d), device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn((V, d), device="cuda", generator=gen) * (2.0 / d ** 0.5)).to(torch.bfloat16)
    labels = torch.tensor(synth.lm_labels(99, T, V, 10), device="cuda")
    rows = torch.empty(T, dtype=torch.float32, device="cuda")
    total = torch.empty(1, dtype=torch.float32, device="cuda")
    good = torch.empty(1, dtype=torch.int64, device="cuda")
    dh = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((V, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(uly.ulysses_logits_loss_workspace_size(shard, V), dtype=torch.uint8,
                     device="cuda")

    def call():
        uly.ulysses_logits_loss(h, w, labels, rows, total, good, dh, dw, ws, 1.0 / T, shard)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    reps = max(args.steps, 3)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        ev[i].record(stream)
        call()
    ev[reps].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
    flop = 6.0 * T * V * d
    tf = flop / (ms * 1e-3) / 1e12
    out = {"ms": ms, "TFLOP/s": tf, "frac_of_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
           "flop": flop, "tokens": T, "hidden": d, "vocab": V, "shard_rows": shard,
           "loss_sum_finite": bool(torch.isfinite(total).item()),
           "method": f"{reps} calls back to back after 2 warm-up calls, HIP events on the "
                     "launch stream; every kernel (matrix-core GEMMs, the row kernel and the loss sum) by libulysses"}
    del h, w, dh, dw, ws
    torch.cuda.empty_cache()
    return out


def measure_tiled_mlp(uly, torch, np, stream, args):
    """The sequence-tiled SwiGLU MLP at the Llama-8B block shape (d = 4096,
    inter = 14336) over the 128K share's 16384 tokens in ceil(T / d) = 4
    shards: forward and backward timed separately with HIP events.
    Algorithmic work: forward 3 products (6 T d I flop), backward 6 products
    (12 T d I); the backward also recomputes g and u (4 T d I more)."""
    T, d, inter = 16384, 4096, 14336
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    bf = torch.bfloat16
    x = torch.randn((T, d), device="cuda", generator=gen).to(bf)
    dy = torch.randn((T, d), device="cuda", generator=gen).to(bf)
    wg = (torch.randn((inter, d), device="cuda", generator=gen) / d ** 0.5).to(bf)
    wu = (torch.randn((inter, d), device="cuda", generator=gen) / d ** 0.5).to(bf)
    wd = (torch.randn((d, inter), device="cuda", generator=gen) / inter ** 0.5).to(bf)
    y = torch.empty((T, d), dtype=bf, device="cuda")
    dx = torch.empty((T, d), dtype=bf, device="cuda")
    dwg = torch.empty((inter, d), device="cuda")
    dwu = torch.empty((inter, d), device="cuda")
    dwd = torch.empty((d, inter), device="cuda")
    ws = torch.empty(uly.ulysses_tiled_mlp_workspace_size(d, d, inter, True), dtype=torch.uint8,
                     device="cuda")

    def fwd():
        uly.ulysses_tiled_mlp_fwd(x, wg, wu, wd, y, ws, d)

    def bwd():
        uly.ulysses_tiled_mlp_bwd(x, wg, wu, wd, dy, dx, dwg, dwu, dwd, ws, d)

    out = {"tokens": T, "hidden": d, "inter": inter, "shard_rows": d}
    reps = max(args.steps, 3)
    for name, fn, flop, executed in (("fwd", fwd, 6.0 * T * d * inter, 6.0 * T * d * inter),
                                     ("bwd", bwd, 12.0 * T * d * inter, 16.0 * T * d * inter)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for i in range(reps):
            ev[i].record(stream)
            fn()
        ev[reps].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = {"ms": ms, "TFLOP/s": tf, "frac_of_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                     "executed_TFLOP/s": executed / (ms * 1e-3) / 1e12}
    out["method"] = (f"{reps} calls each back to back after 2 warm-up calls, HIP events on the "
                     "launch stream; every kernel (matrix-core GEMMs and the SwiGLU row kernels) by libulysses")
    del x, dy, wg, wu, wd, y, dx, dwg, dwu, dwd, ws
    torch.cuda.empty_cache()
    return out


def time_rotated(torch, stream, fns, reps):
    """Average ms of `reps` launches cycling through `fns` (one per buffer
    set), after one warm-up pass over every set; one pair of events on the
    launch stream.  A launch returning a non-zero status raises."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(reps):
        status = fns[i % len(fns)]()
        if status not in (None, 0):
            raise RuntimeError(f"launch failed with status {status}")
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / reps


def measure_merge(w, uly, torch, stream, n_sets, reps):
    """Throughput of the partial-result merge (the combination step of ring /
    blockwise attention, outside the Ulysses step) at the share's forward
    shape: two (O, LSE) partials merged into a third buffer, cycling through
    `n_sets` distinct sets so that every launch reads HBM."""
    lib = uly.load_library()
    N, hl, hd = w.seqlen, w.hq_local, w.head_dim
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261202)
    sets = []
    for _ in range(n_sets):
        o_a, o_b, o = (torch.randn((N, 1, hl, hd), device="cuda", generator=gen).to(torch.bfloat16)
                       for _ in range(3))
        l_a, l_b, l = (8.0 * torch.randn((1, hl, N), device="cuda", generator=gen) for _ in range(3))
        sets.append((o_a, l_a, o_b, l_b, o, l))
    st = stream.cuda_stream

    def caller(t):
        ptrs = [x.data_ptr() for x in t]
        def f():
            return lib.ulysses_attn_merge(ptrs[0], ptrs[1], ptrs[2], ptrs[3], N, 1, hl, hd, uly.BF16,
                                          ptrs[4], ptrs[5], st)
        return f

    ms = time_rotated(torch, stream, [caller(t) for t in sets], reps)
    nbytes = 3.0 * (N * hl * hd * 2 + N * hl * 4)   # two partials read, one result written
    gb = nbytes / (ms * 1e-3) / 1e9
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"ms": ms, "GB/s": gb, "frac_of_hbm_peak": gb / HBM_PEAK_GBPS, "bytes": nbytes,
            "method": f"{reps} back-to-back launches over {n_sets} rotating buffer sets (HBM-cold); "
                      "not part of the step"}


def measure_exchanges(w, uly, torch, stream, n_sets, reps):
    """Throughput of the four layout exchanges of a step, each launched
    `reps` times back to back while cycling through `n_sets` distinct buffer
    sets (every set is larger than the 256 MB Infinity Cache together with
    its neighbour, so each launch finds its data in HBM: cold numbers).  The
    launch arguments are marshalled once per set, so the host stays ahead of
    the GPU.  A device-to-device copy of the same bytes, rotated the same
    way, is the practical ceiling."""
    import ctypes

    import numpy as np

    lib = uly.load_library()
    N, P, n, r = w.seqlen, w.P, w.n_local, w.rank
    hl, kl, hd = w.hq_local, w.hkv_local, w.head_dim
    bf = torch.bfloat16
    st = stream.cuda_stream

    def seq(heads):
        return torch.empty((N, 1, heads, hd), dtype=bf, device="cuda")

    def head(heads):
        return torch.empty((N, 1, heads, hd), dtype=bf, device="cuda")

    def chunks(t):
        return [t[c * n:(c + 1) * n] for c in range(P)]

    def batch_args(pairs):
        descs, keep = uly._batch_descs(pairs)
        return descs, keep

    calls = {"pack_qkv": [], "unpack_o": [], "pack_do": [], "unpack_dqkv": []}
    keep_alive = []
    for _ in range(n_sets):
        sq, sk, sv = seq(w.hq), seq(w.hkv), seq(w.hkv)
        hq_, hk_, hv_ = head(hl), head(kl), head(kl)
        so, ho = seq(w.hq), head(hl)
        sdo, hdo = seq(w.hq), head(hl)
        sdq, sdk, sdv = seq(w.hq), seq(w.hkv), seq(w.hkv)
        hdq, hdk, hdv = head(hl), head(kl), head(kl)
        keep_alive += [sq, sk, sv, hq_, hk_, hv_, so, ho, sdo, hdo, sdq, sdk, sdv, hdq, hdk, hdv]
        d1, k1 = batch_args([(chunks(sq), hq_), (chunks(sk), hk_), (chunks(sv), hv_)])
        d4, k4 = batch_args([(chunks(sdq), hdq), (chunks(sdk), hdk), (chunks(sdv), hdv)])
        co, cdo = uly._ptr_array(chunks(so)), uly._ptr_array(chunks(sdo))
        keep_alive += [d1, k1, d4, k4, co, cdo]
        calls["pack_qkv"].append(lambda d=d1: lib.ulysses_seq_to_head_batch(
            d, 3, P, r, n, 1, hd, uly.BF16, st))
        calls["unpack_o"].append(lambda c=co, h=ho: lib.ulysses_head_to_seq(
            h.data_ptr(), P, r, n, 1, w.hq, hd, uly.BF16, c, st))
        calls["pack_do"].append(lambda c=cdo, h=hdo: lib.ulysses_seq_to_head(
            c, P, r, n, 1, w.hq, hd, uly.BF16, h.data_ptr(), st))
        calls["unpack_dqkv"].append(lambda d=d4: lib.ulysses_head_to_seq_batch(
            d, 3, P, r, n, 1, hd, uly.BF16, st))
    e = 2
    nbytes = {"pack_qkv": 2.0 * N * (hl + 2 * kl) * hd * e, "unpack_o": 2.0 * N * hl * hd * e,
              "pack_do": 2.0 * N * hl * hd * e, "unpack_dqkv": 2.0 * N * (hl + 2 * kl) * hd * e}

    def timed(fns):
        return time_rotated(torch, stream, fns, reps)

    out = {}
    tot_ms, tot_b = 0.0, 0.0
    for name, fns in calls.items():
        ms = timed(fns)
        out[name] = {"ms": ms, "GB/s": nbytes[name] / (ms * 1e-3) / 1e9}
        tot_ms += ms
        tot_b += nbytes[name]
    out["all"] = {"ms": tot_ms, "GB/s": tot_b / (tot_ms * 1e-3) / 1e9,
                  "frac_of_hbm_peak": tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del keep_alive, calls

    # Practical ceiling: a plain device-to-device copy moving the bytes of the
    # Q/K/V pack (read + write), rotated over the same number of buffer sets.
    half = int(nbytes["pack_qkv"] // 2)
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
             torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(n_sets)]
    def copier(src, dst):
        def f():
            dst.copy_(src, non_blocking=True)
        return f

    copy_ms = timed([copier(s_, d_) for s_, d_ in bufs])
    out["d2d_copy_same_bytes"] = {"ms": copy_ms, "GB/s": 2.0 * half / (copy_ms * 1e-3) / 1e9}
    out["method"] = (f"{reps} back-to-back launches per exchange over {n_sets} rotating buffer "
                     "sets (HBM-cold), one pair of HIP events on the launch stream")
    del bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, n_rows):
    """The oracle's forward on a bounded sample of query rows of the same
    workload (all heads), timed on this host's cores; reported in the same
    unit as the GPU (algorithmic TFLOP/s of the rows computed)."""
    import numpy as np

    import oracle
    import synth

    N = w.seqlen
    rows = np.linspace(0, N - 1, n_rows).round().astype(np.int64)
    q = synth.to_f64(w.head_tensor(synth.STREAM_Q, w.hq_local, scale=w.q_prescale), w.dtype)
    k = synth.to_f64(w.head_tensor(synth.STREAM_K, w.hkv_local), w.dtype)
    v = synth.to_f64(w.head_tensor(synth.STREAM_V, w.hkv_local), w.dtype)
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, w.softmax_scale, True, None, rows=rows)
    dt = time.perf_counter() - t0
    flop = 4.0 * w.head_dim * w.hq_local * float(np.sum(rows + 1))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": dt,
            "sample": f"attention forward for {n_rows} evenly spaced query rows of N={N} "
                      f"(all {w.hq_local} heads), fp64, {flop:.3e} algorithmic flop"}


if __name__ == "__main__":
    sys.exit(main())
