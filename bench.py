"""Benchmark of the MSA prefill forward + backward on one MI355X.

One step = the whole path on one batch: forward (k2q CSR, plan, K/V alignment,
forward kernel) then backward (delta preprocessing, task tables, backward: pool
zeroing, main KV-parallel kernel, finalize).  Inputs are resident in HBM before the
timed region.  Prints one JSON line.

Effective FLOPs count only selected blocks: every member block of an (index head,
query) counts its 128 keys for each of the 16 query heads, 4*128 flops per (row, key)
forward and 10*128 backward.  Timing protocol of the pages' operator benchmark:
warmup steps, then a timed loop; per-phase medians come from HIP events.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
WORKLOAD_NAMES = {
    0: "single 512-token document, all causal blocks (dense causal GQA)",
    1: "one packed 16384-token row of 512..6000-token documents, uniform top-16",
    2: "single 16384-token document, diagonal + sink + 14 uniform blocks (top-16)",
    3: "single 65536-token document, diagonal + 3 local + 12 distance-decaying blocks",
    4: "4 packed 16384-token rows of short geometric documents, Zipf-skewed selection",
}


def member_slots(q2k, cu):
    """Count of member slots: ids in [0, blk(t)], first listing in the row."""
    T = int(cu[-1])
    t = np.arange(T)
    doc = np.searchsorted(cu, t, side="right") - 1
    blk = (t - cu[doc]) // 128
    ok = (q2k >= 0) & (q2k <= blk[None, :, None])
    first = np.ones_like(ok)
    for j in range(1, q2k.shape[2]):
        first[:, :, j] = ~np.any(q2k[:, :, :j] == q2k[:, :, j:j + 1], axis=2)
    return int((ok & first).sum())


def visible_keys(q2k, cu):
    """Keys each member slot actually lets its query see (causal): 128 for a block before
    the query's own, pos(t) % 128 + 1 for its own block.  Summed over the slots; the
    whole-block count charges 128 for every slot."""
    T = int(cu[-1])
    t = np.arange(T)
    doc = np.searchsorted(cu, t, side="right") - 1
    pos = t - cu[doc]
    blk = pos // 128
    ok = (q2k >= 0) & (q2k <= blk[None, :, None])
    first = np.ones_like(ok)
    for j in range(1, q2k.shape[2]):
        first[:, :, j] = ~np.any(q2k[:, :, :j] == q2k[:, :, j:j + 1], axis=2)
    keys = np.where(q2k == blk[None, :, None], (pos % 128 + 1)[None, :, None], 128)
    return int((keys * (ok & first)).sum())


def sweep(args, M, WL, torch):
    """Single 16-top-k document at T = 4k, 8k, 16k, 32k tokens (the sequence lengths of
    the pages' operator benchmark), selection as in workload 2 (diagonal + block 0 + 14
    uniform blocks): one JSON line per T with forward / backward medians, effective
    TFLOP/s and the peak device memory of one forward + backward (inputs, outputs and
    every library buffer, the stored dS tiles included), and of the same call sequence in
    the recompute dQ mode, which needs no dS tiles."""
    dev = "cuda:0"
    scale = 1.0 / math.sqrt(128.0)
    for T in (4096, 8192, 16384, 32768):
        cu, q2k = WL.make_custom([T], "sink", 2)
        slots = member_slots(q2k, cu)
        fwd_flops = 4.0 * 128 * 128 * 16 * slots
        bwd_flops = 2.5 * fwd_flops
        peak = {}
        for name, mode in (("recompute", M.DQ_RECOMPUTE), ("stored", M.DQ_STORED)):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            base = torch.cuda.memory_allocated()
            tens = WL.make_tensors(T, 3000 + T, device=dev)
            Q, K, V, dO = tens["Q"], tens["K"], tens["V"], tens["dO"]
            q2k_d = torch.from_numpy(q2k).to(dev)
            m = M.MSA(cu, dq_mode=mode, device=dev)
            O, LSE = m.forward(Q, K, V, q2k_d, scale)
            dQ, dK, dV = m.backward(Q, dO, O, LSE, scale)
            torch.cuda.synchronize()
            peak[name] = (torch.cuda.max_memory_allocated() - base) / 1e9
            if name == "recompute":
                del m, O, LSE, dQ, dK, dV, tens, Q, K, V, dO, q2k_d
        fwd_ms, bwd_ms = [], []
        for k in range(args.warmup + args.steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
            m.forward(Q, K, V, q2k_d, scale, O=O, LSE=LSE)
            ev[1].record()
            m.backward(Q, dO, O, LSE, scale, dQ=dQ, dK=dK, dV=dV)
            ev[2].record()
            torch.cuda.synchronize()
            if k >= args.warmup:
                fwd_ms.append(ev[0].elapsed_time(ev[1]))
                bwd_ms.append(ev[1].elapsed_time(ev[2]))
        f, b = float(np.median(fwd_ms)), float(np.median(bwd_ms))
        print(json.dumps({
            "sweep": "single document, top-16 (diagonal + block 0 + 14 uniform), 64 q / 4 kv heads",
            "tokens": T, "member_slots": slots, "dq_accum": "stored",
            "fwd_ms_median": round(f, 4), "bwd_ms_median": round(b, 4), "ms_per_layer": round(f + b, 4),
            "fwd_tflops": round(fwd_flops / f / 1e9, 2), "bwd_tflops": round(bwd_flops / b / 1e9, 2),
            "tflops": round((fwd_flops + bwd_flops) / (f + b) / 1e9, 2),
            "frac_mfma_peak": round((fwd_flops + bwd_flops) / (f + b) / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "peak_gb": round(peak["stored"], 3), "peak_gb_recompute_mode": round(peak["recompute"], 3),
            "steps": args.steps, "warmup": args.warmup}), flush=True)
        del m, O, LSE, dQ, dK, dV, tens, Q, K, V, dO, q2k_d


def cpu_baseline(cfg, budget_tokens):
    """The fp64 oracle on a bounded sample: the first `budget_tokens` queries of the
    workload's first document with their own selections.  A prefix of a causal
    document attends only to keys inside the prefix, so it is an exact sub-workload."""
    import workloads as WL
    from oracle import oracle as OR
    cu, q2k = WL.make_structure(cfg)
    Tp = min(budget_tokens, int(cu[1]))
    cup = np.array([0, Tp], dtype=np.int32)
    qp = np.ascontiguousarray(q2k[:, :Tp])
    tens = WL.make_tensors(int(cu[-1]), 1000 + cfg)
    Q, K, V, dO = (tens[k][:Tp].float().numpy().astype(np.float64) for k in ("Q", "K", "V", "dO"))
    scale = 1.0 / math.sqrt(128.0)
    OR.build(force=False)
    t0 = time.perf_counter()
    OR.forward(Q, K, V, qp, cup, scale)
    t1 = time.perf_counter()
    OR.backward(Q, K, V, dO, qp, cup, scale)
    t2 = time.perf_counter()
    fwd, bwd, _ = OR.effective_flops(qp, cup)
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": round((fwd + bwd) / (t2 - t0) / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "first %d queries of the first document of workload %d (exact causal "
                      "sub-workload), fp64 forward %.1f s + backward %.1f s" % (Tp, cfg, t1 - t0, t2 - t1)}


# HBM bytes per launch of the main backward kernels at the headline workload (config 2,
# dQ from stored dS tiles), from rocprofv3 FETCH_SIZE / WRITE_SIZE runs scaled by the same counters'
# reading for a plain copy of known size; valid only for the build they were taken on:
# sha256 over every library source the backward launches depend on (the forward's own
# file excepted) and the build script with its compiler flags.
TRAFFIC_SOURCES = ["msa_abi.hip", "msa_backward.hip", "msa_backward_kv.hip", "msa_backward_kv2.hip", "msa_backward_dq.hip",
                   "msa_backward_dqs.hip", "msa_index.hip", "msa_walk.h", "msa_device.h", "msa_launch.h",
                   "../build.py"]
TRAFFIC_RECORD = {"config": 2, "dq_mode": "stored",
                  "sha256": "f6a36f1a09f7b06235e0d2c840e65380a5e38f217482ea17c7d0ad6a8ee6015a",
                  "bytes": 17034090629}  # read 12.516 GB + written 4.518 GB


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.normpath(os.path.join(ROOT, "block_sparse_attention_q2k_amd", "csrc", f)), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(cfg, dq_mode):
    r = TRAFFIC_RECORD
    if r is None or cfg != r["config"] or dq_mode != r["dq_mode"] or sources_digest() != r["sha256"]:
        return None
    return r["bytes"]


def time_index_select(M, WL, torch, cu, m, dev, reps=10):
    """The indexer's block selection on the same layout (synthetic index-Q / index-K):
    kept out of `value`, as the pages' timing excludes selection."""
    T = int(cu[-1])
    it = WL.make_index_tensors(T, 4242, device=dev)
    q2k = torch.empty((4, T, 16), dtype=torch.int32, device=dev)
    for _ in range(3):
        m.select(it["IQ"], it["IK"], q2k)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        m.select(it["IQ"], it["IK"], q2k)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    # every causal (query, block) pair scored over all 128 keys: 2 * 128 * 128 flop
    pairs = sum(int(p // 128) + 1 for d in range(len(cu) - 1) for p in range(int(cu[d + 1] - cu[d])))
    tflop = 4 * pairs * 2.0 * 128 * 128 / 1e12
    return {"ms": round(ms, 4), "tflop": round(tflop, 4), "tflops": round(tflop / (ms * 1e-3), 2),
            "note": "not part of value: the pages time the operator without selection"}


def copy_probe(mib):
    """A plain device copy of mib MiB, five times: what the HBM byte counters read for
    it calibrates them (read mib MiB, write mib MiB per launch)."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--dq-mode", choices=["stored", "recompute", "fp32", "bf16x2", "f16x2"], default="stored")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="single-document sequence sweep (T = 4k..32k) with peak memory, one line per T")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer a few times (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the operator runs on a single MI355X and this "
              "build has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    import block_sparse_attention_q2k_amd as M
    import workloads as WL
    if not os.path.exists(M._LIB_PATH):
        from block_sparse_attention_q2k_amd import build
        build.build()
    M.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.sweep:
        sweep(args, M, WL, torch)
        return
    cu, q2k = WL.make_structure(args.config)
    T = int(cu[-1])
    tens = WL.make_tensors(T, 1000 + args.config, device=dev)
    Q, K, V, dO = tens["Q"], tens["K"], tens["V"], tens["dO"]
    q2k_d = torch.from_numpy(q2k).to(dev)
    scale = 1.0 / math.sqrt(128.0)
    mode = {"stored": M.DQ_STORED, "recompute": M.DQ_RECOMPUTE, "fp32": M.DQ_ACCUM_FP32,
            "bf16x2": M.DQ_ACCUM_BF16X2, "f16x2": M.DQ_ACCUM_F16X2}[args.dq_mode]
    m = M.MSA(cu, grid=args.grid or None, dq_mode=mode, device=dev)
    O = torch.empty_like(Q)
    LSE = torch.empty((T, 64), dtype=torch.float32, device=dev)
    dQ = torch.empty_like(Q)
    dK = torch.empty_like(K)
    dV = torch.empty_like(V)

    slots = member_slots(q2k, cu)
    fwd_flops = 4.0 * 128 * 128 * 16 * slots
    bwd_flops = 2.5 * fwd_flops
    causal_fraction = visible_keys(q2k, cu) / (128.0 * slots)  # keys a query can see / charged keys

    def step(ev=None):
        if ev:
            ev[0].record()
        m.forward(Q, K, V, q2k_d, scale, O=O, LSE=LSE)
        if ev:
            ev[1].record()
        m.backward(Q, dO, O, LSE, scale, dQ=dQ, dK=dK, dV=dV)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(M.TIMING_EVENTS)] for _ in range(args.steps)]
    for row in kev:  # torch creates the HIP event on its first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        M.msa_set_timing_events(kev[k])
        step(evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    M.msa_set_timing_events(None)
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    split = mode in (M.DQ_RECOMPUTE, M.DQ_STORED)  # separate query-parallel dQ kernel
    recompute = mode == M.DQ_RECOMPUTE
    kern_ms = {"fwd": float(np.mean([e[0].elapsed_time(e[1]) for e in kev])),
               "kv": float(np.mean([e[2].elapsed_time(e[3]) for e in kev])),
               "dq": float(np.mean([e[4].elapsed_time(e[5]) for e in kev])) if split else 0.0}
    ms_step = elapsed * 1e3 / args.steps
    total_flops = fwd_flops + bwd_flops
    value = total_flops / (ms_step * 1e-3) / 1e12
    # Main backward: the KV-parallel kernel and (stored / recompute modes) the
    # query-parallel dQ kernel, back to back; together they do the backward's algorithmic
    # contractions.
    main_ms = kern_ms["kv"] + kern_ms["dq"]
    achieved = bwd_flops / (main_ms * 1e-3) / 1e12
    status = int(m.status[0].item())
    unit = 2.0 * 128 * 128 * 16 * slots  # one 128-dim contraction over all member (row, key) pairs
    kernels = [
        {"kernel": "fwd_kernel", "avg_ms": round(kern_ms["fwd"], 4), "algorithmic_tflop": round(2 * unit / 1e12, 4),
         "executed_tflop": round(2 * unit / 1e12, 4),
         "frac_mfma_peak": round(2 * unit / (kern_ms["fwd"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        {"kernel": ("bwd_kv2_kernel" if mode == M.DQ_STORED else "bwd_kv_kernel") if split else "bwd_kernel",
         "avg_ms": round(kern_ms["kv"], 4),
         "algorithmic_tflop": round((4 if split else 5) * unit / 1e12, 4),
         "executed_tflop": round((4 if split else 5) * unit / 1e12, 4),
         "frac_mfma_peak": round((4 if split else 5) * unit / (kern_ms["kv"] * 1e-3) / 1e12
                                 / MFMA_BF16_PEAK_TFLOPS, 4)},
    ]
    if split:
        kernels.append({"kernel": "dq_kernel" if recompute else "dqs_kernel", "avg_ms": round(kern_ms["dq"], 4),
                        "algorithmic_tflop": round(unit / 1e12, 4),
                        "executed_tflop": round((3 if recompute else 1) * unit / 1e12, 4),
                        "frac_mfma_peak": round(unit / (kern_ms["dq"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)})
    traffic = recorded_traffic(args.config, args.dq_mode)
    index_select = time_index_select(M, WL, torch, cu, m, dev)

    out = {
        "metric": "MSA fwd+bwd effective TFLOP/s + ms/layer at 16k packed tokens, 1 MI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; see workloads.py)",
        "config": {"workload": "config %d: %s" % (args.config, WORKLOAD_NAMES[args.config]),
                   "tokens": T, "documents": len(cu) - 1, "q_heads": 64, "kv_heads": 4,
                   "index_heads": 4, "head_dim": 128, "block": 128, "topk": 16,
                   "dq_accum": args.dq_mode, "grid": m.grid, "member_slots": slots},
        "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
        "bwd_ms_median": round(float(np.median(bwd_ms)), 4),
        "fwd_tflops": round(fwd_flops / (np.median(fwd_ms) * 1e-3) / 1e12, 3),
        "bwd_tflops": round(bwd_flops / (np.median(bwd_ms) * 1e-3) / 1e12, 3),
        "fwd_frac_mfma_peak": round(fwd_flops / (np.median(fwd_ms) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "bwd_frac_mfma_peak": round(bwd_flops / (np.median(bwd_ms) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "q2k_status": status,
        "flop_convention": "every member block counts all 128 keys for its 16 heads (4*128 flop per "
                           "(row, key) forward, 10*128 backward); keys a query can causally see are "
                           "causal_fraction of those",
        "causal_fraction": round(causal_fraction, 4),
        "causal_tflops": round(value * causal_fraction, 3),
        "roofline": {"kernel": "main backward: " + " + ".join(k["kernel"] for k in kernels[1:]),
                     "bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "avg_launch_ms": round(main_ms, 4), "traffic": traffic},
        "kernels": kernels,
        "index_select": index_select,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
