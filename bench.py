"""Throughput of one batched Kolibri-1 block-drafter round on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config I] [--no-cpu-baseline]

A step is one kd_round over every stream of the workload (tap fuse, row build,
4 layers with spine and cross-attention, restricted NVFP4 head, argmax), for
the ingesting workload preceded by the kd_ingest of each stream's new context
rows, with every input already resident in HBM. The default workload is the 4-stream
configuration: 4 streams, 2048 context rows each, FP8 body, NVFP4 head.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "drafter rounds/s & draft tokens/s at B streams; % of HBM roofline"
HBM_PEAK_GBS = 8000.0
# the kernel of each small-batch path: path 2 launches k_small_phase once per
# phase (30 launches per 4-layer round), path 3 runs the whole round in
# one launch
KERNEL_NAME = {2: "kd::k_small_phase", 3: "kd::k_small_mega"}
LAUNCHES_PER_ROUND = {2: 30, 3: 1}


def algorithmic_bytes(dims, lens, streams, ingest=0, kv="bf16", head="nvfp4", body="fp8"):
    """Bytes a step must move: weights once (block-FP8 body with scales, or an
    NVFP4 / bf16 body in its own format, NVFP4
    head with block and tensor scales, fp32 vectors), 40,960 B of bf16 K/V per
    visible context row per stream (4 layers x K,V x 20 heads x 128 x 2 B;
    with the rotated 4-bit cache 10,880 B: 64 code bytes and a 4-byte fp16
    scale and offset per layer, K/V, head), and per stream its tapped states,
    4 embedding rows, ids, length and outputs. A bf16 head slice reads 2 B
    per value instead of the NVFP4 head's codes and scales.
    With `ingest` new context rows per stream ahead of the round: their tapped
    states, next-token ids and embedding rows, and the 40,960 B of K/V each
    writes (the weights they use are the round's, counted once); `lens` are the
    lengths the round sees."""
    import synth
    mb = synth.model_bytes(dims, body)
    if head == "bf16":
        mb["head"] = dims.draft_vocab * dims.hidden * 2
    elif head == "fp8":
        mb["head"] = dims.draft_vocab * dims.hidden + dims.draft_vocab * dims.hidden // 64 * 4
    if kv == "int4":
        kv_row = dims.layers * 2 * dims.heads * (dims.head_dim // 2 + 4)
    else:
        kv_row = dims.layers * 2 * dims.heads * dims.head_dim * 2
    vis = sum(min(int(l), dims.window) for l in lens)
    per_stream = (dims.taps * dims.hidden * 2 + dims.block * dims.hidden * 2
                  + 4 * (1 + (dims.block - 1) + 1 + dims.block))
    ingest_bytes = streams * ingest * (dims.taps * dims.hidden * 2 + 4 + dims.hidden * 2 + kv_row)
    total = mb["body"] + mb["head"] + mb["vectors"] + kv_row * vis + per_stream * streams + ingest_bytes
    return dict(total=total, body=mb["body"], head=mb["head"], kv=kv_row * vis, ingest=ingest_bytes)


# the sources the small-batch round kernels are compiled from
SMALL_SOURCES = ("kd_device.h", "kd_runtime.h", "kd_small.h", "kd_small.hip")


def kernel_source_hash():
    """sha256 over the sources of the small-batch round kernels with comments
    and blank space removed, first 12 hex digits: identifies the kernels a
    counter measurement was taken on (an edit of comments alone, or of the
    general path's sources, keeps it)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in [os.path.join(ROOT, "block_draft_model_amd", "csrc", n) for n in SMALL_SOURCES]:
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:12]


def measured_traffic(workload, kernel):
    """HBM bytes per round moved by the round's launches of `kernel`, from the
    rocprofv3 counter summary, if it was taken on the kernels as they are now
    (same source hash), else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    sha = kernel_source_hash()
    for line in lines:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 9 and cells[0] == workload and cells[1] == kernel and cells[2] == sha:
            return int(cells[7].replace(",", ""))
    return None


GAP_MIN = 1e-2        # rows whose top-2 logit gap is at most this may pick either id
REL_L2_MAX = 1e-2     # per-row relative L2 bound of the logits


def cpu_baseline(model, inp, gpu_logits=None, gpu_ids=None, max_seconds=20.0, max_rounds=8):
    """The oracle, as it stands, on this host: rounds of the same workload
    until about max_seconds have passed. Weight decoding to fp64 is timed as a
    separate one-off load step. With the GPU's logits and ids of the same
    inputs, also the parity of that round against the oracle's first round:
    per-row relative L2 of the logits, and the ids on every row whose top-2
    gap exceeds GAP_MIN."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    t0 = time.perf_counter()
    M = oracle.OracleModel(synth.to_numpy_model(model))
    load_s = time.perf_counter() - t0
    inp_np = synth.to_numpy_inputs(inp)
    times = []
    first = None
    t_start = time.perf_counter()
    while len(times) < max_rounds and (time.perf_counter() - t_start) < max_seconds:
        t1 = time.perf_counter()
        out = oracle.oracle_round(M, inp_np)
        times.append(time.perf_counter() - t1)
        first = out if first is None else first
    per_round = sum(times) / len(times)
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    base = {"value": 1.0 / per_round, "unit": "rounds/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} full rounds of the same workload in fp64 NumPy "
                      f"({per_round:.2f} s/round); weight decode to fp64 {load_s:.1f} s "
                      f"as a separate load step; host CPU: {cpu}"}
    parity = None
    if gpu_logits is not None:
        ref_logits, ref_ids = first
        g = np.asarray(gpu_logits, dtype=np.float64).reshape(-1, ref_logits.shape[-1])
        r = np.asarray(ref_logits).reshape(g.shape)
        rel = np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)
        top2 = -np.sort(-r, axis=1)[:, :2]
        gated = (top2[:, 0] - top2[:, 1]) > GAP_MIN
        differ = np.asarray(gpu_ids).reshape(-1) != np.asarray(ref_ids).reshape(-1)
        parity = {"rows": int(len(rel)), "max_rel_l2": float(rel.max()), "rel_l2_bound": REL_L2_MAX,
                  "gated_rows": int(gated.sum()), "mismatches": int(np.sum(differ & gated)),
                  "exempt_near_tie_rows": int(np.sum(~gated)),
                  "exempt_rows_differing": int(np.sum(differ & ~gated)),
                  "finite": bool(np.all(np.isfinite(g)))}
    return base, parity


# the cold-cache variant sweeps (reads and writes) this many float32 values
# before each step: 1 GiB, four times the 256 MB last-level cache (MALL) of
# MI355X, so the step finds neither its weights nor its cache rows in L2 or MALL
COLD_FLUSH_ELEMS = 1 << 28


def run_workload(kdraft, synth, torch, drafter, model, cfg, steps, warmup, kv_fmt, head, keep=False,
                 cold_steps=0):
    """Times `steps` rounds of one workload after `warmup`: HIP events around
    the whole timed region (ms per step) and around each step (p10/p50/p90).
    cold_steps: afterwards, time that many steps one by one, each after a
    sweep over a 1 GiB buffer (events around the step only).
    keep: also return the inputs, for a parity round outside the timed region."""
    dims = synth.FULL
    inp = synth.make_inputs(cfg, dims, device="cuda", vocab=model["vocab"], kv=kv_fmt)
    B = inp["streams"]
    stream = torch.cuda.current_stream()
    if kv_fmt == "int4":
        kv = kdraft.kv_struct_int4(inp["k"], inp["v"], inp["k_so"], inp["v_so"])
    else:
        kv = kdraft.kv_struct(inp["k"], inp["v"])
    ids = torch.empty(B, 4, dtype=torch.int32, device="cuda")
    n_ingest = cfg.get("ingest", 0)
    # the lengths the timed rounds see (an ingesting step appends its rows
    # first; the window keeps the visible rows at min(len, 2048) as they grow)
    lens_host = [l + n_ingest for l in inp["lens"].cpu().tolist()]

    def step():
        if n_ingest:
            drafter.ingest(B, n_ingest, inp["ingest_taps"], inp["ingest_ids"], kv, inp["lens"])
        drafter.round(B, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids, None)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[-1]) / steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    q = lambda f: per[min(len(per) - 1, int(f * len(per)))]
    res = dict(B=B, ms=ms, p10=q(0.1), p50=q(0.5), p90=q(0.9), wall=wall, lens=lens_host,
               ingest=n_ingest, path=drafter.last_path())
    if cold_steps:
        flush = torch.zeros(COLD_FLUSH_ELEMS, dtype=torch.float32, device="cuda")
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(cold_steps)]
        for e0, e1 in cev:
            flush.add_(1.0)
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        cper = sorted(e0.elapsed_time(e1) for e0, e1 in cev)
        cq = lambda f: cper[min(len(cper) - 1, int(f * len(cper)))]
        res["cold"] = dict(steps=cold_steps, p10=cq(0.1), p50=cq(0.5), p90=cq(0.9),
                           flush_bytes_per_step=2 * 4 * COLD_FLUSH_ELEMS)
        del flush
    if keep:
        res["inp"], res["kv"] = inp, kv
    else:
        del inp, kv
    return res


PATH_NAME = {1: "general multi-kernel", 2: "small-batch phases, one launch each",
             3: "small-batch persistent kernel"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=None,
                    help="time only this workload (index into the five); default: the 4-stream "
                         "workload as the headline, then every workload in the configs list")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=30,
                    help="steps of the headline workload timed one by one after a 1 GiB cache sweep (0: none)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB 5 times and "
                         "exit: the calibration kernel for HBM byte counters")
    ap.add_argument("--kv", choices=("bf16", "int4"), default="bf16",
                    help="context cache format: bf16, or rotated 4-bit codes with an fp16 "
                         "scale and offset per row (read by the general path)")
    ap.add_argument("--head", choices=("nvfp4", "bf16", "fp8"), default="nvfp4",
                    help="head slice format: NVFP4, or bf16 / block-FP8 (read by the general path)")
    ap.add_argument("--body", choices=("fp8", "nvfp4", "bf16"), default="fp8",
                    help="body weight format: block-FP8, or NVFP4 / bf16 (read by the general path)")
    ap.add_argument("--path", type=int, default=0,
                    help="0 automatic; 1 general multi-kernel; 2 small-batch phases as "
                         "separate launches; 3 small-batch persistent kernel")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the round shards by stream with no collectives; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from block_draft_model_amd import kdraft

    if not torch.cuda.is_available():
        print("bench.py: no GPU available", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src_t = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst_t = torch.empty_like(src_t)
        torch.cuda.synchronize()
        for _ in range(5):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return
    dims = synth.FULL
    quant = {"nvfp4": kdraft.KD_QUANT_NVFP4, "bf16": kdraft.KD_QUANT_BF16, "fp8": kdraft.KD_QUANT_FP8_BLOCK64}
    head_q, body_q = quant[args.head], quant[args.body]
    stream = torch.cuda.current_stream()
    models, drafters = {}, {}

    def drafter_for(name):
        if name not in drafters:
            models[name] = synth.make_model(dims, name, device="cuda", head=args.head, body=args.body)
            d = kdraft.Drafter(max_streams=max(c["streams"] for c in synth.CONFIGS), stream=stream,
                               head_quant=head_q, body_quant=body_q)
            d.load_weights(models[name])
            d.debug_set_path(args.path)
            drafters[name] = d
        return drafters[name], models[name]

    head_i = 1 if args.config is None else args.config
    cfg = synth.CONFIGS[head_i]
    drafter, model = drafter_for(cfg["model"])
    r = run_workload(kdraft, synth, torch, drafter, model, cfg, args.steps, args.warmup, args.kv, args.head,
                     keep=not args.no_cpu_baseline, cold_steps=args.cold_steps)
    B, ms, path = r["B"], r["ms"], r["path"]
    ab = algorithmic_bytes(dims, r["lens"], B, r["ingest"], args.kv, args.head, args.body)
    rounds_s = 1000.0 / ms
    # roofline of the round's kernel: algorithmic bytes per launch over the
    # average launch duration (the HIP-event time of the timed rounds on the
    # stream the kernels run on, divided by the launches of a round)
    launches = LAUNCHES_PER_ROUND.get(path, 1)
    per_launch = ab["total"] / launches
    launch_us = ms * 1e3 / launches
    achieved = per_launch / (launch_us * 1e-6) / 1e9
    traffic_round = measured_traffic(cfg["name"], KERNEL_NAME.get(path, ""))
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic_round is None else round(traffic_round / launches),
                "kernel": KERNEL_NAME.get(path, "several kernels per round"),
                "launches_per_round": launches, "bytes_per_launch": round(per_launch),
                "avg_launch_us": round(launch_us, 3)}
    n_ingest = r["ingest"]
    out = {"metric": METRIC, "value": round(rounds_s, 2), "unit": "rounds/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           # matrix products take f16 inputs (FP8 / NVFP4 weights decoded exactly) and
           # accumulate in fp32; norms, softmax and the residual stream are fp32
           "dtype": "f16",
           "data": "synthetic",
           "config": {"workload": f"{cfg['name']}: {B} streams x 1 round"
                                  + (f" after ingesting {n_ingest} context rows per stream" if n_ingest else "")
                                  + ", draft block 4, "
                                  f"context rows per stream {sorted(set(min(l, 2048) for l in r['lens']))}, "
                                  f"{dict(nvfp4='NVFP4', bf16='bf16', fp8='block-FP8')[args.body]} body, "
                                  f"{dict(nvfp4='NVFP4', bf16='bf16', fp8='block-FP8')[args.head]} head (60,614 rows)"
                                  + (", rotated 4-bit K/V cache" if args.kv == "int4" else ""),
                      "streams": B, "draft_tokens_per_round": 4 * B, "kv_cache": args.kv, "head": args.head,
                      "body": args.body,
                      "path": PATH_NAME[path]},
           "draft_tokens_per_s": round(4 * B * rounds_s, 1),
           "bytes_per_round": ab, "hbm_roofline_frac": round(achieved / HBM_PEAK_GBS, 4),
           "wall_s": round(r["wall"], 3), "roofline": roofline}
    if "cold" in r:
        c = r["cold"]
        out["cold_cache"] = {"note": "each step after a read-write sweep of 1 GiB (L2 and the 256 MB MALL "
                                     "evicted); HIP events around the step only",
                             "steps": c["steps"], "ms_p10": round(c["p10"], 4), "ms_p50": round(c["p50"], 4),
                             "ms_p90": round(c["p90"], 4),
                             "hbm_roofline_frac_p50": round(ab["total"] / (c["p50"] * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}

    # the parity round of the headline workload (outside the timed region)
    gpu_logits = gpu_ids = None
    if not args.no_cpu_baseline:
        inp, kv = r["inp"], r["kv"]
        lg = torch.empty(B, 4, dims.draft_vocab, dtype=torch.float32, device="cuda")
        ids = torch.empty(B, 4, dtype=torch.int32, device="cuda")
        drafter.round(B, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids, lg)
        torch.cuda.synchronize()
        gpu_logits, gpu_ids = lg.cpu().numpy(), ids.cpu().numpy()
        del lg
    head_inp = r.pop("inp", None)
    r.pop("kv", None)

    # every workload: median and spread of the round time, throughput, roofline
    if args.config is None:
        rows = []
        for i, c in enumerate(synth.CONFIGS):
            if i == head_i:
                rr = r
            else:
                d, m = drafter_for(c["model"])
                big = c["streams"] >= 64
                rr = run_workload(kdraft, synth, torch, d, m, c, min(args.steps, 30) if big else args.steps,
                                  min(args.warmup, 5) if big else args.warmup, args.kv, args.head)
                torch.cuda.empty_cache()
            b = algorithmic_bytes(dims, rr["lens"], rr["B"], rr["ingest"], args.kv, args.head, args.body)["total"]
            rows.append({"workload": c["name"], "streams": rr["B"],
                         "ingest_rows_per_stream": rr["ingest"],
                         "steps": args.steps if i == head_i or rr["B"] < 64 else min(args.steps, 30),
                         "ms_p10": round(rr["p10"], 4), "ms_p50": round(rr["p50"], 4),
                         "ms_p90": round(rr["p90"], 4), "ms_mean": round(rr["ms"], 4),
                         "rounds_per_s": round(1000.0 / rr["p50"], 1),
                         "draft_tokens_per_s": round(4 * rr["B"] * 1000.0 / rr["p50"], 1),
                         "bytes_per_round": b,
                         "hbm_roofline_frac": round(b / (rr["p50"] * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                         "path": PATH_NAME[rr["path"]]})
        out["configs"] = rows
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(model, head_inp, gpu_logits, gpu_ids)
        out["cpu_baseline"] = base
        out["parity"] = dict(parity, workload=cfg["name"],
                             rule="per row relative L2 <= 1e-2; ids equal where the oracle's top-2 gap > 1e-2")
    print(json.dumps(out), flush=True)
    for d in drafters.values():
        d.close()


if __name__ == "__main__":
    main()
