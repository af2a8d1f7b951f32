#!/usr/bin/env python3
"""Throughput of the W4A16 INT4 grouped MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload decode|prefill|skew|ep|tp8_decode|tp8_prefill|tiny]

Default workload (the one the metric is quoted on): one Kimi-K2.6-shape MoE
layer (hidden 7168, moe_intermediate 2048, 384 int4 group-32 experts, top-8,
one bf16 shared expert) in decode, batches of 1, 8, 32 and 64 tokens. A step is
one forward at each of the four batch sizes; every batch size has its own copy
of the weights, so a call never finds weights left in L2/MALL by the previous
call. Inputs are seeded synthetic data, resident in HBM before timing starts.

Prints one JSON line: tokens/s over the timed steps, the dominant kernel's
roofline (algorithmic bytes or FLOPs per launch over its average duration,
timed with HIP events that the library records around that kernel on its
launch stream during the timed steps), the HBM traffic measured by rocprofv3
counters when it was taken on the current kernel source, and the fp64 CPU
oracle timed on a bounded sample of the same workload. `per_batch` adds a
per-stage breakdown from a short pass with all stage events after the timed
region (`us_per_call` there includes those extra event packets), and the time
of the router step (scores -> top-k ids and weights) that would precede the
layer, measured on its own (it is not part of the timed step: the layer takes
ids and weights as inputs).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 MoE layer tokens/s; decode HBM GB/s and prefill TFLOP/s vs roofline"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
# block_m of the paths whose gate_up launch also carries the shared expert
# (small-batch and tiled kernels); prefill-sized blocks give it its own launch
SINGLE_LAUNCH_BLOCK_M = (4, 16, 64)
GEMM_SRCS = [os.path.join(ROOT, "w4a16_int4_grouped_moe_amd", "csrc", f)
             for f in ("gemm.hip", "gemm_small.hip", "gemm_prefill.hip")]


# ----------------------------------------------------------------------------
# algorithmic work (what the layer must read, write and compute)
# ----------------------------------------------------------------------------
def w13_bytes(H, I):   # one expert's gate/up: int4 codes + bf16 group scales
    return 2 * I * H // 2 + 2 * I * (H // 32) * 2


def w2_bytes(H, I):
    return H * I // 2 + H * (I // 32) * 2


def work(T, H, I, k, ids, n_local, base, shared, shared_in_kernel=True):
    """Bytes the layer must move and FLOPs it must do; gate_up_* are those of the
    launch that carries the routed experts' gate_up (it also carries the shared
    expert unless that runs in a launch of its own: shared_in_kernel False)."""
    import numpy as np

    flat = np.asarray(ids).ravel()
    local = (flat >= base) & (flat < base + n_local)
    P = int(local.sum())
    U = int(np.unique(flat[local]).size)
    s13 = 2 * I * H * 2 if shared else 0
    s2 = H * I * 2 if shared else 0
    ts = T if shared else 0
    layer_bytes = U * (w13_bytes(H, I) + w2_bytes(H, I)) + s13 + s2 + 2 * T * H * 2 + T * k * 8
    layer_flops = (P + ts) * (2 * (2 * I) * H + 2 * H * I)
    ks = ts if shared_in_kernel else 0
    gate_up_bytes = U * w13_bytes(H, I) + (s13 if ks else 0) + T * H * 2 + (P + ks) * I * 2
    gate_up_flops = (P + ks) * 2 * (2 * I) * H
    return dict(P=P, U=U, gate_up_bytes=gate_up_bytes, layer_bytes=layer_bytes,
                gate_up_flops=gate_up_flops, layer_flops=layer_flops)


# ----------------------------------------------------------------------------
# HIP events (raw handles, recorded by the library on its launch stream)
# ----------------------------------------------------------------------------
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def traffic_record(workload):
    """rocprofv3 FETCH_SIZE / WRITE_SIZE of the gate_up kernel, if the record in
    profiles/ was taken on the current GEMM sources (workload: the record's
    name, e.g. "prefill" or "prefill_prepacked")."""
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(f, "rb").read())
    sha = h.hexdigest()
    path = os.path.join(ROOT, "profiles", f"gate_up_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        m = re.match(r"\s*traffic_record:\s*(\{.*\})\s*$", line)
        if m:
            rec = json.loads(m.group(1))
            if rec.get("gemm_sources_sha256") == sha:
                return rec
    return None


def cpu_baseline(calls, shared, n_tokens, seconds):
    """The fp64 oracle on a bounded sample of the same workload: the first
    n_tokens tokens of each batch, batch after batch, until `seconds` of wall
    time have passed (at least one pass over every batch)."""
    import numpy as np

    import moe_inputs as mi
    import oracle

    threads = oracle.oracle.default_threads()
    jobs = []
    for c in calls:
        w = c["w"]
        rows = np.arange(min(n_tokens, w.T))
        used, remap = mi.compact_routing(c["ids_np"], rows, w.expert_base, w.n_local)
        bank = mi.weight_bank(w.seed_bank, w.geo.hidden, w.geo.inter, used or [0])
        jobs.append((c["x_np"][rows], remap, c["wts_np"][rows], bank))
    done, n_calls, t0 = 0, 0, time.perf_counter()
    while True:
        for x, remap, wts, bank in jobs:
            oracle.forward(x, remap, wts, bank.packed_w13, bank.scales_w13, bank.packed_w2,
                           bank.scales_w2, shared, 0, threads=threads)
            done += x.shape[0]
            n_calls += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    w = calls[0]["w"]
    return {"value": round(done / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} tokens: {n_calls} oracle calls on the first <= {n_tokens} tokens of "
                      f"each {w.name} batch ({[c['T'] for c in calls]}), fp64 C oracle, "
                      f"{dt:.1f} s wall on {threads} threads"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "skew", "ep", "tp8_decode", "tp8_prefill",
                             "tiny"])
    ap.add_argument("--tokens", type=int, default=0,
                    help="token count of a single-batch workload (default: the workload's own)")
    ap.add_argument("--cpu-tokens", type=int, default=32,
                    help="tokens per batch of the CPU-oracle sample (0 disables it)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the CPU-oracle sample (repeated passes)")
    ap.add_argument("--prepacked", action="store_true",
                    help="run the layer on prepacked weights (moe_w4a16_prepack, once per "
                         "weight copy, before the timed region)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this layer build has no multi-GPU path "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_inputs as mi
    import w4a16_int4_grouped_moe_amd as moe

    dev = torch.device("cuda:0")
    hip = Hip()
    if args.workload in ("decode", "tp8_decode"):
        batches = [1, 8, 32, 64]
    else:
        batches = [args.tokens or mi.workload(args.workload).T]
    w0 = mi.workload(args.workload, batches[0])
    g = w0.geo
    t_setup = time.perf_counter()
    bank = mi.device_bank(w0.seed_bank, g.hidden, g.inter, w0.bank_experts(), dev)
    shared_np = mi.shared_weights(w0.seed_bank, g.hidden, g.inter) if g.shared else None
    shared = mi.to_device(shared_np, dev) if g.shared else None

    calls = []
    for i, T in enumerate(batches):
        w = mi.workload(args.workload, T)
        x = mi.activations(w.seed_x + w.T, w.T, g.hidden)
        ids, wts = mi.make_routing(w)
        b = bank if i == 0 else {k: v.clone() for k, v in bank.items()}
        s = shared if (i == 0 or shared is None) else shared.clone()
        p = moe.problem(T, g.hidden, g.inter, w.n_local, g.top_k, w.expert_base)
        bm = moe.forward_block_m(p)
        calls.append(dict(
            w=w, T=T, x_np=x, ids_np=ids, wts_np=wts,
            args=(mi.to_device(x, dev), mi.to_device(ids, dev), mi.to_device(wts, dev),
                  b["packed_w13"], b["scales_w13"], b["packed_w2"], b["scales_w2"], s),
            out=torch.empty((T, g.hidden), dtype=torch.bfloat16, device=dev),
            ws=torch.empty(max(moe.workspace_size(p), 1), dtype=torch.uint8, device=dev),
            work=work(T, g.hidden, g.inter, g.top_k, ids, w.n_local, w.expert_base, g.shared,
                      shared_in_kernel=bm in SINGLE_LAUNCH_BLOCK_M),
            bm=bm, base=w.expert_base))
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    print(f"[bench] setup {t_setup:.1f} s; workload {args.workload} batches {batches}",
          file=sys.stderr, flush=True)

    if args.prepacked:
        for c in calls:  # the weight copies are replaced by their prepacked form
            a = c["args"]
            c["pk"] = moe.prepack(a[3], a[4], a[5], a[6])
            c["args"] = a[:3] + (None, None, None, None) + a[7:]
        torch.cuda.synchronize()

    def run(c, events=None):
        if args.prepacked:
            x, ids, wts = c["args"][:3]
            moe.forward_prepacked(x, ids, wts, c["pk"], c["args"][7], out=c["out"],
                                  expert_base=c["base"], workspace=c["ws"], stage_events=events)
        else:
            moe.forward(*c["args"], out=c["out"], expert_base=c["base"], workspace=c["ws"],
                        stage_events=events)

    for _ in range(args.warmup):
        for c in calls:
            run(c)
    torch.cuda.synchronize()

    # timed region: only the two events that bracket the dominant kernel (the
    # routed experts' gate_up launch) are recorded, so that event packets add
    # little to the step time
    events = [[[None, hip.event(), None, None, None, hip.event(), None] for _ in calls]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for step in range(args.steps):
        for c, ev in zip(calls, events[step]):
            run(c, ev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_step = sum(batches)
    value = tokens_per_step / (ms_per_step / 1e3)

    # after the timed region: a short pass with all stage events, for the
    # per-stage breakdown (these extra event packets lengthen the calls a little)
    n_diag = min(5, args.steps)
    diag = [[[hip.event() for _ in range(7)] for _ in calls] for _ in range(n_diag)]
    for step in range(n_diag):
        for c, ev in zip(calls, diag[step]):
            run(c, ev)
    torch.cuda.synchronize()

    # the router step in front of the layer (scores of all the model's experts
    # -> top-k ids and weights), timed on its own per batch size: HIP events
    # around single calls on the launch stream
    route_us = []
    for c in calls:
        w = c["w"]
        sc = torch.from_numpy(mi.router_scores(600 + w.T, w.T, g.n_experts)).to(dev)
        rid = torch.empty((w.T, g.top_k), dtype=torch.int32, device=dev)
        rw = torch.empty((w.T, g.top_k), dtype=torch.float32, device=dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_diag + 1)]
        for i in range(n_diag + 1):
            ev[i][0].record()
            moe.route(sc, g.top_k, num_experts=w.n_local, expert_base=w.expert_base,
                      topk_ids=rid, topk_weights=rw)
            ev[i][1].record()
        torch.cuda.synchronize()
        route_us.append(float(np.median([a.elapsed_time(b) for a, b in ev[1:]])) * 1e3)

    # the same steps with the weights in prepacked form (moe_w4a16_prepack, a
    # one-time load step outside the timing), where the widths allow it; the
    # headline above stays on the checkpoint-layout weights the layer's entry
    # point takes
    prepacked = None
    if not args.prepacked:
        try:
            pks = [moe.prepack(*c["args"][3:7]) for c in calls]
        except (ValueError, moe.MoeError):
            pks = None
        if pks:
            def run_pk(c, pk, ev=None):
                x, ids, wts = c["args"][:3]
                moe.forward_prepacked(x, ids, wts, pk, c["args"][7], out=c["out"],
                                      expert_base=c["base"], workspace=c["ws"], stage_events=ev)

            for _ in range(args.warmup):
                for c, pk in zip(calls, pks):
                    run_pk(c, pk)
            ev_pk = [[[None, hip.event(), None, None, None, hip.event(), None] for _ in calls]
                     for _ in range(args.steps)]
            torch.cuda.synchronize()
            t2 = time.perf_counter()
            for step in range(args.steps):
                for c, pk, ev in zip(calls, pks, ev_pk[step]):
                    run_pk(c, pk, ev)
            torch.cuda.synchronize()
            ms_pk = (time.perf_counter() - t2) * 1e3 / args.steps
            prepacked = {
                "value": round(tokens_per_step / (ms_pk / 1e3), 1), "ms_per_step": round(ms_pk, 4),
                "gate_up_us": [round(float(np.mean([hip.elapsed_ms(ev_pk[s][ci][1], ev_pk[s][ci][5])
                                                    for s in range(args.steps)])) * 1e3, 2)
                               for ci in range(len(calls))],
                "note": "same steps with the weights prepacked once (moe_w4a16_prepack) and "
                        "moe_w4a16_forward_prepacked; results identical bit for bit"}
            del pks

    stage_names = ["align", "gate_up", "down", "combine"]
    per_batch = []
    gate_up_ms, gate_up_bytes, gate_up_flops = [], [], []
    for ci, c in enumerate(calls):
        gu = np.array([hip.elapsed_ms(events[s][ci][1], events[s][ci][5])
                       for s in range(args.steps)])
        st = np.array([[hip.elapsed_ms(diag[s][ci][j], diag[s][ci][j + 1]) for j in range(4)]
                       for s in range(n_diag)])
        call_ms = st.sum(1)
        wk = c["work"]
        avg = st.mean(0)
        per_batch.append(dict(
            T=c["T"], us_per_call=round(float(np.median(call_ms)) * 1e3, 2),
            tokens_per_s=round(c["T"] / (float(np.median(call_ms)) / 1e3), 1),
            layer_hbm_gbs=round(wk["layer_bytes"] / (float(np.median(call_ms)) / 1e3) / 1e9, 1),
            layer_tflops=round(wk["layer_flops"] / (float(np.median(call_ms)) / 1e3) / 1e12, 2),
            experts_hit=wk["U"], pairs=wk["P"],
            gate_up_us=round(float(gu.mean()) * 1e3, 2),
            routed_us={"gate_up": round(float(np.mean([hip.elapsed_ms(diag[s][ci][1], diag[s][ci][5])
                                                       for s in range(n_diag)])) * 1e3, 2),
                       "down": round(float(np.mean([hip.elapsed_ms(diag[s][ci][2], diag[s][ci][6])
                                                    for s in range(n_diag)])) * 1e3, 2)},
            stage_us={n: round(float(v) * 1e3, 2) for n, v in zip(stage_names, avg)},
            router_us=round(route_us[ci], 2)))
        gate_up_ms.append(float(gu.mean()))
        gate_up_bytes.append(wk["gate_up_bytes"])
        gate_up_flops.append(wk["gate_up_flops"])

    # dominant kernel: the gate_up GEMM (two thirds of the routed weight bytes
    # and of the FLOPs); per-launch averages over the timed steps
    mean_s = float(np.mean(gate_up_ms)) / 1e3
    rec = traffic_record(args.workload + ("_prepacked" if args.prepacked else ""))
    traffic = None
    if rec is not None:
        traffic = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    if args.workload in ("prefill", "tp8_prefill"):
        ach = float(np.mean(gate_up_flops)) / mean_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        ach = float(np.mean(gate_up_bytes)) / mean_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
    bms = [moe.forward_block_m(moe.problem(T, g.hidden, g.inter, w0.n_local, g.top_k))
           for T in batches]
    if all(b == 4 for b in bms):
        roof["kernel"] = ("small_gemm_kernel<gate_up>: routed + shared experts, int4 dequant + "
                          "MFMA 4x4x4, fused SwiGLU")
    elif all(b in SINGLE_LAUNCH_BLOCK_M for b in bms):
        roof["kernel"] = ("grouped_gemm_kernel<gate_up>: routed + shared experts, int4 dequant + "
                          "MFMA 16x16x32, fused SwiGLU")
    else:
        roof["kernel"] = ("prefill_gemm_kernel<gate_up>: routed experts, int4 dequant + "
                          "MFMA 16x16x32, fused SwiGLU")
    roof["algorithmic_per_launch"] = (float(np.mean(gate_up_flops)) if roof["bound"] == "mfma"
                                      else float(np.mean(gate_up_bytes)))
    roof["avg_launch_us"] = round(mean_s * 1e6, 2)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(calls, shared_np, args.cpu_tokens, args.cpu_seconds)

    if args.workload == "decode":
        wl = ("Kimi-K2.6-shape W4A16 MoE layer decode: hidden 7168, moe_intermediate 2048, "
              "384 int4 g32 experts, top-8, bf16 shared expert; batches 1/8/32/64 tokens")
    elif args.workload.startswith("tp8"):
        wl = ("one GPU's share of the Kimi-K2.6-shape W4A16 MoE layer under 8-way tensor "
              "parallelism: hidden 7168, moe_intermediate 256, 384 int4 g32 experts, top-8, "
              f"bf16 shared expert (intermediate 256); batches {'/'.join(map(str, batches))}")
    else:
        wl = f"Kimi-K2.6-shape W4A16 MoE layer, {args.workload} workload, T={batches[0]}"
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded: int4 codes uniform, bf16 scales U(0.005,0.02), "
                "x N(0,1), uniform distinct top-k routing, softmax weights)",
        "config": {"workload": wl, "batches": batches, "hidden": g.hidden, "inter": g.inter,
                   "weights": "prepacked" if args.prepacked else "checkpoint layout",
                   "experts": w0.n_local, "top_k": g.top_k, "shared_expert": g.shared,
                   "block_m": [moe.forward_block_m(moe.problem(T, g.hidden, g.inter, w0.n_local,
                                                               g.top_k)) for T in batches]},
        "per_batch": per_batch,
        "roofline": roof,
        "cpu_baseline": cpu,
        "prepacked": prepacked,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
