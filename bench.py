"""Benchmark of the fused multi-LoRA MoE expert layer on one MI355X.

One step = one full layer call (route, align, gate_up shrink, gate_up
projection with fused LoRA expand + SwiGLU, down shrink, down projection with
fused LoRA expand, weighted combine) over one batch of synthetic tokens whose
inputs are already resident in HBM.

Default workload: the decode-shaped layer (16 tokens, hidden = intermediate =
2880, 32 experts top-4, 8 adapters of rank 32). The prefill-shaped layer
(4 x 1600 tokens, same dims) is measured in the same run and reported in the
"prefill" object of the same JSON line; the wide-expert, many-adapter, tiny
and dense (one expert) layers follow in "other_workloads".

Weight copies are rotated between calls so that the working set of
consecutive calls exceeds the 256 MB Infinity Cache. Where a layer runs the
16-row projection kernels (decode-sized batches) it is given packed copies of
its base weights, as a serving process would prepare once at load time
(--row-layout: without them); config.launch.packed_weights says which.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

from lora_mixture_experts_amd.profsum import read_traffic


HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
WORKLOAD_NAMES = {"decode": "decode-shaped MoE-LoRA layer (T=16, H=I=2880, E=32 top-4, L=8, r=32)",
                  "prefill": "prefill-shaped MoE-LoRA layer (T=6400=4x1600, H=I=2880, E=32 top-4, L=8, r=32)",
                  "wide": "wide-expert layer (T=64, H=4096, I=11008, E=8 top-2, L=8, r=32)",
                  "many": "many-adapter layer (T=512, H=I=2880, E=32 top-4, L=128, r=64)",
                  "tiny": "tiny MoE-LoRA layer (T=16, H=256, I=512, E=8 top-2, L=2, r=8)",
                  "dense": "dense multi-LoRA MLP (T=16, H=5120, I=25600, one expert, L=8, r=32)"}
RIDGE_FLOP_PER_BYTE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def routing_stats(case, ids):
    """Touched experts / (expert, adapter) segments of the sampled routing."""
    T, k, L = case.T, case.top_k, case.L
    experts = np.unique(ids)
    segs = set()
    p_lora = 0
    for t in range(T):
        a = int(case.adapter_ids[t])
        if 0 <= a < L:
            p_lora += k
            for e in ids[t]:
                segs.add((a, int(e)))
    return dict(n_experts=len(experts), n_segments=len(segs), P=T * k, P_lora=p_lora)


def algorithmic(case, st):
    """Algorithmic bytes / flops per kernel (inputs read once, outputs written
    once, intermediates counted only where a kernel must read/write them)."""
    H, I, r, T, k = case.H, case.I, case.r, case.T, case.top_k
    P, PL, ne, ns = st["P"], st["P_lora"], st["n_experts"], st["n_segments"]
    b = {}
    b["shrink_gate_up"] = ns * r * H * 2 + PL * H * 2 + PL * r * 4
    b["gemm_gate_up"] = ne * 2 * I * H * 2 + ns * 2 * I * r * 2 + T * H * 2 + PL * r * 4 + P * I * 2
    b["shrink_down"] = ns * r * I * 2 + PL * I * 2 + PL * r * 4
    b["gemm_down"] = ne * H * I * 2 + ns * H * r * 2 + P * I * 2 + PL * r * 4 + P * H * 4
    b["combine"] = P * H * 4 + T * H * 4 + P * 8
    b["route"] = T * case.E * 4 + P * 8
    b["align"] = P * 4 + T * 4
    f = {}
    f["gemm_gate_up"] = 2.0 * P * 2 * I * H + 2.0 * PL * 2 * I * r
    f["gemm_down"] = 2.0 * P * H * I + 2.0 * PL * H * r
    f["shrink_gate_up"] = 2.0 * PL * r * H
    f["shrink_down"] = 2.0 * PL * r * I
    layer_bytes = ne * 3 * H * I * 2 + ns * r * (2 * H + 3 * I) * 2 + T * H * 2 + T * case.E * 4 + T * H * 4
    layer_flops = 6.0 * H * I * P + 2.0 * r * (2 * H + 3 * I) * PL
    return b, f, layer_bytes, layer_flops


SHRINK_OF = {"gemm_gate_up": "shrink_gate_up", "gemm_down": "shrink_down"}


def shrinks_fused(kus):
    """True when the shrinks had no launch of their own: the library then
    reports 0 us for them (they ran inside the projection launches)."""
    return all(kus.get(s, 0.0) == 0.0 for s in SHRINK_OF.values())


def combine_fused(kus):
    """True when the weighted combine had no launch of its own (the down
    projection added its weighted rows into the output: the library reports
    0 us for the combine)."""
    return kus.get("combine", 0.0) == 0.0


def fold_fused(kus, b, f, T=None, H=None, P=None):
    """Per-kernel bytes/flops with each shrink's work counted in the
    projection launch that ran it (when the shrinks have no launch of their
    own), and, when the combine is folded into the down projection, that
    launch writing the fp32 output [T][H] once instead of its fp32 rows
    [P][H] (the routing launch then also clears the output)."""
    b, f = dict(b), dict(f)
    if shrinks_fused(kus):
        for g, s in SHRINK_OF.items():
            b[g] += b.pop(s)
            f[g] += f.pop(s)
            b[s] = f[s] = 0
    if combine_fused(kus) and T is not None:
        # drop the fp32 rows [P][H]; write out [T][H] once and read the P
        # routing weights; the routing launch's clearing of out is its own
        b["gemm_down"] += -P * H * 4 + T * H * 4 + P * 4
        b["route"] += T * H * 4
        b["combine"] = 0
    return b, f


def lora_kernels_summary(kus, b):
    """HBM rate of the kernels that carry the LoRA shrink and expand (the two
    shrinks, when launched, and the two projections with the fused expand)."""
    names = ("shrink_gate_up", "gemm_gate_up", "shrink_down", "gemm_down")
    us = sum(kus[n] for n in names)
    by = sum(b[n] for n in names)
    gbs = by / (us * 1e-6) / 1e9 if us else None
    return {"shrinks": "inside the projection launches" if shrinks_fused(kus) else "own launches",
            "kernels_us": round(us, 2), "bytes": int(by),
            "achieved_gbs": round(gbs, 1) if gbs else None,
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4) if gbs else None}


def run_workload(name, steps, warmup, rotate, dev, table=None, packed=True):
    import torch

    import oracle
    from lora_mixture_experts_amd import moe_lora as ml
    from lora_mixture_experts_amd import workloads as wl

    t0 = time.time()
    case = wl.make_case(name)
    ids, _ = oracle.route(case.logits, case.top_k)
    st = routing_stats(case, ids)
    log(f"[{name}] inputs drawn in {time.time() - t0:.1f}s; {st}")
    base = wl.device_tensors(case, dev)
    layers = []
    for i in range(rotate):
        tens = base if i == 0 else {k: v.clone() for k, v in base.items()}
        layers.append((ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r,
                                tens["w_gate_up"], tens["w_down"], tens["a_gate_up"],
                                tens["b_gate_up"], tens["a_down"], tens["b_down"], tuning=table,
                                packed_weights=packed), tens))
    layer0 = layers[0][0]
    bm_b, bm_l = ml.block_sizes(layer0.desc)
    launch = {"block_m_base": bm_b, "block_m_lora": bm_l,
              "shrink_launch": bool(layer0.desc.flags & ml.FLAG_SHRINK_LAUNCH),
              "combine": ("own launch, fixed order" if layer0.keeps_down_rows
                          else "in the down projection's epilogue (fp32 atomic adds)"),
              "from_tuning_table": layer0.tuned is not None,
              "packed_weights": layer0.packed}
    out = torch.empty((case.T, case.H), dtype=torch.float32, device=dev)

    def step(i):
        layer, tens = layers[i % rotate]
        layer(tens["x"], tens["logits"], tens["adapter_ids"], out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # five repeats of the same `steps` calls; the reported time is their median
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    repeats = []
    for _ in range(5):
        ev0.record()
        for i in range(steps):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        repeats.append(ev0.elapsed_time(ev1) / steps)
    ms = float(np.median(repeats))
    # the status word of each weight copy's last call: nonzero means some
    # projection wave stopped waiting for the shrink waves of its launch and
    # computed its own shrink (valid output, slower); reported, not hidden
    status_words = [layer.status() for layer, _ in layers]
    if any(status_words):
        log(f"[{name}] status words {status_words}: some projection waves computed their own shrink")

    # per-kernel durations: HIP events recorded by the library around each
    # kernel on the launch stream, over a second pass of the same steps
    ml.timing_enable(steps)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    kms, ncalls = ml.timing_read()
    ml.timing_enable(0)
    kernel_us = {n: 1000.0 * v / max(ncalls, 1) for n, v in zip(ml.kernel_names(), kms)}
    b, f, layer_bytes, layer_flops = algorithmic(case, st)
    del layers, base
    torch.cuda.empty_cache()
    launch["status_words"] = status_words
    return case, ids, st, ms, kernel_us, b, f, layer_bytes, layer_flops, repeats, launch


def workload_summary(name, c, st, ms, kus, b, f, lb, lf, repeats_ms, launch=None):
    """One workload's object: throughput, per-kernel times, layer roofline and
    the dominant projection kernel against its bound."""
    b, f = fold_fused(kus, b, f, c.T, c.H, c.T * c.top_k)
    dom = max(("gemm_gate_up", "gemm_down"), key=lambda n: kus[n])
    mfma = lf / lb > RIDGE_FLOP_PER_BYTE
    roof_us = max(lb / (HBM_PEAK_GBS * 1e9), lf / (BF16_PEAK_TFLOPS * 1e12)) * 1e6
    traffic = read_traffic(os.path.join(ROOT, "profiles", f"hbm_traffic_{name}.md"), dom)
    if mfma:
        achieved = f[dom] / (kus[dom] * 1e-6) / 1e12
        roof = dict(kernel=dom, bound="mfma", achieved=round(achieved, 1), peak=BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / BF16_PEAK_TFLOPS, 4), traffic=traffic,
                    flops_per_launch=f[dom], bytes_per_launch=b[dom], us_per_launch=round(kus[dom], 2))
    else:
        achieved = b[dom] / (kus[dom] * 1e-6) / 1e9
        roof = dict(kernel=dom, bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    bytes_per_launch=b[dom], us_per_launch=round(kus[dom], 2))
    gemm_us = kus["gemm_gate_up"] + kus["gemm_down"]
    out = {"workload": WORKLOAD_NAMES[name], "value": round(c.T / (ms * 1e-3), 1), "unit": "tokens/s",
           "us_per_call": round(ms * 1e3, 2),
           "us_per_call_repeats": [round(v * 1e3, 2) for v in repeats_ms],
           "layer_bound": "mfma" if mfma else "hbm",
           "layer_roofline_frac": round(roof_us / (ms * 1e3), 4),
           "kernel_us": {k: round(v, 2) for k, v in kus.items()}, "routing": st, "roofline": roof,
           "lora_shrink_expand_kernels": lora_kernels_summary(kus, b)}
    if launch is not None:
        out["launch"] = launch
    if mfma:
        tf = (f["gemm_gate_up"] + f["gemm_down"]) / (gemm_us * 1e-6) / 1e12
        out["base_gemms_tflops"] = round(tf, 1)
        out["base_gemms_mfma_frac"] = round(tf / BF16_PEAK_TFLOPS, 4)
    else:
        gb = (b["gemm_gate_up"] + b["gemm_down"]) / (gemm_us * 1e-6) / 1e9
        out["projection_kernels_gbs"] = round(gb, 1)
        out["projection_kernels_hbm_frac"] = round(gb / HBM_PEAK_GBS, 4)
    return out


def cpu_baseline(case, budget_s, single_budget_s, chunk=None):
    """The fp64 C oracle timed on the host cores over a bounded sample of the
    workload: consecutive chunks of `chunk` tokens (default: the whole batch)
    until `budget_s` seconds have passed."""
    import oracle
    ids_, w = oracle.route(case.logits, case.top_k)
    cores = oracle.default_threads()
    n_tok = min(chunk or case.T, case.T)

    def timed(threads, budget):
        done, t0, c = 0, time.perf_counter(), 0
        while True:
            lo = (c * n_tok) % case.T
            toks = np.arange(lo, min(lo + n_tok, case.T), dtype=np.int32)
            oracle.forward(case, ids_, w, tokens=toks, threads=threads)
            done += len(toks)
            c += 1
            if time.perf_counter() - t0 >= budget:
                break
        return done, time.perf_counter() - t0

    done, dt = timed(cores, budget_s)
    what = (f"{done // n_tok} full {case.name} batches of {n_tok}" if n_tok == case.T
            else f"{done // n_tok} chunks of {n_tok} consecutive tokens of the {case.T}-token {case.name} batch")
    out = dict(value=done / dt, unit="tokens/s", cores=cores, kind="oracle",
               us_per_call=round(case.T / (done / dt) * 1e6, 1),
               sample=f"{done} tokens ({what}) through the fp64 C oracle in {dt:.1f}s")
    if single_budget_s > 0:
        d1, t1 = timed(1, single_budget_s)
        out["single_thread"] = dict(value=d1 / t1, unit="tokens/s", cores=1,
                                    sample=f"{d1} tokens in {t1:.1f}s")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=list(WORKLOAD_NAMES))
    ap.add_argument("--cpu-single-budget", type=float, default=3.0,
                    help="seconds of the one-thread oracle run reported beside the all-core one")
    ap.add_argument("--also", default="prefill,wide,many,tiny,dense",
                    help="comma list of further workloads reported in the same line ('none' = none)")
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--tuning", default=None, metavar="DIR",
                    help="tuning folder (per-shape block sizes and shrink placement); default: the "
                         "package's configs folder when it exists")
    ap.add_argument("--no-tuning", action="store_true", help="use the library's default choices")
    ap.add_argument("--row-layout", action="store_true",
                    help="do not give the 16-row kernels packed copies of the base weights")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="first run one plain device-to-device copy of this size, as the "
                         "reference dispatch for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is a design, not a built path)", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    if args.calibrate_copy > 0:
        # reference dispatches of known size for the HBM byte counters: the
        # runtime's device-to-device copy, then an elementwise kernel that
        # streams the same bytes in and out with ordinary vector loads/stores
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    from lora_mixture_experts_amd import tuning
    table, table_dir = None, None
    if not args.no_tuning:
        table_dir = args.tuning or tuning.DEFAULT_FOLDER
        if args.tuning or os.path.isdir(table_dir):
            table = tuning.load(table_dir)
        else:
            table_dir = None
    case, ids, st, ms, kus, b, f, lbytes, lflops, reps, launch = run_workload(
        args.workload, args.steps, args.warmup, args.rotate, dev, table, not args.row_layout)
    main_obj = workload_summary(args.workload, case, st, ms, kus, b, f, lbytes, lflops, reps, launch)
    line = {
        "metric": "MoE-LoRA layer tokens/s + us/call (decode 16 tok, prefill 6400 tok); % roofline",
        "value": main_obj["value"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "us_per_call": main_obj["us_per_call"],
        "us_per_call_repeats": main_obj["us_per_call_repeats"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded, N(0,1) activations/logits, N(0,0.02) weights)",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "global_batch": case.T, "seq_len": 1,
                   "parallelism": "none (1 GPU)", "rotated_weight_copies": args.rotate,
                   "tuning_table": os.path.relpath(table_dir, ROOT) if table_dir else None,
                   "launch": launch},
        "layer_roofline_frac": main_obj["layer_roofline_frac"],
        "kernel_us": main_obj["kernel_us"],
        "lora_shrink_expand_kernels": main_obj["lora_shrink_expand_kernels"],
        "routing": st,
        "roofline": main_obj["roofline"],
    }
    others = [w for w in args.also.split(",") if w and w != "none" and w != args.workload]
    prefill_case = None
    for name in others:
        steps2 = max(5, args.steps // 5) if name in ("prefill", "many") else max(10, args.steps // 2)
        res = run_workload(name, steps2, max(2, args.warmup // 2), args.rotate, dev, table, not args.row_layout)
        obj = workload_summary(name, res[0], res[2], *res[3:])
        if name == "prefill":
            line["prefill"] = obj
            prefill_case = res[0]
        else:
            line.setdefault("other_workloads", {})[name] = obj
        del res
    if args.cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_budget, args.cpu_single_budget)
        if prefill_case is not None:
            # the prefill-shaped layer on the host: chunks of 400 tokens (a
            # quarter of one 1600-token request) for about the same budget
            line["prefill"]["cpu_baseline"] = cpu_baseline(prefill_case, args.cpu_budget, 0, chunk=400)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
