"""Tune the launch configuration of the MoE-LoRA layer per shape, on the GPU.

For each workload it times every valid (base-view rows, LoRA-view rows, shrink
placement) choice on the workload's seeded synthetic inputs, with weight
copies rotated between calls as in bench.py, and stores the fastest choice
in the shape's JSON file of the tuning folder (lora_mixture_experts_amd/tuning.py
describes the format). This is the per-shape tuning of the AWS ML Blog post
"Efficiently serve dozens of fine-tuned models with vLLM on Amazon SageMaker
AI and Amazon Bedrock", section "Tuning kernel configurations for Amazon
SageMaker AI and Amazon Bedrock", with the choices this library exposes.

    python -m lora_mixture_experts_amd.tune --workload decode --workload prefill
"""
import argparse
import json
import os
import sys
import time

from . import moe_lora as ml
from . import tuning
from . import workloads as wl


def candidates(L):
    for bm_b in tuning.POW2_BLOCKS:
        for bm_l in (16, 32, 64):
            yield bm_b, bm_l, False
            # the shrink placement only differs where the library would run
            # the shrinks inside the projections (16-row base blocks)
            if bm_b == 16 and L > 0:
                yield bm_b, bm_l, True


DOWN_KSPLITS = (1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 25, 32, 50)


def split_candidates(case, plan):
    """Values of each split-K field to try around a resolved plan (the
    library's own value excluded); the caller keeps whichever is fastest,
    one field at a time."""
    out = {"down_ksplit": [d for d in DOWN_KSPLITS
                           if d != plan["down_ksplit"] and (case.I // 64) % d == 0 and case.I // 64 // d >= 8]}
    out["shrink_ksplit"] = ([v for v in (1, 2, 3, 4) if v != plan["shrink_ksplit"]]
                            if case.L > 0 and not plan["shrinks_in_projections"] else [])
    for f in ("waves_gate_up", "waves_down"):
        out[f] = [v for v in (1, 2, 4) if v != plan[f]] if plan["block_m_base"] == 16 else []
    out["frags_gate_up"] = ([v for v in (4, 8) if v != plan["frags_gate_up"]]
                            if plan["block_m_base"] == 16 and case.I % 64 == 0 else [])
    return out


def time_choice(case, copies, out, choice, steps, warmup, launch=None, packed=True):
    import torch
    bm_b, bm_l, sep = choice
    layers = []
    for t in copies:
        layers.append(ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r,
                               t["w_gate_up"], t["w_down"], t["a_gate_up"], t["b_gate_up"],
                               t["a_down"], t["b_down"], block_m_base=bm_b, block_m_lora=bm_l,
                               shrink_launch=sep, packed_weights=packed, **(launch or {})))

    def step(i):
        t = copies[i % len(copies)]
        layers[i % len(copies)](t["x"], t["logits"], t["adapter_ids"], out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    reps = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) * 1000.0 / steps)
    # a nonzero status word means some projection wave stopped waiting for
    # the shrink waves of its launch and computed its own shrink: the output
    # is valid and the time includes that slow path, so the choice stays a
    # candidate on its measured time
    if any(layer.status() != 0 for layer in layers):
        print(json.dumps({"workload": case.name, "choice": list(choice), "launch": launch or {},
                          "note": "status word set: shrink fallback ran"}), flush=True)
    del layers
    return sorted(reps)[1]


def tune_workload(name, folder, rotate=3, steps=None, packed=True):
    """packed: time every choice with packed weight copies (as the bench
    runs the 16-row kernels); False: the row layout only."""
    import torch
    dev = torch.device("cuda:0")
    case = wl.make_case(name)
    base = wl.device_tensors(case, dev)
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(rotate - 1)]
    out = torch.empty((case.T, case.H), dtype=torch.float32, device=dev)
    heavy = case.T * case.top_k > 4096
    steps = steps or (5 if heavy else 30)
    results = []
    for choice in candidates(case.L):
        d = ml.make_desc(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, choice[0], choice[1],
                         ml.FLAG_SHRINK_LAUNCH if choice[2] else 0)
        if ml.validate(d) != ml.OK:
            continue
        us = time_choice(case, copies, out, choice, steps, warmup=2 if heavy else 5, packed=packed)
        print(json.dumps({"workload": name, "block_m_base": choice[0], "block_m_lora": choice[1],
                          "shrink_launch": choice[2], "us": None if us is None else round(us, 2)}),
              flush=True)
        if us is not None:
            results.append((us, choice))
    d0 = ml.make_desc(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r)
    default = ml.block_sizes(d0)
    us_default = next((us for us, c in results if c == (default[0], default[1], False)), None)
    if not results:
        raise RuntimeError(f"{name}: no launch choice produced a valid call")
    us, best = min(results)
    # then the split-K fields of the best choice, one at a time
    flags = ml.FLAG_SHRINK_LAUNCH if best[2] else 0
    plan = ml.plan(ml.make_desc(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, best[0], best[1],
                                flags))
    launch = {}
    for field, values in split_candidates(case, plan).items():
        for v in values:
            trial = dict(launch, **{field: v})
            d = ml.make_desc(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, best[0], best[1],
                             flags, **trial)
            if ml.validate(d) != ml.OK:
                continue
            us_v = time_choice(case, copies, out, best, steps, warmup=2 if heavy else 5, launch=trial,
                               packed=packed)
            print(json.dumps({"workload": name, "block_m_base": best[0], "block_m_lora": best[1],
                              "shrink_launch": best[2], **trial,
                              "us": None if us_v is None else round(us_v, 2)}), flush=True)
            # keep a change only if it gains more than 1 % (run-to-run noise)
            if us_v is not None and us_v < 0.99 * us:
                us, launch = us_v, trial
    shape = {k: getattr(case, k) for k in tuning.SHAPE_KEYS}
    entry = {"T_max": case.T, "block_m_base": best[0], "block_m_lora": best[1], "shrink_launch": best[2],
             **{k: launch.get(k, 0) for k in tuning.SPLIT_KEYS},
             "us": round(us, 2),
             "us_library_default": None if us_default is None else round(us_default, 2)}
    path = tuning.save_entry(folder, shape, entry)
    print(json.dumps({"workload": name, "best": entry, "file": os.path.relpath(path)}), flush=True)
    del copies, base
    torch.cuda.empty_cache()
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", action="append", choices=list(wl.CONFIGS), required=True)
    ap.add_argument("--out", default=tuning.DEFAULT_FOLDER)
    ap.add_argument("--steps", type=int, default=0)
    ap.add_argument("--row-layout", action="store_true",
                    help="time without packed weight copies (the bench gives them to 16-row plans)")
    args = ap.parse_args()
    t0 = time.time()
    for name in args.workload:
        tune_workload(name, args.out, steps=args.steps or None, packed=not args.row_layout)
    print(f"tuned {len(args.workload)} workload(s) in {time.time() - t0:.0f}s", file=sys.stderr)


if __name__ == "__main__":
    main()
