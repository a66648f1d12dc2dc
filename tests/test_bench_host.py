"""Host-side checks of bench.py: the algorithmic byte/flop model, the bound
selection, and the one-GPU contract (no GPU needed)."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def small_case():
    # 4 tokens, top-2 of 3 experts; adapters: 1, none, 0, 1 (L = 2)
    return SimpleNamespace(name="t", T=4, H=64, I=128, E=3, top_k=2, L=2, r=8,
                           adapter_ids=np.array([1, -1, 0, 1], np.int32))


def test_routing_stats_counts_touched_experts_and_segments():
    c = small_case()
    ids = np.array([[0, 1], [2, 0], [1, 2], [0, 1]], np.int32)
    st = bench.routing_stats(c, ids)
    # segments (adapter, expert): (1,0), (1,1), (0,1), (0,2); token 1 has none
    assert st == dict(n_experts=3, n_segments=4, P=8, P_lora=6)


def test_algorithmic_model_matches_the_layer_definition():
    c = small_case()
    st = dict(n_experts=3, n_segments=4, P=8, P_lora=6)
    b, f, lb, lf = bench.algorithmic(c, st)
    H, I, r = c.H, c.I, c.r
    # projections: 2 flops per multiply-add, base rows for every pair, LoRA
    # expand for pairs with an adapter
    assert f["gemm_gate_up"] == 2 * 8 * 2 * I * H + 2 * 6 * 2 * I * r
    assert f["gemm_down"] == 2 * 8 * H * I + 2 * 6 * H * r
    # layer: touched base weights (6HI bytes per expert), touched LoRA
    # (2r(2H+3I) per segment), x, logits, fp32 out
    assert lb == 3 * 6 * H * I + 4 * 2 * r * (2 * H + 3 * I) + 4 * H * 2 + 4 * 3 * 4 + 4 * H * 4
    assert lf == 6 * H * I * 8 + 2 * r * (2 * H + 3 * I) * 6
    # the gate_up kernel streams the touched experts' W_gu once
    assert b["gemm_gate_up"] >= 3 * 2 * I * H * 2


def test_bound_selection_uses_the_ridge_point():
    assert abs(bench.RIDGE_FLOP_PER_BYTE - 312.5) < 1e-9
    c = small_case()
    st = dict(n_experts=3, n_segments=4, P=8, P_lora=6)
    b, f, lb, lf = bench.algorithmic(c, st)
    kus = {k: 10.0 for k in ("route", "align", "shrink_gate_up", "gemm_gate_up", "shrink_down",
                             "gemm_down", "combine")}
    obj = bench.workload_summary("decode", c, st, 0.05, kus, b, f, lb, lf, [0.05] * 5)
    assert obj["layer_bound"] == "hbm" and obj["roofline"]["bound"] == "hbm"
    assert obj["roofline"]["unit"] == "GB/s" and obj["roofline"]["peak"] == 8000.0
    assert abs(obj["roofline"]["frac"] - obj["roofline"]["achieved"] / 8000.0) < 1e-3
    assert obj["value"] == round(4 / 0.05e-3, 1)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_shrink_work_is_counted_in_the_launch_that_ran_it():
    c = small_case()
    st = dict(n_experts=3, n_segments=4, P=8, P_lora=6)
    b, f, lb, lf = bench.algorithmic(c, st)
    names = ("route", "align", "shrink_gate_up", "gemm_gate_up", "shrink_down", "gemm_down", "combine")
    # shrinks with launches of their own: per-kernel figures unchanged
    kus = {k: 10.0 for k in names}
    assert not bench.shrinks_fused(kus)
    assert bench.fold_fused(kus, b, f) == (b, f)
    # shrinks inside the projections (the library reports exactly 0 for them):
    # their bytes and flops move into the projection launches, totals kept
    kus_f = dict(kus, shrink_gate_up=0.0, shrink_down=0.0)
    assert bench.shrinks_fused(kus_f)
    b2, f2 = bench.fold_fused(kus_f, b, f)
    assert b2["gemm_gate_up"] == b["gemm_gate_up"] + b["shrink_gate_up"]
    assert b2["gemm_down"] == b["gemm_down"] + b["shrink_down"]
    assert f2["gemm_down"] == f["gemm_down"] + f["shrink_down"]
    assert b2["shrink_gate_up"] == 0 and b2["shrink_down"] == 0
    assert sum(b2.values()) == sum(b.values())
    summ = bench.lora_kernels_summary(kus_f, b2)
    assert summ["shrinks"] == "inside the projection launches"
    assert summ["bytes"] == sum(b[n] for n in ("shrink_gate_up", "gemm_gate_up", "shrink_down", "gemm_down"))


def test_fold_fused_moves_the_combine_into_the_down_projection():
    c = small_case()
    st = dict(n_experts=3, n_segments=4, P=8, P_lora=6)
    b, f, lb, lf = bench.algorithmic(c, st)
    names = ("route", "align", "shrink_gate_up", "gemm_gate_up", "shrink_down", "gemm_down", "combine")
    kus = {k: 10.0 for k in names}
    # every kernel launched: nothing moves
    b2, _ = bench.fold_fused(kus, b, f, c.T, c.H, 8)
    assert b2 == b
    # combine folded: the down launch writes out [T][H] fp32 instead of its
    # rows [P][H] and reads the P weights; the routing launch clears out
    kus["combine"] = 0.0
    b3, _ = bench.fold_fused(kus, b, f, c.T, c.H, 8)
    assert b3["combine"] == 0
    assert b3["gemm_down"] == b["gemm_down"] - 8 * c.H * 4 + c.T * c.H * 4 + 8 * 4
    assert b3["route"] == b["route"] + c.T * c.H * 4
    # shrinks folded as well
    kus["shrink_gate_up"] = kus["shrink_down"] = 0.0
    b4, f4 = bench.fold_fused(kus, b, f, c.T, c.H, 8)
    assert b4["shrink_gate_up"] == b4["shrink_down"] == 0
    assert b4["gemm_gate_up"] == b["gemm_gate_up"] + b["shrink_gate_up"]
    assert f4["gemm_down"] == f["gemm_down"] + f["shrink_down"]
