"""Parity of the HIP path (called through the C ABI) against the CPU oracle.

Integer work (routing ids, alignment) is compared bit for bit; the layer
output must satisfy max|gpu-ref|/max|ref| <= 1e-2 and
mean|gpu-ref|/mean|ref| <= 2e-3 (bf16 inputs, fp32 accumulation, h in bf16).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from lora_mixture_experts_amd import moe_lora as ml
from lora_mixture_experts_amd import workloads as wl

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 1e-2, 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return torch.device("cuda:0")


def metrics(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    return err.max() / np.abs(ref).max(), err.mean() / np.abs(ref).mean()


def build_case(name, dims=None, seed=None, touched_only=True):
    """Draw a case; with touched_only only the experts / LoRA blocks the routing
    uses get values (the rest hold bf16 NaN, so a stray read shows up)."""
    if dims is None:
        dims = wl.CONFIGS[name]
    logits, x, ad, _ = wl.routing_only(name, seed=seed, dims=dims)
    ids, _ = oracle.route(logits, dims["top_k"])
    experts = set(np.unique(ids).tolist())
    blocks = set()
    for t in range(dims["T"]):
        a = int(ad[t])
        if 0 <= a < dims["L"]:
            for e in ids[t]:
                blocks.add((a, int(e)))
    if not touched_only:
        experts, blocks = None, None
    return wl.make_case(name, seed=seed, dims=dims, experts=experts, lora_blocks=blocks)


def run_gpu(case, dev, bm_b=0, bm_l=0, shrink_launch=False, tuning=None, fused_combine=False,
            packed_weights=False):
    t = wl.device_tensors(case, dev)
    layer = ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r,
                     t["w_gate_up"], t["w_down"], t["a_gate_up"], t["b_gate_up"], t["a_down"],
                     t["b_down"], block_m_base=bm_b, block_m_lora=bm_l, shrink_launch=shrink_launch,
                     tuning=tuning, fused_combine=fused_combine, packed_weights=packed_weights)
    out = layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    return layer, t, out


def sample_tokens(case, n):
    if case.T <= n:
        return np.arange(case.T, dtype=np.int32)
    rng = np.random.default_rng(1234)
    pick = set(rng.choice(case.T, size=n - 2, replace=False).tolist()) | {0, case.T - 1}
    return np.array(sorted(pick), dtype=np.int32)


# ----------------------------------------------------------------------------- route / align

# boundary shapes: 64 experts x 8 picks, 7 experts, 65 experts, 9 picks
ROUTE_CASES = [("tiny", {}), ("decode", {}), ("prefill", {}), ("wide", {}), ("many", {}),
               ("odd", dict(T=37, H=64, I=64, E=70, top_k=7, L=3, r=8)),
               ("one", dict(T=1, H=64, I=64, E=1, top_k=1, L=0, r=8)),
               ("lane_max", dict(T=300, H=64, I=64, E=64, top_k=8, L=2, r=8)),
               ("lane_e7", dict(T=257, H=64, I=64, E=7, top_k=3, L=2, r=8)),
               ("wave_e65", dict(T=33, H=64, I=64, E=65, top_k=8, L=2, r=8)),
               ("wave_k9", dict(T=33, H=64, I=64, E=64, top_k=9, L=2, r=8))]


@pytest.mark.parametrize("name,dims", ROUTE_CASES)
def test_route_parity(dev, name, dims):
    log(f"route {name}")
    dims = dims or wl.CONFIGS[name]
    logits, _, _, _ = wl.routing_only(name, dims=dims)
    ref_ids, ref_w = oracle.route(logits, dims["top_k"])
    d = ml.make_desc(dims["T"], dims["H"], dims["I"], dims["E"], dims["top_k"], dims["L"], dims["r"])
    lg = torch.from_numpy(logits).to(dev)
    ids = torch.empty((dims["T"], dims["top_k"]), dtype=torch.int32, device=dev)
    w = torch.empty((dims["T"], dims["top_k"]), dtype=torch.float32, device=dev)
    ml.route(d, lg, ids, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=0, atol=2e-6)


def test_route_ties(dev):
    log("route ties")
    logits = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 3.0],
                       [0.5] * 6,
                       [-1.0, -2.0, -1.0, -2.0, -3.0, -1.0]], np.float32)
    logits = np.concatenate([logits, np.repeat(logits[:1], 70, axis=0)])
    # 6 experts (one logit per lane) and the same ties spread over 72 experts
    # (two logits on some lanes)
    wide = np.tile(logits, (1, 12))
    for lg in (logits, wide):
        for k in (1, 2, 4, 6):
            ref_ids, _ = oracle.route(lg, k)
            d = ml.make_desc(lg.shape[0], 64, 64, lg.shape[1], k, 0, 8)
            ids = torch.empty((lg.shape[0], k), dtype=torch.int32, device=dev)
            w = torch.empty((lg.shape[0], k), dtype=torch.float32, device=dev)
            ml.route(d, torch.from_numpy(np.ascontiguousarray(lg)).to(dev), ids, w)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)


def gpu_align(dev, ids, ad, dims, bm_b, bm_l, workspace=True):
    d = ml.make_desc(dims["T"], dims["H"], dims["I"], dims["E"], dims["top_k"], dims["L"], dims["r"],
                     bm_b, bm_l)
    C_b, C_l = ml.align_capacity(d)
    bb, bl = ml.block_sizes(d)
    z = lambda n: torch.full((n,), -7, dtype=torch.int32, device=dev)
    out = dict(sorted_b=z(C_b), blk_e_b=z(C_b // bb), n_b=z(1), sorted_l=z(C_l), blk_e_l=z(C_l // bl),
               blk_a_l=z(C_l // bl), n_l=z(1))
    ws = torch.full((ml.workspace_bytes(d),), 0xA5, dtype=torch.uint8, device=dev) if workspace else None
    ml.align(d, torch.from_numpy(ids).to(dev), torch.from_numpy(ad).to(dev), workspace=ws, **out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, (bb, bl)


ALIGN_CASES = [("tiny", {}, (16, 16)), ("decode", {}, (16, 16)), ("decode", {}, (64, 32)),
               ("prefill", {}, (128, 64)), ("prefill", {}, (16, 256)), ("wide", {}, (32, 16)),
               ("many", {}, (128, 16)), ("many", {}, (16, 64)),
               ("odd", dict(T=37, H=64, I=64, E=70, top_k=7, L=3, r=8), (16, 16)),
               ("noL", dict(T=300, H=64, I=64, E=5, top_k=2, L=0, r=8), (32, 16)),
               ("big", dict(T=20000, H=64, I=64, E=64, top_k=8, L=16, r=8), (256, 128)),
               # key counts near the limit: one histogram range, one wave scatters
               ("keys", dict(T=300, H=64, I=64, E=256, top_k=8, L=32, r=8), (16, 16)),
               ("maxkeys", dict(T=4000, H=64, I=64, E=607, top_k=8, L=15, r=8), (32, 16)),
               # beyond one workgroup's histogram rows: the multi-launch path
               ("keys256", dict(T=2000, H=64, I=64, E=256, top_k=8, L=128, r=8), (16, 16)),
               ("keys256b", dict(T=6400, H=64, I=64, E=256, top_k=8, L=128, r=8), (128, 64)),
               ("keystop", dict(T=4000, H=64, I=64, E=1024, top_k=8, L=35, r=8), (32, 16)),
               ("keysfew", dict(T=5, H=64, I=64, E=256, top_k=4, L=40, r=8), (16, 16)),
               ("keys9720", dict(T=3000, H=64, I=64, E=972, top_k=8, L=9, r=8), (64, 32))]


@pytest.mark.parametrize("name,dims,bm", ALIGN_CASES)
def test_align_parity(dev, name, dims, bm):
    log(f"align {name} {bm}")
    dims = dims or wl.CONFIGS[name]
    logits, _, ad, _ = wl.routing_only(name, dims=dims)
    ids, _ = oracle.route(logits, dims["top_k"])
    if name in ("odd", "big", "keys256b"):  # out-of-range adapter ids count as "none"
        ad = ad.copy()
        ad[::5] = dims["L"] + 3
        ad[1::7] = -9
    got, (bb, bl) = gpu_align(dev, ids, ad, dims, *bm)
    ref = oracle.align(ids, ad, dims["E"], dims["L"], bb, bl)
    for key in ("sorted_b", "blk_e_b", "sorted_l", "blk_e_l", "blk_a_l"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    assert int(got["n_b"][0]) == ref["n_b"] and int(got["n_l"][0]) == ref["n_l"]
    again, _ = gpu_align(dev, ids, ad, dims, *bm)
    for key in got:
        np.testing.assert_array_equal(again[key], got[key])
    # without a workspace: the same result where one workgroup suffices,
    # refused where the histograms need the workspace
    if dims["E"] * (dims["L"] + 1) <= 9712:
        nows, _ = gpu_align(dev, ids, ad, dims, *bm, workspace=False)
        for key in got:
            np.testing.assert_array_equal(nows[key], got[key])
    else:
        with pytest.raises(ml.MoeLoraError) as ei:
            gpu_align(dev, ids, ad, dims, *bm, workspace=False)
        assert ei.value.code == ml.EWORKSPACE


# ----------------------------------------------------------------------------- the layer

def check_layer(case, dev, bm=(0, 0), stages=False, stage_tokens=64, shrink_launch=False,
                tuning=None, expect_choice=None, fused_combine=False, packed_weights=False):
    """Run the layer through the C ABI and compare EVERY output element with
    the oracle (max and mean bars over all T x H values); the alignment the
    call used is compared bit for bit. With stages=True the intermediates of
    a sample of stage_tokens tokens (first and last included) are checked
    too."""
    ids, w = oracle.route(case.logits, case.top_k)
    layer, t, out = run_gpu(case, dev, *bm, shrink_launch=shrink_launch, tuning=tuning,
                            fused_combine=fused_combine, packed_weights=packed_weights)
    got = out.cpu().numpy()
    assert layer.status() == 0
    if tuning is not None:
        # the layer ran the table's choice (None: no entry, library defaults)
        assert layer.tuned == expect_choice
        if expect_choice is not None:
            assert ml.block_sizes(layer.desc) == (expect_choice.block_m_base, expect_choice.block_m_lora)
            assert bool(layer.desc.flags & ml.FLAG_SHRINK_LAUNCH) == expect_choice.shrink_launch
    ref = oracle.forward(case, ids, w)
    mx, mean = metrics(got, ref)
    log(f"  {case.name} bm={ml.block_sizes(layer.desc)} tuned={layer.tuned} fused_combine={fused_combine} "
        f"all {case.T} tokens: max {mx:.2e} mean {mean:.2e}")
    assert np.all(np.isfinite(got))
    assert mx <= MAX_TOL and mean <= MEAN_TOL, (mx, mean)
    # the alignment the forward pass used is the oracle's, bit for bit
    bb, bl = ml.block_sizes(layer.desc)
    ref_al = oracle.align(ids, case.adapter_ids, case.E, case.L, bb, bl)
    got_al = {k: v.cpu().numpy() for k, v in layer.alignment().items()}
    for key in ("sorted_b", "blk_e_b", "sorted_l", "blk_e_l", "blk_a_l"):
        np.testing.assert_array_equal(got_al[key], ref_al[key], err_msg=key)
    assert int(got_al["n_b"][0]) == ref_al["n_b"] and int(got_al["n_l"][0]) == ref_al["n_l"]
    if stages:
        toks = sample_tokens(case, stage_tokens)
        _, st = oracle.forward(case, ids, w, tokens=toks, stages=True)
        gs = {k: v.cpu() for k, v in layer.stages().items()}
        rows = (toks[:, None] * case.top_k + np.arange(case.top_k)[None, :]).reshape(-1)
        np.testing.assert_array_equal(gs["topk_ids"].numpy().reshape(case.T, case.top_k), ids)
        s1 = gs["s1"].numpy()[rows]
        s2 = gs["s2"].numpy()[rows]
        h = gs["h"].float().numpy()[rows]
        # the down rows are kept only when a separate launch does the combine
        assert ("dn" in gs) != fused_combine
        dn = gs["dn"].numpy()[rows] if "dn" in gs else None
        del gs
        if case.L > 0 and np.abs(st["s1"]).max() > 0:
            m1 = metrics(s1, st["s1"])
            assert m1[0] < 1e-4, ("s1", m1)
            m2 = metrics(s2, st["s2"])
            assert m2[0] < 2e-2 and m2[1] < 4e-3, ("s2", m2)
        mh = metrics(h, st["h"])
        assert mh[0] < 1e-2 and mh[1] < 4e-3, ("h", mh)
        if dn is not None:
            md = metrics(dn, st["d"])
            assert md[0] < MAX_TOL and md[1] < MEAN_TOL, ("d", md)
        # pairs without adapter have zero shrink rows
        noad = np.array([not (0 <= case.adapter_ids[r // case.top_k] < case.L) for r in rows])
        assert np.all(s1[noad] == 0) and np.all(s2[noad] == 0)
    return out


# Decode-sized batches are aligned inside the gate_up launch (every wave
# derives its rows from the routing launch's picks, or routes the batch from
# the logits itself where the top-k scan is short; the launch's first
# workgroup writes the alignment, and then the routing). The same call with
# the routing and alignment launches must give the same routing, alignment,
# intermediates and output, bit for bit.
LOCAL_CASES = [("tiny", {}, {}), ("decode", {}, {}), ("dense", {}, {}),
               ("decode", {}, dict(fused_combine=True)), ("decode", {}, dict(no_shrink_wait=True)),
               ("k8", dict(T=8, H=128, I=128, E=32, top_k=8, L=5, r=16), {}),
               ("noL", dict(T=16, H=128, I=192, E=20, top_k=4, L=0, r=8), {}),
               ("t1", dict(T=1, H=64, I=64, E=3, top_k=2, L=2, r=8), {}),
               ("t13", dict(T=13, H=64, I=128, E=32, top_k=3, L=40, r=32), {}),
               ("ties", dict(T=16, H=64, I=64, E=24, top_k=4, L=3, r=8), dict(ties=True)),
               ("dense", {}, dict(frags_gate_up=8)),
               ("t13", dict(T=13, H=64, I=128, E=32, top_k=3, L=40, r=32), dict(frags_gate_up=8))]


@pytest.mark.parametrize("name,dims,opts", LOCAL_CASES)
def test_routing_inside_gate_up_matches_routing_launches(dev, name, dims, opts):
    log(f"local routing {name} {opts}")
    opts = dict(opts)
    ties = opts.pop("ties", False)
    case = wl.make_case(name, dims=dims) if dims else wl.make_case(name)
    if ties:  # coarse logits: many equal values, the lower expert id must win
        case.logits[:] = np.round(case.logits * 2) / 2
    t = wl.device_tensors(case, dev)
    layers = [ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, t["w_gate_up"], t["w_down"],
                       t["a_gate_up"], t["b_gate_up"], t["a_down"], t["b_down"], route_launch=rl, **opts)
              for rl in (False, True)]
    modes = [ml.plan(l.desc)["routing_in_gate_up"] for l in layers]
    assert modes[0] in (1, 2) and modes[1] == 0
    assert (modes[0] == 2) == (case.E * case.top_k <= 32)
    outs = [l(t["x"], t["logits"], t["adapter_ids"]).cpu().numpy() for l in layers]
    torch.cuda.synchronize()
    assert all(l.status() == 0 for l in layers) or opts.get("no_shrink_wait")
    if not opts.get("fused_combine"):  # fp32 atomics: the order of adds varies
        np.testing.assert_array_equal(outs[0], outs[1])
    st = [{k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy() for k, v in l.stages().items()}
          for l in layers]
    for key in st[1]:
        np.testing.assert_array_equal(st[0][key].view(np.uint8), st[1][key].view(np.uint8), err_msg=key)
    al = [{k: v.cpu().numpy() for k, v in l.alignment().items()} for l in layers]
    for key in al[1]:
        np.testing.assert_array_equal(al[0][key], al[1][key], err_msg=key)
    # and the oracle's routing
    ids, _ = oracle.route(case.logits, case.top_k)
    np.testing.assert_array_equal(st[0]["topk_ids"].reshape(case.T, case.top_k), ids)
    ref = oracle.forward(case, ids, oracle.route(case.logits, case.top_k)[1])
    mx, mean = metrics(outs[0], ref)
    assert mx <= MAX_TOL and mean <= MEAN_TOL, (mx, mean)


def _table():
    from lora_mixture_experts_amd import tuning
    return tuning.load(tuning.DEFAULT_FOLDER)


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_layer_parity_as_benched(dev, name):
    # each workload with the launch choice bench.py times: the committed
    # tuning table's entry at this shape and token count where there is one,
    # else the library defaults; every token is compared
    from lora_mixture_experts_amd import tuning
    log(f"layer {name} (as benched)")
    table = _table()
    case = build_case(name)
    choice = table.lookup(case.T, *(getattr(case, q) for q in tuning.SHAPE_KEYS))
    check_layer(case, dev, stages=True, tuning=table, expect_choice=choice)


@pytest.mark.parametrize("name", ["decode", "wide", "dense"])
def test_layer_parity_library_default(dev, name):
    # the library's own defaults at the shapes where the committed table
    # chooses differently (every token compared)
    log(f"layer {name} (library defaults)")
    check_layer(build_case(name), dev, stages=True)


@pytest.mark.parametrize("name", ["tiny", "decode", "wide", "many", "dense"])
def test_layer_parity_fused_combine(dev, name):
    # the weighted combine inside the down projection (fp32 atomic adds into
    # out), with the launch choices as benched; agrees with the fixed-order
    # combine to fp32 rounding
    log(f"layer {name} (fused combine)")
    case = build_case(name)
    choice = _table().lookup(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r)
    out = check_layer(case, dev, stages=True, tuning=_table(), fused_combine=True, expect_choice=choice)
    layer, t, ref = run_gpu(case, dev, tuning=_table())
    out2 = layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert torch.equal(ref, out2)  # the fixed-order combine is bitwise repeatable
    mx, mean = metrics(out.cpu().numpy(), ref.cpu().numpy())
    assert mx < 1e-5 and mean < 1e-6, (mx, mean)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("bm", [(16, 16), (32, 16), (64, 64), (128, 32), (256, 256)])
def test_layer_block_sizes(dev, bm, fused):
    log(f"layer block sizes {bm} fused_combine={fused}")
    dims = dict(T=150, H=192, I=320, E=6, top_k=3, L=3, r=16)
    case = build_case("blocks", dims=dims, seed=5)
    check_layer(case, dev, bm=bm, stages=True, fused_combine=fused)


# the split-K launch fields: each value computes the same layer
SPLIT_CASES = [
    # 16-row blocks: waves per tile of each projection, with and without a
    # down K split, and with the shrinks inside the projections (decode)
    ("decode", None, (16, 16), dict(waves_gate_up=2, waves_down=2)),
    ("decode", None, (16, 16), dict(waves_gate_up=4, waves_down=2, down_ksplit=3)),
    ("decode", None, (16, 16), dict(down_ksplit=5)),
    # 8 weight fragments per gate_up wave (64 h columns per tile)
    ("decode", None, (16, 16), dict(frags_gate_up=8)),
    ("dense", None, (16, 16), dict(frags_gate_up=8)),
    # 32- and 64-row blocks: down K ranges and separate shrinks split over K
    ("wide", None, (32, 16), dict(down_ksplit=4, shrink_ksplit=2)),
    ("kdown", dict(T=40, H=256, I=1024, E=3, top_k=2, L=2, r=16), (64, 16), dict(down_ksplit=16, shrink_ksplit=3)),
    # 128-row blocks: a split shrink moves the expand out of the pipeline
    ("kdma", dict(T=300, H=256, I=512, E=2, top_k=1, L=3, r=32), (128, 16), dict(shrink_ksplit=4)),
]


@pytest.mark.parametrize("name,dims,bm,launch", SPLIT_CASES)
def test_split_fields_keep_parity(dev, name, dims, bm, launch):
    log(f"split fields {name} {bm} {launch}")
    case = build_case(name, dims=dims, seed=None if dims is None else 70 + len(name))
    ids, w = oracle.route(case.logits, case.top_k)
    ref = oracle.forward(case, ids, w)
    t = wl.device_tensors(case, dev)
    layer = ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, t["w_gate_up"], t["w_down"],
                     t["a_gate_up"], t["b_gate_up"], t["a_down"], t["b_down"], block_m_base=bm[0],
                     block_m_lora=bm[1], **launch)
    plan = ml.plan(layer.desc)
    for k, v in launch.items():
        assert plan[k] == v, (k, plan)
    out = layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert layer.status() == 0
    mx, mean = metrics(out.cpu().numpy(), ref)
    log(f"  max {mx:.2e} mean {mean:.2e}")
    assert mx <= MAX_TOL and mean <= MEAN_TOL, (mx, mean)
    out2 = layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("bm", [(16, 16), (32, 16)])
def test_fused_combine_with_down_k_split(dev, bm):
    # a long down K (I = 6144) on a small grid: the down projection is cut
    # into K ranges, and every range adds its weighted partial into out
    log(f"fused combine with K split {bm}")
    dims = dict(T=8, H=128, I=6144, E=2, top_k=2, L=2, r=16)
    case = build_case("ksplit", dims=dims, seed=31)
    a = check_layer(case, dev, bm=bm, stages=True, fused_combine=True)
    b = check_layer(case, dev, bm=bm, stages=True)
    mx, mean = metrics(a.cpu().numpy(), b.cpu().numpy())
    assert mx < 1e-5 and mean < 1e-6, (mx, mean)


@pytest.mark.parametrize("r,L,bm,pure", [(8, 3, 128, False), (64, 3, 128, True), (128, 2, 256, False),
                                          (32, 4, 128, False), (128, 4, 128, True),
                                          (32, 6, 128, False), (16, 7, 256, True),
                                          (64, 24, 128, True), (8, 40, 256, False), (32, 20, 64, True),
                                          (16, 33, 32, False)])
def test_pipeline_expand(dev, r, L, bm, pure):
    # 128- and 256-row blocks run the LoRA expand as extra stages of their
    # LDS pipeline, one group of stages per adapter run of the tile (L up to
    # 7 runs here; the epilogue expand is left to split shrinks, see the
    # split-field cases); pure: base weights zero, so the output is the LoRA
    # path alone
    log(f"pipeline expand r={r} L={L} bm={bm} pure={pure}")
    dims = dict(T=300, H=128, I=192, E=2, top_k=1, L=L, r=r)
    case = build_case(f"pipe{r}_{L}", dims=dims, seed=60 + r + L)
    if pure:
        case.w_gate_up[:] = 0
        case.w_down[:] = 0
    check_layer(case, dev, bm=(bm, 16), stages=True)


# 16-row base blocks run the two shrinks as producer waves inside the
# projection launches; the projection waves wait for them before the expand.
# Each case also runs with the shrinks in launches of their own.
FUSED_CASES = [
    ("decode", None, (0, 0), True),
    # gate_up K = 8256: three producer K ranges; down K = 128 (two 64-wide
    # chunks) is then cut into three ranges too, one of them empty
    ("fusedK3", dict(T=12, H=8256, I=128, E=2, top_k=1, L=3, r=16), (16, 16), False),
    ("fusedK2", dict(T=20, H=4160, I=256, E=3, top_k=2, L=2, r=32), (16, 16), True),
    # 64-row LoRA blocks: each producer loops over four row fragments
    ("fusedBL", dict(T=120, H=128, I=192, E=2, top_k=1, L=1, r=32), (16, 64), True),
    # rank 8: the producer's upper 8 columns re-read rows and are never stored
    ("fusedR8", dict(T=20, H=64, I=128, E=4, top_k=2, L=3, r=8), (16, 16), False),
    # rank 128: eight column fragments per LoRA block
    ("fusedR128", dict(T=16, H=128, I=128, E=8, top_k=2, L=2, r=128), (16, 16), False),
]


@pytest.mark.parametrize("name,dims,bm,pure", FUSED_CASES)
def test_shrinks_inside_projections(dev, name, dims, bm, pure):
    log(f"shrinks inside projections {name} bm={bm} pure={pure}")
    case = build_case(name, dims=dims, seed=None if dims is None else 90 + len(name))
    if pure:
        case.w_gate_up[:] = 0
        case.w_down[:] = 0
    out_f = check_layer(case, dev, bm=bm, stages=True)
    out_s = check_layer(case, dev, bm=bm, stages=True, shrink_launch=True)
    # the two agree far inside the oracle bars: they differ only in the
    # shrinks' fp32 summation order, which can move an h value across a bf16
    # rounding boundary (one bf16 step is 2^-8 of that value)
    mx, mean = metrics(out_f.cpu().numpy(), out_s.cpu().numpy())
    assert mx < MAX_TOL / 10 and mean < MEAN_TOL / 10, (mx, mean)
    # and the fused form is repeatable bit for bit
    layer, t, out1 = run_gpu(case, dev, *bm)
    out2 = layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert layer.status() == 0


@pytest.mark.parametrize("name,dims,bm,pure", FUSED_CASES)
def test_projection_waves_compute_their_own_shrink(dev, name, dims, bm, pure):
    # the path a projection wave takes when its bounded wait for the shrink
    # waves of its launch runs out, forced for every wave from the host: each
    # computes the shrink of its own rows, the output still matches the
    # oracle, and the status word reports the slow path
    log(f"own shrink {name} bm={bm} pure={pure}")
    case = build_case(name, dims=dims, seed=None if dims is None else 90 + len(name))
    if pure:
        case.w_gate_up[:] = 0
        case.w_down[:] = 0
    ids, w = oracle.route(case.logits, case.top_k)
    ref = oracle.forward(case, ids, w)
    t = wl.device_tensors(case, dev)
    mk = lambda **kw: ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, t["w_gate_up"],
                               t["w_down"], t["a_gate_up"], t["b_gate_up"], t["a_down"], t["b_down"],
                               block_m_base=bm[0], block_m_lora=bm[1], **kw)
    own = mk(no_shrink_wait=True)
    assert ml.plan(own.desc)["shrinks_in_projections"] == 1
    out = own(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert own.status() == ml.STATUS_SHRINK_FALLBACK
    mx, mean = metrics(out.cpu().numpy(), ref)
    log(f"  max {mx:.2e} mean {mean:.2e}")
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert mx <= MAX_TOL and mean <= MEAN_TOL, (mx, mean)
    # and agrees with the producers' path far inside the oracle bars
    normal = mk()
    out_n = normal(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert normal.status() == 0
    mx, mean = metrics(out.cpu().numpy(), out_n.cpu().numpy())
    assert mx < MAX_TOL / 10 and mean < MEAN_TOL / 10, (mx, mean)


def test_status_word_is_cleared_by_each_call(dev):
    # the status word lives in the workspace and each forward call clears it
    log("status word")
    case = build_case("decode")
    layer, t, _ = run_gpu(case, dev)
    assert layer.status() == 0
    # a call that sets it (every projection wave computes its own shrink),
    # then a normal call on the same workspace clears it again
    own = ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, t["w_gate_up"], t["w_down"],
                   t["a_gate_up"], t["b_gate_up"], t["a_down"], t["b_down"], no_shrink_wait=True)
    own.workspace = layer.workspace
    own(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert layer.status() == ml.STATUS_SHRINK_FALLBACK
    layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert layer.status() == 0
    # poison the whole workspace, including the status word; a forward call
    # writes every workspace entry before it reads it (the alignment fills
    # each view to its capacity, the routing launch clears the counters)
    layer.workspace.view(torch.int32).fill_(-1)
    layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert layer.status() == 0


def _shrink_launch_times(case, dev, bm):
    layer, t, _ = run_gpu(case, dev, *bm)
    ml.timing_enable(2)
    layer(t["x"], t["logits"], t["adapter_ids"])
    layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    ms, n = ml.timing_read()
    ml.timing_enable(0)
    names = ml.kernel_names()
    assert n == 2
    return ms[names.index("shrink_gate_up")], ms[names.index("shrink_down")]


def test_shrink_placement_rule(dev):
    # the shrinks run inside the projection launches (their timing slots read
    # exactly 0) for 16-row base blocks with at most 1024 producer waves, and
    # in launches of their own otherwise
    log("shrink placement")
    dec = build_case("decode")
    assert _shrink_launch_times(dec, dev, (0, 0)) == (0.0, 0.0)
    # 16-row base blocks on a larger batch: LoRA-view capacity
    # (2048 + 256 * 15) / 16 = 368 blocks x 4 column fragments (r = 64)
    # = 1472 > 1024 producer waves
    dims = dict(T=512, H=128, I=128, E=32, top_k=4, L=8, r=64)
    big = build_case("placement", dims=dims, seed=21)
    g, d = _shrink_launch_times(big, dev, (16, 16))
    assert g > 0.0 and d > 0.0
    # 64-row base blocks: always separate launches
    g, d = _shrink_launch_times(build_case("many"), dev, (0, 0))
    assert g > 0.0 and d > 0.0


RANDOM_DIMS = [dict(T=1, H=64, I=64, E=1, top_k=1, L=1, r=8),
               dict(T=3, H=128, I=64, E=4, top_k=4, L=2, r=16),
               dict(T=33, H=64, I=192, E=9, top_k=2, L=4, r=64),
               dict(T=70, H=256, I=128, E=3, top_k=2, L=1, r=128),
               dict(T=19, H=320, I=448, E=16, top_k=5, L=0, r=8),
               dict(T=257, H=128, I=128, E=40, top_k=8, L=5, r=32)]


@pytest.mark.parametrize("i", range(len(RANDOM_DIMS)))
def test_layer_shapes(dev, i):
    dims = RANDOM_DIMS[i]
    log(f"layer shape {dims}")
    case = build_case(f"shape{i}", dims=dims, seed=40 + i)
    check_layer(case, dev, stages=True)


# packed copies of the base weights: read by the 16-row kernels (decode-sized
# batches), with every launch option they take; ignored at larger blocks
# (32/64-row tiled with a down K split, 128/256-row direct loads)
PACKED_CASES = [("decode", None, {}, False), ("dense", None, {}, False), ("tiny", None, {}, False),
                ("odd", dict(T=5, H=320, I=448, E=3, top_k=2, L=2, r=16), {}, False),
                ("decode", None, dict(down_ksplit=3, waves_gate_up=2, waves_down=2), False),
                ("decode", None, {}, True),
                ("decode", None, dict(frags_gate_up=8), False),
                ("dense", None, dict(frags_gate_up=8), False),
                ("odd", dict(T=5, H=320, I=448, E=3, top_k=2, L=2, r=16), dict(frags_gate_up=8), False),
                ("wide", None, {}, False),
                ("wide", None, dict(block_m_base=32, down_ksplit=4), False),
                ("tiles", dict(T=300, H=320, I=448, E=4, top_k=2, L=3, r=32), dict(block_m_base=128), False),
                ("tiles", dict(T=300, H=320, I=448, E=4, top_k=2, L=3, r=32), dict(block_m_base=256), False),
                ("tiles", dict(T=300, H=320, I=448, E=4, top_k=2, L=3, r=32), dict(block_m_base=64), False)]


@pytest.mark.parametrize("name,dims,launch,shrink_launch", PACKED_CASES)
def test_packed_weights_give_bitwise_equal_output(dev, name, dims, launch, shrink_launch):
    log(f"packed weights {name} {dims or ''} {launch} shrink_launch={shrink_launch}")
    case = build_case(name, dims=dims, touched_only=False)
    t = wl.device_tensors(case, dev)
    launch = dict(launch)
    bm = launch.pop("block_m_base", 0)
    layer = ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, t["w_gate_up"], t["w_down"],
                     t["a_gate_up"], t["b_gate_up"], t["a_down"], t["b_down"], shrink_launch=shrink_launch,
                     block_m_base=bm, **launch)
    ref = layer(t["x"], t["logits"], t["adapter_ids"])
    # the same call with packed copies in the weights struct
    gp, dp = torch.empty_like(t["w_gate_up"]), torch.empty_like(t["w_down"])
    ml.pack_weights(layer.desc, t["w_gate_up"], t["w_down"], gp, dp)
    w = layer.weights
    both = ml.Weights(w.w_gate_up, w.w_down, w.a_gate_up, w.b_gate_up, w.a_down, w.b_down, gp.data_ptr(),
                      dp.data_ptr())
    out = torch.empty_like(ref)
    ml.forward(layer.desc, both, t["x"], t["logits"], t["adapter_ids"], out, layer.workspace)
    torch.cuda.synchronize()
    assert torch.equal(ref, out)


def test_layer_parity_packed_weights(dev):
    log("layer packed weights vs oracle")
    check_layer(build_case("decode"), dev, packed_weights=True)


# A seeded sweep: random small shapes crossed with random launch options
# (block sizes of both views, split fields, shrink placement, combine in the
# down projection, bf16 output, packed weight copies), each against the oracle
# on every output. Options the library rejects for a shape are dropped, in
# that order, until the descriptor is valid.
SWEEP_CASES = 40


def _sweep_setup(i):
    rng = np.random.default_rng(5000 + i)
    E = int(rng.integers(1, 17))
    dims = dict(T=int(rng.choice([1, 3, 16, 37, 130, 300])), H=64 * int(rng.integers(1, 13)),
                I=64 * int(rng.integers(1, 13)), E=E, top_k=int(rng.integers(1, min(E, 8) + 1)),
                L=int(rng.integers(0, 6)), r=int(rng.choice([8, 16, 32, 64])))
    while dims["T"] > 1 and dims["T"] * dims["top_k"] * dims["H"] * dims["I"] > 2e8:
        dims["T"] //= 2  # keeps the oracle within a few seconds
    # every block height of both views in turn, the rest drawn
    opts = dict(block_m_base=[0, 16, 32, 64, 128, 256][i % 6],
                block_m_lora=[0, 16, 32, 64][(i // 6) % 4],
                shrink_launch=bool(rng.integers(0, 2)), fused_combine=bool(rng.random() < 0.3),
                out_bf16=bool(rng.random() < 0.2), packed_weights=bool(rng.integers(0, 2)))
    launch = dict(down_ksplit=int(rng.choice([0, 0, 2, 3, 5])), shrink_ksplit=int(rng.choice([0, 0, 2, 4])),
                  waves_gate_up=int(rng.choice([0, 0, 2, 4])), waves_down=int(rng.choice([0, 0, 2, 4])),
                  frags_gate_up=int(rng.choice([0, 0, 8])))

    def valid(o, ln):
        flags = ((ml.FLAG_OUT_BF16 if o["out_bf16"] else 0) | (ml.FLAG_SHRINK_LAUNCH if o["shrink_launch"] else 0) |
                 (ml.FLAG_FUSED_COMBINE if o["fused_combine"] else 0))
        d = ml.make_desc(dims["T"], dims["H"], dims["I"], dims["E"], dims["top_k"], dims["L"], dims["r"],
                         o["block_m_base"], o["block_m_lora"], flags, **ln)
        return ml.validate(d) == ml.OK

    for drop in ("frags_gate_up", "waves_down", "waves_gate_up", "shrink_ksplit", "down_ksplit"):
        if valid(opts, launch):
            break
        launch[drop] = 0
    if not valid(opts, launch):
        opts["out_bf16"] = False
    assert valid(opts, launch), (dims, opts, launch)
    return dims, opts, launch


@pytest.mark.parametrize("i", range(SWEEP_CASES))
def test_layer_random_sweep(dev, i):
    dims, opts, launch = _sweep_setup(i)
    log(f"sweep {i}: {dims} {opts} {launch}")
    case = build_case(f"sweep{i}", dims=dims, seed=6000 + i)
    t = wl.device_tensors(case, dev)
    layer = ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, t["w_gate_up"], t["w_down"],
                     t["a_gate_up"], t["b_gate_up"], t["a_down"], t["b_down"], **opts, **launch)
    out = layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert layer.status() in (0, ml.STATUS_SHRINK_FALLBACK)
    got = out.float().cpu().numpy()
    ids, w = oracle.route(case.logits, case.top_k)
    ref = oracle.forward(case, ids, w)
    mx, mean = metrics(got, ref)
    # bf16 output adds its own rounding (at most 2^-8 relative per element)
    mean_tol = MEAN_TOL + (2e-3 if opts["out_bf16"] else 0.0)
    assert np.all(np.isfinite(got))
    assert mx <= MAX_TOL and mean <= mean_tol, (mx, mean)


def test_layer_many_experts_and_adapters(dev):
    # 256 experts x 40 adapters (10496 keys): the alignment runs on the
    # multi-launch path inside the forward pass
    log("layer 256 experts x 40 adapters")
    dims = dict(T=300, H=64, I=128, E=256, top_k=8, L=40, r=8)
    case = build_case("keyslayer", dims=dims, seed=81)
    check_layer(case, dev, stages=True)


def test_layer_api_maxima(dev):
    # E = 1024 (16 logits per lane in the router), top_k = 32 (the largest
    # choice count), rank 128
    log("layer maxima")
    dims = dict(T=24, H=64, I=128, E=1024, top_k=32, L=2, r=128)
    case = build_case("maxima", dims=dims, seed=77)
    check_layer(case, dev, stages=True)


def test_layer_foreign_adapter_ids(dev):
    # ids outside [0, L) mean "no adapter" in the whole layer, not only in
    # the alignment
    log("layer foreign adapter ids")
    case = build_case("decode", touched_only=False)
    case.adapter_ids[::3] = case.L + 5
    case.adapter_ids[1::4] = -7
    check_layer(case, dev, stages=True)


def test_no_adapter_and_zero_b_agree(dev):
    log("layer no-adapter variants")
    case = build_case("decode", touched_only=False)
    case.adapter_ids[:] = -1
    _, _, out_none = run_gpu(case, dev)
    check_layer(case, dev)
    case2 = build_case("decode", touched_only=False)
    case2.b_gate_up[:] = 0
    case2.b_down[:] = 0
    _, _, out_zero_b = run_gpu(case2, dev)
    # B = 0 adds exact zeros, so the result is bitwise the base-only one
    assert torch.equal(out_none, out_zero_b)


def test_pure_lora(dev):
    """Base weights zero: the output is the LoRA path alone."""
    log("layer pure LoRA")
    case = build_case("decode")
    case.w_gate_up[:] = 0
    case.w_down[:] = 0
    check_layer(case, dev, stages=True)


def test_single_expert(dev):
    log("layer single expert")
    dims = dict(T=40, H=256, I=512, E=1, top_k=1, L=2, r=32)
    case = build_case("single", dims=dims, seed=9)
    check_layer(case, dev, stages=True)


def test_repeat_calls_reuse_workspace(dev):
    log("layer repeat")
    case = build_case("tiny")
    layer, t, out1 = run_gpu(case, dev)
    out2 = layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    # same inputs, same block plan: bitwise identical (no atomics in the path)
    assert torch.equal(out1, out2)
    # the combine inside the down projection (weighted rows added atomically
    # into out) agrees to fp32 rounding, on repeated calls too
    layer_f, t_f, out_f1 = run_gpu(case, dev, fused_combine=True)
    out_f2 = layer_f(t_f["x"], t_f["logits"], t_f["adapter_ids"])
    torch.cuda.synchronize()
    for o in (out_f1, out_f2):
        mx, mean = metrics(o.cpu().numpy(), out1.cpu().numpy())
        assert mx < 1e-5 and mean < 1e-6, (mx, mean)


def test_bf16_output_is_rounded_fp32_output(dev):
    log("bf16 output")
    case = build_case("decode")
    layer, t, out32 = run_gpu(case, dev)
    lb = ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, t["w_gate_up"], t["w_down"],
                  t["a_gate_up"], t["b_gate_up"], t["a_down"], t["b_down"], out_bf16=True)
    outb = lb(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    assert outb.dtype == torch.bfloat16
    # the combine sums in fp32 in a fixed order, so the bf16 form is exactly the
    # round-to-nearest-even of the fp32 output
    np.testing.assert_array_equal(outb.view(torch.int16).cpu().numpy(),
                                  out32.to(torch.bfloat16).view(torch.int16).cpu().numpy())


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replay_matches_eager(dev, fused):
    # the whole layer captured into one HIP graph (no host sync, no allocation,
    # no memset inside the call) replays to the eager result, also after the
    # inputs change in place, with eager calls on the same workspace between
    # replays; bit for bit with the fixed-order combine, to fp32 rounding with
    # the combine in the down projection (which also shows that every replay
    # clears out first)
    log(f"graph replay fused_combine={fused}")
    case = build_case("decode")
    layer, t, out_eager = run_gpu(case, dev, fused_combine=fused)
    ref = out_eager.clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(t["x"], t["logits"], t["adapter_ids"], out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(t["x"], t["logits"], t["adapter_ids"], out=out)
    x0 = t["x"].clone()
    x1 = torch.flip(x0, dims=[0]).contiguous()  # the tokens in reverse order

    def same(a, b):
        if not fused:
            return torch.equal(a, b)
        mx, mean = metrics(a.cpu().numpy(), b.cpu().numpy())
        return mx < 1e-5 and mean < 1e-6

    for i in range(4):
        xi = x0 if i % 2 == 0 else x1
        t["x"].copy_(xi)
        want = layer(t["x"], t["logits"], t["adapter_ids"]).clone()  # eager, same workspace
        out.fill_(12345.0)
        g.replay()
        torch.cuda.synchronize()
        assert same(out, want), i
        if i % 2 == 0:
            assert same(out, ref)
    t["x"].copy_(x0)


def test_zero_tokens_is_noop(dev):
    d = ml.make_desc(0, 64, 64, 2, 1, 0, 8)
    w = torch.zeros(2 * 2 * 64 * 64, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(ml.workspace_bytes(d), 256), dtype=torch.uint8, device=dev)
    out = torch.empty(1, dtype=torch.float32, device=dev)
    x = torch.empty(8, dtype=torch.bfloat16, device=dev)
    lg = torch.empty(2, dtype=torch.float32, device=dev)
    ad = torch.empty(1, dtype=torch.int32, device=dev)
    ml.forward(d, ml.weights_struct(w, w), x, lg, ad, out, ws)
    torch.cuda.synchronize()


def test_zero_tokens_with_adapters_is_noop(dev):
    # T = 0 with a LoRA pool: nothing is launched and the output is untouched
    log("zero tokens with adapters")
    d = ml.make_desc(0, 64, 64, 4, 2, 3, 16)
    w = torch.zeros(4 * 3 * 64 * 64, dtype=torch.bfloat16, device=dev)
    lora = torch.zeros(3 * 4 * 16 * 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(ml.workspace_bytes(d), 256), dtype=torch.uint8, device=dev)
    out = torch.full((4,), 7.0, dtype=torch.float32, device=dev)
    x = torch.empty(8, dtype=torch.bfloat16, device=dev)
    lg = torch.empty(4, dtype=torch.float32, device=dev)
    ad = torch.empty(1, dtype=torch.int32, device=dev)
    ml.forward(d, ml.weights_struct(w, w, lora, lora, lora, lora), x, lg, ad, out, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_tuning_table_choice_is_used_and_keeps_parity(dev, tmp_path):
    # a table entry for the tiny shape that differs from every default: the
    # layer takes its block sizes and shrink placement, and still matches the
    # oracle
    from lora_mixture_experts_amd import tuning
    log("tuning table")
    case = build_case("tiny")
    shape = {k: getattr(case, k) for k in tuning.SHAPE_KEYS}
    tuning.save_entry(str(tmp_path), shape, {"T_max": case.T, "block_m_base": 32, "block_m_lora": 64,
                                             "shrink_launch": True, "down_ksplit": 2, "shrink_ksplit": 2})
    table = tuning.load(str(tmp_path))
    t = wl.device_tensors(case, dev)
    layer = ml.Layer(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r, t["w_gate_up"], t["w_down"],
                     t["a_gate_up"], t["b_gate_up"], t["a_down"], t["b_down"], tuning=table)
    assert layer.tuned == tuning.Choice(32, 64, True, down_ksplit=2, shrink_ksplit=2)
    assert ml.block_sizes(layer.desc) == (32, 64)
    assert layer.desc.flags & ml.FLAG_SHRINK_LAUNCH
    p = ml.plan(layer.desc)
    assert p["down_ksplit"] == 2 and p["shrink_ksplit"] == 2
    out = layer(t["x"], t["logits"], t["adapter_ids"])
    torch.cuda.synchronize()
    ids, w = oracle.route(case.logits, case.top_k)
    ref = oracle.forward(case, ids, w)
    mx, mean = metrics(out.cpu().numpy(), ref)
    assert mx <= MAX_TOL and mean <= MEAN_TOL, (mx, mean)
    assert layer.status() == 0


def test_tuner_writes_a_loadable_table(dev, tmp_path):
    # the tuner end to end on the tiny shape: every candidate runs, the file
    # it writes loads, and the stored choice is the fastest it measured
    from lora_mixture_experts_amd import tune, tuning
    log("tuner")
    entry = tune.tune_workload("tiny", str(tmp_path), steps=5)
    table = tuning.load(str(tmp_path))
    c = wl.CONFIGS["tiny"]
    got = table.lookup(c["T"], c["H"], c["I"], c["E"], c["top_k"], c["L"], c["r"])
    assert got == tuning.choice_of(entry)
    assert entry["us"] <= entry["us_library_default"]


def test_forward_rejects_small_workspace(dev):
    case = build_case("tiny")
    t = wl.device_tensors(case, dev)
    d = ml.make_desc(case.T, case.H, case.I, case.E, case.top_k, case.L, case.r)
    ws = torch.empty(ml.workspace_bytes(d) - 256, dtype=torch.uint8, device=dev)
    out = torch.empty((case.T, case.H), dtype=torch.float32, device=dev)
    wts = ml.weights_struct(t["w_gate_up"], t["w_down"], t["a_gate_up"], t["b_gate_up"], t["a_down"],
                            t["b_down"])
    with pytest.raises(ml.MoeLoraError) as ei:
        ml.forward(d, wts, t["x"], t["logits"], t["adapter_ids"], out, ws)
    assert ei.value.code == ml.EWORKSPACE
