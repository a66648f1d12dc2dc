"""Host-side checks of the C ABI: the library loads, exports every entry point
the header declares, and rejects bad arguments without touching a device."""
import ctypes
import os
import re

import pytest

from lora_mixture_experts_amd import moe_lora as ml
from lora_mixture_experts_amd import workloads as wl
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_lora.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_lora_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert "moe_lora_forward" in names and "moe_lora_align" in names and "moe_lora_route" in names
    assert set(names) == set(ml.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ml.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def desc(**over):
    d = dict(wl.CONFIGS["decode"])
    d.update(over)
    return ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"],
                        d.get("bm_b", 0), d.get("bm_l", 0), d.get("flags", 0))


@pytest.mark.parametrize("over", [dict(H=2881), dict(I=100), dict(top_k=0), dict(top_k=33, E=40),
                                  dict(top_k=5, E=4), dict(r=24), dict(E=0), dict(T=-1), dict(L=-1),
                                  dict(bm_b=48), dict(bm_b=8), dict(bm_l=512), dict(E=1025),
                                  dict(E=128, L=300), dict(E=1024, L=36, top_k=8), dict(flags=32), dict(flags=5),
                                  dict(flags=-1), dict(flags=31)])
def test_validate_rejects(over):
    assert ml.validate(desc(**over)) == ml.EINVAL


def test_validate_accepts_configs_and_checks_workspace():
    for name, d in wl.CONFIGS.items():
        ds = ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"])
        assert ml.validate(ds) == ml.OK, name
        n = ml.workspace_bytes(ds)
        assert n > 0 and n % 256 == 0
        assert ml.validate(ds, None, n) == ml.OK
        assert ml.validate(ds, None, n - 1) == ml.EWORKSPACE


def test_validate_accepts_output_and_shrink_flags():
    assert ml.validate(desc(flags=ml.FLAG_OUT_BF16)) == ml.OK
    assert ml.validate(desc(flags=ml.FLAG_SHRINK_LAUNCH)) == ml.OK
    assert ml.validate(desc(flags=ml.FLAG_OUT_BF16 | ml.FLAG_SHRINK_LAUNCH)) == ml.OK


def test_shrink_launch_flag_keeps_the_decode_workspace_size():
    # decode shape: 16-row base blocks, so the shrinks run inside the
    # projection launches; their S buffers hold one partial per K range of
    # at most 4096, while the separate launch of this shape uses one range
    d = wl.CONFIGS["decode"]
    fused = ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"])
    sep = ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"],
                       flags=ml.FLAG_SHRINK_LAUNCH)
    assert ml.workspace_bytes(fused) == ml.workspace_bytes(sep)


def test_validate_key_limit_edge():
    # up to E * (L + 1) = 9712 keys one workgroup aligns; beyond, up to
    # 36864, the multi-launch path does (e.g. 256 experts x 128 adapters)
    assert ml.validate(desc(E=607, L=15, top_k=8)) == ml.OK     # 9712
    assert ml.validate(desc(E=972, L=9, top_k=8)) == ml.OK      # 9720
    assert ml.validate(desc(E=256, L=128, top_k=8)) == ml.OK    # 33024
    assert ml.validate(desc(E=1024, L=35, top_k=8)) == ml.OK    # 36864
    assert ml.validate(desc(E=1024, L=36, top_k=8)) == ml.EINVAL  # 37888


def test_validate_checks_weight_pointers():
    ds = desc()
    assert ml.validate(ds, ml.Weights(None, 4096, 4096, 4096, 4096, 4096)) == ml.EINVAL
    assert ml.validate(ds, ml.Weights(4096, 4104, 4096, 4096, 4096, 4096)) == ml.EINVAL  # misaligned
    assert ml.validate(ds, ml.Weights(4096, 4096, None, 4096, 4096, 4096)) == ml.EINVAL
    assert ml.validate(ds, ml.Weights(4096, 4096, 4096, 4096, 4096, 4096)) == ml.OK
    ds0 = desc(L=0)
    assert ml.validate(ds0, ml.Weights(4096, 4096, None, None, None, None)) == ml.OK
    # the optional packed copies: accepted when 16-byte aligned
    assert ml.validate(ds, ml.Weights(4096, 4096, 4096, 4096, 4096, 4096, 8192, 8192)) == ml.OK
    assert ml.validate(ds, ml.Weights(4096, 4096, 4096, 4096, 4096, 4096, 8200, None)) == ml.EINVAL
    assert ml.validate(ds, ml.Weights(4096, 4096, 4096, 4096, 4096, 4096, None, 8200)) == ml.EINVAL


def test_pack_weights_refuses_bad_pointers_on_the_host():
    ds = desc()
    f = ml.lib().moe_lora_pack_weights
    P = ctypes.c_void_p
    assert f(ctypes.byref(ds), P(4096), P(4096), P(8200), None, None) == ml.EINVAL   # misaligned output
    assert f(ctypes.byref(ds), P(4104), None, P(8192), None, None) == ml.EINVAL      # misaligned input
    assert f(ctypes.byref(ds), None, P(4096), P(8192), None, None) == ml.EINVAL      # output without input
    assert f(ctypes.byref(desc(H=100)), P(4096), P(4096), P(8192), P(8192), None) == ml.EINVAL
    assert f(ctypes.byref(ds), None, None, None, None, None) == ml.OK                # nothing to pack


def test_zero_tokens_is_valid():
    assert ml.validate(desc(T=0)) == ml.OK


@pytest.mark.parametrize("name", list(wl.CONFIGS))
@pytest.mark.parametrize("bm", [(0, 0), (16, 16), (32, 64), (128, 16), (256, 256)])
def test_capacity_matches_oracle_formula(name, bm):
    d = wl.CONFIGS[name]
    ds = ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"], *bm)
    bm_b, bm_l = ml.block_sizes(ds)
    if bm != (0, 0):
        assert (bm_b, bm_l) == bm
    C_b, C_l = ml.align_capacity(ds)
    assert (C_b, C_l) == oracle.capacities(d["T"] * d["top_k"], d["E"], d["L"], bm_b, bm_l)


def test_default_block_sizes():
    got = {}
    for name, d in wl.CONFIGS.items():
        ds = ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"])
        got[name] = ml.block_sizes(ds)
    assert got["decode"][0] == 16 and got["prefill"][0] == 128


def test_strerror_text():
    assert "workspace" in ml.strerror(ml.EWORKSPACE)
    assert ml.strerror(ml.OK) == "ok"
    assert ml.kernel_names()[0] == "route" and len(ml.kernel_names()) == ml.NKERNELS


def _noalloc_rc(ds):
    # fake, 16-byte aligned device addresses: every refusal tested here is
    # decided on the host before any HIP call or launch
    lib = ml.lib()
    p = ctypes.c_void_p(4096)
    return lib.moe_lora_forward_noalloc(ctypes.byref(ds), ctypes.byref(ml.Weights(*([4096] * 6))),
                                        p, p, p, p, None)


def test_noalloc_refuses_oversized_and_invalid_calls_on_the_host():
    assert "scratch" in ml.strerror(ml.ESCRATCH)
    c = wl.CONFIGS["prefill"]
    big = ml.make_desc(c["T"], c["H"], c["I"], c["E"], c["top_k"], c["L"], c["r"])
    assert ml.workspace_bytes(big) > ml.SCRATCH_BYTES
    assert _noalloc_rc(big) == ml.ESCRATCH
    assert _noalloc_rc(desc(H=2881)) == ml.EINVAL
    assert _noalloc_rc(desc(T=0)) == ml.OK  # a no-op


@pytest.mark.parametrize("name", ["tiny", "decode", "wide", "dense"])
def test_decode_sized_workloads_fit_the_static_scratch(name):
    d = wl.CONFIGS[name]
    ds = ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"])
    assert ml.workspace_bytes(ds) <= ml.SCRATCH_BYTES


def test_header_scratch_size_matches_binding():
    src = open(HEADER).read()
    m = re.search(r"#define MOE_LORA_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == ml.SCRATCH_BYTES


def test_fused_combine_drops_the_down_rows_from_the_workspace():
    # with FUSED_COMBINE the down projection adds its weighted rows into out,
    # so the fp32 [ksplit][C_b][H] buffer is not needed
    for name, d in wl.CONFIGS.items():
        args = [d[k] for k in ("T", "H", "I", "E", "top_k", "L", "r")]
        fused = ml.workspace_bytes(ml.make_desc(*args, flags=ml.FLAG_FUSED_COMBINE))
        kept = ml.workspace_bytes(ml.make_desc(*args))
        bf16 = ml.workspace_bytes(ml.make_desc(*args, flags=ml.FLAG_OUT_BF16))
        C_b, _ = ml.align_capacity(ml.make_desc(*args))
        assert kept == bf16 and kept - fused >= 4 * C_b * d["H"], name


def test_plan_resolves_the_library_defaults():
    d = wl.CONFIGS["decode"]
    p = ml.plan(ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"]))
    assert p["block_m_base"] == 16 and p["down_ksplit"] == 1 and p["waves_gate_up"] == 1
    assert p["frags_gate_up"] == 4
    assert p["shrinks_in_projections"] == 1 and p["combine_in_down"] == 0
    # the decode-shaped batch is aligned inside the gate_up launch (its
    # 4 x 32 top-k scan stays in the routing launch), unless the routing
    # launch or separate shrink launches are asked for; the tiny layer's
    # 2 x 8 scan runs inside the gate_up launch too
    assert p["routing_in_gate_up"] == 1
    tny = wl.CONFIGS["tiny"]
    assert ml.plan(ml.make_desc(tny["T"], tny["H"], tny["I"], tny["E"], tny["top_k"], tny["L"],
                                tny["r"]))["routing_in_gate_up"] == 2
    args = (d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"])
    assert ml.plan(ml.make_desc(*args, flags=ml.FLAG_ROUTE_LAUNCH))["routing_in_gate_up"] == 0
    assert ml.plan(ml.make_desc(*args, flags=ml.FLAG_SHRINK_LAUNCH))["routing_in_gate_up"] == 0
    assert ml.plan(ml.make_desc(*args, waves_gate_up=2))["routing_in_gate_up"] == 0
    assert ml.plan(ml.make_desc(17, *args[1:]))["routing_in_gate_up"] == 0  # T > 16
    d = wl.CONFIGS["prefill"]
    p = ml.plan(ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"]))
    assert p["block_m_base"] == 128 and p["waves_down"] == 0 and p["shrinks_in_projections"] == 0
    assert p["routing_in_gate_up"] == 0


@pytest.mark.parametrize("over", [
    dict(down_ksplit=-1), dict(down_ksplit=7),           # 45 chunks: 7 does not divide
    dict(down_ksplit=2, bm_b=128),                        # direct-load kernels take all of K
    dict(down_ksplit=90),                                 # more ranges than chunks
    dict(shrink_ksplit=5), dict(shrink_ksplit=2),         # decode runs the shrinks in the projections (1)
    dict(waves_gate_up=3), dict(waves_down=8),
    dict(waves_down=2, bm_b=32),                          # waves per tile only for 16-row blocks
    dict(waves_down=4, down_ksplit=3),                    # 15 chunks per range < 4 per wave x 4
    dict(frags_gate_up=6), dict(frags_gate_up=-4),        # 4 or 8 fragments per gate_up wave
    dict(frags_gate_up=8, bm_b=32),                       # only the 16-row kernel has them
    dict(frags_gate_up=8, waves_gate_up=2),               # 8 only with one wave per tile
])
def test_validate_rejects_bad_split_fields(over):
    over = dict(over)
    bm_b = over.pop("bm_b", 0)
    d = wl.CONFIGS["decode"]
    ds = ml.make_desc(d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"], bm_b, 0, **over)
    assert ml.validate(ds) == ml.EINVAL


def test_gate_up_fragments_follow_the_shape():
    # the plan reports the fragments per gate_up wave only for 16-row blocks
    # (8 of them cover 64 h columns; I is always a multiple of 64, the down
    # projection's K chunk)
    d = wl.CONFIGS["decode"]
    args = (d["T"], d["H"], d["I"], d["E"], d["top_k"], d["L"], d["r"])
    assert ml.plan(ml.make_desc(*args, frags_gate_up=8))["frags_gate_up"] == 8
    assert ml.plan(ml.make_desc(*args, frags_gate_up=4))["frags_gate_up"] == 4
    assert ml.plan(ml.make_desc(*args, block_m_base=64))["frags_gate_up"] == 0
    assert ml.validate(ml.make_desc(*args, block_m_base=64, frags_gate_up=4)) == ml.OK


def test_split_fields_change_only_the_plan_and_workspace():
    d = wl.CONFIGS["wide"]
    args = [d[k] for k in ("T", "H", "I", "E", "top_k", "L", "r")]
    base = ml.make_desc(*args, 32, 16)
    more = ml.make_desc(*args, 32, 16, down_ksplit=4, shrink_ksplit=1)  # I/64 = 172 chunks
    assert ml.validate(more) == ml.OK
    p = ml.plan(more)
    assert p["down_ksplit"] == 4 and p["shrink_ksplit"] == 1
    # one fp32 D partial per K range
    C_b, _ = ml.align_capacity(base)
    assert ml.workspace_bytes(more) > ml.workspace_bytes(base)


def test_one_wave_per_tile_takes_any_k():
    # the smallest K (one chunk of 64) with 16-row blocks
    ds = ml.make_desc(37, 64, 64, 70, 7, 3, 8, 16, 16)
    assert ml.validate(ds) == ml.OK
    assert ml.validate(ml.make_desc(37, 64, 64, 70, 7, 3, 8, 16, 16, waves_down=2)) == ml.EINVAL
