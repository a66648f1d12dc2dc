"""Seeded synthetic inputs for the multi-LoRA MoE expert layer.

This module only draws numbers; it computes none of the layer's arithmetic
(no routing, no sorting, no products). Both the HIP library's tests/bench and
the CPU oracle consume exactly the arrays produced here.

Workload shapes follow the pages: the AWS ML Blog post "Efficiently serve
dozens of fine-tuned models with vLLM on Amazon SageMaker AI and Amazon
Bedrock" (section "Implementing multi-LoRA inference for MoE models in vLLM":
1600-token prompts at concurrency 16; Figure 1: hidden 4096, intermediate
11008, rank 32; Figure 3 caption: rank 32 with 8 adapters loaded). Model
dimensions of the GPT-OSS-20B-like layer (hidden = intermediate = 2880,
32 experts, top-4) are taken as given workload parameters.

Storage conventions (all row-major, contiguous):
  x            bf16 bits (uint16) [T][H]
  logits       float32            [T][E]
  adapter_ids  int32              [T]      (-1 = no adapter)
  w_gate_up    bf16 bits          [E][2I][H]   rows 0..I-1 gate, I..2I-1 up
  w_down       bf16 bits          [E][H][I]
  a_gate_up    bf16 bits          [L][E][r][H]
  b_gate_up    bf16 bits          [L][E][2I][r]
  a_down       bf16 bits          [L][E][r][I]
  b_down       bf16 bits          [L][E][H][r]

Every block is drawn from its own PCG64 stream keyed by (seed, tag, index...),
so a block's values do not depend on which other blocks are drawn. Values are
drawn in float32 and rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# name -> shape parameters; seed = position in this table
CONFIGS = {
    "tiny": dict(T=16, H=256, I=512, E=8, top_k=2, L=2, r=8),
    "decode": dict(T=16, H=2880, I=2880, E=32, top_k=4, L=8, r=32),
    "prefill": dict(T=6400, H=2880, I=2880, E=32, top_k=4, L=8, r=32),
    "wide": dict(T=64, H=4096, I=11008, E=8, top_k=2, L=8, r=32),
    "many": dict(T=512, H=2880, I=2880, E=32, top_k=4, L=128, r=64),
    # dense multi-LoRA projection pair (one expert, so routing is trivial):
    # the pages report that the same work also speeds up dense models such as
    # Qwen3 32B (AWS post, first section; Korean summary, "Performance
    # benchmarks and availability"); Qwen3-32B-like MLP dims at decode, one
    # adapter per request as in "decode"
    "dense": dict(T=16, H=5120, I=25600, E=1, top_k=1, L=8, r=32),
}
CONFIG_SEED = {name: i for i, name in enumerate(CONFIGS)}

WEIGHT_STD = 0.02
BF16_NAN = np.uint16(0x7FC0)

# stream tags
_TAG_LOGITS, _TAG_X, _TAG_ADAPTER, _TAG_BIAS = 1, 2, 3, 4
_TAG_WGU, _TAG_WD = 10, 11
_TAG_AGU, _TAG_BGU, _TAG_AD, _TAG_BD = 20, 21, 22, 23


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(key, n, std):
    rng = np.random.default_rng(list(key))
    v = rng.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


@dataclass
class Case:
    """One layer invocation's inputs (host arrays)."""
    name: str
    T: int
    H: int
    I: int
    E: int
    top_k: int
    L: int
    r: int
    x: np.ndarray
    logits: np.ndarray
    adapter_ids: np.ndarray
    w_gate_up: np.ndarray
    w_down: np.ndarray
    a_gate_up: np.ndarray
    b_gate_up: np.ndarray
    a_down: np.ndarray
    b_down: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        return dict(T=self.T, H=self.H, I=self.I, E=self.E, top_k=self.top_k, L=self.L, r=self.r)


# ---------------------------------------------------------------- routing side

def _many_request_lengths(rng, n_req, total, lo, hi):
    """Draw n_req lengths from U{lo..hi}, scale them to sum to `total`, floor,
    then hand out the remainder largest-fraction-first within [lo, hi]."""
    raw = rng.integers(lo, hi + 1, size=n_req).astype(np.float64)
    scaled = raw * (total / raw.sum())
    base = np.clip(np.floor(scaled).astype(np.int64), lo, hi)
    rem = total - int(base.sum())
    frac = scaled - np.floor(scaled)
    order = np.argsort(-frac, kind="stable")
    i = 0
    while rem != 0:
        j = order[i % n_req]
        if rem > 0 and base[j] < hi:
            base[j] += 1
            rem -= 1
        elif rem < 0 and base[j] > lo:
            base[j] -= 1
            rem += 1
        i += 1
    return base


def routing_inputs(name: str, dims: dict, seed: int):
    """logits f32 [T][E], x bf16 bits [T][H], adapter_ids i32 [T], meta."""
    T, H, E, L = dims["T"], dims["H"], dims["E"], dims["L"]
    logits = np.random.default_rng([seed, _TAG_LOGITS]).standard_normal((T, E), dtype=np.float32)
    x = _normal_bf16((seed, _TAG_X), T * H, 1.0).reshape(T, H)
    rng = np.random.default_rng([seed, _TAG_ADAPTER])
    meta = {}
    if name == "tiny":
        ad = rng.integers(-1, 2, size=T)
    elif name in ("decode", "dense"):
        # one token per request, concurrency T; adapter uniform over the L slots
        ad = rng.integers(0, L, size=T)
    elif name == "prefill":
        n_req = 4
        per = rng.integers(0, L, size=n_req)
        ad = np.repeat(per, T // n_req)
        meta["request_lengths"] = [T // n_req] * n_req
    elif name == "wide":
        ad = rng.integers(0, L, size=T)
        ad[rng.random(T) < 0.25] = -1
        # per-expert bias = log-pmf of Zipf(s=1.2) over the ranks of a permutation
        perm = np.random.default_rng([seed, _TAG_BIAS]).permutation(E) + 1
        bias = (-1.2 * np.log(perm.astype(np.float64))).astype(np.float32)
        logits = (logits + bias[None, :]).astype(np.float32)
        meta["expert_bias"] = bias
    elif name == "many":
        n_req = 64
        lens = _many_request_lengths(rng, n_req, T, 1, 32)
        perm = np.random.default_rng([seed, _TAG_BIAS]).permutation(L)
        ranks = np.arange(1, L + 1, dtype=np.float64)
        pmf = ranks ** -1.1
        pmf /= pmf.sum()
        req_rank = rng.choice(L, size=n_req, p=pmf)
        req_adapter = perm[req_rank]
        ad = np.repeat(req_adapter, lens)
        meta["request_lengths"] = lens.tolist()
    else:
        ad = rng.integers(-1, L, size=T) if L > 0 else np.full(T, -1)
    return logits, x, np.ascontiguousarray(ad, dtype=np.int32), meta


# ---------------------------------------------------------------- weights side

def _fill_blocks(out, keys, nper, std, select, fill, workers):
    """out: uint16 [nblk][nper]; keys[i] = stream key of block i."""
    def one(i):
        if select is None or i in select:
            out[i] = _normal_bf16(keys[i], nper, std)
        else:
            out[i] = fill
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(len(keys))))


def make_case(name: str, seed: int | None = None, dims: dict | None = None,
              experts=None, lora_blocks=None, fill=BF16_NAN, workers: int | None = None) -> Case:
    """Build one case.

    name        a key of CONFIGS, or any label when `dims` is given
    experts     optional set of expert ids whose base weights are drawn; the
                rest are filled with `fill` (default: bf16 NaN, so a read of an
                untouched expert poisons the output)
    lora_blocks optional set of (adapter, expert) whose A/B are drawn
    """
    if dims is None:
        dims = CONFIGS[name]
    if seed is None:
        seed = CONFIG_SEED.get(name, 0)
    T, H, I, E, k, L, r = (dims[q] for q in ("T", "H", "I", "E", "top_k", "L", "r"))
    workers = workers or min(16, os.cpu_count() or 1)
    logits, x, ad, meta = routing_inputs(name, dims, seed)

    wgu = np.empty((E, 2 * I * H), np.uint16)
    wd = np.empty((E, H * I), np.uint16)
    sel_e = None if experts is None else set(int(e) for e in experts)
    _fill_blocks(wgu, [(seed, _TAG_WGU, e) for e in range(E)], 2 * I * H, WEIGHT_STD, sel_e, fill, workers)
    _fill_blocks(wd, [(seed, _TAG_WD, e) for e in range(E)], H * I, WEIGHT_STD, sel_e, fill, workers)

    nb = L * E
    sel_l = None if lora_blocks is None else set(int(a) * E + int(e) for a, e in lora_blocks)
    agu = np.empty((nb, r * H), np.uint16)
    bgu = np.empty((nb, 2 * I * r), np.uint16)
    adn = np.empty((nb, r * I), np.uint16)
    bdn = np.empty((nb, H * r), np.uint16)
    blk = [(a, e) for a in range(L) for e in range(E)]
    _fill_blocks(agu, [(seed, _TAG_AGU, a, e) for a, e in blk], r * H, WEIGHT_STD, sel_l, fill, workers)
    _fill_blocks(bgu, [(seed, _TAG_BGU, a, e) for a, e in blk], 2 * I * r, WEIGHT_STD, sel_l, fill, workers)
    _fill_blocks(adn, [(seed, _TAG_AD, a, e) for a, e in blk], r * I, WEIGHT_STD, sel_l, fill, workers)
    _fill_blocks(bdn, [(seed, _TAG_BD, a, e) for a, e in blk], H * r, WEIGHT_STD, sel_l, fill, workers)

    return Case(name=name, T=T, H=H, I=I, E=E, top_k=k, L=L, r=r,
                x=x, logits=logits, adapter_ids=ad,
                w_gate_up=wgu.reshape(E, 2 * I, H), w_down=wd.reshape(E, H, I),
                a_gate_up=agu.reshape(L, E, r, H), b_gate_up=bgu.reshape(L, E, 2 * I, r),
                a_down=adn.reshape(L, E, r, I), b_down=bdn.reshape(L, E, H, r), meta=meta)


def routing_only(name: str, seed: int | None = None, dims: dict | None = None):
    """Just (logits, x, adapter_ids, meta) for a config, without weights."""
    if dims is None:
        dims = CONFIGS[name]
    if seed is None:
        seed = CONFIG_SEED.get(name, 0)
    return routing_inputs(name, dims, seed)


def random_dims(rng: np.random.Generator):
    """Small random shapes for property tests (H, I multiples of 64)."""
    E = int(rng.integers(1, 9))
    k = int(rng.integers(1, E + 1))
    return dict(T=int(rng.integers(1, 40)), H=64 * int(rng.integers(1, 5)),
                I=64 * int(rng.integers(1, 5)), E=E, top_k=min(k, 8),
                L=int(rng.integers(0, 4)), r=int(rng.choice([8, 16, 32])))


def device_tensors(case: Case, device="cuda"):
    """Copy a case to device tensors (bf16 arrays as torch.bfloat16)."""
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    return dict(
        x=bf(case.x), logits=torch.from_numpy(np.ascontiguousarray(case.logits)).to(device),
        adapter_ids=torch.from_numpy(np.ascontiguousarray(case.adapter_ids, dtype=np.int32)).to(device),
        w_gate_up=bf(case.w_gate_up), w_down=bf(case.w_down),
        a_gate_up=bf(case.a_gate_up), b_gate_up=bf(case.b_gate_up),
        a_down=bf(case.a_down), b_down=bf(case.b_down))
