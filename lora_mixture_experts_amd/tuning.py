"""Per-shape launch configurations, loadable from a folder.

The AWS ML Blog post "Efficiently serve dozens of fine-tuned models with vLLM
on Amazon SageMaker AI and Amazon Bedrock" (section "Tuning kernel
configurations for Amazon SageMaker AI and Amazon Bedrock") tunes the MoE-LoRA
kernels per shape and loads the tuned configurations from a user-supplied
folder. Here a configuration is what the C ABI lets a caller choose without
changing results: the row blocks of the two alignment views (which also pick
each projection's tile shape), whether the LoRA shrinks get launches of their
own, the split-K factors (K ranges of the down projection and of the
shrinks, waves per tile of the 16-row projections) and the weight fragments
per 16-row gate_up wave. Any valid choice
computes the same layer (up to fp32 summation order); the table only decides
speed.

A folder holds one JSON file per layer shape (written by
``python -m lora_mixture_experts_amd.tune``)::

    {"shape": {"H": 2880, "I": 2880, "E": 32, "top_k": 4, "L": 8, "r": 32},
     "device": "gfx950",
     "entries": [{"T_max": 16, "block_m_base": 16, "block_m_lora": 16,
                  "shrink_launch": false, "down_ksplit": 0, "shrink_ksplit": 0,
                  "waves_gate_up": 0, "waves_down": 0, "frags_gate_up": 0,
                  "us": 307.9}, ...]}

The five launch keys after shrink_launch are optional (0 or absent = the
library's choice).

An entry covers the token counts ``T_min <= T <= T_max``; ``T_min`` is
optional and defaults to ``T_max // 2 + 1``, so a choice tuned at one batch
size is applied only to batches of about that size (the best block sizes
follow the rows per expert, which grow with T). For a call with T tokens the
covering entry with the smallest ``T_max`` applies; where no entry covers T
the table has no advice and the library's own defaults apply.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass

SHAPE_KEYS = ("H", "I", "E", "top_k", "L", "r")
POW2_BLOCKS = (16, 32, 64, 128, 256)
SPLIT_KEYS = ("down_ksplit", "shrink_ksplit", "waves_gate_up", "waves_down", "frags_gate_up")


@dataclass(frozen=True)
class Choice:
    block_m_base: int
    block_m_lora: int
    shrink_launch: bool
    down_ksplit: int = 0
    shrink_ksplit: int = 0
    waves_gate_up: int = 0
    waves_down: int = 0
    frags_gate_up: int = 0


def choice_of(e) -> Choice:
    return Choice(e["block_m_base"], e["block_m_lora"], bool(e.get("shrink_launch", False)),
                  *(int(e.get(k, 0)) for k in SPLIT_KEYS))


def shape_key(H, I, E, top_k, L, r):
    return (int(H), int(I), int(E), int(top_k), int(L), int(r))


def file_name(H, I, E, top_k, L, r):
    return f"H{H}_I{I}_E{E}_k{top_k}_L{L}_r{r}.json"


def t_min_of(e) -> int:
    """Smallest token count an entry covers."""
    return int(e["T_min"]) if "T_min" in e else e["T_max"] // 2 + 1


def _check_entry(e, where):
    for key in ("T_max", "block_m_base", "block_m_lora"):
        if not isinstance(e.get(key), int):
            raise ValueError(f"{where}: entry needs an integer {key!r}: {e}")
    if e["T_max"] < 1:
        raise ValueError(f"{where}: T_max must be >= 1: {e}")
    if "T_min" in e and (not isinstance(e["T_min"], int) or not 1 <= e["T_min"] <= e["T_max"]):
        raise ValueError(f"{where}: T_min must be an integer in [1, T_max]: {e}")
    for key in ("block_m_base", "block_m_lora"):
        if e[key] not in POW2_BLOCKS:
            raise ValueError(f"{where}: {key} must be one of {POW2_BLOCKS}: {e}")
    if not isinstance(e.get("shrink_launch", False), bool):
        raise ValueError(f"{where}: shrink_launch must be a boolean: {e}")
    for key in SPLIT_KEYS:
        v = e.get(key, 0)
        if not isinstance(v, int) or isinstance(v, bool) or v < 0:
            raise ValueError(f"{where}: {key} must be an integer >= 0: {e}")
    for key in ("waves_gate_up", "waves_down"):
        if e.get(key, 0) not in (0, 1, 2, 4):
            raise ValueError(f"{where}: {key} must be 0, 1, 2 or 4: {e}")
    if e.get("frags_gate_up", 0) not in (0, 4, 8):
        raise ValueError(f"{where}: frags_gate_up must be 0, 4 or 8: {e}")


class Table:
    """Tuned choices by layer shape and token count."""

    def __init__(self):
        self._by_shape: dict[tuple, list[dict]] = {}

    def add(self, shape: dict, entries: list[dict], where: str = "table"):
        key = shape_key(*(shape[k] for k in SHAPE_KEYS))
        for e in entries:
            _check_entry(e, where)
        merged = {e["T_max"]: e for e in self._by_shape.get(key, [])}
        merged.update({e["T_max"]: e for e in entries})
        self._by_shape[key] = sorted(merged.values(), key=lambda e: e["T_max"])

    def lookup(self, T, H, I, E, top_k, L, r) -> Choice | None:
        for e in self._by_shape.get(shape_key(H, I, E, top_k, L, r), []):
            if t_min_of(e) <= T <= e["T_max"]:
                return choice_of(e)
        return None

    def shapes(self):
        return sorted(self._by_shape)

    def entries(self, H, I, E, top_k, L, r):
        return list(self._by_shape.get(shape_key(H, I, E, top_k, L, r), []))

    def __len__(self):
        return sum(len(v) for v in self._by_shape.values())


def load(folder: str) -> Table:
    """Read every ``*.json`` table file of a folder (a missing folder is an
    error; an empty one gives an empty table)."""
    if not os.path.isdir(folder):
        raise FileNotFoundError(f"tuning folder not found: {folder}")
    table = Table()
    for name in sorted(os.listdir(folder)):
        if not name.endswith(".json"):
            continue
        path = os.path.join(folder, name)
        with open(path) as f:
            doc = json.load(f)
        shape = doc.get("shape")
        if not isinstance(shape, dict) or any(not isinstance(shape.get(k), int) for k in SHAPE_KEYS):
            raise ValueError(f"{path}: 'shape' must give integers {SHAPE_KEYS}")
        table.add(shape, doc.get("entries", []), where=path)
    return table


def save_entry(folder: str, shape: dict, entry: dict, device: str = "gfx950") -> str:
    """Insert (or replace, by T_max) one entry in the shape's file."""
    _check_entry(entry, "new entry")
    os.makedirs(folder, exist_ok=True)
    path = os.path.join(folder, file_name(*(shape[k] for k in SHAPE_KEYS)))
    doc = {"shape": {k: int(shape[k]) for k in SHAPE_KEYS}, "device": device, "entries": []}
    if os.path.exists(path):
        with open(path) as f:
            doc = json.load(f)
    entries = {e["T_max"]: e for e in doc.get("entries", [])}
    entries[entry["T_max"]] = entry
    doc["entries"] = sorted(entries.values(), key=lambda e: e["T_max"])
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    return path


DEFAULT_FOLDER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "configs")
