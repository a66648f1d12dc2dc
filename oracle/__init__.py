"""CPU oracle for the multi-LoRA MoE expert layer.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding. It
shares no code with the HIP path; both sides only share the seeded input
generator (which holds none of the layer's arithmetic).

Pieces:
  route()   top-k on the logits + renormalised softmax  (C, fp64 weights)
  align()   the (expert, adapter) grouping of the (token, choice) pairs into
            padded blocks, written as a plain sort in Python
  forward() the per-token, per-choice layer loop in C, fp64 throughout

Pages: the AWS ML Blog post "Efficiently serve dozens of fine-tuned models with
vLLM on Amazon SageMaker AI and Amazon Bedrock" and its Korean summary on
agentlenshq.com. Routing and aggregation: AWS post, section "Implementing
multi-LoRA inference for MoE models in vLLM". Two projections with a shrink and
an expand each: Korean summary, section "Multi-LoRA serving for MoE". The
extra LoRA-index grid axis and the compound expert x adapter sparsity that the
alignment expresses: AWS post, section "Tuning kernel configurations for
Amazon SageMaker AI and Amazon Bedrock", and the Korean summary's description
of fused_moe_lora.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_lora_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C part with gcc (portable x86-64-v3, OpenMP, IEEE math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.oracle_route.argtypes = [i32, i32, i32, P, P, P]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [i32] * 7 + [P] * 10 + [i32, P, P] + [P] * 5 + [i32]
        lib.oracle_forward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ------------------------------------------------------------------ A1 route

def route(logits: np.ndarray, top_k: int):
    """Top-k expert ids per token (ties -> lower id) and fp64 weights that
    are the softmax of the selected logits. Returns (ids int32 [T][k],
    w float64 [T][k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float64)
    rc = _load().oracle_route(T, E, top_k, _ptr(logits), _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    return ids, w


# ------------------------------------------------------------------ A2 align

def capacities(P: int, E: int, L: int, bm_b: int, bm_l: int):
    """Worst-case padded lengths of the two views: every non-empty segment may
    waste up to (block - 1) slots; at most min(#segments, P) are non-empty."""
    def roundup(v, m):
        return (v + m - 1) // m * m
    C_b = roundup(P + min(E, P) * (bm_b - 1), bm_b)
    C_l = roundup(P + min(E * L, P) * (bm_l - 1), bm_l)
    return C_b, C_l


def align(topk_ids: np.ndarray, adapter_ids: np.ndarray, E: int, L: int,
          bm_b: int, bm_l: int):
    """Group the P = T*k pairs p = t*k + j.

    The pairs are ordered by the key (expert, a', p) with a' = adapter if it
    lies in [0, L), else L ("no adapter" sorts last within its expert).
    Base view: for each expert in id order, its pairs in that order, padded
    with the sentinel P to a multiple of bm_b; one block id per bm_b slots.
    LoRA view: the same for the segments (expert, adapter) with adapter < L,
    experts ascending then adapters ascending, padded to bm_l.
    Slots past the used length hold P; unused block entries hold -1.
    """
    topk_ids = np.asarray(topk_ids)
    T, k = topk_ids.shape
    P = T * k
    expert = [int(topk_ids[p // k][p % k]) for p in range(P)]
    aprime = []
    for t in range(T):
        a = int(adapter_ids[t])
        aprime.append(a if 0 <= a < L else L)
    order = sorted(range(P), key=lambda p: (expert[p], aprime[p // k], p))

    C_b, C_l = capacities(P, E, L, bm_b, bm_l)

    by_expert = {}
    by_seg = {}
    for p in order:
        by_expert.setdefault(expert[p], []).append(p)
        a = aprime[p // k]
        if a < L:
            by_seg.setdefault((expert[p], a), []).append(p)

    sorted_b, blk_e_b = [], []
    for e in range(E):
        seg = by_expert.get(e, [])
        if not seg:
            continue
        nblk = (len(seg) + bm_b - 1) // bm_b
        sorted_b += seg + [P] * (nblk * bm_b - len(seg))
        blk_e_b += [e] * nblk
    n_b = len(sorted_b)

    sorted_l, blk_e_l, blk_a_l = [], [], []
    for e in range(E):
        for a in range(L):
            seg = by_seg.get((e, a), [])
            if not seg:
                continue
            nblk = (len(seg) + bm_l - 1) // bm_l
            sorted_l += seg + [P] * (nblk * bm_l - len(seg))
            blk_e_l += [e] * nblk
            blk_a_l += [a] * nblk
    n_l = len(sorted_l)

    def pad(lst, n, v):
        return np.array(lst + [v] * (n - len(lst)), dtype=np.int32)

    return dict(
        sorted_b=pad(sorted_b, C_b, P), blk_e_b=pad(blk_e_b, C_b // bm_b, -1), n_b=n_b,
        sorted_l=pad(sorted_l, C_l, P), blk_e_l=pad(blk_e_l, C_l // bm_l, -1),
        blk_a_l=pad(blk_a_l, C_l // bm_l, -1), n_l=n_l, C_b=C_b, C_l=C_l,
    )


# ------------------------------------------------------------------ the layer

def forward(case, ids: np.ndarray, w: np.ndarray, tokens=None, stages: bool = False,
            threads: int | None = None):
    """Layer output (fp64) for the listed tokens (default: all), given the
    routing (ids, w). With stages=True also returns per-(token, choice) rows
    of s1 [r], g [2I], h [I], s2 [r], d [H] (rows ordered token-list-major)."""
    T, H, I, E, k, L, r = case.T, case.H, case.I, case.E, case.top_k, case.L, case.r
    toks = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, np.int32)
    n = len(toks)
    out = np.empty((n, H), np.float64)
    st = None
    if stages:
        st = dict(s1=np.empty((n * k, r)), g=np.empty((n * k, 2 * I)), h=np.empty((n * k, I)),
                  s2=np.empty((n * k, r)), d=np.empty((n * k, H)))
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    arrs = [np.ascontiguousarray(a) for a in (case.x, case.adapter_ids, case.w_gate_up, case.w_down,
                                               case.a_gate_up, case.b_gate_up, case.a_down, case.b_down)]
    x, ad, wgu, wd, agu, bgu, adn, bdn = arrs
    ad = ad.astype(np.int32)
    rc = _load().oracle_forward(
        T, H, I, E, k, L, r, _ptr(x), _ptr(ids), _ptr(w), _ptr(ad),
        _ptr(wgu), _ptr(wd), _ptr(agu), _ptr(bgu), _ptr(adn), _ptr(bdn),
        n, _ptr(toks), _ptr(out),
        *(_ptr(st[q]) if st else None for q in ("s1", "g", "h", "s2", "d")),
        threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_forward failed ({rc})")
    return (out, st) if stages else out
