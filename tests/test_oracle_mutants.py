"""Plant plausible mistakes in a private copy of the oracle (on the CPU) and
check that at least one pin catches each one. This shows the pins in
test_oracle_pins.py constrain every part of the oracle."""
import importlib.util
import os
import shutil
import subprocess

import numpy as np
import pytest

import tests.test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")

C_MUTANTS = {
    "tie_break_ge": ("row[e] > row[best]", "row[e] >= row[best]"),
    "no_renormalise": ("w[(size_t)t * k + j] /= s;", "(void)s;"),
    "no_max_shift": ("double m = (double)row[ids[(size_t)t * k]];", "double m = 0.0;"),
    "gate_up_swapped": ("h[q] = silu(g[q]) * g[I64 + q];", "h[q] = silu(g[I64 + q]) * g[q];"),
    "drop_gate_up_expand": ("g[n] += t2[n];", "g[n] += 0.0 * t2[n];"),
    "drop_down_expand": ("d[n] += d2[n];", "d[n] += 0.0 * d2[n];"),
    "lora_index_transposed": ("const int64_t ae = (int64_t)a * E64 + e;\n                        /* shrink",
                              "const int64_t ae = e * (int64_t)L + a;\n                        /* shrink"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "combine_first_weight": ("const double wj = w[(int64_t)t * k + j];", "const double wj = w[(int64_t)t * k];"),
}

PY_MUTANTS = {
    "align_ignores_adapter": ("key=lambda p: (expert[p], aprime[p // k], p)", "key=lambda p: (expert[p], p)"),
    "align_no_padding": ("sorted_b += seg + [P] * (nblk * bm_b - len(seg))", "sorted_b += seg"),
    "align_keeps_no_adapter": ("        if a < L:\n            by_seg", "        if a <= L:\n            by_seg",
                               "        for a in range(L):\n            seg = by_seg", "        for a in range(L + 1):\n            seg = by_seg"),
}


def _load_variant(tmp_path, c_mut=None, py_mut=None):
    d = tmp_path / "oracle_variant"
    shutil.copytree(ORACLE_DIR, d, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    if c_mut:
        src = (d / "moe_lora_oracle.c").read_text()
        assert c_mut[0] in src, c_mut[0]
        (d / "moe_lora_oracle.c").write_text(src.replace(c_mut[0], c_mut[1]))
    if py_mut:
        src = (d / "__init__.py").read_text()
        for old, new in zip(py_mut[0::2], py_mut[1::2]):
            assert old in src, old
            src = src.replace(old, new)
        (d / "__init__.py").write_text(src)
    spec = importlib.util.spec_from_file_location("oracle_variant", d / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build(force=True)
    mod._load()
    return mod


def _pin_calls(m):
    yield lambda: pins.test_route_matches_full_sort_and_full_softmax(m, 0)
    yield lambda: pins.test_route_ties_pick_lower_expert(m)
    yield lambda: pins.test_route_k_equals_e_is_full_softmax(m)
    yield lambda: pins.test_route_large_logits_no_overflow(m)
    yield lambda: pins.test_align_handworked(m)
    for s in range(12):
        yield lambda s=s: pins.test_align_invariants_random(m, s)
    yield lambda: pins.test_align_invariants_configs(m, "decode")
    yield lambda: pins.test_forward_matches_dense_merged_weights(m, 0, {})
    yield lambda: pins.test_single_expert_is_textbook_swiglu_mlp(m)
    yield lambda: pins.test_no_adapter_equals_zero_lora(m)


def _caught(m):
    for call in _pin_calls(m):
        try:
            with np.errstate(all="ignore"):
                call()
        except AssertionError:
            return True
    return False


@pytest.fixture(scope="module")
def have_gcc():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")


def test_unmutated_copy_passes(tmp_path, have_gcc):
    assert not _caught(_load_variant(tmp_path))


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_is_caught(tmp_path, have_gcc, name):
    assert _caught(_load_variant(tmp_path, c_mut=C_MUTANTS[name])), name


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_mutant_is_caught(tmp_path, have_gcc, name):
    assert _caught(_load_variant(tmp_path, py_mut=PY_MUTANTS[name])), name
