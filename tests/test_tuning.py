"""Host-side checks of the per-shape tuning table and the tuner's search space
(no GPU needed)."""
import json
import os

import pytest

from lora_mixture_experts_amd import moe_lora as ml
from lora_mixture_experts_amd import tune
from lora_mixture_experts_amd import tuning
from lora_mixture_experts_amd import workloads as wl

SHAPE = dict(H=2880, I=2880, E=32, top_k=4, L=8, r=32)


def entry(T_max, bm_b, bm_l=16, sep=False, us=1.0):
    return {"T_max": T_max, "block_m_base": bm_b, "block_m_lora": bm_l, "shrink_launch": sep, "us": us}


def test_round_trip_and_bucket_lookup(tmp_path):
    d = str(tmp_path)
    tuning.save_entry(d, SHAPE, entry(16, 16, sep=True))
    tuning.save_entry(d, SHAPE, entry(6400, 128, 32))
    tuning.save_entry(d, SHAPE, entry(512, 64))
    t = tuning.load(d)
    assert len(t) == 3
    args = [SHAPE[k] for k in tuning.SHAPE_KEYS]
    # an entry covers (T_max / 2, T_max]
    assert t.lookup(9, *args) == tuning.Choice(16, 16, True)
    assert t.lookup(16, *args) == tuning.Choice(16, 16, True)
    assert t.lookup(257, *args) == tuning.Choice(64, 16, False)
    assert t.lookup(512, *args) == tuning.Choice(64, 16, False)
    assert t.lookup(6400, *args) == tuning.Choice(128, 32, False)
    assert t.lookup(3201, *args) == tuning.Choice(128, 32, False)
    # between entries, below the smallest, beyond the largest, or another
    # shape: no advice (the library's defaults apply)
    for T in (1, 8, 17, 32, 256, 513, 3200, 6401):
        assert t.lookup(T, *args) is None, T
    assert t.lookup(16, 2880, 2880, 32, 4, 8, 64) is None
    # entries are kept sorted and replaced by T_max
    tuning.save_entry(d, SHAPE, entry(512, 32))
    t = tuning.load(d)
    assert [e["T_max"] for e in t.entries(*args)] == [16, 512, 6400]
    assert t.lookup(300, *args) == tuning.Choice(32, 16, False)


def test_explicit_t_min_widens_an_entry(tmp_path):
    d = str(tmp_path)
    e = entry(16, 16, sep=True)
    e["T_min"] = 1
    tuning.save_entry(d, SHAPE, e)
    t = tuning.load(d)
    args = [SHAPE[k] for k in tuning.SHAPE_KEYS]
    assert t.lookup(1, *args) == tuning.Choice(16, 16, True)
    assert t.lookup(17, *args) is None
    for bad in (0, 17, "1"):
        e["T_min"] = bad
        with pytest.raises(ValueError):
            tuning.save_entry(d, SHAPE, e)


def test_a_call_between_committed_entries_gets_the_library_defaults():
    # the committed decode/prefill shape has entries at T = 16 and 6400;
    # a 32-token batch must not inherit the prefill choice (128-row blocks)
    t = tuning.load(tuning.DEFAULT_FOLDER)
    c = wl.CONFIGS["decode"]
    args = [c[k] for k in tuning.SHAPE_KEYS]
    assert t.lookup(16, *args) is not None and t.lookup(6400, *args) is not None
    assert t.lookup(32, *args) is None


def test_every_committed_entry_is_a_benched_workload():
    # the GPU parity suite checks each committed entry at its own shape and
    # token count through the workload of that shape; an entry no workload
    # covers would be timed by no test
    t = tuning.load(tuning.DEFAULT_FOLDER)
    have = {(tuning.shape_key(*(d[k] for k in tuning.SHAPE_KEYS)), d["T"]) for d in wl.CONFIGS.values()}
    for key in t.shapes():
        for e in t.entries(*key):
            assert (key, e["T_max"]) in have, (key, e)


def test_files_are_named_by_shape(tmp_path):
    path = tuning.save_entry(str(tmp_path), SHAPE, entry(16, 16))
    assert os.path.basename(path) == "H2880_I2880_E32_k4_L8_r32.json"
    doc = json.load(open(path))
    assert doc["shape"] == SHAPE and doc["device"] == "gfx950"


@pytest.mark.parametrize("bad", [dict(block_m_base=48), dict(block_m_lora=8), dict(T_max=0), dict(T_min=0),
                                 dict(shrink_launch="yes"), dict(block_m_base=None)])
def test_invalid_entries_are_rejected(tmp_path, bad):
    e = entry(16, 16)
    e.update(bad)
    with pytest.raises(ValueError):
        tuning.save_entry(str(tmp_path), SHAPE, e)
    path = tmp_path / "x.json"
    path.write_text(json.dumps({"shape": SHAPE, "entries": [e]}))
    with pytest.raises(ValueError):
        tuning.load(str(tmp_path))


def test_missing_folder_is_an_error_and_other_files_are_ignored(tmp_path):
    with pytest.raises(FileNotFoundError):
        tuning.load(str(tmp_path / "nope"))
    (tmp_path / "README.txt").write_text("not a table")
    assert len(tuning.load(str(tmp_path))) == 0


def test_committed_table_loads_and_names_valid_choices():
    if not os.path.isdir(tuning.DEFAULT_FOLDER):
        pytest.skip("no committed tuning folder")
    t = tuning.load(tuning.DEFAULT_FOLDER)
    for key in t.shapes():
        for e in t.entries(*key):
            H, I, E, k, L, r = key
            d = ml.make_desc(e["T_max"], H, I, E, k, L, r, e["block_m_base"], e["block_m_lora"],
                             ml.FLAG_SHRINK_LAUNCH if e["shrink_launch"] else 0)
            assert ml.validate(d) == ml.OK, (key, e)


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_search_space_holds_the_library_default(name):
    c = wl.CONFIGS[name]
    cands = list(tune.candidates(c["L"]))
    assert len(set(cands)) == len(cands)
    d0 = ml.make_desc(c["T"], c["H"], c["I"], c["E"], c["top_k"], c["L"], c["r"])
    bm_b, bm_l = ml.block_sizes(d0)
    assert (bm_b, bm_l, False) in cands
    valid = [x for x in cands
             if ml.validate(ml.make_desc(c["T"], c["H"], c["I"], c["E"], c["top_k"], c["L"], c["r"], x[0], x[1],
                                         ml.FLAG_SHRINK_LAUNCH if x[2] else 0)) == ml.OK]
    assert len(valid) >= 10
