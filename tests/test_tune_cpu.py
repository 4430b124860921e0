"""The forward tile-width tuner without a GPU: candidate validity and the table it writes."""

import json
import shutil

from exact_attention_94_amd import tune


def test_candidates_respect_whole_1kb_loads_per_wave():
    assert tune.valid(64, 64) and tune.valid(128, 64) and tune.valid(32, 64)
    assert not tune.valid(32, 32) and tune.valid(64, 32)
    assert not tune.valid(32, 96) and tune.valid(64, 96) and tune.valid(128, 96)


def test_write_picks_the_fastest_width_per_head_dim(tmp_path):
    header = tmp_path / "fa_tune.h"
    shutil.copy(tune.HEADER, header)
    res = {"32": {"64": 2.0, "128": 1.0}, "64": {"32": 3.0, "64": 1.5, "128": 2.5},
           "96": {"64": 1.0, "128": 9.0}, "128": {"32": 2.0, "64": 3.0, "128": 4.0}}
    path = tmp_path / "r.json"
    path.write_text(json.dumps(res))
    best = tune.write(str(path), header=str(header))
    assert best == {32: "128", 64: "64", 96: "64", 128: "32"}
    text = header.read_text()
    for d, k in best.items():
        assert f"#define FA_FWD_BC_{d} {k}\n" in text
