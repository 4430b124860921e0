"""The tile tuner without a GPU: candidate validity, the choice per key, the tables it writes, and
that the committed header holds what the committed measurements choose."""

import json
import os
import re
import shutil

import pytest

from exact_attention_94_amd import tune


def test_candidates_respect_whole_1kb_loads_per_wave():
    assert tune.valid(64, 64) and tune.valid(128, 64) and tune.valid(32, 64)
    assert not tune.valid(32, 32) and tune.valid(64, 32)
    assert not tune.valid(32, 96) and tune.valid(64, 96) and tune.valid(128, 96)
    for f, q, k in tune.CANDIDATE_SETS:
        assert f in tune.FWD_CANDIDATES and q in tune.BWD_CANDIDATES and k in tune.BWD_CANDIDATES


def _parse_table(text, macro):
    """The [4][2][2] initialiser of a table macro as nested lists."""
    start = text.index(f"#define {macro}")
    body = text[start:text.index("}}}", start) + 3].replace("\\\n", " ")
    nums = [int(x) for x in re.findall(r"\d+", body[body.index("{"):])]
    assert len(nums) == 16
    return [[[nums[4 * i + 2 * j + c] for c in range(2)] for j in range(2)] for i in range(4)]


def test_write_picks_the_fastest_tile_per_key(tmp_path):
    header = tmp_path / "fa_tune.h"
    shutil.copy(tune.HEADER, header)
    res = {"fwd": {}, "dkdv": {}, "dq": {}}
    # Make the fastest tile depend on every part of the key, so that a transposed index fails.
    for d in tune.HEAD_DIMS:
        for dt in tune.DTYPES:
            for causal in tune.CAUSAL:
                k = tune.key(d, dt, causal)
                fast = {(32, "f16", False): 128, (64, "bf16", True): 32}.get((d, dt, causal), 64)
                res["fwd"][k] = {str(c): (1.0 if c == fast else 2.0) for c in (32, 64, 128)
                                 if tune.valid(c, d)}
                qfast = 32 if (dt == "bf16" and causal and tune.valid(32, d)) else 64
                res["dkdv"][k] = {str(c): (1.0 if c == qfast else 2.0) for c in (32, 64)
                                  if tune.valid(c, d)}
                kfast = 32 if (d == 128 and not causal) else 64
                res["dq"][k] = {str(c): (1.0 if c == kfast else 2.0) for c in (32, 64)
                                if tune.valid(c, d)}
    path = tmp_path / "r.json"
    path.write_text(json.dumps(res))
    best = tune.write(str(path), header=str(header))
    text = header.read_text()
    fwd = _parse_table(text, "FA_FWD_BC_TABLE")
    dkdv = _parse_table(text, "FA_DKDV_BQ_TABLE")
    dq = _parse_table(text, "FA_DQ_BC_TABLE")
    assert fwd[0][0][0] == 128 and fwd[1][1][1] == 32 and fwd[1][1][0] == 64 and fwd[0][1][0] == 64
    assert dkdv[1][1][1] == 32 and dkdv[1][1][0] == 64 and dkdv[1][0][1] == 64
    assert dkdv[0][1][1] == 64  # d = 32: 32 queries is no candidate
    assert dq[3][0][0] == 32 and dq[3][1][0] == 32 and dq[3][0][1] == 64
    for i, d in enumerate(tune.HEAD_DIMS):
        for j, dt in enumerate(tune.DTYPES):
            for c, causal in enumerate(tune.CAUSAL):
                k = tune.key(d, dt, causal)
                assert fwd[i][j][c] == best["fwd"][k] and dq[i][j][c] == best["dq"][k]
    # The rest of the header is untouched, and writing twice is stable.
    tune.write(str(path), header=str(header))
    assert header.read_text() == text
    assert "#define FA_FWD_PRE 4" in text


def test_committed_header_matches_committed_measurements():
    if not os.path.exists(tune.RESULTS):
        pytest.skip("no committed tuning measurements")
    best = tune.choose(json.load(open(tune.RESULTS)))
    text = open(tune.HEADER, encoding="utf-8").read()
    for table, macro in (("fwd", "FA_FWD_BC_TABLE"), ("dkdv", "FA_DKDV_BQ_TABLE"),
                         ("dq", "FA_DQ_BC_TABLE")):
        got = _parse_table(text, macro)
        for i, d in enumerate(tune.HEAD_DIMS):
            for j, dt in enumerate(tune.DTYPES):
                for c, causal in enumerate(tune.CAUSAL):
                    assert got[i][j][c] == best[table][tune.key(d, dt, causal)], (table, d, dt,
                                                                                  causal)
