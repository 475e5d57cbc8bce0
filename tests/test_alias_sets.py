"""The padded-row alias predictor reproduces the worked example printed on the
FlyDSL conv3d fp8 page, then predicts the packed-varlen alias sets used by the
GPU bounds tests."""
import json
import os

import numpy as np

from alias_sets import conv_fast_path_alias, packed_alias_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "conv3d_padded_row_alias.json")


def test_conv3d_alias_set_matches_page():
    g = json.load(open(GOLDEN))
    off = conv_fast_path_alias(g["npq"], g["tile_m"], g["columns"], g["dhw"])
    assert -(-g["npq"] // g["tile_m"]) == g["grid_m"]
    assert g["grid_m"] * g["tile_m"] - g["npq"] == g["padded_rows"]
    assert len(off) == g["alias_offsets"]
    assert round(100.0 * len(off) / (g["columns"] * g["dhw"]), 2) == g["clobberable_percent"]
    # the page's example: column 0, row 288 lands on column 1, row 0
    assert 288 in off


def test_packed_varlen_alias_rows():
    # causal GQA varlen workload, 128-row tiles
    lens = [4096, 2500, 1, 3969]
    res = packed_alias_rows(lens, 128)
    cu = np.concatenate([[0], np.cumsum(lens)])
    assert len(res[0][0]) == 0 and res[0][1] == 0
    rows1, past1 = res[1]
    assert len(rows1) == 60 and past1 == 0
    assert rows1[0] == cu[2] and rows1[1] == cu[3] and rows1[-1] == cu[3] + 58
    rows2, past2 = res[2]
    assert len(rows2) == 127 and rows2[0] == cu[3] and rows2[-1] == cu[3] + 126
    rows3, past3 = res[3]
    assert len(rows3) == 0 and past3 == 127
    # tiny causal workload: 300 rows in 3 tiles leave 84 padded rows, all past the end
    (r, p), = packed_alias_rows([300], 128)
    assert len(r) == 0 and p == 84
