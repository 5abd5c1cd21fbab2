"""Host logic of the layout cost model (CPU): its share decomposition agrees with
the oracle's pinned Table 2 decomposition, and the chooser picks the cheapest
layout under given share times."""
import json
import os

import pytest

import oracle
from layout_agnostic_latent_amd import layout_model as lm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table2_loads.json")


@pytest.mark.parametrize("layout", lm.LAYOUTS)
@pytest.mark.parametrize("B,T,s,H", [(16, 8, 4096, 128), (16, 8, 65536, 128), (13, 4, 1000, 64), (3, 8, 96, 16),
                                     (64, 8, 512, 128)])
def test_shares_match_oracle_decomposition(layout, B, T, s, H):
    mine = lm.rank_shares(layout, B, T, s, H)
    ref = oracle.layout_shares(layout, B, T, s, H)
    assert len(mine) == len(ref) == T
    # the same multiset of (requests, tokens, heads) per rank
    got = sorted((sh.reqs, sh.tokens, sh.heads) for sh in mine)
    want = sorted((len(r["reqs"]), r["toks"][1] - r["toks"][0], r["heads"][1] - r["heads"][0]) for r in ref)
    assert got == want
    # and the same busiest-rank loads as Table 2's columns
    load = oracle.busiest_rank_load(ref, s, H)
    bs = lm.busiest_share(layout, B, T, s, H)
    assert bs.kv_tokens * bs.heads / (s * H) == pytest.approx(load["attention_work"])
    assert max(sh.kv_tokens for sh in mine) / s == pytest.approx(load["kv_read"])
    # shares cover the step's work exactly once
    assert sum(sh.kv_tokens * sh.heads for sh in mine) == B * s * H


def test_table2_rows():
    """Busiest-rank KV read and attention work of every layout equal Table 2's
    formulas, evaluated at several (B, T)."""
    import math
    rows = json.load(open(GOLDEN))["rows"]
    s, H = 4096, 128
    for B, T in [(16, 8), (16, 4), (13, 4), (3, 8), (64, 8), (9, 2)]:
        env = {"B": B, "T": T, "ceil": math.ceil}
        for row in rows:
            layout = row["layout"]
            bs_kv = max(sh.kv_tokens for sh in lm.rank_shares(layout, B, T, s, H)) / s
            bs = lm.busiest_share(layout, B, T, s, H)
            work = bs.kv_tokens * bs.heads / (s * H)
            assert bs_kv == pytest.approx(eval(row["kv_read"], env)), (B, T, layout)
            assert work == pytest.approx(eval(row["attention_work"], env)), (B, T, layout)


def test_choose_picks_least_time():
    # a share costs its KV tokens plus a fixed 5 units (and 2 per merged part)
    def time_of(sh):
        return sh.kv_tokens * 1e-3 + 5.0 + (2.0 * sh.merge_parts if sh.merge_parts > 1 else 0.0)
    best, times = lm.choose(16, 8, 65536, 128, time_of)
    assert times["TP"] == pytest.approx(16 * 65536e-3 + 5.0)
    assert times["DP-attention"] == times["DOP"] == pytest.approx(2 * 65536e-3 + 5.0)
    assert times["CP"] == pytest.approx(16 * 8192e-3 + 5.0 + 16.0)
    assert best == "DP-attention"
    # with a heavy fixed cost per request, CP (fewer tokens, all requests) never wins here
    assert lm.choose(16, 8, 1024, 128, time_of)[0] == "DP-attention"


def test_bad_arguments():
    with pytest.raises(ValueError):
        lm.rank_shares("XP", 4, 2, 10, 8)
    with pytest.raises(ValueError):
        lm.rank_shares("TP", 4, 0, 10, 8)
