"""Forced split-KV chunks computed by several workgroups (CPU).

With num_splits = S > 1 every request's tiles are cut into S equal chunks;
while B x S x head groups is below the CU count, each chunk is computed by
`sub` workgroups over equal sub-ranges of its tiles (workgroup x takes
sub-range x % sub of chunk x / sub).  This test restates the kernel's index
arithmetic in Python and checks, for many tile counts, that the sub-ranges
of every request cover its tiles exactly once and stay inside their chunk,
and that the host's choice of `sub` (through splash_decode_plan) fills the
CUs without exceeding the chunk's tiles.  The GPU parity tests run the
kernel with these splits (the TP share with 8 chunks, forced 3 and 16).
"""
import pytest

import layout_agnostic_latent_amd as sp

CUS = 256


def subranges(nt, splits, sub, tf=0):
    """[t_begin, t_end) of every workgroup x < splits * sub of one request."""
    chunk = (nt + splits - 1) // splits
    out = []
    for x in range(splits * sub):
        c, k = divmod(x, sub)
        cb = tf + c * chunk
        ce = min(cb + chunk, tf + nt)
        s = (ce - cb + sub - 1) // sub if ce > cb else 0
        tb = cb + k * s
        te = min(tb + s, ce)
        out.append((c, tb, te, cb, ce))
    return out


@pytest.mark.parametrize("splits", [2, 3, 5, 8, 16])
@pytest.mark.parametrize("sub", [1, 2, 3, 4, 7])
def test_subranges_tile_every_request_once(splits, sub):
    for nt in list(range(0, 70)) + [127, 128, 129, 511, 512, 2048, 2049]:
        for tf in (0, 3):
            seen = []
            for c, tb, te, cb, ce in subranges(nt, splits, sub, tf):
                if te > tb:
                    assert cb <= tb and te <= ce, (nt, splits, sub, c)
                    seen.extend(range(tb, te))
            assert sorted(seen) == list(range(tf, tf + nt)), (nt, splits, sub, tf)


@pytest.mark.parametrize("B,heads,splits", [(16, 16, 8), (16, 128, 5), (2, 16, 4), (1, 16, 8), (64, 128, 2),
                                            (16, 128, 1), (300, 16, 8)])
def test_host_choice_of_workgroups_per_chunk(B, heads, splits):
    ctx = 16384
    s, groups, _ = sp.decode_plan(B, 128, 576, 512, 64, ctx // 64, B * (ctx // 64), 0.07, 0, heads, 0, ctx,
                                  num_splits=splits)
    tiles_per_chunk = -(-(ctx // 32) // splits)
    expect = 1 if splits == 1 else max(1, min(CUS // (B * splits * groups), tiles_per_chunk))
    assert s == splits * expect
    if splits > 1:
        assert B * s * groups <= max(CUS, B * splits * groups)


def test_head_groups_of_the_16_head_tile():
    # a 16-head slice is one head group of the 16-head tile; 24 heads take the
    # 32-head tile; G = 8 KV heads of 16 query heads each: 8 groups
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 16, 0, 4096)[1] == 1
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 24, 0, 4096)[1] == 1
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096, num_kv_heads=8)[1] == 8
    # a 16-head range straddling two KV heads of 16: one group on each
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 8, 24, 0, 4096, num_kv_heads=8)[1] == 2
