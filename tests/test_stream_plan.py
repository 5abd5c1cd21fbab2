"""The balanced split-KV plan, as arithmetic (CPU).

The decode kernel cuts a batch's tiles on the device: every request with
work is a run of a header (the cost of starting a segment, counted in tiles;
none when all lengths are equal) and its real tiles; the runs are cut into
ranges of L = ceil(TV / N) tiles, N = min(target, ceil(TV / 4)); a range
walks the requests its real tiles cover, writing whole requests directly
and a cut request's part into slot w (the range's first segment) or
target + w (its last).  The merge finds a request's parts from a record
{first range, last range, slot of the first part}.  This test restates that
arithmetic in Python and checks its invariants on thousands of batches: every
request's tiles are covered exactly once, every index stays in range, a
range holds at most two partial segments, and the records name exactly the
slots the segments write.  (The GPU parity tests run the kernel itself.)
"""
import math
import random

import numpy as np
import pytest

import workloads as W


def plan(tiles, header_cfg, target=256, min_chunk=4):
    nz = [t for t in tiles if t > 0]
    header = 0 if (not nz or min(nz) == max(nz)) else header_cfg
    nv = [t + header if t > 0 else 0 for t in tiles]
    incl = np.cumsum(nv).tolist()
    excl = [incl[i] - nv[i] for i in range(len(nv))]
    TV = incl[-1]
    N = min(-(-TV // min_chunk), target)
    L = -(-TV // N)
    N = -(-TV // L)
    segments = {}
    for w in range(N):
        A, E = w * L, min(w * L + L, TV)
        r = next(i for i in range(len(tiles)) if incl[i] > A)
        V, k, out = excl[r], 0, []
        while True:
            nt = 0
            while V < E and r < len(tiles):
                nt = tiles[r]
                if nt:
                    break
                r += 1
            R0 = V + header
            if V >= E or r >= len(tiles) or R0 >= E:
                break
            s0, s1 = max(A, R0), min(E, R0 + nt)
            out.append((r, s0 - R0, s1 - R0, s0 != R0 or s1 != R0 + nt, target + w if k else w))
            V, r, k = R0 + nt, r + 1, k + 1
        segments[w] = out
    records = []
    for i in range(len(tiles)):
        v0, v1 = excl[i], incl[i]
        if v1 == v0:
            records.append(("empty", []))
            continue
        wa, wb = (v0 + header) // L, (v1 - 1) // L
        if wa == wb:
            records.append(("direct", []))
        else:
            first = wa if wa * L >= v0 else target + wa
            records.append(("parts", [first] + [wa + p for p in range(1, wb - wa + 1)]))
    return segments, records


def batches():
    yield [math.ceil(n / 32) for n in W.loguniform_lengths(5, 64, 512, 65536)]   # the transition batch
    yield [math.ceil(150000 / 32), math.ceil(777 / 32), 0]                       # one long request
    yield [128] * 16                                                             # uniform: no header
    rng = random.Random(3)
    for _ in range(1500):
        B = rng.randint(1, 80)
        yield [rng.choice([0, 0, 1, 2, 3, 5, 17, 100, 1000, rng.randint(0, 5000)]) for _ in range(B)]


@pytest.mark.parametrize("header", [0, 5, 12, 32])
def test_plan_covers_every_tile_once_and_records_match(header):
    for tiles in batches():
        if sum(tiles) == 0:
            continue
        segments, records = plan(tiles, header)
        covered, wrote = {}, {}
        for w, segs in segments.items():
            assert sum(1 for s in segs if s[3]) <= 2           # at most two partial segments per range
            for (r, t0, t1, partial, slot) in segs:
                assert 0 <= r < len(tiles) and 0 <= t0 < t1 <= tiles[r]
                assert 0 <= slot < 2 * 256
                covered.setdefault(r, []).append((t0, t1))
                wrote.setdefault(r, []).append((partial, slot))
        for r, t in enumerate(tiles):
            iv = sorted(covered.get(r, []))
            assert sum(b - a for a, b in iv) == t
            assert all(iv[i][1] == iv[i + 1][0] for i in range(len(iv) - 1))
            kind, parts = records[r]
            if kind == "empty":
                assert r not in wrote
            elif kind == "direct":
                assert len(wrote[r]) == 1 and not wrote[r][0][0]
            else:
                assert all(p for p, _ in wrote[r])
                assert sorted(s for _, s in wrote[r]) == sorted(parts)


def test_uniform_batch_ranges_fall_on_request_boundaries():
    segments, records = plan([128] * 16, 12)
    assert all(len(s) == 1 and s[0][2] - s[0][1] == 8 for s in segments.values())
    assert all(kind == "parts" and len(parts) == 16 for kind, parts in records)


@pytest.mark.parametrize("target", [128, 85, 16])
def test_parts_in_range_order_and_no_slot_written_twice(target):
    """Fewer ranges (wider head groups take 256 / groups of them): the parts
    of a request come one per range, in range order, at the slots its record
    names in that order, and no slot is written by two segments."""
    rng = random.Random(target)
    for _ in range(800):
        tiles = [rng.choice([0, 1, 3, 17, 100, 1000, rng.randint(0, 5000)]) for _ in range(rng.randint(1, 70))]
        if sum(tiles) == 0:
            continue
        segments, records = plan(tiles, 12, target)
        slots, by_req = set(), {}
        for w in sorted(segments):
            segs = segments[w]
            for k, (r, t0, t1, partial, slot) in enumerate(segs):
                if partial:
                    assert k == 0 or k == len(segs) - 1      # only a range's ends are cut
                    assert slot not in slots
                    slots.add(slot)
                    by_req.setdefault(r, []).append(slot)
        for r, (kind, parts) in enumerate(records):
            assert by_req.get(r, []) == (parts if kind == "parts" else [])
