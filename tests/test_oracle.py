"""Pins for the CPU oracle (no GPU).

The oracle is checked against what the pages and the mathematics fix, never
against itself: closed forms (one-token context, equal scores), brute force in
pure Python and 50-digit mpmath on tiny inputs built from a dense logical
cache, invariants (page permutation, convex bounds, LSE bounds), the merge
identities, the layout invariance of the TP / CP / DP-attention shares, and the
busiest-rank loads printed in Appendix Table 2 of the SPLASH pages.

Each pin is a plain function of the implementation under test, so the same
pins also run against deliberately broken copies of the oracle (mutants
planted here, on the CPU) to show that a plausible mistake fails at least one
of them.
"""
import inspect
import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(bits):
    # Independent widening for the brute-force side: go through Python floats.
    return [float(np.frombuffer(np.array([int(b) << 16], dtype=np.uint32).tobytes(), dtype=np.float32)[0])
            for b in np.asarray(bits).ravel()]


def _small_case(seed=11, lens=(5, 33, 1, 64, 40), H=6, d_qk=24, d_v=16, ps=8, std=0.7, **kw):
    return W.make_decode_case("small", seed, list(lens), num_heads=H, d_qk=d_qk, d_v=d_v,
                              page_size=ps, scale=1.0 / math.sqrt(d_qk), std=std, extra_pages=3,
                              keep_dense=True, **kw)


def _run(decode, c, **over):
    args = dict(head_lo=c.head_lo, head_hi=c.head_hi, tok_lo=c.tok_lo, tok_hi=c.tok_hi)
    args.update(over)
    return decode(c.q, c.kv_pages, c.block_table, c.seq_lens, args["head_lo"], args["head_hi"],
                  args["tok_lo"], args["tok_hi"], c.d_v, c.page_size, c.scale,
                  **({"reqs": over["reqs"]} if "reqs" in over else {}))


# ---------------------------------------------------------------------------
# Pins.  Each raises AssertionError when the implementation is wrong.
# ---------------------------------------------------------------------------
def pin_one_token(decode, merge):
    """A one-token context returns that token's V exactly; LSE is its scaled score."""
    c = _small_case(seed=21, lens=(1, 9, 30))
    # request 0 has one token; requests 1, 2 get a one-token range [4, 5)
    for b, (lo, hi) in [(0, (0, 1)), (1, (4, 5)), (2, (29, 30))]:
        out, lse = _run(decode, c, tok_lo=lo, tok_hi=hi, reqs=[b])
        row = c.dense_kv[b][lo]
        v = np.array(_f64(row[:c.d_v]))
        k = _f64(row)
        for h in range(c.num_heads):
            assert np.array_equal(out[b, h], v), "one-token O must equal that token's V"
            qh = _f64(c.q[b, h])
            s = c.scale * math.fsum(x * y for x, y in zip(qh, k))
            assert abs(lse[b, h] - s) <= 1e-13 * max(1.0, abs(s)), (lse[b, h], s)


def pin_equal_scores(decode, merge):
    """Equal scores return the mean of V and LSE = s + ln n (q = 0, and rope-only q)."""
    c = _small_case(seed=22, lens=(7, 40))
    # (a) q = 0: every score is 0
    c.q[:] = 0
    out, lse = _run(decode, c)
    for b in range(c.num_reqs):
        n = int(c.seq_lens[b])
        V = [_f64(c.dense_kv[b][t][:c.d_v]) for t in range(n)]
        mean = [math.fsum(V[t][d] for t in range(n)) / n for d in range(c.d_v)]
        assert np.allclose(out[b], np.array(mean)[None, :], rtol=0, atol=1e-13)
        assert np.allclose(lse[b], math.log(n), rtol=0, atol=1e-13)
    # (b) q nonzero only on the rope dims, every token's rope slice equal:
    #     equal nonzero scores with distinct V.
    c = _small_case(seed=23, lens=(12, 64))
    rope = c.kv_pages[c.block_table[0, 0], 0, c.d_v:].copy()
    for b in range(c.num_reqs):
        n = int(c.seq_lens[b])
        for t in range(n):
            c.kv_pages[c.block_table[b, t // c.page_size], t % c.page_size, c.d_v:] = rope
            c.dense_kv[b][t, c.d_v:] = rope
    c.q[:, :, :c.d_v] = 0
    out, lse = _run(decode, c)
    r = _f64(rope)
    for b in range(c.num_reqs):
        n = int(c.seq_lens[b])
        V = [_f64(c.dense_kv[b][t][:c.d_v]) for t in range(n)]
        mean = np.array([math.fsum(V[t][d] for t in range(n)) / n for d in range(c.d_v)])
        for h in range(c.num_heads):
            s = c.scale * math.fsum(x * y for x, y in zip(_f64(c.q[b, h, c.d_v:]), r))
            assert np.allclose(out[b, h], mean, rtol=0, atol=1e-13)
            assert abs(lse[b, h] - (s + math.log(n))) <= 1e-12


def pin_brute_force(decode, merge):
    """Pure-Python fsum and 50-digit mpmath over the dense logical cache agree to 1e-12."""
    for c in (W.case_tiny(keep_dense=True), _small_case(seed=24)):
        out, lse = _run(decode, c)
        lo = max(c.tok_lo, 0)
        for b in range(c.num_reqs):
            hi = min(c.tok_hi, int(c.seq_lens[b]))
            K = [_f64(c.dense_kv[b][t]) for t in range(lo, hi)]
            for h in range(c.num_q_heads):
                qh = _f64(c.q[b, c.head_lo + h])
                with mpmath.workdps(50):
                    s = [mpmath.mpf(c.scale) * mpmath.fsum(mpmath.mpf(x) * y for x, y in zip(qh, k)) for k in K]
                    w = [mpmath.exp(x) for x in s]
                    Z = mpmath.fsum(w)
                    o = [mpmath.fsum(w[i] * K[i][d] for i in range(len(K))) / Z for d in range(c.d_v)]
                    L = mpmath.log(Z)
                assert abs(float(L) - lse[b, h]) <= 1e-12 * max(1.0, abs(float(L)))
                assert np.allclose(out[b, h], np.array([float(x) for x in o]), rtol=0, atol=1e-12)


def pin_brute_force_kv_heads(decode, merge):
    """G = 2 and G = 4 shared KV heads (query head h reads KV head h*G // H):
    50-digit mpmath over the dense logical cache, all heads and a head slice
    that crosses a group boundary."""
    for G, H, slice_ in ((2, 8, (0, 8)), (4, 8, (1, 6))):
        c = W.make_decode_case("gqa", 30 + G, [9, 1, 23], num_heads=H, d_qk=12, d_v=8, page_size=4,
                               scale=0.37, std=0.7, head_lo=slice_[0], head_hi=slice_[1], extra_pages=2,
                               keep_dense=True, num_kv_heads=G)
        out, lse = _run(decode, c)
        for b in range(c.num_reqs):
            n = int(c.seq_lens[b])
            for j, h in enumerate(range(c.head_lo, c.head_hi)):
                kvh = h * G // H
                K = [_f64(c.dense_kv[b][t][kvh]) for t in range(n)]
                qh = _f64(c.q[b, h])
                with mpmath.workdps(50):
                    sc = [mpmath.mpf(c.scale) * mpmath.fsum(mpmath.mpf(x) * y for x, y in zip(qh, k)) for k in K]
                    w = [mpmath.exp(x) for x in sc]
                    Z = mpmath.fsum(w)
                    o = [mpmath.fsum(w[i] * K[i][d] for i in range(n)) / Z for d in range(c.d_v)]
                    L = mpmath.log(Z)
                assert abs(float(L) - lse[b, j]) <= 1e-12 * max(1.0, abs(float(L)))
                assert np.allclose(out[b, j], np.array([float(x) for x in o]), rtol=0, atol=1e-12)


def pin_layout_invariance(decode, merge):
    """Head slices (TP), token ranges + merge (CP) and request subsets (DP / DOP) equal the whole."""
    c = _small_case(seed=25, lens=(5, 33, 1, 64, 40, 17), H=8)
    full_o, full_l = _run(decode, c)
    # TP: uneven head slices, concatenated
    cuts = [0, 3, 4, 8]
    parts = [_run(decode, c, head_lo=a, head_hi=b) for a, b in zip(cuts, cuts[1:])]
    assert np.allclose(np.concatenate([p[0] for p in parts], axis=1), full_o, rtol=0, atol=1e-12)
    assert np.allclose(np.concatenate([p[1] for p in parts], axis=1), full_l, rtol=0, atol=1e-12)
    # CP: T token ranges (ragged requests: some ranges are empty for short requests), merged
    for T in (2, 4, 7):
        s = int(c.seq_lens.max())
        bounds = [r * s // T for r in range(T + 1)]
        po, pl = zip(*[_run(decode, c, tok_lo=a, tok_hi=b) for a, b in zip(bounds, bounds[1:])])
        B, Hs, dv = full_o.shape
        mo, ml = merge(np.stack(po).reshape(T, B * Hs, dv), np.stack(pl).reshape(T, B * Hs))
        assert np.allclose(mo.reshape(B, Hs, dv), full_o, rtol=0, atol=1e-12)
        assert np.allclose(ml.reshape(B, Hs), full_l, rtol=0, atol=1e-12)
    # DP-attention / DOP: request subsets dealt by count
    for T in (2, 3):
        got_o = np.zeros_like(full_o)
        got_l = np.full_like(full_l, -np.inf)
        for r in range(T):
            mine = [b for b in range(c.num_reqs) if b % T == r]
            o, l = _run(decode, c, reqs=mine)
            got_o[mine], got_l[mine] = o[mine], l[mine]
        assert np.array_equal(got_o, full_o) and np.array_equal(got_l, full_l)


def pin_page_permutation(decode, merge):
    """Moving physical pages (and updating the table) changes nothing."""
    c = _small_case(seed=26)
    o1, l1 = _run(decode, c)
    rng = np.random.default_rng(5)
    perm = rng.permutation(c.num_pages)          # new position of old page p is perm[p]
    new_pool = np.empty_like(c.kv_pages)
    new_pool[perm] = c.kv_pages
    new_table = np.where(c.block_table >= 0, perm[np.maximum(c.block_table, 0)], -1).astype(np.int32)
    c.kv_pages, c.block_table = new_pool, new_table
    o2, l2 = _run(decode, c)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_bounds(decode, merge):
    """O is a convex combination of V; max s <= LSE <= max s + ln n."""
    c = _small_case(seed=27, std=2.0)
    out, lse = _run(decode, c)
    for b in range(c.num_reqs):
        n = int(c.seq_lens[b])
        V = np.array([_f64(c.dense_kv[b][t][:c.d_v]) for t in range(n)])
        K = np.array([_f64(c.dense_kv[b][t]) for t in range(n)])
        assert np.all(out[b] >= V.min(axis=0) - 1e-12) and np.all(out[b] <= V.max(axis=0) + 1e-12)
        for h in range(c.num_heads):
            qh = np.array(_f64(c.q[b, h]))
            smax = max(c.scale * math.fsum(qh * k) for k in K)
            assert smax - 1e-12 <= lse[b, h] <= smax + math.log(n) + 1e-12


def pin_empty_range(decode, merge):
    """An empty clipped range gives O = 0 and LSE = -inf."""
    c = _small_case(seed=28, lens=(5, 33))
    out, lse = _run(decode, c, tok_lo=10, tok_hi=20)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))
    out, lse = _run(decode, c, tok_lo=40, tok_hi=40)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def pin_merge_identities(decode, merge):
    """Merge: identity, arithmetic mean, shift, empty parts, and a two-part closed form."""
    rng = np.random.default_rng(3)
    O = rng.standard_normal((4, 10, 6))
    L = rng.uniform(-5, 5, (4, 10))
    o1, l1 = merge(O[:1], L[:1])
    assert np.array_equal(o1, O[0]) and np.array_equal(l1, L[0])
    Leq = np.repeat(L[:1], 4, axis=0)
    o, l = merge(O, Leq)
    assert np.allclose(o, O.mean(axis=0), rtol=0, atol=1e-14)
    assert np.allclose(l, L[0] + math.log(4), rtol=0, atol=1e-13)
    oa, la = merge(O, L)
    ob, lb = merge(O, L + 2.5)
    assert np.allclose(oa, ob, rtol=0, atol=1e-13) and np.allclose(lb, la + 2.5, rtol=0, atol=1e-13)
    Lm = L.copy()
    Lm[1] = -np.inf
    Om = O.copy()
    Om[1] = np.nan
    oc, lc = merge(Om, Lm)
    od, ld = merge(O[[0, 2, 3]], L[[0, 2, 3]])
    assert np.allclose(oc, od, rtol=0, atol=1e-14) and np.allclose(lc, ld, rtol=0, atol=1e-14)
    oe, le = merge(O[:2], np.full((2, 10), -np.inf))
    assert np.all(oe == 0) and np.all(np.isneginf(le))
    # two parts with LSE 0 and ln 3: weights 1/4 and 3/4, merged LSE ln 4
    o2, l2 = merge(np.array([[[1.0, 0.0]], [[0.0, 1.0]]]), np.array([[0.0], [math.log(3.0)]]))
    assert np.allclose(o2, [[0.25, 0.75]], rtol=0, atol=1e-15)
    assert abs(l2[0] - math.log(4.0)) <= 1e-15


ALL_PINS = [pin_one_token, pin_equal_scores, pin_brute_force, pin_brute_force_kv_heads, pin_layout_invariance,
            pin_page_permutation, pin_bounds, pin_empty_range, pin_merge_identities]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin):
    pin(oracle.decode_attn, oracle.lse_merge)


# ---------------------------------------------------------------------------
# Mutants: plausible mistakes planted in copies of the oracle.  Each must fail
# at least one pin.
# ---------------------------------------------------------------------------
DECODE_MUTANTS = {
    "dropped scale": ("scale * (Q @ K.T)", "(Q @ K.T)"),
    "V from the rope end": ("V = K[:, :d_v]", "V = K[:, -d_v:]"),
    "wrong page slot": ("rows = kv_pages[pages, t % page_size]", "rows = kv_pages[pages, (t + 1) % page_size]"),
    "wrong page index": ("block_table[b, t // page_size]", "block_table[b, (t + 1) // page_size]"),
    "LSE without the max": ("(m + np.log(denom))", "(np.log(denom))"),
    "sign of the max shift": ("np.exp(S - m)", "np.exp(m - S)"),
    "range off by one": ("lo = max(int(tok_lo), 0)", "lo = max(int(tok_lo) + 1, 0)"),
    "range end off by one": ("hi = min(int(tok_hi), int(seq_lens[b]))", "hi = min(int(tok_hi), int(seq_lens[b])) - 1"),
    "transposed operand": ("(Q @ K.T)", "(Q[:, ::-1] @ K.T)"),
    "no normalisation": ("(W @ V) / denom", "(W @ V)"),
    "one KV head for every group": ("rows[:, g, :d_qk]", "rows[:, 0, :d_qk]"),
    "KV heads in reverse": ("rows[:, g, :d_qk]", "rows[:, G - 1 - g, :d_qk]"),
    "group boundary off by one": ("max(head_lo, g * group), min(head_hi, (g + 1) * group)",
                                  "max(head_lo, g * group + 1), min(head_hi, (g + 1) * group + 1)"),
}
MERGE_MUTANTS = {
    "merged LSE sign": ("M_safe + np.log(s_safe)", "M_safe - np.log(s_safe)"),
    "weight sign": ("- M_safe[None, :]), 0.0)", "+ M_safe[None, :]), 0.0)"),
    "no normalisation": ("/ s_safe[:, None]", "/ 1.0"),
    "empty parts counted": ("live = np.isfinite(L)", "live = np.isfinite(L) | True"),
}


def _mutate(fn, old, new):
    src = inspect.getsource(fn)
    assert old in src, f"mutation anchor not found: {old!r}"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[fn.__name__]


def _fails_some_pin(decode, merge):
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(decode, merge)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_mutant_is_caught(name):
    old, new = DECODE_MUTANTS[name]
    assert _fails_some_pin(_mutate(oracle.decode_attn, old, new), oracle.lse_merge), name


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_mutant_is_caught(name):
    old, new = MERGE_MUTANTS[name]
    assert _fails_some_pin(oracle.decode_attn, _mutate(oracle.lse_merge, old, new)), name


# ---------------------------------------------------------------------------
# Appendix Table 2: busiest-rank loads of the layout shares.
# ---------------------------------------------------------------------------
def _eval_table_expr(expr, B, T):
    return {"B": B, "B/T": B / T, "ceil(B/T)": math.ceil(B / T)}[expr]


@pytest.mark.parametrize("B,T", [(16, 8), (17, 8), (5, 8), (8, 2), (16, 4), (3, 3), (64, 8)])
def test_table2_busiest_rank_loads(B, T):
    with open(os.path.join(GOLDEN, "table2_loads.json")) as f:
        table = json.load(f)
    s, H = 64 * T, 16 * T
    for row in table["rows"]:
        load = oracle.busiest_rank_load(oracle.layout_shares(row["layout"], B, T, s, H), s, H)
        assert load["kv_read"] == pytest.approx(_eval_table_expr(row["kv_read"], B, T), abs=1e-12)
        assert load["attention_work"] == pytest.approx(_eval_table_expr(row["attention_work"], B, T), abs=1e-12)
        # Every row of the table stores exactly what it reads.
        assert row["kv_stored"] == row["kv_read"]
        if B % T == 0 and "ceil" in row["kv_read"]:
            assert math.ceil(B / T) == B / T   # the caption's "owner entries equal B/T"


def test_layout_shares_cover_the_work_once():
    """Every layout's shares together cover each (request, head, token) exactly once."""
    B, T, s, H = 5, 4, 32, 8
    for layout in ("TP", "CP", "DP-attention", "DOP"):
        cover = np.zeros((B, H, s), dtype=int)
        for sh in oracle.layout_shares(layout, B, T, s, H):
            for b in sh["reqs"]:
                cover[b, sh["heads"][0]:sh["heads"][1], sh["toks"][0]:sh["toks"][1]] += 1
        assert np.all(cover == 1), layout


# ---------------------------------------------------------------------------
# Repack: bytes.
# ---------------------------------------------------------------------------
def test_repack_bytes_and_round_trip():
    c = _small_case(seed=29)
    rc = W.make_repack_case(c, seed=30)
    dst0 = np.full((rc.dst_num_pages,) + c.kv_pages.shape[1:], rc.dst_fill, dtype=np.uint16)
    dst, copied, rejected = oracle.kv_repack(c.kv_pages, rc.src_table, dst0, rc.dst_table)
    assert rejected == 0 and copied == int((rc.src_table >= 0).sum()) == rc.dst_num_pages
    for i, b in enumerate(rc.moved_reqs):
        n = int(c.seq_lens[b])
        for t in range(n):
            got = dst[rc.dst_table[i, t // c.page_size], t % c.page_size]
            assert np.array_equal(got, c.dense_kv[b][t])
    back = np.zeros_like(c.kv_pages)
    back2, _, _ = oracle.kv_repack(dst, rc.dst_table, back, rc.src_table)
    moved_pages = rc.src_table[rc.src_table >= 0]
    assert np.array_equal(back2[moved_pages], c.kv_pages[moved_pages])


def test_repack_rejects_mismatched_pairs():
    src = np.arange(4 * 3, dtype=np.uint16).reshape(4, 3)
    dst = np.zeros((4, 3), dtype=np.uint16)
    out, copied, rejected = oracle.kv_repack(src, np.array([[0, -1, 2, -1, 9]]), dst,
                                             np.array([[3, 1, -1, -1, 0]]))
    assert copied == 1 and rejected == 3
    assert np.array_equal(out[3], src[0]) and np.all(out[:3] == 0)
