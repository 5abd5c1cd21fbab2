"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Every case uses the seeded generators of ``workloads``.  Bars: attention
output max abs <= 1e-2 and relative L2 <= 5e-3, LSE abs <= 1e-3; repack
bit-exact.  Unused KV slots and unreferenced pages hold NaN, so any unmasked
read shows up as a non-finite output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_close, run_decode, run_oracle, to_dev

import layout_agnostic_latent_amd as sp

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _clean_device_errors():
    sp.device_errors(clear=True)
    yield
    assert sp.device_errors(clear=True) == 0, "a kernel raised a device error bit"


# ---------------------------------------------------------------------------
# tiny: B=2, lens 17/64, H=8, d_qk 80, d_v 64, page 16
# ---------------------------------------------------------------------------
def test_tiny_full():
    c = W.case_tiny()
    _print("case tiny")
    go, gl = run_decode(c)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what="tiny")


@pytest.mark.parametrize("splits", [1, 2, 3, 5])
def test_tiny_forced_splits(splits):
    c = W.case_tiny()
    go, gl = run_decode(c, num_splits=splits)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what=f"tiny splits={splits}")


@pytest.mark.parametrize("heads,toks", [((0, 8), (0, 64)), ((3, 5), (0, 64)), ((0, 8), (5, 40)),
                                        ((7, 8), (16, 17)), ((0, 8), (-7, 3)), ((1, 6), (17, 64)),
                                        ((0, 8), (40, 1000)), ((0, 8), (64, 80))])
def test_tiny_shares(heads, toks):
    c = W.case_tiny()
    go, gl = run_decode(c, head_lo=heads[0], head_hi=heads[1], tok_lo=toks[0], tok_hi=toks[1])
    ro, rl = run_oracle(c, head_lo=heads[0], head_hi=heads[1], tok_lo=toks[0], tok_hi=toks[1])
    assert_close(go, gl, ro, rl, what=f"tiny heads={heads} toks={toks}")


def test_tiny_without_lse():
    c = W.case_tiny()
    go, _ = run_decode(c, with_lse=False)
    ro, rl = run_oracle(c)
    assert_close(go, None, ro, rl, what="tiny no-lse")


# ---------------------------------------------------------------------------
# request-owned share (DP-attention / DOP owner): B=16 x 4,096, 128 heads
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def owner():
    c = W.case_owner()
    return c, to_dev(c), run_oracle(c)


@pytest.mark.parametrize("splits", [0, 1, 4, 16])
def test_owner(owner, splits):
    c, t, (ro, rl) = owner
    _print(f"case owner splits={splits}")
    go, gl = run_decode(c, t, num_splits=splits)
    err, rel = assert_close(go, gl, ro, rl, what=f"owner splits={splits}")
    _print(f"  max abs {err:.2e} rel L2 {rel:.2e}")


def test_owner_deterministic(owner):
    c, t, _ = owner
    a = run_decode(c, t)
    b = run_decode(c, t)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_split_calls_on_two_streams(owner):
    """Split-KV calls on two streams at once, over different data: each
    stream has its own workspace, so neither call's merge reads the other's
    partials (both shares cut into the same 256 ranges and partial slots)."""
    c, t, (ro, rl) = owner
    c2 = W.make_decode_case("owner2", 77, [4096] * 16, num_heads=128, d_qk=576, d_v=512, page_size=64,
                            scale=W.LATENT_SCALE)
    t2 = to_dev(c2)
    ro2, rl2 = run_oracle(c2)
    _print("case owner on two streams")
    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    outs = [torch.full((16, 128, 512), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
    lses = [torch.full((16, 128), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(4):
        for k, (cc, tt) in enumerate(((c, t), (c2, t2))):
            sp.decode_attn(tt["q"], tt["kv"], tt["bt"], tt["sl"], 0, 128, 0, 1 << 30, outs[k], lses[k],
                           d_v=cc.d_v, scale=cc.scale, stream=streams[k])
    torch.cuda.synchronize()
    for k, (o, l) in enumerate(((ro, rl), (ro2, rl2))):
        assert_close(outs[k].cpu().double().numpy(), lses[k].cpu().double().numpy(), o, l, what=f"stream {k}")


def test_owner_request_subsets(owner):
    """DP-attention / DOP: each owner's call over its own requests equals the batch."""
    c, t, (ro, rl) = owner
    T = 3
    for r in range(T):
        mine = [b for b in range(c.num_reqs) if b % T == r]
        idx = torch.tensor(mine, device=DEV)
        sub = dict(q=t["q"][idx].contiguous(), kv=t["kv"], bt=t["bt"][idx].contiguous(), sl=t["sl"][idx].contiguous())
        hs = c.num_q_heads
        out = torch.empty((len(mine), hs, c.d_v), dtype=torch.float32, device=DEV)
        lse = torch.empty((len(mine), hs), dtype=torch.float32, device=DEV)
        sp.decode_attn(sub["q"], sub["kv"], sub["bt"], sub["sl"], 0, hs, 0, c.tok_hi, out, lse,
                       d_v=c.d_v, scale=c.scale)
        torch.cuda.synchronize()
        assert_close(out.cpu().double().numpy(), lse.cpu().double().numpy(), ro[mine], rl[mine],
                     what=f"owner rank {r}")


def test_owner_head_slices_concat(owner):
    """TP: eight 16-head slices, concatenated, equal the all-head result."""
    c, t, (ro, rl) = owner
    outs, lses = [], []
    for r in range(8):
        go, gl = run_decode(c, t, head_lo=16 * r, head_hi=16 * (r + 1))
        outs.append(go)
        lses.append(gl)
    assert_close(np.concatenate(outs, axis=1), np.concatenate(lses, axis=1), ro, rl, what="owner TP slices")


# ---------------------------------------------------------------------------
# head-sliced share (TP rank): B=16 x 16,384, heads [0,16) of 128
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def tp():
    c = W.case_tp()
    return c, to_dev(c), run_oracle(c)


def test_tp_one_call_eight_splits(tp):
    c, t, (ro, rl) = tp
    _print("case tp splits=8")
    go, gl = run_decode(c, t, num_splits=8)
    assert_close(go, gl, ro, rl, what="tp 8 splits")


def test_tp_auto_plan(tp):
    c, t, (ro, rl) = tp
    go, gl = run_decode(c, t)
    assert_close(go, gl, ro, rl, what="tp auto")


def test_tp_eight_ranges_then_merge(tp):
    c, t, (ro, rl) = tp
    s = int(c.seq_lens.max())
    hs = c.num_q_heads
    P = torch.empty((8, c.num_reqs * hs, c.d_v), dtype=torch.float32, device=DEV)
    L = torch.empty((8, c.num_reqs * hs), dtype=torch.float32, device=DEV)
    for r in range(8):
        lo, hi = r * s // 8, (r + 1) * s // 8
        sp.decode_attn(t["q"], t["kv"], t["bt"], t["sl"], c.head_lo, c.head_hi, lo, hi,
                       P[r].view(c.num_reqs, hs, c.d_v), L[r].view(c.num_reqs, hs), d_v=c.d_v, scale=c.scale)
    out = torch.empty((c.num_reqs * hs, c.d_v), dtype=torch.float32, device=DEV)
    lse = torch.empty((c.num_reqs * hs,), dtype=torch.float32, device=DEV)
    sp.lse_merge(P, L, out, lse)
    torch.cuda.synchronize()
    assert_close(out.cpu().double().numpy().reshape(ro.shape), lse.cpu().double().numpy().reshape(rl.shape),
                 ro, rl, what="tp ranges+merge")


# ---------------------------------------------------------------------------
# token-split share (CP rank 3 of 8): B=16 x 65,536, tokens [24,576, 32,768)
# ---------------------------------------------------------------------------
def test_cp_rank_share():
    c = W.case_cp()   # pages outside the range hold NaN
    _print("case cp rank share")
    t = to_dev(c)
    go, gl = run_decode(c, t)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what="cp share")
    del t
    torch.cuda.empty_cache()


def test_cp_merge_seeded_sets():
    m = W.case_cp_merge()
    P = torch.from_numpy(m.partials).to(DEV)
    L = torch.from_numpy(m.lses).to(DEV)
    rows, d_v = m.partials.shape[1:]
    out = torch.empty((rows, d_v), dtype=torch.float32, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    sp.lse_merge(P, L, out, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(m.partials, m.lses)
    assert_close(out.cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, what="cp merge")


def test_cp_eight_ranks_merge_equals_unsplit():
    """CP: the 8 ranks' partials, merged, equal the unsplit 65,536-token result (2 requests)."""
    c = W.case_cp(B=2, live_only_in_range=False)
    t = to_dev(c)
    s = 65536
    hs = c.num_q_heads
    P = torch.empty((8, c.num_reqs * hs, c.d_v), dtype=torch.float32, device=DEV)
    L = torch.empty((8, c.num_reqs * hs), dtype=torch.float32, device=DEV)
    for r in range(8):
        sp.decode_attn(t["q"], t["kv"], t["bt"], t["sl"], 0, hs, r * s // 8, (r + 1) * s // 8,
                       P[r].view(c.num_reqs, hs, c.d_v), L[r].view(c.num_reqs, hs), d_v=c.d_v, scale=c.scale)
    out = torch.empty((c.num_reqs * hs, c.d_v), dtype=torch.float32, device=DEV)
    lse = torch.empty((c.num_reqs * hs,), dtype=torch.float32, device=DEV)
    sp.lse_merge(P, L, out, lse)
    torch.cuda.synchronize()
    ro, rl = run_oracle(c, tok_lo=0, tok_hi=s)
    assert_close(out.cpu().double().numpy().reshape(ro.shape), lse.cpu().double().numpy().reshape(rl.shape),
                 ro, rl, what="cp 8 ranks merged")
    go, gl = run_decode(c, t, tok_lo=0, tok_hi=s)
    assert_close(go, gl, ro, rl, what="cp unsplit")
    del t
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# transition batch: 64 ragged requests, 128 heads; repack of 32 requests
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def transition():
    c = W.case_transition()
    _print("oracle: transition batch, all 64 requests")
    return c, to_dev(c), run_oracle(c)


def test_transition_decode(transition):
    """Every request of the ragged batch, every head, element by element."""
    c, t, (ro, rl) = transition
    _print("case transition decode")
    go, gl = run_decode(c, t)
    assert_close(go, gl, ro, rl, what="transition all 64 requests")
    # and per request, so that one request's error cannot hide in the batch's norm
    for b in range(c.num_reqs):
        assert_close(go[b:b + 1], gl[b:b + 1], ro[b:b + 1], rl[b:b + 1], what=f"transition request {b}",
                     quiet=True)


def _ranges(tiles, target=256, min_chunk=4):
    """The device plan's cut of a batch's tiles: N equal contiguous ranges."""
    T = sum(tiles)
    N = min(target, -(-T // min_chunk))
    return T, N, [w * T // N for w in range(N + 1)]


def test_ragged_batch_packed_ranges():
    """A ragged batch of 64 requests cut into equal ranges of the batch's
    tiles: ranges that hold several whole requests (written directly), and
    requests spread over several ranges (merged); 8 heads of d_qk 80 keep the
    oracle cheap.  Every request is compared."""
    lens = W.loguniform_lengths(71, 64, 40, 9000)
    tiles = [(int(n) + 31) // 32 for n in lens]
    T, N, cut = _ranges(tiles)
    starts = np.concatenate([[0], np.cumsum(tiles)])
    per_range = [int(np.sum((starts[:-1] >= cut[w]) & (starts[1:] <= cut[w + 1]))) for w in range(N)]
    spans = [int(np.searchsorted(cut, starts[r + 1], side="left") - np.searchsorted(cut, starts[r], side="right") + 1)
             for r in range(len(tiles))]
    assert max(per_range) >= 2 and max(spans) >= 3
    c = W.make_decode_case("ragged80", 72, lens, num_heads=8, d_qk=80, d_v=64, page_size=16,
                           scale=1.0 / math.sqrt(80.0), std=0.5, extra_pages=4)
    _print(f"case ragged d_qk 80: 64 requests, {T} tiles in {N} ranges; up to {max(per_range)} whole requests "
           f"in a range, up to {max(spans)} ranges per request")
    go, gl = run_decode(c)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what="ragged d_qk 80, packed ranges")
    for b in range(c.num_reqs):
        assert_close(go[b:b + 1], gl[b:b + 1], ro[b:b + 1], rl[b:b + 1], what=f"ragged80 request {b}", quiet=True)


def test_transition_repack_bit_exact(transition):
    c, t, _ = transition
    _print("case transition repack")
    rc = W.make_repack_case(c, seed=5)
    fill = int(np.int16(np.uint16(rc.dst_fill).view(np.int16)))
    dst = torch.full((rc.dst_num_pages,) + c.kv_pages.shape[1:], fill, dtype=torch.int16, device=DEV)
    errs = torch.zeros((1,), dtype=torch.int32, device=DEV)
    sp.kv_repack(t["kv"], torch.from_numpy(rc.src_table).to(DEV), dst, torch.from_numpy(rc.dst_table).to(DEV), errs)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16)
    want, copied, rejected = oracle.kv_repack(
        c.kv_pages, rc.src_table, np.full((rc.dst_num_pages,) + c.kv_pages.shape[1:], rc.dst_fill, np.uint16),
        rc.dst_table)
    assert int(errs.item()) == rejected == 0
    assert np.array_equal(got, want), "repack not bit-exact"
    moved_tokens = int(c.seq_lens[rc.moved_reqs].sum())
    _print(f"  moved {copied} pages, {moved_tokens} tokens, {copied * c.kv_pages[0].nbytes / 1e9:.3f} GB")
    # round trip back into a fresh pool at the source positions
    back = torch.zeros_like(t["kv"])
    sp.kv_repack(dst, torch.from_numpy(rc.dst_table).to(DEV), back, torch.from_numpy(rc.src_table).to(DEV))
    torch.cuda.synchronize()
    moved = rc.src_table[rc.src_table >= 0]
    assert torch.equal(back[torch.from_numpy(moved).long().to(DEV)], t["kv"][torch.from_numpy(moved).long().to(DEV)])


@pytest.mark.parametrize("G,heads,splits", [(2, (0, 128), 0), (4, (0, 128), 0), (8, (0, 128), 0),
                                            (4, (20, 70), 0), (8, (8, 40), 3), (2, (0, 128), 5)])
def test_few_kv_heads(G, heads, splits):
    """G shared latent KV heads (query head h reads KV head h // (H/G)): one
    launch serves every KV head the share touches, each workgroup reading its
    KV head's rows of the pool."""
    c = W.make_decode_case(f"gqa{G}", 50 + G, [700, 1500, 33, 2100], num_heads=128, d_qk=576, d_v=512,
                           page_size=64, scale=W.LATENT_SCALE, head_lo=heads[0], head_hi=heads[1],
                           extra_pages=3, num_kv_heads=G)
    _print(f"case few KV heads G={G} heads={heads} splits={splits}")
    go, gl = run_decode(c, num_splits=splits)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what=f"G={G} heads={heads}")


def test_few_kv_heads_tiny():
    c = W.make_decode_case("gqa_tiny", 60, [17, 64, 5], num_heads=8, d_qk=80, d_v=64, page_size=16,
                           scale=1.0 / math.sqrt(80.0), std=0.5, head_lo=1, head_hi=7, extra_pages=2, num_kv_heads=2)
    _print("case few KV heads tiny")
    go, gl = run_decode(c)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what="tiny G=2")


def test_background_handoff_concurrent(transition):
    """Decode on one stream while the repack runs in slices on a second
    stream (both default priority), reading the same KV pool: the decode
    output still matches the oracle and every moved page is exact."""
    c, t, (ro, rl) = transition
    _print("case transition handoff on two streams")
    rc = W.make_repack_case(c, seed=6)
    dst = torch.zeros((rc.dst_num_pages,) + c.kv_pages.shape[1:], dtype=torch.int16, device=DEV)
    errs = torch.zeros((1,), dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream(device=DEV)
    main = torch.cuda.current_stream(DEV)
    out = torch.full((c.num_reqs, c.num_q_heads, c.d_v), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((c.num_reqs, c.num_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    rows = np.array_split(np.arange(rc.src_table.shape[0]), 4)
    for r in rows:
        sp.decode_attn(t["q"], t["kv"], t["bt"], t["sl"], 0, c.num_q_heads, 0, 1 << 30, out, lse,
                       d_v=c.d_v, scale=c.scale, stream=main)
        sp.kv_repack(t["kv"], torch.from_numpy(np.ascontiguousarray(rc.src_table[r])).to(DEV), dst,
                     torch.from_numpy(np.ascontiguousarray(rc.dst_table[r])).to(DEV), errs, stream=side)
    torch.cuda.synchronize()
    assert int(errs.item()) == 0
    got = dst.cpu().numpy().view(np.uint16)
    want, copied, rejected = oracle.kv_repack(c.kv_pages, rc.src_table,
                                              np.zeros((rc.dst_num_pages,) + c.kv_pages.shape[1:], np.uint16),
                                              rc.dst_table)
    assert rejected == 0 and np.array_equal(got, want), "repack on the side stream not bit-exact"
    go, gl = out.cpu().double().numpy(), lse.cpu().double().numpy()
    assert_close(go, gl, ro, rl, what="decode during handoff, all 64 requests")
    for b in range(c.num_reqs):
        assert_close(go[b:b + 1], gl[b:b + 1], ro[b:b + 1], rl[b:b + 1], what=f"handoff request {b}", quiet=True)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_many_ragged_requests():
    """1,100 requests (more than one planner pass over the batch), lengths 0..400
    against a 4,800-token capacity, so the chunks are cut on the device."""
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 401, size=1100)
    lens[::97] = 0
    c = W.make_decode_case("many", 41, lens, num_heads=8, d_qk=80, d_v=64, page_size=16,
                           scale=1.0 / np.sqrt(80.0), std=0.5, max_pages_per_req=300)
    _print("case many ragged requests")
    go, gl = run_decode(c)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what="many ragged")


@pytest.mark.parametrize("heads", [(0, 128), (48, 64)])
def test_more_than_64_ragged_latent_requests(heads):
    """100 ragged 576-dim requests: the plan is made by the workgroup, not by
    each wave (which covers at most 64 requests), for the 128-head tile and
    for the 16-head tile."""
    rng = np.random.default_rng(78)
    lens = rng.integers(0, 3001, size=100)
    lens[::17] = 0
    c = W.make_decode_case("many576", 49, lens, num_heads=128, d_qk=576, d_v=512, page_size=64,
                           scale=W.LATENT_SCALE, head_lo=heads[0], head_hi=heads[1])
    _print(f"case 100 ragged latent requests heads={heads}")
    go, gl = run_decode(c)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what=f"100 ragged latent requests, heads {heads}")


def test_one_long_request_many_chunks():
    """A 150,000-token request next to a short and an empty one: about 250
    device-planned chunks of one request, merged by its own part list."""
    c = W.make_decode_case("long1", 42, [150000, 777, 0], num_heads=128, d_qk=576, d_v=512, page_size=64,
                           scale=W.LATENT_SCALE, head_lo=0, head_hi=16)
    _print("case one long request")
    go, gl = run_decode(c)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what="long request")


@pytest.mark.parametrize("n_tok,ps,heads", [(40000, 64, (0, 128)), (70000, 16, (0, 128)), (40000, 64, (0, 32)),
                                             (40000, 64, (0, 64)), (70000, 16, (16, 32))])
def test_unsplit_long_chunks(n_tok, ps, heads):
    """One chunk per request (num_splits = 1) longer than the 128-head tile's
    address table holds: the page ids come from LDS (up to 4,096 pages) or
    through the scalar cache (more, and in the 64- and 32-head variants,
    whose LDS holds the score exchange); the 16-head tile likewise."""
    c = W.make_decode_case("longchunk", 95 + ps, [n_tok, 333], num_heads=128, d_qk=576, d_v=512, page_size=ps,
                           scale=W.LATENT_SCALE, head_lo=heads[0], head_hi=heads[1])
    _print(f"case unsplit long chunk tokens={n_tok} page={ps} heads={heads}")
    go, gl = run_decode(c, num_splits=1)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what=f"unsplit {n_tok} tokens, page {ps}, heads {heads}")


def test_ragged_edges():
    """Zero-length, one-token, unaligned and page-straddling requests in one batch."""
    lens = [0, 1, 31, 32, 33, 63, 64, 65, 200, 1000]
    c = W.make_decode_case("edges", 40, lens, num_heads=128, d_qk=576, d_v=512, page_size=64,
                           scale=W.LATENT_SCALE, extra_pages=5, max_pages_per_req=20)
    t = to_dev(c)
    for toks in [(0, 1 << 30), (5, 70), (31, 33), (64, 65), (-3, 2), (999, 1 << 20), (2000, 3000)]:
        for splits in (0, 1, 3):
            go, gl = run_decode(c, t, tok_lo=toks[0], tok_hi=toks[1], num_splits=splits)
            ro, rl = run_oracle(c, tok_lo=toks[0], tok_hi=toks[1])
            assert_close(go, gl, ro, rl, what=f"edges toks={toks} splits={splits}")


@pytest.mark.parametrize("heads", [(0, 1), (5, 37), (0, 64), (64, 128), (1, 100), (0, 128)])
def test_head_ranges(heads):
    c = W.make_decode_case("heads", 41, [300, 77, 1025], num_heads=128, d_qk=576, d_v=512, page_size=64,
                           scale=W.LATENT_SCALE)
    go, gl = run_decode(c, head_lo=heads[0], head_hi=heads[1])
    ro, rl = run_oracle(c, head_lo=heads[0], head_hi=heads[1])
    assert_close(go, gl, ro, rl, what=f"heads={heads}")


@pytest.mark.parametrize("tok_lo", [16, 48, 80, 17])
def test_page16_range_starting_mid_tile(tok_lo):
    """Page size 16 with a token range that starts in the second half of a
    32-token tile: the block-table entries before the range are -1 (a rank
    that does not hold those pages) and must not be read, so no bad-page bit
    is raised (the autouse fixture checks the device error word)."""
    c = W.make_decode_case("p16mid", 46, [300, 129, 96], num_heads=8, d_qk=80, d_v=64, page_size=16,
                           scale=1.0 / math.sqrt(80.0), std=0.5, tok_lo=tok_lo, tok_hi=1000,
                           live_only_in_range=True, extra_pages=2)
    bt = c.block_table.copy()
    bt[:, :tok_lo // 16] = -1
    c2 = W.DecodeCase(**{**c.__dict__, "block_table": bt})
    for splits in (0, 1, 2):
        go, gl = run_decode(c2, num_splits=splits)
        ro, rl = run_oracle(c2)
        assert_close(go, gl, ro, rl, what=f"page 16, tok_lo {tok_lo}, splits {splits}")


@pytest.mark.parametrize("ps", [16, 32, 64, 128, 256])
def test_head16_tile_pages_ranges_and_groups(ps):
    """Shares of at most 16 heads run on the 16x16x32 tile: page sizes 16 to
    256; a token range starting in the second half of a 32-token tile with
    the block-table entries before it -1 (never read: the autouse fixture
    checks that no bad-page bit is set); full, partial (8 and 12 heads) and
    KV-head-crossing head groups; unsplit, forced and planned splits."""
    tok_lo = 48 if ps == 16 else 3 * ps // 2
    c = W.make_decode_case("h16", 47 + ps, [700, 1, 129, 300, 1000], num_heads=128, d_qk=576, d_v=512,
                           page_size=ps, scale=W.LATENT_SCALE, tok_lo=tok_lo, tok_hi=900,
                           live_only_in_range=True, extra_pages=2)
    bt = c.block_table.copy()
    bt[:, :tok_lo // ps] = -1
    c2 = W.DecodeCase(**{**c.__dict__, "block_table": bt})
    t = to_dev(c2)
    for heads in ((16, 32), (120, 128), (3, 15)):
        ro, rl = run_oracle(c2, head_lo=heads[0], head_hi=heads[1])
        for splits in (0, 1, 3):
            _print(f"case head16 ps={ps} heads={heads} splits={splits}")
            go, gl = run_decode(c2, t, head_lo=heads[0], head_hi=heads[1], num_splits=splits)
            assert_close(go, gl, ro, rl, what=f"16-head tile, page {ps}, heads {heads}, splits {splits}")


def test_head16_tile_rescale():
    """Growing scores on the 16-head tile: the running max moves many times
    (rope dims only, so the output keeps its scale)."""
    c = W.make_decode_case("grow16", 48, [4096, 2500], num_heads=128, d_qk=576, d_v=512, page_size=64,
                           scale=W.LATENT_SCALE)
    for b in range(c.num_reqs):
        n = int(c.seq_lens[b])
        for tkn in range(n):
            p, s = c.block_table[b, tkn // 64], tkn % 64
            rope = (c.kv_pages[p, s, c.d_v:].astype(np.uint32) << 16).view(np.float32) * (1.0 + tkn / 64.0)
            c.kv_pages[p, s, c.d_v:] = W.bf16_bits(rope)
    for splits in (0, 1):
        _print(f"case head16 growing scores splits={splits}")
        go, gl = run_decode(c, head_lo=32, head_hi=48, num_splits=splits)
        ro, rl = run_oracle(c, head_lo=32, head_hi=48)
        assert_close(go, gl, ro, rl, what=f"16-head tile, growing scores, splits {splits}")


@pytest.mark.parametrize("ps", [16, 32, 128, 256])
def test_128_head_tile_page_sizes(ps):
    """The 128-head tile (four waves, the tile-address table) on every page
    size: each wave's 8-row group of a tile lies in one page, whose offset the
    table holds; ranges starting mid-tile and mid-page, with the entries
    before them -1; unsplit, forced and planned splits."""
    tok_lo = 16 + ps
    c = W.make_decode_case("p128h", 90 + ps, [1500, 40, 700, 2], num_heads=128, d_qk=576, d_v=512,
                           page_size=ps, scale=W.LATENT_SCALE, tok_lo=tok_lo, tok_hi=1400,
                           live_only_in_range=True, extra_pages=2)
    bt = c.block_table.copy()
    bt[:, :tok_lo // ps] = -1
    c2 = W.DecodeCase(**{**c.__dict__, "block_table": bt})
    t = to_dev(c2)
    ro, rl = run_oracle(c2)
    for splits in (0, 1, 3):
        _print(f"case 128-head tile ps={ps} splits={splits}")
        go, gl = run_decode(c2, t, num_splits=splits)
        assert_close(go, gl, ro, rl, what=f"128-head tile, page {ps}, splits {splits}")


@pytest.mark.parametrize("ps", [16, 32, 128, 256])
def test_other_page_sizes(ps):
    c = W.make_decode_case("pages", 42, [700, 1, 129, 300], num_heads=40, d_qk=576, d_v=512, page_size=ps,
                           scale=W.LATENT_SCALE, extra_pages=3)
    go, gl = run_decode(c)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what=f"page_size={ps}")


def test_large_scores_rescale():
    """Scores that grow along the context force the running max to move many times.

    Only the rope dims (not part of V) grow with the token index, so the
    output stays on the N(0,1) scale the bars are set for."""
    c = W.make_decode_case("grow", 43, [4096, 2500], num_heads=128, d_qk=576, d_v=512, page_size=64,
                           scale=W.LATENT_SCALE)
    for b in range(c.num_reqs):
        n = int(c.seq_lens[b])
        for tkn in range(n):
            p, s = c.block_table[b, tkn // 64], tkn % 64
            rope = (c.kv_pages[p, s, c.d_v:].astype(np.uint32) << 16).view(np.float32) * (1.0 + tkn / 64.0)
            c.kv_pages[p, s, c.d_v:] = W.bf16_bits(rope)
    go, gl = run_decode(c)
    ro, rl = run_oracle(c)
    assert_close(go, gl, ro, rl, what="growing scores")


@pytest.mark.parametrize("heads", [16, 32, 128])
def test_bad_page_index_is_flagged_not_faulted(heads):
    """A block-table entry outside the pool is read as page 0 and raises the
    device error bit: the 16-head tile, the 32-head one, and the 128-head one
    (whose tile-address table checks the entries in its prologue)."""
    c = W.make_decode_case("bad", 44, [130], num_heads=128, d_qk=576, d_v=512, page_size=64,
                           scale=W.LATENT_SCALE, head_hi=heads)
    bt = c.block_table.copy()
    bt[0, 1] = c.num_pages + 1000
    c2 = W.DecodeCase(**{**c.__dict__, "block_table": bt})
    _print(f"case bad page heads={heads}")
    run_decode(c2)
    assert sp.device_errors(clear=True) & sp.DEVERR_BAD_PAGE


@pytest.mark.parametrize("f", [1e5, 1e30])
def test_split_partials_keep_the_range(f):
    """Split-KV partial outputs are kept in fp16 with a power-of-two scale per
    row, so a split share keeps the range of any finite input.  V values near
    f (q scaled down by f, so the scores keep their N(0,1)-input scale): with
    and without splits the result matches the oracle (compared at 1/f) and no
    device error bit is raised."""
    c = W.make_decode_case("big_v", 45, [700, 300], num_heads=128, d_qk=576, d_v=512, page_size=64,
                           scale=W.LATENT_SCALE)
    kv = c.kv_pages.copy()
    kv[..., :c.d_v] = W.bf16_bits((kv[..., :c.d_v].astype(np.uint32) << 16).view(np.float32) * np.float32(f))
    q = W.bf16_bits((c.q.astype(np.uint32) << 16).view(np.float32) / np.float32(f))
    c2 = W.DecodeCase(**{**c.__dict__, "kv_pages": kv, "q": q})
    ro, rl = run_oracle(c2)
    for splits in (1, 4, 0):
        go, gl = run_decode(c2, num_splits=splits)
        assert_close(go / f, gl, ro / f, rl, what=f"V near {f:.0e}, splits={splits}")


@pytest.mark.parametrize("d_v", [512, 516])  # one wave per row; the workgroup form (d_v not a multiple of 8)
def test_merge_edges(d_v):
    rows = 5
    P = torch.randn((3, rows, d_v), dtype=torch.float32, device=DEV)
    L = torch.tensor([[0.0, -math.inf, 1.0, -math.inf, 2.0],
                      [1.0, -math.inf, -math.inf, -math.inf, 2.0],
                      [-math.inf, -math.inf, 0.5, 3.0, 2.0]], dtype=torch.float32, device=DEV)
    P[0, 1] = float("nan")  # a part with LSE -inf contributes nothing, whatever its row holds
    out = torch.empty((rows, d_v), dtype=torch.float32, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    sp.lse_merge(P, L, out, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(P.cpu().numpy(), L.cpu().numpy())
    assert_close(out.cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, what=f"merge edges d_v={d_v}")
    o1 = torch.empty_like(out)
    sp.lse_merge(P[:1].contiguous(), L[:1].contiguous(), o1)
    torch.cuda.synchronize()
    live = torch.isfinite(L[0])
    assert torch.allclose(o1[live], P[0][live], atol=1e-6, rtol=0)


@pytest.mark.parametrize("n_parts,rows,d_v", [(300, 7, 512), (3000, 3, 64), (17, 33, 512), (1, 4, 64),
                                              (3000, 3, 12), (300, 7, 1028)])
def test_merge_many_parts(n_parts, rows, d_v):
    """Part counts past one batch (16) and past the workgroup form's LDS
    weight store (2,048); widths that take the workgroup form (d_v not a
    multiple of 8, or above 512); some parts empty."""
    g = torch.Generator(device="cpu").manual_seed(n_parts)
    P = torch.randn((n_parts, rows, d_v), generator=g, dtype=torch.float32).to(DEV)
    L = (torch.rand((n_parts, rows), generator=g, dtype=torch.float32) * 20 - 10).to(DEV)
    L[::7, 0] = -math.inf
    out = torch.empty((rows, d_v), dtype=torch.float32, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    sp.lse_merge(P, L, out, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(P.cpu().numpy(), L.cpu().numpy())
    assert_close(out.cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, what=f"merge {n_parts} parts")


def test_repack_rejects_bad_pairs():
    src = torch.arange(6 * 4 * 8, dtype=torch.int16, device=DEV).view(6, 4, 8)
    dst = torch.full((5, 4, 8), -1, dtype=torch.int16, device=DEV)
    st = torch.tensor([[0, -1, 2, -1, 9, 3]], dtype=torch.int32, device=DEV)
    dt = torch.tensor([[4, 1, -1, -1, 0, 0]], dtype=torch.int32, device=DEV)
    errs = torch.zeros((1,), dtype=torch.int32, device=DEV)
    sp.kv_repack(src, st, dst, dt, errs)
    torch.cuda.synchronize()
    want, copied, rejected = oracle.kv_repack(src.cpu().numpy(), st.cpu().numpy(),
                                              np.full((5, 4, 8), -1, np.int16), dt.cpu().numpy())
    assert int(errs.item()) == rejected == 3 and copied == 2
    assert np.array_equal(dst.cpu().numpy(), want)
    assert sp.device_errors(clear=True) & sp.DEVERR_REPACK_PAIR


def test_repack_unaligned_page_bytes():
    """Pages whose size is not a multiple of 16 bytes take the byte-copy path."""
    src = torch.randint(-100, 100, (7, 3, 5), dtype=torch.int16, device=DEV)  # 30-byte pages
    dst = torch.zeros((7, 3, 5), dtype=torch.int16, device=DEV)
    st = torch.tensor([[6, 0, 3], [1, -1, 2]], dtype=torch.int32, device=DEV)
    dt = torch.tensor([[0, 6, 1], [2, -1, 3]], dtype=torch.int32, device=DEV)
    sp.kv_repack(src, st, dst, dt)
    torch.cuda.synchronize()
    want, _, _ = oracle.kv_repack(src.cpu().numpy(), st.cpu().numpy(), np.zeros((7, 3, 5), np.int16),
                                  dt.cpu().numpy())
    assert np.array_equal(dst.cpu().numpy(), want)


# ---------------------------------------------------------------------------
# measured peaks (roofline context; no part of the path)
# ---------------------------------------------------------------------------
def test_measure_peaks_is_plausible():
    buf = torch.ones(256 << 20, dtype=torch.uint8, device=DEV)
    _print("case measure_peaks over 256 MiB")
    pk = sp.measure_peaks(buf)
    _print(f"  {pk}")
    # dense bf16 MFMA: below the 2.5 PFLOP/s published peak, far above a
    # broken loop; the shader clock within the part's range; the read rate
    # below the 256 MiB Infinity Cache's bandwidth and above a trickle
    assert 500.0 < pk["mfma_bf16_tflops"] < 2600.0
    assert 0.5 < pk["mfma_clock_ghz"] < 2.6
    assert 500.0 < pk["hbm_read_gbps"] < 20000.0
    with pytest.raises(sp.SplashError):
        sp.measure_peaks(buf[:1000])   # under 1 MiB


# ---------------------------------------------------------------------------
# HIP graph replay of a step (decode with its split-KV merge, then a repack)
# ---------------------------------------------------------------------------
def test_graph_replay_matches_eager():
    """The step captured into a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager result bit for bit."""
    c = W.case_owner(B=4, ctx=2048)
    t = to_dev(c)
    rc = W.make_repack_case(c, seed=11)
    st, dt = torch.from_numpy(rc.src_table).to(DEV), torch.from_numpy(rc.dst_table).to(DEV)
    fill = int(np.int16(rc.dst_fill.view(np.int16)))
    shape = (rc.dst_num_pages,) + c.kv_pages.shape[1:]
    hs = c.num_q_heads

    def run(out, lse, dst):
        sp.decode_attn(t["q"], t["kv"], t["bt"], t["sl"], c.head_lo, c.head_hi, c.tok_lo, c.tok_hi, out, lse,
                       d_v=c.d_v, scale=c.scale)
        sp.kv_repack(t["kv"], st, dst, dt)

    out_e = torch.empty((c.num_reqs, hs, c.d_v), dtype=torch.float32, device=DEV)
    lse_e = torch.empty((c.num_reqs, hs), dtype=torch.float32, device=DEV)
    dst_e = torch.full(shape, fill, dtype=torch.int16, device=DEV)
    # the library keeps one split-KV workspace per stream: the eager call on
    # the capture stream sizes that stream's workspace before the capture
    cap = torch.cuda.Stream(device=DEV)
    cap.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(cap):
        run(out_e, lse_e, dst_e)
    torch.cuda.synchronize()

    out_g, lse_g = torch.empty_like(out_e), torch.empty_like(lse_e)
    dst_g = torch.full(shape, fill, dtype=torch.int16, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        run(out_g, lse_g, dst_g)
    torch.cuda.synchronize()
    scratch_o, scratch_l = torch.empty_like(out_e), torch.empty_like(lse_e)
    for r in range(3):
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        dst_g.fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        # eager work of the program between replays
        sp.decode_attn(t["q"], t["kv"], t["bt"], t["sl"], c.head_lo, c.head_hi, 0, 1000, scratch_o, scratch_l,
                       d_v=c.d_v, scale=c.scale)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {r}: output differs from eager"
        assert torch.equal(lse_g, lse_e), f"replay {r}: LSE differs from eager"
        assert torch.equal(dst_g, dst_e), f"replay {r}: repack differs from eager"
    ro, rl = run_oracle(c)
    assert_close(out_g.cpu().double().numpy(), lse_g.cpu().double().numpy(), ro, rl, what="graph replay")
