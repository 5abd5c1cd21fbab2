"""splash_decode_attn_noalloc through the C ABI against splash_decode_attn.

The allocation-free entry point keeps its split-KV workspace in the
library's static per-device scratch array.  Two calls in a row, the second
with a smaller input (the scratch still holds the first call's partials),
each compared with the allocating entry point at the parity bars, plus a
forced-split share and one without splits.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DEV, assert_close, to_dev

import layout_agnostic_latent_amd as sp

pytestmark = pytest.mark.gpu


def _both(case, num_splits=0):
    t = to_dev(case)
    hs = case.num_q_heads
    res = []
    for fn in (sp.decode_attn, sp.decode_attn_noalloc):
        out = torch.full((case.num_reqs, hs, case.d_v), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((case.num_reqs, hs), float("nan"), dtype=torch.float32, device=DEV)
        fn(t["q"], t["kv"], t["bt"], t["sl"], case.head_lo, case.head_hi, case.tok_lo, case.tok_hi, out, lse,
           d_v=case.d_v, scale=case.scale, num_splits=num_splits)
        torch.cuda.synchronize()
        res.append((out.cpu().double().numpy(), lse.cpu().double().numpy()))
    return res


def test_noalloc_two_calls_second_smaller():
    sp.device_errors(clear=True)
    big = W.case_owner()                                 # 16 x 4,096 tokens, 128 heads: split-KV
    small = W.case_owner(seed=9, B=3, ctx=1500)          # fewer requests, shorter, ragged tail
    for case in (big, small):
        plan = sp.decode_plan(case.num_reqs, case.num_heads, case.d_qk, case.d_v, case.page_size,
                              case.max_pages_per_req, case.num_pages, case.scale, case.head_lo, case.head_hi,
                              case.tok_lo, case.tok_hi)
        print(f"case noalloc {case.name} B={case.num_reqs}: splits {plan[0]}, workspace {plan[2]} B", flush=True)
        assert plan[0] > 1 and 0 < plan[2] <= 72 << 20
        (ro, rl), (go, gl) = _both(case)
        assert_close(go, gl, ro, rl, what=f"noalloc vs decode_attn, {case.name} B={case.num_reqs}")
    assert sp.device_errors(clear=True) == 0


def test_noalloc_forced_splits_and_unsplit():
    sp.device_errors(clear=True)
    case = W.make_decode_case("noalloc_mix", 47, [900, 33, 0, 2500], num_heads=128, d_qk=576, d_v=512,
                              page_size=64, scale=W.LATENT_SCALE, head_lo=5, head_hi=100)
    for splits in (3, 1):
        print(f"case noalloc forced splits={splits}", flush=True)
        (ro, rl), (go, gl) = _both(case, num_splits=splits)
        assert_close(go, gl, ro, rl, what=f"noalloc vs decode_attn, splits={splits}")
    tiny = W.case_tiny()
    (ro, rl), (go, gl) = _both(tiny)
    assert_close(go, gl, ro, rl, what="noalloc vs decode_attn, tiny")
    assert sp.device_errors(clear=True) == 0


def test_noalloc_16_head_tile():
    """A 16-head share (the 16x16x32 tile) through the allocation-free entry
    point, planned and forced splits."""
    sp.device_errors(clear=True)
    case = W.make_decode_case("noalloc_h16", 48, [3000, 700, 65, 1800], num_heads=128, d_qk=576, d_v=512,
                              page_size=64, scale=W.LATENT_SCALE, head_lo=16, head_hi=32)
    for splits in (0, 3):
        print(f"case noalloc 16-head tile splits={splits}", flush=True)
        (ro, rl), (go, gl) = _both(case, num_splits=splits)
        assert_close(go, gl, ro, rl, what=f"noalloc vs decode_attn, 16-head tile, splits={splits}")
    assert sp.device_errors(clear=True) == 0
