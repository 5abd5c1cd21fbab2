"""Per-layout attention time of one decode step, from measured share times.

SPLASH picks a parallel layout per phase of serving.  Its pages give, for each
layout, what one rank's attention share of a decode step is (thelatestinai
page, Appendix, Table 2 and its caption); the time model that turns those
shares into step time (the caption's Eqs. 1 and 10) is not on the pages.  This
module stands in for it on the attention part only: a rank's share is a
(requests, tokens per request, query heads) shape, its time is measured with
libsplash_attn at that shape, and a layout's attention time per step is the
busiest rank's.

Shares, for B requests of s tokens, H query heads and T ranks:
  * TP: heads [r*H/T, (r+1)*H/T) of every request over all s tokens;
  * CP: a contiguous 1/T of every request's tokens, all heads, whose partial
    outputs are then merged over the T ranks (each rank merging H/T heads
    after a reduce-scatter);
  * DP-attention and DOP: whole requests, dealt to ranks by count, all heads.
    DOP differs from DP-attention in how the weights are sharded, which this
    attention-only model does not see.

The model therefore cannot reproduce the pages' end-to-end crossovers at
short inputs (Tables 4-6), where sharded weight reads favour TP; it shows the
attention side, where reading every history on every rank makes TP lose as
contexts grow.

Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of Attention with
Seamless Handoff for LLM Serving" (weekinpapers.com); the thelatestinai page is that paper's
summary with its appendix tables (thelatestinai.com).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, List, Tuple

LAYOUTS = ("TP", "CP", "DP-attention", "DOP")


@dataclass(frozen=True)
class Share:
    """One rank's attention share of a decode step."""
    reqs: int         # requests in the rank's batch
    tokens: int       # history tokens per request that the rank attends over
    heads: int        # query heads
    merge_parts: int  # > 1: outputs are partial and merged over this many ranks

    @property
    def kv_tokens(self) -> int:
        return self.reqs * self.tokens


def rank_shares(layout: str, B: int, T: int, s: int, H: int) -> List[Share]:
    """The T ranks' shares under `layout` (Table 2's decomposition)."""
    if T < 1 or B < 0 or s < 0 or H < 1:
        raise ValueError("need T >= 1, B >= 0, s >= 0, H >= 1")
    if layout == "TP":
        return [Share(B, s, (r + 1) * H // T - r * H // T, 1) for r in range(T)]
    if layout == "CP":
        return [Share(B, (r + 1) * s // T - r * s // T, H, T) for r in range(T)]
    if layout in ("DP-attention", "DOP"):
        base, extra = divmod(B, T)
        return [Share(base + (1 if r < extra else 0), s, H, 1) for r in range(T)]
    raise ValueError(f"unknown layout {layout!r}")


def busiest_share(layout: str, B: int, T: int, s: int, H: int) -> Share:
    """The share with the most attention work (KV tokens x heads)."""
    return max(rank_shares(layout, B, T, s, H), key=lambda sh: (sh.kv_tokens * sh.heads, sh.kv_tokens))


def attention_time(layout: str, B: int, T: int, s: int, H: int, time_of: Callable[[Share], float]) -> float:
    """Attention time of one decode step: the busiest rank's share time."""
    return max(time_of(sh) for sh in set(rank_shares(layout, B, T, s, H)))


def choose(B: int, T: int, s: int, H: int, time_of: Callable[[Share], float],
           layouts=LAYOUTS) -> Tuple[str, Dict[str, float]]:
    """The layout with the least attention time, and every layout's time."""
    times = {L: attention_time(L, B, T, s, H, time_of) for L in layouts}
    return min(times, key=lambda L: (times[L], layouts.index(L))), times
