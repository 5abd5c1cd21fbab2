"""CPU oracle for one rank's share of decode attention over a paged latent KV head.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, float64 statement
of what the HIP path computes.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library
never calls it and shares no code with it; the two meet only in the seeded
input generators of ``workloads``.

What is computed, and where the pages fix it
--------------------------------------------
SPLASH (weekinpapers page, Abstract) rests on attention whose query heads
share one or a few KV heads: every query head of a request attends to one shared latent KV row per
token, so where a request's cache lives is independent of how the attention
weights are sharded.  One rank's share of a decode step is then

* a slice of the query heads over every request's whole history (TP),
* a contiguous token range of every request, emitted as a partial output plus
  its log-sum-exp and merged afterwards (CP, tokens split evenly),
* or the whole histories of the requests the rank owns (DP-attention, DOP,
  requests dealt to the ranks in equal numbers),

as laid out in thelatestinai page, Appendix Table 2 and its caption.  The
merge of partial results across ranks is the cross-node attention merge that
the zot.news page on Decode Token Parallelism names (its "How it works"
figure).  The KV movement at a layout handoff (Abstract: state that is not yet
in place is moved in the background and handed off at a batch boundary) is a
page copy.

Readings where the pages are silent (each is also listed in the design notes):
* attention is softmax(scale * q . k) . v over the tokens of the share, with
  the natural-log LSE = log(sum_t exp(scale * q . k_t));
* V is the first d_v dims of the same latent row as K (no extra V storage);
* the decode query attends to every token in [lo, hi); seq_len already counts
  the current token; no other mask;
* an empty range gives O = 0 and LSE = -inf, and the merge ignores such parts.

Parity pins (tests/test_oracle.py): one-token context, equal scores, the
layout-invariance of all three shares, brute force in pure Python / mpmath on
tiny inputs, page-permutation invariance, bounds, the merge identities, and the
busiest-rank loads of Table 2 (tests/golden/table2_loads.json).  No function
here is "parity unpinned".

Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of Attention with
Seamless Handoff for LLM Serving" (weekinpapers.com); the thelatestinai page is that paper's
summary with its appendix tables (thelatestinai.com); the zot.news page is "Decoupling attention
from model weights speeds large-language-model serving by up to 2x" (zot.news).
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

__all__ = ["widen_bf16", "decode_attn", "lse_merge", "kv_repack", "layout_shares",
           "busiest_rank_load"]


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_attn(q: np.ndarray, kv_pages: np.ndarray, block_table: np.ndarray,
                seq_lens: np.ndarray, head_lo: int, head_hi: int, tok_lo: int, tok_hi: int,
                d_v: int, page_size: int, scale: float,
                reqs: Sequence[int] | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention of one share, by definition, in float64.

    q           uint16 bf16 bits [B, H, d_qk]
    kv_pages    uint16 bf16 bits [num_pages, page_size, d_qk] (one latent KV
                head), or [num_pages, page_size, G, d_qk] (G shared KV heads)
    block_table int32 [B, max_pages]: logical page j of request b -> physical page
    seq_lens    int32 [B]
    Returns (out float64 [B, head_hi-head_lo, d_v], lse float64 [B, head_hi-head_lo]).
    Requests not listed in ``reqs`` (default: all) are left as O = 0, LSE = -inf.

    Per request b and head h of the slice (h an index of q's H heads):
      g = h // (H / G), the KV head that query head h shares with its group
      lo = max(tok_lo, 0), hi = min(tok_hi, seq_len[b]); empty -> O = 0, LSE = -inf
      k_t = kv[block_table[b][t // page_size], t % page_size, (g,) :d_qk], v_t = k_t[:d_v]
      s_t = scale * q[b,h] . k_t
      O   = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m),  m = max_t s_t
      LSE = m + log(sum_t exp(s_t - m))
    The premise is attention whose query heads share one or a few KV heads (weekinpapers page,
    Abstract); with G > 1 the query heads are taken to share KV heads in
    contiguous groups of H / G.
    """
    B, H, d_qk = q.shape
    G = 1 if kv_pages.ndim == 3 else kv_pages.shape[2]
    if H % G:
        raise ValueError("the query heads must split evenly over the KV heads")
    group = H // G
    Hs = head_hi - head_lo
    out = np.zeros((B, Hs, d_v), dtype=np.float64)
    lse = np.full((B, Hs), -np.inf, dtype=np.float64)
    for b in (range(B) if reqs is None else reqs):
        lo = max(int(tok_lo), 0)
        hi = min(int(tok_hi), int(seq_lens[b]))
        if lo >= hi:
            continue
        t = np.arange(lo, hi)
        pages = block_table[b, t // page_size]
        rows = kv_pages[pages, t % page_size]                     # [n, d_qk] or [n, G, d_qk]
        for g in range(G):
            h0, h1 = max(head_lo, g * group), min(head_hi, (g + 1) * group)
            if h0 >= h1:
                continue
            K = widen_bf16(rows[:, :d_qk] if G == 1 else rows[:, g, :d_qk])   # [n, d_qk]
            V = K[:, :d_v]                                           # [n, d_v]
            Q = widen_bf16(q[b, h0:h1, :])                           # [h1-h0, d_qk]
            S = scale * (Q @ K.T)                                    # [h1-h0, n]
            m = S.max(axis=1, keepdims=True)
            W = np.exp(S - m)
            denom = W.sum(axis=1, keepdims=True)
            out[b, h0 - head_lo:h1 - head_lo] = (W @ V) / denom
            lse[b, h0 - head_lo:h1 - head_lo] = (m + np.log(denom))[:, 0]
    return out, lse


def lse_merge(partials: np.ndarray, lses: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Merge n_parts partial softmax results over disjoint token sets, in float64.

    partials [n_parts, rows, d_v], lses [n_parts, rows].  Per row:
      M = max_p L_p over parts with finite L_p
      L = M + log(sum_p exp(L_p - M)),  O = sum_p exp(L_p - L) O_p
    Parts with L_p = -inf carry no tokens and count for nothing; a row whose
    parts are all empty gets O = 0, L = -inf.
    """
    P = np.asarray(partials, dtype=np.float64)
    L = np.asarray(lses, dtype=np.float64)
    live = np.isfinite(L)
    any_live = live.any(axis=0)
    M = np.where(live, L, -np.inf).max(axis=0)
    M_safe = np.where(any_live, M, 0.0)
    w = np.where(live, np.exp(np.where(live, L, 0.0) - M_safe[None, :]), 0.0)   # [n, rows]
    s = w.sum(axis=0)
    s_safe = np.where(any_live, s, 1.0)
    L_out = np.where(any_live, M_safe + np.log(s_safe), -np.inf)
    Pz = np.where(live[:, :, None], P, 0.0)
    O_out = (w[:, :, None] * Pz).sum(axis=0) / s_safe[:, None]
    O_out[~any_live] = 0.0
    return O_out, L_out


def kv_repack(src_pages: np.ndarray, src_table: np.ndarray, dst_pages: np.ndarray,
              dst_table: np.ndarray) -> Tuple[np.ndarray, int, int]:
    """Copy whole pages dst[dst_table[r][j]] <- src[src_table[r][j]].

    A pair (-1, -1) is padding.  A pair with exactly one -1, or an index
    outside its pool, is a caller error: it is skipped and counted.
    Returns (new destination pool, pages copied, pairs rejected).
    """
    dst = np.array(dst_pages, copy=True)
    copied = rejected = 0
    ns, nd = src_pages.shape[0], dst.shape[0]
    for s, d in zip(np.asarray(src_table).ravel().tolist(), np.asarray(dst_table).ravel().tolist()):
        if s < 0 and d < 0:
            continue
        if s < 0 or d < 0 or s >= ns or d >= nd:
            rejected += 1
            continue
        dst[d] = src_pages[s]
        copied += 1
    return dst, copied, rejected


# ---------------------------------------------------------------------------
# Layout shares (thelatestinai page, Appendix Table 2 and caption): B
# equal-length requests of s tokens on T ranks.
# ---------------------------------------------------------------------------
def layout_shares(layout: str, B: int, T: int, s: int, H: int) -> List[Dict]:
    """Per-rank share of a decode step under one layout.

    Each share is {'reqs': [...], 'heads': (lo, hi), 'toks': (lo, hi)}.
    * TP: rank r holds heads [r*H/T, (r+1)*H/T) of every request, all tokens.
    * CP: rank r holds tokens [r*s/T, (r+1)*s/T) of every request, all heads
      (the tokens split evenly over the ranks).
    * DP-attention and DOP: requests are dealt to owners by count (request b
      to rank b mod T, equal numbers per rank); each owner holds
      all heads and all tokens of its requests.  DOP differs from DP-attention
      only in how the weights are sharded, not in the attention share.
    """
    shares = []
    for r in range(T):
        if layout == "TP":
            shares.append({"reqs": list(range(B)), "heads": (r * H // T, (r + 1) * H // T),
                           "toks": (0, s)})
        elif layout == "CP":
            shares.append({"reqs": list(range(B)), "heads": (0, H),
                           "toks": (r * s // T, (r + 1) * s // T)})
        elif layout in ("DP-attention", "DOP"):
            shares.append({"reqs": [b for b in range(B) if b % T == r], "heads": (0, H),
                           "toks": (0, s)})
        else:
            raise ValueError(layout)
    return shares


def busiest_rank_load(shares: List[Dict], s: int, H: int) -> Dict[str, float]:
    """Busiest-rank KV read and attention work of a set of shares.

    KV read counts histories of s tokens the rank must read (a head slice
    still reads the whole history of every request, since all heads share the
    one latent row).  Attention work counts one request's full attention
    (all heads over all tokens) as 1.
    """
    kv_read = []
    work = []
    for sh in shares:
        toks = sh["toks"][1] - sh["toks"][0]
        heads = sh["heads"][1] - sh["heads"][0]
        n = len(sh["reqs"])
        kv_read.append(n * toks / s)
        work.append(n * toks * heads / (s * H))
    return {"kv_read": max(kv_read), "attention_work": max(work)}
