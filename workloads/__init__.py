"""Seeded synthetic inputs for decode attention over a paged, shared latent KV head.

This module is shared by the CPU oracle (``oracle/``) and the HIP path (tests,
bench, smoke).  It draws random numbers and lays them out; it holds none of the
attention arithmetic.

Shapes follow the workloads of the SPLASH pages: batches of B requests with
context lengths from about 1k to 64k tokens (thelatestinai page, Appendix
Tables 4-6, the input-length sweep at B=16), each rank holding one layout's
share of the work (Appendix Table 2: a head slice for TP, a token range for
CP, whole requests for DP-attention and DOP).  The model shapes (128 query
heads sharing one latent KV row of 512+64 dims, page size 64) are those of the
DeepSeek-V3 family named in Table 3's caption; the pages themselves give no
dimensions.

Conventions
-----------
* bf16 tensors are ``numpy.uint16`` arrays holding the raw bf16 bit patterns.
  Values are drawn as float32 from ``numpy.random.Generator(PCG64)`` and
  rounded to nearest-even bf16.
* Unused KV slots (the tail of a request's last page) and pages nobody
  references are filled with a quiet-NaN bit pattern, so any read of them that
  is not masked shows up in the result.
* Every tensor of a case gets its own child of ``SeedSequence(seed)``.

Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of Attention with
Seamless Handoff for LLM Serving" (weekinpapers.com); the thelatestinai page is that paper's
summary with its appendix tables (thelatestinai.com).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)

# Child-seed slots of a case's SeedSequence (fixed order: never reorder).
_SEED_Q, _SEED_KV, _SEED_PERM, _SEED_LENS, _SEED_MERGE_O, _SEED_MERGE_L, _SEED_REPACK, _SEED_DSTPERM = range(8)
_N_SEED_SLOTS = 8


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    r[nan] = BF16_QNAN
    return r


def _children(seed: int) -> List[np.random.Generator]:
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(_N_SEED_SLOTS)]


def _normal_bf16(gen: np.random.Generator, shape, std: float) -> np.ndarray:
    x = gen.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


@dataclasses.dataclass
class DecodeCase:
    """One rank's decode-attention share over a paged latent KV pool."""

    name: str
    seed: int
    num_reqs: int
    num_heads: int          # H: q's head count (its row stride)
    d_qk: int               # latent + rope dims of a KV row
    d_v: int                # V = first d_v dims of the same row
    page_size: int
    max_pages_per_req: int  # block_table row stride
    num_pages: int          # pool size in pages
    scale: float
    head_lo: int
    head_hi: int
    tok_lo: int
    tok_hi: int
    q: np.ndarray            # uint16 [B, H, d_qk]
    kv_pages: np.ndarray     # uint16 [num_pages, page_size, d_qk], or [.., G, d_qk] with G latent heads
    block_table: np.ndarray  # int32  [B, max_pages_per_req]; -1 = no page
    seq_lens: np.ndarray     # int32  [B]
    dense_kv: Optional[List[np.ndarray]] = None  # per request, logical order (optional)
    num_kv_heads: int = 1    # G latent KV heads per token; query head h reads head h // (H / G)

    @property
    def num_q_heads(self) -> int:
        return self.head_hi - self.head_lo

    def kv_tokens(self) -> int:
        """Number of (request, token) pairs the share attends over."""
        lo = max(self.tok_lo, 0)
        return int(sum(max(0, min(self.tok_hi, int(s)) - lo) for s in self.seq_lens))


def make_decode_case(name: str, seed: int, seq_lens, num_heads: int, d_qk: int, d_v: int,
                     page_size: int, scale: float, std: float = 1.0,
                     head_lo: int = 0, head_hi: Optional[int] = None,
                     tok_lo: int = 0, tok_hi: Optional[int] = None,
                     extra_pages: int = 0, live_only_in_range: bool = False,
                     max_pages_per_req: Optional[int] = None, keep_dense: bool = False,
                     num_kv_heads: int = 1) -> DecodeCase:
    """Build a paged decode case.

    Every request gets ceil(len/page_size) physical pages, placed at a random
    permutation of the pool.  ``extra_pages`` NaN pages nobody references are
    added to the pool.  With ``live_only_in_range`` only pages overlapping
    [tok_lo, tok_hi) receive random data; the rest of each request's pages are
    NaN (a share must never read outside its range).  With ``keep_dense`` the
    case also carries each request's rows in logical token order
    (``dense_kv[b]``, uint16 [len_b, d_qk]), drawn before any page placement.
    With ``num_kv_heads`` G > 1 every token holds G latent rows: the pool is
    [num_pages, page_size, G, d_qk] (and dense rows [len_b, G, d_qk]).
    """
    gens = _children(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = int(seq_lens.shape[0])
    if head_hi is None:
        head_hi = num_heads
    if tok_hi is None:
        tok_hi = int(seq_lens.max()) if B else 0
    pages_per_req = [(int(s) + page_size - 1) // page_size for s in seq_lens]
    if max_pages_per_req is None:
        max_pages_per_req = max(pages_per_req) if B else 1
    n_live = sum(pages_per_req)
    num_pages = n_live + extra_pages
    perm = gens[_SEED_PERM].permutation(num_pages).astype(np.int32)

    q = _normal_bf16(gens[_SEED_Q], (B, num_heads, d_qk), std)
    G = int(num_kv_heads)
    row_shape = (d_qk,) if G == 1 else (G, d_qk)
    kv = np.full((num_pages, page_size) + row_shape, BF16_QNAN, dtype=np.uint16)
    block_table = np.full((B, max_pages_per_req), -1, dtype=np.int32)

    # Draw the KV values request by request, in logical order, so that the
    # values a token holds do not depend on where its page landed.
    kv_gen = gens[_SEED_KV]
    dense = [] if keep_dense else None
    cursor = 0
    for b in range(B):
        n = int(seq_lens[b])
        rows = []
        for j in range(pages_per_req[b]):
            phys = int(perm[cursor])
            cursor += 1
            block_table[b, j] = phys
            t0 = j * page_size
            used = min(page_size, n - t0)
            if live_only_in_range and (t0 + page_size <= tok_lo or t0 >= tok_hi):
                if keep_dense:
                    rows.append(np.full((used,) + row_shape, BF16_QNAN, dtype=np.uint16))
                continue
            vals = _normal_bf16(kv_gen, (used,) + row_shape, std)
            kv[phys, :used] = vals
            if keep_dense:
                rows.append(vals)
        if keep_dense:
            dense.append(np.concatenate(rows, axis=0) if rows else np.zeros((0,) + row_shape, np.uint16))
    return DecodeCase(name=name, seed=seed, num_reqs=B, num_heads=num_heads, d_qk=d_qk, d_v=d_v,
                      page_size=page_size, max_pages_per_req=max_pages_per_req, num_pages=num_pages,
                      scale=scale, head_lo=head_lo, head_hi=head_hi, tok_lo=tok_lo, tok_hi=tok_hi,
                      q=q, kv_pages=kv, block_table=block_table, seq_lens=seq_lens, dense_kv=dense,
                      num_kv_heads=G)


def loguniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """floor(exp(U[ln lo, ln hi])) clipped to [lo, hi]."""
    g = _children(seed)[_SEED_LENS]
    x = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), size=n)))
    return np.clip(x, lo, hi).astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads and the sweep.  Latent 512 + rope 64 => d_qk 576, d_v 512,
# softmax scale 1/sqrt(128 + 64) = 1/sqrt(192).
# ---------------------------------------------------------------------------
LATENT_QK, LATENT_V, LATENT_SCALE = 576, 512, 1.0 / math.sqrt(192.0)


def case_tiny(seed: int = 1, keep_dense: bool = False) -> DecodeCase:
    """B=2, lengths 17 and 64, H=8, d_qk 80 (64 latent + 16 rope), d_v 64, page 16.

    6 live pages in an 8-page pool (2 NaN pages), shuffled table, N(0, 0.5^2)."""
    return make_decode_case("tiny", seed, [17, 64], num_heads=8, d_qk=80, d_v=64, page_size=16,
                            scale=1.0 / math.sqrt(80.0), std=0.5, extra_pages=2, keep_dense=keep_dense)


def case_owner(seed: int = 2, B: int = 16, ctx: int = 4096, num_kv_heads: int = 1) -> DecodeCase:
    """Request-owned share (DP-attention / DOP owner): B x ctx tokens, all 128 heads
    (over num_kv_heads shared latent KV heads)."""
    return make_decode_case("owner", seed, [ctx] * B, num_heads=128, d_qk=LATENT_QK, d_v=LATENT_V,
                            page_size=64, scale=LATENT_SCALE, num_kv_heads=num_kv_heads)


def case_tp(seed: int = 3, B: int = 16, ctx: int = 16384, heads=(0, 16)) -> DecodeCase:
    """Head-sliced share (one TP rank): heads [0,16) of 128, all tokens."""
    return make_decode_case("tp", seed, [ctx] * B, num_heads=128, d_qk=LATENT_QK, d_v=LATENT_V,
                            page_size=64, scale=LATENT_SCALE, head_lo=heads[0], head_hi=heads[1])


def case_cp(seed: int = 4, B: int = 16, ctx: int = 65536, rank: int = 3, ranks: int = 8,
            live_only_in_range: bool = True) -> DecodeCase:
    """Token-split share (one CP rank): tokens [rank*ctx/T, (rank+1)*ctx/T) of every request."""
    lo, hi = rank * ctx // ranks, (rank + 1) * ctx // ranks
    return make_decode_case("cp", seed, [ctx] * B, num_heads=128, d_qk=LATENT_QK, d_v=LATENT_V,
                            page_size=64, scale=LATENT_SCALE, tok_lo=lo, tok_hi=hi,
                            live_only_in_range=live_only_in_range)


def case_transition(seed: int = 5, n: int = 64, lo: int = 512, hi: int = 65536) -> DecodeCase:
    """Ragged transition batch: n requests, log-uniform lengths in [lo, hi], all 128 heads."""
    lens = loguniform_lengths(seed, n, lo, hi)
    return make_decode_case("transition", seed, lens, num_heads=128, d_qk=LATENT_QK, d_v=LATENT_V,
                            page_size=64, scale=LATENT_SCALE)


def sweep_case(share: str, ctx: int, seed: int = 6, B: int = 16) -> DecodeCase:
    """The B=16 input-length sweep, one rank's share: 'owner', 'tp' or 'cp' (rank 3 of 8);
    'gqa<G>' is the owner share over G shared latent KV heads."""
    if share == "owner":
        return case_owner(seed=seed, B=B, ctx=ctx)
    if share.startswith("gqa"):
        return case_owner(seed=seed, B=B, ctx=ctx, num_kv_heads=int(share[3:]))
    if share == "tp":
        return case_tp(seed=seed, B=B, ctx=ctx)
    if share == "cp":
        return case_cp(seed=seed, B=B, ctx=ctx)
    raise ValueError(share)


SWEEP_CONTEXTS = (1024, 4096, 16384, 32768, 65536)


@dataclasses.dataclass
class MergeCase:
    partials: np.ndarray  # float32 [n_parts, rows, d_v]
    lses: np.ndarray      # float32 [n_parts, rows]


def make_merge_case(seed: int, n_parts: int, rows: int, d_v: int, lse_lo: float = -5.0,
                    lse_hi: float = 5.0) -> MergeCase:
    """Synthetic partial (O, LSE) sets: O ~ N(0,1), LSE ~ U[lse_lo, lse_hi], float32."""
    g = _children(seed)
    O = g[_SEED_MERGE_O].standard_normal(size=(n_parts, rows, d_v), dtype=np.float32)
    L = g[_SEED_MERGE_L].uniform(lse_lo, lse_hi, size=(n_parts, rows)).astype(np.float32)
    return MergeCase(partials=O, lses=L)


def case_cp_merge(seed: int = 4, B: int = 16, H: int = 128, parts: int = 8, d_v: int = 512) -> MergeCase:
    """The CP rank's merge: 8 seeded (O, LSE) sets over B*H rows, LSE ~ U[-5, 5]."""
    return make_merge_case(seed + 1000, parts, B * H, d_v)


@dataclasses.dataclass
class RepackCase:
    src_pages: np.ndarray   # uint16 [src_num_pages, page_size, d]
    src_table: np.ndarray   # int32 [n_reqs, max_pages]; -1 = padding
    dst_num_pages: int
    dst_table: np.ndarray   # int32 [n_reqs, max_pages]; -1 = padding
    moved_reqs: np.ndarray  # int32 indices into the batch
    dst_fill: np.uint16     # sentinel bit pattern of the fresh destination pool


def make_repack_case(case: DecodeCase, seed: int, fraction: float = 0.5,
                     dst_fill: int = 0x5A5A) -> RepackCase:
    """Move a seeded random subset of the requests (all of their pages) to a fresh pool.

    The destination pool holds exactly the moved pages, at a fresh random
    permutation; every other destination byte keeps the sentinel ``dst_fill``.
    """
    g = _children(seed)
    B = case.num_reqs
    k = max(1, int(round(B * fraction)))
    moved = np.sort(g[_SEED_REPACK].choice(B, size=k, replace=False)).astype(np.int32)
    src_table = np.full((k, case.max_pages_per_req), -1, dtype=np.int32)
    n_moved_pages = 0
    for i, b in enumerate(moved):
        n = (int(case.seq_lens[b]) + case.page_size - 1) // case.page_size
        src_table[i, :n] = case.block_table[b, :n]
        n_moved_pages += n
    dst_perm = g[_SEED_DSTPERM].permutation(n_moved_pages).astype(np.int32)
    dst_table = np.full_like(src_table, -1)
    c = 0
    for i in range(k):
        for j in range(case.max_pages_per_req):
            if src_table[i, j] >= 0:
                dst_table[i, j] = dst_perm[c]
                c += 1
    return RepackCase(src_pages=case.kv_pages, src_table=src_table, dst_num_pages=n_moved_pages,
                      dst_table=dst_table, moved_reqs=moved, dst_fill=np.uint16(dst_fill))


CONFIGS: Dict[str, str] = {
    "tiny": "B=2, lens 17/64, H=8, d_qk 80, d_v 64, page 16, N(0,0.25), scale 1/sqrt(80)",
    "owner": "B=16 x 4,096, H=128, 576/512, page 64, N(0,1), scale 1/sqrt(192)",
    "tp": "B=16 x 16,384, heads [0,16) of 128, split into 8 chunks + merge",
    "cp": "B=16 x 65,536, tokens [24,576, 32,768), 128 heads; merge of 8 seeded (O, LSE) sets",
    "transition": "64 requests, log-uniform [512, 65,536], 128 heads; repack of 32 requests",
}
