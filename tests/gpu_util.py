"""Helpers shared by the GPU parity tests: move seeded cases to the GPU, run the
library through the C ABI binding, and compare with the oracle."""
import numpy as np
import torch

import layout_agnostic_latent_amd as sp
import oracle

DEV = torch.device("cuda:0")

# Bars for floating-point parity against the float64 oracle.
MAX_ABS = 1e-2
REL_L2 = 5e-3
LSE_ABS = 1e-3


def to_dev(case):
    return dict(q=torch.from_numpy(case.q.view(np.int16)).to(DEV),
                kv=torch.from_numpy(case.kv_pages.view(np.int16)).to(DEV),
                bt=torch.from_numpy(case.block_table).to(DEV),
                sl=torch.from_numpy(case.seq_lens).to(DEV))


def run_decode(case, t=None, head_lo=None, head_hi=None, tok_lo=None, tok_hi=None, num_splits=0,
               with_lse=True):
    t = t or to_dev(case)
    head_lo = case.head_lo if head_lo is None else head_lo
    head_hi = case.head_hi if head_hi is None else head_hi
    tok_lo = case.tok_lo if tok_lo is None else tok_lo
    tok_hi = case.tok_hi if tok_hi is None else tok_hi
    hs = head_hi - head_lo
    out = torch.full((case.num_reqs, hs, case.d_v), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((case.num_reqs, hs), float("nan"), dtype=torch.float32, device=DEV) if with_lse else None
    sp.decode_attn(t["q"], t["kv"], t["bt"], t["sl"], head_lo, head_hi, tok_lo, tok_hi, out, lse,
                   d_v=case.d_v, scale=case.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), (lse.cpu().double().numpy() if with_lse else None)


def run_oracle(case, head_lo=None, head_hi=None, tok_lo=None, tok_hi=None, reqs=None):
    head_lo = case.head_lo if head_lo is None else head_lo
    head_hi = case.head_hi if head_hi is None else head_hi
    tok_lo = case.tok_lo if tok_lo is None else tok_lo
    tok_hi = case.tok_hi if tok_hi is None else tok_hi
    return oracle.decode_attn(case.q, case.kv_pages, case.block_table, case.seq_lens, head_lo, head_hi,
                              tok_lo, tok_hi, case.d_v, case.page_size, case.scale, reqs=reqs)


def assert_close(go, gl, ro, rl, rows=None, what="", quiet=False):
    """Attention output within max-abs and relative-L2 bars, LSE within its bar.

    ``rows``: request indices to compare (default all).  -inf LSEs must match
    exactly (empty ranges), and their outputs must be exactly 0.
    """
    if rows is not None:
        go, ro = go[rows], ro[rows]
        if gl is not None:
            gl, rl = gl[rows], rl[rows]
    assert np.all(np.isfinite(go)), f"{what}: non-finite output"
    err = np.abs(go - ro).max() if go.size else 0.0
    denom = np.linalg.norm(ro)
    rel = np.linalg.norm(go - ro) / denom if denom > 0 else np.linalg.norm(go)
    lerr = float("nan")
    if gl is not None:
        live = ~np.isneginf(rl)
        if live.any():
            lerr = float(np.abs(gl[live] - rl[live]).max())
    # the margins, shown by `pytest -rP`
    if not quiet:
        print(f"parity {what}: max abs {err:.2e} (bar {MAX_ABS:.0e}), rel L2 {rel:.2e} (bar {REL_L2:.0e}), "
              f"LSE {lerr:.2e} (bar {LSE_ABS:.0e})", flush=True)
    assert err <= MAX_ABS, f"{what}: max abs error {err:.3e}"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e}"
    if gl is not None:
        empty = np.isneginf(rl)
        assert np.array_equal(np.isneginf(gl), empty), f"{what}: empty-range rows differ"
        assert np.all(go[empty] == 0), f"{what}: empty-range output not 0"
        if (~empty).any():
            assert lerr <= LSE_ABS, f"{what}: LSE abs error {lerr:.3e}"
    return err, rel
