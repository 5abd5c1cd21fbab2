"""Python binding of libsplash_attn (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libsplash_attn.so``.  torch is used for device memory and
streams.  Import fails loudly if the library has not been built
(``python -m layout_agnostic_latent_amd.build``).

Functions mirror the C ABI in include/splash_attn.h:
  decode_attn(q, kv_pages, block_table, seq_lens, head_lo, head_hi, tok_lo, tok_hi, out, lse, ...)
  decode_attn_noalloc(...)  (same arguments; split-KV workspace in a static scratch array)
  lse_merge(partials, lses, out, lse_out)
  kv_repack(src_pages, src_table, dst_pages, dst_table, err_count=None)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = ["LIB_PATH", "SplashError", "lib", "library_info", "decode_attn", "decode_attn_noalloc", "decode_plan", "lse_merge", "kv_repack",
           "device_errors", "release_workspace", "profile_start", "profile_stop", "measure_peaks", "DEVERR_BAD_PAGE",
           "DEVERR_REPACK_PAIR", "DEVERR_PARTIAL_RANGE"]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# The in-tree build.  SPLASH_LIB may only name a library inside this package
# (so that a result can never come from a build made elsewhere).
LIB_PATH = os.path.join(_PKG_DIR, "libsplash_attn.so")
if os.environ.get("SPLASH_LIB"):
    _alt = os.path.realpath(os.environ["SPLASH_LIB"])
    if os.path.dirname(_alt) != os.path.realpath(_PKG_DIR):
        raise ImportError(f"SPLASH_LIB={os.environ['SPLASH_LIB']} is outside the package directory {_PKG_DIR}")
    LIB_PATH = _alt

OK, EINVAL, EUNSUPPORTED, EHIP = 0, -1, -2, -3
DEVERR_BAD_PAGE, DEVERR_REPACK_PAIR, DEVERR_PARTIAL_RANGE = 1, 2, 4


class SplashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libsplash_attn error {code}: {msg}")
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages_per_req", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("num_splits", ctypes.c_int32), ("scale", ctypes.c_float),
                ("num_kv_heads", ctypes.c_int32)]


class Profile(ctypes.Structure):
    _fields_ = [("decode_launches", ctypes.c_int32), ("merge_launches", ctypes.c_int32),
                ("repack_launches", ctypes.c_int32), ("decode_ms", ctypes.c_double),
                ("merge_ms", ctypes.c_double), ("repack_ms", ctypes.c_double),
                ("lse_merge_launches", ctypes.c_int32), ("lse_merge_ms", ctypes.c_double)]


class Peaks(ctypes.Structure):
    _fields_ = [("mfma_bf16_tflops", ctypes.c_double), ("mfma_clock_ghz", ctypes.c_double),
                ("hbm_read_gbps", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsplash_attn.so (once).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m layout_agnostic_latent_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, fp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        L.splash_decode_attn.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, i32, i32, i32, i32, fp, fp, vp]
        L.splash_decode_attn.restype = ctypes.c_int
        L.splash_decode_attn_noalloc.argtypes = L.splash_decode_attn.argtypes
        L.splash_decode_attn_noalloc.restype = ctypes.c_int
        L.splash_lse_merge.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
        L.splash_lse_merge.restype = ctypes.c_int
        L.splash_kv_repack.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, vp]
        L.splash_kv_repack.restype = ctypes.c_int
        L.splash_last_error.argtypes = []
        L.splash_last_error.restype = ctypes.c_char_p
        L.splash_device_errors.argtypes = [ctypes.POINTER(i32), i32]
        L.splash_device_errors.restype = ctypes.c_int
        L.splash_release_workspace.argtypes = []
        L.splash_release_workspace.restype = ctypes.c_int
        L.splash_decode_plan.argtypes = [ctypes.POINTER(Desc), i32, i32, i32, i32, ctypes.POINTER(i32),
                                         ctypes.POINTER(i32), ctypes.POINTER(i64)]
        L.splash_decode_plan.restype = ctypes.c_int
        L.splash_profile_start.argtypes = []
        L.splash_profile_start.restype = ctypes.c_int
        L.splash_profile_stop.argtypes = [ctypes.POINTER(Profile)]
        L.splash_profile_stop.restype = ctypes.c_int
        L.splash_measure_peaks.argtypes = [vp, i64, ctypes.POINTER(Peaks), vp]
        L.splash_measure_peaks.restype = ctypes.c_int
        _lib = L
    return _lib


def library_info() -> dict:
    """Path and SHA-256 (first 16 hex digits) of the library file this process loads."""
    import hashlib
    with open(LIB_PATH, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    return {"path": os.path.relpath(LIB_PATH, os.path.dirname(_PKG_DIR)), "sha256_16": digest}


def _check(rc: int) -> None:
    if rc != OK:
        raise SplashError(rc, lib().splash_last_error().decode())


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


def make_desc(num_reqs, num_heads, d_qk, d_v, page_size, max_pages_per_req, num_pages, scale,
              num_splits=0, num_kv_heads=1) -> Desc:
    return Desc(num_reqs, num_heads, d_qk, d_v, page_size, max_pages_per_req, num_pages, num_splits, scale,
                num_kv_heads)


def _desc_from(q, kv_pages, block_table, d_v, scale, num_splits) -> Desc:
    B, H, d_qk = q.shape
    if kv_pages.dim() == 3:   # one latent KV head
        (num_pages, ps, d_row), G = kv_pages.shape, 1
    else:                     # [P, ps, G, d_qk]: G shared KV heads
        num_pages, ps, G, d_row = kv_pages.shape
    if d_row != d_qk:
        raise ValueError(f"kv row width {d_row} != q width {d_qk}")
    return make_desc(B, H, d_qk, d_v, ps, block_table.shape[1], num_pages, scale, num_splits, G)


def _require(t, name, dtypes, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {ndim}-d tensor, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")


def decode_attn(q, kv_pages, block_table, seq_lens, head_lo: int, head_hi: int, tok_lo: int, tok_hi: int,
                out, lse=None, *, d_v: int, scale: float, num_splits: int = 0, stream=None) -> None:
    """splash_decode_attn.  q bf16 [B,H,d_qk]; kv_pages bf16 [P,ps,d_qk] or [P,ps,G,d_qk] (G shared KV heads);
    block_table int32 [B,max_pages]; seq_lens int32 [B]; out fp32 [B, head_hi-head_lo, d_v];
    lse fp32 [B, head_hi-head_lo] or None."""
    _decode("splash_decode_attn", q, kv_pages, block_table, seq_lens, head_lo, head_hi, tok_lo, tok_hi, out, lse,
            d_v, scale, num_splits, stream)


def decode_attn_noalloc(q, kv_pages, block_table, seq_lens, head_lo: int, head_hi: int, tok_lo: int, tok_hi: int,
                        out, lse=None, *, d_v: int, scale: float, num_splits: int = 0, stream=None) -> None:
    """splash_decode_attn_noalloc: as decode_attn, with the split-KV workspace in the library's static
    per-device scratch (no device allocation; overlapping calls on one GPU race)."""
    _decode("splash_decode_attn_noalloc", q, kv_pages, block_table, seq_lens, head_lo, head_hi, tok_lo, tok_hi, out,
            lse, d_v, scale, num_splits, stream)


def _decode(entry, q, kv_pages, block_table, seq_lens, head_lo, head_hi, tok_lo, tok_hi, out, lse, d_v, scale,
            num_splits, stream):
    import torch
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    _require(q, "q", bf, 3)
    _require(kv_pages, "kv_pages", bf, 4 if getattr(kv_pages, "ndim", 3) == 4 else 3)
    _require(block_table, "block_table", (torch.int32,), 2)
    _require(seq_lens, "seq_lens", (torch.int32,), 1)
    _require(out, "out", (torch.float32,), 3)
    if lse is not None:
        _require(lse, "lse", (torch.float32,), 2)
    B, H, _ = q.shape
    hs = head_hi - head_lo
    if tuple(out.shape) != (B, hs, d_v) or (lse is not None and tuple(lse.shape) != (B, hs)):
        raise ValueError("out / lse shape does not match [B, head_hi-head_lo(, d_v)]")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table / seq_lens rows != B")
    d = _desc_from(q, kv_pages, block_table, d_v, scale, num_splits)
    _check(getattr(lib(), entry)(ctypes.byref(d), _ptr(q), _ptr(kv_pages), _ptr(block_table), _ptr(seq_lens),
                                 head_lo, head_hi, tok_lo, tok_hi, _ptr(out), _ptr(lse), _stream(stream)))


def decode_plan(num_reqs, num_heads, d_qk, d_v, page_size, max_pages_per_req, num_pages, scale,
                head_lo, head_hi, tok_lo, tok_hi, num_splits=0, num_kv_heads=1) -> Tuple[int, int, int]:
    """(split-KV chunks, head groups, workspace bytes) the library would use.  Host only."""
    d = make_desc(num_reqs, num_heads, d_qk, d_v, page_size, max_pages_per_req, num_pages, scale, num_splits,
                  num_kv_heads)
    s, g, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib().splash_decode_plan(ctypes.byref(d), head_lo, head_hi, tok_lo, tok_hi, ctypes.byref(s),
                                    ctypes.byref(g), ctypes.byref(w)))
    return s.value, g.value, w.value


def lse_merge(partials, lses, out, lse_out=None, *, stream=None) -> None:
    """splash_lse_merge.  partials fp32 [n,rows,d_v]; lses fp32 [n,rows]; out fp32 [rows,d_v]."""
    import torch
    _require(partials, "partials", (torch.float32,), 3)
    _require(lses, "lses", (torch.float32,), 2)
    _require(out, "out", (torch.float32,), 2)
    n, rows, d_v = partials.shape
    if tuple(lses.shape) != (n, rows) or tuple(out.shape) != (rows, d_v):
        raise ValueError("shape mismatch between partials, lses and out")
    if lse_out is not None:
        _require(lse_out, "lse_out", (torch.float32,), 1)
    _check(lib().splash_lse_merge(_ptr(partials), _ptr(lses), n, rows, d_v, _ptr(out), _ptr(lse_out),
                                  _stream(stream)))


def kv_repack(src_pages, src_table, dst_pages, dst_table, err_count=None, *, stream=None) -> None:
    """splash_kv_repack over whole pages (the leading dim of src_pages / dst_pages)."""
    import torch
    for name, pool in (("src_pages", src_pages), ("dst_pages", dst_pages)):
        if not isinstance(pool, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if not pool.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if not pool.is_contiguous() or pool.dim() < 1:
            raise ValueError(f"{name} must be a contiguous tensor of pages (leading dimension)")
    if src_pages.device != dst_pages.device:
        raise ValueError("src_pages and dst_pages are on different devices")
    if src_pages.dtype != dst_pages.dtype:
        raise TypeError(f"pool dtypes differ: {src_pages.dtype} and {dst_pages.dtype}")
    _require(src_table, "src_table", (torch.int32,), 2)
    _require(dst_table, "dst_table", (torch.int32,), 2)
    if src_table.device != src_pages.device or dst_table.device != src_pages.device:
        raise ValueError("the block tables must be on the pools' device")
    if tuple(src_table.shape) != tuple(dst_table.shape):
        raise ValueError("src_table and dst_table shapes differ")
    page_bytes = src_pages[0].numel() * src_pages.element_size() if src_pages.shape[0] else \
        (dst_pages[0].numel() * dst_pages.element_size())
    dst_page_bytes = dst_pages[0].numel() * dst_pages.element_size() if dst_pages.shape[0] else page_bytes
    if page_bytes != dst_page_bytes:
        raise ValueError("source and destination page sizes differ")
    if err_count is not None:
        _require(err_count, "err_count", (torch.int32,), 1)
        if err_count.numel() < 1 or err_count.device != src_pages.device:
            raise ValueError("err_count must hold at least one int32 on the pools' device")
    n, m = src_table.shape
    _check(lib().splash_kv_repack(_ptr(src_pages), _ptr(src_table), _ptr(dst_pages), _ptr(dst_table), n, m,
                                  page_bytes, src_pages.shape[0], dst_pages.shape[0], _ptr(err_count),
                                  _stream(stream)))


def device_errors(clear: bool = True) -> int:
    """Synchronise the device; return (and by default clear) its SPLASH_DEVERR_* bits."""
    v = ctypes.c_int32()
    _check(lib().splash_device_errors(ctypes.byref(v), 1 if clear else 0))
    return v.value


def release_workspace() -> None:
    _check(lib().splash_release_workspace())


def profile_start() -> None:
    """Bracket every kernel the library launches with HIP events until profile_stop()."""
    _check(lib().splash_profile_start())


def profile_stop() -> dict:
    """Synchronise and return launch counts and summed kernel durations (ms) per kind."""
    p = Profile()
    _check(lib().splash_profile_stop(ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in Profile._fields_}


def measure_peaks(buf, stream=None) -> dict:
    """splash_measure_peaks over the device tensor `buf` (>= 1 MiB; use >= 1 GiB): measured bf16 MFMA
    TFLOP/s, the shader clock during it (GHz), and the streaming HBM read rate (GB/s)."""
    import torch
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    p = Peaks()
    _check(lib().splash_measure_peaks(_ptr(buf), buf.numel() * buf.element_size(), ctypes.byref(p), _stream(stream)))
    return {"mfma_bf16_tflops": p.mfma_bf16_tflops, "mfma_clock_ghz": p.mfma_clock_ghz,
            "hbm_read_gbps": p.hbm_read_gbps}
