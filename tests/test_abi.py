"""The C ABI without a GPU: the library loads, exports every function the
header declares, rejects bad host arguments before any HIP call, and plans
launches (split-KV chunks, head groups, workspace) as a pure host function."""
import ctypes
import os
import re

import pytest

import layout_agnostic_latent_amd as sp

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "splash_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(splash_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("splash_decode_attn", "splash_lse_merge", "splash_kv_repack", "splash_last_error"):
        assert required in names


def test_library_exports_every_declared_function(splash):
    L = splash.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in the header but not exported"


def _desc(**kw):
    d = dict(num_reqs=16, num_heads=128, d_qk=576, d_v=512, page_size=64, max_pages_per_req=64,
             num_pages=1024, scale=0.0721, num_splits=0)
    d.update(kw)
    return sp.make_desc(**d)


def _decode_rc(splash, desc, head_lo=0, head_hi=128, tok_lo=0, tok_hi=4096, ptr=0x1000, out=0x2000):
    L = splash.lib()
    return L.splash_decode_attn(ctypes.byref(desc), ptr, ptr, ptr, ptr, head_lo, head_hi, tok_lo, tok_hi, out,
                                None, None)


@pytest.mark.parametrize("kw,args,code", [
    (dict(), dict(head_lo=5, head_hi=5), sp.EINVAL),
    (dict(), dict(head_lo=-1), sp.EINVAL),
    (dict(), dict(head_hi=129), sp.EINVAL),
    (dict(), dict(tok_lo=10, tok_hi=9), sp.EINVAL),
    (dict(num_heads=0), dict(head_hi=1), sp.EINVAL),
    (dict(num_reqs=-1), dict(), sp.EINVAL),
    (dict(num_pages=0), dict(), sp.EINVAL),
    (dict(max_pages_per_req=0), dict(), sp.EINVAL),
    (dict(num_splits=-2), dict(), sp.EINVAL),
    (dict(scale=float("nan")), dict(), sp.EINVAL),
    (dict(scale=float("inf")), dict(), sp.EINVAL),
    (dict(d_qk=128, d_v=128), dict(), sp.EUNSUPPORTED),
    (dict(d_v=256), dict(), sp.EUNSUPPORTED),
    (dict(page_size=48), dict(), sp.EUNSUPPORTED),
    (dict(num_kv_heads=-1), dict(), sp.EINVAL),
    (dict(num_kv_heads=3), dict(), sp.EINVAL),   # 128 heads do not split over 3 KV heads
    (dict(page_size=8), dict(), sp.EUNSUPPORTED),
    (dict(), dict(ptr=0), sp.EINVAL),
    (dict(), dict(out=0), sp.EINVAL),
    (dict(), dict(ptr=0x1008), sp.EINVAL),
])
def test_decode_rejects_bad_arguments(splash, kw, args, code):
    rc = _decode_rc(splash, _desc(**kw), **args)
    assert rc == code
    assert splash.lib().splash_last_error().decode()


def test_merge_rejects_bad_arguments(splash):
    L = splash.lib()
    assert L.splash_lse_merge(0x1000, 0x1000, 0, 4, 512, 0x1000, None, None) == sp.EINVAL
    assert L.splash_lse_merge(0x1000, 0x1000, 2, -1, 512, 0x1000, None, None) == sp.EINVAL
    assert L.splash_lse_merge(0x1000, 0x1000, 2, 4, 510, 0x1000, None, None) == sp.EINVAL
    assert L.splash_lse_merge(None, 0x1000, 2, 4, 512, 0x1000, None, None) == sp.EINVAL
    assert L.splash_lse_merge(0x1004, 0x1000, 2, 4, 512, 0x1000, None, None) == sp.EINVAL


def test_repack_rejects_bad_arguments(splash):
    L = splash.lib()
    p = 0x1000
    assert L.splash_kv_repack(None, p, p, p, 1, 1, 16, 1, 1, None, None) == sp.EINVAL
    assert L.splash_kv_repack(p, p, p, p, -1, 1, 16, 1, 1, None, None) == sp.EINVAL
    assert L.splash_kv_repack(p, p, p, p, 1, 1, 0, 1, 1, None, None) == sp.EINVAL
    assert L.splash_kv_repack(p, p, p, p, 1, 1, 16, -1, 1, None, None) == sp.EINVAL
    assert L.splash_kv_repack(p, p, p, p, 1 << 20, 1 << 12, 16, 1, 1, None, None) == sp.EINVAL


def test_plan_shapes(splash, monkeypatch):
    # request-owned, 128 heads, 4,096 tokens: one head group, split to fill 256 CUs
    s, g, w = sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096)
    # unforced splits are cut on the device from the real lengths into at
    # most 256 equal ranges of the batch's tiles, each leaving at most two
    # partials: 512 partial rows per head, each 512 fp16 values and an
    # 8-byte {LSE, scale} record per 256-column group, plus each request's
    # 16-byte merge record
    assert g == 1 and s == 16
    per_part = 128 * (512 * 2 + 2 * 8)
    assert 512 * per_part + 16 * 16 <= w <= 512 * per_part + 1024
    # forced splits: fp16 outputs, then the records (each 256-byte aligned);
    # a 16-head slice stores 128-column groups
    # 16 requests x 8 chunks leave 128 of 256 CUs idle: each chunk is
    # computed by two workgroups, 16 partials per request
    s, g, w = sp.decode_plan(16, 128, 576, 512, 64, 256, 4096, 0.07, 0, 16, 0, 16384, num_splits=8)
    assert s == 16 and g == 1 and w == 16 * 16 * 16 * 512 * 2 + 4 * 16 * 16 * 16 * 8
    monkeypatch.setenv("SPLASH_CHUNK_WORKGROUPS", "1")
    s, g, w = sp.decode_plan(16, 128, 576, 512, 64, 256, 4096, 0.07, 0, 16, 0, 16384, num_splits=8)
    assert s == 8 and w == 8 * 16 * 16 * 512 * 2 + 4 * 8 * 16 * 16 * 8
    monkeypatch.delenv("SPLASH_CHUNK_WORKGROUPS")
    # no more workgroups per chunk than the chunk has tiles (2 tiles each here)
    assert sp.decode_plan(1, 128, 576, 512, 64, 256, 4096, 0.07, 0, 16, 0, 512, num_splits=8)[0] == 16
    # a 64-head slice uses 32-head x 2 waves groups
    s, g, _ = sp.decode_plan(2, 128, 576, 512, 64, 8, 16, 0.07, 0, 64, 0, 512)
    assert g == 1
    # 100 heads -> one 128-head group; 129..256 heads -> two groups
    assert sp.decode_plan(2, 256, 576, 512, 64, 8, 16, 0.07, 0, 200, 0, 512)[1] == 2
    # a tiny share needs no split and no workspace
    s, g, w = sp.decode_plan(2, 8, 80, 64, 16, 4, 8, 0.1, 0, 8, 0, 64)
    assert s == 1 and g == 1 and w == 0
    # 256 requests fill the CUs with one chunk each
    s, g, w = sp.decode_plan(256, 128, 576, 512, 64, 64, 20000, 0.07, 0, 128, 0, 4096)
    assert s == 1 and w == 0
    # 16 x 65,536 tokens: one round of 256 workgroups, 128-tile (4,096-token) chunks
    assert sp.decode_plan(16, 128, 576, 512, 64, 1024, 20000, 0.07, 0, 128, 0, 65536)[0] == 16
    # chunks never exceed 128 tiles: one 1M-token request still gets 256 of them
    assert sp.decode_plan(1, 128, 576, 512, 64, 16384, 20000, 0.07, 0, 128, 0, 1 << 20)[0] == 256


def test_plan_kv_heads(splash):
    # G = 2: 64 query heads per KV head -> one 64-head workgroup per KV head
    s, g, w = sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096, num_kv_heads=2)
    assert g == 2
    # G = 8: 16 heads per KV head; heads [8, 40) touch KV heads 0, 1 and 2
    s8, g8, w8 = sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 8, 40, 0, 4096, num_kv_heads=8)
    assert g8 == 3 and w8 > 0
    # G = 4 over all heads: 32 heads per KV head, four workgroups along the heads
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096, num_kv_heads=4)[1] == 4
    # a slice inside one KV head plans like G = 1 with that slice
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 64, 96, 0, 4096, num_kv_heads=2) == \
        sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 64, 96, 0, 4096)
    # G = 1 and G = 0 are the same single latent head
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096, num_kv_heads=0) == \
        sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096, num_kv_heads=1)


def test_plan_env_override(splash, monkeypatch):
    monkeypatch.setenv("SPLASH_NUM_SPLITS", "5")
    # 16 requests x 5 chunks = 80 workgroups: three per chunk fill 240 CUs
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096)[0] == 15
    monkeypatch.setenv("SPLASH_CHUNK_WORKGROUPS", "1")
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096)[0] == 5
    # an explicit num_splits in the descriptor wins
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096, num_splits=3)[0] == 3
    # one chunk always runs unsplit, whatever the workgroups-per-chunk override
    monkeypatch.setenv("SPLASH_CHUNK_WORKGROUPS", "3")
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096, num_splits=1)[:3:2] == (1, 0)


def test_product_path_does_not_touch_the_oracle():
    """The HIP package never imports the CPU oracle (the oracle is test infrastructure)."""
    pkg = os.path.dirname(sp.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_measure_peaks_rejects_bad_arguments_without_a_gpu(splash):
    L = splash.lib()
    p = sp.Peaks()
    assert L.splash_measure_peaks(None, 1 << 30, ctypes.byref(p), None) == sp.EINVAL
    assert b"measure_peaks" in L.splash_last_error()
    assert L.splash_measure_peaks(0x1000, 1000, ctypes.byref(p), None) == sp.EINVAL   # under 1 MiB
    assert L.splash_measure_peaks(0x1001, 1 << 30, ctypes.byref(p), None) == sp.EINVAL  # misaligned
    assert L.splash_measure_peaks(0x1000, 1 << 30, None, None) == sp.EINVAL


def test_repack_binding_rejects_host_pools():
    """A pool in host memory would hand a host pointer to the copy kernel: the
    binding refuses it before anything reaches the library."""
    import torch
    src = torch.zeros((4, 2, 8), dtype=torch.int16)
    dst = torch.zeros((4, 2, 8), dtype=torch.int16)
    tab = torch.zeros((1, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="src_pages must be on the GPU"):
        sp.kv_repack(src, tab, dst, tab)


def test_library_info_names_the_in_tree_build(splash):
    info = sp.library_info()
    assert info["path"] == os.path.join("layout_agnostic_latent_amd", "libsplash_attn.so")
    assert len(info["sha256_16"]) == 16


def test_splash_lib_outside_the_package_is_refused(tmp_path):
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SPLASH_LIB=str(tmp_path / "libsplash_attn.so"), PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", "import layout_agnostic_latent_amd"], env=env, capture_output=True,
                       text=True)
    assert r.returncode != 0 and "outside the package directory" in r.stderr


def test_noalloc_rejects_a_share_beyond_its_scratch(splash):
    """A share whose split-KV workspace exceeds the static scratch is refused
    on the host, before any HIP call."""
    L = splash.lib()
    # 64 forced chunks x 16 requests x 128 heads x 512 fp16 values = 128 MiB of partials
    d = _desc(num_splits=64)
    p = 0x1000
    rc = L.splash_decode_attn_noalloc(ctypes.byref(d), p, p, p, p, 0, 128, 0, 4096, p, None, None)
    assert rc == sp.EINVAL and b"scratch" in L.splash_last_error()
    assert sp.decode_plan(16, 128, 576, 512, 64, 64, 1024, 0.07, 0, 128, 0, 4096, num_splits=64)[2] > 72 << 20
