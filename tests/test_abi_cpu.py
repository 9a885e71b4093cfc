"""Host-side checks of libftmoe.so that need no GPU: the library loads, exports
every entry point include/ftmoe.h declares, and its host validation rejects bad
arguments with the documented status codes before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ftmoe.h")


def _lib_path():
    from nvfp4_mixture_experts_amd import build
    if not os.path.exists(build.LIB_PATH):
        build.build()
    return build.LIB_PATH


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ft_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("ft_moe_route", "ft_moe_nvfp4_decode", "ft_moe_nvfp4_prefill", "ft_nvfp4_repack",
              "ft_nvfp4_dequant", "ft_moe_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    path = _lib_path()
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (ft_[a-z0-9_]+)$", out, flags=re.M))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(path)
    for n in _declared():
        assert hasattr(lib, n)


@pytest.fixture(scope="module")
def ft():
    _lib_path()
    from nvfp4_mixture_experts_amd import ftmoe
    return ftmoe


def test_abi_version(ft):
    assert ft.ft_abi_version() == ft.FT_ABI_VERSION == 1


def test_repacked_sizes(ft):
    H, I, n = 2048, 768, 288
    assert ft.ft_nvfp4_repacked_bytes(H, I, n, 0) == n * 2 * I * H // 2
    assert ft.ft_nvfp4_repacked_bytes(H, I, n, 1) == n * 2 * I * H // 16
    assert ft.ft_nvfp4_repacked_bytes(H, I, n, 2) == n * H * I // 2
    assert ft.ft_nvfp4_repacked_bytes(H, I, n, 3) == n * H * I // 16
    assert ft.ft_nvfp4_repacked_bytes(H, I, n, 4) == 0
    assert ft.ft_nvfp4_repacked_bytes(0, I, n, 0) == 0


def test_workspace_bytes_and_desc_validation(ft):
    good = ft.make_desc(288, 2048, 768, 8, 1)
    for path in (0, 1, 2):
        assert ft.ft_moe_workspace_bytes(good, 1, path) > 0
    assert ft.ft_moe_workspace_bytes(good, 32, 1) > ft.ft_moe_workspace_bytes(good, 1, 1)
    assert ft.ft_moe_workspace_bytes(good, -1, 1) == 0
    assert ft.ft_moe_workspace_bytes(good, 1, 3) == 0
    bad = [
        ft.make_desc(8, 2048, 768, 9, 1),      # k > E
        ft.make_desc(8, 2048, 768, 0, 1),      # k = 0
        ft.make_desc(2048, 2048, 768, 8, 1),   # E > 1024
        ft.make_desc(288, 2048, 768, 17, 1),   # k > 16
        ft.make_desc(288, 2000, 768, 8, 1),    # H not a multiple of 256
        ft.make_desc(288, 2048, 760, 8, 1),    # I not a multiple of 64
        ft.make_desc(288, 2048, 768, 8, 2),    # act
        ft.make_desc(288, 2048, 768, 8, 1, shared_inter=100),
    ]
    for d in bad:
        assert ft.ft_moe_workspace_bytes(d, 1, 1) == 0


def test_workspace_bytes_never_shrink_with_tokens(ft):
    """A workspace sized for T tokens serves every smaller T (the header's
    contract): the size is non-decreasing in T on every path, across the token
    counts where the router and the grouped path change form (4/5, 7/8, 23/24,
    63/64/65, 1023/1024) and across the split router's token-block boundaries."""
    descs = [ft.make_desc(288, 2048, 768, 8, 1),
             ft.make_desc(512, 2048, 512, 10, 1, shared_inter=512),
             ft.make_desc(1024, 4096, 1024, 16, 1, shared_inter=256),
             ft.make_desc(8, 256, 128, 2, 0)]
    Ts = list(range(0, 130)) + list(range(130, 1100, 7)) + [1023, 1024, 1025, 4096, 8192]
    for d in descs:
        for path in (0, 1, 2):
            sizes = [ft.ft_moe_workspace_bytes(d, T, path) for T in sorted(set(Ts))]
            assert all(b >= a for a, b in zip(sizes, sizes[1:])), (path, sizes[:8])


def _raw(ft):
    return ft._lib


def test_host_validation_status_codes(ft):
    lib = _raw(ft)
    d = ft.make_desc(288, 2048, 768, 8, 1)
    dp = ctypes.byref(d)
    # NULL descriptor
    assert lib.ft_moe_route(None, 1, 16, 16, None, 16, 16, 256, 1 << 20, None) == ft.FT_EINVAL
    assert "desc" in ft.ft_last_error()
    # NULL x
    assert lib.ft_moe_route(dp, 1, None, 16, None, 16, 16, 256, 1 << 20, None) == ft.FT_EINVAL
    # misaligned x
    assert lib.ft_moe_route(dp, 1, 18, 16, None, 16, 16, 256, 1 << 20, None) == ft.FT_EINVAL
    # workspace too small / misaligned / NULL
    assert lib.ft_moe_route(dp, 1, 16, 16, None, 16, 16, 256, 8, None) == ft.FT_EWORKSPACE
    assert lib.ft_moe_route(dp, (1 << 21) + 1, 16, 16, None, 16, 16, 256, 1 << 62,
                            None) == ft.FT_EUNSUPPORTED
    assert lib.ft_moe_route(dp, 1, 16, 16, None, 16, 16, 272, 1 << 20, None) == ft.FT_EWORKSPACE
    assert lib.ft_moe_route(dp, 1, 16, 16, None, 16, 16, None, 1 << 20, None) == ft.FT_EWORKSPACE
    # decode token range
    bank = ft.FtNvfp4Experts(256, 256, 256, 256, 256)
    b = ctypes.byref(bank)
    args = (16, None, b, None, None, None, None, 16, 256, 1 << 24, None)
    assert lib.ft_moe_nvfp4_decode(dp, 0, 16, *args) == ft.FT_EINVAL
    assert lib.ft_moe_nvfp4_decode(dp, 65, 16, *args) == ft.FT_EUNSUPPORTED
    # shared expert declared but no bank
    ds = ft.make_desc(512, 2048, 512, 10, 1, shared_inter=512)
    assert lib.ft_moe_nvfp4_decode(ctypes.byref(ds), 1, 16, 16, None, b, None, 16, None, None,
                                   16, 256, 1 << 24, None) == ft.FT_EINVAL
    assert "shared" in ft.ft_last_error()
    # routed bank with a NULL part
    nb = ft.FtNvfp4Experts(256, None, 256, 256, 256)
    assert lib.ft_moe_nvfp4_decode(dp, 1, 16, 16, None, ctypes.byref(nb), None, None, None,
                                   None, 16, 256, 1 << 24, None) == ft.FT_EINVAL
    # prefill needs routes
    assert lib.ft_moe_nvfp4_prefill(dp, 4, 16, None, 16, b, None, None, 16, 256, 1 << 24,
                                    None) == ft.FT_EINVAL
    # dequant argument checks
    assert lib.ft_nvfp4_dequant(2048, 768, 8, b, 8, 0, 0, 16, None) == ft.FT_EINVAL
    assert lib.ft_nvfp4_dequant(2048, 768, 8, b, 0, 3, 0, 16, None) == ft.FT_EINVAL
    assert lib.ft_nvfp4_dequant(2048, 768, 8, b, 0, 0, 5, 16, None) == ft.FT_EINVAL
    assert lib.ft_nvfp4_dequant(2048, 768, 8, b, 0, 0, 2, 24, None) == ft.FT_EINVAL  # alignment
    assert lib.ft_nvfp4_dequant(2000, 768, 8, b, 0, 0, 0, 16, None) == ft.FT_EUNSUPPORTED
    # repack argument checks
    assert lib.ft_nvfp4_repack(2048, 768, 8, *([16] * 7), None, None) == ft.FT_EINVAL
    assert lib.ft_nvfp4_repack(2048, 100, 8, *([16] * 8), None) == ft.FT_EUNSUPPORTED


def test_attn_cache_scale_validation(ft):
    lib = _raw(ft)
    for fmt, ks, vs in ((1, 0.0, 1.0), (2, 1.0, -0.5), (2, float("inf"), 1.0), (1, 1.0, float("nan"))):
        c = ft.FtKvCache(fmt, 64, 256, 256, 256, 256, ks, vs)
        assert lib.ft_attn_extend(8, 8, 2, 64, 0, 256, 256, 256, ctypes.byref(c), 256,
                                  None) == ft.FT_EINVAL
        assert "k_scale and v_scale" in ft.ft_last_error()


def test_device_status_and_wait_limit_validation(ft):
    lib = _raw(ft)
    assert lib.ft_moe_device_status(None, 1 << 20, 16, None) == ft.FT_EINVAL
    assert lib.ft_moe_device_status(256, 1 << 20, None, None) == ft.FT_EINVAL
    assert lib.ft_moe_device_status(272, 1 << 20, 16, None) == ft.FT_EWORKSPACE
    assert lib.ft_moe_device_status(256, 128, 16, None) == ft.FT_EWORKSPACE
    assert lib.ft_moe_device_status(256, 1 << 20, 18, None) == ft.FT_EINVAL
    assert lib.ft_set_wait_limit(-1) == ft.FT_EINVAL
    assert lib.ft_set_wait_limit(0) == ft.FT_OK


def test_zero_tokens_route_enqueues_nothing(ft):
    lib = _raw(ft)
    d = ft.make_desc(288, 2048, 768, 8, 1)
    n = ft.ft_moe_workspace_bytes(d, 0, 0)
    assert lib.ft_moe_route(ctypes.byref(d), 0, 16, 16, None, 16, 16, 256, n, None) == ft.FT_OK
