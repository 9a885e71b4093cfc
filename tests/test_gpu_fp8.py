"""GPU parity of the block-fp8 expert codec (e4m3 weights, one fp32 scale per
128 x 128 block) through ft_moe_fp8_decode and the ft_fp8_dequant export, against
the CPU oracle, through the C ABI.  Dequantised weights bit-exact (both device
routines, every byte including the NaN encodings); top-k ids bit-exact; routing
weights within 2 fp32 ulp; bf16 outputs within max_abs_rel 1e-2, rel_l2 2e-3."""
import ctypes
import functools

import numpy as np
import pytest
import torch

import oracle
from nvfp4_mixture_experts_amd import synth
from tests.gpu_util import assert_output_close, f32_ulp_diff, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_mixture_experts_amd import device, ftmoe
    ftmoe.ft_init(0)
    return device


@functools.lru_cache(maxsize=2)
def _host(name, **over):
    w = synth.WORKLOADS[name]
    if over:
        w = synth.dataclasses.replace(w, **over)
    return synth.make_fp8_layer(w)


def _bits_equal_with_nan(got, want):
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn)
    assert np.array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32))


@pytest.mark.parametrize("mode", [0, 1])   # down-GEMV routine, gate|up-GEMV routine
def test_fp8_dequant_bit_exact_every_byte(gpu, mode):
    from nvfp4_mixture_experts_amd import ftmoe
    H, I, n = 256, 128, 2
    rng = np.random.default_rng(21)
    w13c = np.tile(np.arange(256, dtype=np.uint8), (n, 2 * I, H // 256))   # every byte, NaNs too
    w13c = np.ascontiguousarray(w13c[:, :, rng.permutation(H)])
    w13s = (rng.random((n, 2 * I // 128, H // 128)) * 3e-3 + 1e-5).astype(np.float32)
    w2c = rng.integers(0, 256, (n, H, I), dtype=np.uint8)
    w2s = (rng.random((n, H // 128, I // 128)) * 3e-3 + 1e-5).astype(np.float32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bank = ftmoe.ft_fp8_repack(H, I, n, d(w13c), d(w13s), d(w2c), d(w2s))
    for e in range(n):
        for tensor in (0, 1, 2):
            rows, K = (H, I) if tensor == 2 else (I, H)
            out = torch.empty((rows, K), dtype=torch.float32, device="cuda")
            ftmoe.ft_fp8_dequant(bank, e, tensor, out, mode=mode)
            torch.cuda.synchronize()
            if tensor == 2:
                want = oracle.fp8_dequant_matrix(w2c[e], w2s[e])
            else:
                sl = slice(0, I) if tensor == 0 else slice(I, 2 * I)
                bs = slice(0, I // 128) if tensor == 0 else slice(I // 128, 2 * I // 128)
                want = oracle.fp8_dequant_matrix(w13c[e, sl], w13s[e, bs])
            _bits_equal_with_nan(out.cpu().numpy(), want)


@pytest.mark.parametrize("tokens,rows", [(1, None), (3, None), (7, [0, 3, 6])])
def test_fp8_decode_matches_oracle(gpu, tokens, rows):
    from tests.gpu_util import decode_checked  # noqa: F401  (status checked below)
    name = "decode_e512_top10_shared_fp8"
    w = synth.WORKLOADS[name]
    L = _host(name)
    dl = gpu.upload_fp8_layer(L)
    x = synth.make_tokens(w, tokens=tokens, stream="fp8")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    y, ids, wt = gpu.decode_fp8(dl, gpu.tokens_to_device(x), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rows = list(range(tokens)) if rows is None else rows
    ref = oracle.moe_layer_fp8(L, x[rows])
    assert np.array_equal(ids.cpu().numpy()[rows], ref["ids"])
    assert f32_ulp_diff(wt.cpu().numpy()[rows], ref["weights"]).max() <= 2
    assert_output_close(gpu.bf16_bits(y)[rows], ref["y"], f"{name} T={tokens}")


@pytest.mark.parametrize("H,I,E,k,Is", [(1024, 256, 40, 6, 0), (4096, 128, 24, 4, 128),
                                         (3072, 384, 32, 8, 256)])
def test_fp8_decode_other_shapes(gpu, H, I, E, k, Is):
    L = _host("decode_e512_top10_shared_fp8", hidden=H, inter=I, num_experts=E, top_k=k,
              shared_inter=Is)
    x = synth.make_tokens(L.workload, tokens=2, stream="fp8s")
    dl = gpu.upload_fp8_layer(L)
    y, ids, _ = gpu.decode_fp8(dl, gpu.tokens_to_device(x))
    torch.cuda.synchronize()
    ref = oracle.moe_layer_fp8(L, x)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_output_close(gpu.bf16_bits(y), ref["y"], f"fp8 H={H} I={I} E={E} k={k} Is={Is}")


def test_fp8_decode_is_deterministic_and_rejects_grouped_counts(gpu):
    from nvfp4_mixture_experts_amd import ftmoe
    name = "decode_e512_top10_shared_fp8"
    L = _host(name)
    dl = gpu.upload_fp8_layer(L)
    x = gpu.tokens_to_device(synth.make_tokens(L.workload, tokens=2, stream="fp8d"))
    a, _, _ = gpu.decode_fp8(dl, x)
    b, _, _ = gpu.decode_fp8(dl, x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    bank = ftmoe.FtFp8Experts(256, 256, 256, 256)
    st = ftmoe._lib.ft_moe_fp8_decode(ctypes.byref(dl.desc), 8, 16, 16, None, ctypes.byref(bank),
                                      ctypes.byref(bank), 16, None, None, 16, 256, 1 << 24, None)
    assert st == ftmoe.FT_EUNSUPPORTED
