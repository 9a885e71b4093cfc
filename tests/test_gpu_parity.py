"""GPU parity of libftmoe.so against the CPU oracle, through the C ABI.

Bit-exact: dequantised weights (all 16 codes x all 256 scale bytes, and random
banks through the repack) and top-k expert ids.  Routing weights: within 2 fp32
ulps.  bf16 layer outputs: max_abs_rel <= 1e-2 and rel_l2 <= 2e-3 against the
oracle's bf16-rounded output.
"""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_mixture_experts_amd import synth
from tests.gpu_util import (assert_output_close, decode_checked, f32_ulp_diff, host_layer,
                            oracle_layer_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_mixture_experts_amd import device, ftmoe
    ftmoe.ft_init(0)
    say(f"libftmoe: {ftmoe.library_path()}")
    return device


_uploaded = {}


def dev_layer(gpu, name, **overrides):
    key = (name, tuple(sorted(overrides.items())))
    if key not in _uploaded:
        if len(_uploaded) >= 3:
            _uploaded.clear()
            torch.cuda.empty_cache()
        say(f"  upload {name} {overrides}")
        _uploaded[key] = gpu.upload_layer(host_layer(name, **overrides))
    return _uploaded[key]


# ---------------------------------------------------------------- dequant --

def _all_codes_bank(H=256, I=64, n=2, g=(1.0, 0.3, 2.0 ** -6)):
    """Gate rows 0..15 of expert 0 carry all 256 scale bytes, each block all 16 codes."""
    rng = np.random.default_rng(42)
    w13c = rng.integers(0, 256, (n, 2 * I, H // 2), dtype=np.uint8)
    w13s = synth.SCALE_BYTES[rng.integers(0, 7, (n, 2 * I, H // 16))]
    w13c[0, :16, :] = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE],
                                       np.uint8), H // 16)
    w13s[0, :16, :] = np.arange(256, dtype=np.uint8).reshape(16, 16)
    w2c = rng.integers(0, 256, (n, H, I // 2), dtype=np.uint8)
    w2s = synth.SCALE_BYTES[rng.integers(0, 7, (n, H, I // 16))]
    w2s[0, :64, :] = np.arange(256, dtype=np.uint8).reshape(64, 4)
    gsc = np.tile(np.array(g, np.float32), (n, 1))
    return dict(w13_codes=w13c, w13_scales=w13s, w2_codes=w2c, w2_scales=w2s, global_scale=gsc)


def _bits_equal_with_nan(got, want):
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn)
    assert np.array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32))


def _check_f16_tile(bank, e, tensor, rows, K, want1):
    """ft_nvfp4_dequant mode 4 (the fp16 MFMA tile builder) against the oracle's
    code x scale: every value is exactly representable in fp16, so the converted
    oracle value must match bit for bit (NaN where the scale is NaN)."""
    from nvfp4_mixture_experts_amd import ftmoe
    out16 = torch.empty((rows, K), dtype=torch.float16, device="cuda")
    ftmoe.ft_nvfp4_dequant(bank, e, tensor, out16, mode=ftmoe.DEQ_TILE_F16)
    torch.cuda.synchronize()
    got = out16.cpu().numpy()
    n1 = np.isnan(want1)
    want16 = want1.astype(np.float16)
    assert np.array_equal(want16[~n1].astype(np.float32), want1[~n1])  # exact in fp16
    assert np.array_equal(np.isnan(got), n1)
    assert np.array_equal(got[~n1].view(np.uint16), want16[~n1].view(np.uint16))


@pytest.mark.parametrize("tensor", [0, 1, 2])
def test_dequant_bit_exact_all_codes_and_scales(gpu, tensor):
    from nvfp4_mixture_experts_amd import ftmoe
    H, I, n = 256, 64, 2
    b = _all_codes_bank(H, I, n)
    dev = lambda a: torch.from_numpy(a).cuda()
    bank = ftmoe.ft_nvfp4_repack(H, I, n, dev(b["w13_codes"]), dev(b["w13_scales"]),
                                 dev(b["w2_codes"]), dev(b["w2_scales"]), dev(b["global_scale"]))
    for e in range(n):
        rows, K = (H, I) if tensor == 2 else (I, H)
        out = torch.empty((rows, K), dtype=torch.float32, device="cuda")
        ftmoe.ft_nvfp4_dequant(bank, e, tensor, out)
        outb = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
        ftmoe.ft_nvfp4_dequant(bank, e, tensor, outb)
        torch.cuda.synchronize()
        g = float(b["global_scale"][e, tensor])
        if tensor == 2:
            want = oracle.dequant_matrix(b["w2_codes"][e], b["w2_scales"][e], g)
        else:
            sl = slice(0, I) if tensor == 0 else slice(I, 2 * I)
            want = oracle.dequant_matrix(b["w13_codes"][e, sl], b["w13_scales"][e, sl], g)
        got = out.cpu().numpy()
        _bits_equal_with_nan(got, want)
        wantb = np.array([oracle.bf16_from_double(float(v)) for v in want.ravel()],
                         np.uint16).reshape(want.shape)
        gotb = outb.cpu().view(torch.int16).numpy().view(np.uint16)
        nanb = np.isnan(want)
        assert np.array_equal(gotb[~nanb], wantb[~nanb])
        # the one-launch decode kernel's gate|up routine (codes -> bf16 pairs)
        outg = torch.empty((rows, K), dtype=torch.float32, device="cuda")
        ftmoe.ft_nvfp4_dequant(bank, e, tensor, outg, mode=ftmoe.DEQ_GATEUP_F32)
        # the grouped / prefill MFMA tile builder: bf16 code x scale, no global scale
        outt = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
        ftmoe.ft_nvfp4_dequant(bank, e, tensor, outt, mode=ftmoe.DEQ_TILE_BF16)
        torch.cuda.synchronize()
        _bits_equal_with_nan(outg.cpu().numpy(), want)
        if tensor == 2:
            want1 = oracle.dequant_matrix(b["w2_codes"][e], b["w2_scales"][e], 1.0)
        else:
            want1 = oracle.dequant_matrix(b["w13_codes"][e, sl], b["w13_scales"][e, sl], 1.0)
        n1 = np.isnan(want1)
        # code x scale is exact in bf16: the oracle's fp32 value has empty low halves
        assert np.all(want1[~n1].view(np.uint32) & 0xFFFF == 0)
        gott = outt.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(gott[~n1], (want1[~n1].view(np.uint32) >> 16).astype(np.uint16))
        tv = (gott.astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(np.isnan(tv), n1)
        # the fp16 tile builder of the down GEMMs (h in fp16): code x scale is exact in
        # fp16 as well, so its bits are the oracle's value converted
        _check_f16_tile(bank, e, tensor, rows, K, want1)


def test_dequant_bit_exact_workload_bank(gpu):
    """Every tensor of two experts of the 288-expert decode layer, after the repack."""
    from nvfp4_mixture_experts_amd import ftmoe
    dl = dev_layer(gpu, "decode_e288_top8")
    L = host_layer("decode_e288_top8")
    I, H = L.inter, L.hidden
    for e in (0, 287):
        for tensor in (0, 1, 2):
            rows, K = (H, I) if tensor == 2 else (I, H)
            out = torch.empty((rows, K), dtype=torch.float32, device="cuda")
            ftmoe.ft_nvfp4_dequant(dl.routed, e, tensor, out)
            outg = torch.empty((rows, K), dtype=torch.float32, device="cuda")
            ftmoe.ft_nvfp4_dequant(dl.routed, e, tensor, outg, mode=ftmoe.DEQ_GATEUP_F32)
            outt = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
            ftmoe.ft_nvfp4_dequant(dl.routed, e, tensor, outt, mode=ftmoe.DEQ_TILE_BF16)
            g = float(L.global_scale[e, tensor])
            if tensor == 2:
                want = oracle.dequant_matrix(L.w2_codes[e], L.w2_scales[e], g)
                want1 = oracle.dequant_matrix(L.w2_codes[e], L.w2_scales[e], 1.0)
            else:
                sl = slice(0, I) if tensor == 0 else slice(I, 2 * I)
                want = oracle.dequant_matrix(L.w13_codes[e, sl], L.w13_scales[e, sl], g)
                want1 = oracle.dequant_matrix(L.w13_codes[e, sl], L.w13_scales[e, sl], 1.0)
            assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
            assert np.array_equal(outg.cpu().numpy().view(np.uint32), want.view(np.uint32))
            gott = outt.cpu().view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(gott, (want1.view(np.uint32) >> 16).astype(np.uint16))
            _check_f16_tile(dl.routed, e, tensor, rows, K, want1)


# ------------------------------------------------------------------ route --

def _check_routes(ids, w, ref_ids, ref_w, what):
    ids = ids.cpu().numpy()
    w = w.cpu().numpy()
    assert np.array_equal(ids, ref_ids), f"{what}: ids differ"
    ulps = f32_ulp_diff(w, ref_w)
    say(f"  {what}: ids exact, weights max ulp diff {ulps.max()}, exact {np.mean(ulps == 0):.4f}")
    assert ulps.max() <= 2


@pytest.mark.parametrize("name,tokens", [("tiny_e8_top2", 1), ("decode_e288_top8", 1),
                                         ("decode_e512_top10_shared", 1),
                                         ("batched_decode_t32_hot64", 32),
                                         ("decode_e512_top10_shared", 64),
                                         ("decode_e512_top10_shared", 333),
                                         # split-K router; 289 rows (not a multiple of 64)
                                         ("decode_e288_top8", 100),
                                         # MFMA router; experts not a multiple of 64
                                         ("decode_e288_top8", 1100)])
def test_route_matches_oracle(gpu, name, tokens):
    w = synth.WORKLOADS[name]
    dl = dev_layer(gpu, name)
    L = host_layer(name)
    x = synth.make_tokens(w, tokens=tokens, stream=f"route{tokens}")
    ids, wt = gpu.route(dl, gpu.tokens_to_device(x))
    torch.cuda.synchronize()
    logits = oracle.router_logits(x, L.w_router, L.bias)
    ref_ids, ref_w = oracle.topk(logits, w.top_k)
    _check_routes(ids, wt, ref_ids, ref_w, f"{name} T={tokens}")


@pytest.mark.parametrize("tokens", [16, 40, 1100])  # row, split-K and bounded routers
def test_route_ties_go_to_lowest_index(gpu, tokens):
    """Duplicated router rows give exactly equal logits; the lower index must win."""
    from nvfp4_mixture_experts_amd import ftmoe
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e288_top8"], num_experts=96)
    L = synth.make_layer(w)
    wr = L.w_router.copy()
    wr[50:96] = wr[0:46]                      # experts 50.. duplicate 0..45
    wr[10] = wr[70]                           # and a tie inside the copy
    x = synth.make_tokens(w, tokens=tokens, stream="ties")
    xd = gpu.tokens_to_device(x)
    desc = ftmoe.make_desc(96, w.hidden, w.inter, w.top_k, 1)
    wsp = ftmoe.alloc_workspace(desc, tokens, ftmoe.PATH_ROUTE)
    ids = torch.empty((tokens, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((tokens, w.top_k), dtype=torch.float32, device="cuda")
    ftmoe.ft_moe_route(desc, xd, torch.from_numpy(wr).cuda(), None, ids, wt, wsp)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.topk(oracle.router_logits(x, wr), w.top_k)
    # every token must have at least one tie inside its top-k for the test to bite
    lg = oracle.router_logits(x, wr)
    ties = sum(len(set(lg[t, ref_ids[t]].tolist())) < w.top_k for t in range(tokens))
    assert ties > 0
    _check_routes(ids, wt, ref_ids, ref_w, "ties")


def _zero_nan_router(E, H, rng):
    """Router rows whose logits round to +0 or -0 (one tiny product of either sign,
    or an all-zero row), NaN (a NaN weight), or clearly negative numbers, for tokens
    whose elements are positive and whose element 0 is tiny."""
    wr = -np.abs(rng.standard_normal((E, H)).astype(np.float32) * np.float32(0.02))
    for e in range(10):                          # +0 / -0 / exact zero
        wr[e] = 0.0
        wr[e, 0] = [1e-30, -1e-30, 0.0][e % 3]
    for e in range(10, 14):
        wr[e, 5] = np.nan
    return wr


def _zero_nan_tokens(T, H, rng):
    xf = np.abs(rng.standard_normal((T, H)).astype(np.float32)) + np.float32(0.05)
    xf[:, 0] = np.float32(1e-30)
    return synth.bf16_bits_from_f32(xf)


def _routes_nan_aware(ids, w, ref_ids, ref_w, what):
    ids = ids.cpu().numpy()
    w = w.cpu().numpy()
    assert np.array_equal(ids, ref_ids), f"{what}: ids differ\n{ids}\n{ref_ids}"
    assert np.array_equal(np.isnan(w), np.isnan(ref_w)), what
    ok = ~np.isnan(ref_w)
    assert f32_ulp_diff(w[ok], ref_w[ok]).max(initial=0) <= 2, what
    say(f"  {what}: ids exact")


@pytest.mark.parametrize("E,k", [(24, 16), (18, 16), (64, 12)])
@pytest.mark.parametrize("tokens", [1, 3, 16, 40, 1100])   # every router and top-k kernel
def test_route_signed_zero_and_nan_logits(gpu, E, k, tokens):
    """Logits of +0 and -0 compare equal (the lower index wins), a NaN logit ranks
    below every number; the oracle decides."""
    from nvfp4_mixture_experts_amd import ftmoe
    H = 256
    rng = np.random.default_rng(100 + E + tokens)
    wr = _zero_nan_router(E, H, rng)
    x = _zero_nan_tokens(tokens, H, rng)
    logits = oracle.router_logits(x, wr)
    assert np.all(np.signbit(logits[:, 1]) & (logits[:, 1] == 0))      # -0 logits
    assert np.all((logits[:, 0] == 0) & ~np.signbit(logits[:, 0]))     # +0 logits
    assert np.all(np.isnan(logits[:, 10:14]))
    ref_ids, ref_w = oracle.topk(logits, k)
    desc = ftmoe.make_desc(E, H, 128, k, 1)
    ws = ftmoe.alloc_workspace(desc, tokens, ftmoe.PATH_ROUTE)
    ids = torch.empty((tokens, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((tokens, k), dtype=torch.float32, device="cuda")
    ftmoe.ft_moe_route(desc, gpu.tokens_to_device(x), torch.from_numpy(wr).cuda(), None, ids, wt,
                       ws)
    torch.cuda.synchronize()
    _routes_nan_aware(ids, wt, ref_ids, ref_w, f"route E={E} k={k} T={tokens}")


@pytest.mark.parametrize("E", [24, 18])        # 18: two NaN logits among the top 16
@pytest.mark.parametrize("tokens", [1, 4, 12])   # fused kernel (one token, several), grouped
def test_decode_routes_signed_zero_and_nan_logits(gpu, E, tokens):
    k, H = 16, 256
    w = synth.dataclasses.replace(synth.WORKLOADS["tiny_e8_top2"], num_experts=E, top_k=k,
                                  hidden=H, inter=128)
    layer = synth.make_layer(w)
    rng = np.random.default_rng(7 + tokens)
    layer.w_router = _zero_nan_router(E, H, rng)
    x = _zero_nan_tokens(tokens, H, rng)
    ref_ids, ref_w = oracle.topk(oracle.router_logits(x, layer.w_router), k)
    dl = gpu.upload_layer(layer)
    y, ids, wt = decode_checked(gpu, dl, gpu.tokens_to_device(x))
    _routes_nan_aware(ids, wt, ref_ids, ref_w, f"decode E={E} k={k} T={tokens}")
    if not np.isnan(ref_w).any():
        ref = oracle.moe_layer(layer, x)
        assert_output_close(gpu.bf16_bits(y), ref["y"], f"decode, zero logits, T={tokens}")


@pytest.mark.parametrize("tokens", [16, 64])   # the one-launch routing of a decode batch
def test_decode_routes_ties_go_to_lowest_index(gpu, tokens):
    """Duplicated router rows give exactly equal logits: the routing kernel of a decode
    batch must pick the lower index, as the oracle does; the layer output follows."""
    w = synth.dataclasses.replace(synth.WORKLOADS["tiny_e8_top2"], num_experts=96, top_k=8,
                                  hidden=512, inter=128)
    layer = synth.make_layer(w)
    wr = layer.w_router.copy()
    wr[50:96] = wr[0:46]                      # experts 50.. duplicate 0..45
    wr[10] = wr[70]                           # and a tie inside the copy
    layer.w_router = wr
    x = synth.make_tokens(w, tokens=tokens, stream="ties")
    lg = oracle.router_logits(x, wr)
    ref_ids, ref_w = oracle.topk(lg, w.top_k)
    assert sum(len(set(lg[t, ref_ids[t]].tolist())) < w.top_k for t in range(tokens)) > 0
    dl = gpu.upload_layer(layer)
    y, ids, wt = decode_checked(gpu, dl, gpu.tokens_to_device(x))
    _check_routes(ids, wt, ref_ids, ref_w, f"decode ties T={tokens}")
    ref = oracle.moe_layer(layer, x)
    assert_output_close(gpu.bf16_bits(y), ref["y"], f"decode ties T={tokens}")


@pytest.mark.parametrize("num_experts", [1000, 1024])
def test_decode_batch_many_experts(gpu, num_experts):
    """40 tokens over 1000 / 1024 experts with a router bias and a shared expert: the
    routing kernel's two logits per selecting thread, four K splits over 63 / 64 row
    tiles (the last one partial for 1000), and the grouping of 400 pairs."""
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"],
                                  num_experts=num_experts, hidden=512, inter=128,
                                  shared_inter=128, tokens=40)
    layer = synth.make_layer(w)
    layer.bias = (np.random.default_rng(num_experts).standard_normal(num_experts)
                  * 0.05).astype(np.float32)
    x = synth.make_tokens(w)
    dl = gpu.upload_layer(layer)
    y, ids, wt = decode_checked(gpu, dl, gpu.tokens_to_device(x))
    ref = oracle.moe_layer(layer, x)
    _check_routes(ids, wt, ref["ids"], ref["weights"], f"decode E={num_experts} T=40")
    assert_output_close(gpu.bf16_bits(y), ref["y"], f"decode E={num_experts} T=40")


@pytest.mark.parametrize("num_experts", [1000, 1024])
def test_route_many_experts_split_router(gpu, num_experts):
    """40 tokens (split-K router) with 1000 and 1024 experts and a router bias: the
    widest split-router blocks (8 waves), two row passes in the per-token top-k, and
    for 1024 (a multiple of the top-k block's 512 threads) row E loaded by lanes."""
    from nvfp4_mixture_experts_amd import ftmoe
    tokens = 40
    w = synth.dataclasses.replace(synth.WORKLOADS["batched_decode_t32_hot64"],
                                  num_experts=num_experts)
    wr, bias = synth.make_router(w)
    assert bias is not None
    x = synth.make_tokens(w, tokens=tokens, stream="many_experts")
    desc = ftmoe.make_desc(num_experts, w.hidden, w.inter, w.top_k, 1)
    wsp = ftmoe.alloc_workspace(desc, tokens, ftmoe.PATH_ROUTE)
    ids = torch.empty((tokens, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((tokens, w.top_k), dtype=torch.float32, device="cuda")
    ftmoe.ft_moe_route(desc, gpu.tokens_to_device(x), torch.from_numpy(wr).cuda(),
                       torch.from_numpy(bias).cuda(), ids, wt, wsp)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.topk(oracle.router_logits(x, wr, bias), w.top_k)
    _check_routes(ids, wt, ref_ids, ref_w, f"E={num_experts} T={tokens}")


@pytest.mark.parametrize("num_experts", [1000, 1024, 200])
def test_route_bounded_many_tokens(gpu, num_experts):
    """1100 tokens (the bounded router: bf16 approximations, exact recheck of the
    experts the error bound leaves in play) with 1000, 1024 and 200 experts and a
    router bias, every token against the oracle."""
    from nvfp4_mixture_experts_amd import ftmoe
    tokens = 1100
    w = synth.dataclasses.replace(synth.WORKLOADS["batched_decode_t32_hot64"],
                                  num_experts=num_experts, hot_experts=min(64, num_experts // 4))
    wr, bias = synth.make_router(w)
    assert bias is not None
    x = synth.make_tokens(w, tokens=tokens, stream="bounded")
    desc = ftmoe.make_desc(num_experts, w.hidden, w.inter, w.top_k, 1)
    wsp = ftmoe.alloc_workspace(desc, tokens, ftmoe.PATH_ROUTE)
    ids = torch.empty((tokens, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((tokens, w.top_k), dtype=torch.float32, device="cuda")
    ftmoe.ft_moe_route(desc, gpu.tokens_to_device(x), torch.from_numpy(wr).cuda(),
                       torch.from_numpy(bias).cuda(), ids, wt, wsp)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.topk(oracle.router_logits(x, wr, bias), w.top_k)
    _check_routes(ids, wt, ref_ids, ref_w, f"bounded E={num_experts} T={tokens}")


def test_route_bounded_nonfinite_tokens(gpu):
    """Tokens with an infinite or NaN activation among 1100 finite ones: those tokens
    take every expert exactly (their logits are infinite or NaN), the others the
    bounded candidates; the oracle decides ids (ties of +inf to the lower index) and
    which weights are NaN."""
    from nvfp4_mixture_experts_amd import ftmoe
    tokens, E, k, H = 1100, 64, 6, 512
    rng = np.random.default_rng(77)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    xf = rng.standard_normal((tokens, H)).astype(np.float32)
    xf[3, 10] = np.inf
    xf[700, 0] = -np.inf
    xf[5, 99] = np.nan
    x = synth.bf16_bits_from_f32(xf)
    logits = oracle.router_logits(x, wr)
    ref_ids, ref_w = oracle.topk(logits, k)
    assert np.isinf(logits[3]).all() and np.isnan(logits[5]).all()
    desc = ftmoe.make_desc(E, H, 128, k, 1)
    ws = ftmoe.alloc_workspace(desc, tokens, ftmoe.PATH_ROUTE)
    ids = torch.empty((tokens, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((tokens, k), dtype=torch.float32, device="cuda")
    ftmoe.ft_moe_route(desc, gpu.tokens_to_device(x), torch.from_numpy(wr).cuda(), None, ids, wt,
                       ws)
    torch.cuda.synchronize()
    _routes_nan_aware(ids, wt, ref_ids, ref_w, "bounded router, non-finite tokens")


# ----------------------------------------------------------------- decode --

@pytest.mark.parametrize("name,tokens,sample", [
    ("tiny_e8_top2", 1, None),
    ("decode_e288_top8", 1, None),
    ("decode_e512_top10_shared", 1, None),
    ("batched_decode_t32_hot64", 32, None),        # every token of the batched workload
    ("decode_e288_top8", 2, None),                # fused kernel, several tokens, I = 768
    ("batched_decode_t32_hot64", 7, [0, 6]),     # largest count on the fused kernel
    ("batched_decode_t32_hot64", 8, [0, 7]),     # smallest count on the grouped path
    ("tiny_e8_top2", 64, [0, 63]),
])
def test_decode_matches_oracle(gpu, name, tokens, sample):
    w = synth.WORKLOADS[name]
    dl = dev_layer(gpu, name)
    L = host_layer(name)
    x = synth.make_tokens(w, tokens=tokens)
    y, ids, wt = decode_checked(gpu, dl, gpu.tokens_to_device(x))
    torch.cuda.synchronize()
    yb = gpu.bf16_bits(y)
    rows = list(range(tokens)) if sample is None else sample
    ref = oracle_layer_rows(L, x, rows)
    assert np.array_equal(ids.cpu().numpy()[rows], ref["ids"])
    assert f32_ulp_diff(wt.cpu().numpy()[rows], ref["weights"]).max() <= 2
    assert_output_close(yb[rows], ref["y"], f"{name} T={tokens}")
    if sample is not None:   # the other tokens: routes checked against the oracle router
        ref_ids, _ = oracle.topk(oracle.router_logits(x, L.w_router, L.bias), w.top_k)
        assert np.array_equal(ids.cpu().numpy(), ref_ids)


def _host_layer_of(w, d):
    """The oracle's inputs (a host Layer) from a layer instance drawn on the device."""
    def host(t):
        return None if t is None else t.cpu().numpy()
    L = synth.Layer(workload=w, w_router=host(d["w_router"]).astype(np.float32),
                    bias=host(d["bias"]), **{k: host(v) for k, v in d["routed"].items()})
    if d["shared"] is not None:
        sb = d["shared"]
        L.s13_codes, L.s13_scales = host(sb["w13_codes"]), host(sb["w13_scales"])
        L.s2_codes, L.s2_scales = host(sb["w2_codes"]), host(sb["w2_scales"])
        L.s_global = host(sb["global_scale"])
        L.shared_gate = d["shared_gate"].cpu().view(torch.int16).numpy().view(np.uint16)
    return L


@pytest.mark.parametrize("name,instances,tokens,rows", [
    ("decode_e288_top8", (1, 23, 45), 1, [0]),
    ("decode_e512_top10_shared", (1, 23, 45), 1, [0]),
    ("batched_decode_t32_hot64", (1, 11), 32, [0, 5, 13, 31]),
])
def test_decode_timed_instances_match_oracle(gpu, name, instances, tokens, rows):
    """Layer instances that the benchmark times (drawn on the device; the last of them
    among these), downloaded as the oracle's inputs: the routes of every token, and the
    routing weights and outputs of the sampled ones."""
    w = synth.WORKLOADS[name]
    for inst in instances:
        d = synth.make_layer_device(w, inst, torch.device("cuda"))
        dl = gpu.upload_canonical(w, d["w_router"], d["bias"], d["routed"], d["shared"],
                                  d["shared_gate"], "cuda")
        L = _host_layer_of(w, d)
        del d
        x = synth.make_tokens(w, instance=inst, tokens=tokens)
        y, ids, wt = decode_checked(gpu, dl, gpu.tokens_to_device(x))
        ref = oracle_layer_rows(L, x, rows)
        assert np.array_equal(ids.cpu().numpy()[rows], ref["ids"])
        assert f32_ulp_diff(wt.cpu().numpy()[rows], ref["weights"]).max() <= 2
        assert_output_close(gpu.bf16_bits(y)[rows], ref["y"], f"{name} instance {inst}")
        if tokens > 1:
            ref_ids, _ = oracle.topk(oracle.router_logits(x, L.w_router, L.bias), w.top_k)
            assert np.array_equal(ids.cpu().numpy(), ref_ids)
        del dl, L
        torch.cuda.empty_cache()


def test_decode_all_experts_selected(gpu):
    """k = E: the layer is the dense softmax mixture of every expert."""
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"], num_experts=16,
                                  top_k=16, global_scale=2.0 ** -4)
    L = synth.make_layer(w)
    dl = gpu.upload_layer(L)
    x = synth.make_tokens(w, tokens=3)
    y, ids, _ = decode_checked(gpu, dl, gpu.tokens_to_device(x))
    torch.cuda.synchronize()
    ref = oracle.moe_layer(L, x)
    assert np.array_equal(np.sort(ids.cpu().numpy(), axis=1), np.tile(np.arange(16), (3, 1)))
    assert_output_close(gpu.bf16_bits(y), ref["y"], "all experts")


def test_decode_shapes_outside_the_workloads(gpu):
    """H = 512 (16 lanes per row), I = 192, shared I = 128 != I, T = 5, plain SwiGLU."""
    w = synth.Workload("odd_shapes", 24, 512, 192, 5, 5, False, 2.0 ** -5, seed=77,
                       shared_inter=128)
    L = synth.make_layer(w)
    dl = gpu.upload_layer(L)
    x = synth.make_tokens(w)
    y, ids, _ = decode_checked(gpu, dl, gpu.tokens_to_device(x))
    torch.cuda.synchronize()
    ref = oracle.moe_layer(L, x)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_output_close(gpu.bf16_bits(y), ref["y"], "odd shapes")


def test_grouped_decode_shapes_outside_the_workloads(gpu):
    """Grouped path with H = 768 (8 lanes x 3 chunks per row), I = 192, shared
    I = 128 != I, T = 12, clamped SwiGLU; and H = 4096 (64 lanes x 2 chunks)."""
    for H, I, Is, seed in ((768, 192, 128, 78), (4096, 128, 64, 79)):
        w = synth.Workload(f"odd_{H}", 20, H, I, 4, 12, True, 2.0 ** -6, seed=seed,
                           shared_inter=Is)
        L = synth.make_layer(w)
        dl = gpu.upload_layer(L)
        x = synth.make_tokens(w)
        y, ids, _ = decode_checked(gpu, dl, gpu.tokens_to_device(x))
        torch.cuda.synchronize()
        ref = oracle.moe_layer(L, x)
        assert np.array_equal(ids.cpu().numpy(), ref["ids"])
        assert_output_close(gpu.bf16_bits(y), ref["y"], f"grouped odd shapes H={H}")


@pytest.mark.parametrize("H,I,Is,T", [(1024, 768, 768, 16), (3072, 1024, 1024, 24),
                                      (2048, 512, 0, 40), (4096, 512, 512, 64)])
def test_grouped_decode_pipelined_shapes(gpu, H, I, Is, T):
    """The few-token grouped kernels at every width they are unrolled for: gate|up
    with H / 512 = 2, 6, 4, 8 K blocks, down with I / 128 = 6, 8, 4, 4 pieces (one
    case without a shared expert), T up to 64."""
    w = synth.Workload(f"pipe_{H}_{I}", 24, H, I, 4, T, True, 2.0 ** -6, seed=H + I + T,
                       shared_inter=Is)
    L = synth.make_layer(w)
    dl = gpu.upload_layer(L)
    x = synth.make_tokens(w)
    y, ids, _ = decode_checked(gpu, dl, gpu.tokens_to_device(x))
    torch.cuda.synchronize()
    ref = oracle.moe_layer(L, x)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_output_close(gpu.bf16_bits(y), ref["y"], f"grouped pipelined H={H} I={I}")


@pytest.mark.parametrize("name,tokens", [("tiny_e8_top2", 1), ("tiny_e8_top2", 3),
                                         ("decode_e512_top10_shared", 1)])
def test_decode_consecutive_calls_on_one_workspace(gpu, name, tokens):
    """Several fused calls in a row on one workspace, each with new tokens, each
    against the oracle.  Every block of the fused kernel must advance its own call
    counter on every call, also blocks with no gate|up rows (the tiny layer has
    256 rows for 2048 waves), or the next call's hand-offs never match."""
    from nvfp4_mixture_experts_amd import ftmoe
    w = synth.WORKLOADS[name]
    dl = dev_layer(gpu, name)
    L = host_layer(name)
    ws = ftmoe.alloc_workspace(dl.desc, tokens, ftmoe.PATH_DECODE)
    for i in range(4):
        x = synth.make_tokens(w, tokens=tokens, stream=f"seq{i}")
        y, ids, _ = gpu.decode(dl, gpu.tokens_to_device(x), workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.moe_layer(L, x)
        assert np.array_equal(ids.cpu().numpy(), ref["ids"]), i
        assert_output_close(gpu.bf16_bits(y), ref["y"], f"{name} T={tokens} call {i}")


@pytest.mark.parametrize("tokens", [4, 16, 40])   # fused kernel, grouped path (row, split router)
def test_decode_is_deterministic(gpu, tokens):
    """Same inputs -> same bits, across workspace addresses and streams."""
    from nvfp4_mixture_experts_amd import ftmoe
    name = "decode_e512_top10_shared"
    dl = dev_layer(gpu, name)
    x = gpu.tokens_to_device(synth.make_tokens(synth.WORKLOADS[name], tokens=tokens,
                                               stream="det"))
    n = ftmoe.ft_moe_workspace_bytes(dl.desc, tokens, ftmoe.PATH_DECODE)
    span = (n + 255) // 256 * 256 + 1024
    big = torch.zeros(3 * span, dtype=torch.uint8, device="cuda")
    # disjoint workspaces at different offsets; calls ordered (a workspace is never
    # shared by calls that may run at the same time)
    y0, _, _ = decode_checked(gpu, dl, x)
    y1, _, _ = decode_checked(gpu, dl, x, workspace=big[1024:1024 + n])
    main = torch.cuda.current_stream()
    s = torch.cuda.Stream()
    s.wait_stream(main)
    with torch.cuda.stream(s):
        y2, _, _ = gpu.decode(dl, x, workspace=big[span + 2048:span + 2048 + n], stream=s)
    main.wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(y0.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("tokens", [1, 12, 40])   # fused kernel, grouped path (row, split router)
def test_decode_graph_replays_match_eager(gpu, tokens):
    from nvfp4_mixture_experts_amd import ftmoe
    name = "decode_e288_top8"
    w = synth.WORKLOADS[name]
    dl = dev_layer(gpu, name)
    xs = [gpu.tokens_to_device(synth.make_tokens(w, tokens=tokens, stream=f"g{i}"))
          for i in range(3)]
    ws = ftmoe.alloc_workspace(dl.desc, tokens, ftmoe.PATH_DECODE)
    eager = []
    for x in xs:
        y, _, _ = decode_checked(gpu, dl, x, workspace=ws)
        eager.append(y.clone())
    torch.cuda.synchronize()
    xin = xs[0].clone()
    yout = torch.empty_like(eager[0])
    ids = torch.empty((tokens, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((tokens, w.top_k), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            ftmoe.ft_moe_nvfp4_decode(dl.desc, xin, dl.w_router, dl.bias, dl.routed, dl.shared,
                                      dl.shared_gate, yout, ws, ids, wt, stream=s)
    torch.cuda.synchronize()
    for rep in range(6):
        i = rep % 3
        xin.copy_(xs[i])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(yout.view(torch.int16), eager[i].view(torch.int16)), rep
        # eager work between replays
        decode_checked(gpu, dl, xs[(i + 1) % 3], workspace=ws)


# ---------------------------------------------------------------- prefill --

def test_prefill_matches_oracle_small(gpu):
    w = synth.dataclasses.replace(synth.WORKLOADS["prefill_t8192"], num_experts=32, tokens=97)
    L = synth.make_layer(w)
    dl = gpu.upload_layer(L)
    x = synth.make_tokens(w)
    xd = gpu.tokens_to_device(x)
    ids, wt = gpu.route(dl, xd)
    y = gpu.prefill(dl, xd, ids, wt)
    torch.cuda.synchronize()
    rows = [0, 1, 48, 96]
    ref = oracle.moe_layer(L, x[rows])
    assert np.array_equal(ids.cpu().numpy()[rows], ref["ids"])
    assert_output_close(gpu.bf16_bits(y)[rows], ref["y"], "prefill T=97")


def test_prefill_uses_given_routes(gpu):
    """Routes passed in (not the router's) decide which experts run."""
    w = synth.dataclasses.replace(synth.WORKLOADS["prefill_t8192"], num_experts=16, tokens=8)
    L = synth.make_layer(w)
    dl = gpu.upload_layer(L)
    x = synth.make_tokens(w)
    rng = np.random.default_rng(3)
    ids = np.stack([rng.permutation(16)[: w.top_k] for _ in range(8)]).astype(np.int32)
    wts = rng.dirichlet(np.ones(w.top_k), size=8).astype(np.float32)
    y = gpu.prefill(dl, gpu.tokens_to_device(x), torch.from_numpy(ids).cuda(),
                    torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    ref = oracle.moe_layer(L, x, ids=ids, weights=wts)
    assert_output_close(gpu.bf16_bits(y), ref["y"], "prefill given routes")


@pytest.mark.parametrize("tokens", [24, 300])   # grouped decode, prefill
def test_token_order_does_not_change_results(gpu, tokens):
    """Permuting the tokens permutes the outputs bit for bit: where a pair lands in
    its expert's group (which the grouping leaves unspecified) changes nothing."""
    name = "decode_e512_top10_shared"
    w = synth.WORKLOADS[name]
    dl = dev_layer(gpu, name)
    x = synth.make_tokens(w, tokens=tokens, stream="perm")
    perm = np.random.default_rng(9).permutation(tokens)
    xd, xpd = gpu.tokens_to_device(x), gpu.tokens_to_device(x[perm])
    if tokens <= 64:
        y, _, _ = decode_checked(gpu, dl, xd)
        yp, _, _ = decode_checked(gpu, dl, xpd)
    else:
        ids, wt = gpu.route(dl, xd)
        y = gpu.prefill(dl, xd, ids, wt)
        idsp, wtp = gpu.route(dl, xpd)
        yp = gpu.prefill(dl, xpd, idsp, wtp)
    torch.cuda.synchronize()
    assert np.array_equal(gpu.bf16_bits(y)[perm], gpu.bf16_bits(yp))
