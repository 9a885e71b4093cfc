"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against what the format or the mathematics fixes:
the published E2M1/E4M3 tables, a library decoder (torch's float8_e4m3fn), the
exactness of the code x scale product, library routines (numpy matmul and
argsort, scipy softmax) on the special cases that reduce to them, a
hand-derived worked example, and closed forms.  Together they are chosen so
that a plausible slip in the oracle (swapped nibbles, a wrong scale-block index,
gate and up swapped, a missing clamp, a wrong sign, double rounding to bf16,
ties broken toward the higher index) fails at least one of them.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from nvfp4_mixture_experts_amd import synth
from tests.conftest import GOLDEN


def _golden_e2m1():
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, v = line.split()
            vals.append((int(code), float(v)))
    assert [c for c, _ in vals] == list(range(16))
    return np.array([v for _, v in vals], dtype=np.float64)


E2M1 = _golden_e2m1()


def _torch_e4m3_all():
    b = torch.arange(256, dtype=torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


E4M3 = _torch_e4m3_all()


def _f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


# ------------------------------------------------------------------ codecs --

def test_e2m1_matches_published_table_bitwise():
    got = np.array([oracle.e2m1(c) for c in range(16)])
    # bitwise (so -0.0 for code 8 is checked too)
    assert np.array_equal(got.view(np.uint64), E2M1.view(np.uint64))


def test_e4m3_matches_torch_for_all_256_bytes():
    got = np.array([oracle.e4m3(b) for b in range(256)])
    nan = np.isnan(E4M3)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan].view(np.uint64), E4M3[~nan].view(np.uint64))


def test_e4m3_named_points():
    with open(os.path.join(GOLDEN, "e4m3_points.txt")) as f:
        rows = [ln.split()[:2] for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for hexbyte, val in rows:
        got = oracle.e4m3(int(hexbyte, 16))
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), hexbyte


def test_synthetic_scale_bytes_are_the_powers_of_two_the_workloads_name():
    got = [oracle.e4m3(int(b)) for b in synth.SCALE_BYTES]
    assert got == [2.0 ** n for n in range(-4, 3)]


@pytest.mark.parametrize("g", [1.0, 2.0 ** -6, 0.3, 3.0e-3])
def test_dequant_is_one_rounding_of_the_exact_product(g):
    g32 = np.float32(g)
    for b in range(256):
        s = E4M3[b]
        if math.isnan(s):
            continue
        for c in range(16):
            exact = E2M1[c] * s
            # code x scale is exact in fp32 (at most 6 significant bits)
            assert np.float64(np.float32(exact)) == exact
            want = np.float32(exact) * g32            # numpy: one IEEE fp32 multiply
            got = oracle.dequant_value(c, b, float(g32))
            assert _f32_bits(got) == _f32_bits(want), (c, b, g)


def test_dequant_matrix_nibble_order_and_block_index():
    rng = np.random.default_rng(7)
    rows, K = 5, 64
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = synth.SCALE_BYTES[rng.integers(0, 7, (rows, K // 16))]
    g = np.float32(2.0 ** -6)
    got = oracle.dequant_matrix(codes, scales, float(g))
    # independent unpack: low nibble -> even k, high nibble -> odd k; block k // 16
    nib = np.empty((rows, K), np.int64)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    blk = np.repeat(scales, 16, axis=1)
    want = (E2M1[nib] * E4M3[blk]).astype(np.float32) * g
    assert np.array_equal(_f32_bits(got), _f32_bits(want))


# ------------------------------------------------------------- bf16 output --

def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # torch rounds fp32 -> bf16 to nearest-even; on fp32 inputs one rounding is all there is
    want = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rounding_is_a_single_rounding_from_binary64():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125: ties to even -> 1.0
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80
    # just above the tie rounds up; via fp32 the 2^-40 would be lost and tie down
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.bf16_from_double(-0.0) == 0x8000
    assert oracle.bf16_from_double(3.5e38) == 0x7F80
    assert oracle.bf16_from_double(2.0 ** -133) == 0x0001   # smallest subnormal
    assert oracle.bf16_from_double(2.0 ** -135) == 0x0000   # below half of it


# ------------------------------------------------------------------ router --

def test_router_logits_exact_on_integer_data():
    # small integers: every partial sum is exact in binary64 whatever the order,
    # so numpy's matmul must agree bit for bit
    rng = np.random.default_rng(3)
    T, E, H = 3, 37, 256
    xf = rng.integers(-4, 5, (T, H)).astype(np.float32)
    x = synth.bf16_bits_from_f32(xf)
    W = rng.integers(-8, 9, (E, H)).astype(np.float32)
    bias = rng.integers(-3, 4, E).astype(np.float32)
    got = oracle.router_logits(x, W, bias)
    want = (xf.astype(np.float64) @ W.astype(np.float64).T + bias).astype(np.float32)
    assert np.array_equal(got, want)


def test_router_logits_match_library_matmul():
    w = synth.WORKLOADS["decode_e288_top8"]
    L = synth.make_layer(w, num_experts=64)
    x = synth.make_tokens(w, tokens=4)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.router_logits(x, L.w_router)
    want = (xf @ L.w_router.astype(np.float64).T).astype(np.float32)
    ulps = np.abs(_f32_bits(got).astype(np.int64) - _f32_bits(want).astype(np.int64))
    assert ulps.max() <= 1 and (ulps == 0).mean() > 0.99


def test_topk_matches_stable_argsort_with_ties():
    rng = np.random.default_rng(5)
    T, E = 200, 50
    # few distinct values -> many exact ties; lowest index must win
    logits = rng.integers(0, 6, (T, E)).astype(np.float32) * np.float32(0.25)
    for k in (1, 3, 10, 16, 50):
        ids, w = oracle.topk(logits, k)
        want = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, want), k


def test_topk_weights_softmax_and_renormalisation():
    rng = np.random.default_rng(9)
    T, E = 64, 288
    logits = rng.standard_normal((T, E)).astype(np.float32)
    for k in (1, 2, 8, 10, E):
        ids, w = oracle.topk(logits, k)
        sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
        want = scipy.special.softmax(sel, axis=1)
        assert np.allclose(w, want, rtol=2 ** -23, atol=0)
        # renormalising a softmax over all experts gives the same weights
        full = scipy.special.softmax(logits.astype(np.float64), axis=1)
        ren = np.take_along_axis(full, ids, axis=1)
        ren /= ren.sum(axis=1, keepdims=True)
        assert np.allclose(w, ren, rtol=2 ** -22, atol=0)
        assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= k * 2.0 ** -24)
        if k == 1:
            assert np.all(w == 1.0)


def test_topk_nan_ranks_last():
    logits = np.array([[np.nan, 1.0, np.nan, 0.5]], np.float32)
    ids, _ = oracle.topk(logits, 3)
    assert ids.tolist() == [[1, 3, 0]]


# ------------------------------------------------------------- activations --

def test_silu_closed_forms():
    getcontext().prec = 40
    s7 = Decimal(7) / (1 + Decimal(-7).exp())
    assert oracle.silu(7.0) == pytest.approx(float(s7), rel=1e-15)
    assert oracle.silu(0.0) == 0.0
    for z in (-1000.0, -800.0):
        v = oracle.silu(z)
        assert not math.isnan(v) and v == 0.0 and math.copysign(1, v) < 0
    assert oracle.silu(1000.0) == 1000.0


def test_swiglu_clamps():
    s7 = oracle.silu(7.0)
    # clamped: gate capped above at 7, up clamped to [-7, 7]
    assert oracle.swiglu(1, 100.0, 100.0) == s7 * 7.0
    assert oracle.swiglu(1, 100.0, -100.0) == -s7 * 7.0
    assert oracle.swiglu(1, 3.0, 2.0) == oracle.silu(3.0) * 2.0
    assert oracle.swiglu(1, -50.0, 5.0) == oracle.silu(-50.0) * 5.0   # no lower gate clamp
    # plain: no clamps, gate and up are not interchangeable
    assert oracle.swiglu(0, 100.0, 100.0) == pytest.approx(100.0 * 100.0, rel=1e-15)
    assert oracle.swiglu(0, 2.0, 5.0) != oracle.swiglu(0, 5.0, 2.0)
    assert math.isnan(oracle.swiglu(1, float("nan"), 1.0))


# ---------------------------------------------------------- whole layer --

def _bf16_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()


def _unpack(codes, scales, g):
    """Dense fp32 [rows, K] from canonical codes/scales, by table lookup (numpy only)."""
    rows = codes.shape[0]
    nib = np.empty((rows, codes.shape[1] * 2), np.int64)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    return (E2M1[nib] * E4M3[np.repeat(scales, 16, axis=1)]).astype(np.float32) * np.float32(g)


def _dense_mlp(layer, xf, w13c, w13s, w2c, w2s, g3, I):
    """One expert's MLP on fp64 token rows xf [T, H] with numpy matmuls and scipy's
    expit; returns (output [T, H], whether a clamp engaged)."""
    wg = _unpack(w13c[:I], w13s[:I], g3[0]).astype(np.float64)
    wu = _unpack(w13c[I:], w13s[I:], g3[1]).astype(np.float64)
    wd = _unpack(w2c, w2s, g3[2]).astype(np.float64)
    gate = xf @ wg.T
    up = xf @ wu.T
    clamped = False
    if layer.act == 1:
        clamped = bool((gate > layer.gate_max).any() or (np.abs(up) > layer.up_absmax).any())
        gate = np.minimum(gate, layer.gate_max)
        up = np.clip(up, -layer.up_absmax, layer.up_absmax)
    h = scipy.special.expit(gate) * gate * up
    return h @ wd.T, clamped


def _dense_shared(layer, xf):
    """gamma [T] = expit(x . gate vector) and the shared expert's output [T, H]."""
    gs = _bf16_to_f64(layer.shared_gate)
    gamma = scipy.special.expit(xf @ gs)
    o, _ = _dense_mlp(layer, xf, layer.s13_codes[0], layer.s13_scales[0], layer.s2_codes[0],
                      layer.s2_scales[0], layer.s_global[0], layer.shared_inter)
    return gamma, o


def _dense_reference(layer, x):
    """k = E: y = sum_e softmax_e(logits) * MLP_e(x) (+ expit(gs . x) * MLP_s(x) with a
    shared expert), from library routines only."""
    H, I, E = layer.hidden, layer.inter, layer.num_experts
    xf = _bf16_to_f64(x)
    logits = (xf @ layer.w_router.astype(np.float64).T).astype(np.float32)
    probs = scipy.special.softmax(logits.astype(np.float64), axis=1).astype(np.float32)
    y = np.zeros((x.shape[0], H))
    clamped = False
    for e in range(E):
        o, c = _dense_mlp(layer, xf, layer.w13_codes[e], layer.w13_scales[e], layer.w2_codes[e],
                          layer.w2_scales[e], layer.global_scale[e], I)
        clamped |= c
        y += probs[:, e:e + 1].astype(np.float64) * o
    if layer.shared_inter > 0:
        gamma, o = _dense_shared(layer, xf)
        y += gamma[:, None] * o
    return y, clamped


@pytest.mark.parametrize("name", ["tiny_e8_top2", "decode_e288_top8"])
def test_all_experts_selected_equals_dense_layer(name):
    w = synth.WORKLOADS[name]
    E = 8 if name == "tiny_e8_top2" else 6
    # the clamped case uses a larger global scale so that both clamps engage
    g = w.global_scale if w.act == 0 else 2.0 ** -3
    w = synth.dataclasses.replace(w, num_experts=E, top_k=E, hidden=256, inter=128,
                                  global_scale=g)
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=2)
    got = oracle.moe_layer(layer, x)
    want, clamped = _dense_reference(layer, x)
    scale = np.abs(want).max()
    assert np.abs(got["y64"] - want).max() <= 1e-12 * scale
    assert clamped == (w.act == 1)


def test_clamp_engages_on_decode_workload_shape():
    # with global scale 2^-6 some pre-activations exceed 7: dropping the clamp changes y
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e288_top8"], num_experts=4, top_k=4)
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=1)
    clamped = oracle.moe_layer(layer, x)["y64"]
    w_plain = synth.dataclasses.replace(w, clamped=False)
    plain = oracle.moe_layer(synth.dataclasses.replace(layer, workload=w_plain), x)["y64"]
    assert not np.allclose(clamped, plain, rtol=1e-6)


def test_worked_example():
    spec = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    sh = spec["shape"]
    E, H, I = sh["num_experts"], sh["hidden"], sh["inter"]
    w = synth.Workload("worked_example", E, H, I, sh["top_k"], 1, True, 1.0, seed=0)
    w13c = np.full((E, 2 * I, H // 2), 0x77, np.uint8)
    w13s = np.full((E, 2 * I, H // 16), 0x38, np.uint8)
    w2c = np.full((E, H, I // 2), 0x77, np.uint8)
    w2s = np.full((E, H, I // 16), 0x38, np.uint8)
    gsc = np.ones((E, 3), np.float32)
    w13c[0, :I] = 0x62
    w13s[0, :I] = [0x38, 0x30]
    w13c[0, I:] = 0xB3
    w13s[0, I:] = [0x38, 0x38]
    w2c[0] = 0x02
    w2s[0, 0::2] = 0x40
    w2s[0, 1::2] = 0x48
    gsc[0] = [0.5, 1.0, 0.25]
    wr = np.empty((E, H), np.float32)
    wr[0] = 0.01
    wr[1] = -0.01
    layer = synth.Layer(w, wr, None, w13c, w13s, w2c, w2s, gsc)
    x = np.zeros((1, H), np.uint16)
    x[0, 0::2] = 0x3F80
    out = oracle.moe_layer(layer, x)
    ex = spec["expected"]
    assert out["ids"].tolist() == [ex["ids"]]
    assert out["weights"].tolist() == [ex["weights"]]
    assert np.allclose(out["y64"][0, 0::2], ex["y64_even_c"], rtol=1e-14, atol=0)
    assert np.allclose(out["y64"][0, 1::2], ex["y64_odd_c"], rtol=1e-14, atol=0)
    assert np.all(out["y"][0, 0::2] == int(ex["y_bf16_even_c"], 16))
    assert np.all(out["y"][0, 1::2] == int(ex["y_bf16_odd_c"], 16))


def test_shared_gate_of_zero_vector_is_one_half():
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"], num_experts=12,
                                  hidden=256, inter=128, shared_inter=128)
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=1)
    layer.shared_gate = np.zeros_like(layer.shared_gate)
    with_shared = oracle.moe_layer(layer, x)
    w0 = synth.dataclasses.replace(w, shared_inter=0)
    routed_only = oracle.moe_layer(synth.dataclasses.replace(layer, workload=w0), x)
    o_s = oracle.expert_output(layer, 0, x[0], shared=True)
    diff = with_shared["y64"][0] - routed_only["y64"][0]
    assert np.allclose(diff, 0.5 * o_s, rtol=1e-9, atol=1e-12 * np.abs(o_s).max())
    assert np.array_equal(with_shared["ids"], routed_only["ids"])


@pytest.mark.parametrize("z", [-4.0, -0.5, 1.5, 6.0])
def test_shared_gate_direction_on_one_hot_token(z):
    # x = e_{h0} (one-hot, 1.0) and gate vector entry gs[h0] = z (exact in bf16): the
    # gate's argument is exactly z, so the shared expert enters y with weight
    # expit(z), which is above 1/2 for z > 0 and below it for z < 0 (a sign slip in
    # the sigmoid turns expit(z) into expit(-z) and fails here).
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"], num_experts=12,
                                  hidden=256, inter=128, shared_inter=128,
                                  global_scale=2.0 ** -2)
    layer = synth.make_layer(w)
    h0 = 37
    x = np.zeros((1, w.hidden), np.uint16)
    x[0, h0] = 0x3F80                                  # bf16 1.0
    gs = np.zeros(w.hidden, np.uint16)
    gs[h0] = synth.bf16_bits_from_f32(np.array([z], np.float32))[0]
    assert _bf16_to_f64(gs)[h0] == z
    layer.shared_gate = gs
    with_shared = oracle.moe_layer(layer, x)
    w0 = synth.dataclasses.replace(w, shared_inter=0)
    routed_only = oracle.moe_layer(synth.dataclasses.replace(layer, workload=w0), x)
    diff = with_shared["y64"][0] - routed_only["y64"][0]
    # the shared expert's output from numpy/scipy alone (not the oracle)
    gamma, o_s = _dense_shared(layer, _bf16_to_f64(x))
    want_gamma = scipy.special.expit(z)
    assert gamma[0] == pytest.approx(want_gamma, rel=1e-15)
    assert (want_gamma > 0.5) == (z > 0)
    assert np.abs(o_s[0]).max() > 0
    assert np.allclose(diff, want_gamma * o_s[0], rtol=1e-9, atol=1e-12 * np.abs(o_s).max())
    # the ratio itself identifies the gate's value and direction
    big = np.abs(o_s[0]) > 0.1 * np.abs(o_s[0]).max()
    ratio = diff[big] / o_s[0][big]
    assert np.allclose(ratio, want_gamma, rtol=1e-9)
    assert np.array_equal(with_shared["ids"], routed_only["ids"])


def test_all_experts_selected_with_shared_expert_equals_dense_layer():
    # k = E plus a shared expert whose gate argument is far from 0 for every token
    # (gate vector N(0, 0.5), so |z| is typically ~8): the whole layer, shared
    # expert included, against a dense numpy/scipy reference.
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"], num_experts=5,
                                  top_k=5, hidden=256, inter=128, shared_inter=128,
                                  global_scale=2.0 ** -3, shared_gate_std=0.5)
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=3)
    got = oracle.moe_layer(layer, x)
    want, clamped = _dense_reference(layer, x)
    gamma, _ = _dense_shared(layer, _bf16_to_f64(x))
    assert np.all(np.abs(gamma - 0.5) > 0.05), gamma   # the gate is not near its midpoint
    scale = np.abs(want).max()
    assert np.abs(got["y64"] - want).max() <= 1e-12 * scale
    assert clamped


def test_given_routes_reproduce_computed_routes():
    w = synth.WORKLOADS["tiny_e8_top2"]
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=3)
    a = oracle.moe_layer(layer, x)
    b = oracle.moe_layer(layer, x, ids=a["ids"], weights=a["weights"])
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["y64"], b["y64"])


def test_expert_output_matches_layer_with_single_route():
    w = synth.WORKLOADS["tiny_e8_top2"]
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=1)
    ids = np.array([[5, 2]], np.int32)
    wts = np.array([[1.0, 0.0]], np.float32)
    out = oracle.moe_layer(layer, x, ids=ids, weights=wts)
    o5 = oracle.expert_output(layer, 5, x[0])
    assert np.array_equal(out["y64"][0], o5)


def test_openmp_timing_copy_gives_identical_bits():
    # the OpenMP build only spreads independent rows over threads
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"], num_experts=24)
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=2)
    a = oracle.moe_layer(layer, x)
    b = oracle.moe_layer(layer, x, openmp=True)
    for key in ("ids", "weights", "y64", "y"):
        assert np.array_equal(a[key], b[key]), key
    assert oracle.threads(False) == 1 and oracle.threads(True) >= 1


# ------------------------------------------------- expert-slot indirection --

def _bank_of(layer):
    return dict(w13_codes=layer.w13_codes, w13_scales=layer.w13_scales,
                w2_codes=layer.w2_codes, w2_scales=layer.w2_scales,
                global_scale=layer.global_scale)


def _slot_bank(layer, experts):
    """A bank whose slot s holds expert experts[s]."""
    b = _bank_of(layer)
    return {key: np.ascontiguousarray(v[np.asarray(experts)]) for key, v in b.items()}


def _slot_case(tokens=3):
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"], num_experts=40,
                                  hidden=256, inter=128, shared_inter=128, global_scale=2.0 ** -3)
    return synth.make_layer(w), synth.make_tokens(w, tokens=tokens)


def test_slots_identity_map_is_the_plain_layer():
    layer, x = _slot_case()
    E = layer.num_experts
    got = oracle.moe_layer_slots(layer, x, np.arange(E, dtype=np.int32), _bank_of(layer))
    want = oracle.moe_layer(layer, x)
    for key in ("ids", "weights", "y64", "y"):
        assert np.array_equal(got[key], want[key]), key
    assert np.all(got["miss"] == -1)


def test_slots_permuted_partial_bank_is_the_plain_layer():
    # only the selected experts resident, in a shuffled order, in a bank smaller than E
    layer, x = _slot_case()
    E = layer.num_experts
    sel = np.unique(oracle.moe_layer(layer, x)["ids"])
    rng = np.random.default_rng(3)
    order = rng.permutation(sel)
    slot_of = np.full(E, -1, np.int32)
    slot_of[order] = np.arange(len(order), dtype=np.int32)
    got = oracle.moe_layer_slots(layer, x, slot_of, _slot_bank(layer, order))
    want = oracle.moe_layer(layer, x)
    assert len(order) < E
    for key in ("ids", "weights", "y64", "y"):
        assert np.array_equal(got[key], want[key]), key
    assert np.all(got["miss"] == -1)


def test_slots_missing_experts_contribute_nothing_and_are_reported():
    # a missing expert equals a resident one whose codes are all zero (every weight
    # +0, so its output is exactly 0): routing and every other term unchanged
    layer, x = _slot_case(tokens=4)
    E = layer.num_experts
    ids = oracle.moe_layer(layer, x)["ids"]
    missing = np.unique(ids[:, [1, 4]])            # some experts of places 1 and 4
    slot_of = np.arange(E, dtype=np.int32)
    slot_of[missing[0::2]] = -1
    slot_of[missing[1::2]] = E + 7                 # outside [0, n_slots) as well
    got = oracle.moe_layer_slots(layer, x, slot_of, _bank_of(layer))
    zeroed = synth.dataclasses.replace(layer, w13_codes=layer.w13_codes.copy(),
                                       w2_codes=layer.w2_codes.copy())
    zeroed.w13_codes[missing] = 0
    zeroed.w2_codes[missing] = 0
    want = oracle.moe_layer(zeroed, x)
    assert np.array_equal(got["ids"], want["ids"])
    assert np.array_equal(got["weights"], want["weights"])
    assert np.array_equal(got["y64"], want["y64"])
    assert np.array_equal(got["y"], want["y"])
    expect_miss = np.where(np.isin(ids, missing), ids, -1)
    assert np.array_equal(got["miss"], expect_miss)
    assert (got["miss"] >= 0).sum() >= 2
    # and the output differs from the full layer (the dropped terms were not zero)
    full = oracle.moe_layer(layer, x)
    assert not np.array_equal(got["y64"], full["y64"])


# ------------------------------------------------------------- block-fp8 --

def test_fp8_dequant_is_one_rounding_matching_torch():
    # torch's float8_e4m3fn decode (library routine) times the fp32 scale in fp32
    # (one rounding), for every finite byte and scales that make the product round
    rng = np.random.default_rng(8)
    scales = np.concatenate([np.float32([1.0, 2.0 ** -9, 448.0]),
                             (rng.random(40) * 3e-3 + 1e-4).astype(np.float32)])
    bytes_ = synth.FP8_FINITE_BYTES
    dec = torch.from_numpy(bytes_.copy()).view(torch.float8_e4m3fn).to(torch.float32)
    rounded = 0
    for sc in scales:
        want = (dec * torch.tensor(sc, dtype=torch.float32)).numpy()
        got = np.array([oracle.fp8_dequant_value(int(b), float(sc)) for b in bytes_], np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), sc
        exact = E4M3[bytes_] * np.float64(sc)
        rounded += int(np.sum(exact != got.astype(np.float64)))
    assert rounded > 1000          # the products do round: the single rounding is exercised


def test_fp8_dequant_matrix_block_index_and_partial_blocks():
    rng = np.random.default_rng(9)
    rows, K = 300, 200                     # partial blocks in both directions
    codes = synth.FP8_FINITE_BYTES[rng.integers(0, 254, (rows, K))]
    scales = (rng.random((3, 2)) + 0.5).astype(np.float32)
    got = oracle.fp8_dequant_matrix(codes, scales)
    full = np.repeat(np.repeat(scales, 128, axis=0), 128, axis=1)[:rows, :K]
    want = (E4M3[codes].astype(np.float32) * full).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # a transposed scale index would read scales[c // 128, r // 128]: it differs here
    assert not np.array_equal(scales[:2, :2], scales[:2, :2].T)


def _dense_fp8_mlp(layer, xf, w13c, w13s, w2c, w2s, I):
    def dq(c, s):
        full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:c.shape[0], :c.shape[1]]
        return (E4M3[c].astype(np.float32) * full).astype(np.float64)
    wg = dq(w13c[:I], w13s[: I // 128])
    wu = dq(w13c[I:], w13s[I // 128:])
    wd = dq(w2c, w2s)
    gate = np.minimum(xf @ wg.T, layer.gate_max)
    up = np.clip(xf @ wu.T, -layer.up_absmax, layer.up_absmax)
    return (scipy.special.expit(gate) * gate * up) @ wd.T


def test_fp8_layer_all_experts_selected_equals_dense_layer():
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared_fp8"], num_experts=4,
                                  top_k=4, hidden=256, inter=128, shared_inter=128,
                                  shared_gate_std=0.5)
    layer = synth.make_fp8_layer(w)
    x = synth.make_tokens(w, tokens=2)
    got = oracle.moe_layer_fp8(layer, x)
    xf = _bf16_to_f64(x)
    logits = (xf @ layer.w_router.astype(np.float64).T).astype(np.float32)
    probs = scipy.special.softmax(logits.astype(np.float64), axis=1).astype(np.float32)
    want = np.zeros((2, w.hidden))
    for e in range(w.num_experts):
        want += probs[:, e:e + 1].astype(np.float64) * _dense_fp8_mlp(
            layer, xf, layer.w13_codes[e], layer.w13_scales[e], layer.w2_codes[e],
            layer.w2_scales[e], w.inter)
    gamma = scipy.special.expit(xf @ _bf16_to_f64(layer.shared_gate))
    want += gamma[:, None] * _dense_fp8_mlp(layer, xf, layer.s13_codes[0], layer.s13_scales[0],
                                            layer.s2_codes[0], layer.s2_scales[0],
                                            w.shared_inter)
    assert np.abs(got["y64"] - want).max() <= 1e-12 * np.abs(want).max()


def test_fp8_workload_clamps_engage():
    # the synthetic fp8 draws put pre-activations in the range where the clamps act
    w = synth.WORKLOADS["decode_e512_top10_shared_fp8"]
    layer = synth.make_fp8_layer(synth.dataclasses.replace(w, num_experts=12))
    x = synth.make_tokens(w, tokens=1)
    xf = _bf16_to_f64(x)
    c = layer.w13_codes[0]
    full = np.repeat(np.repeat(layer.w13_scales[0], 128, 0), 128, 1)
    pre = xf @ (E4M3[c] * full).T
    assert 0.3 < np.std(pre) < 30 and np.mean(np.abs(pre) > 7) > 0.001


# ------------------------------------------------ fp8 per-tensor W8A8 linear --

def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_encoder_round_trip_and_torch_rounding():
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F])
    for b in finite:                                   # decode then encode is the identity
        assert oracle.e4m3_encode(oracle.e4m3(b)) == b
    # midpoints between neighbouring magnitudes (exact ties: round to the even code)
    mags = np.array(sorted({abs(oracle.e4m3(b)) for b in range(0x7F)}))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal((mags[:-1] + mags[1:]) / 2, mids.astype(np.float64))   # exact in fp32
    rng = np.random.default_rng(12)
    vals = np.concatenate([mids, -mids, (rng.standard_normal(4000) * 40).astype(np.float32),
                           (rng.random(1000) * 0.02).astype(np.float32), np.float32([0.0, -0.0])])
    vals = vals[np.abs(vals) <= 448]
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, _torch_e4m3(vals))
    assert oracle.e4m3_encode(1e6) == 0x7E and oracle.e4m3_encode(-1e6) == 0xFE   # saturate


def test_fp8_activation_quantisation():
    w = synth.WORKLOADS["fp8_linear_qkv_t32"]
    x = synth.make_tokens(w, tokens=6, stream="q")
    codes, s = oracle.fp8_quantize(x)
    xf = _bf16_to_f64(x).astype(np.float32)
    amax = np.float32(np.abs(xf).max())
    assert s == amax / np.float32(448.0)
    assert np.array_equal(codes, _torch_e4m3(xf / s))
    assert codes.view(np.int8).max() == 0x7E or (codes & 0x7F).max() == 0x7E   # amax -> 448


def test_fp8_linear_equals_exact_matmul_and_per_part_concatenation():
    w = synth.WORKLOADS["fp8_linear_qkv_t32"]
    lin = synth.make_fp8_linear(synth.dataclasses.replace(w, hidden=512,
                                                          parts=(256, 64, 64)))
    x = synth.make_tokens(lin.workload, tokens=5, stream="lin")
    xq, s_x = oracle.fp8_quantize(x)
    rows = lin.row_scales()
    got = oracle.fp8_linear(xq, s_x, lin.w, rows)
    a = E4M3[xq].astype(np.float64)
    b = E4M3[lin.w].astype(np.float64)
    want = ((a @ b.T) * np.float64(s_x)) * rows.astype(np.float64)[None, :]
    assert np.array_equal(got["y64"], want)            # the fp64 sums are exact
    # one tensor-wise product per part over its row slice, concatenated
    parts = []
    for (r0, r1), sc in zip(lin.part_ranges(), lin.part_scales):
        parts.append(oracle.fp8_linear(xq, s_x, lin.w[r0:r1],
                                       np.full(r1 - r0, sc, np.float32))["y"])
    assert np.array_equal(np.concatenate(parts, axis=1), got["y"])


# ---------------------------------------------- extend attention over a cache --

def _cache_values(cache, key, Hkv, d):
    """Dequantised cache K or V [P, Hkv, d] in fp64, from torch / numpy tables."""
    c = cache[key]
    if cache["format"] == 0:
        return _bf16_to_f64(c)
    if cache["format"] == 1:
        dec = torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).to(
            torch.float64).numpy()
        return dec * cache[key + "_scale"]
    nib = np.empty(c.shape[:-1] + (d,), np.int64)
    nib[..., 0::2] = c & 0x0F
    nib[..., 1::2] = c >> 4
    bs = E4M3[np.repeat(cache[key + "_bscale"], 16, axis=-1)]
    return E2M1[nib] * bs * cache[key + "_scale"]


def _sdpa_reference(case, window):
    """torch's scaled_dot_product_attention in fp64 over [cache; new] with the visible
    set as a boolean mask (key p visible to query t iff p <= P + t and, with a
    window, P + t - p < window); kv heads repeated for the query-head groups."""
    q = _bf16_to_f64(case["q"])
    n_new, Hq, d = q.shape
    Hkv = case["k_new"].shape[1]
    P = case["cache"]["prefix"]
    k = np.concatenate([_cache_values(case["cache"], "k", Hkv, d), _bf16_to_f64(case["k_new"])])
    v = np.concatenate([_cache_values(case["cache"], "v", Hkv, d), _bf16_to_f64(case["v_new"])])
    rep = Hq // Hkv
    kt = torch.from_numpy(np.repeat(k, rep, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, rep, axis=1)).permute(1, 0, 2)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    pos_q = P + np.arange(n_new)[:, None]
    pos_k = np.arange(P + n_new)[None, :]
    vis = pos_k <= pos_q
    if window:
        vis &= (pos_q - pos_k) < window
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt,
                                                           attn_mask=torch.from_numpy(vis))
    return out.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("window", [0, 7])
def test_attn_extend_equals_sdpa_over_dequantised_cache(fmt, window):
    case = synth.make_attn_case(fmt, 64, prefix=37, n_new=9)
    got = oracle.attn_extend(case["q"], case["k_new"], case["v_new"], case["cache"], window)
    want = _sdpa_reference(case, window)
    assert np.abs(got["out64"] - want).max() <= 1e-12 * np.abs(want).max()


def test_attn_extend_without_prefix_is_library_causal_attention():
    case = synth.make_attn_case(0, 64, prefix=0, n_new=11)
    got = oracle.attn_extend(case["q"], case["k_new"], case["v_new"], case["cache"], 0)
    q = torch.from_numpy(_bf16_to_f64(case["q"])).permute(1, 0, 2)
    k = torch.from_numpy(np.repeat(_bf16_to_f64(case["k_new"]), 4, axis=1)).permute(1, 0, 2)
    v = torch.from_numpy(np.repeat(_bf16_to_f64(case["v_new"]), 4, axis=1)).permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    assert np.allclose(got["out64"], want.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_attn_extend_window_special_cases():
    case = synth.make_attn_case(2, 128, prefix=20, n_new=6)
    args = (case["q"], case["k_new"], case["v_new"], case["cache"])
    one = oracle.attn_extend(*args, window=1)      # each query sees only itself
    v_self = np.repeat(_bf16_to_f64(case["v_new"]), 4, axis=1)
    assert np.array_equal(one["out64"], v_self)
    a = oracle.attn_extend(*args, window=0)
    b = oracle.attn_extend(*args, window=1000)     # wider than every sequence position
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["out64"], b["out64"])
