"""GPU parity of ft_attn_extend (extend attention over a bf16 / fp8 / NVFP4 KV-cache
prefix and the new tokens, causal, optional window) against the CPU oracle's
dequantised-cache attention, through the C ABI.  The case matrix is the pages' own
check: cache formats 16-bit, fp8 and NVFP4; head dims 64 and 128; prefixes 37, 200
and 1000; windows 0 and 100.  bf16 outputs within max_abs_rel 1e-2, rel_l2 2e-3."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_mixture_experts_amd import synth
from tests.gpu_util import assert_output_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ft():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_mixture_experts_amd import ftmoe
    ftmoe.ft_init(0)
    return ftmoe


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _u8(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(ft, case, window):
    c = case["cache"]
    fmt = c["format"]
    n_new, Hq, d = case["q"].shape
    out = torch.full((n_new, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    kc = vc = None
    if c["prefix"] > 0:
        kc, vc = (_bf16(c["k"]), _bf16(c["v"])) if fmt == 0 else (_u8(c["k"]), _u8(c["v"]))
    ft.ft_attn_extend(_bf16(case["q"]), _bf16(case["k_new"]), _bf16(case["v_new"]), fmt,
                      c["prefix"], kc, vc, out, window=window,
                      k_block_scale=_u8(c.get("k_bscale")), v_block_scale=_u8(c.get("v_bscale")),
                      k_scale=c.get("k_scale", 1.0), v_scale=c.get("v_scale", 1.0))
    torch.cuda.synchronize()
    return out.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("prefix", [37, 200, 1000])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_attn_extend_matches_dequantised_cache_reference(ft, fmt, head_dim, prefix, window):
    case = synth.make_attn_case(fmt, head_dim, prefix)
    got = _run(ft, case, window)
    ref = oracle.attn_extend(case["q"], case["k_new"], case["v_new"], case["cache"], window)
    assert_output_close(got.reshape(-1, head_dim), ref["out"].reshape(-1, head_dim),
                        f"attn fmt={fmt} d={head_dim} prefix={prefix} window={window}")


@pytest.mark.parametrize("fmt", [0, 2])
def test_attn_extend_edges(ft, fmt):
    # no prefix; a window of one position; one new token; q heads == kv heads
    for prefix, window, n_new, hq, hkv in [(0, 0, 17, 8, 2), (64, 1, 5, 4, 4),
                                           (300, 0, 1, 6, 3), (130, 65, 70, 2, 1)]:
        case = synth.make_attn_case(fmt, 64, prefix, n_new=n_new, q_heads=hq, kv_heads=hkv)
        got = _run(ft, case, window)
        ref = oracle.attn_extend(case["q"], case["k_new"], case["v_new"], case["cache"], window)
        assert_output_close(got.reshape(-1, 64), ref["out"].reshape(-1, 64),
                            f"attn edge fmt={fmt} prefix={prefix} window={window} n={n_new}")


@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("fmt", [0, 2])
def test_attn_extend_scores_that_keep_growing(ft, fmt, window):
    """Scores that rise along the cache, so that a row's running maximum moves by far
    more than 2^8 from one 64-key chunk to the next (and, for the NVFP4 cache, barely
    moves over its first chunks): every rescaling of the output and normaliser, and
    long stretches of none, against the reference."""
    rng = np.random.default_rng(41 + fmt + window)
    prefix, n_new, Hq, Hkv, d = 1000, 24, 8, 2, 64
    q = np.ones((n_new, Hq, d), np.float32) * (1.0 + 0.5 * rng.random((n_new, Hq, 1), np.float32))
    case = {"q": synth.bf16_bits_from_f32(q),
            "k_new": synth.bf16_bits_from_f32(rng.standard_normal((n_new, Hkv, d), np.float32)),
            "v_new": synth.bf16_bits_from_f32(rng.standard_normal((n_new, Hkv, d), np.float32)),
            "cache": {"format": fmt, "prefix": prefix}}
    c = case["cache"]
    pos = np.arange(prefix, dtype=np.float32)[:, None, None]
    if fmt == 0:
        # score ~ q x position / 8: +8 q (natural), 11.5 q (base 2) or more per chunk
        k = np.broadcast_to(pos / 64.0, (prefix, Hkv, d)) * (1.0 + 0.1 * rng.random((prefix, Hkv, d), np.float32))
        c["k"] = synth.bf16_bits_from_f32(k.astype(np.float32))
        c["v"] = synth.bf16_bits_from_f32(rng.standard_normal((prefix, Hkv, d), np.float32))
    else:
        # every key code +6 (0x7 in both nibbles), block scales rising one e4m3 step per
        # 8 positions from 2^-6 to 448: tiny scores first, then jumps of ~2.5x a chunk
        c["k"] = np.full((prefix, Hkv, d // 2), 0x77, np.uint8)
        steps = np.minimum(0x08 + np.arange(prefix) // 8, 0x7E).astype(np.uint8)
        c["k_bscale"] = np.ascontiguousarray(np.broadcast_to(steps[:, None, None], (prefix, Hkv, d // 16)))
        c["v"] = synth._codes(rng, (prefix, Hkv, d // 2))
        c["v_bscale"] = synth.SCALE_BYTES[rng.integers(0, 5, (prefix, Hkv, d // 16))]
        c["k_scale"], c["v_scale"] = 0.25, 0.25
    got = _run(ft, case, window)
    ref = oracle.attn_extend(case["q"], case["k_new"], case["v_new"], c, window)
    assert_output_close(got.reshape(-1, d), ref["out"].reshape(-1, d),
                        f"attn growing scores fmt={fmt} window={window}")
