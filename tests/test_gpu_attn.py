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
