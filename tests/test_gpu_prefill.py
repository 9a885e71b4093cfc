"""GPU parity of the many-token path (ft_moe_route + ft_moe_nvfp4_prefill) against
the CPU oracle, through the C ABI.

The prefill path groups the routed (token, slot) pairs by expert and runs each
expert's tokens as MFMA tiles of at most 256 tokens; these cases cover experts
with several tiles, ragged tails, a shared expert of another width, every expert
selected, a single token, the full 8192-token chunk (sampled tokens) and
run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_mixture_experts_amd import synth
from tests.gpu_util import (assert_output_close, cover_rows, f32_ulp_diff, host_layer,
                            oracle_layer_rows, oracle_routes, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_mixture_experts_amd import device, ftmoe
    ftmoe.ft_init(0)
    return device


def _run(gpu, L, x, ids, wts):
    dl = gpu.upload_layer(L)
    y = gpu.prefill(dl, gpu.tokens_to_device(x), torch.from_numpy(ids).cuda(),
                    torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    return gpu.bf16_bits(y)


def _skewed_routes(T, E, k, seed):
    """Every token picks expert 0 (three 256-token tiles at T = 600), every 35th
    token expert 1 (a ragged 18-token tile), the rest at random."""
    rng = np.random.default_rng(seed)
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        first = [0, 1] if t % 35 == 0 else [0]
        rest = rng.permutation(np.arange(2, E))[: k - len(first)]
        ids[t] = np.concatenate([first, rest])
    wts = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    return ids, wts


def test_prefill_multi_tile_experts_and_ragged_tails(gpu):
    w = synth.dataclasses.replace(synth.WORKLOADS["prefill_t8192"], num_experts=16, hidden=512,
                                  inter=128, top_k=4, tokens=600, shared_inter=192)
    L = synth.make_layer(w)
    x = synth.make_tokens(w)
    ids, wts = _skewed_routes(w.tokens, w.num_experts, w.top_k, seed=11)
    say(f"  tokens of expert 0: {(ids == 0).sum()}, expert 1: {(ids == 1).sum()}")
    y = _run(gpu, L, x, ids, wts)
    rows = [0, 1, 35, 255, 256, 257, 300, 511, 512, 513, 525, 560, 598, 599]
    ref = oracle.moe_layer(L, x[rows], ids=ids[rows], weights=wts[rows])
    assert_output_close(y[rows], ref["y"], "prefill T=600 skewed")


def test_prefill_plain_swiglu_no_shared(gpu):
    w = synth.dataclasses.replace(synth.WORKLOADS["tiny_e8_top2"], tokens=300)
    L = synth.make_layer(w)
    x = synth.make_tokens(w)
    rng = np.random.default_rng(2)
    ids = np.stack([rng.permutation(8)[:2] for _ in range(300)]).astype(np.int32)
    wts = rng.dirichlet(np.ones(2), size=300).astype(np.float32)
    y = _run(gpu, L, x, ids, wts)
    rows = list(range(0, 300, 23)) + [299]
    ref = oracle.moe_layer(L, x[rows], ids=ids[rows], weights=wts[rows])
    assert_output_close(y[rows], ref["y"], "prefill tiny T=300")


def test_prefill_all_experts_selected(gpu):
    w = synth.dataclasses.replace(synth.WORKLOADS["prefill_t8192"], num_experts=16, top_k=16,
                                  tokens=40, hidden=256, inter=64, shared_inter=64)
    L = synth.make_layer(w)
    x = synth.make_tokens(w)
    dl = gpu.upload_layer(L)
    xd = gpu.tokens_to_device(x)
    ids, wt = gpu.route(dl, xd)
    y = gpu.prefill(dl, xd, ids, wt)
    torch.cuda.synchronize()
    rows = [0, 13, 39]
    ref = oracle.moe_layer(L, x[rows])
    assert np.array_equal(ids.cpu().numpy()[rows], ref["ids"])
    assert_output_close(gpu.bf16_bits(y)[rows], ref["y"], "prefill k=E=16")


def test_prefill_single_token(gpu):
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"], tokens=1)
    L = host_layer("decode_e512_top10_shared")
    x = synth.make_tokens(w)
    dl = gpu.upload_layer(L)
    xd = gpu.tokens_to_device(x)
    ids, wt = gpu.route(dl, xd)
    y = gpu.prefill(dl, xd, ids, wt)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(L, x)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_output_close(gpu.bf16_bits(y), ref["y"], "prefill T=1")


def test_prefill_is_deterministic(gpu):
    w = synth.dataclasses.replace(synth.WORKLOADS["prefill_t8192"], num_experts=64, tokens=700)
    L = synth.make_layer(w)
    x = synth.make_tokens(w)
    dl = gpu.upload_layer(L)
    xd = gpu.tokens_to_device(x)
    ids, wt = gpu.route(dl, xd)
    from nvfp4_mixture_experts_amd import ftmoe
    ws_a = ftmoe.alloc_workspace(dl.desc, w.tokens, ftmoe.PATH_PREFILL, xd.device)
    ws_b = ftmoe.alloc_workspace(dl.desc, w.tokens, ftmoe.PATH_PREFILL, xd.device)
    ya = gpu.prefill(dl, xd, ids, wt, workspace=ws_a)
    yb = gpu.prefill(dl, xd, ids, wt, workspace=ws_b)
    yc = gpu.prefill(dl, xd, ids, wt, workspace=ws_a)
    torch.cuda.synchronize()
    a, b, c = gpu.bf16_bits(ya), gpu.bf16_bits(yb), gpu.bf16_bits(yc)
    assert np.array_equal(a, b) and np.array_equal(a, c)


@pytest.mark.parametrize("H,Is,clamped", [(1024, 512, True), (2048, 512, True), (4096, 0, True),
                                         (2048, 512, False)])
def test_prefill_unrolled_widths(gpu, H, Is, clamped):
    """The many-token kernels with the unrolled gate|up K loop (H / 256 = 4, 8, 16
    super-slabs) and the whole-tile down product (I = 512 for both banks; one case
    without a shared expert): T = 300, so the shared unit holds 256 tokens.  The
    clamped activation hands h to the down product in fp16, the plain one as a
    bf16 (hi, lo) pair."""
    w = synth.dataclasses.replace(synth.WORKLOADS["prefill_t8192"], num_experts=16, top_k=4,
                                  tokens=300, hidden=H, inter=512, shared_inter=Is,
                                  clamped=clamped, seed=600 + H + Is + int(clamped))
    L = synth.make_layer(w)
    x = synth.make_tokens(w)
    dl = gpu.upload_layer(L)
    xd = gpu.tokens_to_device(x)
    ids, wt = gpu.route(dl, xd)
    y = gpu.prefill(dl, xd, ids, wt)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 127, 128, 200, 255, 256, 299]
    ref = oracle.moe_layer(L, x[rows])
    assert np.array_equal(ids.cpu().numpy()[rows], ref["ids"])
    assert_output_close(gpu.bf16_bits(y)[rows], ref["y"],
                        f"prefill unrolled H={H} clamped={clamped}")


@pytest.mark.parametrize("clamped", [True, False])
def test_grouped_few_tokens_both_h_forms(gpu, clamped):
    """The few-token grouped kernels (units of at most 16 tokens) with h in fp16
    (clamped activation) and as a bf16 pair (plain), every token against the oracle:
    24 tokens over 32 experts, top-4, a shared expert, I = 512 (the pipelined down
    product) and I = 192 (the looped one, with a trailing 64-K piece)."""
    for inter in (512, 192):
        w = synth.dataclasses.replace(synth.WORKLOADS["batched_decode_t32_hot64"], num_experts=32,
                                      top_k=4, tokens=24, inter=inter, shared_inter=inter,
                                      hot_experts=4, clamped=clamped, seed=700 + inter)
        L = synth.make_layer(w)
        x = synth.make_tokens(w)
        dl = gpu.upload_layer(L)
        xd = gpu.tokens_to_device(x)
        ids, wt = gpu.route(dl, xd)
        y = gpu.prefill(dl, xd, ids, wt)
        torch.cuda.synchronize()
        ref = oracle.moe_layer(L, x)
        assert np.array_equal(ids.cpu().numpy(), ref["ids"])
        assert_output_close(gpu.bf16_bits(y), ref["y"], f"grouped T=24 I={inter} clamped={clamped}")


@pytest.mark.slow
def test_prefill_full_chunk_sampled(gpu):
    """The 8192-token chunk at full size: the routes of every token bit-exact against
    the oracle router; outputs against the oracle on rows that together reach every
    one of the 512 experts and both ends of every 256-token unit of the shared
    expert; every output finite."""
    name = "prefill_t8192"
    w = synth.WORKLOADS[name]
    L = host_layer(name)
    x = synth.make_tokens(w)
    dl = gpu.upload_layer(L)
    xd = gpu.tokens_to_device(x)
    ids, wt = gpu.route(dl, xd)
    y = gpu.prefill(dl, xd, ids, wt)
    torch.cuda.synchronize()
    yb = gpu.bf16_bits(y)
    yf = (yb.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isfinite(yf))
    ids_np = ids.cpu().numpy()
    ref_ids, ref_w = oracle_routes(x, L.w_router, L.bias, w.top_k)
    assert np.array_equal(ids_np, ref_ids)
    assert f32_ulp_diff(wt.cpu().numpy(), ref_w).max() <= 2
    counts = np.bincount(ids_np.ravel(), minlength=w.num_experts)
    say(f"  routes of all {w.tokens} tokens exact; tokens per expert: min {counts.min()} "
        f"max {counts.max()} mean {counts.mean():.1f}")
    ends = [t for j in range(w.tokens // 256) for t in (256 * j, 256 * j + 255)]
    rows = cover_rows(ids_np, w.num_experts, must=ends)
    say(f"  comparing {len(rows)} rows with the oracle (all {w.num_experts} experts reached)")
    assert len(np.unique(ids_np[rows])) == w.num_experts
    ref = oracle_layer_rows(L, x, rows)
    assert np.array_equal(ids_np[rows], ref["ids"])
    assert_output_close(yb[rows], ref["y"], f"prefill T=8192, {len(rows)} rows")
