"""GPU parity of ft_moe_nvfp4_decode_slots (routed experts in a bank of expert slots,
with an expert -> slot map; a non-resident selected expert contributes nothing and
is reported) against the CPU oracle's slot layer, through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from nvfp4_mixture_experts_amd import synth
from tests.gpu_util import assert_output_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_mixture_experts_amd import device, ftmoe
    ftmoe.ft_init(0)
    return device


def _slot_bank_host(layer, experts):
    b = dict(w13_codes=layer.w13_codes, w13_scales=layer.w13_scales, w2_codes=layer.w2_codes,
             w2_scales=layer.w2_scales, global_scale=layer.global_scale)
    return {key: np.ascontiguousarray(v[np.asarray(experts)]) for key, v in b.items()}


def _upload_bank(layer, bank):
    from nvfp4_mixture_experts_amd import ftmoe
    n = bank["w13_codes"].shape[0]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return ftmoe.ft_nvfp4_repack(layer.hidden, layer.inter, n, d(bank["w13_codes"]),
                                 d(bank["w13_scales"]), d(bank["w2_codes"]),
                                 d(bank["w2_scales"]), d(bank["global_scale"]))


def _run_slots(gpu, layer, dl, x, slot_bank, slot_of):
    from nvfp4_mixture_experts_amd import ftmoe
    T = x.shape[0]
    xd = gpu.tokens_to_device(x)
    ws = ftmoe.alloc_workspace(dl.desc, T, ftmoe.PATH_DECODE)
    y = torch.empty((T, layer.hidden), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, layer.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, layer.top_k), dtype=torch.float32, device="cuda")
    miss = torch.full((T, layer.top_k), -7, dtype=torch.int32, device="cuda")
    ftmoe.ft_moe_nvfp4_decode_slots(dl.desc, xd, dl.w_router, dl.bias, slot_bank,
                                    torch.from_numpy(slot_of).cuda(), dl.shared, dl.shared_gate,
                                    y, ws, ids, w, miss)
    st = ftmoe.device_status(ws)
    torch.cuda.synchronize()
    assert st == 0
    return gpu.bf16_bits(y), ids.cpu().numpy(), w.cpu().numpy(), miss.cpu().numpy()


def _case(name, tokens, **over):
    w = synth.dataclasses.replace(synth.WORKLOADS[name], **over) if over else synth.WORKLOADS[name]
    layer = synth.make_layer(w)
    return layer, synth.make_tokens(w, tokens=tokens, stream="slots")


@pytest.mark.parametrize("tokens", [1, 3])
def test_slots_partial_permuted_bank_equals_plain_decode(gpu, tokens):
    """Only the selected experts (plus a few others) resident, shuffled into a smaller
    bank: the same bits as the plain decode over the full bank."""
    layer, x = _case("decode_e512_top10_shared", tokens)
    dl = gpu.upload_layer(layer)
    y_ref, ids_ref, w_ref = gpu.decode(dl, gpu.tokens_to_device(x))
    torch.cuda.synchronize()
    sel = np.unique(ids_ref.cpu().numpy())
    rng = np.random.default_rng(tokens)
    extra = rng.choice(np.setdiff1d(np.arange(layer.num_experts), sel), 6, replace=False)
    order = rng.permutation(np.concatenate([sel, extra]))
    slot_of = np.full(layer.num_experts, -1, np.int32)
    slot_of[order] = np.arange(len(order), dtype=np.int32)
    bank = _upload_bank(layer, _slot_bank_host(layer, order))
    y, ids, w, miss = _run_slots(gpu, layer, dl, x, bank, slot_of)
    assert np.array_equal(ids, ids_ref.cpu().numpy())
    assert np.array_equal(w.view(np.uint32), w_ref.cpu().numpy().view(np.uint32))
    assert np.all(miss == -1)
    assert np.array_equal(y, gpu.bf16_bits(y_ref))
    say(f"  T={tokens}: {len(order)} resident slots, bits equal to the plain decode")


@pytest.mark.parametrize("name,tokens,over", [
    ("decode_e512_top10_shared", 1, {}),
    ("decode_e288_top8", 1, {}),
    ("decode_e512_top10_shared", 5, {}),
    # grouped path (8 or more tokens), n_slots <= E
    ("decode_e512_top10_shared", 12, dict(num_experts=48, hidden=1024, inter=256,
                                          shared_inter=256, top_k=6)),
    ("decode_e512_top10_shared", 24, dict(num_experts=48, hidden=1024, inter=256,
                                          shared_inter=256, top_k=6)),
])
def test_slots_missing_experts_match_oracle(gpu, name, tokens, over):
    layer, x = _case(name, tokens, **over)
    E = layer.num_experts
    ids_full = oracle.topk(oracle.router_logits(x, layer.w_router, layer.bias), layer.top_k)[0]
    sel = np.unique(ids_full)
    rng = np.random.default_rng(17 + tokens)
    missing = rng.choice(sel, max(2, len(sel) // 4), replace=False)
    resident = rng.permutation(np.setdiff1d(np.arange(E), missing))[: min(E - len(missing), 40)]
    resident = np.union1d(resident, np.setdiff1d(sel, missing))
    order = rng.permutation(resident)
    slot_of = np.full(E, -1, np.int32)
    slot_of[order] = np.arange(len(order), dtype=np.int32)
    slot_of[missing[::2]] = len(order) + 3          # out of range above, too
    host_bank = _slot_bank_host(layer, order)
    ref = oracle.moe_layer_slots(layer, x, slot_of, host_bank)
    dl = gpu.upload_layer(layer)
    y, ids, w, miss = _run_slots(gpu, layer, dl, x, _upload_bank(layer, host_bank), slot_of)
    assert np.array_equal(ids, ref["ids"])
    assert np.array_equal(miss, ref["miss"])
    assert (miss >= 0).sum() >= 2
    assert_output_close(y, ref["y"], f"{name} T={tokens} slots, {len(missing)} missing")


def test_slots_bank_larger_than_the_expert_count(gpu):
    """A bank of more slots than the layer has experts (a shared expert cache)."""
    layer, x = _case("decode_e512_top10_shared", 1, num_experts=64, hidden=512, inter=128,
                     shared_inter=128)
    E, n_slots = 64, 300
    rng = np.random.default_rng(5)
    where = rng.choice(n_slots, E, replace=False).astype(np.int32)  # slot of each expert
    experts_in_slot = np.zeros(n_slots, np.int64)
    experts_in_slot[where] = np.arange(E)
    fill = np.setdiff1d(np.arange(n_slots), where)
    experts_in_slot[fill] = rng.integers(0, E, len(fill))           # other layers' experts
    host_bank = _slot_bank_host(layer, experts_in_slot)
    ref = oracle.moe_layer_slots(layer, x, where, host_bank)
    dl = gpu.upload_layer(layer)
    y, ids, _, miss = _run_slots(gpu, layer, dl, x, _upload_bank(layer, host_bank), where)
    assert np.array_equal(ids, ref["ids"]) and np.all(miss == -1)
    assert_output_close(y, ref["y"], "300-slot bank, 64 experts")


def test_slots_grouped_path_rejects_a_bank_larger_than_the_expert_count(gpu):
    from nvfp4_mixture_experts_amd import ftmoe
    lib = ftmoe._lib
    d = ftmoe.make_desc(64, 512, 128, 4, 1)
    bank = ftmoe.FtNvfp4Experts(256, 256, 256, 256, 256)
    st = lib.ft_moe_nvfp4_decode_slots(ctypes.byref(d), 8, 16, 16, None, ctypes.byref(bank), 65,
                                       16, None, None, None, None, None, 16, 256, 1 << 24, None)
    assert st == ftmoe.FT_EUNSUPPORTED
    st = lib.ft_moe_nvfp4_decode_slots(ctypes.byref(d), 1, 16, 16, None, ctypes.byref(bank), 4,
                                       None, None, None, None, None, None, 16, 256, 1 << 24, None)
    assert st == ftmoe.FT_EINVAL
