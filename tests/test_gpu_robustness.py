"""GPU behaviour on caller errors that only exist in device memory.

Routes passed to ft_moe_nvfp4_prefill live in device memory and cannot be
checked on the host without a synchronisation.  An id outside [0, E) must not
make a kernel read outside the expert bank: that token's output becomes NaN and
every other token is unaffected.
"""
import numpy as np
import pytest
import torch

from nvfp4_mixture_experts_amd import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_prefill_out_of_range_ids_poison_only_their_token():
    assert torch.cuda.is_available()
    from nvfp4_mixture_experts_amd import device, ftmoe
    ftmoe.ft_init(0)
    w = synth.dataclasses.replace(synth.WORKLOADS["prefill_t8192"], num_experts=16, tokens=6)
    L = synth.make_layer(w)
    dl = device.upload_layer(L)
    x = device.tokens_to_device(synth.make_tokens(w))
    rng = np.random.default_rng(5)
    ids = np.stack([rng.permutation(16)[: w.top_k] for _ in range(6)]).astype(np.int32)
    wts = np.full((6, w.top_k), 1.0 / w.top_k, np.float32)
    good = device.prefill(dl, x, torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda())
    bad_ids = ids.copy()
    bad_ids[2, 3] = 16            # one past the end
    bad_ids[4, 0] = -7
    bad = device.prefill(dl, x, torch.from_numpy(bad_ids).cuda(), torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    g = good.float().cpu().numpy()
    b = bad.float().cpu().numpy()
    say(f"  nan rows: {sorted(set(np.nonzero(np.isnan(b))[0].tolist()))}")
    assert np.isnan(b[2]).all() and np.isnan(b[4]).all()
    keep = [0, 1, 3, 5]
    assert np.array_equal(b[keep], g[keep])


@pytest.mark.parametrize("tokens", [1, 16])   # one-launch decode kernel; decode routing kernel
def test_decode_wait_give_up_is_reported_and_the_next_workspace_is_clean(tokens):
    """The one-launch decode kernel's blocks (and those of the routing kernel of a
    decode batch) agree on a call's generation by each counting its own calls;
    values handed between blocks carry that generation.
    Here the per-block counters of one workspace are set to unequal values from
    the host, so no hand-off can complete: with a small wait limit every wait
    gives up after a bounded number of polls, the kernel finishes, and
    ft_moe_device_status reports it (and clears it).  A fresh workspace then
    gives the oracle's result with a clean status."""
    import oracle
    from nvfp4_mixture_experts_amd import device, ftmoe
    from tests.gpu_util import assert_output_close
    assert torch.cuda.is_available()
    ftmoe.ft_init(0)
    w = synth.dataclasses.replace(synth.WORKLOADS["decode_e512_top10_shared"], num_experts=32,
                                  hidden=256, inter=128, shared_inter=128)
    L = synth.make_layer(w)
    dl = device.upload_layer(L)
    xh = synth.make_tokens(w, tokens=tokens)
    x = device.tokens_to_device(xh)
    ref = oracle.moe_layer(L, xh)

    ws = ftmoe.alloc_workspace(dl.desc, tokens, ftmoe.PATH_DECODE, "cuda")
    y, ids, _ = device.decode(dl, x, ws)
    assert ftmoe.device_status(ws) == 0
    # per-block call counters: bytes [256, 256 + 4 * 1024) of a decode workspace
    rng = np.random.default_rng(11)
    ws[256:256 + 4096] = torch.from_numpy(rng.integers(0, 256, 4096, dtype=np.uint8)).cuda()
    say("  desynchronised the block counters; wait limit 64 polls")
    try:
        ftmoe.ft_set_wait_limit(64)
        device.decode(dl, x, ws)
        torch.cuda.synchronize()
    finally:
        ftmoe.ft_set_wait_limit(0)
    st = ftmoe.device_status(ws)
    say(f"  status after the desynchronised call: {st:#x}")
    assert st != 0 and (st & ~0x1F) == 0
    assert ftmoe.device_status(ws) == 0           # the read cleared it

    ws2 = ftmoe.alloc_workspace(dl.desc, tokens, ftmoe.PATH_DECODE, "cuda")
    y2, ids2, _ = device.decode(dl, x, ws2)
    torch.cuda.synchronize()
    assert ftmoe.device_status(ws2) == 0
    assert np.array_equal(ids2.cpu().numpy(), ref["ids"])
    assert_output_close(device.bf16_bits(y2), ref["y"], "fresh workspace after a give-up")
    assert np.array_equal(device.bf16_bits(y2), device.bf16_bits(y))
