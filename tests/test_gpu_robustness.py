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
