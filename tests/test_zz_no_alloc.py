"""ft_moe_nvfp4_decode_noalloc (the decode call that allocates nothing and runs on
the library's static scratch) against ft_moe_nvfp4_decode with a workspace of its
own: identical outputs, routes and weights, on consecutive calls of decreasing size
and of different layer shapes, with every device-side wait completed."""
import ctypes

import numpy as np
import pytest
import torch

from nvfp4_mixture_experts_amd import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _both(device, ftmoe, dl, xh):
    x = device.tokens_to_device(xh)
    T = x.shape[0]
    y_ref, ids_ref, w_ref = device.decode(dl, x)
    y = torch.empty_like(y_ref)
    ids = torch.full_like(ids_ref, -1)
    w = torch.full_like(w_ref, -1.0)
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ftmoe.ft_moe_nvfp4_decode_noalloc(dl.desc, x, dl.w_router, dl.bias, dl.routed, dl.shared,
                                      dl.shared_gate, y, ids, w, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(ids, ids_ref), T
    assert torch.equal(w.view(torch.int32), w_ref.view(torch.int32)), T
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), T
    say(f"  T={T}: no-alloc call equals the workspace call bit for bit")


def test_decode_noalloc_matches_decode_on_consecutive_calls():
    assert torch.cuda.is_available()
    from nvfp4_mixture_experts_amd import device, ftmoe
    ftmoe.ft_init(0)
    w2 = synth.WORKLOADS["decode_e512_top10_shared"]
    dl2 = device.upload_layer(synth.make_layer(w2))
    # two calls in a row, the second smaller, then a layer of another shape, then
    # the first layer again
    _both(device, ftmoe, dl2, synth.make_tokens(w2, tokens=5, stream="na0"))
    _both(device, ftmoe, dl2, synth.make_tokens(w2, tokens=1, stream="na1"))
    w1 = synth.WORKLOADS["decode_e288_top8"]
    dl1 = device.upload_layer(synth.make_layer(w1))
    _both(device, ftmoe, dl1, synth.make_tokens(w1, tokens=1, stream="na2"))
    _both(device, ftmoe, dl2, synth.make_tokens(w2, tokens=3, stream="na3"))


def test_decode_noalloc_rejects_what_it_cannot_hold():
    from nvfp4_mixture_experts_amd import ftmoe
    ftmoe.ft_init(0)
    lib = ftmoe._lib
    d = ftmoe.make_desc(288, 2048, 768, 8, 1)
    bank = ftmoe.FtNvfp4Experts(256, 256, 256, 256, 256)
    b = ctypes.byref(bank)
    args = (16, 16, None, b, None, None, None, None, 16, None, None)
    assert lib.ft_moe_nvfp4_decode_noalloc(ctypes.byref(d), 8, *args) == ftmoe.FT_EUNSUPPORTED
    assert lib.ft_moe_nvfp4_decode_noalloc(ctypes.byref(d), 0, *args) == ftmoe.FT_EINVAL
    big = ftmoe.make_desc(1024, 8192, 4096, 16, 1, shared_inter=4096)
    assert ftmoe.ft_moe_workspace_bytes(big, 7, ftmoe.PATH_DECODE) > (4 << 20)
    assert lib.ft_moe_nvfp4_decode_noalloc(ctypes.byref(big), 7, *args) == ftmoe.FT_EWORKSPACE
    assert "scratch" in ftmoe.ft_last_error()
