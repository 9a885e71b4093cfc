"""Device-side plumbing around the C ABI: upload canonical NVFP4 layer weights,
repack them with ft_nvfp4_repack, and run the layer entry points.

Only torch allocations and copies happen here; the layer itself is computed by
libftmoe.so.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import ftmoe


def _dev(a, device, dtype=None):
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.to(device)
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


@dataclasses.dataclass
class DeviceLayer:
    desc: ftmoe.FtMoeDesc
    w_router: torch.Tensor
    bias: Optional[torch.Tensor]
    routed: ftmoe.Bank
    shared: Optional[ftmoe.Bank]
    shared_gate: Optional[torch.Tensor]

    @property
    def hidden(self) -> int:
        return self.desc.hidden

    @property
    def top_k(self) -> int:
        return self.desc.top_k


def desc_of(workload) -> ftmoe.FtMoeDesc:
    return ftmoe.make_desc(workload.num_experts, workload.hidden, workload.inter, workload.top_k,
                           workload.act, workload.gate_max, workload.up_absmax,
                           workload.shared_inter)


def upload_canonical(workload, w_router, bias, routed: dict, shared: Optional[dict],
                     shared_gate, device="cuda") -> DeviceLayer:
    """``routed``/``shared``: dicts of canonical tensors (w13_codes, w13_scales, w2_codes,
    w2_scales, global_scale) as numpy arrays or device tensors."""
    desc = desc_of(workload)

    def bank(b, inter, n):
        return ftmoe.ft_nvfp4_repack(
            workload.hidden, inter, n,
            _dev(b["w13_codes"], device).contiguous(), _dev(b["w13_scales"], device).contiguous(),
            _dev(b["w2_codes"], device).contiguous(), _dev(b["w2_scales"], device).contiguous(),
            _dev(b["global_scale"], device).contiguous())

    r = bank(routed, workload.inter, workload.num_experts)
    s = bank(shared, workload.shared_inter, 1) if shared is not None else None
    sg = _dev(shared_gate, device, torch.bfloat16) if shared_gate is not None else None
    if sg is not None and sg.dtype != torch.bfloat16:
        sg = sg.view(torch.bfloat16)
    return DeviceLayer(desc, _dev(w_router, device).contiguous(),
                       _dev(bias, device) if bias is not None else None, r, s,
                       sg.contiguous() if sg is not None else None)


def upload_layer(layer, device="cuda") -> DeviceLayer:
    """Upload a host ``synth.Layer``."""
    routed = dict(w13_codes=layer.w13_codes, w13_scales=layer.w13_scales,
                  w2_codes=layer.w2_codes, w2_scales=layer.w2_scales,
                  global_scale=layer.global_scale)
    shared = None
    if layer.shared_inter > 0:
        shared = dict(w13_codes=layer.s13_codes, w13_scales=layer.s13_scales,
                      w2_codes=layer.s2_codes, w2_scales=layer.s2_scales,
                      global_scale=layer.s_global)
    return upload_canonical(layer.workload, layer.w_router, layer.bias, routed, shared,
                            layer.shared_gate, device)


def tokens_to_device(x_bits: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bits (uint16 numpy) -> bf16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(
        torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def decode(dl: DeviceLayer, x: torch.Tensor, workspace: Optional[torch.Tensor] = None,
           stream=None, status: Optional[torch.Tensor] = None):
    """Returns (y bf16 [T, H], topk_ids, topk_w) on the device.  With ``status`` (int32
    device tensor of one element), the workspace's give-up reasons are copied there
    after the call (0 = every device-side wait completed)."""
    T = x.shape[0]
    if workspace is None:
        workspace = ftmoe.alloc_workspace(dl.desc, T, ftmoe.PATH_DECODE, x.device)
    y = torch.empty((T, dl.hidden), dtype=torch.bfloat16, device=x.device)
    ids = torch.empty((T, dl.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, dl.top_k), dtype=torch.float32, device=x.device)
    ftmoe.ft_moe_nvfp4_decode(dl.desc, x, dl.w_router, dl.bias, dl.routed, dl.shared,
                              dl.shared_gate, y, workspace, ids, w, stream=stream)
    if status is not None:
        ftmoe.ft_moe_device_status(workspace, status, stream)
    return y, ids, w


def route(dl: DeviceLayer, x: torch.Tensor, workspace: Optional[torch.Tensor] = None,
          stream=None):
    T = x.shape[0]
    if workspace is None:
        workspace = ftmoe.alloc_workspace(dl.desc, T, ftmoe.PATH_ROUTE, x.device)
    ids = torch.empty((T, dl.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, dl.top_k), dtype=torch.float32, device=x.device)
    ftmoe.ft_moe_route(dl.desc, x, dl.w_router, dl.bias, ids, w, workspace, stream=stream)
    return ids, w


def prefill(dl: DeviceLayer, x: torch.Tensor, ids: torch.Tensor, w: torch.Tensor,
            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T = x.shape[0]
    if workspace is None:
        workspace = ftmoe.alloc_workspace(dl.desc, T, ftmoe.PATH_PREFILL, x.device)
    y = torch.empty((T, dl.hidden), dtype=torch.bfloat16, device=x.device)
    ftmoe.ft_moe_nvfp4_prefill(dl.desc, x, ids, w, dl.routed, dl.shared, dl.shared_gate, y,
                               workspace, stream=stream)
    return y


def upload_fp8_canonical(w, w_router, bias, routed: dict, shared: Optional[dict], shared_gate,
                         device="cuda") -> DeviceLayer:
    """Block-fp8 banks given as dicts of canonical arrays or device tensors (w13_codes,
    w13_scales, w2_codes, w2_scales), repacked with ft_fp8_repack."""
    desc = desc_of(w)

    def bank(b, inter, n):
        d = lambda a: _dev(a, device).contiguous()
        return ftmoe.ft_fp8_repack(w.hidden, inter, n, d(b["w13_codes"]),
                                   d(b["w13_scales"]).float(), d(b["w2_codes"]),
                                   d(b["w2_scales"]).float())

    r = bank(routed, w.inter, w.num_experts)
    s = bank(shared, w.shared_inter, 1) if shared is not None else None
    sg = _dev(shared_gate, device, torch.bfloat16) if shared_gate is not None else None
    if sg is not None and sg.dtype != torch.bfloat16:
        sg = sg.view(torch.bfloat16)
    return DeviceLayer(desc, _dev(w_router, device).contiguous(),
                       _dev(bias, device) if bias is not None else None, r, s,
                       sg.contiguous() if sg is not None else None)


def upload_fp8_layer(layer, device="cuda") -> DeviceLayer:
    """Upload a host ``synth.Fp8Layer`` (block-fp8 banks, repacked with ft_fp8_repack)."""
    w = layer.workload
    routed = dict(w13_codes=layer.w13_codes, w13_scales=layer.w13_scales,
                  w2_codes=layer.w2_codes, w2_scales=layer.w2_scales)
    shared = None
    if w.shared_inter > 0:
        shared = dict(w13_codes=layer.s13_codes, w13_scales=layer.s13_scales,
                      w2_codes=layer.s2_codes, w2_scales=layer.s2_scales)
    return upload_fp8_canonical(w, layer.w_router, layer.bias, routed, shared, layer.shared_gate,
                                device)


def decode_fp8(dl: DeviceLayer, x: torch.Tensor, workspace: Optional[torch.Tensor] = None,
               stream=None, status: Optional[torch.Tensor] = None):
    """ft_moe_fp8_decode; returns (y, topk_ids, topk_w) on the device."""
    T = x.shape[0]
    if workspace is None:
        workspace = ftmoe.alloc_workspace(dl.desc, T, ftmoe.PATH_DECODE, x.device)
    y = torch.empty((T, dl.hidden), dtype=torch.bfloat16, device=x.device)
    ids = torch.empty((T, dl.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, dl.top_k), dtype=torch.float32, device=x.device)
    ftmoe.ft_moe_fp8_decode(dl.desc, x, dl.w_router, dl.bias, dl.routed, dl.shared,
                            dl.shared_gate, y, workspace, ids, w, stream=stream)
    if status is not None:
        ftmoe.ft_moe_device_status(workspace, status, stream)
    return y, ids, w
