"""Python binding of libftmoe.so (the C ABI in include/ftmoe.h).

Argument marshalling only: every function takes torch tensors (or plain ints),
checks dtype, device and contiguity, and passes raw pointers plus the current
HIP stream to the function of the same name in the library.  All compute runs in
the library's gfx950 kernels; there is no fallback: if libftmoe.so is missing or
cannot be loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libftmoe.so")
FT_ABI_VERSION = 1

FT_OK = 0
FT_EINVAL = -1
FT_EUNSUPPORTED = -2
FT_EWORKSPACE = -3
FT_EHIP = -4

# Decode calls of at least this many tokens take the grouped path inside
# ft_moe_nvfp4_decode (the library's kGroupedDecodeMinTokens; informational).
GROUPED_DECODE_MIN_TOKENS = 8
PATH_ROUTE, PATH_DECODE, PATH_PREFILL = 0, 1, 2


class FtError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where} failed with status {status}: {message}")
        self.status = status


class FtMoeDesc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("top_k", ctypes.c_int32), ("act", ctypes.c_int32),
                ("gate_max", ctypes.c_float), ("up_absmax", ctypes.c_float),
                ("shared_inter", ctypes.c_int32)]


class FtNvfp4Experts(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p)]


class FtFp8Experts(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


class FtKvCache(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("prefix", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_block_scale", ctypes.c_void_p), ("v_block_scale", ctypes.c_void_p),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run nvfp4_mixture_experts_amd.build.build() "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(FtMoeDesc)
    B = ctypes.POINTER(FtNvfp4Experts)
    F8 = ctypes.POINTER(FtFp8Experts)
    sig = {
        "ft_abi_version": (I32, []),
        "ft_last_error": (ctypes.c_char_p, []),
        "ft_init": (I32, [I32]),
        "ft_nvfp4_repacked_bytes": (SZ, [I32, I32, I32, I32]),
        "ft_nvfp4_repack": (I32, [I32, I32, I32] + [P] * 8 + [P]),
        "ft_moe_workspace_bytes": (SZ, [D, I64, I32]),
        "ft_moe_route": (I32, [D, I64, P, P, P, P, P, P, SZ, P]),
        "ft_moe_nvfp4_decode": (I32, [D, I64, P, P, P, B, B, P, P, P, P, P, SZ, P]),
        "ft_moe_nvfp4_prefill": (I32, [D, I64, P, P, P, B, B, P, P, P, SZ, P]),
        "ft_nvfp4_dequant": (I32, [I32, I32, I32, B, I32, I32, I32, P, P]),
        "ft_moe_device_status": (I32, [P, SZ, P, P]),
        "ft_set_wait_limit": (I32, [I32]),
        "ft_moe_nvfp4_decode_noalloc": (I32, [D, I64, P, P, P, B, B, P, P, P, P, P, P]),
        "ft_moe_nvfp4_decode_slots": (I32, [D, I64, P, P, P, B, I32, P, B, P, P, P, P, P, P,
                                            SZ, P]),
        "ft_fp8_repacked_bytes": (SZ, [I32, I32, I32, I32]),
        "ft_fp8_repack": (I32, [I32, I32, I32] + [P] * 8 + [P]),
        "ft_moe_fp8_decode": (I32, [D, I64, P, P, P, F8, F8, P, P, P, P, P, SZ, P]),
        "ft_fp8_dequant": (I32, [I32, I32, I32, F8, I32, I32, I32, P, P]),
        "ft_fp8_linear_workspace_bytes": (SZ, [I64, I64]),
        "ft_fp8_quantize": (I32, [I64, I64, P, P, P, P, SZ, P]),
        "ft_fp8_linear": (I32, [I64, I64, I64, P, P, P, P, P, SZ, P]),
        "ft_fp8_linear_parts": (I32, [I64, I64, P, P, I32, P, P, P, P, SZ, P]),
        "ft_fp8_scale_runs": (I32, [P, I64, P, P, I32]),
        "ft_attn_extend": (I32, [I32, I32, I32, I32, I32, P, P, P,
                                 ctypes.POINTER(FtKvCache), P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.ft_abi_version() != FT_ABI_VERSION:
        raise ImportError(f"libftmoe.so ABI {lib.ft_abi_version()} != {FT_ABI_VERSION}")
    return lib


_lib = _load()
EXPORTED = ("ft_abi_version", "ft_last_error", "ft_init", "ft_nvfp4_repacked_bytes",
            "ft_nvfp4_repack", "ft_moe_workspace_bytes", "ft_moe_route", "ft_moe_nvfp4_decode",
            "ft_moe_nvfp4_prefill", "ft_nvfp4_dequant", "ft_moe_device_status",
            "ft_set_wait_limit", "ft_moe_nvfp4_decode_noalloc", "ft_moe_nvfp4_decode_slots",
            "ft_fp8_repacked_bytes", "ft_fp8_repack", "ft_moe_fp8_decode", "ft_fp8_dequant",
            "ft_fp8_linear_workspace_bytes", "ft_fp8_quantize", "ft_fp8_linear",
            "ft_fp8_linear_parts", "ft_fp8_scale_runs", "ft_attn_extend")


def library_path() -> str:
    return _LIB_PATH


def _check(status: int, where: str) -> None:
    if status != FT_OK:
        raise FtError(status, where, _lib.ft_last_error().decode())


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live in device memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_desc(num_experts: int, hidden: int, inter: int, top_k: int, act: int,
              gate_max: float = 7.0, up_absmax: float = 7.0, shared_inter: int = 0) -> FtMoeDesc:
    return FtMoeDesc(num_experts, hidden, inter, top_k, act, gate_max, up_absmax, shared_inter)


class Bank:
    """A repacked NVFP4 expert bank (device tensors) and its C view."""

    def __init__(self, hidden: int, inter: int, n: int, w13, w13_scale, w2, w2_scale,
                 global_scale):
        self.hidden, self.inter, self.n = hidden, inter, n
        self.w13, self.w13_scale, self.w2, self.w2_scale = w13, w13_scale, w2, w2_scale
        self.global_scale = global_scale
        self.c = FtNvfp4Experts(_ptr(w13, torch.uint8, "w13"), _ptr(w13_scale, torch.uint8),
                                _ptr(w2, torch.uint8, "w2"), _ptr(w2_scale, torch.uint8),
                                _ptr(global_scale, torch.float32, "global_scale"))

    def ref(self):
        return ctypes.byref(self.c)


# ------------------------------------------------------------- entry points --

def ft_abi_version() -> int:
    return _lib.ft_abi_version()


def ft_last_error() -> str:
    return _lib.ft_last_error().decode()


def ft_init(device: int = 0) -> None:
    _check(_lib.ft_init(device), "ft_init")


def ft_nvfp4_repacked_bytes(hidden: int, inter: int, n_experts: int, part: int) -> int:
    return _lib.ft_nvfp4_repacked_bytes(hidden, inter, n_experts, part)


def ft_nvfp4_repack(hidden: int, inter: int, n_experts: int, w13, w13_scale, w2, w2_scale,
                    global_scale, stream=None) -> Bank:
    """Repack a canonical bank (device uint8 tensors) into newly allocated device buffers."""
    dev = w13.device
    outs = [torch.empty(ft_nvfp4_repacked_bytes(hidden, inter, n_experts, p), dtype=torch.uint8,
                        device=dev) for p in range(4)]
    _check(_lib.ft_nvfp4_repack(hidden, inter, n_experts,
                                _ptr(w13, torch.uint8, "w13"), _ptr(w13_scale, torch.uint8),
                                _ptr(w2, torch.uint8, "w2"), _ptr(w2_scale, torch.uint8),
                                *[o.data_ptr() for o in outs], _stream(stream)),
           "ft_nvfp4_repack")
    return Bank(hidden, inter, n_experts, *outs, global_scale.contiguous())


def ft_moe_workspace_bytes(desc: FtMoeDesc, tokens: int, path: int) -> int:
    return _lib.ft_moe_workspace_bytes(ctypes.byref(desc), tokens, path)


def alloc_workspace(desc: FtMoeDesc, tokens: int, path: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (zero fill is required once, before first use)."""
    n = ft_moe_workspace_bytes(desc, tokens, path)
    if n == 0:
        raise FtError(FT_EINVAL, "ft_moe_workspace_bytes", "invalid descriptor or token count")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def ft_moe_route(desc: FtMoeDesc, x, w_router, bias, topk_ids, topk_w, workspace,
                 stream=None) -> None:
    _check(_lib.ft_moe_route(ctypes.byref(desc), x.shape[0], _ptr(x, torch.bfloat16, "x"),
                             _ptr(w_router, torch.float32, "w_router"),
                             _ptr(bias, torch.float32, "bias"),
                             _ptr(topk_ids, torch.int32, "topk_ids"),
                             _ptr(topk_w, torch.float32, "topk_w"),
                             _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                             _stream(stream)), "ft_moe_route")


def ft_moe_nvfp4_decode(desc: FtMoeDesc, x, w_router, bias, routed: Bank, shared: Optional[Bank],
                        shared_gate, y, workspace, topk_ids_out=None, topk_w_out=None,
                        stream=None) -> None:
    _check(_lib.ft_moe_nvfp4_decode(ctypes.byref(desc), x.shape[0], _ptr(x, torch.bfloat16, "x"),
                                    _ptr(w_router, torch.float32, "w_router"),
                                    _ptr(bias, torch.float32, "bias"), routed.ref(),
                                    shared.ref() if shared is not None else None,
                                    _ptr(shared_gate, torch.bfloat16, "shared_gate"),
                                    _ptr(topk_ids_out, torch.int32, "topk_ids_out"),
                                    _ptr(topk_w_out, torch.float32, "topk_w_out"),
                                    _ptr(y, torch.bfloat16, "y"),
                                    _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                    _stream(stream)), "ft_moe_nvfp4_decode")


def ft_moe_nvfp4_prefill(desc: FtMoeDesc, x, topk_ids, topk_w, routed: Bank,
                         shared: Optional[Bank], shared_gate, y, workspace, stream=None) -> None:
    _check(_lib.ft_moe_nvfp4_prefill(ctypes.byref(desc), x.shape[0], _ptr(x, torch.bfloat16, "x"),
                                     _ptr(topk_ids, torch.int32, "topk_ids"),
                                     _ptr(topk_w, torch.float32, "topk_w"), routed.ref(),
                                     shared.ref() if shared is not None else None,
                                     _ptr(shared_gate, torch.bfloat16, "shared_gate"),
                                     _ptr(y, torch.bfloat16, "y"),
                                     _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                     _stream(stream)), "ft_moe_nvfp4_prefill")


# ft_nvfp4_dequant modes (see include/ftmoe.h)
DEQ_F32, DEQ_BF16, DEQ_TILE_BF16, DEQ_GATEUP_F32, DEQ_TILE_F16 = 0, 1, 2, 3, 4


def ft_nvfp4_dequant(bank: Bank, expert: int, tensor: int, out, stream=None,
                     mode: Optional[int] = None) -> None:
    """out: fp32, bf16 or fp16 [rows][K] device tensor (gate/up [I][H], down [H][I]).
    ``mode`` defaults to DEQ_F32 for fp32 ``out`` and DEQ_BF16 for bf16 ``out``."""
    want = {DEQ_F32: torch.float32, DEQ_BF16: torch.bfloat16, DEQ_TILE_BF16: torch.bfloat16,
            DEQ_GATEUP_F32: torch.float32, DEQ_TILE_F16: torch.float16}
    if mode is None:
        if out.dtype == torch.float32:
            mode = DEQ_F32
        elif out.dtype == torch.bfloat16:
            mode = DEQ_BF16
        else:
            raise TypeError("out must be float32 or bfloat16")
    if mode not in want:
        raise ValueError(f"unknown dequant mode {mode}")
    if out.dtype != want[mode]:
        raise TypeError(f"mode {mode} writes {want[mode]}, out is {out.dtype}")
    dt = mode
    _check(_lib.ft_nvfp4_dequant(bank.hidden, bank.inter, bank.n, bank.ref(), expert, tensor, dt,
                                 _ptr(out, None, "out"), _stream(stream)), "ft_nvfp4_dequant")


# reasons ft_moe_device_status reports (OR-ed)
WAIT_LOGITS, WAIT_GATE, WAIT_H, WAIT_PARTIAL = 1, 2, 4, 8


def ft_moe_device_status(workspace, status, stream=None) -> None:
    """Enqueue: copy the decode workspace's give-up reasons to ``status`` (int32 device
    tensor, one element) and clear them."""
    _check(_lib.ft_moe_device_status(_ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                     _ptr(status, torch.int32, "status"), _stream(stream)),
           "ft_moe_device_status")


def device_status(workspace, stream=None) -> int:
    """Reads and clears the give-up reasons of a decode workspace (synchronises)."""
    st = torch.zeros(1, dtype=torch.int32, device=workspace.device)
    ft_moe_device_status(workspace, st, stream)
    return int(st.item())


def ft_set_wait_limit(polls: int) -> None:
    _check(_lib.ft_set_wait_limit(int(polls)), "ft_set_wait_limit")


def ft_moe_nvfp4_decode_noalloc(desc: FtMoeDesc, x, w_router, bias, routed: Bank,
                                shared: Optional[Bank], shared_gate, y, topk_ids_out=None,
                                topk_w_out=None, status=None, stream=None) -> None:
    """ft_moe_nvfp4_decode on the library's static scratch (1..7 tokens, no workspace)."""
    _check(_lib.ft_moe_nvfp4_decode_noalloc(
        ctypes.byref(desc), x.shape[0], _ptr(x, torch.bfloat16, "x"),
        _ptr(w_router, torch.float32, "w_router"), _ptr(bias, torch.float32, "bias"),
        routed.ref(), shared.ref() if shared is not None else None,
        _ptr(shared_gate, torch.bfloat16, "shared_gate"),
        _ptr(topk_ids_out, torch.int32, "topk_ids_out"),
        _ptr(topk_w_out, torch.float32, "topk_w_out"), _ptr(y, torch.bfloat16, "y"),
        _ptr(status, torch.int32, "status"), _stream(stream)), "ft_moe_nvfp4_decode_noalloc")


def ft_moe_nvfp4_decode_slots(desc: FtMoeDesc, x, w_router, bias, slots: Bank, slot_of,
                              shared: Optional[Bank], shared_gate, y, workspace,
                              topk_ids_out=None, topk_w_out=None, miss_out=None,
                              stream=None) -> None:
    """ft_moe_nvfp4_decode over a bank of expert slots; ``slot_of`` int32 [E] device."""
    _check(_lib.ft_moe_nvfp4_decode_slots(
        ctypes.byref(desc), x.shape[0], _ptr(x, torch.bfloat16, "x"),
        _ptr(w_router, torch.float32, "w_router"), _ptr(bias, torch.float32, "bias"),
        slots.ref(), slots.n, _ptr(slot_of, torch.int32, "slot_of"),
        shared.ref() if shared is not None else None,
        _ptr(shared_gate, torch.bfloat16, "shared_gate"),
        _ptr(topk_ids_out, torch.int32, "topk_ids_out"),
        _ptr(topk_w_out, torch.float32, "topk_w_out"), _ptr(miss_out, torch.int32, "miss_out"),
        _ptr(y, torch.bfloat16, "y"), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream)), "ft_moe_nvfp4_decode_slots")


# ------------------------------------------------------------- block-fp8 --

class Fp8Bank:
    """A repacked block-fp8 expert bank (device tensors) and its C view."""

    def __init__(self, hidden: int, inter: int, n: int, w13, w13_scale, w2, w2_scale):
        self.hidden, self.inter, self.n = hidden, inter, n
        self.w13, self.w13_scale, self.w2, self.w2_scale = w13, w13_scale, w2, w2_scale
        self.c = FtFp8Experts(_ptr(w13, torch.uint8, "w13"), _ptr(w13_scale, torch.float32),
                              _ptr(w2, torch.uint8, "w2"), _ptr(w2_scale, torch.float32))

    def ref(self):
        return ctypes.byref(self.c)


def ft_fp8_repacked_bytes(hidden: int, inter: int, n_experts: int, part: int) -> int:
    return _lib.ft_fp8_repacked_bytes(hidden, inter, n_experts, part)


def ft_fp8_repack(hidden: int, inter: int, n_experts: int, w13, w13_scale, w2, w2_scale,
                  stream=None) -> Fp8Bank:
    """Repack a canonical block-fp8 bank (device tensors) into newly allocated buffers."""
    dev = w13.device
    nb = [ft_fp8_repacked_bytes(hidden, inter, n_experts, p) for p in range(4)]
    outs = [torch.empty(nb[0], dtype=torch.uint8, device=dev),
            torch.empty(nb[1] // 4, dtype=torch.float32, device=dev),
            torch.empty(nb[2], dtype=torch.uint8, device=dev),
            torch.empty(nb[3] // 4, dtype=torch.float32, device=dev)]
    _check(_lib.ft_fp8_repack(hidden, inter, n_experts, _ptr(w13, torch.uint8, "w13"),
                              _ptr(w13_scale, torch.float32, "w13_scale"),
                              _ptr(w2, torch.uint8, "w2"), _ptr(w2_scale, torch.float32, "w2_scale"),
                              *[o.data_ptr() for o in outs], _stream(stream)), "ft_fp8_repack")
    return Fp8Bank(hidden, inter, n_experts, *outs)


def ft_moe_fp8_decode(desc: FtMoeDesc, x, w_router, bias, routed: Fp8Bank,
                      shared: Optional[Fp8Bank], shared_gate, y, workspace, topk_ids_out=None,
                      topk_w_out=None, stream=None) -> None:
    _check(_lib.ft_moe_fp8_decode(ctypes.byref(desc), x.shape[0], _ptr(x, torch.bfloat16, "x"),
                                  _ptr(w_router, torch.float32, "w_router"),
                                  _ptr(bias, torch.float32, "bias"), routed.ref(),
                                  shared.ref() if shared is not None else None,
                                  _ptr(shared_gate, torch.bfloat16, "shared_gate"),
                                  _ptr(topk_ids_out, torch.int32, "topk_ids_out"),
                                  _ptr(topk_w_out, torch.float32, "topk_w_out"),
                                  _ptr(y, torch.bfloat16, "y"),
                                  _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                  _stream(stream)), "ft_moe_fp8_decode")


def ft_fp8_dequant(bank: Fp8Bank, expert: int, tensor: int, out, mode: int = 0,
                   stream=None) -> None:
    _check(_lib.ft_fp8_dequant(bank.hidden, bank.inter, bank.n, bank.ref(), expert, tensor, mode,
                               _ptr(out, torch.float32, "out"), _stream(stream)), "ft_fp8_dequant")


# ------------------------------------------------ per-tensor FP8 W8A8 linear --

def fp8_linear_workspace(M: int, K: int, device="cuda") -> torch.Tensor:
    n = _lib.ft_fp8_linear_workspace_bytes(M, K)
    if n == 0:
        raise FtError(FT_EUNSUPPORTED, "ft_fp8_linear_workspace_bytes", f"M={M} K={K}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def ft_fp8_quantize(x, xq, x_scale, workspace, stream=None) -> None:
    M, K = x.shape
    _check(_lib.ft_fp8_quantize(M, K, _ptr(x, torch.bfloat16, "x"), _ptr(xq, torch.uint8, "xq"),
                                _ptr(x_scale, torch.float32, "x_scale"),
                                _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                _stream(stream)), "ft_fp8_quantize")


def ft_fp8_linear(x, w, w_scale_rows, y, workspace, stream=None) -> None:
    M, K = x.shape
    N = w.shape[0]
    _check(_lib.ft_fp8_linear(M, N, K, _ptr(x, torch.bfloat16, "x"), _ptr(w, torch.uint8, "w"),
                              _ptr(w_scale_rows, torch.float32, "w_scale_rows"),
                              _ptr(y, torch.bfloat16, "y"), _ptr(workspace, torch.uint8,
                                                                 "workspace"),
                              workspace.numel(), _stream(stream)), "ft_fp8_linear")


def ft_fp8_scale_runs(w_scale_rows, max_parts: int = 64):
    """Host: (part_rows int64 [n + 1], part_scales float32 [n]) of a host scale vector."""
    import numpy as np
    rows = np.ascontiguousarray(np.asarray(w_scale_rows, dtype=np.float32))
    pr = np.zeros(max_parts + 1, np.int64)
    ps = np.zeros(max_parts, np.float32)
    n = _lib.ft_fp8_scale_runs(rows.ctypes.data, rows.size, pr.ctypes.data, ps.ctypes.data,
                               max_parts)
    if n < 0:
        raise FtError(FT_EINVAL, "ft_fp8_scale_runs", "bad arguments or too many runs")
    return pr[:n + 1].copy(), ps[:n].copy()


def ft_fp8_linear_parts(x, w, part_rows, part_scales, y, workspace, stream=None) -> None:
    import numpy as np
    M, K = x.shape
    pr = np.ascontiguousarray(np.asarray(part_rows, dtype=np.int64))
    ps = np.ascontiguousarray(np.asarray(part_scales, dtype=np.float32))
    _check(_lib.ft_fp8_linear_parts(M, K, _ptr(x, torch.bfloat16, "x"), _ptr(w, torch.uint8, "w"),
                                    len(ps), pr.ctypes.data, ps.ctypes.data,
                                    _ptr(y, torch.bfloat16, "y"),
                                    _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                    _stream(stream)), "ft_fp8_linear_parts")


# -------------------------------------------------- extend attention, KV cache --

def ft_attn_extend(q, k_new, v_new, cache_format: int, prefix: int, k_cache, v_cache, out,
                   window: int = 0, k_block_scale=None, v_block_scale=None, k_scale: float = 1.0,
                   v_scale: float = 1.0, stream=None) -> None:
    """q bf16 [n_new, Hq, d]; k_new / v_new bf16 [n_new, Hkv, d]; cache tensors as in
    include/ftmoe.h (None when prefix == 0); out bf16 [n_new, Hq, d]."""
    n_new, Hq, d = q.shape
    Hkv = k_new.shape[1]
    cdt = torch.bfloat16 if cache_format == 0 else torch.uint8
    c = FtKvCache(cache_format, prefix, _ptr(k_cache, cdt, "k_cache"), _ptr(v_cache, cdt, "v_cache"),
                  _ptr(k_block_scale, torch.uint8, "k_block_scale"),
                  _ptr(v_block_scale, torch.uint8, "v_block_scale"), k_scale, v_scale)
    _check(_lib.ft_attn_extend(n_new, Hq, Hkv, d, window, _ptr(q, torch.bfloat16, "q"),
                               _ptr(k_new, torch.bfloat16, "k_new"),
                               _ptr(v_new, torch.bfloat16, "v_new"), ctypes.byref(c),
                               _ptr(out, torch.bfloat16, "out"), _stream(stream)),
           "ft_attn_extend")
