"""CPU oracle for the NVFP4 mixture-of-experts layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports, links or runs it, and it never imports the
product: the two sides meet only in the seeded input arrays of
``nvfp4_mixture_experts_amd.synth``.

The arithmetic lives in ``ftmoe_oracle.c`` (plain C, binary64, one element at a
time); this module only compiles it with gcc and marshals numpy arrays through
ctypes.  Definitions and the readings taken where the pages are silent are
documented at the top of the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ftmoe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_ftmoe_oracle.so")
# the same source built with OpenMP: only for timing the oracle on every host core
_OMP_LIB_PATH = os.path.join(_HERE, "_ftmoe_oracle_omp.so")
_libs = {}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_F64 = ctypes.c_double


_CFLAGS = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared"]


def build() -> str:
    """Compile the oracle into ``oracle/_ftmoe_oracle.so`` (gcc, no fast-math, no contraction;
    the OpenMP pragmas ignored) and the OpenMP timing copy ``oracle/_ftmoe_oracle_omp.so``."""
    cmd = _CFLAGS + ["-Wno-unknown-pragmas", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    cmd = _CFLAGS + ["-fopenmp", _SRC, "-o", _OMP_LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_OMP_LIB_PATH + ".tmp", _OMP_LIB_PATH)
    return _LIB_PATH


def _load(omp: bool = False):
    if omp in _libs:
        return _libs[omp]
    path = _OMP_LIB_PATH if omp else _LIB_PATH
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    lib.or_e2m1.restype = _F64
    lib.or_e2m1.argtypes = [ctypes.c_uint32]
    lib.or_e4m3.restype = _F64
    lib.or_e4m3.argtypes = [ctypes.c_uint32]
    lib.or_dequant_value.restype = _F32
    lib.or_dequant_value.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _F32]
    lib.or_dequant_matrix.restype = None
    lib.or_dequant_matrix.argtypes = [_P, _P, _I64, _I64, _F32, _P]
    lib.or_bf16_to_double.restype = _F64
    lib.or_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.or_bf16_from_double.restype = ctypes.c_uint16
    lib.or_bf16_from_double.argtypes = [_F64]
    lib.or_router_logits.restype = None
    lib.or_router_logits.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P]
    lib.or_topk.restype = None
    lib.or_topk.argtypes = [_I64, _I32, _I32, _P, _P, _P]
    lib.or_silu.restype = _F64
    lib.or_silu.argtypes = [_F64]
    lib.or_swiglu.restype = _F64
    lib.or_swiglu.argtypes = [_I32, _F64, _F64, _F64, _F64]
    lib.or_expert_output.restype = None
    lib.or_expert_output.argtypes = [_I32, _I32, _I64, _P, _P, _P, _P, _P, _I32, _F32, _F32,
                                     _P, _P]
    lib.or_threads.restype = _I32
    lib.or_threads.argtypes = []
    lib.or_moe_layer.restype = _I32
    lib.or_moe_layer.argtypes = ([_I32, _I32, _I32, _I32, _I32, _F32, _F32, _I64, _P, _P, _P]
                                 + [_P] * 5 + [_I32] + [_P] * 6 + [_P] * 6)
    lib.or_moe_layer_slots.restype = _I32
    lib.or_moe_layer_slots.argtypes = ([_I32, _I32, _I32, _I32, _I32, _F32, _F32, _I64, _P, _P, _P,
                                        _I32, _P] + [_P] * 5 + [_I32] + [_P] * 6 + [_P] * 5)
    lib.or_fp8_dequant_value.restype = _F32
    lib.or_fp8_dequant_value.argtypes = [ctypes.c_uint32, _F32]
    lib.or_fp8_dequant_matrix.restype = None
    lib.or_fp8_dequant_matrix.argtypes = [_P, _P, _I64, _I64, _P]
    lib.or_moe_layer_fp8.restype = _I32
    lib.or_moe_layer_fp8.argtypes = ([_I32, _I32, _I32, _I32, _I32, _F32, _F32, _I64, _P, _P, _P]
                                     + [_P] * 4 + [_I32] + [_P] * 5 + [_P] * 4)
    lib.or_e4m3_encode.restype = ctypes.c_uint32
    lib.or_e4m3_encode.argtypes = [_F32]
    lib.or_fp8_quantize.restype = None
    lib.or_fp8_quantize.argtypes = [_I64, _I64, _P, _P, _P]
    lib.or_fp8_linear.restype = None
    lib.or_fp8_linear.argtypes = [_I64, _I64, _I64, _P, _F32, _P, _P, _P, _P]
    lib.or_attn_extend.restype = _I32
    lib.or_attn_extend.argtypes = ([_I32] * 6 + [_P] * 3 + [_I32] + [_P] * 4 + [_F32, _F32]
                                   + [_P, _P])
    _libs[omp] = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous arrays"
    return a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def threads(openmp: bool = False) -> int:
    """Threads the oracle's row loops use (1 for the plain build)."""
    return int(_load(openmp).or_threads())


# ------------------------------------------------------------------ codecs --

def e2m1(code: int) -> float:
    return _load().or_e2m1(int(code))


def e4m3(byte: int) -> float:
    return _load().or_e4m3(int(byte))


def dequant_value(code: int, scale_byte: int, g: float) -> np.float32:
    return np.float32(_load().or_dequant_value(int(code), int(scale_byte), float(g)))


def dequant_matrix(codes: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    """codes u8 [rows, K/2], scales u8 [rows, K/16] -> fp32 [rows, K]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, half = codes.shape
    K = 2 * half
    assert scales.shape == (rows, K // 16)
    out = np.empty((rows, K), np.float32)
    _load().or_dequant_matrix(_ptr(codes), _ptr(scales), rows, K, float(g), _ptr(out))
    return out


def bf16_to_double(b: int) -> float:
    return _load().or_bf16_to_double(int(b))


def bf16_from_double(v: float) -> int:
    return int(_load().or_bf16_from_double(float(v)))


# ------------------------------------------------------------------ router --

def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """x bf16 bits u16 [T, H]; w_router fp32 [E, H]; bias fp32 [E] or None -> fp32 [T, E]."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = w_router.shape[0]
    out = np.empty((T, E), np.float32)
    _load().or_router_logits(T, E, H, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(out))
    return out


def topk(logits: np.ndarray, k: int):
    """fp32 [T, E] -> (ids int32 [T, k], weights fp32 [T, k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().or_topk(T, E, int(k), _ptr(logits), _ptr(ids), _ptr(w))
    return ids, w


def silu(z: float) -> float:
    return _load().or_silu(float(z))


def swiglu(act: int, g: float, u: float, gate_max: float = 7.0, up_absmax: float = 7.0) -> float:
    return _load().or_swiglu(int(act), float(g), float(u), float(gate_max), float(up_absmax))


# ------------------------------------------------------------------ layer --

def expert_output(layer, e: int, x_row: np.ndarray, shared: bool = False) -> np.ndarray:
    """One expert's binary64 output [H] for one bf16 token row."""
    x_row = _c(x_row, np.uint16)
    if shared:
        I = layer.shared_inter
        bank = (layer.s13_codes, layer.s13_scales, layer.s2_codes, layer.s2_scales,
                layer.s_global)
    else:
        I = layer.inter
        bank = (layer.w13_codes, layer.w13_scales, layer.w2_codes, layer.w2_scales,
                layer.global_scale)
    bank = [_c(a, np.uint8) for a in bank[:4]] + [_c(bank[4], np.float32)]
    out = np.empty(layer.hidden, np.float64)
    _load().or_expert_output(layer.hidden, I, int(e), *[_ptr(a) for a in bank], layer.act,
                             layer.gate_max, layer.up_absmax, _ptr(x_row), _ptr(out))
    return out


def moe_layer(layer, x: np.ndarray, ids=None, weights=None, openmp: bool = False) -> dict:
    """Run the whole layer for the tokens in ``x`` (bf16 bits u16 [T, H]).

    ``layer`` carries the weights (see ``nvfp4_mixture_experts_amd.synth.Layer``).
    With ``ids``/``weights`` given, those routes are used instead of the router.
    ``openmp`` runs the OpenMP build of the same source (for timing on all cores;
    same bits).  Returns ``{"ids", "weights", "y64", "y"}``.
    """
    x = _c(x, np.uint16)
    T = x.shape[0]
    k = layer.top_k
    ids_in = _c(ids, np.int32)
    w_in = _c(weights, np.float32)
    ids_out = np.empty((T, k), np.int32)
    w_out = np.empty((T, k), np.float32)
    y64 = np.empty((T, layer.hidden), np.float64)
    y = np.empty((T, layer.hidden), np.uint16)
    Is = layer.shared_inter
    sh = [None] * 6
    if Is > 0:
        sh = [_c(layer.s13_codes, np.uint8), _c(layer.s13_scales, np.uint8),
              _c(layer.s2_codes, np.uint8), _c(layer.s2_scales, np.uint8),
              _c(layer.s_global, np.float32), _c(layer.shared_gate, np.uint16)]
    bank = [_c(layer.w13_codes, np.uint8), _c(layer.w13_scales, np.uint8),
            _c(layer.w2_codes, np.uint8), _c(layer.w2_scales, np.uint8),
            _c(layer.global_scale, np.float32)]
    wr = _c(layer.w_router, np.float32)
    bias = _c(layer.bias, np.float32)
    rc = _load(openmp).or_moe_layer(layer.num_experts, layer.hidden, layer.inter, k, layer.act,
                              layer.gate_max, layer.up_absmax, T, _ptr(x), _ptr(wr), _ptr(bias),
                              *[_ptr(a) for a in bank], Is, *[_ptr(a) for a in sh],
                              _ptr(ids_in), _ptr(w_in), _ptr(ids_out), _ptr(w_out), _ptr(y64),
                              _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected the layer shape")
    return {"ids": ids_out, "weights": w_out, "y64": y64, "y": y}


def moe_layer_slots(layer, x: np.ndarray, slot_of: np.ndarray, slot_bank: dict,
                    openmp: bool = False) -> dict:
    """The layer with its routed experts in a bank of expert slots: ``slot_bank`` holds
    canonical arrays of n_slots experts (w13_codes, w13_scales, w2_codes, w2_scales,
    global_scale); ``slot_of`` int32 [E] names the slot of each expert, or a value
    outside [0, n_slots) when it is not resident.  Routing uses ``layer``'s router.
    Returns ``{"ids", "weights", "miss", "y64", "y"}``; ``miss[t, i]`` is the id of a
    selected expert that is not resident, else -1."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    k = layer.top_k
    slot_of = _c(slot_of, np.int32)
    assert slot_of.shape == (layer.num_experts,)
    bank = [_c(slot_bank["w13_codes"], np.uint8), _c(slot_bank["w13_scales"], np.uint8),
            _c(slot_bank["w2_codes"], np.uint8), _c(slot_bank["w2_scales"], np.uint8),
            _c(slot_bank["global_scale"], np.float32)]
    n_slots = bank[0].shape[0]
    Is = layer.shared_inter
    sh = [None] * 6
    if Is > 0:
        sh = [_c(layer.s13_codes, np.uint8), _c(layer.s13_scales, np.uint8),
              _c(layer.s2_codes, np.uint8), _c(layer.s2_scales, np.uint8),
              _c(layer.s_global, np.float32), _c(layer.shared_gate, np.uint16)]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    miss = np.empty((T, k), np.int32)
    y64 = np.empty((T, layer.hidden), np.float64)
    y = np.empty((T, layer.hidden), np.uint16)
    rc = _load(openmp).or_moe_layer_slots(
        layer.num_experts, layer.hidden, layer.inter, k, layer.act, layer.gate_max,
        layer.up_absmax, T, _ptr(x), _ptr(_c(layer.w_router, np.float32)),
        _ptr(_c(layer.bias, np.float32)), n_slots, _ptr(slot_of), *[_ptr(a) for a in bank], Is,
        *[_ptr(a) for a in sh], _ptr(ids), _ptr(w), _ptr(miss), _ptr(y64), _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected the layer shape")
    return {"ids": ids, "weights": w, "miss": miss, "y64": y64, "y": y}


# --------------------------------------------------------- block-fp8 codec --

FP8_BLOCK = 128


def fp8_dequant_value(byte: int, scale: float) -> np.float32:
    return np.float32(_load().or_fp8_dequant_value(int(byte), float(scale)))


def fp8_dequant_matrix(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes u8 [rows, K], scales f32 [ceil(rows/128), ceil(K/128)] -> fp32 [rows, K]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    rows, K = codes.shape
    assert scales.shape == (-(-rows // FP8_BLOCK), -(-K // FP8_BLOCK))
    out = np.empty((rows, K), np.float32)
    _load().or_fp8_dequant_matrix(_ptr(codes), _ptr(scales), rows, K, _ptr(out))
    return out


def moe_layer_fp8(layer, x: np.ndarray, openmp: bool = False) -> dict:
    """The layer with block-fp8 experts: ``layer`` is a ``synth.Fp8Layer`` (routed bank
    w13_codes u8 [E, 2I, H], w13_scales f32 [E, 2I/128, H/128], w2_codes u8 [E, H, I],
    w2_scales f32 [E, H/128, I/128], and the shared expert likewise with n = 1).
    Returns ``{"ids", "weights", "y64", "y"}``."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    k = layer.top_k
    bank = [_c(layer.w13_codes, np.uint8), _c(layer.w13_scales, np.float32),
            _c(layer.w2_codes, np.uint8), _c(layer.w2_scales, np.float32)]
    Is = layer.shared_inter
    sh = [None] * 5
    if Is > 0:
        sh = [_c(layer.s13_codes, np.uint8), _c(layer.s13_scales, np.float32),
              _c(layer.s2_codes, np.uint8), _c(layer.s2_scales, np.float32),
              _c(layer.shared_gate, np.uint16)]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    y64 = np.empty((T, layer.hidden), np.float64)
    y = np.empty((T, layer.hidden), np.uint16)
    rc = _load(openmp).or_moe_layer_fp8(
        layer.num_experts, layer.hidden, layer.inter, k, layer.act, layer.gate_max,
        layer.up_absmax, T, _ptr(x), _ptr(_c(layer.w_router, np.float32)),
        _ptr(_c(layer.bias, np.float32)), *[_ptr(a) for a in bank], Is, *[_ptr(a) for a in sh],
        _ptr(ids), _ptr(w), _ptr(y64), _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected the layer shape")
    return {"ids": ids, "weights": w, "y64": y64, "y": y}


# ---------------------------------------------- fp8 per-tensor W8A8 linear --

def e4m3_encode(v: float) -> int:
    return int(_load().or_e4m3_encode(float(v)))


def fp8_quantize(x: np.ndarray, openmp: bool = False):
    """bf16 bits u16 [M, K] -> (e4m3 codes u8 [M, K], fp32 per-tensor scale)."""
    x = _c(x, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K), np.uint8)
    scale = np.empty(1, np.float32)
    _load(openmp).or_fp8_quantize(M, K, _ptr(x), _ptr(codes), _ptr(scale))
    return codes, np.float32(scale[0])


def fp8_linear(xq: np.ndarray, s_x: float, w: np.ndarray, w_scale_rows: np.ndarray,
               openmp: bool = False) -> dict:
    """y = bf16(s_x * s_w[n] * sum_k e4m3(xq[m,k]) e4m3(w[n,k])): returns {"y64", "y"}."""
    xq = _c(xq, np.uint8)
    w = _c(w, np.uint8)
    ws = _c(w_scale_rows, np.float32)
    M, K = xq.shape
    N = w.shape[0]
    assert w.shape == (N, K) and ws.shape == (N,)
    y64 = np.empty((M, N), np.float64)
    y = np.empty((M, N), np.uint16)
    _load(openmp).or_fp8_linear(M, N, K, _ptr(xq), float(s_x), _ptr(w), _ptr(ws), _ptr(y64),
                                _ptr(y))
    return {"y64": y64, "y": y}


# ---------------------------------------------------- extend attention, cache --

def attn_extend(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, cache: dict,
                window: int = 0, openmp: bool = False) -> dict:
    """Extend attention of n_new query tokens over a cached prefix and the new tokens.
    q bf16 bits u16 [n_new, Hq, d]; k_new, v_new u16 [n_new, Hkv, d]; ``cache`` =
    {"format": 0|1|2, "prefix": P, "k", "v" (codes), "k_bscale", "v_bscale" (NVFP4),
    "k_scale", "v_scale"} (see the C source for the layouts).  Returns {"out64", "out"}
    of shape [n_new, Hq, d]."""
    q = _c(q, np.uint16)
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    n_new, Hq, d = q.shape
    Hkv = k_new.shape[1]
    fmt = int(cache["format"])
    dt = np.uint16 if fmt == 0 else np.uint8
    kc = _c(cache["k"], dt)
    vc = _c(cache["v"], dt)
    kb = _c(cache.get("k_bscale"), np.uint8)
    vb = _c(cache.get("v_bscale"), np.uint8)
    out64 = np.empty((n_new, Hq, d), np.float64)
    out = np.empty((n_new, Hq, d), np.uint16)
    rc = _load(openmp).or_attn_extend(n_new, int(cache["prefix"]), Hq, Hkv, d, int(window),
                                      _ptr(q), _ptr(k_new), _ptr(v_new), fmt, _ptr(kc), _ptr(vc),
                                      _ptr(kb), _ptr(vb), float(cache.get("k_scale", 1.0)),
                                      float(cache.get("v_scale", 1.0)), _ptr(out64), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the attention shape")
    return {"out64": out64, "out": out}
