"""Seeded synthetic inputs for the NVFP4 mixture-of-experts layer.

This module only draws random inputs of the right shapes, dtypes and
distributions; it holds none of the layer's arithmetic.  Both the HIP path and
the CPU oracle are fed from it (it is the only code they share).

Distributions (per workload):
  * activations x: bf16 draws of N(0, 1) (fp32 draw, converted by torch);
  * router weight: fp32 N(0, 0.02) (0.02 is the standard deviation), [E, H];
  * router bias: absent, or +hot_bias on ``hot_experts`` experts picked at random;
  * expert codes: uniform random bytes (two uniform 4-bit e2m1 codes per byte);
  * block scales: one e4m3 byte per 16 K-elements, uniform over the encodings
    of 2^-4 .. 2^2 (exponent field n + 7, mantissa 0);
  * per-tensor global scales (gate, up, down) all equal to ``global_scale``;
  * shared-expert gate vector: bf16 draws of N(0, 0.02);
  * block-fp8 workloads (codec "fp8"): e4m3 code bytes uniform over the 254 finite
    encodings, one fp32 scale per 128 x 128 block drawn as 2^-11 * (1 + U[0, 1)).

Canonical weight layout (what ``ft_nvfp4_repack`` takes):
  w13 codes [n, 2I, H/2] (gate rows 0..I-1, then up rows), w13 scales [n, 2I, H/16],
  w2 codes [n, H, I/2], w2 scales [n, H, I/16], global scales fp32 [n, 3];
  byte k/2 of a row holds element k in its low nibble when k is even.

Layer instance ``l`` of a workload uses seed ``workload.seed + 7919 * l``.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional

import numpy as np

# e4m3 encodings of 2^-4, 2^-3, ..., 2^2: sign 0, exponent field n + 7, mantissa 0.
SCALE_BYTES = np.array([(n + 7) << 3 for n in range(-4, 3)], dtype=np.uint8)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_experts: int
    hidden: int
    inter: int
    top_k: int
    tokens: int
    clamped: bool
    global_scale: float
    seed: int
    shared_inter: int = 0
    hot_experts: int = 0
    hot_bias: float = 0.0
    gate_max: float = 7.0
    up_absmax: float = 7.0
    router_std: float = 0.02
    shared_gate_std: float = 0.02
    codec: str = "nvfp4"          # routed/shared expert weights: "nvfp4" or "fp8" (block-fp8)

    @property
    def act(self) -> int:
        return 1 if self.clamped else 0


WORKLOADS = {
    w.name: w
    for w in [
        # Tiny layer: 8 experts, H=256, I=128, top-2, plain SwiGLU, global scale 1.
        Workload("tiny_e8_top2", 8, 256, 128, 2, 1, False, 1.0, seed=1000),
        # Batch-1 decode over the 288-expert layer: H=2048, I=768, top-8, clamped.
        Workload("decode_e288_top8", 288, 2048, 768, 8, 1, True, 2.0 ** -6, seed=1001),
        # Batch-1 decode over the 512-expert layer with a gated shared expert.
        Workload("decode_e512_top10_shared", 512, 2048, 512, 10, 1, True, 2.0 ** -6,
                 seed=1002, shared_inter=512),
        # 32 concurrent decode tokens; 64 seeded hot experts get +2.0 on their logit.
        Workload("batched_decode_t32_hot64", 512, 2048, 512, 10, 32, True, 2.0 ** -6,
                 seed=1003, shared_inter=512, hot_experts=64, hot_bias=2.0),
        # Prefill chunk of 8192 tokens through the 512-expert layer.
        Workload("prefill_t8192", 512, 2048, 512, 10, 8192, True, 2.0 ** -6, seed=1004,
                 shared_inter=512),
        # The 512-expert decode layer with block-fp8 routed and shared experts.
        Workload("decode_e512_top10_shared_fp8", 512, 2048, 512, 10, 1, True, 1.0, seed=1005,
                 shared_inter=512, codec="fp8"),
    ]
}


# ------------------------------------------------------ fp8 W8A8 projections --

@dataclasses.dataclass(frozen=True)
class LinearWorkload:
    """A fused per-tensor-FP8 projection: parts of `parts` output rows each (q, k, v)
    stacked along N, input width `hidden`, `tokens` rows of activations."""
    name: str
    hidden: int
    parts: tuple
    tokens: int
    seed: int

    @property
    def out_rows(self) -> int:
        return int(sum(self.parts))


@dataclasses.dataclass
class Fp8Linear:
    workload: LinearWorkload
    w: np.ndarray              # u8 [N, K] e4m3 codes (parts stacked)
    part_scales: np.ndarray    # f32 [n_parts] per-part (per-tensor) weight scales

    def part_ranges(self):
        edges = np.concatenate([[0], np.cumsum(self.workload.parts)])
        return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:])]

    def row_scales(self) -> np.ndarray:
        """The per-row scale vector (each row carries its part's scale)."""
        return np.repeat(self.part_scales, self.workload.parts).astype(np.float32)


def make_fp8_linear(w: LinearWorkload) -> Fp8Linear:
    """Uniform e4m3 weight codes over the finite encodings; per-part scales drawn as
    2^-9 * (1 + U[0, 1)) (distinct parts, so a wrong part boundary changes rows)."""
    rng = _rng(w.seed, "fp8_linear_w")
    codes = _fp8_codes(rng, (w.out_rows, w.hidden))
    scales = (np.float32(2.0 ** -9) * (1 + _rng(w.seed, "fp8_linear_s").random(
        len(w.parts), dtype=np.float32))).astype(np.float32)
    return Fp8Linear(w, codes, scales)


LINEAR_WORKLOADS = {
    lw.name: lw
    for lw in [
        # q (32 heads x 128) | k (4 x 128) | v (4 x 128) over hidden 2048
        LinearWorkload("fp8_linear_qkv_t1", 2048, (4096, 512, 512), 1, seed=2001),
        LinearWorkload("fp8_linear_qkv_t32", 2048, (4096, 512, 512), 32, seed=2002),
        LinearWorkload("fp8_linear_qkv_t8192", 2048, (4096, 512, 512), 8192, seed=2003),
    ]
}
WORKLOADS.update(LINEAR_WORKLOADS)

# ---------------------------------------------------------------- block-fp8 --

FP8_BLOCK = 128
# every e4m3 byte but the two NaN encodings (S.1111.111)
FP8_FINITE_BYTES = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)


@dataclasses.dataclass
class Fp8Layer:
    """One layer with block-fp8 experts (canonical layout): codes are e4m3 bytes, one
    fp32 scale per 128 x 128 block (bank [n][ceil(rows/128)][ceil(K/128)])."""
    workload: Workload
    w_router: np.ndarray
    bias: Optional[np.ndarray]
    w13_codes: np.ndarray    # u8 [E, 2I, H]
    w13_scales: np.ndarray   # f32 [E, 2I/128, H/128]
    w2_codes: np.ndarray     # u8 [E, H, I]
    w2_scales: np.ndarray    # f32 [E, H/128, I/128]
    s13_codes: Optional[np.ndarray] = None
    s13_scales: Optional[np.ndarray] = None
    s2_codes: Optional[np.ndarray] = None
    s2_scales: Optional[np.ndarray] = None
    shared_gate: Optional[np.ndarray] = None

    num_experts = property(lambda s: s.workload.num_experts)
    hidden = property(lambda s: s.workload.hidden)
    inter = property(lambda s: s.workload.inter)
    top_k = property(lambda s: s.workload.top_k)
    act = property(lambda s: s.workload.act)
    gate_max = property(lambda s: s.workload.gate_max)
    up_absmax = property(lambda s: s.workload.up_absmax)
    shared_inter = property(lambda s: s.workload.shared_inter)


def _blocks(n: int) -> int:
    return -(-n // FP8_BLOCK)


def _fp8_codes(rng, shape):
    return FP8_FINITE_BYTES[rng.integers(0, len(FP8_FINITE_BYTES), size=shape)]


def _fp8_scales(rng, shape):
    # 2^-11 * (1 + u), u ~ U[0, 1): pre-activations of a few units at H = 2048
    return (np.float32(2.0 ** -11) * (1 + rng.random(shape, dtype=np.float32))).astype(np.float32)


def _fp8_bank(seed: int, prefix: str, n: int, H: int, I: int):
    return dict(
        w13_codes=_fp8_codes(_rng(seed, prefix + "w13_codes"), (n, 2 * I, H)),
        w13_scales=_fp8_scales(_rng(seed, prefix + "w13_scales"), (n, _blocks(2 * I), _blocks(H))),
        w2_codes=_fp8_codes(_rng(seed, prefix + "w2_codes"), (n, H, I)),
        w2_scales=_fp8_scales(_rng(seed, prefix + "w2_scales"), (n, _blocks(H), _blocks(I))),
    )


def make_fp8_layer(w: Workload, instance: int = 0) -> Fp8Layer:
    """Host (numpy) block-fp8 weights of layer instance ``instance``."""
    seed = w.seed + 7919 * instance
    wr, bias = make_router(w, instance)
    layer = Fp8Layer(workload=w, w_router=wr, bias=bias,
                     **_fp8_bank(seed, "fp8_", w.num_experts, w.hidden, w.inter))
    if w.shared_inter > 0:
        sb = _fp8_bank(seed, "fp8_shared_", 1, w.hidden, w.shared_inter)
        layer.s13_codes, layer.s13_scales = sb["w13_codes"], sb["w13_scales"]
        layer.s2_codes, layer.s2_scales = sb["w2_codes"], sb["w2_scales"]
        gs = _rng(seed, "shared_gate").standard_normal(w.hidden, dtype=np.float32)
        layer.shared_gate = bf16_bits_from_f32(gs * np.float32(w.shared_gate_std))
    return layer


@dataclasses.dataclass
class Layer:
    """One layer's weights (numpy, canonical layout) plus its workload shape."""
    workload: Workload
    w_router: np.ndarray
    bias: Optional[np.ndarray]
    w13_codes: np.ndarray
    w13_scales: np.ndarray
    w2_codes: np.ndarray
    w2_scales: np.ndarray
    global_scale: np.ndarray
    s13_codes: Optional[np.ndarray] = None
    s13_scales: Optional[np.ndarray] = None
    s2_codes: Optional[np.ndarray] = None
    s2_scales: Optional[np.ndarray] = None
    s_global: Optional[np.ndarray] = None
    shared_gate: Optional[np.ndarray] = None

    # shape accessors used by the oracle wrapper and the binding
    num_experts = property(lambda s: s.workload.num_experts)
    hidden = property(lambda s: s.workload.hidden)
    inter = property(lambda s: s.workload.inter)
    top_k = property(lambda s: s.workload.top_k)
    act = property(lambda s: s.workload.act)
    gate_max = property(lambda s: s.workload.gate_max)
    up_absmax = property(lambda s: s.workload.up_absmax)
    shared_inter = property(lambda s: s.workload.shared_inter)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([seed, zlib.crc32(name.encode())])


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 draws to bf16 (torch's conversion, nearest-even) and return the bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _codes(rng, shape):
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def _scales(rng, shape):
    return SCALE_BYTES[rng.integers(0, len(SCALE_BYTES), size=shape)]


def _bank(seed: int, prefix: str, n: int, H: int, I: int, g: float):
    return dict(
        w13_codes=_codes(_rng(seed, prefix + "w13_codes"), (n, 2 * I, H // 2)),
        w13_scales=_scales(_rng(seed, prefix + "w13_scales"), (n, 2 * I, H // 16)),
        w2_codes=_codes(_rng(seed, prefix + "w2_codes"), (n, H, I // 2)),
        w2_scales=_scales(_rng(seed, prefix + "w2_scales"), (n, H, I // 16)),
        global_scale=np.full((n, 3), g, dtype=np.float32),
    )


def make_router(w: Workload, instance: int = 0, num_experts: Optional[int] = None):
    """Router weights [E, H] and bias [E] (or None) of layer instance ``instance``:
    the same values ``make_layer`` gives, without the expert banks."""
    seed = w.seed + 7919 * instance
    E = w.num_experts if num_experts is None else num_experts
    wr = (_rng(seed, "w_router").standard_normal((E, w.hidden), dtype=np.float32)
          * np.float32(w.router_std)).astype(np.float32)
    bias = None
    if w.hot_experts > 0:
        bias = np.zeros(E, np.float32)
        hot = _rng(seed, "hot").choice(E, size=min(w.hot_experts, E), replace=False)
        bias[hot] = np.float32(w.hot_bias)
    return wr, bias


def make_layer(w: Workload, instance: int = 0, num_experts: Optional[int] = None) -> Layer:
    """Host (numpy) weights of layer instance ``instance``.

    ``num_experts`` overrides the routed bank size (tests use it to build small
    variants of a workload); by default the workload's own count is used.
    """
    seed = w.seed + 7919 * instance
    E = w.num_experts if num_experts is None else num_experts
    if num_experts is not None:
        w = dataclasses.replace(w, num_experts=E)
    H, I = w.hidden, w.inter
    wr, bias = make_router(w, instance)
    bank = _bank(seed, "", E, H, I, w.global_scale)
    layer = Layer(workload=w, w_router=wr, bias=bias, **bank)
    if w.shared_inter > 0:
        sb = _bank(seed, "shared_", 1, H, w.shared_inter, w.global_scale)
        layer.s13_codes = sb["w13_codes"]
        layer.s13_scales = sb["w13_scales"]
        layer.s2_codes = sb["w2_codes"]
        layer.s2_scales = sb["w2_scales"]
        layer.s_global = sb["global_scale"]
        gs = _rng(seed, "shared_gate").standard_normal(H, dtype=np.float32)
        layer.shared_gate = bf16_bits_from_f32(gs * np.float32(w.shared_gate_std))
    return layer


def make_tokens(w: Workload, instance: int = 0, tokens: Optional[int] = None,
                stream: str = "x") -> np.ndarray:
    """bf16 bits u16 [T, H] of N(0, 1) draws."""
    T = w.tokens if tokens is None else tokens
    seed = w.seed + 7919 * instance
    a = _rng(seed, stream).standard_normal((T, w.hidden), dtype=np.float32)
    return bf16_bits_from_f32(a)


def make_layer_device(w: Workload, instance: int, device):
    """Draw one layer instance directly in device memory with torch's generator.

    Same shapes and distributions as ``make_layer`` (different draws); used to
    fill many distinct layer instances for timing without host round trips.
    Returns a dict of torch tensors in the canonical layout.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 7919 * instance)
    E, H, I = w.num_experts, w.hidden, w.inter
    table = torch.tensor(SCALE_BYTES, dtype=torch.uint8, device=device)

    def codes(shape):
        return torch.randint(0, 256, shape, generator=gen, device=device, dtype=torch.uint8)

    def scales(shape):
        idx = torch.randint(0, len(SCALE_BYTES), shape, generator=gen, device=device)
        return table[idx]

    def bank(n, inter):
        return dict(w13_codes=codes((n, 2 * inter, H // 2)),
                    w13_scales=scales((n, 2 * inter, H // 16)),
                    w2_codes=codes((n, H, inter // 2)),
                    w2_scales=scales((n, H, inter // 16)),
                    global_scale=torch.full((n, 3), w.global_scale, dtype=torch.float32,
                                            device=device))

    out = dict(w_router=torch.randn((E, H), generator=gen, device=device) * w.router_std,
               bias=None, routed=bank(E, I), shared=None, shared_gate=None)
    if w.hot_experts > 0:
        bias = torch.zeros(E, dtype=torch.float32, device=device)
        hot = torch.randperm(E, generator=gen, device=device)[: w.hot_experts]
        bias[hot] = w.hot_bias
        out["bias"] = bias
    if w.shared_inter > 0:
        out["shared"] = bank(1, w.shared_inter)
        out["shared_gate"] = (torch.randn(H, generator=gen, device=device)
                              * w.shared_gate_std).to(torch.bfloat16)
    return out


# ------------------------------------------------- extend attention cases --

# e4m3 bytes of magnitude at most 15 (exponent field <= 10), both signs, no NaN
FP8_CACHE_BYTES = np.array([b for b in range(256) if ((b >> 3) & 15) <= 10], dtype=np.uint8)


def make_attn_case(fmt: int, head_dim: int, prefix: int, n_new: int = 24, q_heads: int = 8,
                   kv_heads: int = 2, seed: int = 3000) -> dict:
    """One sequence for extend attention: q, k_new, v_new (bf16 bits, N(0, 1)) and a
    cached prefix in format ``fmt`` (0 bf16 N(0, 1); 1 e4m3 bytes uniform over the
    magnitudes <= 15 with tensor scales 1/8; 2 NVFP4: uniform codes, e4m3 block
    scales 2^U{-4..0}, tensor scales 1/4)."""
    rng = _rng(seed + 97 * fmt + 7 * head_dim + prefix, "attn")
    d, Hq, Hkv = head_dim, q_heads, kv_heads

    def bf16(shape):
        return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))

    case = {"q": bf16((n_new, Hq, d)), "k_new": bf16((n_new, Hkv, d)),
            "v_new": bf16((n_new, Hkv, d)), "cache": {"format": fmt, "prefix": prefix}}
    c = case["cache"]
    if fmt == 0:
        c["k"], c["v"] = bf16((prefix, Hkv, d)), bf16((prefix, Hkv, d))
    elif fmt == 1:
        pick = lambda: FP8_CACHE_BYTES[rng.integers(0, len(FP8_CACHE_BYTES), (prefix, Hkv, d))]
        c["k"], c["v"] = pick(), pick()
        c["k_scale"], c["v_scale"] = 0.125, 0.125
    else:
        codes = lambda: _codes(rng, (prefix, Hkv, d // 2))
        bscale = lambda: SCALE_BYTES[rng.integers(0, 5, (prefix, Hkv, d // 16))]
        c["k"], c["v"] = codes(), codes()
        c["k_bscale"], c["v_bscale"] = bscale(), bscale()
        c["k_scale"], c["v_scale"] = 0.25, 0.25
    return case



def make_fp8_layer_device(w: Workload, instance: int, device):
    """A block-fp8 layer instance drawn on the device (torch's generator; the same
    distributions as make_fp8_layer, different draws): canonical tensors."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 7919 * instance)
    E, H, I = w.num_experts, w.hidden, w.inter
    table = torch.tensor(FP8_FINITE_BYTES, dtype=torch.uint8, device=device)

    def codes(shape):
        return table[torch.randint(0, len(FP8_FINITE_BYTES), shape, generator=gen, device=device)]

    def scales(shape):
        return (2.0 ** -11) * (1 + torch.rand(shape, generator=gen, device=device))

    def bank(n, inter):
        return dict(w13_codes=codes((n, 2 * inter, H)),
                    w13_scales=scales((n, _blocks(2 * inter), _blocks(H))),
                    w2_codes=codes((n, H, inter)), w2_scales=scales((n, _blocks(H), _blocks(inter))))

    out = dict(w_router=torch.randn((E, H), generator=gen, device=device) * w.router_std,
               bias=None, routed=bank(E, I), shared=None, shared_gate=None)
    if w.shared_inter > 0:
        out["shared"] = bank(1, w.shared_inter)
        out["shared_gate"] = (torch.randn(H, generator=gen, device=device)
                              * w.shared_gate_std).to(torch.bfloat16)
    return out
