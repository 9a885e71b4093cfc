"""Shared helpers of the GPU parity tests (imported only by GPU tests)."""
import functools
import sys

import numpy as np

from nvfp4_mixture_experts_amd import synth

# Output tolerance for bf16 results against the oracle's bf16-rounded output
# (fp32 accumulation in a different order, then one bf16 rounding on each side).
MAX_ABS_REL = 1e-2
REL_L2 = 2e-3


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def output_errors(y_bits, ref_bits):
    y = bf16_to_f64(y_bits)
    r = bf16_to_f64(ref_bits)
    err = y - r
    mar = np.abs(err).max() / np.abs(r).max()
    l2 = np.linalg.norm(err) / np.linalg.norm(r)
    return float(mar), float(l2)


def assert_output_close(y_bits, ref_bits, what=""):
    assert np.all(np.isfinite(bf16_to_f64(y_bits))), f"{what}: non-finite output"
    mar, l2 = output_errors(y_bits, ref_bits)
    say(f"  {what}: max_abs_rel={mar:.3e} rel_l2={l2:.3e}")
    assert mar <= MAX_ABS_REL, (what, mar)
    assert l2 <= REL_L2, (what, l2)


def f32_ulp_diff(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


@functools.lru_cache(maxsize=4)
def host_layer(name: str, **overrides):
    w = synth.WORKLOADS[name]
    if overrides:
        w = synth.dataclasses.replace(w, **overrides)
    return synth.make_layer(w)
