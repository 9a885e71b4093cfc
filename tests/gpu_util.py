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


def decode_checked(device, dl, x, workspace=None, stream=None):
    """device.decode plus a check that every device-side wait of the call completed."""
    import torch
    st = torch.full((1,), -1, dtype=torch.int32, device=x.device)
    out = device.decode(dl, x, workspace, stream, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, f"device-side wait gave up (status {int(st.item()):#x})"
    return out


def _threads():
    import os
    return max(1, min(16, os.cpu_count() or 1))


def oracle_layer_rows(layer, x, rows):
    """oracle.moe_layer on the token rows ``rows`` of ``x``, with the rows split over a
    thread pool (ctypes releases the GIL; tokens are independent in the oracle)."""
    import concurrent.futures
    import oracle
    rows = list(rows)
    n = _threads()
    chunks = [rows[i::n] for i in range(n) if rows[i::n]]
    with concurrent.futures.ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(lambda c: oracle.moe_layer(layer, x[c]), chunks))
    out = {}
    for key in ("ids", "weights", "y64", "y"):
        full = np.empty((len(rows),) + parts[0][key].shape[1:], parts[0][key].dtype)
        for i, part in enumerate(parts):
            full[i::len(chunks)] = part[key]
        out[key] = full
    return out


def oracle_routes(x, w_router, bias, k):
    """oracle.topk(oracle.router_logits(...)) for every token, over a thread pool."""
    import concurrent.futures
    import oracle
    T = x.shape[0]
    n = min(_threads(), T)
    bounds = np.linspace(0, T, n + 1).astype(int)
    def run(i):
        lo, hi = bounds[i], bounds[i + 1]
        return oracle.topk(oracle.router_logits(x[lo:hi], w_router, bias), k)
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(run, range(n)))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


def cover_rows(ids, num_experts, must=()):
    """Token rows, starting with ``must``, chosen greedily until every expert id in
    [0, num_experts) appears in some chosen row's routes."""
    rows = list(dict.fromkeys(int(r) for r in must))
    covered = np.zeros(num_experts, bool)
    for r in rows:
        covered[ids[r]] = True
    gain = np.zeros(ids.shape[0], np.int64)
    while not covered.all():
        gain[:] = (~covered[ids]).sum(axis=1)
        gain[rows] = -1
        r = int(np.argmax(gain))
        if gain[r] <= 0:
            break
        rows.append(r)
        covered[ids[r]] = True
    return rows
