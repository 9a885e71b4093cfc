"""GPU parity of the per-tensor FP8 W8A8 projection (ft_fp8_quantize,
ft_fp8_linear, ft_fp8_linear_parts, ft_fp8_scale_runs) against the CPU oracle,
through the C ABI.  Activation codes and scale bit-exact (both sides divide in fp32
and round to the nearest e4m3, ties to even); bf16 outputs within max_abs_rel 1e-2
and rel_l2 2e-3; the per-part form equal to the row-wise form bit for bit."""
import concurrent.futures

import numpy as np
import pytest
import torch

import oracle
from nvfp4_mixture_experts_amd import synth
from tests.gpu_util import assert_output_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ft():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_mixture_experts_amd import ftmoe
    ftmoe.ft_init(0)
    return ftmoe


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _oracle_rows(xq, s_x, w, rows_scale, rows):
    n = 16
    chunks = [rows[i::n] for i in range(n) if rows[i::n]]
    with concurrent.futures.ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(lambda c: oracle.fp8_linear(xq[c], s_x, w, rows_scale)["y"], chunks))
    out = np.empty((len(rows), w.shape[0]), np.uint16)
    for i, p in enumerate(parts):
        out[i::len(chunks)] = p
    return out


def test_fp8_quantize_codes_bit_exact_with_ties(ft):
    # amax 448 gives s_x = 1 exactly, so the other elements are divided by 1 and every
    # midpoint between neighbouring e4m3 magnitudes is an exact tie
    mags = np.array(sorted({abs(oracle.e4m3(b)) for b in range(0x7F)}))
    mids = ((mags[:-1] + mags[1:]) / 2)
    K = 512
    vals = np.concatenate([[448.0], mids, -mids])
    x = np.zeros((2, K), np.float32)
    x.flat[: len(vals)] = vals
    x[1] = np.random.default_rng(4).standard_normal(K) * 30
    xb = synth.bf16_bits_from_f32(x)
    assert np.array_equal((xb.astype(np.uint32) << 16).view(np.float32).ravel()[: len(vals)],
                          vals.astype(np.float32))                   # exact in bf16
    want_q, want_s = oracle.fp8_quantize(xb)
    assert want_s == 1.0
    ws = ft.fp8_linear_workspace(2, K)
    q = torch.empty((2, K), dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    ft.ft_fp8_quantize(_dev_bf16(xb), q, s, ws)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), want_q)
    assert s.item() == want_s


def test_fp8_quantize_many_rows_bit_exact_with_ties(ft):
    # 77 x 1024 values: the e4m3 midpoints (exact ties at s_x = 1) spread over the rows,
    # the amax 448 as the very last element, the rest normal * 30
    mags = np.array(sorted({abs(oracle.e4m3(b)) for b in range(0x7F)}))
    mids = ((mags[:-1] + mags[1:]) / 2)
    M, K = 77, 1024
    x = np.random.default_rng(11).standard_normal((M, K)).astype(np.float32) * 30
    vals = np.concatenate([mids, -mids])
    for j, r in enumerate((0, 38, 76)):
        x[r, 100 * j: 100 * j + len(vals)] = vals
    x[-1, -1] = -448.0
    xb = synth.bf16_bits_from_f32(x)
    want_q, want_s = oracle.fp8_quantize(xb)
    assert want_s == 1.0
    ws = ft.fp8_linear_workspace(M, K)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    # the kernels read x in 16-byte pieces: an x one element off is refused
    buf = torch.zeros(M * K + 8, dtype=torch.bfloat16, device="cuda")
    buf[1: 1 + M * K] = _dev_bf16(xb.ravel())
    with pytest.raises(ft.FtError, match="aligned"):
        ft.ft_fp8_quantize(buf[1: 1 + M * K].view(M, K), q, s, ws)
    ft.ft_fp8_quantize(_dev_bf16(xb), q, s, ws)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), want_q)
    assert s.item() == want_s


@pytest.mark.parametrize("tokens", [1, 2, 8, 32, 77, 128, 300])   # GEMV (<= 8 rows), 64- and 128-row MFMA GEMMs
def test_fp8_linear_matches_oracle_and_parts_equal_rowwise(ft, tokens):
    w = synth.WORKLOADS["fp8_linear_qkv_t32"]
    lin = synth.make_fp8_linear(w)
    x = synth.make_tokens(w, tokens=tokens, stream=f"lin{tokens}")
    xq, s_x = oracle.fp8_quantize(x)
    rows = lin.row_scales()
    want = _oracle_rows(xq, s_x, lin.w, rows, list(range(tokens)))
    xd = _dev_bf16(x)
    wd = torch.from_numpy(lin.w).cuda()
    ws = ft.fp8_linear_workspace(tokens, w.hidden)
    y = torch.empty((tokens, w.out_rows), dtype=torch.bfloat16, device="cuda")
    ft.ft_fp8_linear(xd, wd, torch.from_numpy(rows).cuda(), y, ws)
    part_rows, part_scales = ft.ft_fp8_scale_runs(rows)
    assert part_rows.tolist() == [0, 4096, 4608, 5120]
    assert np.array_equal(part_scales, lin.part_scales)
    yp = torch.full_like(y, float("nan"))
    ft.ft_fp8_linear_parts(xd, wd, part_rows, part_scales, yp, ws)
    q = torch.empty((tokens, w.hidden), dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    ft.ft_fp8_quantize(xd, q, s, ws)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), xq) and s.item() == s_x
    assert_output_close(_bits(y), want, f"fp8 linear q|k|v T={tokens}")
    assert np.array_equal(_bits(yp), _bits(y))


@pytest.mark.parametrize("tokens,hidden", [(19, 1024), (5, 1024), (3, 1088), (130, 1088),
                                          (2, 4096), (8, 3072)])   # few rows past the one-launch form
def test_fp8_linear_ragged_parts_and_rows(ft, tokens, hidden):
    # parts whose row counts are not multiples of the 64- or 128-row tiles (nor of the
    # GEMV's 16 rows per block); K = 1088: 68 16-byte chunks, so most GEMV lanes hold
    # one, and the 128-row GEMM's last 128-byte K slab is half past K
    w = synth.dataclasses.replace(synth.WORKLOADS["fp8_linear_qkv_t32"], hidden=hidden,
                                  parts=(100, 37, 200), tokens=tokens)
    lin = synth.make_fp8_linear(w)
    x = synth.make_tokens(w, stream="ragged")
    xq, s_x = oracle.fp8_quantize(x)
    rows = lin.row_scales()
    want = _oracle_rows(xq, s_x, lin.w, rows, list(range(w.tokens)))
    xd, wd = _dev_bf16(x), torch.from_numpy(lin.w).cuda()
    ws = ft.fp8_linear_workspace(w.tokens, w.hidden)
    y = torch.empty((w.tokens, w.out_rows), dtype=torch.bfloat16, device="cuda")
    ft.ft_fp8_linear(xd, wd, torch.from_numpy(rows).cuda(), y, ws)
    pr, ps = ft.ft_fp8_scale_runs(rows)
    yp = torch.full_like(y, float("nan"))
    ft.ft_fp8_linear_parts(xd, wd, pr, ps, yp, ws)
    torch.cuda.synchronize()
    assert_output_close(_bits(y), want, f"fp8 linear ragged T={tokens} K={hidden}")
    assert np.array_equal(_bits(yp), _bits(y))


def test_fp8_linear_prefill_chunk_sampled(ft):
    """8192 tokens x 2048 -> 5120: codes of every token bit-exact, outputs of sampled
    rows (first, last, both ends of one 128-row tile in every band of 1024, and the
    rows either side of a tile boundary) against the oracle."""
    w = synth.WORKLOADS["fp8_linear_qkv_t8192"]
    lin = synth.make_fp8_linear(w)
    x = synth.make_tokens(w)
    xq, s_x = oracle.fp8_quantize(x)
    rows = lin.row_scales()
    xd, wd = _dev_bf16(x), torch.from_numpy(lin.w).cuda()
    ws = ft.fp8_linear_workspace(w.tokens, w.hidden)
    y = torch.empty((w.tokens, w.out_rows), dtype=torch.bfloat16, device="cuda")
    ft.ft_fp8_linear(xd, wd, torch.from_numpy(rows).cuda(), y, ws)
    q = torch.empty((w.tokens, w.hidden), dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    ft.ft_fp8_quantize(xd, q, s, ws)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), xq) and s.item() == s_x
    sample = sorted({0, 8191} | {t for j in range(8) for t in (1024 * j, 1024 * j + 63,
                                                               1024 * j + 127, 1024 * j + 128)}
                    | {4321, 6000, 7777})
    want = _oracle_rows(xq, s_x, lin.w, rows, sample)
    say(f"  comparing {len(sample)} rows of the 8192-token chunk")
    assert_output_close(_bits(y)[sample], want, "fp8 linear T=8192 sampled")
