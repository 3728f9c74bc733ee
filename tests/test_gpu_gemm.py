"""Batched dequantise-and-multiply on MFMA (vbq_gemm) against the CPU oracle
(needs an MI355X).

The matrix cores multiply bfloat16 weights, so y = x . bf16(s*q + o)^T.
Bars:
  - within 1e-5 relative L2 of the oracle's product with the weights first
    rounded to bfloat16 (the difference is fp32 accumulation order only);
  - every output within its rounding bound of the exact fp64 product:
    |y - y64| <= (2^-8 + K 2^-23) sum_k |x_k| |w_nk|  (half a bfloat16 ulp of
    each weight, plus fp32 accumulation);
  - within 2e-3 relative L2 of the fp64 oracle over outputs enough for the
    statistics to settle (>= 4096 outputs; expected about 1.7e-3 from the
    weight rounding alone);
  - integer inputs give exact results.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 2e-3
TOL_BF16_W = 1e-5


@pytest.fixture(scope="module")
def vbq():
    import torch
    assert torch.cuda.is_available()
    import packed_decode_gemv_amd as m
    return m


def _t(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def _case(M, N, K, seed, p=(0.55, 0.2, 0.15, 0.1)):
    r = np.random.default_rng(seed)
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64), p=list(p))
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    xb = synth.x_bf16(seed, (77,), M, K)
    return W, widths, xb


GEMM_CASES = [
    (64, 128, 4096),      # one workgroup row of tokens, one weight tile column
    (100, 1000, 4160),    # ragged tokens, rows (not a multiple of 16) and a 1-group second k-tile
    (256, 264, 8192),     # two k-tiles, two token tiles
    (130, 48, 256),       # short K, fewer rows than a workgroup
    (1, 16, 64),          # smallest shape
    (300, 130, 1024),     # three token tiles
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=[f"{m}x{n}x{k}" for m, n, k in GEMM_CASES])
def test_gemm_parity(vbq, case):
    import torch
    M, N, K = case
    W, widths, xb = _case(M, N, K, seed=M * 7 + N + K)
    print(f"case gemm M={M} N={N} K={K}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    y = vbq.vbq_gemm(pm, _t(xb, torch.bfloat16)).cpu().numpy()
    q, s, o = oracle.quantize_matrix(W, widths)
    assert y.shape == (M, N)
    check_gemm(y, q, s, o, xb)


def check_gemm(y, q, s, o, xb):
    ref = oracle.gemv(q, s, o, xb, bf16=True)
    assert rel_l2(y, oracle.gemm_bf16_weights(q, s, o, xb)) <= TOL_BF16_W
    K = q.shape[1]
    absw = np.abs(oracle.bf16_to_f64(oracle.dequant_bf16(q, s, o))) * (1 + 2.0 ** -8)
    bound = (np.abs(oracle.bf16_to_f64(xb)) @ absw.T) * (2.0 ** -8 + K * 2.0 ** -23)
    assert np.all(np.abs(y - ref) <= bound)
    if y.size >= 4096:
        assert rel_l2(y, ref) <= TOL


def test_gemm_exact_integer(vbq):
    """8-bit codes 0..255 with 0 and 255 in every group give s = 1, o = 0
    exactly; x in {-2..2} is exact in bfloat16 and every partial sum stays
    below 2^24, so the result is the exact integer product."""
    import torch
    r = np.random.default_rng(12)
    M, N, K = 192, 272, 768
    Wi = r.integers(0, 256, (N, K))
    Wi[:, 0::64] = 0
    Wi[:, 1::64] = 255
    widths = np.full((N, K // 64), 8, np.uint8)
    xi = r.integers(-2, 3, (M, K))
    xb = (xi.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # exact: small integers
    pm = vbq.vbq_pack(_t(Wi.astype(np.float32)), widths)
    y = vbq.vbq_gemm(pm, _t(xb, torch.bfloat16)).cpu().numpy()
    assert np.array_equal(y.astype(np.int64), xi @ Wi.T)


def test_gemm_repeatable(vbq):
    import torch
    W, widths, xb = _case(160, 200, 4096 + 128, seed=5)
    pm = vbq.vbq_pack(_t(W), widths)
    xt = _t(xb, torch.bfloat16)
    a = vbq.vbq_gemm(pm, xt)
    b = vbq.vbq_gemm(pm, xt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_workload_gemm_full_size_sampled(vbq):
    """M = 256 tokens, K = 4096, N = 14336 with the default width mix: the
    whole product on the GPU, sampled rows against the oracle."""
    import torch
    proj = synth.C4.projs[0]
    M = synth.C4.gemm_m
    key = synth.proj_key(4, 0, 0)
    N, K = proj.n, proj.k
    widths = synth.widths(synth.SEED, key, N, K // 64, proj.mix)
    W = synth.weights(synth.SEED, key, N, K)
    xb = synth.x_bf16(synth.SEED, key, M, K)
    print(f"case workload 4 gemm M={M} N={N} K={K}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    y = vbq.vbq_gemm(pm, _t(xb, torch.bfloat16)).cpu().numpy()
    r = np.random.default_rng(4)
    rows = np.array(sorted(set(r.choice(N, 96, replace=False).tolist()) | {0, N - 1}), np.int64)
    q, s, o = oracle.quantize_matrix(W[rows], widths[rows])
    check_gemm(y[:, rows], q, s, o, xb)
