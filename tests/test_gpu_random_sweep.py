"""GPU parity over seeded random cases: every weight format, random shapes, column
counts and activation distributions, each compared in full with the CPU oracle.

The hand-picked shapes of test_gpu_parity.py sit on the kernels' switch points;
these cases land anywhere between them (rows of one to several thousand, rows of
one to 400 blocks of 32 or 60 superblocks, one to 70 columns), with activations drawn from mixtures the
fixed rows do not cover: per-block scales spread over eight decades, mostly-zero
columns, exact rounding ties, heavy tails.  Bars as everywhere: activation blocks,
per-block int32 sums and dequantized values bit-exact; y within 1e-5 * L (the
L1 of the oracle's block terms).  Every case prints its parameters before it runs.
"""
import numpy as np
import pytest

import quantized_gemv_quantize_amd as qk
from quantized_gemv_quantize_amd import synth
from oracle import oracle as orc

from test_gpu_parity import (_oracle_gemv, _oracle_sums, assert_swiglu, assert_y, dev, host, say,  # noqa: F401
                             torch_cuda, weights)

pytestmark = pytest.mark.gpu

FORMATS = (qk.QK_TYPE_Q8_0, qk.QK_TYPE_Q4_0, qk.QK_TYPE_Q5_0, qk.QK_TYPE_Q4_1, qk.QK_TYPE_Q5_1,
           qk.QK_TYPE_Q2_K, qk.QK_TYPE_Q3_K, qk.QK_TYPE_Q4_K, qk.QK_TYPE_Q5_K, qk.QK_TYPE_Q6_K)
COLS = (1, 1, 1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 48, 63, 64, 65, 70)
MAX_WORK = 12_000_000  # weights x columns per case: the threaded oracle stays within seconds
CASES_PER_FORMAT = 6


def _activations(rng, ncols, n, be):
    """ncols rows of n finite f32 values, each row from one of several mixtures."""
    X = np.empty((ncols, n), np.float32)
    for c in range(ncols):
        kind = int(rng.integers(0, 6))
        if kind == 0:
            v = rng.standard_normal(n)
        elif kind == 1:  # per-block scales over eight decades
            v = rng.standard_normal(n) * np.repeat(10.0 ** rng.uniform(-6, 2, n // be), be)
        elif kind == 2:  # mostly zero, some whole zero blocks
            v = rng.standard_normal(n) * (rng.random(n) < 0.3)
            v.reshape(-1, be)[rng.random(n // be) < 0.25] = 0.0
        elif kind == 3:  # exact ties of the code rounding: amax 127 per block, halves
            v = rng.integers(-126, 126, n) + 0.5
            v[::be] = 127.0
        elif kind == 4:  # heavy tails (finite)
            v = np.clip(rng.standard_cauchy(n), -1e6, 1e6)
        else:            # one constant block value per block
            v = np.repeat(rng.uniform(-4, 4, n // be), be)
        X[c] = v.astype(np.float32)
    return X


def _case(t, k):
    """Shape and column count of case k of format t (seeded, reproducible)."""
    rng = np.random.default_rng(9000 + 100 * t + k)
    be = qk.qk_block_elems(t)
    max_blocks = min(qk.qk_max_n_in(t) // be, 400 if be == 32 else 60)
    nb = int(rng.integers(1, max_blocks + 1))
    n_in = nb * be
    ncols = int(COLS[rng.integers(0, len(COLS))])
    n_out = int(rng.choice([rng.integers(1, 64), rng.integers(64, 1024), rng.integers(1024, 6000)]))
    n_out = max(1, min(n_out, MAX_WORK // (n_in * ncols)))
    return n_out, n_in, ncols, rng


@pytest.mark.parametrize("k", range(CASES_PER_FORMAT))
@pytest.mark.parametrize("t", FORMATS)
def test_random_gemv_case(torch_cuda, t, k):
    n_out, n_in, ncols, rng = _case(t, k)
    at = orc.act_type(t)
    say("random gemv", t, k, n_out, n_in, ncols)
    W = weights(rng, t, n_out, n_in)
    X = _activations(rng, ncols, n_in, qk.qk_block_elems(at))
    xq = orc.quantize(at, X)
    Wd = dev(torch_cuda, W)
    xd = qk.qk_quantize_act(at, dev(torch_cuda, X))
    assert np.array_equal(host(xd), xq), "activation blocks differ"
    sums = host(qk.qk_gemv_block_sums(t, Wd, n_out, n_in, xd, ncols))
    want = _oracle_sums(t, W, xq, n_out, n_in, ncols).reshape(sums.shape)
    bad = np.argwhere(sums != want)
    assert bad.size == 0, f"{len(bad)} block sums differ, first [column, row, block, k] {bad[:4].tolist()}"
    y = host(qk.qk_gemv(t, Wd, n_out, n_in, xd, ncols))
    y_o, l1 = _oracle_gemv(t, W, n_out, n_in, xq, ncols)
    assert_y(y, y_o, l1, f"type {t} {n_out}x{n_in} ncols {ncols}")
    # the typed entry point takes the same path
    y2 = host(qk.qk_gemv_typed(t, at, Wd, n_out, n_in, xd, ncols))
    assert np.array_equal(y2.view(np.uint32), y.view(np.uint32))
    # and dequantize of a random run of whole rows is bit-exact
    r0 = int(rng.integers(0, n_out))
    r1 = int(min(n_out, r0 + 1 + rng.integers(0, 8)))
    rb = qk.qk_row_bytes(t, n_in)
    src = W.reshape(n_out, -1)[r0:r1].reshape(-1)
    got = host(qk.qk_dequantize_row(t, dev(torch_cuda, src), (r1 - r0) * n_in))
    assert src.size == (r1 - r0) * rb
    assert np.array_equal(got.view(np.uint32), orc.dequantize(t, src, (r1 - r0) * n_in).view(np.uint32))


@pytest.mark.parametrize("k", range(4))
@pytest.mark.parametrize("t", [qk.QK_TYPE_Q4_K, qk.QK_TYPE_Q5_K])
def test_random_pair_case(torch_cuda, t, k):
    # the gate / up pair over random shapes: both products in one launch against two
    # GEMVs of the oracle, and SwiGLU of them within the bound the y bars imply
    rng = np.random.default_rng(9500 + 10 * t + k)
    nb = int(rng.integers(1, 49))
    n_in = 256 * nb
    ncols = int(rng.choice([1, 1, 2, 3, 5]))
    n_out = int(max(1, min(int(rng.integers(1, 3000)), MAX_WORK // (2 * n_in * ncols))))
    say("random pair", t, k, n_out, n_in, ncols)
    W1, W2 = weights(rng, t, n_out, n_in), weights(rng, t, n_out, n_in)
    X = _activations(rng, ncols, n_in, 256)
    xq = orc.quantize(orc.Q8_K, X)
    W1d, W2d, xd = dev(torch_cuda, W1), dev(torch_cuda, W2), dev(torch_cuda, xq)
    pair = host(qk.qk_gemv_pair(t, W1d, W2d, n_out, n_in, xd, ncols)).reshape(ncols, 2, n_out)
    g_o, l1g = _oracle_gemv(t, W1, n_out, n_in, xq, ncols)
    u_o, l1u = _oracle_gemv(t, W2, n_out, n_in, xq, ncols)
    assert_y(pair[:, 0], g_o, l1g, "pair y1")
    assert_y(pair[:, 1], u_o, l1u, "pair y2")
    h = host(qk.qk_gemv_pair(t, W1d, W2d, n_out, n_in, xd, ncols, qk.QK_EPI_SWIGLU))
    assert_swiglu(h, g_o, u_o, l1g, l1u, "pair SwiGLU")


@pytest.mark.parametrize("act", [qk.QK_TYPE_Q8_0, qk.QK_TYPE_Q8_1, qk.QK_TYPE_Q8_K])
def test_random_quantize_act_cases(torch_cuda, act):
    rng = np.random.default_rng(9700 + act)
    be = qk.qk_block_elems(act)
    for k in range(8):
        n = be * int(rng.integers(1, 200 if be == 32 else 50))
        ncols = int(rng.integers(1, 20))
        say("random quantize", act, k, n, ncols)
        X = _activations(rng, ncols, n, be)
        assert np.array_equal(host(qk.qk_quantize_act(act, dev(torch_cuda, X))), orc.quantize(act, X))


@pytest.mark.parametrize("t", [qk.QK_TYPE_Q8_0, qk.QK_TYPE_Q4_0, qk.QK_TYPE_Q4_1, qk.QK_TYPE_Q5_0])
def test_random_quantize_row_cases(torch_cuda, t):
    rng = np.random.default_rng(9800 + t)
    for k in range(8):
        n = 32 * int(rng.integers(1, 3000))
        say("random quantize_row", t, k, n)
        x = _activations(rng, 1, n, 32)[0] * np.float32(0.02)
        got = host(qk.qk_quantize_row(t, dev(torch_cuda, x)))
        assert np.array_equal(got, orc.quantize(t, x)), (t, k, n)
