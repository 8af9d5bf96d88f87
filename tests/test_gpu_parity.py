"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars (per the method's definition):
  - activation blocks (qk_quantize_act): bit-exact;
  - per-block int32 sums of the GEMV kernels: bit-exact;
  - dequantized values: bit-exact (every product is exact in f32);
  - y: |y_gpu - y_oracle| <= 1e-5 * L per output, where L is the sum over blocks of
    the absolute float terms of the oracle's block steps: |c_b| for the one-term
    formats, |(dx d) S_q| + |(dx dmin) S_m| for Q4_K and Q5_K (a relative bound that
    stays meaningful when a random dot product, or one block's two terms, cancel;
    codeloopback Example 10 reports its error against the sum of |a*b| for the same
    reason).  The GPU sums the same terms in a different order (and may fuse
    multiply-adds), which stays far inside it.
Inputs are seeded (numpy) and synthetic; see quantized_gemv_quantize_amd/synth.py.
"""
import os

import numpy as np
import pytest

import quantized_gemv_quantize_amd as qk
from quantized_gemv_quantize_amd import synth
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

T8_0, T4_0, T4K, T6K, T8K = (qk.QK_TYPE_Q8_0, qk.QK_TYPE_Q4_0, qk.QK_TYPE_Q4_K,
                             qk.QK_TYPE_Q6_K, qk.QK_TYPE_Q8_K)
T4_1, T5_0, T5_1, T5K = qk.QK_TYPE_Q4_1, qk.QK_TYPE_Q5_0, qk.QK_TYPE_Q5_1, qk.QK_TYPE_Q5_K
T8_1 = qk.QK_TYPE_Q8_1
T2K, T3K = qk.QK_TYPE_Q2_K, qk.QK_TYPE_Q3_K
Y_TOL = 1e-5


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    qk.lib()
    return torch


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def say(*a):
    print("[case]", *a, flush=True)


def assert_y(y_gpu, y_orc, l1, what):
    """y within 1e-5 * L where the oracle's y is finite; where it is not (a block term
    that overflows, e.g. a Q8_1 sum field rounded to f16 infinity), the GPU must give
    the same value: the same infinity, or NaN for NaN."""
    yg, yo = y_gpu.astype(np.float64), y_orc.astype(np.float64)
    assert yg.shape == yo.shape, f"{what}: shape {yg.shape} against {yo.shape}"
    fin = np.isfinite(yo)
    nf = ~fin
    same = (yg[nf] == yo[nf]) | (np.isnan(yg[nf]) & np.isnan(yo[nf]))
    assert same.all(), f"{what}: {int((~same).sum())} non-finite oracle outputs not reproduced"
    err = np.abs(yg[fin] - yo[fin])
    l1f = l1[fin]
    bad = ~(err <= Y_TOL * l1f)  # NaN in err counts as a failure
    ratio = np.max(err / np.maximum(l1f, 1e-300), initial=0.0)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond 1e-5 * L (worst {ratio:.3g})"


def weights(rng, t, n_out, n_in):
    if t == T8_0:
        return orc.quantize(orc.Q8_0, synth.gaussian(rng, (n_out, n_in), 0.02))
    return synth.weight_blocks(rng, t, n_out, n_in)


# ---------------------------------------------------------------------------
# qk_quantize_act
# ---------------------------------------------------------------------------

def _special_rows(n, rng):
    """Activation rows that exercise the edge semantics of the quantizer."""
    rows = []
    rows.append(rng.standard_normal(n).astype(np.float32))
    rows.append((rng.standard_normal(n) * 1e3).astype(np.float32))
    rows.append(np.zeros(n, np.float32))                          # d = 0 -> codes 0
    z = rng.standard_normal(n).astype(np.float32)
    z[::7] = np.nan                                               # NaN ignored / coded 0
    rows.append(z)
    w = rng.standard_normal(n).astype(np.float32)
    w[5] = np.inf                                                 # inf amax -> d = inf
    w[n // 2 + 3] = -np.inf
    rows.append(w)
    rows.append((rng.standard_normal(n) * 1e-39).astype(np.float32))   # subnormal f32
    rows.append((rng.standard_normal(n) * 1e-42).astype(np.float32))   # 1/d overflows
    rows.append((rng.standard_normal(n) * 2e-6).astype(np.float32))    # f16 subnormal d
    rows.append((rng.standard_normal(n) * 9e6).astype(np.float32))     # f16 d -> inf
    # exact ties: values (k + 0.5) * d with d = 1 -> amax 127 so id = 1/ (127/127)
    t = (rng.integers(-126, 126, n) + 0.5).astype(np.float32)
    t[::32] = 127.0
    rows.append(t)
    rows.append(np.full(n, -3.25, np.float32))
    allnan = rng.standard_normal(n).astype(np.float32)
    allnan[:256] = np.nan                                         # whole blocks of NaN -> d = 0
    rows.append(allnan)
    rows.append(np.float32(1.0) * (np.arange(n) % 256 - 128).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("act", [T8_0, T8_1, T8K])
@pytest.mark.parametrize("n", [256, 4096, 11008])
def test_quantize_act_bit_exact(torch_cuda, act, n):
    say("quantize", act, n)
    rng = np.random.default_rng(1000 + n + act)
    X = _special_rows(n, rng)
    got = host(qk.qk_quantize_act(act, dev(torch_cuda, X)))
    want = orc.quantize(act, X)
    torch_cuda.cuda.synchronize()
    assert got.shape == want.shape
    mism = np.nonzero((got != want).any(axis=1))[0]
    assert mism.size == 0, f"rows {mism.tolist()} differ"


def test_quantize_act_many_columns(torch_cuda):
    say("quantize many columns")
    rng = np.random.default_rng(7)
    X = rng.standard_normal((64, 4096)).astype(np.float32)
    for act in (T8_0, T8_1, T8K):
        assert np.array_equal(host(qk.qk_quantize_act(act, dev(torch_cuda, X))),
                              orc.quantize(act, X))


# ---------------------------------------------------------------------------
# qk_quantize_row (weight quantizers)
# ---------------------------------------------------------------------------

def _cl_inputs(n):
    # codeloopback Example 14's inputs: ((i * 7919) mod 1001 - 500) / 337 in f32
    i = np.arange(n)
    return (((i * 7919) % 1001) - 500).astype(np.float32) / np.float32(337)


def _weight_rows(rng, n):
    """Finite weight rows (n a multiple of 32) that exercise the quantizers' edges:
    ties for the largest magnitude, signed zeros, constant and all-zero blocks,
    f16-subnormal and f16-overflowing scales, f32 subnormals."""
    rows = [rng.standard_normal(n).astype(np.float32) * np.float32(0.02),
            (rng.standard_normal(n) * 50).astype(np.float32),
            np.zeros(n, np.float32),
            np.full(n, -0.0, np.float32),
            np.full(n, 0.75, np.float32),
            (rng.standard_normal(n) * 1e-39).astype(np.float32),     # 1/d overflows
            (rng.standard_normal(n) * 3e-37).astype(np.float32),     # 1/d near FLT_MAX
            (rng.standard_normal(n) * 1e-6).astype(np.float32),
            (rng.standard_normal(n) * 3e5).astype(np.float32),
            (rng.standard_normal(n) * 1e37).astype(np.float32),
            rng.integers(-16, 16, n).astype(np.float32)]
    t = rng.standard_normal(n).astype(np.float32)
    blocks = t.reshape(-1, 32)
    for b in range(blocks.shape[0]):
        i, j = rng.choice(32, 2, replace=False)
        a = np.float32(3.0 + b % 5)
        blocks[b, i], blocks[b, j] = a, -a          # equal magnitudes, opposite signs
    rows.append(t)
    z = rng.standard_normal(n).astype(np.float32)
    z[rng.integers(0, 2, n) == 1] = 0.0
    z[::3] = -0.0
    zb = z.reshape(-1, 32)
    zb[::2] = np.where(rng.integers(0, 2, zb[::2].shape) == 1, -0.0, 0.0)  # all-zero blocks
    rows.append(z)
    s = np.abs(rng.standard_normal(n)).astype(np.float32) + np.float32(2)   # min > 0
    rows.append(s)
    return np.stack(rows)


@pytest.mark.parametrize("t", [T8_0, T4_0, T4_1, T5_0])
def test_quantize_row_bit_exact(torch_cuda, t):
    rng = np.random.default_rng(500 + t)
    for n in (32, 96, 4096, 32 * 1001):
        say("quantize_row", t, n)
        X = _weight_rows(rng, n)
        for r in range(X.shape[0]):
            got = host(qk.qk_quantize_row(t, dev(torch_cuda, X[r])))
            want = orc.quantize(t, X[r])
            bad = np.nonzero((got.reshape(-1, orc.block_bytes(t)) !=
                              want.reshape(-1, orc.block_bytes(t))).any(axis=1))[0]
            assert bad.size == 0, f"type {t} n {n} row {r}: blocks {bad[:8].tolist()} differ"


def test_quantize_row_page_hex_example_14(torch_cuda):
    # the printed block bytes of codeloopback Example 14, straight from the GPU
    from golden_io import rows
    say("quantize_row Example 14")
    x = _cl_inputs(64)
    x[40] = np.float32(9.5)
    types = {"Q8_0": T8_0, "Q4_0": T4_0, "Q4_1": T4_1, "Q5_0": T5_0}
    xd = dev(torch_cuda, x)
    for blk, name, hexs in rows("hex_crosscheck.txt"):
        got = host(qk.qk_quantize_row(types[name], xd))
        bb = len(hexs) // 2
        assert got[int(blk) * bb:(int(blk) + 1) * bb].tobytes().hex() == hexs, (blk, name)


def test_quantize_row_full_4096x11008(torch_cuda):
    # a whole weight matrix quantized in one call, as a model loader would
    rng = np.random.default_rng(512)
    Wf = synth.f32_weights_4096x11008()["W_f32"]
    Wd = dev(torch_cuda, Wf)
    for t in (T4_0, T4_1, T5_0, T8_0):
        say("quantize_row full", t)
        got = host(qk.qk_quantize_row(t, Wd)).reshape(4096, -1)
        pick = np.unique(np.concatenate([np.arange(8), rng.integers(0, 4096, 24), [4095]]))
        want = orc.quantize(t, Wf[pick])
        assert np.array_equal(got[pick], want.reshape(len(pick), -1)), t


# ---------------------------------------------------------------------------
# qk_dequantize_row
# ---------------------------------------------------------------------------

def _edge_scale_blocks(t, rng, nblocks):
    """Blocks with unusual f16 scales: subnormal, negative, largest finite."""
    n = nblocks * synth.BLOCK_ELEMS[t]
    b = weights(rng, t, 1, n).reshape(nblocks, -1).copy()
    specials = np.array([0x0001, 0x03FF, 0x8001, 0x7BFF, 0xFBFF, 0x3C00, 0xBC00, 0x0000],
                        dtype=np.uint16).view(np.uint8).reshape(-1, 2)
    offs = {T8_0: [0], T4_0: [0], T4_1: [0, 2], T5_0: [0], T5_1: [0, 2], T4K: [0, 2], T5K: [0, 2],
            T6K: [208], T2K: [80, 82], T3K: [108]}[t]
    for i in range(nblocks):
        for o in offs:
            b[i, o:o + 2] = specials[(i + o) % len(specials)]
    return b.reshape(-1)


@pytest.mark.parametrize("t", [T8_0, T4_0, T4_1, T5_0, T5_1, T2K, T3K, T4K, T5K, T6K])
def test_dequantize_bit_exact(torch_cuda, t):
    rng = np.random.default_rng(200 + t)
    for nblocks in (1, 3, 17, 1000):
        say("dequantize", t, nblocks)
        n = nblocks * synth.BLOCK_ELEMS[t]
        for src in (weights(rng, t, 1, n).reshape(-1), _edge_scale_blocks(t, rng, nblocks)):
            got = host(qk.qk_dequantize_row(t, dev(torch_cuda, src), n))
            want = orc.dequantize(t, src, n)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (t, nblocks)


# ---------------------------------------------------------------------------
# qk_gemv: per-block integer sums and y
# ---------------------------------------------------------------------------

SHAPES = {
    T4K: [(1, 256), (5, 512), (67, 4096), (9, 4352), (13, 11008), (3, 12544), (6, 28672)],
    T6K: [(1, 256), (5, 512), (67, 4096), (9, 4352), (13, 11008), (3, 12544), (6, 28672)],
    T5K: [(1, 256), (5, 512), (67, 4096), (9, 4352), (13, 11008), (3, 12544), (6, 28672)],
    T2K: [(1, 256), (5, 512), (67, 4096), (9, 4352), (13, 11008), (3, 12544), (6, 28672)],
    T3K: [(1, 256), (5, 512), (67, 4096), (9, 4352), (13, 11008), (3, 12544), (6, 28672)],
    T8_0: [(1, 32), (5, 96), (67, 1024), (9, 2048), (13, 4096), (3, 4128), (4, 10240), (7, 11008), (6, 28672)],
    T4_0: [(1, 32), (5, 96), (67, 1024), (9, 2048), (13, 4096), (3, 4128), (4, 10240), (7, 11008), (6, 28672)],
    T5_0: [(1, 32), (5, 96), (67, 1024), (9, 2048), (13, 4096), (3, 4128), (4, 10240), (7, 11008), (6, 28672)],
    T4_1: [(1, 32), (5, 96), (67, 1024), (9, 2048), (13, 4096), (3, 4128), (4, 10240), (7, 11008), (6, 28672)],
    T5_1: [(1, 32), (5, 96), (67, 1024), (9, 2048), (13, 4096), (3, 4128), (4, 10240), (7, 11008), (6, 28672)],
}


def _row_chunks(n_out):
    """Row ranges that split a matrix over the host's threads (the C oracle's
    calls release the GIL, so large full-size cases run on every core)."""
    parts = min(n_out, 4 * _THREADS)
    edges = np.linspace(0, n_out, parts + 1).astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_sums(t, W, xq, n_out, n_in, ncols):
    """Per-block integer sums of every (column, row): [ncols, n_out, blocks, k]."""
    from concurrent.futures import ThreadPoolExecutor
    W2 = W.reshape(n_out, -1)
    with ThreadPoolExecutor(_THREADS) as ex:
        parts = list(ex.map(lambda rr: orc.gemv_block_sums(t, W2[rr[0]:rr[1]], rr[1] - rr[0], n_in, xq, ncols),
                            _row_chunks(n_out)))
    return np.concatenate(parts, axis=1)


def _oracle_gemv(t, W, n_out, n_in, xq, ncols):
    """orc.gemv over all rows, split over the host's threads: (y, l1) [ncols, n_out]."""
    from concurrent.futures import ThreadPoolExecutor
    W2 = W.reshape(n_out, -1)
    with ThreadPoolExecutor(_THREADS) as ex:
        parts = list(ex.map(lambda rr: orc.gemv(t, W2[rr[0]:rr[1]], rr[1] - rr[0], n_in, xq, ncols),
                            _row_chunks(n_out)))
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


@pytest.mark.parametrize("t", [T8_0, T4_0, T5_0, T4_1, T5_1, T2K, T3K, T4K, T5K, T6K])
def test_gemv_block_sums_and_y(torch_cuda, t):
    rng = np.random.default_rng(300 + t)
    at = orc.act_type(t)
    for n_out, n_in in SHAPES[t]:
        for ncols in (1, 3):
            say("gemv", t, n_out, n_in, ncols)
            W = weights(rng, t, n_out, n_in)
            X = rng.standard_normal((ncols, n_in)).astype(np.float32)
            xq = orc.quantize(at, X)
            Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
            # activation blocks from the GPU quantizer equal the oracle's
            assert np.array_equal(host(qk.qk_quantize_act(at, dev(torch_cuda, X))), xq)
            sums = host(qk.qk_gemv_block_sums(t, Wd, n_out, n_in, xd, ncols))
            want = _oracle_sums(t, W, xq, n_out, n_in, ncols).reshape(sums.shape)
            bad = np.argwhere(sums != want)
            assert bad.size == 0, (f"type {t} {n_out}x{n_in} ncols {ncols}: {len(bad)} sums differ, "
                                   f"first [column, row, block, k] {bad[:4].tolist()}: "
                                   f"got {sums[tuple(bad[0])]}, want {want[tuple(bad[0])]}")
            y = host(qk.qk_gemv(t, Wd, n_out, n_in, xd, ncols))
            y_o, l1 = orc.gemv(t, W, n_out, n_in, xq, ncols)
            assert_y(y, y_o, l1, f"type {t} {n_out}x{n_in} ncols {ncols}")


# Q4_K with several activation columns runs on the matrix cores (16-token tiles,
# up to 64 columns per pass), or for 2 (3) columns on the multi-column GEMV
# kernel: ragged row counts, every tile count and the column counts around each
# tile, pass and kernel boundary.
BATCHED = [(1, 256, 2), (17, 512, 16), (33, 1024, 17), (45, 4096, 33), (70, 2304, 48),
           (31, 11008, 64), (50, 768, 65), (21, 4352, 130), (129, 256, 7),
           # past the row counts that switch to 64-row workgroups, ragged
           (8300, 256, 9), (4200, 256, 24), (4160, 256, 40), (8300, 1024, 40), (2100, 2560, 64),
           # small batches: the multi-column GEMV kernel (2 columns; 3 up to 8192
           # rows) and, past 8192 rows, the matrix cores at 3 columns
           (37, 2304, 3), (8300, 256, 3), (4100, 11008, 2),
           # up to 16 columns on tall matrices with rows of at most 16 superblocks:
           # one superblock per wavefront, two to four row tiles per workgroup
           (7000, 2048, 13), (6500, 4096, 16), (9001, 4096, 5), (11008, 4096, 16),
           # 33 to 64 columns on the same tall matrices: two superblocks per
           # wavefront (an odd count leaves the last one alone), two to four row tiles
           (6500, 4096, 33), (9001, 2304, 50), (5000, 768, 47), (11008, 4096, 64)]


@pytest.mark.parametrize("n_out,n_in,ncols", BATCHED)
def test_batched_q4_K_block_sums_and_y(torch_cuda, n_out, n_in, ncols):
    say("batched Q4_K", n_out, n_in, ncols)
    rng = np.random.default_rng(n_out * 7 + ncols)
    W = synth.q4_K_blocks(rng, n_out, n_in)
    X = rng.standard_normal((ncols, n_in)).astype(np.float32)
    X[ncols // 2] = 0.0                      # an all-zero column: d = 0, codes 0
    xq = orc.quantize(T8K, X)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    sums = host(qk.qk_gemv_block_sums(T4K, Wd, n_out, n_in, xd, ncols))
    want = _oracle_sums(T4K, W, xq, n_out, n_in, ncols)
    assert np.array_equal(sums, want.reshape(sums.shape))
    y = host(qk.qk_gemv(T4K, Wd, n_out, n_in, xd, ncols))
    y_o, l1 = _oracle_gemv(T4K, W, n_out, n_in, xq, ncols)
    assert_y(y, y_o, l1, f"batched Q4_K {n_out}x{n_in} ncols {ncols}")
    assert not y[ncols // 2].any()


@pytest.mark.parametrize("n_out,n_in,ncols", [(40, 1024, 20), (4200, 1024, 64)])
def test_batched_q4_K_extreme_codes(torch_cuda, n_out, n_in, ncols):
    # every nibble 15, every 6-bit scale and min 63, activations at +-127: the
    # largest integer sums the format allows, on both MFMA products
    say("batched Q4_K extreme codes", n_out, n_in, ncols)
    rng = np.random.default_rng(77)
    W = synth.q4_K_blocks(rng, n_out, n_in).reshape(n_out, n_in // 256, 144)
    W[:, :, 4:] = 0xFF
    W = W.reshape(n_out, -1)
    X = np.where(rng.integers(0, 2, (ncols, n_in)) == 1, 1.0, -1.0).astype(np.float32)
    X[1] = 1.0
    X[2] = -1.0
    xq = orc.quantize(T8K, X)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    sums = host(qk.qk_gemv_block_sums(T4K, Wd, n_out, n_in, xd, ncols))
    want = _oracle_sums(T4K, W, xq, n_out, n_in, ncols)
    assert np.array_equal(sums, want.reshape(sums.shape))
    assert np.abs(want).max() == 256 * 15 * 63 * 127
    y = host(qk.qk_gemv(T4K, Wd, n_out, n_in, xd, ncols))
    y_o, l1 = orc.gemv(T4K, W, n_out, n_in, xq, ncols)
    assert_y(y, y_o, l1, "batched Q4_K extreme codes")


def test_gemv_max_row_length(torch_cuda):
    rng = np.random.default_rng(31)
    for t in (T4K, T5K, T6K, T8_0, T4_0, T5_0, T4_1, T5_1, T2K, T3K):
        n_in = qk.qk_max_n_in(t)
        say("gemv max n_in", t, n_in)
        W = weights(rng, t, 3, n_in)
        X = rng.standard_normal((1, n_in)).astype(np.float32)
        xq = orc.quantize(orc.act_type(t), X)
        y = host(qk.qk_gemv(t, dev(torch_cuda, W), 3, n_in, dev(torch_cuda, xq), 1))
        y_o, l1 = orc.gemv(t, W, 3, n_in, xq, 1)
        assert_y(y, y_o, l1, f"type {t} max n_in {n_in}")


def test_lds_budget_matches_device(torch_cuda):
    # the one-column kernels stage rows up to 160 KB of activation blocks in one
    # workgroup's LDS: the device must let a workgroup address that much
    props = torch_cuda.cuda.get_device_properties(0)
    say("sharedMemPerBlock", props.shared_memory_per_block)
    assert props.shared_memory_per_block >= 163840
    n = qk.qk_max_n_in(T4K)
    assert n // 256 * 292 <= 163840 < (n // 256 + 1) * 292


def test_long_rows_beyond_64KB_lds(torch_cuda):
    # rows whose activation blocks need more than 64 KB of LDS: the launches opt in
    # to the larger dynamic LDS; every path that takes such rows (one column, column
    # groups falling back to one column per launch, the matrix-core kernel over a
    # long K, the gate / up pair) against the oracle
    rng = np.random.default_rng(33)
    n_in = qk.qk_max_n_in(T4K)
    assert n_in // 256 * 292 > 65536
    n_out = 37
    W = weights(rng, T4K, n_out, n_in)
    X = rng.standard_normal((16, n_in)).astype(np.float32)
    xq = orc.quantize(orc.Q8_K, X)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    for ncols in (1, 3, 16):
        say("long rows Q4_K", n_in, ncols)
        sums = host(qk.qk_gemv_block_sums(T4K, Wd, n_out, n_in, xd, ncols))
        assert np.array_equal(sums, _oracle_sums(T4K, W, xq[:ncols], n_out, n_in, ncols).reshape(sums.shape))
        y = host(qk.qk_gemv(T4K, Wd, n_out, n_in, xd, ncols))
        y_o, l1 = orc.gemv(T4K, W, n_out, n_in, xq[:ncols], ncols)
        assert_y(y, y_o, l1, f"Q4_K n_in {n_in} ncols {ncols}")
    say("long rows pair", n_in)
    W2 = weights(rng, T4K, n_out, n_in)
    out = host(qk.qk_gemv_pair(T4K, Wd, dev(torch_cuda, W2), n_out, n_in, xd, 1, qk.QK_EPI_NONE))
    y1, l1a = orc.gemv(T4K, W, n_out, n_in, xq[:1], 1)
    y2, l1b = orc.gemv(T4K, W2, n_out, n_in, xq[:1], 1)
    assert_y(out.reshape(2, n_out)[0], y1[0], l1a[0], "pair y1 long rows")
    assert_y(out.reshape(2, n_out)[1], y2[0], l1b[0], "pair y2 long rows")
    for t in (T8_0, T4_1, T6K):
        n_t = qk.qk_max_n_in(t)
        say("long rows", t, n_t)
        Wt = weights(rng, t, 5, n_t)
        Xt = rng.standard_normal((2, n_t)).astype(np.float32)
        xt = orc.quantize(orc.act_type(t), Xt)
        y = host(qk.qk_gemv(t, dev(torch_cuda, Wt), 5, n_t, dev(torch_cuda, xt), 2))
        y_o, l1 = orc.gemv(t, Wt, 5, n_t, xt, 2)
        assert_y(y, y_o, l1, f"type {t} n_in {n_t} ncols 2")


def test_gemv_zero_activation_gives_zero(torch_cuda):
    # rml ZeroActivationsGiveZero
    rng = np.random.default_rng(5)
    for t in (T4K, T5K, T6K, T8_0, T4_0, T5_0, T4_1, T5_1, T2K, T3K):
        W = weights(rng, t, 8, 1024)
        xq = qk.qk_quantize_act(orc.act_type(t), torch_cuda.zeros((1, 1024), device="cuda"))
        y = host(qk.qk_gemv(t, dev(torch_cuda, W), 8, 1024, xq, 1))
        assert not y.any()


def test_gemv_typed_is_gemv_with_a_pairing_check(torch_cuda):
    # the stated activation type only adds the pairing check: y is qk_gemv's, bit for
    # bit, and a mismatched type fails before anything is enqueued (y untouched)
    rng = np.random.default_rng(17)
    for t in (T4K, T5K, T6K, T8_0, T4_0, T5_0, T4_1, T5_1, T2K, T3K):
        say("qk_gemv_typed", t)
        W = dev(torch_cuda, weights(rng, t, 37, 1024))
        at = qk.qk_act_type(t)
        xq = qk.qk_quantize_act(at, torch_cuda.randn((2, 1024), device="cuda"))
        want = host(qk.qk_gemv(t, W, 37, 1024, xq, 2))
        got = host(qk.qk_gemv_typed(t, at, W, 37, 1024, xq, 2))
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        y = torch_cuda.full((2, 37), 7.0, device="cuda")
        for other in (qk.QK_TYPE_Q8_0, qk.QK_TYPE_Q8_1, qk.QK_TYPE_Q8_K):
            if other == at:
                continue
            with pytest.raises(qk.QKError) as e:
                qk.qk_gemv_typed(t, other, W, 37, 1024, xq, 2, y=y)
            assert e.value.status == 2
        assert bool((y == 7.0).all())


def test_empty_calls_touch_nothing(torch_cuda):
    # zero rows, zero columns or zero elements: QK_OK, nothing launched, buffers intact
    torch = torch_cuda
    say("empty calls")
    L = qk.lib()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    W = torch.zeros(4 * 144, dtype=torch.uint8, device="cuda")
    xq = torch.zeros(292, dtype=torch.uint8, device="cuda")
    x = torch.zeros(256, dtype=torch.float32, device="cuda")
    y = torch.full((16,), 7.0, dtype=torch.float32, device="cuda")
    blk = torch.full((64,), 0xAB, dtype=torch.uint8, device="cuda")
    assert L.qk_gemv(T4K, p(W), 0, 256, p(xq), 1, p(y), st) == 0
    assert L.qk_gemv(T4K, p(W), 4, 256, p(xq), 0, p(y), st) == 0
    assert L.qk_gemv_block_sums(T6K, p(W), 0, 256, p(xq), 1, p(y), st) == 0
    assert L.qk_gemv_pair(T4K, p(W), p(W), 0, 256, p(xq), 1, 1, p(y), st) == 0
    assert L.qk_quantize_act(T8K, p(x), p(blk), 256, 0, st) == 0
    assert L.qk_quantize_row(T4_0, p(x), p(blk), 0, st) == 0
    assert L.qk_dequantize_row(T4K, p(W), p(y), 0, st) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and torch.all(blk == 0xAB)


def test_gemv_rejects_misaligned_view(torch_cuda):
    rng = np.random.default_rng(6)
    W = dev(torch_cuda, weights(rng, T4K, 4, 512))
    xq = qk.qk_quantize_act(T8K, dev(torch_cuda, rng.standard_normal((1, 512)).astype(np.float32)))
    with pytest.raises(qk.QKError) as e:
        qk.qk_gemv(T4K, W.reshape(-1)[8:], 3, 512, xq, 1)
    assert e.value.status == 4
    with pytest.raises(qk.QKError) as e:
        qk.qk_gemv(T8K, W, 4, 512, xq, 1)
    assert e.value.status == 1


def test_gemv_timed_matches_untimed(torch_cuda):
    rng = np.random.default_rng(8)
    W = dev(torch_cuda, weights(rng, T4K, 256, 4096))
    xq = qk.qk_quantize_act(T8K, dev(torch_cuda, rng.standard_normal((2, 4096)).astype(np.float32)))
    y0 = qk.qk_gemv(T4K, W, 256, 4096, xq, 2)
    e0 = torch_cuda.cuda.Event(enable_timing=True)
    e1 = torch_cuda.cuda.Event(enable_timing=True)
    e0.record()  # torch creates the underlying hipEvent_t on first record
    e1.record()
    y1 = torch_cuda.empty_like(y0)
    qk.qk_gemv_timed(T4K, W, 256, 4096, xq, 2, y1, e0, e1)
    e1.synchronize()
    assert e0.elapsed_time(e1) > 0
    assert torch_cuda.equal(y0, y1)


def test_quantize_act_timed_matches_untimed(torch_cuda):
    rng = np.random.default_rng(14)
    for act, n, ncols in ((T8K, 11008, 1), (T8_0, 4096, 3)):
        say("quantize_act_timed", act, n, ncols)
        x = dev(torch_cuda, rng.standard_normal((ncols, n)).astype(np.float32))
        want = host(qk.qk_quantize_act(act, x))
        xq = torch_cuda.zeros((ncols, qk.qk_row_bytes(act, n)), dtype=torch_cuda.uint8, device="cuda")
        e0 = torch_cuda.cuda.Event(enable_timing=True)
        e1 = torch_cuda.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()
        qk.qk_quantize_act_timed(act, x, xq, e0, e1)
        torch_cuda.cuda.synchronize()
        assert np.array_equal(host(xq), want)
        assert e0.elapsed_time(e1) > 0


def test_gemv_pair_timed_matches_untimed(torch_cuda):
    rng = np.random.default_rng(9)
    for n_in in (4096, 11008):  # the register kernel and the LDS kernel
        W1 = dev(torch_cuda, synth.q4_K_blocks(rng, 64, n_in))
        W2 = dev(torch_cuda, synth.q4_K_blocks(rng, 64, n_in))
        xq = qk.qk_quantize_act(T8K, dev(torch_cuda, rng.standard_normal((2, n_in)).astype(np.float32)))
        for epi in (qk.QK_EPI_NONE, qk.QK_EPI_SWIGLU):
            say("gemv_pair_timed", n_in, epi)
            out0 = qk.qk_gemv_pair(T4K, W1, W2, 64, n_in, xq, 2, epi)
            e0 = torch_cuda.cuda.Event(enable_timing=True)
            e1 = torch_cuda.cuda.Event(enable_timing=True)
            e0.record()
            e1.record()
            out1 = torch_cuda.empty_like(out0)
            qk.qk_gemv_pair_timed(T4K, W1, W2, 64, n_in, xq, 2, epi, out1, e0, e1)
            e1.synchronize()
            assert e0.elapsed_time(e1) > 0
            assert torch_cuda.equal(out0, out1)


@pytest.mark.parametrize("nbytes", [16, 2048, 5 * 2048 + 7 * 16, 25_362_432])
def test_read_probe_xor_of_each_group(torch_cuda, nbytes):
    say("read_probe", nbytes)
    rng = np.random.default_rng(10)
    buf = rng.integers(0, 256, size=nbytes + 4096, dtype=np.uint8)  # bytes past nbytes must not count
    out = host(qk.qk_read_probe(dev(torch_cuda, buf), nbytes)).view(np.uint32)
    ng = (nbytes + 2047) // 2048
    words = np.zeros(ng * 512, dtype=np.uint32)
    words[:nbytes // 4] = buf[:nbytes].view("<u4")
    assert out.shape == (ng,)
    assert np.array_equal(out, np.bitwise_xor.reduce(words.reshape(ng, 512), axis=1))


@pytest.mark.parametrize("kb,grid,nt", [(1, 0, 0), (4, 0, 1), (8, 0, 0), (16, 0, 0), (2, 3, 0), (4, 256, 1),
                                         (16, 1, 0)])
def test_read_probe_ex_xor_of_each_group(torch_cuda, kb, grid, nt):
    # every load pattern of the probe reads exactly the bytes asked for: the XOR of
    # each kb-kilobyte group (a persistent grid of `grid` workgroups strides over them)
    for nbytes in (16, 1024 * kb * 37 + 7 * 16, 3_000_000):
        say("read_probe_ex", kb, grid, nt, nbytes)
        rng = np.random.default_rng(11)
        buf = rng.integers(0, 256, size=nbytes + 4096, dtype=np.uint8)
        out = host(qk.qk_read_probe_ex(dev(torch_cuda, buf), nbytes, kb, grid, nt)).view(np.uint32)
        gw = 256 * kb
        ng = (nbytes + 4 * gw - 1) // (4 * gw)
        words = np.zeros(ng * gw, dtype=np.uint32)
        words[:nbytes // 4] = buf[:nbytes].view("<u4")
        assert out.shape == (ng,)
        assert np.array_equal(out, np.bitwise_xor.reduce(words.reshape(ng, gw), axis=1))


def test_c_abi_from_a_host_program(torch_cuda):
    # the C ABI without Python or torch: a host program allocates with the HIP
    # runtime, calls include/qk.h and checks every result against the C oracle
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_check")
    assert os.path.exists(exe), "tests/c/abi_check is not built (run __graft_entry__.build())"
    say("c abi_check")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check ok" in r.stdout


def test_two_streams_concurrently(torch_cuda):
    # the library keeps no state between calls beyond a per-device cache of the CU
    # count: calls on two streams at once (different formats, launch shapes and
    # inputs, outputs in separate buffers) give what each gives alone
    torch = torch_cuda
    rng = np.random.default_rng(91)
    cases = [(T6K, 9000, 4096, 1), (T4K, 4096, 11008, 1), (T4_0, 5000, 4096, 3), (T4K, 3000, 4096, 16)]
    bufs, want = [], []
    for t, n_out, n_in, nc in cases:
        W = dev(torch, weights(rng, t, n_out, n_in))
        x = dev(torch, rng.standard_normal((nc, n_in)).astype(np.float32))
        at = qk.qk_act_type(t)
        xq = qk.qk_quantize_act(at, x)
        want.append(qk.qk_gemv(t, W, n_out, n_in, xq, nc).clone())
        bufs.append((t, n_out, n_in, nc, W, x, at))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    outs = [[] for _ in cases]
    for rep in range(5):
        for i, (t, n_out, n_in, nc, W, x, at) in enumerate(bufs):
            with torch.cuda.stream(streams[i % 2]):
                xq = qk.qk_quantize_act(at, x)
                outs[i].append(qk.qk_gemv(t, W, n_out, n_in, xq, nc))
    torch.cuda.synchronize()
    for i, (t, n_out, n_in, nc, *_rest) in enumerate(bufs):
        say("two streams", t, n_out, n_in, nc)
        for y in outs[i]:
            assert torch.equal(y.view(torch.int32), want[i].view(torch.int32)), (t, n_out, n_in, nc)


def test_graph_capture_replays_match_eager(torch_cuda):
    # quantize + GEMV captured into a HIP graph; several replays, with eager work
    # and synchronizations between them, must each equal the eager result.
    torch = torch_cuda
    rng = np.random.default_rng(9)
    cases = [(T4K, 64, 11008, 1), (T4K, 300, 4096, 1), (T6K, 70, 4096, 1), (T8_0, 50, 4096, 1),
             (T4_0, 33, 1024, 1), (T5_0, 41, 4096, 1), (T4K, 200, 4096, 16),
             (T4K, 90, 2048, 64), (T5K, 57, 11008, 1), (T5K, 40, 4096, 3), (T6K, 48, 4096, 4), (T5_0, 36, 2048, 3),
             # more rows than the row-walking grid has wavefronts: each walks several
             (T6K, 7000, 4096, 1), (T4K, 6500, 2048, 1), (T8_0, 5000, 1024, 1)]
    bufs = []
    for t, n_out, n_in, nc in cases:
        W = dev(torch, weights(rng, t, n_out, n_in))
        x = dev(torch, rng.standard_normal((nc, n_in)).astype(np.float32))
        at = qk.qk_act_type(t)
        xq = torch.empty((nc, qk.qk_row_bytes(at, n_in)), dtype=torch.uint8, device="cuda")
        y = torch.empty((nc, n_out), dtype=torch.float32, device="cuda")
        bufs.append((t, n_out, n_in, nc, W, x, at, xq, y))
    want = []
    for t, n_out, n_in, nc, W, x, at, xq, y in bufs:
        qk.qk_quantize_act(at, x, xq)
        want.append(qk.qk_gemv(t, W, n_out, n_in, xq, nc).clone())
    # gate / up pair with the SwiGLU epilogue on the first Q4_K case's activations
    W2p = dev(torch, weights(rng, T4K, 64, 11008))
    hp = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    want_h = qk.qk_gemv_pair(T4K, bufs[0][4], W2p, 64, 11008, bufs[0][7], 1, qk.QK_EPI_SWIGLU).clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t, n_out, n_in, nc, W, x, at, xq, y in bufs:
            qk.qk_quantize_act(at, x, xq)
            qk.qk_gemv(t, W, n_out, n_in, xq, nc, y)
        qk.qk_gemv_pair(T4K, bufs[0][4], W2p, 64, 11008, bufs[0][7], 1, qk.QK_EPI_SWIGLU, hp)
    for rep in range(4):
        for b in bufs:
            b[8].fill_(float("nan"))
            b[7].zero_()
        hp.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (t, n_out, n_in, nc, W, x, at, xq, y), w in zip(bufs, want):
            assert torch.equal(y, w), (rep, t, n_out, n_in, nc)
        assert torch.equal(hp, want_h), rep


def test_native_library_is_the_one_loaded(torch_cuda):
    maps = open("/proc/self/maps").read()
    assert os.path.realpath(qk.LIB_PATH) in maps
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip


# ---------------------------------------------------------------------------
# qk_gemv_pair: gate and up in one launch, optional SwiGLU epilogue
# ---------------------------------------------------------------------------

SILU_SLOPE = 1.0998  # max |d/dv v*sigmoid(v)|


def silu64(v):
    v = v.astype(np.float64)
    with np.errstate(over="ignore"):  # e^-v = inf for very negative v gives the limit 0
        return v / (1.0 + np.exp(-v))


def assert_swiglu(h_gpu, g_o, u_o, l1g, l1u, what):
    """|h_gpu - silu(g)u| within what the R12 bounds on g and u allow, plus a few
    f32 roundings of the epilogue itself."""
    h_o = orc.swiglu(g_o, u_o)
    dg, du = Y_TOL * l1g, Y_TOL * l1u
    bound = (SILU_SLOPE * (np.abs(u_o) + du) * dg + (np.abs(silu64(g_o)) + SILU_SLOPE * dg) * du
             + 8 * 2.0 ** -24 * np.abs(h_o) + 1e-30)
    hg = h_gpu.astype(np.float64)
    fin = np.isfinite(h_o) & np.isfinite(bound)
    same = (hg[~fin] == h_o[~fin]) | (np.isnan(hg[~fin]) & np.isnan(h_o[~fin]))
    assert same.all(), f"{what}: {int((~same).sum())} non-finite oracle outputs not reproduced"
    err = np.abs(hg[fin] - h_o[fin])
    bad = ~(err <= bound[fin])  # NaN in err counts as a failure
    worst = np.max(err / bound[fin], initial=0.0)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond the bound (worst {worst:.3g})"


PAIR_SHAPES = [(1, 256), (7, 4096), (130, 4096), (33, 8192), (9, 11008), (5, 28672)]


@pytest.mark.parametrize("t", [T4K, T5K])
@pytest.mark.parametrize("n_out,n_in", PAIR_SHAPES)
def test_gemv_pair_and_swiglu(torch_cuda, n_out, n_in, t):
    rng = np.random.default_rng(600 + n_out + n_in + t)
    for ncols in (1, 3):
        say("gemv_pair", t, n_out, n_in, ncols)
        W1 = synth.weight_blocks(rng, t, n_out, n_in)
        W2 = synth.weight_blocks(rng, t, n_out, n_in)
        X = rng.standard_normal((ncols, n_in)).astype(np.float32)
        xq = orc.quantize(T8K, X)
        W1d, W2d, xd = dev(torch_cuda, W1), dev(torch_cuda, W2), dev(torch_cuda, xq)
        pair = host(qk.qk_gemv_pair(t, W1d, W2d, n_out, n_in, xd, ncols))
        g_o, l1g = orc.gemv(t, W1, n_out, n_in, xq, ncols)
        u_o, l1u = orc.gemv(t, W2, n_out, n_in, xq, ncols)
        assert_y(pair[:, 0], g_o, l1g, f"pair y1 {n_out}x{n_in} ncols {ncols}")
        assert_y(pair[:, 1], u_o, l1u, f"pair y2 {n_out}x{n_in} ncols {ncols}")
        if ncols == 1:  # the one-column GEMV kernels' own arithmetic
            assert np.array_equal(pair[:, 0], host(qk.qk_gemv(t, W1d, n_out, n_in, xd, 1)))
            assert np.array_equal(pair[:, 1], host(qk.qk_gemv(t, W2d, n_out, n_in, xd, 1)))
        h = host(qk.qk_gemv_pair(t, W1d, W2d, n_out, n_in, xd, ncols, qk.QK_EPI_SWIGLU))
        assert h.shape == (ncols, n_out)
        assert_swiglu(h, g_o, u_o, l1g, l1u, f"swiglu {n_out}x{n_in} ncols {ncols}")


def test_swiglu_extreme_gates(torch_cuda):
    # gates far into both tails: e^-g overflows to inf (h -> -0) or vanishes (h -> g u)
    say("swiglu extreme gates")
    rng = np.random.default_rng(610)
    n_out, n_in = 64, 512
    W1 = synth.q4_K_blocks(rng, n_out, n_in, d_range=(0.5, 2.0))   # large |g|
    W2 = synth.q4_K_blocks(rng, n_out, n_in)
    X = rng.standard_normal((1, n_in)).astype(np.float32) * 40
    xq = orc.quantize(T8K, X)
    h = host(qk.qk_gemv_pair(T4K, dev(torch_cuda, W1), dev(torch_cuda, W2), n_out, n_in,
                             dev(torch_cuda, xq), 1, qk.QK_EPI_SWIGLU))
    g_o, l1g = orc.gemv(T4K, W1, n_out, n_in, xq, 1)
    u_o, l1u = orc.gemv(T4K, W2, n_out, n_in, xq, 1)
    assert np.abs(g_o).max() > 200  # the tails are reached
    assert np.all(np.isfinite(h))
    assert_swiglu(h, g_o, u_o, l1g, l1u, "swiglu extreme gates")


@pytest.mark.parametrize("gt", [T4K, T5K])
def test_ffn_swiglu_step_7b(torch_cuda, gt):
    # the FFN decode step as the library runs it: quantize x, gate + up with the
    # SwiGLU epilogue, quantize h on the GPU, down projection.  Each stage is
    # checked against the oracle on the GPU's own input to that stage.  Gate / up
    # are Q4_K (Q4_K_M layout) or Q5_K (Q5_K_M layout); down is Q6_K in both.
    torch = torch_cuda
    d = synth.ffn_7b() if gt == T4K else synth.ffn_7b_q5_K()
    say("FFN step 7B: gate/up pair", gt)
    x = d["x"][None, :]
    xq = qk.qk_quantize_act(T8K, dev(torch, x))
    assert np.array_equal(host(xq), orc.quantize(T8K, x))
    h = qk.qk_gemv_pair(gt, dev(torch, d["gate"]), dev(torch, d["up"]), 11008, 4096, xq, 1,
                        qk.QK_EPI_SWIGLU)
    xq_h = host(xq)
    g_o, l1g = orc.gemv(gt, d["gate"], 11008, 4096, xq_h, 1)
    u_o, l1u = orc.gemv(gt, d["up"], 11008, 4096, xq_h, 1)
    h_host = host(h)
    assert_swiglu(h_host, g_o, u_o, l1g, l1u, "FFN h")
    say("FFN step 7B: quantize h, down")
    hq = qk.qk_quantize_act(T8K, h)
    hq_o = orc.quantize(T8K, h_host)
    assert np.array_equal(host(hq), hq_o)
    y = host(qk.qk_gemv(T6K, dev(torch, d["down"]), 4096, 11008, hq, 1))
    y_o, l1 = orc.gemv(T6K, d["down"], 4096, 11008, hq_o, 1)
    assert_y(y, y_o, l1, "FFN down")


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times.
# ---------------------------------------------------------------------------

def _check_full(torch, t, W, n_out, n_in, X, what=""):
    """GEMV over the full matrix on the GPU, every output and every per-block sum
    against the oracle."""
    at = orc.act_type(t)
    ncols = X.shape[0]
    xq_gpu = qk.qk_quantize_act(at, dev(torch, X))
    xq = orc.quantize(at, X)
    assert np.array_equal(host(xq_gpu), xq), what
    Wd = dev(torch, W)
    y = host(qk.qk_gemv(t, Wd, n_out, n_in, xq_gpu, ncols))
    y_o, l1 = _oracle_gemv(t, W, n_out, n_in, xq, ncols)
    assert_y(y, y_o, l1, what)
    sums = host(qk.qk_gemv_block_sums(t, Wd, n_out, n_in, xq_gpu, ncols))
    want = _oracle_sums(t, W, xq, n_out, n_in, ncols)
    assert np.array_equal(sums, want.reshape(sums.shape)), what
    return y


def test_full_q8_0_256x1024(torch_cuda):
    say("full Q8_0 256x1024")
    d = synth.q8_0_gemv_256x1024()
    # the weights are quantized on each side by its own quantizer
    Wg = host(qk.qk_quantize_act(T8_0, dev(torch_cuda, d["W_f32"])))
    W = orc.quantize(orc.Q8_0, d["W_f32"])
    assert np.array_equal(Wg, W)
    _check_full(torch_cuda, T8_0, W, 256, 1024, d["x"][None, :], what="Q8_0 256x1024")


def test_full_q4_0_and_q4_K_4096x4096(torch_cuda):
    d = synth.q4_gemv_4096x4096()
    say("full Q4_0 4096x4096")
    _check_full(torch_cuda, T4_0, d["W_q4_0"], 4096, 4096, d["x"][None, :], what="Q4_0 4096^2")
    say("full Q4_K 4096x4096")
    _check_full(torch_cuda, T4K, d["W_q4_K"], 4096, 4096, d["x"][None, :], what="Q4_K 4096^2")


def test_full_q5_0_4096x4096(torch_cuda):
    d = synth.q5_0_gemv_4096x4096()
    say("full Q5_0 4096x4096")
    _check_full(torch_cuda, T5_0, d["W"], 4096, 4096, d["x"][None, :], what="Q5_0 4096^2")


def test_full_ffn_7b(torch_cuda):
    d = synth.ffn_7b()
    say("full FFN gate/up Q4_K 11008x4096")
    _check_full(torch_cuda, T4K, d["gate"], 11008, 4096, d["x"][None, :], what="gate")
    _check_full(torch_cuda, T4K, d["up"], 11008, 4096, d["x"][None, :], what="up")
    say("full FFN down Q6_K 4096x11008")
    _check_full(torch_cuda, T6K, d["down"], 4096, 11008, d["x2"][None, :], what="down")


def test_full_q6_K_head_and_dequantize(torch_cuda):
    d = synth.q6_K_head_32000x4096()
    say("full Q6_K head 32000x4096")
    _check_full(torch_cuda, T6K, d["W"], 32000, 4096, d["x"][None, :], what="Q6_K head")
    say("full Q6_K dequantize 32000x4096")
    Wd = dev(torch_cuda, d["W"])
    out = qk.qk_dequantize_row(T6K, Wd, 32000 * 4096)
    rb = orc.row_bytes(orc.Q6_K, 4096)
    for r0 in range(0, 32000, 4000):
        want = orc.dequantize(orc.Q6_K, d["W"][r0:r0 + 4000].reshape(-1), 4000 * 4096)
        got = host(out[r0 * 4096:(r0 + 4000) * 4096])
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), r0
    del rb


@pytest.mark.parametrize("ncols", [16, 64])
def test_full_q4_K_batched_14336x4096(torch_cuda, ncols):
    d = synth.q4_K_batched_14336x4096()
    say("full Q4_K batched 14336x4096", ncols)
    _check_full(torch_cuda, T4K, d["W"], 14336, 4096, d["X"][:ncols], what=f"Q4_K batched {ncols}")


def test_full_q5_K_decode_4096x11008(torch_cuda):
    d = synth.q5_K_decode_4096x11008()
    say("full Q5_K 4096x11008")
    _check_full(torch_cuda, T5K, d["W"], 4096, 11008, d["x"][None, :], what="Q5_K 4096x11008")


def test_q5_K_extreme_codes(torch_cuda):
    # every code 31 (all nibbles and fifth bits set) and largest 6-bit scales and
    # mins against activations of +-127: the largest |S_q| and |S_m| the format
    # can produce, computed exactly.
    rng = np.random.default_rng(55)
    n_out, n_in = 19, 11008
    W = weights(rng, T5K, n_out, n_in).reshape(n_out, -1, 176).copy()
    W[:, :, 4:16] = 0xFF
    W[:, :, 16:176] = 0xFF
    W[::2, :, 16:48] = 0x00  # half the rows: fifth bits clear (codes 15)
    W = W.reshape(n_out, -1)
    X = np.where(rng.random((2, n_in)) < 0.5, 127.0, -127.0).astype(np.float32)
    X[1] = 127.0
    xq = orc.quantize(orc.Q8_K, X)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    for ncols in (1, 2):
        say("Q5_K extreme codes", ncols)
        sums = host(qk.qk_gemv_block_sums(T5K, Wd, n_out, n_in, xd, ncols))
        want = _oracle_sums(T5K, W, xq, n_out, n_in, ncols).reshape(sums.shape)
        assert np.array_equal(sums, want)
        y = host(qk.qk_gemv(T5K, Wd, n_out, n_in, xd, ncols))
        y_o, l1 = orc.gemv(T5K, W, n_out, n_in, xq, ncols)
        assert_y(y, y_o, l1, "Q5_K extreme codes")


# Q8_0, Q4_0, Q5_0, Q5_K and Q6_K with several columns: the multi-column GEMV
# kernels in groups of up to 4 columns (fewer where the rows are too long for 4
# activation rows in LDS: Q8_K rows of 28672 take 2; Q8_0 rows of 11008 take 3, of
# 14336 2, and of 28672 run one column per launch), a ragged last group, one to
# fourteen passes per row and the rows past one workgroup.
SMALL_BATCH = [(37, 2304, 2), (129, 4096, 4), (8300, 256, 5), (45, 11008, 9),
               (3, 28672, 3), (50, 768, 7), (70, 14336, 4)]


@pytest.mark.parametrize("t", [T8_0, T4_0, T5_0, T4_1, T5_1, T2K, T3K, T5K, T6K])
@pytest.mark.parametrize("n_out,n_in,ncols", SMALL_BATCH)
def test_small_batch_gemv_kernels(torch_cuda, t, n_out, n_in, ncols):
    say("small batch", t, n_out, n_in, ncols)
    rng = np.random.default_rng(n_out * 11 + ncols + t)
    W = weights(rng, t, n_out, n_in)
    X = rng.standard_normal((ncols, n_in)).astype(np.float32)
    X[ncols // 2] = 0.0                      # an all-zero column: d = 0, codes 0
    xq = orc.quantize(orc.act_type(t), X)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    sums = host(qk.qk_gemv_block_sums(t, Wd, n_out, n_in, xd, ncols))
    want = _oracle_sums(t, W, xq, n_out, n_in, ncols).reshape(sums.shape)
    assert np.array_equal(sums, want)
    y = host(qk.qk_gemv(t, Wd, n_out, n_in, xd, ncols))
    y_o, l1 = orc.gemv(t, W, n_out, n_in, xq, ncols)
    assert_y(y, y_o, l1, f"small batch type {t} {n_out}x{n_in} ncols {ncols}")
    assert not y[ncols // 2].any()


@pytest.mark.parametrize("t", [T8_0, T4_0, T5_0])
def test_q80_family_extreme_codes(torch_cuda, t):
    # the ends of each code range (Q8_0 -128 / +127, Q4_0 -8 / +7, Q5_0 -16 / +15)
    # against activations of +-127, one to four columns: the largest block sums
    # the 32-element formats can produce, and the signed-byte conversion of the
    # multi-column kernel at both ends.
    rng = np.random.default_rng(57)
    n_out, n_in = 21, 4096
    bb = {T8_0: 34, T4_0: 18, T5_0: 22}[t]
    W = weights(rng, t, n_out, n_in).reshape(n_out, -1, bb).copy()
    if t == T8_0:
        W[0::2, :, 2:] = 0x80
        W[1::2, :, 2:] = 0x7F
    else:
        W[0::2, :, 2:] = 0xFF                # Q5_0: qh set too, code 31
        W[1::2, :, 2:] = 0x00
    W = W.reshape(n_out, -1)
    X = np.where(rng.random((4, n_in)) < 0.5, 127.0, -127.0).astype(np.float32)
    X[1] = 127.0
    X[2] = -127.0
    xq = orc.quantize(orc.Q8_0, X)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    for ncols in (1, 2, 3, 4):
        say("extreme codes", t, ncols)
        sums = host(qk.qk_gemv_block_sums(t, Wd, n_out, n_in, xd, ncols))
        want = _oracle_sums(t, W, xq, n_out, n_in, ncols).reshape(sums.shape)
        assert np.array_equal(sums, want)
        y = host(qk.qk_gemv(t, Wd, n_out, n_in, xd, ncols))
        y_o, l1 = orc.gemv(t, W, n_out, n_in, xq, ncols)
        assert_y(y, y_o, l1, f"type {t} extreme codes")


@pytest.mark.parametrize("t", [T4_1, T5_1])
def test_q4_1_q5_1_extreme_codes(torch_cuda, t):
    # the ends of each code range (Q4_1 0 / 15, Q5_1 0 / 31) against activations of
    # +-127, with negative and positive minimums: the largest block sums these
    # formats produce, and the minimum term against the Q8_1 sum field at its ends.
    rng = np.random.default_rng(58)
    n_out, n_in = 22, 4096
    bb = {T4_1: 20, T5_1: 24}[t]
    W = weights(rng, t, n_out, n_in).reshape(n_out, -1, bb).copy()
    W[0::2, :, 4:] = 0xFF                    # Q5_1: qh set too, code 31
    W[1::2, :, 4:] = 0x00
    W[2::4, :, 2:4] = np.frombuffer(np.float16(0.02).tobytes(), np.uint8)
    W = W.reshape(n_out, -1)
    X = np.where(rng.random((3, n_in)) < 0.5, 127.0, -127.0).astype(np.float32)
    X[1] = 127.0
    X[2] = -127.0
    xq = orc.quantize(T8_1, X)
    assert np.array_equal(host(qk.qk_quantize_act(T8_1, dev(torch_cuda, X))), xq)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    for ncols in (1, 3):
        say("Q4_1 / Q5_1 extreme codes", t, ncols)
        sums = host(qk.qk_gemv_block_sums(t, Wd, n_out, n_in, xd, ncols))
        want = _oracle_sums(t, W, xq, n_out, n_in, ncols).reshape(sums.shape)
        assert np.array_equal(sums, want)
        y = host(qk.qk_gemv(t, Wd, n_out, n_in, xd, ncols))
        y_o, l1 = orc.gemv(t, W, n_out, n_in, xq, ncols)
        assert_y(y, y_o, l1, f"type {t} extreme codes")


@pytest.mark.parametrize("t", [T2K, T3K])
def test_q2_K_q3_K_extreme_codes(torch_cuda, t):
    # codes at both ends (Q2_K 0 / 3, Q3_K -4 / +3), the largest scales and mins (Q2_K
    # nibbles 15; Q3_K scale fields 0 and 63, i.e. -32 and +31) against activations of
    # +-127: the largest |S| these formats produce, exactly.
    rng = np.random.default_rng(59)
    n_out, n_in = 24, 11008
    bb = {T2K: 84, T3K: 110}[t]
    W = weights(rng, t, n_out, n_in).reshape(n_out, -1, bb).copy()
    if t == T2K:
        W[:, :, 0:16] = 0xFF                 # scale 15, min 15
        W[0::2, :, 16:80] = 0xFF             # code 3
        W[1::2, :, 16:80] = 0x00             # code 0
    else:
        W[0::2, :, 0:96] = 0xFF              # code 7 - 4 = +3
        W[1::2, :, 0:96] = 0x00              # code -4
        W[0::4, :, 96:108] = 0xFF            # scale 63 - 32 = +31
        W[1::4, :, 96:108] = 0x00            # scale -32
    W = W.reshape(n_out, -1)
    X = np.where(rng.random((3, n_in)) < 0.5, 127.0, -127.0).astype(np.float32)
    X[1] = 127.0
    X[2] = -127.0
    xq = orc.quantize(orc.Q8_K, X)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    for ncols in (1, 3):
        say("Q2_K / Q3_K extreme codes", t, ncols)
        sums = host(qk.qk_gemv_block_sums(t, Wd, n_out, n_in, xd, ncols))
        want = _oracle_sums(t, W, xq, n_out, n_in, ncols).reshape(sums.shape)
        assert np.array_equal(sums, want)
        y = host(qk.qk_gemv(t, Wd, n_out, n_in, xd, ncols))
        y_o, l1 = orc.gemv(t, W, n_out, n_in, xq, ncols)
        assert_y(y, y_o, l1, f"type {t} extreme codes")


def test_q6_K_extreme_codes(torch_cuda):
    # codes 63 and 0 (q - 32 = 31 and -32) with scales +127 and -128 against
    # activations of +-127: the largest |S| the format can produce, exactly.
    rng = np.random.default_rng(56)
    n_out, n_in = 23, 11008
    W = weights(rng, T6K, n_out, n_in).reshape(n_out, -1, 210).copy()
    W[:, :, 0:192] = 0xFF                    # every code 63
    W[1::2, :, 0:192] = 0x00                 # odd rows: every code 0
    W[:, :, 192:208] = np.where(np.arange(16) % 2 == 0, 0x7F, 0x80).astype(np.uint8)
    W = W.reshape(n_out, -1)
    X = np.where(rng.random((3, n_in)) < 0.5, 127.0, -127.0).astype(np.float32)
    X[1] = 127.0
    X[2] = -127.0
    xq = orc.quantize(orc.Q8_K, X)
    Wd, xd = dev(torch_cuda, W), dev(torch_cuda, xq)
    for ncols in (1, 2, 3):
        say("Q6_K extreme codes", ncols)
        sums = host(qk.qk_gemv_block_sums(T6K, Wd, n_out, n_in, xd, ncols))
        want = _oracle_sums(T6K, W, xq, n_out, n_in, ncols).reshape(sums.shape)
        assert np.array_equal(sums, want)
        y = host(qk.qk_gemv(T6K, Wd, n_out, n_in, xd, ncols))
        y_o, l1 = orc.gemv(T6K, W, n_out, n_in, xq, ncols)
        assert_y(y, y_o, l1, "Q6_K extreme codes")


@pytest.mark.parametrize("ncols", [2, 16, 64])
def test_q4_K_batched_4096x11008(torch_cuda, ncols):
    # few rows and long rows: the 16-row workgroup shapes of the batched kernel
    d = synth.q4_K_decode_4096x11008()
    rng = np.random.default_rng(45)
    X = rng.standard_normal((ncols, 11008)).astype(np.float32)
    say("batched Q4_K 4096x11008", ncols)
    _check_full(torch_cuda, T4K, d["W"], 4096, 11008, X, what=f"Q4_K 4096x11008 x {ncols}")


def test_full_q2_K_and_q3_K_decode_4096x11008(torch_cuda):
    for t, d in ((T2K, synth.q2_K_decode_4096x11008()), (T3K, synth.q3_K_decode_4096x11008())):
        say("full", qk.TYPE_NAMES[t], "4096x11008")
        _check_full(torch_cuda, t, d["W"], 4096, 11008, d["x"][None, :], what=f"{qk.TYPE_NAMES[t]} 4096x11008")


def test_full_q4_1_and_q5_1_decode_4096x11008(torch_cuda):
    for t, d in ((T4_1, synth.q4_1_decode_4096x11008()), (T5_1, synth.q5_1_decode_4096x11008())):
        say("full", qk.TYPE_NAMES[t], "4096x11008")
        _check_full(torch_cuda, t, d["W"], 4096, 11008, d["x"][None, :], what=f"{qk.TYPE_NAMES[t]} 4096x11008")


def test_full_q4_K_decode_4096x11008(torch_cuda):
    d = synth.q4_K_decode_4096x11008()
    say("full Q4_K 4096x11008")
    _check_full(torch_cuda, T4K, d["W"], 4096, 11008, d["x"][None, :], what="Q4_K 4096x11008")
