"""Seeded synthetic inputs (numpy) for the GEMV workloads.

This module only draws random numbers and lays them into the GGUF block byte
layouts; it holds none of the method's arithmetic (no quantization, no
dequantization, no dot products).  Tests feed the same arrays to the CPU oracle
and to the HIP library; the benchmark uses them for its weight copies.

Recipes (one numpy default_rng(seed) per workload, drawn in the order listed):
  f16 fields "U[a, b]": f64 uniform draw, rounded to f16 (numpy, RNE).
  "uniform bytes": every byte iid U{0..255}, so Q4_K's and Q5_K's 6-bit
  scales/mins, nibbles and fifth bits are uniform; Q6_K scales int8 U{-64..63}
  inclusive.
"""
import numpy as np

Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q8_1 = 2, 3, 6, 7, 8, 9
Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, Q8_K = 10, 11, 12, 13, 14, 15
BLOCK_ELEMS = {Q4_0: 32, Q4_1: 32, Q5_0: 32, Q5_1: 32, Q8_0: 32, Q8_1: 32, Q2_K: 256, Q3_K: 256,
               Q4_K: 256, Q5_K: 256, Q6_K: 256, Q8_K: 256}
BLOCK_BYTES = {Q4_0: 18, Q4_1: 20, Q5_0: 22, Q5_1: 24, Q8_0: 34, Q8_1: 36, Q2_K: 84, Q3_K: 110,
               Q4_K: 144, Q5_K: 176, Q6_K: 210, Q8_K: 292}


def uniform_bytes(rng, shape):
    """iid U{0..255} bytes, cut from full-range uint32 draws (exactly uniform)."""
    count = int(np.prod(shape))
    words = rng.integers(0, 2**32, size=(count + 3) // 4, dtype=np.uint32)
    return words.view(np.uint8)[:count].reshape(shape).copy()


def uniform_int8(rng, shape, lo, hi):
    """iid integers U{lo..hi} with hi - lo + 1 a power of two dividing 2^32."""
    span = hi - lo + 1
    words = rng.integers(0, 2**32, size=shape, dtype=np.uint32)
    return ((words % np.uint32(span)).astype(np.int32) + lo).astype(np.int8)


def _f16_bytes(vals):
    return np.ascontiguousarray(vals.astype(np.float16)).view(np.uint8).reshape(*vals.shape, 2)


def q4_0_blocks(rng, n_out, n_in, d_range=(1e-3, 4e-3)):
    """Q4_0 rows: f16 d ~ U[d_range], 16 uniform qs bytes per block."""
    nb = n_in // 32
    b = uniform_bytes(rng, (n_out, nb, 18))
    b[:, :, 0:2] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 18)


def q4_1_blocks(rng, n_out, n_in, d_range=(1e-3, 4e-3), m_range=(-0.03, -0.005)):
    """Q4_1 rows: f16 d ~ U[d_range], f16 m ~ U[m_range], 16 uniform qs bytes."""
    nb = n_in // 32
    b = uniform_bytes(rng, (n_out, nb, 20))
    b[:, :, 0:2] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    b[:, :, 2:4] = _f16_bytes(rng.uniform(*m_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 20)


def q5_1_blocks(rng, n_out, n_in, d_range=(5e-4, 2e-3), m_range=(-0.03, -0.005)):
    """Q5_1 rows: f16 d ~ U[d_range], f16 m ~ U[m_range]; the 4 qh and 16 qs bytes uniform."""
    nb = n_in // 32
    b = uniform_bytes(rng, (n_out, nb, 24))
    b[:, :, 0:2] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    b[:, :, 2:4] = _f16_bytes(rng.uniform(*m_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 24)


def q5_0_blocks(rng, n_out, n_in, d_range=(5e-4, 2e-3)):
    """Q5_0 rows: f16 d ~ U[d_range]; the 4 qh bytes and 16 qs bytes uniform."""
    nb = n_in // 32
    b = uniform_bytes(rng, (n_out, nb, 22))
    b[:, :, 0:2] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 22)


def q4_K_blocks(rng, n_out, n_in, d_range=(1e-4, 1e-3)):
    """Q4_K rows: f16 d, dmin ~ U[d_range]; 12 scale bytes and 128 qs bytes uniform."""
    nb = n_in // 256
    b = uniform_bytes(rng, (n_out, nb, 144))
    b[:, :, 0:2] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    b[:, :, 2:4] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 144)


def q5_K_blocks(rng, n_out, n_in, d_range=(1e-4, 1e-3)):
    """Q5_K rows: f16 d, dmin ~ U[d_range]; 12 scale, 32 qh and 128 qs bytes uniform."""
    nb = n_in // 256
    b = uniform_bytes(rng, (n_out, nb, 176))
    b[:, :, 0:2] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    b[:, :, 2:4] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 176)


def q6_K_blocks(rng, n_out, n_in, d_range=(1e-4, 1e-3)):
    """Q6_K rows: ql/qh bytes uniform, int8 scales ~ U{-64..63}, f16 d ~ U[d_range]."""
    nb = n_in // 256
    b = uniform_bytes(rng, (n_out, nb, 210))
    b[:, :, 192:208] = uniform_int8(rng, (n_out, nb, 16), -64, 63).view(np.uint8)
    b[:, :, 208:210] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 210)


def q2_K_blocks(rng, n_out, n_in, d_range=(1e-4, 1e-3)):
    """Q2_K rows: 16 scale bytes and 64 qs bytes uniform, f16 d, dmin ~ U[d_range]."""
    nb = n_in // 256
    b = uniform_bytes(rng, (n_out, nb, 84))
    b[:, :, 80:82] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    b[:, :, 82:84] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 84)


def q3_K_blocks(rng, n_out, n_in, d_range=(1e-4, 1e-3)):
    """Q3_K rows: hmask, qs and scale bytes uniform, f16 d ~ U[d_range]."""
    nb = n_in // 256
    b = uniform_bytes(rng, (n_out, nb, 110))
    b[:, :, 108:110] = _f16_bytes(rng.uniform(*d_range, size=(n_out, nb)))
    return b.reshape(n_out, nb * 110)


def weight_blocks(rng, t, n_out, n_in):
    return {Q4_0: q4_0_blocks, Q4_1: q4_1_blocks, Q5_0: q5_0_blocks, Q5_1: q5_1_blocks,
            Q2_K: q2_K_blocks, Q3_K: q3_K_blocks, Q4_K: q4_K_blocks, Q5_K: q5_K_blocks,
            Q6_K: q6_K_blocks}[t](rng, n_out, n_in)


def gaussian(rng, shape, std=1.0):
    return (rng.standard_normal(size=shape) * std).astype(np.float32)


# ---------------------------------------------------------------------------
# Named workloads.  Each returns a dict of numpy arrays; "W_f32" entries are f32
# weights still to be quantized (Q8_0), "W" entries are finished block bytes.
# ---------------------------------------------------------------------------

def q8_0_gemv_256x1024():
    """Q8_0 GEMV 256x1024: W f32 ~N(0, 0.02) to be quantized to Q8_0; x ~N(0,1)."""
    rng = np.random.default_rng(0)
    return {"W_f32": gaussian(rng, (256, 1024), 0.02), "x": gaussian(rng, (1024,))}


def q4_gemv_4096x4096():
    """Q4_0 and Q4_K GEMV 4096x4096; x ~N(0,1)[4096]."""
    rng = np.random.default_rng(1)
    w40 = q4_0_blocks(rng, 4096, 4096)
    w4k = q4_K_blocks(rng, 4096, 4096)
    return {"W_q4_0": w40, "W_q4_K": w4k, "x": gaussian(rng, (4096,))}


def ffn_7b():
    """7B-shape FFN: gate, up Q4_K 11008x4096; down Q6_K 4096x11008; x[4096], x2[11008]."""
    rng = np.random.default_rng(2)
    gate = q4_K_blocks(rng, 11008, 4096)
    up = q4_K_blocks(rng, 11008, 4096)
    down = q6_K_blocks(rng, 4096, 11008)
    return {"gate": gate, "up": up, "down": down, "x": gaussian(rng, (4096,)),
            "x2": gaussian(rng, (11008,))}


def ffn_7b_q5_K():
    """7B-shape FFN as a Q5_K_M file stores it: gate, up Q5_K 11008x4096; down Q6_K
    4096x11008; x[4096], x2[11008]."""
    rng = np.random.default_rng(9)
    gate = q5_K_blocks(rng, 11008, 4096)
    up = q5_K_blocks(rng, 11008, 4096)
    down = q6_K_blocks(rng, 4096, 11008)
    return {"gate": gate, "up": up, "down": down, "x": gaussian(rng, (4096,)),
            "x2": gaussian(rng, (11008,))}


def q6_K_head_32000x4096():
    """Q6_K output head 32000x4096; x[4096]."""
    rng = np.random.default_rng(3)
    return {"W": q6_K_blocks(rng, 32000, 4096), "x": gaussian(rng, (4096,))}


def q5_0_gemv_4096x4096():
    """Q5_0 GEMV 4096x4096 (Q8_0 activations); x ~N(0,1)[4096]."""
    rng = np.random.default_rng(6)
    return {"W": q5_0_blocks(rng, 4096, 4096), "x": gaussian(rng, (4096,))}


def f32_weights_4096x11008():
    """f32 weights N(0, 0.02) [4096, 11008], to be quantized to GGUF blocks."""
    rng = np.random.default_rng(7)
    return {"W_f32": gaussian(rng, (4096, 11008), 0.02)}


def q4_K_batched_14336x4096():
    """Q4_K 14336x4096 with 64 token columns X[64, 4096] (16-column case = first 16)."""
    rng = np.random.default_rng(4)
    return {"W": q4_K_blocks(rng, 14336, 4096), "X": gaussian(rng, (64, 4096))}


def q4_K_decode_4096x11008(seed=5):
    """Q4_K decode GEMV, 4096 rows x 11008 columns (43 superblocks per row); x[11008]."""
    rng = np.random.default_rng(seed)
    return {"W": q4_K_blocks(rng, 4096, 11008), "x": gaussian(rng, (11008,))}


def q4_1_decode_4096x11008(seed=9):
    """Q4_1 GEMV, 4096 rows x 11008 columns (344 blocks per row, Q8_1 activations); x[11008]."""
    rng = np.random.default_rng(seed)
    return {"W": q4_1_blocks(rng, 4096, 11008), "x": gaussian(rng, (11008,))}


def q5_1_decode_4096x11008(seed=10):
    """Q5_1 GEMV, 4096 rows x 11008 columns (344 blocks per row, Q8_1 activations); x[11008]."""
    rng = np.random.default_rng(seed)
    return {"W": q5_1_blocks(rng, 4096, 11008), "x": gaussian(rng, (11008,))}


def q2_K_decode_4096x11008(seed=11):
    """Q2_K decode GEMV, 4096 rows x 11008 columns (43 superblocks per row); x[11008]."""
    rng = np.random.default_rng(seed)
    return {"W": q2_K_blocks(rng, 4096, 11008), "x": gaussian(rng, (11008,))}


def q3_K_decode_4096x11008(seed=12):
    """Q3_K decode GEMV, 4096 rows x 11008 columns (43 superblocks per row); x[11008]."""
    rng = np.random.default_rng(seed)
    return {"W": q3_K_blocks(rng, 4096, 11008), "x": gaussian(rng, (11008,))}


def q5_K_decode_4096x11008(seed=8):
    """Q5_K decode GEMV, 4096 rows x 11008 columns (43 superblocks per row); x[11008]."""
    rng = np.random.default_rng(seed)
    return {"W": q5_K_blocks(rng, 4096, 11008), "x": gaussian(rng, (11008,))}


def random_copies(t, n_out, n_in, count, seed):
    """`count` independent weight matrices of one shape (for cache rotation)."""
    rng = np.random.default_rng(seed)
    return [weight_blocks(rng, t, n_out, n_in) for _ in range(count)]
