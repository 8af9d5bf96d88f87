"""Pins of the CPU oracle against what the pages fix (no GPU needed).

Every check here compares the oracle with something other than itself: values
printed on the pages (tests/golden/, each file citing its page and section),
a library routine for a textbook case (numpy's IEEE binary16 conversion),
structural properties the pages state in prose, and f64 brute force on tiny
rows.  Sources are cited by page title and section.
"""
import math

import numpy as np
import pytest

from golden_io import keyvals, rows
from jrandom import JavaRandom
from oracle import oracle as o

F32 = np.float32


# --------------------------------------------------------------------------
# Type table and row geometry
# --------------------------------------------------------------------------

def test_type_table_matches_printed_geometry():
    # candle "量化格式" GgmlDType table; codeloopback lesson format table.  Elements,
    # bytes and bits per weight are printed there; the id column is a reading (the
    # pages say the ids follow ggml's enum without printing them), so it is checked
    # for consistency with the oracle's constants only, not as a pin.
    ids = {"Q4_0": o.Q4_0, "Q4_1": o.Q4_1, "Q5_0": o.Q5_0, "Q5_1": o.Q5_1, "Q8_0": o.Q8_0, "Q2_K": o.Q2_K,
           "Q3_K": o.Q3_K, "Q4_K": o.Q4_K, "Q5_K": o.Q5_K, "Q6_K": o.Q6_K, "Q8_K": o.Q8_K}
    for name, gid, elems, nbytes, bpw in rows("type_table.txt"):
        t = ids[name]
        assert o.block_elems(t) == int(elems)
        assert o.block_bytes(t) == int(nbytes)
        assert f"{o.block_bytes(t) * 8 / o.block_elems(t):.4f}" == bpw


def test_type_ids_reading_is_consistent():
    # reading, not a pin: the GGUF enum values used as ids (type_table.txt header)
    ids = {"Q4_0": o.Q4_0, "Q4_1": o.Q4_1, "Q5_0": o.Q5_0, "Q5_1": o.Q5_1, "Q8_0": o.Q8_0, "Q2_K": o.Q2_K,
           "Q3_K": o.Q3_K, "Q4_K": o.Q4_K, "Q5_K": o.Q5_K, "Q6_K": o.Q6_K, "Q8_K": o.Q8_K}
    for name, gid, _, _, _ in rows("type_table.txt"):
        assert ids[name] == int(gid)


def test_row_bytes_whole_blocks_no_padding():
    # codeloopback Example 9: 64 x 4096 tensor is 278,528 B in Q8_0 and 147,456 B in
    # Q4_0; row strides 4352 and 2304.  Example 15: a 100-element row is rejected.
    assert 64 * o.row_bytes(o.Q8_0, 4096) == 278528
    assert 64 * o.row_bytes(o.Q4_0, 4096) == 147456
    assert o.row_bytes(o.Q8_0, 4096) == 4352
    assert o.row_bytes(o.Q4_0, 4096) == 2304
    assert o.row_bytes(o.Q4_0, 100) == 0
    assert o.row_bytes(o.Q4_K, 11008) == 43 * 144
    assert o.row_bytes(o.Q6_K, 11008) == 43 * 210
    assert o.row_bytes(o.Q5_K, 11008) == 43 * 176
    assert o.row_bytes(o.Q4_K, 4096 + 32) == 0
    assert o.row_bytes(99, 256) == 0


def test_pairing_table():
    # candle VecDotType table; codeloopback Example 11 (Q4_0 -> Q8_0).
    assert o.act_type(o.Q4_0) == o.Q8_0
    assert o.act_type(o.Q8_0) == o.Q8_0
    assert o.act_type(o.Q4_K) == o.Q8_K
    assert o.act_type(o.Q6_K) == o.Q8_K
    assert o.act_type(o.Q5_K) == o.Q8_K
    assert o.act_type(o.Q2_K) == o.Q8_K   # "Q2K 到 Q6K" -> BlockQ8K
    assert o.act_type(o.Q3_K) == o.Q8_K
    assert o.act_type(o.Q8_K) == -1
    # the same table pairs Q4_1 and Q5_1 with BlockQ8_1, an activation-only block
    assert o.act_type(o.Q4_1) == o.Q8_1
    assert o.act_type(o.Q5_1) == o.Q8_1
    assert o.act_type(o.Q8_1) == -1
    assert o.act_type(4) == -1


# --------------------------------------------------------------------------
# binary16 conversion
# --------------------------------------------------------------------------

def test_f16_decode_all_patterns_against_numpy():
    # IEEE 754 binary16 decode is a textbook routine; numpy implements it.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([o.f16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_against_numpy_rne():
    rng = np.random.default_rng(1234)
    # random f32 bit patterns over the whole range, plus every f16 boundary and
    # midpoint (ties), subnormals and overflow edges.
    vals = [rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32)]
    h = np.arange(0, 0x7C01, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2  # exact in f64; the f32 casts below hit ties and neighbours
    m32 = mids.astype(np.float32)
    vals += [h.astype(np.float32), m32, np.nextafter(m32, np.float32(np.inf)),
             np.nextafter(m32, np.float32(0)),
             np.array([65504, 65519.996, 65520, 65536, 1e-8, 2.98e-8, 2.9802322e-8,
                       5.96e-8, 6.1e-5], dtype=np.float32)]
    v = np.concatenate(vals)
    v = np.concatenate([v, -v])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = np.array([o.f32_to_f16(float(x)) for x in v], dtype=np.uint16)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_f16_printed_scales():
    kv = keyvals("q8_0_blocks.txt")
    # codeloopback Example 2: d = 0.011682516 -> f16 0x21FB = 0.011680603.
    assert o.f32_to_f16(float(F32(kv["cl_ex2.d_f32"]))) == int(kv["cl_ex2.d_f16_bits"], 16)
    assert f"{o.f16_to_f32(0x21FB):.9f}" == kv["cl_ex2.d_f16"]
    # candle: [40, 22] -> 0x2240 = 0.012207031.
    assert f"{o.f16_to_f32(0x2240):.9f}" == kv["candle.d"]
    # rml Q4_0 example: 0.25 -> 0x3400; codeloopback Example 14: 9.5 / -8 -> 0xBCC0.
    kq = keyvals("q4_0_blocks.txt")
    assert o.f32_to_f16(0.25) == int(kq["rml.d_f16_bits"], 16)
    assert o.f32_to_f16(float(F32(9.5) / F32(-8))) == int(kq["cl_ex14_read.d_f16_bits"], 16)


# --------------------------------------------------------------------------
# quantize_row_q8_0 / q4_0 against printed bytes
# --------------------------------------------------------------------------

def _cl_inputs(n):
    i = np.arange(n)
    return (((i * 7919) % 1001) - 500).astype(np.float32) / np.float32(337)


def test_q8_0_candle_block():
    kv = keyvals("q8_0_blocks.txt")
    x = (np.arange(32, dtype=np.float32) - F32(15.5)) / F32(10)
    b = o.quantize(o.Q8_0, x)
    assert b[:2].tobytes().hex() == kv["candle.d_bytes_hex"]
    assert [int(c) for c in b[2:].view(np.int8)] == [int(c) for c in kv["candle.qs"].split()]
    back = o.dequantize(o.Q8_0, b, 32)
    assert np.array_equal(back[:4], np.array(kv["candle.back4"].split(), dtype=np.float32))
    assert f"{o.f16_to_f32(int(b[0]) | int(b[1]) << 8):.9f}" == kv["candle.d"]


def test_q8_0_codeloopback_examples_2_3_4():
    kv = keyvals("q8_0_blocks.txt")
    x = _cl_inputs(32)
    b = o.quantize(o.Q8_0, x)
    assert [int(c) for c in b[2:].view(np.int8)] == [int(c) for c in kv["cl_ex2.qs"].split()]
    assert b.tobytes().hex() == kv["cl_ex2.hex"]
    assert f"{np.abs(x).max() / F32(127):.9f}" == kv["cl_ex2.d_f32"]
    y = o.dequantize(o.Q8_0, b, 32)
    assert y[0] == F32(kv["cl_ex2.y0"])  # printed as the shortest f32 repr
    # Example 3: error with the f32 scale and with the stored f16 scale.
    d = np.abs(x).max() / F32(127)
    codes = b[2:].view(np.int8).astype(np.float32)
    err_f32 = np.max(np.abs(codes * d - x).astype(np.float64))
    err_f16 = np.max(np.abs((y - x).astype(np.float64)))
    rmse = 100 * math.sqrt(np.sum((y - x).astype(np.float64) ** 2) / np.sum((x * x).astype(np.float64)))
    assert f"{err_f32:.6f}" == kv["cl_ex3.max_err_f32_d"]
    assert f"{err_f16:.6f}" == kv["cl_ex3.max_err_f16_d"]
    assert f"{rmse:.4f}" == kv["cl_ex3.rel_rmse_pct"]


def test_hex_crosscheck_example_14():
    x = _cl_inputs(64)
    x[40] = F32(9.5)
    types = {"Q8_0": o.Q8_0, "Q4_0": o.Q4_0, "Q4_1": o.Q4_1, "Q5_0": o.Q5_0}
    for blk, name, hexs in rows("hex_crosscheck.txt"):
        blk = int(blk)
        assert o.quantize(types[name], x[32 * blk:32 * blk + 32]).tobytes().hex() == hexs


def _rel_rmse_pct(x, y):
    x64, y64 = x.astype(np.float64), y.astype(np.float64)
    return 100 * math.sqrt(np.sum((y64 - x64) ** 2) / np.sum(x64 * x64))


def test_q4_1_codeloopback_example_7():
    kv = keyvals("q4_1_q5_0_examples.txt")
    centered = _cl_inputs(32)
    shifted = F32(2) + np.abs(centered)
    for name, x in (("centered", centered), ("shifted", shifted)):
        b = o.quantize(o.Q4_1, x)
        assert b.size == 20
        mn, mx = x.min(), x.max()
        assert f"{mn:.3f}" == kv[f"ex7.{name}.min"] and f"{mx:.3f}" == kv[f"ex7.{name}.max"]
        assert f"{(mx - mn) / F32(15):.4f}" == kv[f"ex7.{name}.d"]
        # stored m is the f16 of min; the page prints min itself
        assert f"{mn:.4f}" == kv[f"ex7.{name}.m"]
        assert o.f16_to_f32(int(b[2]) | int(b[3]) << 8) == float(np.float16(mn))
        y = o.dequantize(o.Q4_1, b, 32)
        assert f"{_rel_rmse_pct(x, y):.3f}" == kv[f"ex7.{name}.rmse"]
    assert f"{20 * 8 / 32.0}" == kv["ex7.bpw"]


def test_q5_0_codeloopback_example_8():
    kv = keyvals("q4_1_q5_0_examples.txt")
    x = _cl_inputs(32)
    b = o.quantize(o.Q5_0, x)
    assert b.tobytes().hex() == kv["ex8.block"]
    qh = int.from_bytes(b[2:6].tobytes(), "little")
    assert format(qh, "032b") == kv["ex8.qh_bits"]
    amax_i = int(np.argmax(np.abs(x)))  # first index of the largest magnitude
    assert f"{x[amax_i]:.4f}" == kv["ex8.max"]
    assert f"{x[amax_i] / F32(-16):.5f}" == kv["ex8.d"]
    y = o.dequantize(o.Q5_0, b, 32)
    assert f"{_rel_rmse_pct(x, y):.3f}" == kv["ex8.rmse"]


def test_weight_codes_when_the_inverse_scale_overflows():
    # codeloopback Examples 5, 7, 8 convert codes with the listings' (int) cast:
    # toward zero, saturating, NaN -> 0.  A block of f32 subnormals has a scale
    # below 2^-128, so 1/d is +inf; the bytes below are worked out by hand from
    # that rule: x * inf is +-inf (NaN for x = 0), +inf saturates to the top
    # code, -inf to INT_MIN whose low bits are 0, NaN to 0.
    x = np.zeros(32, np.float32)
    x[0], x[1], x[17] = F32(-1e-39), F32(5e-40), F32(-2e-40)
    q40 = "0000" + "000f" + "00" * 14                 # d -> f16 +0; only x[1] -> 15
    q50 = "0000" + "02000000" + "000f" + "00" * 14    # code 31 for x[1]: qh bit 1
    q41 = "00000080" + "f0" + "ff" * 15               # m = -0; x[0] -> NaN -> 0
    assert o.quantize(o.Q4_0, x).tobytes().hex() == q40
    assert o.quantize(o.Q5_0, x).tobytes().hex() == q50
    assert o.quantize(o.Q4_1, x).tobytes().hex() == q41


def test_q5_0_and_q4_1_each_code_bit_is_one_element():
    # codeloopback Example 8: bit e of qh is the fifth bit of element e; a nibble of
    # byte j holds element j (low) or j + 16 (high), as Q4_0.  Flipping any one code
    # bit must move exactly one element, by d * 2^k (Q5_0) or d * 2^k (Q4_1).
    rng = np.random.default_rng(9)
    for t, qs_off, hdr in ((o.Q5_0, 6, 22), (o.Q4_1, 4, 20)):
        b = rng.integers(0, 256, hdr, dtype=np.uint8)
        b[0:2] = np.frombuffer(np.float16(0.25).tobytes(), np.uint8)
        if t == o.Q4_1:
            b[2:4] = np.frombuffer(np.float16(-1.0).tobytes(), np.uint8)
        base = o.dequantize(t, b, 32).astype(np.float64)
        seen = set()
        bits = [(j, k) for j in range(qs_off, hdr) for k in range(8)]
        if t == o.Q5_0:
            bits += [(j, k) for j in range(2, 6) for k in range(8)]
        for j, k in bits:
            c = b.copy()
            c[j] ^= np.uint8(1 << k)
            d = o.dequantize(t, c, 32).astype(np.float64) - base
            moved = np.nonzero(d)[0]
            assert moved.size == 1, (t, j, k)
            e = int(moved[0])
            if j >= qs_off:  # nibble bit: element j' (low) or j' + 16 (high)
                jj = j - qs_off
                assert e == (jj if k < 4 else jj + 16)
                assert abs(d[e]) == 0.25 * 2 ** (k % 4)
            else:  # qh bit: element 8 * (j - 2) + k, weight 16
                assert e == 8 * (j - 2) + k
                assert abs(d[e]) == 0.25 * 16
            seen.add((e, (k % 4) if j >= qs_off else 4))
        assert len(seen) == (32 * 5 if t == o.Q5_0 else 32 * 4)


def test_q4_0_rml_worked_example():
    kv = keyvals("q4_0_blocks.txt")
    x = np.zeros(32, dtype=np.float32)
    x[:4] = np.array(kv["rml.x4"].split(), dtype=np.float32)
    b = o.quantize(o.Q4_0, x)
    assert b[:6].tobytes().hex() == kv["rml.head_hex"]
    y = o.dequantize(o.Q4_0, b, 32)
    assert y[0] == F32(-2.0)          # the extreme value is exact
    assert y[2] == F32(kv["rml.decoded_2_0"])  # 2.0 comes back as 1.75


def test_q4_0_nibble_reading_example_14():
    # Second Q4_0 block of Example 14: byte 0x79 holds code 9 for value 32 (low
    # nibble) and code 7 for value 48 (high nibble); d = 0xBCC0.
    kv = keyvals("q4_0_blocks.txt")
    x = _cl_inputs(64)
    x[40] = F32(9.5)
    b = o.quantize(o.Q4_0, x[32:64])
    assert b[2] == int(kv["cl_ex14_read.byte0"], 16)
    d = o.f16_to_f32(int(kv["cl_ex14_read.d_f16_bits"], 16))
    y = o.dequantize(o.Q4_0, b, 32)
    assert y[0] == F32(9 - 8) * F32(d)
    assert y[16] == F32(7 - 8) * F32(d)


def test_q4_0_example_6_errors():
    kv = keyvals("q4_0_blocks.txt")
    x = _cl_inputs(32)
    for t, key in ((o.Q4_0, "q4_0"), (o.Q8_0, "q8_0")):
        y = o.dequantize(t, o.quantize(t, x), 32)
        assert " ".join(f"{v:.4f}" for v in y[:4]) == kv[f"cl_ex6.{key}_first4"]
        diff = (y - x).astype(np.float64)
        assert f"{np.max(np.abs(diff)):.4f}" == kv[f"cl_ex6.{key}_max_err"]
        rmse = 100 * math.sqrt(np.sum(diff ** 2) / np.sum((x * x).astype(np.float64)))
        assert f"{rmse:.3f}" == kv[f"cl_ex6.{key}_rel_rmse_pct"]


def _fmt_out(v):
    if np.isnan(v):
        return "nan"
    if np.isinf(v):
        return "inf" if v > 0 else "-inf"
    return repr(float(v)) if v != 0 else "0.0"


def test_q8_0_edge_table():
    # candle "一些边界值": NaN ignored by amax and coded 0; inf amax -> d = inf ->
    # NaN block; d below the f16 subnormal range -> 0; d above 65504 -> inf.
    for label, A, special, outs in rows("q8_edge.txt", sep="|"):
        A = F32(A)
        x = (A * np.arange(32, dtype=np.float32) / F32(31)).astype(np.float32)
        if special == "x1=nan":
            x[1] = np.nan
        elif special == "x1=inf":
            x[1] = np.inf
        y = o.dequantize(o.Q8_0, o.quantize(o.Q8_0, x), 32)
        expect = outs.split()
        for got, want in zip(y[:3], expect):
            if want in ("nan", "inf"):
                assert _fmt_out(got) == want, label
            else:
                assert got == F32(want), (label, got, want)


def test_q8_0_fixed_point_and_bound():
    # codeloopback Example 4: requantizing dequantized values gives the same bytes;
    # rontolisp quantize: a value moves by at most half a step (amax / 254 before
    # the scale is rounded to f16).
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(32 * 500) * rng.choice([0.02, 1, 30], 32 * 500)).astype(np.float32)
    b = o.quantize(o.Q8_0, x)
    y = o.dequantize(o.Q8_0, b, x.size)
    assert np.array_equal(o.quantize(o.Q8_0, y), b)
    xb = x.reshape(-1, 32)
    d = np.abs(xb).max(axis=1, keepdims=True) / F32(127)
    codes = b.reshape(-1, 34)[:, 2:].view(np.int8).astype(np.float32)
    assert np.all(np.abs(codes * d - xb) <= np.abs(xb).max(axis=1, keepdims=True) / 254 * (1 + 1e-6))
    bq = o.quantize(o.Q4_0, x)
    assert np.array_equal(o.quantize(o.Q4_0, o.dequantize(o.Q4_0, bq, x.size)), bq)


def test_zero_block_gives_zero():
    # rml ZeroActivationsGiveZero; codeloopback Example 2 (d = 0 -> id = 0).
    z = np.zeros(512, dtype=np.float32)
    b8 = o.quantize(o.Q8_0, z)
    assert not b8.any()
    bk = o.quantize(o.Q8_K, z)
    assert not bk.any()
    rng = np.random.default_rng(3)
    w = rng.integers(0, 256, o.row_bytes(o.Q4_K, 512), dtype=np.uint8)
    w.reshape(-1, 144)[:, 0:2] = np.frombuffer(np.float16(0.01).tobytes(), np.uint8)
    w.reshape(-1, 144)[:, 2:4] = np.frombuffer(np.float16(0.02).tobytes(), np.uint8)
    y, l1 = o.vec_dot(o.Q4_K, w, bk, 512)
    assert y == 0.0 and l1 == 0.0


# --------------------------------------------------------------------------
# Q8_K invariants (its scale rule is not on the pages; these hold for any rule)
# --------------------------------------------------------------------------

def test_q8_K_layout_invariants():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(256 * 64).astype(np.float32) * rng.choice([1e-3, 1, 50], 256 * 64).astype(np.float32)
    b = o.quantize(o.Q8_K, x).reshape(-1, 292)
    d = b[:, 0:4].copy().view(np.float32)[:, 0]
    qs = b[:, 4:260].view(np.int8).astype(np.int32)
    bsums = b[:, 260:292].copy().view(np.int16).astype(np.int32)
    assert np.array_equal(bsums, qs.reshape(-1, 16, 16).sum(axis=2))  # candle BlockQ8K
    assert np.all(np.abs(qs) <= 127)
    amax = np.abs(x.reshape(-1, 256)).max(axis=1)
    # every block uses its full code range and codes are within half a step
    assert np.all(np.abs(qs).max(axis=1) == 127)
    err = np.abs(qs * d[:, None].astype(np.float64) - x.reshape(-1, 256))
    assert np.all(err <= (amax / 254 * (1 + 1e-5))[:, None])
    y = o.dequantize(o.Q8_K, b, x.size).reshape(-1, 256)
    assert np.array_equal(y, (qs.astype(np.float32) * d[:, None]).astype(np.float32))


def _q8_K_fields(b):
    b = b.reshape(-1, 292)
    return (b[:, 0:4].tobytes(), b[:, 4:260].view(np.int8).astype(np.int32),
            b[:, 260:292].copy().view("<i2").astype(np.int32))


def test_q8_K_exact_ties_round_away_from_zero():
    # codeloopback "Building Q8_0 and Q4_0 Like ggml", Example 2 prints roundf(2.5) = 3
    # and roundf(-2.5) = -3: a scaled value halfway between two codes goes away from
    # zero.  In a Q8_K block whose largest magnitude is 127 the scale is 127 / 127 =
    # 1 exactly and 1/d = 1, so x itself is the scaled value and each k + 1/2 is an
    # exact tie.  Worked by hand: codes 127, 3, -3, 1, -1, 5, -5, 127, -127, 2, -2,
    # 0 elsewhere; d's four bytes are f32 1.0 (00 00 80 3F); bsums[0] is the sum of
    # those codes (129 + ...), the other fifteen 0.  Round-half-even would give 2, -2,
    # 0, 0, 4, -4, 126, -126, 2, -2.
    x = np.zeros(256, np.float32)
    vals = [127.0, 2.5, -2.5, 0.5, -0.5, 4.5, -4.5, 126.5, -126.5, 1.5, -1.5]
    x[:len(vals)] = vals
    d, qs, bsums = _q8_K_fields(o.quantize(o.Q8_K, x))
    want = [127, 3, -3, 1, -1, 5, -5, 127, -127, 2, -2]
    assert d == bytes([0x00, 0x00, 0x80, 0x3F])
    assert qs[0, :len(want)].tolist() == want and not qs[0, len(want):].any()
    assert bsums[0].tolist() == [sum(want)] + [0] * 15
    # the same ties in the second block of a row, mirrored, with another block first
    x2 = np.concatenate([np.linspace(-1, 1, 256, dtype=np.float32), -x])
    d2, qs2, bs2 = _q8_K_fields(o.quantize(o.Q8_K, x2))
    assert d2[4:8] == bytes([0x00, 0x00, 0x80, 0x3F])
    assert qs2[1, :len(want)].tolist() == [-w for w in want]
    assert bs2[1].tolist() == [-sum(want)] + [0] * 15


def test_q8_K_scale_is_stored_as_f32():
    # candle "量化格式", section "块结构": BlockQ8K's d is an f32 (BlockQ8_0's an f16).
    # A block whose largest magnitude is 1 has d = fl32(1/127), worked by hand:
    # 1/127 = 2^-7 * 128/127 = 2^-7 * (1 + 1/127), 23-bit fraction round(2^23 / 127) =
    # round(66052.03) = 66052 = 0x10204, biased exponent 120 -> bits 0x3C010204, bytes
    # 04 02 01 3C.  Rounded to f16 first it would be 2^-7 * (1 + 8/1024) = 0x3C010000.
    # 1/d = 2^30 / 8454660 = 127 + 4/8454660 rounds to 127 exactly in f32 (half an ulp
    # at 127 is 2^-17), so the codes are x * 127 rounded: 1 -> 127, 0.5 -> 63.5 -> 64
    # (a tie, away from zero), -0.25 -> -31.75 -> -32, 0.125 -> 15.875 -> 16.
    x = np.zeros(256, np.float32)
    x[:4] = [1.0, 0.5, -0.25, 0.125]
    d, qs, bsums = _q8_K_fields(o.quantize(o.Q8_K, x))
    assert d == bytes([0x04, 0x02, 0x01, 0x3C])
    assert qs[0, :4].tolist() == [127, 64, -32, 16] and not qs[0, 4:].any()
    assert bsums[0].tolist() == [127 + 64 - 32 + 16] + [0] * 15
    # dequantized through the stored f32 d: 64 * d = 64 * 8454660 * 2^-30 exactly
    y = o.dequantize(o.Q8_K, o.quantize(o.Q8_K, x), 256)
    assert y[1] == np.float32(8454660 * 2.0 ** -24)


# --------------------------------------------------------------------------
# Q4_K: rml element-200 trace and candle get_scale_min_k4 prose
# --------------------------------------------------------------------------

def _q4k_block(rng):
    b = rng.integers(0, 256, 144, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.float16(rng.uniform(0.01, 0.1)).tobytes(), np.uint8)
    b[2:4] = np.frombuffer(np.float16(rng.uniform(0.01, 0.1)).tobytes(), np.uint8)
    return b


def test_q4_K_element_200_trace():
    # rml "Unpacking the packed fields": element 200 is in sub-block 6, chunk 3,
    # position 8 -> low nibble of qs[104]; scale = (s[10] & 0xF) | ((s[2] >> 6) << 4),
    # min = (s[10] >> 4) | ((s[6] >> 6) << 4); x = d * scale * q - dmin * min.
    rng = np.random.default_rng(200)
    for _ in range(50):
        b = np.zeros(144, dtype=np.uint8)
        d, dmin = np.float16(rng.uniform(0.01, 0.2)), np.float16(rng.uniform(0.01, 0.2))
        b[0:2] = np.frombuffer(d.tobytes(), np.uint8)
        b[2:4] = np.frombuffer(dmin.tobytes(), np.uint8)
        s = b[4:16]
        s[2], s[6], s[10] = rng.integers(0, 256, 3)
        b[16 + 104] = rng.integers(0, 256)
        scale = (int(s[10]) & 0xF) | ((int(s[2]) >> 6) << 4)
        mn = (int(s[10]) >> 4) | ((int(s[6]) >> 6) << 4)
        q = int(b[16 + 104]) & 0xF
        want = F32(d) * F32(scale) * F32(q) - F32(dmin) * F32(mn)
        y = o.dequantize(o.Q4_K, b, 256)
        assert y[200] == want
        # every other byte (besides d, dmin and the four above) leaves y[200] alone
        for k in range(4, 144):
            if k in (4 + 2, 4 + 6, 4 + 10, 16 + 104):
                continue
            b2 = b.copy()
            b2[k] ^= rng.integers(1, 256)
            assert o.dequantize(o.Q4_K, b2, 256)[200] == y[200], k


def _sub_block_effect(b, k, mask):
    """Which (sub-block, kind) values change when byte k of a Q4_K block is
    XORed with mask.  kind 'sc' is seen through dmin = 0, 'm' through d = 0."""
    out = set()
    for kind in ("sc", "m"):
        bb = b.copy()
        if kind == "sc":
            bb[2:4] = 0
        else:
            bb[0:2] = 0
        y0 = o.dequantize(o.Q4_K, bb, 256)
        bb[k] ^= mask
        y1 = o.dequantize(o.Q4_K, bb, 256)
        for j in range(8):
            if not np.array_equal(y0[32 * j:32 * j + 32], y1[32 * j:32 * j + 32]):
                out.add((j, kind))
    return out


def test_q4_K_scale_min_bit_positions():
    # candle 块结构 (get_scale_min_k4): sub-blocks 0-3 keep scale and min in the low
    # 6 bits of bytes 0-7; sub-blocks 4-7 keep their low 4 bits in bytes 8-11 and
    # borrow the high 2 bits from the top 2 bits of bytes 0-7.  rml's trace fixes
    # which of those belong to the scale (low nibble / bytes 0-3) and which to the
    # min (high nibble / bytes 4-7).
    rng = np.random.default_rng(5)
    b = _q4k_block(rng)
    b[16:] = 0x11  # q = 1 everywhere so a scale change shows in every element
    for t in range(4):
        assert _sub_block_effect(b, 4 + t, 0x3F) == {(t, "sc")}
        assert _sub_block_effect(b, 4 + t, 0xC0) == {(t + 4, "sc")}
        assert _sub_block_effect(b, 8 + t, 0x3F) == {(t, "m")}
        assert _sub_block_effect(b, 8 + t, 0xC0) == {(t + 4, "m")}
        assert _sub_block_effect(b, 12 + t, 0x0F) == {(t + 4, "sc")}
        assert _sub_block_effect(b, 12 + t, 0xF0) == {(t + 4, "m")}


def test_q4_K_each_nibble_is_one_element():
    # rml trace: element e of chunk c = e/64 at p = e%64 is the low nibble of
    # qs[32c + p] when p < 32, else (the complement) the high nibble of qs[32c+p-32].
    rng = np.random.default_rng(9)
    b = _q4k_block(rng)
    b[4:16] = 0x21  # nonzero scales in every sub-block
    y0 = o.dequantize(o.Q4_K, b, 256)
    for k in range(128):
        c, p = divmod(k, 32)
        for nib, e in ((0x0F, 64 * c + p), (0xF0, 64 * c + p + 32)):
            bb = b.copy()
            bb[16 + k] ^= nib
            changed = np.nonzero(o.dequantize(o.Q4_K, bb, 256) != y0)[0]
            assert list(changed) == [e], (k, nib)


# --------------------------------------------------------------------------
# Q6_K: only invariants (bit arrangement is not on the pages: parity unpinned)
# --------------------------------------------------------------------------

def test_q6_K_structure_invariants():
    # candle 块结构: ql = low 4 bits, qh = high 2 bits, 16 int8 scales for 16-element
    # sub-blocks, value d * sc[j] * (q - 32).  Properties any arrangement satisfies:
    # every ql nibble and every qh bit pair controls exactly one element, each element
    # is controlled by exactly one of each, and the scale of element e is sc[e / 16].
    rng = np.random.default_rng(6)
    b = rng.integers(0, 256, 210, dtype=np.uint8)
    b[192:208] = rng.integers(1, 100, 16).astype(np.int8).view(np.uint8)
    b[208:210] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    y0 = o.dequantize(o.Q6_K, b, 256)
    owner_low, owner_high = {}, {}
    for k in range(128):
        for nib in (0x0F, 0xF0):
            bb = b.copy()
            bb[k] ^= nib
            ch = np.nonzero(o.dequantize(o.Q6_K, bb, 256) != y0)[0]
            assert len(ch) == 1
            assert int(ch[0]) not in owner_low
            owner_low[int(ch[0])] = (k, nib)
    for k in range(64):
        for sh in range(4):
            bb = b.copy()
            bb[128 + k] ^= 3 << (2 * sh)
            ch = np.nonzero(o.dequantize(o.Q6_K, bb, 256) != y0)[0]
            assert len(ch) == 1
            assert int(ch[0]) not in owner_high
            owner_high[int(ch[0])] = (k, sh)
    assert len(owner_low) == 256 and len(owner_high) == 256
    d = F32(0.5)
    for j in range(16):
        bb = b.copy()
        bb[192 + j] = np.uint8(np.int8(-1).view(np.uint8))  # sc = -1
        y = o.dequantize(o.Q6_K, bb, 256)
        ch = np.nonzero(y != y0)[0]
        assert set(ch) <= set(range(16 * j, 16 * j + 16))
        # value = d * sc * (q - 32) -> with sc = -1, y = -d * (q - 32); q = 32 +- 32 range
        q = -y[16 * j:16 * j + 16] / d + 32
        assert np.all(q == np.round(q)) and np.all((q >= 0) & (q <= 63))
    bb = b.copy()
    bb[:192] = 0
    # q = 0 everywhere: value = -32 * d * sc
    sc = bb[192:208].view(np.int8).astype(np.float32)
    assert np.array_equal(o.dequantize(o.Q6_K, bb, 256), np.repeat(F32(-32) * d * sc, 16))


# --------------------------------------------------------------------------
# Q2_K and Q3_K: the pages give their size (candle GgmlDType table: 84 and 110
# bytes per 256 elements), that the K-quants split a superblock into 16 sub-blocks
# of 16 (or 8 of 32) whose small integer scales multiply the f16 d (rml summary,
# candle 块结构 prose), and that Q2K..Q6K pair with BlockQ8K; the field order and
# bit arrangement are GGUF's (parity unpinned).  Pinned here: structure any
# arrangement of those fields has.
# --------------------------------------------------------------------------

def _field_owners(t, b, fields):
    """For each (byte, mask) field: the elements a flip of it changes."""
    y0 = o.dequantize(t, b, 256)
    out = []
    for k, mask in fields:
        bb = b.copy()
        bb[k] ^= mask
        out.append(np.nonzero(o.dequantize(t, bb, 256) != y0)[0])
    return y0, out


def test_q2_K_structure_invariants():
    rng = np.random.default_rng(12)
    b = rng.integers(0, 256, 84, dtype=np.uint8)
    b[0:16] = rng.integers(1, 16, 16) | (rng.integers(1, 16, 16) << 4)   # sc, m nonzero
    b[80:82] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    b[82:84] = np.frombuffer(np.float16(0.25).tobytes(), np.uint8)
    # the 256 two-bit code fields of the 64 code bytes: each moves exactly one
    # element, and each element is moved by exactly one
    y0, owners = _field_owners(o.Q2_K, b, [(16 + k, 3 << (2 * f)) for k in range(64) for f in range(4)])
    assert all(len(c) == 1 for c in owners)
    assert sorted(int(c[0]) for c in owners) == list(range(256))
    # each scale byte's nibbles act on exactly one run of 16 consecutive elements,
    # the 16 runs tile the superblock (every code 1, so the scale shows everywhere)
    b1 = b.copy()
    b1[16:80] = 0x55
    _, sc_owners = _field_owners(o.Q2_K, b1, [(j, 0x0F) for j in range(16)])
    _, m_owners = _field_owners(o.Q2_K, b1, [(j, 0xF0) for j in range(16)])
    runs = sorted(tuple(c) for c in sc_owners)
    assert runs == [tuple(range(16 * j, 16 * j + 16)) for j in range(16)]
    assert all(np.array_equal(a, c) for a, c in zip(sc_owners, m_owners))
    # codes 0: value -dmin * m of the element's sub-block; codes 3: 3 d sc - dmin m
    for fill, mult in ((0x00, 0), (0xFF, 3)):
        bb = b.copy()
        bb[16:80] = fill
        y = o.dequantize(o.Q2_K, bb, 256)
        vals = sorted(set(np.round(y.astype(np.float64), 6)))
        want = sorted(set(np.round([mult * 0.5 * (s & 15) - 0.25 * (s >> 4) for s in b[0:16]], 6)))
        assert vals == want


def test_q3_K_structure_invariants():
    rng = np.random.default_rng(13)
    b = rng.integers(0, 256, 110, dtype=np.uint8)
    b[108:110] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    # no sub-block scale of 32 (a zero multiplier would hide its elements)
    while any(o.dequantize(o.Q3_K, b, 256)[16 * j:16 * j + 16].tolist() == [0.0] * 16 for j in range(16)):
        b[96:108] = rng.integers(0, 256, 12, dtype=np.uint8)
    # two-bit code fields of qs and the single hmask bits: each moves exactly one
    # element; both families cover all 256 elements once
    _, lo = _field_owners(o.Q3_K, b, [(32 + k, 3 << (2 * f)) for k in range(64) for f in range(4)])
    _, hi = _field_owners(o.Q3_K, b, [(k, 1 << f) for k in range(32) for f in range(8)])
    assert all(len(c) == 1 for c in lo + hi)
    assert sorted(int(c[0]) for c in lo) == list(range(256))
    assert sorted(int(c[0]) for c in hi) == list(range(256))
    # the high code bit is worth 4 steps of the element's scale
    y0 = o.dequantize(o.Q3_K, b, 256).astype(np.float64)
    for k, f in ((0, 0), (5, 3), (31, 7)):
        bb = b.copy()
        bb[k] ^= 1 << f
        y1 = o.dequantize(o.Q3_K, bb, 256).astype(np.float64)
        e = int(np.nonzero(y1 != y0)[0][0])
        lowbb = b.copy()
        # the same element's low field moved by one step, for the step size
        step = None
        for kk in range(64):
            for ff in range(4):
                c = lowbb.copy()
                c[32 + kk] ^= 1 << (2 * ff)
                yc = o.dequantize(o.Q3_K, c, 256).astype(np.float64)
                if yc[e] != y0[e]:
                    step = abs(yc[e] - y0[e])
        assert abs(abs(y1[e] - y0[e]) - 4 * step) == 0
    # the 96 scale bits: each acts on exactly one run of 16 consecutive elements, each
    # run is acted on by exactly 6 bits
    _, sc = _field_owners(o.Q3_K, b, [(96 + k, 1 << f) for k in range(12) for f in range(8)])
    runs = {}
    for c in sc:
        assert len(c) >= 1
        j = int(c[0]) // 16
        assert set(int(x) for x in c) <= set(range(16 * j, 16 * j + 16))
        runs[j] = runs.get(j, 0) + 1
    assert runs == {j: 6 for j in range(16)}
    # every code at its middle value (low bits 0, high bit set) or every scale at its
    # middle value gives zero: codes and scales are offset by half their range
    bb = b.copy()
    bb[32:96] = 0
    bb[0:32] = 0xFF
    assert not o.dequantize(o.Q3_K, bb, 256).any()


# --------------------------------------------------------------------------
# Round-trip statistics printed on the candle formats page ("往返误差"): the only
# numbers the pages give that depend on the Q8_K scale rule (its bytes are never
# printed).  Quantize + dequantize of 262144 N(0,1) values (and the same with one
# value per 256 scaled by 20) must reproduce the printed rel RMSE within the
# sampling spread of a different draw (1 % of the value for N(0,1), 3 % with
# outliers; measured over seeds 0-5: 0.3 % and 1.6 %) and max |err| within 25 %.
# This fixes each rule's resolution (block size, levels, round to nearest), not its
# last bit.  Planted in the Q8_K rule, each of these fails: a divisor of 128 (the
# extreme value saturates at 127, so max |err| is a whole step), 63 or 255,
# truncation instead of rounding, an amax over the first 32 values only.
# --------------------------------------------------------------------------

def _roundtrip(t, x):
    if t == o.Q8_K:
        b = o.quantize(o.Q8_K, x.reshape(-1, 256)).reshape(-1, 292)
        d = b[:, 0:4].copy().view(np.float32)[:, 0]
        y = (b[:, 4:260].view(np.int8).astype(np.float32) * d[:, None]).reshape(-1)
    else:
        y = o.dequantize(t, o.quantize(t, x), x.size)
    e = y.astype(np.float64) - x.astype(np.float64)
    return 100 * math.sqrt(np.mean(e ** 2) / np.mean(x.astype(np.float64) ** 2)), float(np.max(np.abs(e)))


@pytest.mark.parametrize("row", rows("candle_roundtrip.txt", sep="|"), ids=lambda r: r[0])
def test_candle_roundtrip_statistics(row):
    name, rmse, maxerr, rmse_o, _ = row
    t = {"Q4_0": o.Q4_0, "Q4_1": o.Q4_1, "Q5_0": o.Q5_0, "Q8_0": o.Q8_0, "Q8_K": o.Q8_K}[name]
    rng = np.random.default_rng(2025)
    x = rng.standard_normal(262144).astype(np.float32)
    got, gmax = _roundtrip(t, x)
    assert abs(got - float(rmse)) <= 0.01 * float(rmse), (name, got)
    assert abs(gmax - float(maxerr)) <= 0.25 * float(maxerr), (name, gmax)
    if rmse_o != "-":
        xo = x.copy().reshape(-1, 256)
        xo[np.arange(xo.shape[0]), rng.integers(0, 256, xo.shape[0])] *= np.float32(20)
        got_o, _ = _roundtrip(t, xo.reshape(-1))
        assert abs(got_o - float(rmse_o)) <= 0.03 * float(rmse_o), (name, got_o)


# --------------------------------------------------------------------------
# Q5_1 (dequantize only): size from candle's table, "the _1 types add an f16 min"
# from its block prose; field order not on the pages (parity unpinned beyond the
# reduction to the pinned Q4_1 decoder and the fifth-bit structure).
# --------------------------------------------------------------------------

def test_q5_1_without_fifth_bits_is_q4_1():
    rng = np.random.default_rng(71)
    for _ in range(50):
        b = rng.integers(0, 256, 24, dtype=np.uint8)
        b[0:2] = np.frombuffer(np.float16(rng.uniform(1e-3, 4e-3)).tobytes(), np.uint8)
        b[2:4] = np.frombuffer(np.float16(rng.uniform(-0.03, 0.03)).tobytes(), np.uint8)
        b[4:8] = 0
        q41 = np.concatenate([b[0:4], b[8:24]])
        assert np.array_equal(o.dequantize(o.Q5_1, b, 32), o.dequantize(o.Q4_1, q41, 32))


def test_q5_1_fifth_bit_e_is_element_e():
    # bit e of qh is bit 4 of element e, as in Q5_0 (codeloopback Example 8's qh
    # string pins that arrangement for Q5_0); with m = 0 it adds exactly 16 d.
    rng = np.random.default_rng(72)
    b = rng.integers(0, 256, 24, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.float16(0.25).tobytes(), np.uint8)
    b[2:4] = 0
    b[4:8] = 0
    y0 = o.dequantize(o.Q5_1, b, 32).astype(np.float64)
    for e in range(32):
        bb = b.copy()
        bb[4 + e // 8] |= 1 << (e % 8)
        y1 = o.dequantize(o.Q5_1, bb, 32).astype(np.float64)
        assert list(np.nonzero(y1 != y0)[0]) == [e]
        assert y1[e] - y0[e] == 16 * 0.25


# --------------------------------------------------------------------------
# Q8_1 and the Q4_1 / Q5_1 dot products.  candle "量化格式", VecDotType table:
# Q4_1 and Q5_1 pair with BlockQ8_1, whose layout the pages do not print.  Reading:
# d f16 @0, s f16 @2, 32 int8 codes @4; d and the codes by the Q8_0 rule (pinned
# below by the printed Q8_0 bytes), s = f16(sum of codes * the unrounded f32 d).
# --------------------------------------------------------------------------

def _q8_1_fields(b):
    return (b[0:2].tobytes().hex(), b[2:4].tobytes().hex(), [int(c) for c in b[4:36].view(np.int8)])


def test_q8_1_d_and_codes_are_the_printed_q8_0_bytes():
    kv = keyvals("q8_0_blocks.txt")
    assert o.block_elems(o.Q8_1) == 32 and o.block_bytes(o.Q8_1) == 36
    # codeloopback Example 2's block: the printed Q8_0 hex is d (2 bytes) + 32 codes
    b = o.quantize(o.Q8_1, _cl_inputs(32))
    assert b[0:2].tobytes().hex() + b[4:].tobytes().hex() == kv["cl_ex2.hex"]
    # candle's Q8_0 block
    d, _, codes = _q8_1_fields(o.quantize(o.Q8_1, (np.arange(32, dtype=np.float32) - F32(15.5)) / F32(10)))
    assert d == kv["candle.d_bytes_hex"]
    assert codes == [int(c) for c in kv["candle.qs"].split()]


def test_q8_1_sum_field_hand_worked():
    # amax 127: d = 1 exactly, codes are roundf(x) (ties away from zero, codeloopback
    # Example 2), s = f16(sum).  127 + 3 - 3 + 1 = 128 = 2^7: f16 0x5800.
    x = np.zeros(32, np.float32)
    x[:4] = [127.0, 2.5, -2.5, 1.4]
    d, s_, codes = _q8_1_fields(o.quantize(o.Q8_1, x))
    assert d == "003c" and codes[:4] == [127, 3, -3, 1] and s_ == "0058"
    # -127 - 100 = -227 = -1.7734375 * 2^7: sign, exponent 22, fraction 792: 0xdb18.
    x[:4] = [-127.0, -100.0, 0.0, 0.0]
    assert _q8_1_fields(o.quantize(o.Q8_1, x))[1] == "18db"
    # amax 1: d = fl32(1/127) = 0.0078740157; codes 127, -127, 16 (0.125 * 127 =
    # 15.875), 1 (0.0078125 * 127 = 0.99); sum 17.  17 * d = 0.13385826 lies between
    # the f16 neighbours 0x3048 = 0.13378906 and 0x3049 = 0.13391113, nearer 0x3049.
    # With d first rounded to f16 (0.0078735352) the product, 0.13385010, would be
    # nearer 0x3048: the sum is scaled by the unrounded d.
    x[:4] = [1.0, -1.0, 0.125, 0.0078125]
    d, s_, codes = _q8_1_fields(o.quantize(o.Q8_1, x))
    assert codes[:4] == [127, -127, 16, 1] and sum(codes) == 17
    assert s_ == "4930"
    assert o.quantize(o.Q8_1, np.zeros(32, np.float32)).tobytes() == bytes(36)
    # an infinity: d = inf (f16 0x7c00), every code 0 (finite * 0, and inf * 0 = NaN
    # coded 0), so s = 0 * inf, stored as the quiet NaN 0x7e00
    x[:4] = [np.inf, 1.0, -2.0, 0.0]
    d, s_, codes = _q8_1_fields(o.quantize(o.Q8_1, x))
    assert d == "007c" and not any(codes) and s_ == "007e"


def _blocks_with_min(t, nblocks, rng, zero_min=False):
    nb = o.block_bytes(t)
    w = rng.integers(0, 256, (nblocks, nb), dtype=np.uint8)
    w[:, 0:2] = np.frombuffer(rng.uniform(1e-3, 4e-3, nblocks).astype(np.float16).tobytes(), np.uint8).reshape(-1, 2)
    m = np.zeros(nblocks) if zero_min else rng.uniform(-0.05, 0.05, nblocks)
    w[:, 2:4] = np.frombuffer(m.astype(np.float16).tobytes(), np.uint8).reshape(-1, 2)
    return w.reshape(-1)


@pytest.mark.parametrize("t", [o.Q4_1, o.Q5_1])
def test_q4_1_q5_1_block_sums_are_exact(t):
    # with m = 0 every decoded value is code * d exactly (code < 32, d f16), so the
    # codes come back from the dequantizer (pinned by codeloopback Examples 7 and 14
    # for Q4_1) and the block's integer is their dot product with the Q8_1 codes.
    rng = np.random.default_rng(80 + t)
    n = 256
    w = _blocks_with_min(t, n // 32, rng, zero_min=True)
    xq = o.quantize(o.Q8_1, rng.standard_normal(n).astype(np.float32))
    d = np.repeat(w.reshape(-1, o.block_bytes(t))[:, 0:2].copy().view(np.float16).astype(np.float64)[:, 0], 32)
    q = o.dequantize(t, w, n).astype(np.float64) / d
    assert np.array_equal(q, np.round(q)) and q.min() >= 0 and q.max() < (16 if t == o.Q4_1 else 32)
    a = xq.reshape(-1, 36)[:, 4:].view(np.int8).astype(np.int64).reshape(-1)
    want = (q.astype(np.int64) * a).reshape(-1, 32).sum(axis=1)
    assert np.array_equal(o.block_sums(t, w, xq, n)[:, 0], want)


@pytest.mark.parametrize("t", [o.Q4_1, o.Q5_1])
def test_q4_1_q5_1_vec_dot_brute_force(t):
    # sum over elements of (code d_w + m_w) (d_x a), in f64 from the dequantized
    # values.  The oracle's minimum term uses the stored s = f16(d_x32 sum a), where
    # d_x32 is the unrounded scale that the dequantizer sees rounded to f16: the two
    # differ by at most 2^-10 |m_w d_x sum a| per block (two f16 roundings); the
    # rest is f32 rounding of the block steps and their sum.
    rng = np.random.default_rng(90 + t)
    for nblk in (1, 8, 96):
        n = 32 * nblk
        w = _blocks_with_min(t, nblk, rng)
        x = rng.standard_normal(n).astype(np.float32)
        xq = o.quantize(o.Q8_1, x)
        xb = xq.reshape(-1, 36)
        dx = xb[:, 0:2].copy().view(np.float16).astype(np.float64)[:, 0]
        a = xb[:, 4:].view(np.int8).astype(np.int64)
        brute = np.sum(o.dequantize(t, w, n).astype(np.float64) * np.repeat(dx, 32) * a.reshape(-1))
        mw = w.reshape(nblk, -1)[:, 2:4].copy().view(np.float16).astype(np.float64)[:, 0]
        bound = np.sum(np.abs(mw * dx * a.sum(axis=1))) * 2.0 ** -10 * 1.01
        y, l1 = o.vec_dot(t, w, xq, n)
        assert abs(y - brute) <= bound + 2 * nblk * 2.0 ** -23 * l1 + 1e-30, (t, n, y, brute)
        # dropping the minimum term, or taking it with the wrong sign, is far outside
        assert np.sum(np.abs(mw * dx * a.sum(axis=1))) > 50 * bound


# --------------------------------------------------------------------------
# Q5_K: the pages give its size and that it shares Q4K's d, dmin and 6-bit
# (scale, min) pairs; field order and fifth-bit arrangement are not on the pages
# (parity unpinned).  Pinned: the reduction to the pinned Q4_K decoder when no
# fifth bit is set, and structure any arrangement of the fifth bits satisfies.
# --------------------------------------------------------------------------

def _q5k_block(rng):
    b = rng.integers(0, 256, 176, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.float16(rng.uniform(0.01, 0.1)).tobytes(), np.uint8)
    b[2:4] = np.frombuffer(np.float16(rng.uniform(0.01, 0.1)).tobytes(), np.uint8)
    return b


def test_q5_K_without_fifth_bits_is_q4_K():
    # candle 块结构: Q5K is Q4K's (d, dmin, 6-bit scales and mins, 4-bit low codes)
    # plus one more bit per code.  With every fifth bit clear, each element must be
    # the Q4_K element of the block made of the same d, dmin, scales and nibbles.
    rng = np.random.default_rng(13)
    for _ in range(20):
        b = _q5k_block(rng)
        b[16:48] = 0
        q4 = np.concatenate([b[0:16], b[48:176]])
        assert np.array_equal(o.dequantize(o.Q5_K, b, 256), o.dequantize(o.Q4_K, q4, 256))


def test_q5_K_each_fifth_bit_is_one_element():
    # 256 fifth bits for 256 elements: every qh bit controls exactly one element,
    # every element exactly one bit, and setting it adds 16 to that element's code:
    # seen through dmin = 0, the value moves from d*sc*q to d*sc*(q + 16).
    rng = np.random.default_rng(14)
    b = _q5k_block(rng)
    b[2:4] = 0  # dmin = 0: the value is d * sc * q, exact in f32
    b[4:16] = 0x21  # scale 33 in sub-blocks 0-3, 1 in sub-blocks 4-7
    b[16:48] = 0
    y0 = o.dequantize(o.Q5_K, b, 256).astype(np.float64)
    d = float(np.frombuffer(b[0:2].tobytes(), np.float16)[0])
    owner = {}
    for k in range(32):
        for bit in range(8):
            bb = b.copy()
            bb[16 + k] |= 1 << bit
            y1 = o.dequantize(o.Q5_K, bb, 256).astype(np.float64)
            ch = np.nonzero(y1 != y0)[0]
            assert len(ch) == 1, (k, bit)
            e = int(ch[0])
            assert e not in owner
            owner[e] = (k, bit)
            sc = 33 if e < 128 else 1
            assert y1[e] - y0[e] == d * sc * 16
    assert len(owner) == 256
    # fifth bits of consecutive elements of one 32-element sub-block share a bit
    # position and run over consecutive qh bytes (the Q4_K nibble order, one bit plane
    # per sub-block)
    for j in range(8):
        bits = {owner[e][1] for e in range(32 * j, 32 * j + 32)}
        assert len(bits) == 1
        assert [owner[e][0] for e in range(32 * j, 32 * j + 32)] == list(range(32))


def test_q5_K_codes_span_0_to_31():
    # A 5-bit code: with d = 1, dmin = 0 and every scale 1, the values are the codes,
    # all of 0..31 reachable; all-ones low nibbles and fifth bits give 31.
    b = np.zeros(176, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    b[4:8] = 1
    b[12:16] = 1
    b[16:48] = 0xFF
    b[48:176] = 0xFF
    assert np.array_equal(o.dequantize(o.Q5_K, b, 256), np.full(256, 31, np.float32))
    rng = np.random.default_rng(15)
    b[16:48] = rng.integers(0, 256, 32)
    b[48:176] = rng.integers(0, 256, 128)
    y = o.dequantize(o.Q5_K, b, 256)
    assert np.all(y == np.round(y)) and y.min() >= 0 and y.max() <= 31
    assert len(set(y.tolist())) > 24


# --------------------------------------------------------------------------
# VecDot: brute force against the dequantized values, and the seeded examples
# --------------------------------------------------------------------------

def _random_weights(t, nblocks, rng):
    nb = o.block_bytes(t)
    w = rng.integers(0, 256, nb * nblocks, dtype=np.uint8).reshape(nblocks, nb)
    h = lambda lo, hi: np.frombuffer(rng.uniform(lo, hi, nblocks).astype(np.float16).tobytes(), np.uint8).reshape(nblocks, 2)
    if t in (o.Q8_0, o.Q4_0, o.Q5_0):
        w[:, 0:2] = h(0.001, 0.05)
    elif t in (o.Q4_K, o.Q5_K):
        w[:, 0:2] = h(1e-3, 1e-2)
        w[:, 2:4] = h(1e-3, 1e-2)
    elif t == o.Q6_K:
        w[:, 192:208] = rng.integers(-64, 64, (nblocks, 16)).astype(np.int8).view(np.uint8)
        w[:, 208:210] = h(1e-3, 1e-2)
    elif t == o.Q2_K:
        w[:, 80:82] = h(1e-3, 1e-2)
        w[:, 82:84] = h(1e-3, 1e-2)
    elif t == o.Q3_K:
        w[:, 108:110] = h(1e-3, 1e-2)
    return w.reshape(-1)


def _act_parts(at, xq, n):
    """(per-element f64 scale, per-element int code) of an activation row."""
    if at == o.Q8_0:
        blk = xq.reshape(-1, 34)
        d = blk[:, 0:2].copy().view(np.float16).astype(np.float64)[:, 0]
        return np.repeat(d, 32), blk[:, 2:].view(np.int8).astype(np.int64).reshape(-1)
    blk = xq.reshape(-1, 292)
    d = blk[:, 0:4].copy().view(np.float32).astype(np.float64)[:, 0]
    return np.repeat(d, 256), blk[:, 4:260].view(np.int8).astype(np.int64).reshape(-1)


@pytest.mark.parametrize("t", [o.Q8_0, o.Q4_0, o.Q5_0, o.Q4_K, o.Q5_K, o.Q6_K, o.Q2_K, o.Q3_K])
def test_vec_dot_brute_force(t):
    rng = np.random.default_rng(100 + t)
    at = o.act_type(t)
    for nblocks_k in (1, 2, 3):
        n = nblocks_k * 256
        w = _random_weights(t, n // o.block_elems(t), rng)
        x = rng.standard_normal(n).astype(np.float32)
        xq = o.quantize(at, x)
        wdeq = o.dequantize(t, w, n).astype(np.float64)
        dx, qx = _act_parts(at, xq, n)
        terms = wdeq * (dx * qx)
        brute = terms.sum()
        # f64 evaluation of the oracle's exact block integers with the block scales
        sums = o.block_sums(t, w, xq, n).astype(np.float64)
        wb = w.reshape(n // o.block_elems(t), -1)
        f16 = lambda a, off: a[:, off:off + 2].copy().view(np.float16).astype(np.float64)[:, 0]
        if t in (o.Q8_0, o.Q4_0, o.Q5_0):
            exact = np.sum(sums[:, 0] * f16(wb, 0) * dx[::32])
        elif t in (o.Q4_K, o.Q5_K, o.Q2_K):
            off = 80 if t == o.Q2_K else 0
            exact = np.sum(dx[::256] * (f16(wb, off) * sums[:, 0] - f16(wb, off + 2) * sums[:, 1]))
        else:
            exact = np.sum(dx[::256] * f16(wb, 108 if t == o.Q3_K else 208) * sums[:, 0])
        scale = np.abs(terms).sum()
        # Q8_0, Q4_0, Q5_0, Q3_K, Q6_K decoded values are exact in f32; the K-quants
        # with a min (d*sc*q - dmin*m) round once per element.
        tol = 1e-12 if t not in (o.Q4_K, o.Q5_K, o.Q2_K) else 1e-7
        assert abs(exact - brute) <= tol * scale, (t, n, exact, brute)
        y, l1 = o.vec_dot(t, w, xq, n)
        nbk = n // o.block_elems(t)
        assert abs(y - exact) <= nbk * 2.0 ** -23 * l1 + 1e-30


def _examples_10_11():
    kv = keyvals("seeded_examples.txt")
    n = 4096
    r = JavaRandom(22)
    a = np.empty(n, np.float32)
    b = np.empty(n, np.float32)
    for i in range(n):
        a[i] = F32(r.next_gaussian()) * F32(0.02)
        b[i] = F32(r.next_gaussian())
    y10, _ = o.vec_dot(o.Q8_0, o.quantize(o.Q8_0, a), o.quantize(o.Q8_0, b), n)
    exact10 = float(np.dot(a.astype(np.float64), b.astype(np.float64)))
    r = JavaRandom(23)
    w = np.empty(n, np.float32)
    x = np.empty(n, np.float32)
    for i in range(n):
        w[i] = F32(r.next_gaussian()) * F32(0.02)
        x[i] = F32(r.next_gaussian())
    qw = o.quantize(o.Q4_0, w)
    y11, _ = o.vec_dot(o.Q4_0, qw, o.quantize(o.Q8_0, x), n)
    wo11 = float(np.dot(o.dequantize(o.Q4_0, qw, n).astype(np.float64), x.astype(np.float64)))
    exact11 = float(np.dot(w.astype(np.float64), x.astype(np.float64)))
    return kv, (y10, exact10, y11, wo11, exact11)


def test_codeloopback_examples_10_11_vec_dot():
    kv, (y10, exact10, y11, wo11, exact11) = _examples_10_11()
    assert f"{y10:.6f}" == kv["ex10.q8_0_dot"]
    assert f"{exact10:.6f}" == kv["ex10.exact"]
    assert f"{y11:.6f}" == kv["ex11.q4_0_q8_0_kernel"]
    assert f"{wo11:.6f}" == kv["ex11.q4_0_weights_f32_x"]
    assert f"{exact11:.6f}" == kv["ex11.exact"]


def _outlier_weights(r, count):
    w = np.empty(count, np.float32)
    for i in range(count):
        g = F32(r.next_gaussian()) * F32(0.02)
        w[i] = g * (F32(10) if r.next_int(500) == 0 else F32(1))
    return w


def _fake(t, x):
    if t == "F16":
        return x.astype(np.float16).astype(np.float32)
    tt = {"Q8_0": o.Q8_0, "Q4_0": o.Q4_0, "Q4_1": o.Q4_1, "Q5_0": o.Q5_0}[t]
    return o.dequantize(tt, o.quantize(tt, x), x.size)


def test_codeloopback_example_12_error_table():
    kv = keyvals("seeded_examples.txt")
    x = _outlier_weights(JavaRandom(24), 65536)
    p = np.sum((x * x).astype(np.float64))
    for t in ("F16", "Q8_0", "Q5_0", "Q4_1", "Q4_0"):
        y = _fake(t, x)
        e = np.sum(((y - x).astype(np.float64)) ** 2)
        assert f"{100 * math.sqrt(e / p):.4f}" == kv[f"ex12.{t}"], t


def test_codeloopback_example_13_output_error():
    kv = keyvals("seeded_examples.txt")
    rows_, cols = 256, 4096
    r = JavaRandom(25)
    w = _outlier_weights(r, rows_ * cols).reshape(rows_, cols)
    x = np.array([F32(r.next_gaussian()) for _ in range(cols)], dtype=np.float32)
    xq = _fake("Q8_0", x)
    ref = w.astype(np.float64) @ x.astype(np.float64)
    for t in ("F16", "Q8_0", "Q4_0"):
        wq = _fake(t, w.reshape(-1)).reshape(rows_, cols)
        act = x if t == "F16" else xq
        y = wq.astype(np.float64) @ act.astype(np.float64)
        err = 100 * math.sqrt(np.sum((y - ref) ** 2) / np.sum(ref ** 2))
        assert f"{err:.4f}" == kv[f"ex13.{t}"], t


def test_codeloopback_example_15_project_report():
    kv = keyvals("seeded_examples.txt")
    rows_, cols = 512, 2048
    r = JavaRandom(26)
    w = _outlier_weights(r, rows_ * cols)
    x = np.array([F32(r.next_gaussian()) for _ in range(cols)], dtype=np.float32)
    for name, t in (("Q8_0", o.Q8_0), ("Q4_0", o.Q4_0)):
        q = o.quantize(t, w.reshape(rows_, cols))
        wq = o.dequantize(t, q, w.size)
        e = np.sum(((wq - w).astype(np.float64)) ** 2)
        p = np.sum((w * w).astype(np.float64))
        assert f"{100 * math.sqrt(e / p):.3f}" == kv[f"ex15.{name}.weight_rmse"]
        y = w.reshape(rows_, cols).astype(np.float64) @ x.astype(np.float64)
        yq = wq.reshape(rows_, cols).astype(np.float64) @ x.astype(np.float64)
        oe = 100 * math.sqrt(np.sum((yq - y) ** 2) / np.sum(y ** 2))
        assert f"{oe:.3f}" == kv[f"ex15.{name}.output_err"]
        assert np.array_equal(o.quantize(t, wq.reshape(rows_, cols)), q)  # stable


def test_gemv_is_vec_dot_per_row_and_column():
    # sipllm matmul_quant: y[o] = VecDot(row o, x) for each output row; every
    # activation column is independent.
    rng = np.random.default_rng(21)
    for t in (o.Q8_0, o.Q4_0, o.Q4_K, o.Q5_K, o.Q6_K):
        n_out, n_in, ncols = 5, 512, 3
        W = _random_weights(t, n_out * n_in // o.block_elems(t), rng)
        X = rng.standard_normal((ncols, n_in)).astype(np.float32)
        xq = o.quantize(o.act_type(t), X)
        y, l1 = o.gemv(t, W, n_out, n_in, xq, ncols)
        rb = o.row_bytes(t, n_in)
        for c in range(ncols):
            for r_ in range(n_out):
                v, s = o.vec_dot(t, W[rb * r_:rb * (r_ + 1)], xq[c], n_in)
                assert y[c, r_] == F32(v) and l1[c, r_] == s


# --------------------------------------------------------------------------
# SwiGLU epilogue of the FFN step (not on the pages: silu(g) * u, silu(v) =
# v * sigmoid(v)); pinned by closed forms of the logistic function.
# --------------------------------------------------------------------------

def test_swiglu_closed_forms():
    ln3 = math.log(3.0)
    g = np.array([0.0, ln3, -ln3, 50.0, -50.0, 2.0, -2.0, 1e-3], dtype=np.float32)
    u = np.ones_like(g)
    h = o.swiglu(g, u)
    gd = g.astype(np.float64)
    assert h[0] == 0.0
    # sigmoid(ln 3) = 3/4 with slope 3/16 there; g holds ln 3 rounded to f32
    d1 = gd[1] - ln3
    assert abs(h[1] - gd[1] * (0.75 + 0.1875 * d1)) <= 1e-14
    assert abs(h[2] - gd[2] * (0.25 - 0.1875 * d1)) <= 1e-14
    assert abs(h[3] - 50.0) <= 1e-15 * 50 and abs(h[4]) < 1e-19                     # tails
    # odd part: silu(v) - silu(-v) = v exactly in the reals
    assert abs((h[5] - h[6]) - gd[5]) <= 1e-15
    assert abs(h[7] - gd[7] * (0.5 + gd[7] / 4)) <= 1e-12                           # slope 1/2 at 0
    # linear in u, sign follows u
    u2 = np.array([2, -3, 0.5, 1, 1, -1, 4, 1], dtype=np.float32)
    h2 = o.swiglu(g, u2)
    assert np.allclose(h2, h * u2.astype(np.float64), rtol=1e-15, atol=0)


def test_swiglu_large_negative_gate_is_zero_not_nan():
    g = np.array([-1e30, -3.4e38, -89.0], dtype=np.float32)
    h = o.swiglu(g, np.full(3, 7.0, np.float32))
    assert np.all(np.isfinite(h)) and np.all(np.abs(h) < 1e-30)
