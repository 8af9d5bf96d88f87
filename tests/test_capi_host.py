"""Host-side checks of libqk.so (no GPU): it loads, exports every function that
include/qk.h declares, its geometry and pairing match the printed type table,
and argument validation rejects bad calls before anything is enqueued.

Every call below fails validation by construction (bad type, shape, pointer or
alignment), so no kernel is launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_gemv_quantize_amd as qk
from golden_io import rows

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qk.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qk_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = qk.lib()
    names = _declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qk.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qk_[a-z0-9_]+)", out))
    assert set(names) <= exported


def test_c_host_program_links_the_library_and_the_oracle():
    # tests/c/abi_check (built by __graft_entry__.build()) resolves libqk.so and the
    # oracle in-tree through its rpaths; running it needs a GPU (a gpu test does)
    exe = os.path.join(ROOT, "tests", "c", "abi_check")
    if not os.path.exists(exe):
        pytest.skip("tests/c/abi_check is not built")
    out = subprocess.run(["ldd", exe], capture_output=True, text=True, check=True).stdout
    libs = {line.split("=>")[0].strip(): line.split("=>")[1].split("(")[0].strip()
            for line in out.splitlines() if "=>" in line}
    assert os.path.realpath(libs["libqk.so"]) == os.path.realpath(qk.DEFAULT_LIB_PATH)
    assert os.path.realpath(libs["liboracle.so"]) == os.path.join(ROOT, "oracle", "liboracle.so")


def test_library_is_built_for_gfx950_only():
    # the offload bundle ids embedded in the library name every device target
    data = open(qk.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[-a-z0-9:+]*?(gfx[0-9a-f]+)", data))
    assert targets == {b"gfx950"}, targets


def test_geometry_matches_type_table():
    ids = {"Q4_0": qk.QK_TYPE_Q4_0, "Q4_1": qk.QK_TYPE_Q4_1, "Q5_0": qk.QK_TYPE_Q5_0, "Q5_1": qk.QK_TYPE_Q5_1,
           "Q8_0": qk.QK_TYPE_Q8_0, "Q2_K": qk.QK_TYPE_Q2_K, "Q3_K": qk.QK_TYPE_Q3_K,
           "Q4_K": qk.QK_TYPE_Q4_K, "Q5_K": qk.QK_TYPE_Q5_K,
           "Q6_K": qk.QK_TYPE_Q6_K, "Q8_K": qk.QK_TYPE_Q8_K}
    for name, gid, elems, nbytes, _ in rows("type_table.txt"):
        assert ids[name] == int(gid)
        assert qk.qk_block_elems(ids[name]) == int(elems)
        assert qk.qk_block_bytes(ids[name]) == int(nbytes)
    assert qk.qk_row_bytes(qk.QK_TYPE_Q8_0, 4096) == 4352
    assert qk.qk_row_bytes(qk.QK_TYPE_Q4_K, 11008) == 6192
    assert qk.qk_row_bytes(qk.QK_TYPE_Q6_K, 11008) == 9030
    assert qk.qk_row_bytes(qk.QK_TYPE_Q5_K, 11008) == 7568
    assert qk.qk_row_bytes(qk.QK_TYPE_Q4_0, 100) == 0
    assert qk.qk_row_bytes(99, 256) == 0
    assert qk.qk_row_bytes(qk.QK_TYPE_Q5_0, 4096) == 2816
    assert qk.qk_row_bytes(qk.QK_TYPE_Q4_1, 4096) == 2560
    # Q8_1: named on the pages, never laid out; 36 bytes is the reading (f16 d, f16 s,
    # 32 codes) that the oracle's layout takes too
    assert qk.qk_block_elems(qk.QK_TYPE_Q8_1) == 32 and qk.qk_block_bytes(qk.QK_TYPE_Q8_1) == 36
    assert qk.qk_row_bytes(qk.QK_TYPE_Q8_1, 4096) == 4608
    assert qk.qk_block_elems(16) == 0


def test_pairing():
    assert qk.qk_act_type(qk.QK_TYPE_Q4_0) == qk.QK_TYPE_Q8_0
    assert qk.qk_act_type(qk.QK_TYPE_Q8_0) == qk.QK_TYPE_Q8_0
    assert qk.qk_act_type(qk.QK_TYPE_Q4_K) == qk.QK_TYPE_Q8_K
    assert qk.qk_act_type(qk.QK_TYPE_Q6_K) == qk.QK_TYPE_Q8_K
    assert qk.qk_act_type(qk.QK_TYPE_Q5_K) == qk.QK_TYPE_Q8_K
    assert qk.qk_act_type(qk.QK_TYPE_Q5_0) == qk.QK_TYPE_Q8_0
    assert qk.qk_act_type(qk.QK_TYPE_Q8_K) == -1
    assert qk.qk_act_type(qk.QK_TYPE_Q4_1) == qk.QK_TYPE_Q8_1
    assert qk.qk_act_type(qk.QK_TYPE_Q5_1) == qk.QK_TYPE_Q8_1
    assert qk.qk_act_type(qk.QK_TYPE_Q8_1) == -1
    assert qk.qk_act_type(qk.QK_TYPE_Q2_K) == qk.QK_TYPE_Q8_K
    assert qk.qk_act_type(qk.QK_TYPE_Q3_K) == qk.QK_TYPE_Q8_K


def test_max_n_in_covers_llm_shapes():
    for t in qk.WEIGHT_TYPES:
        m = qk.qk_max_n_in(t)
        assert m >= 28672 and m % qk.qk_block_elems(t) == 0
    # one workgroup stages up to 160 KB of activation blocks: 561 Q8_K blocks
    assert qk.qk_max_n_in(qk.QK_TYPE_Q4_K) == 561 * 256
    assert qk.qk_max_n_in(qk.QK_TYPE_Q8_K) == 0
    assert qk.qk_max_n_in(qk.QK_TYPE_Q8_1) == 0


P = ctypes.c_void_p
GOOD = P(0x10000)     # aligned, never dereferenced: every call below fails validation
ODD = P(0x10008)      # 8-byte aligned only


def _status(fn, *args):
    return getattr(qk.lib(), fn)(*args)


@pytest.mark.parametrize("timed", [False, True])
def test_quantize_validation(timed):
    def st(*a):
        return _status("qk_quantize_act_timed", *a, None, None) if timed else _status("qk_quantize_act", *a)
    assert st(qk.QK_TYPE_Q4_K, GOOD, GOOD, 256, 1, None) == 1  # weight type
    assert st(99, GOOD, GOOD, 256, 1, None) == 1
    assert st(qk.QK_TYPE_Q8_0, GOOD, GOOD, 33, 1, None) == 3
    assert st(qk.QK_TYPE_Q8_1, GOOD, GOOD, 48, 1, None) == 3
    assert st(qk.QK_TYPE_Q8_1, GOOD, ODD, 32, 1, None) == 4
    assert st(qk.QK_TYPE_Q8_K, GOOD, GOOD, 0, 1, None) == 3
    assert st(qk.QK_TYPE_Q8_K, GOOD, GOOD, 256, -1, None) == 3
    assert st(qk.QK_TYPE_Q8_K, None, GOOD, 256, 1, None) == 5
    assert st(qk.QK_TYPE_Q8_K, GOOD, ODD, 256, 1, None) == 4
    assert st(qk.QK_TYPE_Q8_K, GOOD, GOOD, 256, 0, None) == 0  # no-op


def test_quantize_row_validation():
    f = "qk_quantize_row"
    assert _status(f, qk.QK_TYPE_Q4_K, GOOD, GOOD, 256, None) == 1   # only 32-element types
    assert _status(f, qk.QK_TYPE_Q8_K, GOOD, GOOD, 256, None) == 1
    assert _status(f, 99, GOOD, GOOD, 32, None) == 1
    assert _status(f, qk.QK_TYPE_Q4_1, GOOD, GOOD, 48, None) == 3
    assert _status(f, qk.QK_TYPE_Q5_0, GOOD, GOOD, -32, None) == 3
    assert _status(f, qk.QK_TYPE_Q4_0, None, GOOD, 32, None) == 5
    assert _status(f, qk.QK_TYPE_Q4_0, GOOD, None, 32, None) == 5
    assert _status(f, qk.QK_TYPE_Q8_0, ODD, GOOD, 32, None) == 4
    assert _status(f, qk.QK_TYPE_Q8_0, GOOD, ODD, 32, None) == 4
    assert _status(f, qk.QK_TYPE_Q5_0, None, None, 0, None) == 0     # no-op


def test_gemv_validation():
    f = "qk_gemv"
    assert _status(f, qk.QK_TYPE_Q8_K, GOOD, 4, 256, GOOD, 1, GOOD, None) == 1
    assert _status(f, qk.QK_TYPE_Q8_1, GOOD, 4, 256, GOOD, 1, GOOD, None) == 1  # activation only
    assert _status(f, qk.QK_TYPE_Q4_1, GOOD, 4, 48, GOOD, 1, GOOD, None) == 3
    assert _status(f, qk.QK_TYPE_Q5_1, GOOD, 4, 256, GOOD, 1, ODD, None) == 4
    assert _status(f, 5, GOOD, 4, 256, GOOD, 1, GOOD, None) == 1
    assert _status(f, qk.QK_TYPE_Q4_K, GOOD, 4, 255, GOOD, 1, GOOD, None) == 3
    assert _status(f, qk.QK_TYPE_Q4_K, GOOD, 4, 0, GOOD, 1, GOOD, None) == 3
    assert _status(f, qk.QK_TYPE_Q4_K, GOOD, -1, 256, GOOD, 1, GOOD, None) == 3
    assert _status(f, qk.QK_TYPE_Q4_K, GOOD, 4, 256, GOOD, -2, GOOD, None) == 3
    big = qk.qk_max_n_in(qk.QK_TYPE_Q4_K) + 256
    assert _status(f, qk.QK_TYPE_Q4_K, GOOD, 4, big, GOOD, 1, GOOD, None) == 7
    assert _status(f, qk.QK_TYPE_Q8_0, None, 4, 64, GOOD, 1, GOOD, None) == 5
    assert _status(f, qk.QK_TYPE_Q8_0, GOOD, 4, 64, None, 1, GOOD, None) == 5
    assert _status(f, qk.QK_TYPE_Q8_0, GOOD, 4, 64, GOOD, 1, None, None) == 5
    assert _status(f, qk.QK_TYPE_Q6_K, ODD, 4, 256, GOOD, 1, GOOD, None) == 4
    assert _status(f, qk.QK_TYPE_Q6_K, GOOD, 4, 256, ODD, 1, GOOD, None) == 4
    assert _status(f, qk.QK_TYPE_Q6_K, GOOD, 4, 256, GOOD, 1, ODD, None) == 4
    assert _status(f, qk.QK_TYPE_Q6_K, GOOD, 0, 256, GOOD, 1, GOOD, None) == 0   # no-op
    assert _status(f, qk.QK_TYPE_Q6_K, None, 0, 256, None, 1, None, None) == 0   # no-op
    assert _status("qk_gemv_block_sums", qk.QK_TYPE_Q4_0, GOOD, 4, 64, GOOD, 1, None, None) == 5
    assert _status("qk_gemv_timed", qk.QK_TYPE_Q4_0, GOOD, 4, 64, GOOD, 1, ODD, None, None,
                   None) == 4


def test_gemv_typed_validation():
    # every weight type against every activation type: QK_E_PAIR unless it is the
    # weight type's pairing, which then passes on to qk_gemv (n_out = 0: a no-op)
    f = "qk_gemv_typed"
    acts = (qk.QK_TYPE_Q8_0, qk.QK_TYPE_Q8_1, qk.QK_TYPE_Q8_K)
    for w in qk.WEIGHT_TYPES:
        blk = qk.qk_block_elems(w)
        for a in acts:
            want = 0 if a == qk.qk_act_type(w) else 2
            assert _status(f, w, a, GOOD, 0, blk, GOOD, 1, GOOD, None) == want, (w, a)
        assert sum(a == qk.qk_act_type(w) for a in acts) == 1
    assert _status(f, qk.QK_TYPE_Q8_K, qk.QK_TYPE_Q8_K, GOOD, 4, 256, GOOD, 1, GOOD, None) == 1
    assert _status(f, qk.QK_TYPE_Q4_K, qk.QK_TYPE_Q4_K, GOOD, 4, 256, GOOD, 1, GOOD, None) == 1
    assert _status(f, qk.QK_TYPE_Q4_K, 99, GOOD, 4, 256, GOOD, 1, GOOD, None) == 1
    # after the pairing, qk_gemv's own checks
    assert _status(f, qk.QK_TYPE_Q4_K, qk.QK_TYPE_Q8_K, GOOD, 4, 255, GOOD, 1, GOOD, None) == 3
    assert _status(f, qk.QK_TYPE_Q4_0, qk.QK_TYPE_Q8_0, GOOD, 4, 64, GOOD, 1, ODD, None) == 4
    assert _status(f, qk.QK_TYPE_Q4_1, qk.QK_TYPE_Q8_1, None, 4, 64, GOOD, 1, GOOD, None) == 5


@pytest.mark.parametrize("f", ["qk_gemv_pair", "qk_gemv_pair_timed"])
def test_gemv_pair_validation(f):
    T4K = qk.QK_TYPE_Q4_K
    ev = (None, None) if f.endswith("_timed") else ()

    def st(*a):
        return _status(f, *a, *ev)
    assert st(qk.QK_TYPE_Q6_K, GOOD, GOOD, 4, 256, GOOD, 1, 0, GOOD, None) == 1  # Q4_K / Q5_K only
    assert st(T4K, GOOD, GOOD, 4, 256, GOOD, 1, 2, GOOD, None) == 8     # epilogue
    assert st(T4K, GOOD, GOOD, 4, 255, GOOD, 1, 0, GOOD, None) == 3
    assert st(T4K, GOOD, GOOD, -1, 256, GOOD, 1, 1, GOOD, None) == 3
    assert st(T4K, GOOD, GOOD, 4, 256, GOOD, 65536, 1, GOOD, None) == 7  # columns
    big = qk.qk_max_n_in(T4K) + 256
    assert st(T4K, GOOD, GOOD, 4, big, GOOD, 1, 1, GOOD, None) == 7
    assert st(T4K, GOOD, None, 4, 256, GOOD, 1, 1, GOOD, None) == 5
    assert st(T4K, None, GOOD, 4, 256, GOOD, 1, 1, GOOD, None) == 5
    assert st(T4K, GOOD, GOOD, 4, 256, GOOD, 1, 1, None, None) == 5
    assert st(T4K, GOOD, ODD, 4, 256, GOOD, 1, 1, GOOD, None) == 4
    assert st(T4K, GOOD, GOOD, 4, 256, ODD, 1, 0, GOOD, None) == 4
    assert st(T4K, GOOD, GOOD, 0, 256, GOOD, 1, 1, GOOD, None) == 0     # no-op
    assert st(T4K, None, None, 4, 256, None, 0, 0, None, None) == 0     # no-op


def test_read_probe_validation():
    f = "qk_read_probe"
    assert _status(f, GOOD, 0, GOOD, None, None, None) == 3
    assert _status(f, GOOD, -16, GOOD, None, None, None) == 3
    assert _status(f, GOOD, 24, GOOD, None, None, None) == 3      # not whole 16-byte units
    assert _status(f, None, 4096, GOOD, None, None, None) == 5
    assert _status(f, GOOD, 4096, None, None, None, None) == 5
    assert _status(f, ODD, 4096, GOOD, None, None, None) == 4
    assert _status(f, GOOD, 4096, ODD, None, None, None) == 4


def test_read_probe_ex_validation():
    f = "qk_read_probe_ex"
    for kb in (0, 3, 32, -1):
        assert _status(f, GOOD, 4096, GOOD, kb, 0, 0, None, None, None) == 8
    assert _status(f, GOOD, 4096, GOOD, 2, -1, 0, None, None, None) == 8
    assert _status(f, GOOD, 4096, GOOD, 2, 0, 2, None, None, None) == 8
    assert _status(f, GOOD, 24, GOOD, 2, 0, 0, None, None, None) == 3
    assert _status(f, None, 4096, GOOD, 2, 0, 0, None, None, None) == 5
    assert _status(f, GOOD, 4096, ODD, 16, 256, 1, None, None, None) == 4


def test_dequantize_validation():
    f = "qk_dequantize_row"
    assert _status(f, qk.QK_TYPE_Q8_K, GOOD, GOOD, 256, None) == 1   # activation-only type
    assert _status(f, 9, GOOD, GOOD, 32, None) == 1   # Q8_1: never laid out on the pages
    assert _status(f, qk.QK_TYPE_Q4_0, GOOD, GOOD, 48, None) == 3
    assert _status(f, qk.QK_TYPE_Q4_0, GOOD, GOOD, -32, None) == 3
    assert _status(f, qk.QK_TYPE_Q4_0, None, GOOD, 32, None) == 5
    assert _status(f, qk.QK_TYPE_Q4_0, GOOD, ODD, 32, None) == 4
    assert _status(f, qk.QK_TYPE_Q4_0, GOOD, GOOD, 0, None) == 0


def test_launch_size_limit():
    # sizes whose grid would exceed one launch's 32-bit work-item count are refused
    # with QK_E_LIMIT before any HIP call (the fake pointers are never touched)
    big = 1 << 40
    assert _status("qk_dequantize_row", qk.QK_TYPE_Q8_0, GOOD, GOOD, big, None) == 7
    assert _status("qk_dequantize_row", qk.QK_TYPE_Q6_K, GOOD, GOOD, big, None) == 7
    assert _status("qk_quantize_row", qk.QK_TYPE_Q4_0, GOOD, GOOD, big, None) == 7
    assert _status("qk_quantize_act", qk.QK_TYPE_Q8_K, GOOD, GOOD, 256, 1 << 27, None) == 7
    assert _status("qk_quantize_act", qk.QK_TYPE_Q8_0, GOOD, GOOD, 32, 1 << 30, None) == 7
    assert _status("qk_read_probe", GOOD, big, GOOD, None, None, None) == 7
    # one wavefront per row (rows beyond one pass): 2^26 rows of 64 lanes is the limit
    assert _status("qk_gemv", qk.QK_TYPE_Q4_K, GOOD, 1 << 27, 11008, GOOD, 1, GOOD, None) == 7
    # the batched kernel: 64 rows per 512-thread workgroup
    assert _status("qk_gemv", qk.QK_TYPE_Q4_K, GOOD, (1 << 31) - 1, 4096, GOOD, 16, GOOD, None) == 7


def test_status_strings():
    for s in (0, 1, 2, 3, 4, 5, 6, 7, 8):
        assert qk.status_str(s) and qk.status_str(s) != "unknown status"
    assert qk.status_str(42) == "unknown status"


def _imports(path):
    src = open(path).read()
    return set(re.findall(r"^\s*(?:from|import)\s+([A-Za-z_][\w.]*)", src, flags=re.M))


def test_oracle_and_product_are_independent():
    # The product path never imports the oracle, and the oracle never imports the
    # product; they share no source file.
    pkg = os.path.join(ROOT, "quantized_gemv_quantize_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            p = os.path.join(dirpath, f)
            if f.endswith(".py"):
                assert not any(m.split(".")[0] == "oracle" for m in _imports(p)), p
            if f.endswith((".hip", ".h", ".cpp")):
                assert "oracle" not in open(p).read().lower().replace("oracle-free", ""), p
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        p = os.path.join(ROOT, "oracle", f)
        if f.endswith(".py"):
            assert not any("quantized_gemv_quantize_amd" in m for m in _imports(p)), p
        if f.endswith((".c", ".h")):
            txt = open(p).read()
            assert "#include \"../" not in txt and "qk.h\"" not in txt, p
