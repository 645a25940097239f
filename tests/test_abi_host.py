"""Host-side checks of the C ABI (no GPU needed, no kernel is launched):
the library loads, exports every entry point include/bsfp.h declares, and
rejects bad arguments with a status and a message before touching the GPU."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsfp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsfp_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def blib():
    import block_scaled_bit_fp_amd as b
    return b


def test_header_declares_the_boundary():
    fns = declared_functions()
    for f in ("bsfp_quantize", "bsfp_dequantize", "bsfp_qmv", "bsfp_qmm", "bsfp_amax",
              "bsfp_qmm_workspace_bytes", "bsfp_time_next_launch", "bsfp_last_error",
              "bsfp_version"):
        assert f in fns


def test_library_exports_every_declared_symbol(blib):
    out = subprocess.run(["nm", "-D", "--defined-only", blib.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (bsfp_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    L = blib.lib()
    for f in declared_functions():
        assert hasattr(L, f)
    assert "gfx950" in blib.version()


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "bsfp.h"\nint main(void){bsfp_qtensor q; (void)q; return 0;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    "-c", str(src), "-o", str(tmp_path / "t.o")], check=True)


FAKE = 0x10000  # 16-byte aligned fake device address; never dereferenced


def desc(blib, mode=2, bits=4, group=16, rows=4, cols=64, codes=FAKE, scales=FAKE,
         biases=None, gs=None, amax=None):
    return blib.QTensorDesc(mode, bits, group, rows, cols, codes, scales, biases, gs, amax)


def status(blib, rc):
    return blib.STATUS[rc], blib.lib().bsfp_last_error().decode()


@pytest.mark.parametrize("mode,bits,group", [(3, 4, 16), (3, 8, 16), (2, 8, 16), (2, 4, 32),
                                             (1, 4, 16), (1, 8, 32), (0, 4, 16), (0, 8, 256),
                                             (0, 2, 64), (4, 4, 32), (-1, 4, 64)])
def test_unsupported_formats_are_reported_not_thrown(blib, mode, bits, group):
    d = desc(blib, mode, bits, group)
    rc = blib.lib().bsfp_quantize(C.c_void_p(FAKE), C.byref(d), 0, None)
    st, msg = status(blib, rc)
    assert st == "BSFP_ERR_UNSUPPORTED"
    assert "supported" in msg and "(nvfp4, 4, 16)" in msg and "(mxfp8, 8, 32)" in msg
    rc = blib.lib().bsfp_qmv(C.c_void_p(FAKE), 1, C.byref(d), C.c_void_p(FAKE), None)
    assert status(blib, rc)[0] == "BSFP_ERR_UNSUPPORTED"


@pytest.mark.parametrize("mode,bits,group", [(3, 8, 32), (0, 4, 32), (0, 4, 128), (0, 8, 32),
                                             (0, 8, 64), (0, 8, 128)])
def test_format_variants_routing(blib, mode, bits, group):
    """Variants pass the descriptor check; bsfp_qmm sends them to the dense
    path and bsfp_qmv rejects an x beyond its 64 KB LDS copy, both before
    anything is launched."""
    L = blib.lib()
    d = desc(blib, mode, bits, group, rows=4, cols=256, biases=FAKE if mode == 0 else None)
    rc = L.bsfp_qmm(C.c_void_p(FAKE), 4, C.byref(d), 0, None, 0, C.c_void_p(FAKE), None)
    st, msg = status(blib, rc)
    assert st == "BSFP_ERR_UNSUPPORTED" and "bsfp_qmm_dense" in msg
    big = desc(blib, mode, bits, group, rows=4, cols=32768, biases=FAKE if mode == 0 else None)
    rc = L.bsfp_qmv(C.c_void_p(FAKE), 2, C.byref(big), C.c_void_p(FAKE), None)
    st, msg = status(blib, rc)
    assert st == "BSFP_ERR_UNSUPPORTED" and "64 KB" in msg


def test_bad_arguments(blib):
    L = blib.lib()
    X = C.c_void_p(FAKE)
    # cols not a multiple of the group
    d = desc(blib, cols=40)
    assert status(blib, L.bsfp_quantize(X, C.byref(d), 0, None))[0] == "BSFP_ERR_ARG"
    # null codes
    d = desc(blib, codes=None)
    assert status(blib, L.bsfp_dequantize(C.byref(d), X, None))[0] == "BSFP_ERR_ARG"
    # misaligned codes / x
    d = desc(blib, codes=FAKE + 4)
    assert status(blib, L.bsfp_dequantize(C.byref(d), X, None))[0] == "BSFP_ERR_ARG"
    d = desc(blib)
    assert status(blib, L.bsfp_quantize(C.c_void_p(FAKE + 2), C.byref(d), 0, None))[0] == "BSFP_ERR_ARG"
    # NVFP4 global scale requested without buffers
    assert status(blib, L.bsfp_quantize(X, C.byref(d), 1, None))[0] == "BSFP_ERR_ARG"
    d2 = desc(blib, gs=FAKE)
    assert status(blib, L.bsfp_quantize(X, C.byref(d2), 1, None))[0] == "BSFP_ERR_ARG"
    assert status(blib, L.bsfp_quantize(X, C.byref(d2), 7, None))[0] == "BSFP_ERR_ARG"
    # affine without biases
    d = desc(blib, mode=0, group=64)
    assert status(blib, L.bsfp_dequantize(C.byref(d), X, None))[0] == "BSFP_ERR_ARG"
    # qmv M range
    d = desc(blib)
    for M in (0, 9, -1):
        assert status(blib, L.bsfp_qmv(X, M, C.byref(d), X, None))[0] == "BSFP_ERR_ARG"
    # null descriptor
    assert status(blib, L.bsfp_qmv(X, 1, None, X, None))[0] == "BSFP_ERR_ARG"
    # amax
    assert status(blib, L.bsfp_amax(X, -1, X, None))[0] == "BSFP_ERR_ARG"
    assert status(blib, L.bsfp_amax(X, 8, None, None))[0] == "BSFP_ERR_ARG"
    # qmm: bad activation mode, K not a multiple of 32, missing workspace
    assert status(blib, L.bsfp_qmm(X, 4, C.byref(d), 5, None, 0, X, None))[0] == "BSFP_ERR_ARG"
    d48 = desc(blib, cols=48)
    assert status(blib, L.bsfp_qmm(X, 4, C.byref(d48), 0, None, 0, X, None))[0] in (
        "BSFP_ERR_ARG", "BSFP_ERR_UNSUPPORTED")
    need = L.bsfp_qmm_workspace_bytes(2, 4, 64, 1)
    if need:
        rc = L.bsfp_qmm(X, 4, C.byref(d), 1, X, need - 1, X, None)
        assert status(blib, rc)[0] == "BSFP_ERR_ARG"


def test_workspace_query(blib):
    L = blib.lib()
    assert L.bsfp_qmm_workspace_bytes(9, 4, 64, 0) == 0
    assert L.bsfp_qmm_workspace_bytes(2, -1, 64, 0) == 0
    assert L.bsfp_qmm_workspace_bytes(2, 4, 64, 3) == 0
    assert L.bsfp_qmm_workspace_bytes(2, 4, 64, 0) == 0  # weight-only needs none


def test_no_cpu_fallback_in_product(blib):
    """The product package never reaches the oracle (no import, no call)."""
    pkg = os.path.dirname(blib.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, f


def test_time_next_launch_set_and_clear(blib):
    """The measurement hook only stores the pair (no GPU work): OK either way."""
    L = blib.lib()
    assert L.bsfp_time_next_launch(None, None) == 0
    assert L.bsfp_time_next_launch(FAKE, FAKE) == 0
    assert L.bsfp_time_next_launch(None, None) == 0


def test_qmm_size_limits(blib):
    """Shapes beyond the GEMM entry points' limits (M, N <= 2^30, M * N <=
    2^33, K <= 2^22) are refused before anything is launched."""
    L = blib.lib()
    X = C.c_void_p(FAKE)
    S = C.c_void_p(FAKE)
    cases = [((1 << 30) + 1, 4, 64, "2^30"),     # M
             (4, (1 << 30) + 1, 64, "2^30"),     # N
             (1 << 20, 1 << 14, 64, "2^33"),     # M * N = 2^34
             ((1 << 19) + 1, 1 << 14, 64, "2^33"),
             (4, 4, (1 << 22) + 64, "2^22")]     # K
    for M, N, K, word in cases:
        d = desc(blib, rows=N, cols=K)
        st, msg = status(blib, L.bsfp_qmm(X, M, C.byref(d), 0, None, 0, X, None))
        assert st == "BSFP_ERR_UNSUPPORTED" and word in msg, (M, N, K, msg)
        st, msg = status(blib, L.bsfp_qmm_dense(X, M, C.byref(d), S, 1 << 62, X, None))
        assert st == "BSFP_ERR_UNSUPPORTED" and word in msg, (M, N, K, msg)


def test_element_count_limit(blib):
    """A descriptor of more than 2^40 elements is refused by every entry
    point before rows * cols is used."""
    L = blib.lib()
    X = C.c_void_p(FAKE)
    for rows, cols in (((1 << 40) // 64 + 1, 64), (1 << 62, 1 << 40)):
        d = desc(blib, rows=rows, cols=cols)
        for rc in (L.bsfp_quantize(X, C.byref(d), 0, None), L.bsfp_dequantize(C.byref(d), X, None),
                   L.bsfp_qmv(X, 1, C.byref(d), X, None),
                   L.bsfp_qmm(X, 4, C.byref(d), 0, None, 0, X, None)):
            st, msg = status(blib, rc)
            assert st == "BSFP_ERR_UNSUPPORTED" and "2^40" in msg, msg


def test_noalloc_checks_before_touching_the_gpu(blib):
    """bsfp_qmm_noalloc applies bsfp_qmm's argument checks, and refuses a
    product whose workspace exceeds its static array, before it looks up the
    array or launches anything."""
    L = blib.lib()
    X = C.c_void_p(FAKE)
    d = desc(blib, rows=64, cols=5120)
    assert status(blib, L.bsfp_qmm_noalloc(X, 4, C.byref(d), 5, X, None))[0] == "BSFP_ERR_ARG"
    assert status(blib, L.bsfp_qmm_noalloc(None, 4, C.byref(d), 1, X, None))[0] == "BSFP_ERR_ARG"
    assert status(blib, L.bsfp_qmm_noalloc(X, 4, C.byref(d), 1, None, None))[0] == "BSFP_ERR_ARG"
    assert status(blib, L.bsfp_qmm_noalloc(X, -1, C.byref(d), 1, X, None))[0] == "BSFP_ERR_ARG"
    # nothing to compute: OK without any GPU work
    assert status(blib, L.bsfp_qmm_noalloc(X, 0, C.byref(d), 1, X, None))[0] == "BSFP_OK"
    # NVFP4 qq at M = 3277, K = 5120: 33.6 MB of workspace > 32 MiB
    M = blib.NOALLOC_WORKSPACE_BYTES // (2 * 5120) + 1
    assert L.bsfp_qmm_workspace_bytes(2, M, 5120, 1) > blib.NOALLOC_WORKSPACE_BYTES
    st, msg = status(blib, L.bsfp_qmm_noalloc(X, M, C.byref(d), 1, X, None))
    assert st == "BSFP_ERR_UNSUPPORTED" and "static" in msg and str(M) in msg, msg


def test_noalloc_size_matches_header(blib):
    text = open(HEADER).read()
    m = re.search(r"#define BSFP_NOALLOC_WORKSPACE_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == blib.NOALLOC_WORKSPACE_BYTES


def test_qmv_batch_checks_before_touching_the_gpu(blib):
    """bsfp_qmv_batch refuses a bad count, null arrays or entries, matrices
    that differ in format or K, and what bsfp_qmv refuses, before launching."""
    L = blib.lib()
    X = C.c_void_p(FAKE)
    QP = C.POINTER(blib.QTensorDesc)

    def call(descs, M=1, count=None, ys=None):
        darr = (QP * max(1, len(descs)))(*[C.pointer(d) if d is not None else QP() for d in descs])
        n = len(descs) if count is None else count
        yarr = (C.c_void_p * max(1, len(descs)))(*([FAKE] * len(descs) if ys is None else ys))
        return status(blib, L.bsfp_qmv_batch(X, M, darr, n, yarr, None))

    a, b = desc(blib, rows=4, cols=256), desc(blib, rows=8, cols=256)
    for n in (0, 5, -1):
        assert call([a, b], count=n)[0] == "BSFP_ERR_ARG"
    assert status(blib, L.bsfp_qmv_batch(X, 1, None, 1, None, None))[0] == "BSFP_ERR_ARG"
    assert call([a, None])[0] == "BSFP_ERR_ARG"
    st, msg = call([a, desc(blib, rows=4, cols=512)])
    assert st == "BSFP_ERR_ARG" and "differs" in msg
    st, msg = call([a, desc(blib, mode=1, group=32, rows=4, cols=256)])
    assert st == "BSFP_ERR_ARG" and "differs" in msg
    assert call([a, b], ys=[FAKE, None])[0] == "BSFP_ERR_ARG"
    assert call([a, b], ys=[FAKE, FAKE + 8])[0] == "BSFP_ERR_ARG"  # not 16-byte aligned
    assert call([a, b], M=9)[0] == "BSFP_ERR_ARG"
    big = desc(blib, 3, 8, 32, rows=4, cols=1 << 16)
    st, msg = call([big, big], M=2)
    assert st == "BSFP_ERR_UNSUPPORTED" and "64 KB" in msg


def test_quantize_ws_checks_before_touching_the_gpu(blib):
    """bsfp_quantize_ws needs its workspace only for NVFP4 with a computed
    global scale, and refuses a missing, misaligned or short one; it keeps
    bsfp_quantize_sr's checks when rbits is given."""
    L = blib.lib()
    X = C.c_void_p(FAKE)
    need = blib.QUANTIZE_WS_BYTES
    nv = desc(blib, gs=FAKE, amax=FAKE + 16)

    def call(d, gs=1, rbits=None, ws=FAKE, nbytes=need):
        return status(blib, L.bsfp_quantize_ws(X, C.byref(d), gs, rbits, ws, nbytes, None))

    assert call(nv, ws=None)[0] == "BSFP_ERR_ARG"
    assert call(nv, ws=FAKE + 2)[0] == "BSFP_ERR_ARG"
    st, msg = call(nv, nbytes=need - 4)
    assert st == "BSFP_ERR_ARG" and str(need) in msg
    assert call(desc(blib, gs=FAKE))[0] == "BSFP_ERR_ARG"          # no amax buffer
    assert call(nv, gs=7)[0] == "BSFP_ERR_ARG"                      # bad flag
    assert call(desc(blib, cols=40, gs=FAKE, amax=FAKE))[0] == "BSFP_ERR_ARG"
    assert call(nv, rbits=FAKE + 4)[0] == "BSFP_ERR_ARG"            # rbits misaligned
    aff = desc(blib, mode=0, group=64, biases=FAKE)
    assert call(aff, gs=0, rbits=FAKE, ws=None, nbytes=0)[0] == "BSFP_ERR_UNSUPPORTED"


def test_quantize_ws_size_matches_header(blib):
    text = open(HEADER).read()
    m = re.search(r"#define BSFP_QUANTIZE_WS_BYTES (\d+)", text)
    assert m and int(m.group(1)) == blib.QUANTIZE_WS_BYTES
