"""The C-ABI library loads, exports what include/slim.h declares, and rejects
bad arguments before it touches the GPU (CPU only: no compute call runs).

Every call below fails validation, so nothing is enqueued; the pointers are
never dereferenced."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "slim.h")

pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "post_mixed_precision_amd", "libslim.so")),
    reason="libslim.so not built (run __graft_entry__.build())")


@pytest.fixture(scope="module")
def lib():
    from post_mixed_precision_amd import _lib
    return _lib.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(slim_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 16
    for name in names:
        assert hasattr(lib, name), name


def test_binding_covers_header():
    from post_mixed_precision_amd import _lib
    assert sorted(_lib._SIGS) == declared_functions()


def test_version_and_status_strings(lib):
    assert lib.slim_version() == 1
    for code in range(0, -8, -1):
        s = lib.slim_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.slim_status_string(-99).decode() == "unknown status"
    assert lib.slim_last_hip_error() == 0


FAKE = ctypes.c_void_p(4096)   # aligned, never dereferenced (validation fails first)


def test_hessian_validation(lib):
    assert lib.slim_hessian(FAKE, 0, 10, 16, None, 0, FAKE, 1 << 30, None) == -1
    assert lib.slim_hessian(FAKE, 7, 10, 16, FAKE, 0, FAKE, 1 << 30, None) == -3
    assert lib.slim_hessian(FAKE, 1, -1, 16, FAKE, 0, FAKE, 1 << 30, None) == -2
    assert lib.slim_hessian(FAKE, 1, 10, 0, FAKE, 0, FAKE, 1 << 30, None) == -2
    assert lib.slim_hessian(ctypes.c_void_p(4098), 1, 10, 16, FAKE, 0, FAKE, 1 << 30, None) == -7
    assert lib.slim_hessian(FAKE, 1, 10, 16, FAKE, 0, FAKE, 1, None) == -5
    assert lib.slim_hessian_workspace(4096, 4096, 1) > 0
    assert lib.slim_hessian_workspace(-1, 4096, 1) == 0
    assert lib.slim_hessian_workspace(4096, 4096, 5) == 0


def test_salience_validation(lib):
    args = lambda **kw: [kw.get("H", FAKE), kw.get("m", 256), kw.get("damp", 0.01), FAKE, kw.get("wdt", 1),
                         kw.get("n", 64), kw.get("g", 128), FAKE, FAKE, None, kw.get("info", FAKE), FAKE,
                         kw.get("ws", 1 << 40), None]
    assert lib.slim_salience(*args(H=None)) == -1
    assert lib.slim_salience(*args(info=None)) == -1
    assert lib.slim_salience(*args(wdt=3)) == -3
    assert lib.slim_salience(*args(m=200)) == -2           # m % g != 0
    assert lib.slim_salience(*args(g=96)) == -2
    assert lib.slim_salience(*args(n=0)) == -2
    assert lib.slim_salience(*args(damp=-1.0)) == -4
    assert lib.slim_salience(*args(ws=16)) == -5
    assert lib.slim_salience_workspace(64, 256, 128) > 0
    assert lib.slim_salience_workspace(64, 250, 128) == 0


def test_salience_u_validation(lib):
    def call(**kw):
        return lib.slim_salience_u(kw.get("H", FAKE), kw.get("m", 256), kw.get("damp", 0.01), FAKE, kw.get("wdt", 1),
                                   kw.get("n", 64), kw.get("g", 128), FAKE, FAKE, None, kw.get("U", FAKE),
                                   kw.get("info", FAKE), FAKE, kw.get("ws", 1 << 40), None)
    assert call(H=None) == -1 and call(U=None) == -1 and call(info=None) == -1
    assert call(wdt=3) == -3
    assert call(m=200) == -2 and call(g=96) == -2 and call(n=0) == -2
    assert call(damp=-1.0) == -4
    assert call(ws=16) == -5
    assert call(U=ctypes.c_void_p(4100)) == -7


def test_group_salience_validation(lib):
    def call(**kw):
        return lib.slim_group_salience(kw.get("hinv", FAKE), kw.get("m", 256), kw.get("W", FAKE), kw.get("wdt", 1),
                                       kw.get("n", 64), kw.get("g", 128), kw.get("gsal", FAKE), None,
                                       kw.get("info", FAKE), FAKE, kw.get("ws", 1 << 40), None)
    assert call(hinv=None) == -1 and call(W=None) == -1 and call(gsal=None) == -1 and call(info=None) == -1
    assert call(wdt=3) == -3
    assert call(m=200) == -2 and call(g=96) == -2 and call(n=0) == -2 and call(m=0) == -2
    assert call(ws=16) == -5
    assert call(hinv=ctypes.c_void_p(4100)) == -7
    # one float64 partial per (64-row block, group), rounded up to 256 bytes
    assert lib.slim_group_salience_workspace(130, 256, 128) == 256
    assert lib.slim_group_salience_workspace(64 * 40, 4096, 32) == 40 * 128 * 8
    assert lib.slim_group_salience_workspace(64, 250, 128) == 0


def test_sba_validation(lib):
    def call(**kw):
        return lib.slim_sba_search(FAKE, kw.get("xdt", 1), kw.get("t", 100), FAKE, kw.get("wdt", 1),
                                   kw.get("n", 64), kw.get("m", 256), kw.get("g", 128), FAKE, kw.get("N", 2),
                                   FAKE, FAKE, kw.get("rs", FAKE), FAKE, kw.get("ws", 1 << 40), None)
    assert call(rs=None) == -1
    assert call(xdt=0, wdt=1) == -3
    assert call(t=0) == -2
    assert call(m=96) == -2
    assert call(m=32 * 4096, g=32) == -2                   # beyond the width limit
    assert call(N=1) == -4 and call(N=8) == -4
    assert call(ws=10) == -5
    assert lib.slim_sba_workspace(262144, 4096, 4096, 128, 1) > 0


def test_sqc_and_pack_validation(lib):
    assert lib.slim_sqc_calibrate(FAKE, 1, 0, 256, 128, FAKE, FAKE, 0.1, 50, FAKE, FAKE, FAKE, FAKE, None,
                                  None) == 0                 # n = 0 is a no-op
    assert lib.slim_sqc_calibrate(FAKE, 1, 4, 256, 128, FAKE, FAKE, 0.1, 0, FAKE, FAKE, FAKE, FAKE, None,
                                  None) == -4
    assert lib.slim_sqc_calibrate(FAKE, 1, 4, 256, 128, FAKE, FAKE, 1.5, 50, FAKE, FAKE, FAKE, FAKE, None,
                                  None) == -4
    assert lib.slim_sqc_calibrate(None, 1, 4, 256, 128, FAKE, FAKE, 0.1, 50, FAKE, FAKE, FAKE, FAKE, None,
                                  None) == -1
    assert lib.slim_pack(FAKE, 4, 256, 128, FAKE, 9, FAKE, None, None) == -4
    assert lib.slim_pack(FAKE, 4, 250, 128, FAKE, 2, FAKE, None, None) == -2
    assert lib.slim_pack(FAKE, 0, 256, 128, FAKE, 2, FAKE, None, None) == 0
    assert lib.slim_pack_words(4096, 4096, 2) == 4096 * 4096 * 2 // 32


def test_tau_table_matches_oracle_grid(lib):
    from post_mixed_precision_amd import _lib
    for lam, nt in ((0.1, 50), (0.1, 20), (0.25, 7), (0.0, 1)):
        np.testing.assert_array_equal(_lib.tau_table(lam, nt), oracle.tau_grid(lam, nt))


def test_timing_interface(lib):
    from post_mixed_precision_amd import _lib
    _lib.timing_reset()
    assert _lib.timing_read("sba_klgemm") == (0.0, 0)
    ms, cnt = ctypes.c_double(), ctypes.c_int64()
    assert lib.slim_timing_read(b"nope", ctypes.byref(ms), ctypes.byref(cnt)) == -4
    assert lib.slim_timing_select(b"nope", 0) == -4
    assert lib.slim_timing_select(None, 0) == -1
    assert lib.slim_timing_select(b"chol_update", 0) == 0
    assert lib.slim_timing_enable(0) == 0


def test_sba_variant_validation(lib):
    def call(**kw):
        return lib.slim_sba_search_ex(FAKE, 1, 100, FAKE, 1, 64, 256, 128, kw.get("S", FAKE), kw.get("order", None),
                                      2, kw.get("obj", 0), FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert call(S=None, order=None) == -1
    assert call(obj=2) == -4 and call(obj=-1) == -4
    assert lib.slim_sba_search_ex(FAKE, 1, 100, FAKE, 1, 64, 96, 128, FAKE, None, 2, 0, FAKE, FAKE, FAKE, FAKE,
                                  1 << 40, None) == -2


def test_qlinear_validation(lib):
    def call(**kw):
        return lib.slim_qlinear(kw.get("X", FAKE), kw.get("xdt", 1), kw.get("t", 1), kw.get("m", 256), FAKE, FAKE,
                                kw.get("N", 2), FAKE, FAKE, kw.get("n", 64), kw.get("g", 128), FAKE, FAKE,
                                kw.get("ws", 1 << 40), None)
    assert call(X=None) == -1
    assert call(xdt=3) == -3
    assert call(t=0) == -2 and call(t=65537) == -2   # above SLIM_QLINEAR_MAX_T
    assert call(m=96) == -2
    assert call(N=9) == -4
    assert call(ws=0) == -5
    assert lib.slim_qlinear_workspace(1, 4096, 4096, 128) > 0
    assert lib.slim_qlinear_workspace(65537, 4096, 4096, 128) == 0
    # prefill sizes: the group sums of X, t * k floats
    assert lib.slim_qlinear_workspace(2048, 4096, 4096, 128) == 2048 * 32 * 4


def test_gptq_validation(lib):
    def call(**kw):
        return lib.slim_gptq_quantize(kw.get("H", FAKE), kw.get("m", 256), kw.get("damp", 0.01), kw.get("W", FAKE),
                                      kw.get("wdt", 1), kw.get("n", 64), kw.get("g", 128), FAKE, FAKE,
                                      kw.get("lam", 0.1), kw.get("n_tau", 50), FAKE, FAKE, FAKE, FAKE, None,
                                      kw.get("info", FAKE), kw.get("ws", FAKE), kw.get("wsb", 1 << 40), None)
    assert call(H=None) == -1 and call(W=None) == -1 and call(info=None) == -1
    assert call(wdt=3) == -3
    assert call(n=0) == -2 and call(m=200) == -2 and call(g=96) == -2
    assert call(damp=-1.0) == -4 and call(n_tau=0) == -4 and call(lam=1.0) == -4
    assert call(ws=None) == -5 and call(wsb=16) == -5
    assert call(H=ctypes.c_void_p(4100)) == -7
    assert lib.slim_gptq_workspace(64, 256, 128) > lib.slim_salience_workspace(64, 256, 128)

    def call_u(**kw):
        return lib.slim_gptq_quantize_u(kw.get("U", FAKE), kw.get("m", 256), kw.get("W", FAKE), kw.get("wdt", 1),
                                        kw.get("n", 64), kw.get("g", 128), FAKE, FAKE, kw.get("lam", 0.1),
                                        kw.get("n_tau", 50), FAKE, FAKE, FAKE, FAKE, None, kw.get("info", FAKE),
                                        kw.get("ws", FAKE), kw.get("wsb", 1 << 40), None)
    assert call_u(U=None) == -1 and call_u(W=None) == -1 and call_u(info=None) == -1
    assert call_u(wdt=3) == -3
    assert call_u(n=0) == -2 and call_u(m=200) == -2 and call_u(g=96) == -2
    assert call_u(n_tau=0) == -4 and call_u(lam=1.0) == -4
    assert call_u(ws=None) == -5 and call_u(wsb=16) == -5
    assert call_u(U=ctypes.c_void_p(4100)) == -7
    assert lib.slim_gptq_workspace(64, 250, 128) == 0
