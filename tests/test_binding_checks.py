"""The Python binding checks every tensor argument's dtype and shape on the
host before it calls the library (CPU only: every call below is rejected
before a pointer is passed, so no kernel is launched).

The C ABI receives raw pointers and the sizes passed beside them; a tensor of
the wrong length would otherwise be read or written out of bounds on the
device.  Each case below gets one argument wrong and expects the wrapper's
error naming that argument."""
import os

import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "post_mixed_precision_amd", "libslim.so")),
    reason="libslim.so not built (run __graft_entry__.build())")


@pytest.fixture(scope="module")
def L():
    from post_mixed_precision_amd import _lib
    _lib.load_library()
    return _lib


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def raises(L, fn, *words):
    with pytest.raises(L.SlimError) as e:
        fn()
    msg = str(e.value)
    for w in words:
        assert w in msg, msg


def test_hessian_checks(L):
    raises(L, lambda: L.hessian(torch.zeros((8, 16), dtype=torch.float16)), "X", "dtype")
    raises(L, lambda: L.hessian(bf(8, 16), H=f32(16, 15)), "H", "shape")
    raises(L, lambda: L.hessian(bf(8, 16), H=torch.zeros((16, 16), dtype=torch.float64)), "H", "dtype")
    raises(L, lambda: L.hessian(bf(8, 16), accumulate=True), "accumulate")
    raises(L, lambda: L.hessian(bf(8, 16)), "GPU")          # right shapes, host memory


def test_salience_checks(L):
    raises(L, lambda: L.salience(f32(256, 256), bf(8, 256), 96), "group")
    raises(L, lambda: L.salience(f32(256, 255), bf(8, 256), 128), "H", "shape")
    raises(L, lambda: L.salience(f32(128, 128), bf(8, 256), 128), "H", "shape")


def test_group_salience_checks(L):
    raises(L, lambda: L.group_salience(f32(255), bf(8, 256), 128), "hinv", "shape")
    raises(L, lambda: L.group_salience(torch.zeros(256, dtype=torch.float64), bf(8, 256), 128), "hinv", "dtype")
    raises(L, lambda: L.group_salience(f32(256), bf(8, 256), 96), "group")
    raises(L, lambda: L.group_salience(f32(256), bf(8, 256), 128), "GPU")


def test_sba_checks(L):
    X, W, S = bf(32, 256), bf(8, 256), torch.zeros(2, dtype=torch.float64)
    raises(L, lambda: L.sba_search(X, bf(8, 384), S, 128, 2), "W", "shape")
    raises(L, lambda: L.sba_search(X, W, torch.zeros(2, dtype=torch.float32), 128, 2), "group_sal", "dtype")
    raises(L, lambda: L.sba_search(X, W, torch.zeros(3, dtype=torch.float64), 128, 2), "group_sal", "shape")
    raises(L, lambda: L.sba_search(X, W, S, 100, 2), "group")
    raises(L, lambda: L.sba_search_ex(X, W, 128, 2, order=torch.zeros(3, dtype=torch.int32)), "order", "shape")
    raises(L, lambda: L.sba_search_ex(X, W, 128, 2, order=torch.zeros(2, dtype=torch.int64)), "order", "dtype")
    raises(L, lambda: L.sba_search_ex(X, W, 128, 2), "group_sal")


def test_sqc_and_gptq_checks(L):
    W = bf(8, 256)
    bits, hinv = torch.full((2,), 2, dtype=torch.int8), f32(256)
    raises(L, lambda: L.sqc_calibrate(W, bits.to(torch.int32), hinv, 128), "bits", "dtype")
    raises(L, lambda: L.sqc_calibrate(W, torch.full((3,), 2, dtype=torch.int8), hinv, 128), "bits", "shape")
    raises(L, lambda: L.sqc_calibrate(W, bits, f32(128), 128), "hinv", "shape")
    raises(L, lambda: L.gptq_quantize(f32(255, 255), W, bits, hinv, 128), "H", "shape")
    raises(L, lambda: L.gptq_quantize(None, W, bits, hinv, 128), "U")
    raises(L, lambda: L.gptq_quantize(None, W, bits, hinv, 128, U=f32(256, 256)), "U", "dtype")


def test_pack_and_qlinear_checks(L):
    codes = torch.zeros((8, 256), dtype=torch.uint8)
    bits = torch.full((2,), 2, dtype=torch.int8)
    raises(L, lambda: L.pack(codes.to(torch.int8), bits, 128, 2), "codes", "dtype")
    raises(L, lambda: L.pack(codes, torch.full((4,), 2, dtype=torch.int8), 128, 2), "bits", "shape")
    words = 8 * 256 * 2 // 32
    packed = torch.zeros(words, dtype=torch.int32)
    s, z = f32(8, 2), f32(8, 2)
    raises(L, lambda: L.qlinear(bf(1, 256), packed[:-1], bits, s, z, 128, 2), "packed")
    raises(L, lambda: L.qlinear(bf(1, 256), packed, bits, s, f32(8, 3), 128, 2), "zero", "shape")
    raises(L, lambda: L.qlinear(bf(1, 256), packed, bits, f32(8, 4), z, 128, 2), "scale", "shape")
    raises(L, lambda: L.qlinear(bf(1, 256), packed, bits, s.double(), z, 128, 2), "scale", "dtype")
