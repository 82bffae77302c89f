"""slim_qlinear_noalloc (partial sums in the library's fixed device scratch)
against slim_qlinear (partial sums in a caller workspace), through the C ABI.

Both run the same plan and kernels, so the bar is bit equality.  Two calls in
a row on one GPU, the second with a smaller layer and batch: the scratch then
still holds the first call's partial sums, which the second must not see.
Both layers are split into several runs of groups, so the scratch is used.
"""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    from post_mixed_precision_amd import _lib
    return _lib.load_library()


def _layer(n, m, g, N, t, seed):
    """Random planes (every bit pattern is a valid code), widths N+1 on the
    first third of the groups and N-1 on the last third, positive scales,
    zeros inside the code range, and a bf16 batch."""
    rng = np.random.default_rng(seed)
    k = m // g
    bits = np.full(k, N, dtype=np.int8)
    bits[: k // 3] = N + 1
    bits[k - k // 3:] = N - 1
    words = n * m * N // 32
    packed = rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32).view(np.int32)
    scale = rng.uniform(1e-3, 2e-2, size=(n, k)).astype(np.float32)
    zero = (rng.uniform(0, 1, size=(n, k)) * (2.0 ** bits[None, :] - 1)).astype(np.float32)
    X = rng.standard_normal((t, m)).astype(np.float32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")  # noqa: E731
    return d(X).to(torch.bfloat16), d(packed), d(bits), d(scale), d(zero)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(lib, n, m, g, N, t, seed):
    X, packed, bits, scale, zero = _layer(n, m, g, N, t, seed)
    ws_bytes = lib.slim_qlinear_workspace(t, n, m, g)
    assert 256 < ws_bytes <= lib.slim_qlinear_noalloc_scratch_bytes(), ws_bytes   # several runs, within the scratch
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    Y_ref = torch.empty((t, n), dtype=torch.float32, device="cuda:0")
    Y_na = torch.full((t, n), float("nan"), dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.slim_qlinear(_p(X), 1, t, m, _p(packed), _p(bits), N, _p(scale), _p(zero), n, g, _p(Y_ref), _p(ws),
                          ws_bytes, stream)
    assert st == 0, st
    st = lib.slim_qlinear_noalloc(_p(X), 1, t, m, _p(packed), _p(bits), N, _p(scale), _p(zero), n, g, _p(Y_na),
                                  stream)
    assert st == 0, st
    torch.cuda.synchronize()
    a, b = Y_ref.cpu().numpy(), Y_na.cpu().numpy()
    assert np.all(np.isfinite(a))
    np.testing.assert_array_equal(b, a)
    return a


def test_noalloc_two_calls_match_workspace_entry(lib):
    print("qlinear_noalloc: t=8 n=1000 m=2048 g=128 N=2, then t=2 n=300 m=1024 g=64 N=3", flush=True)
    _both(lib, 1000, 2048, 128, 2, 8, seed=1)     # matrix-core kernel, 8 runs of groups
    _both(lib, 300, 1024, 64, 3, 2, seed=2)       # table kernel, smaller layer and batch


def test_noalloc_rejects_oversize_before_launch(lib):
    # partial sums of 16 runs x 8 tokens x 131072 rows = 64 MiB > the 32 MiB scratch
    fake = ctypes.c_void_p(4096)
    assert lib.slim_qlinear_workspace(8, 131072, 16384, 128) > lib.slim_qlinear_noalloc_scratch_bytes()
    st = lib.slim_qlinear_noalloc(fake, 1, 8, 16384, fake, fake, 2, fake, fake, 131072, 128, fake, None)
    assert st == -5, st
