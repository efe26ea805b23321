"""CPU oracle against its pins (golden examples, closed forms, a library
convolution, identities).  No GPU involved."""
import pytest

import oracle
import oracle_pins

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.get())


def test_thread_count_does_not_change_result():
    import numpy as np
    o = oracle.get()
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 5, 9, 9))
    w = rng.standard_normal((6, 5, 3, 3))
    a = o.conv(x, w, 1, 1, nthreads=1)
    b = o.conv(x, w, 1, 1, nthreads=4)
    np.testing.assert_array_equal(a, b)


def test_fused_loop_equals_unfused_passes():
    """The page's claim that fusing leaves the arithmetic unchanged: an
    element-at-a-time loop that applies batch norm and SiLU right after each
    output's conv sum (same summation order) equals the three-pass oracle
    bit for bit."""
    import math
    import numpy as np
    o = oracle.get()
    rng = np.random.default_rng(4)
    N, C, H, W, O, K, s, p = 1, 2, 5, 4, 3, 3, 2, 1
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((O, C, K, K))
    scale, bias = rng.uniform(0.5, 1.5, O), rng.standard_normal(O)
    y = o.forward(x, w, scale, bias, s, p)
    OH, OW = y.shape[2:]
    for n in range(N):
        for co in range(O):
            for oh in range(OH):
                for ow in range(OW):
                    acc = 0.0
                    for ci in range(C):
                        for kh in range(K):
                            for kw in range(K):
                                ih, iw = oh * s - p + kh, ow * s - p + kw
                                xv = x[n, ci, ih, iw] if (0 <= ih < H and 0 <= iw < W) else 0.0
                                acc += float(xv) * float(w[co, ci, kh, kw])
                    v = acc * float(scale[co]) + float(bias[co])
                    assert y[n, co, oh, ow] == v * (1.0 / (1.0 + math.exp(-v)))
