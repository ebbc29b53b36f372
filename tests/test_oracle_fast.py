"""Pin the full-size oracle variants (float64 matrix product as the primitive
step, oracle/fast.py) to the plain-C oracle loops: identical int32 results on
shapes with ragged sizes, for every linear, conv and DFP-16 role."""
import numpy as np
import pytest

import ionn_synth
import oracle
from oracle import fast


@pytest.mark.parametrize("B,IN,OUT", [(1, 1, 1), (17, 33, 10), (64, 200, 96), (130, 70, 260)])
def test_linear_fast_equals_c(B, IN, OUT):
    d = ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=B)
    X, W, dY = d["X"], d["W"], d["dY"]
    np.testing.assert_array_equal(fast.linear_fwd(X, W), oracle.linear_fwd(X, W))
    np.testing.assert_array_equal(fast.linear_dgrad(dY, W), oracle.linear_dgrad(dY, W))
    np.testing.assert_array_equal(fast.linear_wgrad(dY, X), oracle.linear_wgrad(dY, X))


def test_fast_wraps_like_c():
    K = 1 << 18
    X = np.full((1, K), 127, np.int8)
    np.testing.assert_array_equal(fast.linear_fwd(X, X), oracle.linear_fwd(X, X))


@pytest.mark.parametrize("N,H,W,Cin,Cout,P,K", [(2, 5, 7, 16, 16, 1, 3), (1, 9, 9, 32, 48, 1, 3),
                                                (2, 6, 5, 3, 4, 0, 3), (1, 7, 7, 2, 2, 2, 5),
                                                (1, 1, 1, 16, 16, 1, 3)])
def test_conv_fast_equals_c(N, H, W, Cin, Cout, P, K):
    rng = np.random.default_rng(N + H + Cin)
    X = rng.integers(-128, 128, (N, H, W, Cin)).astype(np.int8)
    Wt = rng.integers(-128, 128, (Cout, K, K, Cin)).astype(np.int8)
    Ho, Wo = H + 2 * P - K + 1, W + 2 * P - K + 1
    dY = rng.integers(-128, 128, (N, Ho, Wo, Cout)).astype(np.int8)
    np.testing.assert_array_equal(fast.conv_fwd(X, Wt, P), oracle.conv_fwd(X, Wt, P))
    np.testing.assert_array_equal(fast.conv_dgrad(dY, Wt, X.shape, P), oracle.conv_dgrad(dY, Wt, X.shape, P))
    np.testing.assert_array_equal(fast.conv_wgrad(dY, X, K, K, P), oracle.conv_wgrad(dY, X, K, K, P))


@pytest.mark.parametrize("M,K,N", [(3, 64, 5), (17, 40, 9), (40, 256, 24), (30, 200, 70), (9, 1000, 5)])
def test_dfp_fast_equals_c(M, K, N):
    d = ionn_synth.dfp16_gemm(M=M, K=K, N=N, seed=M)
    X, W, dY = d["X"], d["W"], d["dY"]
    for f_fast, f_c, args in ((fast.dfp16_fwd, oracle.dfp16_fwd, (X, d["eX"], W, d["eW"])),
                              (fast.dfp16_dgrad, oracle.dfp16_dgrad, (dY, d["edY"], W, d["eW"])),
                              (fast.dfp16_wgrad, oracle.dfp16_wgrad, (dY, d["edY"], X, d["eX"]))):
        a, b = f_fast(*args), f_c(*args)
        np.testing.assert_array_equal(a[0], b[0])
        assert a[1] == b[1]
        np.testing.assert_array_equal(a[2], b[2])
