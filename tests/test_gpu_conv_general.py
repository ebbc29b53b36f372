"""GPU parity: stride-1 conv contractions of other geometries (any KH x KW,
zero padding, any channel counts) on the direct kernels and on the kernels
that stage whole small samples in LDS, including the 16 x 2 "valid" filter
bank of the TI page's arc-fault example network, against the oracle,
bit-exact with every max-abs."""
import numpy as np
import pytest
import torch

import oracle
from integer_only_nn_amd import ops
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu

GEOMS = [(8, 64, 2, 1, 3, 16, 2, 0),     # the page's example: 64x2x1 -> 49x1x3
         (2, 5, 4, 3, 2, 1, 3, 1), (1, 9, 6, 2, 5, 4, 2, 1), (3, 7, 7, 4, 3, 5, 1, 0),
         (2, 10, 10, 3, 8, 3, 3, 1),     # 3x3 / pad 1 with 3 input channels
         (4, 8, 8, 16, 16, 1, 1, 0),     # 1x1
         (16, 28, 28, 8, 16, 5, 5, 2),   # 6 KB per sample: the direct kernels
         (2, 40, 40, 4, 8, 3, 3, 1),     # the direct kernels again
         (1000, 64, 2, 1, 3, 16, 2, 0),  # the example network's layer, a ragged last sample group
         (6, 10, 10, 8, 12, 3, 3, 1),    # 864 weights: four weight chunks in the staged wgrad
         (5, 12, 12, 8, 16, 3, 3, 0),    # 1152 weights: staged fwd/dgrad, direct wgrad
         (1, 1, 1, 1, 1, 1, 1, 0),
         # full-row windows (no padding, KW = W): the row kernels, with odd
         # sample sizes, every channel count up to 8, and one channel past it
         (7, 10, 3, 2, 5, 4, 3, 0), (3, 9, 1, 4, 8, 3, 1, 0), (4096, 64, 2, 1, 3, 16, 2, 0),
         (2, 6, 2, 2, 9, 3, 2, 0), (5, 33, 2, 2, 1, 1, 2, 0)]


def _u32(t):
    return int(host(t).astype(np.int64)[0]) & 0xFFFFFFFF


@pytest.mark.parametrize("N,H,W,Cin,Cout,KH,KW,P", GEOMS)
def test_conv_general_vs_oracle(N, H, W, Cin, Cout, KH, KW, P):
    say("conv general", N, H, W, Cin, Cout, KH, KW, P)
    rng = np.random.default_rng(N * 1000 + H * 10 + KH + 7 * KW)
    X = rng.integers(-128, 128, (N, H, W, Cin), dtype=np.int64).astype(np.int8)
    Wt = rng.integers(-128, 128, (Cout, KH, KW, Cin), dtype=np.int64).astype(np.int8)
    Ho, Wo = H + 2 * P - KH + 1, W + 2 * P - KW + 1
    dY = rng.integers(-128, 128, (N, Ho, Wo, Cout), dtype=np.int64).astype(np.int8)
    desc = ops.conv_desc(N, H, W, Cin, Cout, KH=KH, KW=KW, pad=P)
    Xd, Wd, dYd = to_dev(X), to_dev(Wt), to_dev(dY)
    Y = torch.empty(N, Ho, Wo, Cout, dtype=torch.int32, device=dev())
    dX = torch.empty(N, H, W, Cin, dtype=torch.int32, device=dev())
    G = torch.empty(Cout, KH, KW, Cin, dtype=torch.int32, device=dev())
    am = torch.zeros(3, dtype=torch.int32, device=dev())
    ops.int_conv_fwd(Xd, Wd, Y, desc, absmax_Y=am[0:1])
    ops.int_conv_dgrad(dYd, Wd, dX, desc, absmax_dX=am[1:2])
    ops.int_conv_wgrad(dYd, Xd, G, desc, absmax_G=am[2:3])
    nws = ops.int_conv_wgrad_workspace_bytes(desc)
    if nws:  # the partial-sums form: the same G and max
        G2 = torch.full_like(G, 7)
        am2 = torch.zeros(1, dtype=torch.int32, device=dev())
        ops.int_conv_wgrad(dYd, Xd, G2, desc, absmax_G=am2,
                           workspace=torch.empty(nws, dtype=torch.uint8, device=dev()))
        np.testing.assert_array_equal(host(G2), host(G))
        assert _u32(am2) == _u32(am[2:3])
    Yo = oracle.conv_fwd(X, Wt, P)
    dXo = oracle.conv_dgrad(dY, Wt, X.shape, P)
    Go = oracle.conv_wgrad(dY, X, KH, KW, P)
    np.testing.assert_array_equal(host(Y), Yo)
    np.testing.assert_array_equal(host(dX), dXo)
    np.testing.assert_array_equal(host(G), Go)
    a = host(am).astype(np.int64) & 0xFFFFFFFF
    assert a.tolist() == [oracle.absmax(Yo), oracle.absmax(dXo), oracle.absmax(Go)]
