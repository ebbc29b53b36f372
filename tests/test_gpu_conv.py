"""GPU parity: 3x3 / stride 1 / pad 1 NHWC conv contractions (implicit GEMM)
and the whole conv NITI step against the oracle, bit-exact with every shift;
the 128x56x56x64 workload checked on sampled outputs plus properties."""
import numpy as np
import pytest
import torch

import ionn_synth
import oracle
from oracle import fast
from oracle import steps as osteps
from integer_only_nn_amd import ops, steps
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,H,W,Cin,Cout", [(1, 3, 3, 16, 16), (2, 9, 7, 16, 32), (1, 1, 1, 16, 16),
                                            (3, 17, 13, 32, 48), (2, 16, 16, 64, 64),
                                            (4, 32, 32, 64, 64), (1, 5, 70, 48, 16),
                                            # 64 -> 64 channels take the halo-tiled kernel:
                                            # W = 1, 2 (many rows per tile), ragged last tiles,
                                            # W = 100 (largest halo that fits), tiles > grid
                                            (3, 5, 1, 64, 64), (2, 7, 2, 64, 64), (5, 13, 11, 64, 64),
                                            (1, 100, 100, 64, 64), (2, 1, 57, 64, 64),
                                            (40, 20, 20, 64, 64)])
def test_conv_step_vs_oracle(N, H, W, Cin, Cout):
    say("conv", N, H, W, Cin, Cout)
    d = ionn_synth.conv3x3(N=N, H=H, W=W, Cin=Cin, Cout=Cout, seed=N * H + Cin)
    dY = np.ascontiguousarray(d["dY"][..., :Cout]) if d["dY"].shape[3] != Cout else d["dY"]
    want = osteps.conv_step(d["X"], d["W"], dY)
    Wt = to_dev(d["W"])
    buf = steps.ConvStepBuffers.make(N, H, W, Cin, Cout, dev(), with_gq=True)
    steps.conv_step(to_dev(d["X"]), Wt, to_dev(dY), buf)
    for k, t in (("Y32", buf.Y), ("y8", buf.y8), ("dX32", buf.dX), ("dx8", buf.dx8), ("G", buf.G),
                 ("Gq", buf.gq)):
        np.testing.assert_array_equal(host(t), want[k], err_msg=k)
    np.testing.assert_array_equal(host(Wt), want["W_new"])
    sc = host(buf.scal).tolist()
    assert sc[3:7] == [want["s_y"], want["s_dx"], want["s"], want["ws"]]


def test_conv_workload_full():
    """128x56x56x64 -> 64, the whole conv step, every element and shift
    against the oracle (float64-product variant)."""
    say("generating conv inputs")
    d = ionn_synth.conv3x3()
    X, W, dY = d["X"], d["W"], d["dY"]
    N, H, Wd, C = X.shape
    Wt = to_dev(W)
    buf = steps.ConvStepBuffers.make(N, H, Wd, C, 64, dev(), with_gq=True)
    steps.conv_step(to_dev(X), Wt, to_dev(dY), buf)
    sc = host(buf.scal).astype(np.int64) & 0xFFFFFFFF
    say("oracle: forward")
    Yo = fast.conv_fwd(X, W)
    np.testing.assert_array_equal(host(buf.Y), Yo)
    y8, s_y = oracle.niti_requant(Yo, 7)
    np.testing.assert_array_equal(host(buf.y8), y8)
    assert (sc[0], sc[3]) == (oracle.absmax(Yo), s_y)
    del Yo, y8
    say("oracle: dgrad")
    dXo = fast.conv_dgrad(dY, W, X.shape)
    np.testing.assert_array_equal(host(buf.dX), dXo)
    dx8, s_dx = oracle.niti_requant(dXo, 7)
    np.testing.assert_array_equal(host(buf.dx8), dx8)
    assert (sc[1], sc[4]) == (oracle.absmax(dXo), s_dx)
    del dXo, dx8
    say("oracle: wgrad + update")
    Go = fast.conv_wgrad(dY, X)
    np.testing.assert_array_equal(host(buf.G), Go)
    Wo, gqo, s, ws = oracle.niti_update(Go, W, 8, 2)
    assert (sc[2], sc[5], sc[6]) == (oracle.absmax(Go), s, ws)
    np.testing.assert_array_equal(host(buf.gq), gqo)
    np.testing.assert_array_equal(host(Wt), Wo)
