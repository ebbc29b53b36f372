"""GPU parity: the one-launch NITI step of a small Linear layer
(int_linear_step_small) against the oracle's single-layer step, bit-exact:
Y, dX, the propagated delta, G, Gq, the updated W, the three maxima and the
three shifts.  Shapes from 1x1x1 to the 32 KiB operand limit, long
reductions on each side, consecutive steps with W moving, int8 extremes,
and the step replayed from a captured HIP graph."""
import numpy as np
import pytest
import torch

import ionn_synth
import oracle
from oracle import steps as osteps
from integer_only_nn_amd import ops, steps
from gpu_helpers import dev, host, say, to_dev, u32

pytestmark = pytest.mark.gpu


def _check(buf, W, want, X, dY):
    np.testing.assert_array_equal(host(buf.Y), want["Y32"])
    np.testing.assert_array_equal(host(buf.dX), want["dX32"])
    np.testing.assert_array_equal(host(buf.delta), want["delta"])
    np.testing.assert_array_equal(host(buf.G), want["G"])
    np.testing.assert_array_equal(host(buf.gq), want["Gq"])
    np.testing.assert_array_equal(host(W), want["W_new"])
    sc = host(buf.scal).astype(np.int64) & 0xFFFFFFFF
    assert sc[0:3].tolist() == [oracle.absmax(want["Y32"]), oracle.absmax(want["dX32"]), oracle.absmax(want["G"])]
    assert sc[3:6].tolist() == [want["s_d"], want["s"], want["ws"]]


@pytest.mark.parametrize("B,IN,OUT", [(16, 64, 32), (1, 1, 1), (3, 5, 7), (17, 33, 10), (8, 100, 40),
                                      (48, 255, 63), (128, 128, 64), (1, 16383, 1), (4096, 1, 4)])
def test_step_small_vs_oracle(B, IN, OUT):
    say("linear step small", B, IN, OUT)
    assert ops.int_linear_step_small_fits(B, IN, OUT)
    d = ionn_synth.single_linear() if (B, IN, OUT) == (16, 64, 32) else \
        ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=B + 2 * IN + 3 * OUT)
    X, W0, dY = d["X"], d["W"], d["dY"]
    want = osteps.linear_step(X, W0, dY)
    W = to_dev(W0)
    buf = steps.LinearStepBuffers.make(B, IN, OUT, dev(), with_gq=True)
    steps.linear_step_small(to_dev(X), W, to_dev(dY), buf)
    _check(buf, W, want, X, dY)


def test_step_small_consecutive_steps_and_extremes():
    """Three steps on one layer, W moving between them, operands at the int8
    extremes (saturating updates)."""
    rng = np.random.default_rng(21)
    pick = np.array([-128, -127, 127, 126, 0, 1, -1, 64, -64], np.int8)
    B, IN, OUT = 24, 40, 12
    X = pick[rng.integers(0, len(pick), (B, IN))]
    Wh = pick[rng.integers(0, len(pick), (OUT, IN))]
    dY = pick[rng.integers(0, len(pick), (B, OUT))]
    W = to_dev(Wh)
    buf = steps.LinearStepBuffers.make(B, IN, OUT, dev(), with_gq=True)
    Xd, dYd = to_dev(X), to_dev(dY)
    for k in range(3):
        want = osteps.linear_step(X, Wh, dY, tb_w=5, mu=1)
        steps.linear_step_small(Xd, W, dYd, buf, tb_w=5, mu=1)
        _check(buf, W, want, X, dY)
        Wh = want["W_new"]
    assert (Wh == -128).any() or (Wh == 127).any()


def test_step_small_matches_the_launch_by_launch_step():
    d = ionn_synth.single_linear(B=20, IN=70, OUT=30, seed=4)
    a, b = to_dev(d["W"]), to_dev(d["W"])
    ba = steps.LinearStepBuffers.make(20, 70, 30, dev(), with_gq=True)
    bb = steps.LinearStepBuffers.make(20, 70, 30, dev(), with_gq=True)
    X, dY = to_dev(d["X"]), to_dev(d["dY"])
    steps.linear_step(X, a, dY, ba)
    steps.linear_step_small(X, b, dY, bb)
    for t in ("Y", "dX", "delta", "G", "gq"):
        np.testing.assert_array_equal(host(getattr(ba, t)), host(getattr(bb, t)))
    np.testing.assert_array_equal(host(a), host(b))
    assert host(ba.scal)[3:6].tolist() == host(bb.scal)[3:6].tolist()


def test_step_small_replayed_from_graph():
    """Two steps captured in one HIP graph, replayed three times with W
    carried over; every replay against the oracle, eager work in between."""
    d = ionn_synth.single_linear()
    X, Wh, dY = d["X"], d["W"], d["dY"]
    W = to_dev(Wh)
    buf = steps.LinearStepBuffers.make(16, 64, 32, dev(), with_gq=True)
    Xd, dYd = to_dev(X), to_dev(dY)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    W_cap = W.clone()
    with torch.cuda.stream(s):
        steps.linear_step_small(Xd, W, dYd, buf, stream=s.cuda_stream)
        torch.cuda.synchronize()
        W.copy_(W_cap)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            steps.linear_step_small(Xd, W, dYd, buf, stream=s.cuda_stream)
            steps.linear_step_small(Xd, W, dYd, buf, stream=s.cuda_stream)
    torch.cuda.synchronize()
    W.copy_(W_cap)
    torch.cuda.synchronize()
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        first = osteps.linear_step(X, Wh, dY)
        want = osteps.linear_step(X, first["W_new"], dY)
        _check(buf, W, want, X, dY)
        Wh = want["W_new"]
        buf.Y.zero_()
        buf.G.zero_()
        torch.cuda.synchronize()


def test_step_small_refuses_large_layers():
    assert not ops.int_linear_step_small_fits(256, 784, 256)
    assert not ops.int_linear_step_small_fits(1, 16384, 1)
    assert not ops.int_linear_step_small_fits(0, 4, 4)
    X = torch.zeros(256, 784, dtype=torch.int8, device=dev())
    W = torch.zeros(256, 784, dtype=torch.int8, device=dev())
    dY = torch.zeros(256, 256, dtype=torch.int8, device=dev())
    buf = steps.LinearStepBuffers.make(256, 784, 256, dev())
    with pytest.raises(RuntimeError):
        steps.linear_step_small(X, W, dY, buf)
