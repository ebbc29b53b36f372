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


# ---------------------------------------------------------------------------
# The requantisation fused into the 64 -> 64 contractions (the int32 sums
# never stored), on both paths: one contraction pass plus the streaming pass
# (with the workspace) and two contraction passes (without): y8 / dx8 and
# every shift against the oracle.
# ---------------------------------------------------------------------------

FAST64 = [(2, 16, 16), (4, 32, 32), (3, 5, 3), (2, 7, 2), (5, 13, 11), (1, 100, 100), (2, 1, 57),
          (40, 20, 20)]


@pytest.mark.parametrize("one_pass", [True, False])
@pytest.mark.parametrize("N,H,W", FAST64)
def test_conv_step_fused_vs_oracle(N, H, W, one_pass):
    say("conv fused", N, H, W, "one pass" if one_pass else "two passes")
    d = ionn_synth.conv3x3(N=N, H=H, W=W, Cin=64, Cout=64, seed=N * H + 64)
    want = osteps.conv_step(d["X"], d["W"], d["dY"])
    Wt = to_dev(d["W"])
    buf = steps.ConvStepBuffers.make(N, H, W, 64, 64, dev(), with_gq=True, one_pass=one_pass)
    assert (buf.rws is not None) == one_pass
    steps.conv_step_fused(to_dev(d["X"]), Wt, to_dev(d["dY"]), buf)
    for k, t in (("y8", buf.y8), ("dx8", buf.dx8), ("G", buf.G), ("Gq", buf.gq)):
        np.testing.assert_array_equal(host(t), want[k], err_msg=k)
    np.testing.assert_array_equal(host(Wt), want["W_new"])
    sc = host(buf.scal).astype(np.int64) & 0xFFFFFFFF
    assert (sc[0], sc[1]) == (oracle.absmax(want["Y32"]), oracle.absmax(want["dX32"]))
    assert sc[3:7].tolist() == [want["s_y"], want["s_dx"], want["s"], want["ws"]]


@pytest.mark.parametrize("fused", [True, False])
def test_conv_steps_alternating_scalar_sets(fused):
    """Five steps with the maxima alternating between two scalar sets (each
    step's update clears the set the next one uses; no fill kernel), each
    against the oracle's step on the weights the previous one left."""
    N, H, W = 2, 10, 9
    d = ionn_synth.conv3x3(N=N, H=H, W=W, Cin=64, Cout=64, seed=91)
    X, Wt0, dY = d["X"], d["W"], d["dY"]
    Wt, Xd, dYd = to_dev(Wt0), to_dev(X), to_dev(dY)
    buf = steps.ConvStepBuffers.make(N, H, W, 64, 64, dev(), with_gq=True, alternate=True)
    run = steps.conv_step_fused if fused else steps.conv_step
    for k in range(5):
        say("conv alternating step", k, "fused" if fused else "int32")
        run(Xd, Wt, dYd, buf)
        want = osteps.conv_step(X, Wt0, dY)
        for name, t in (("y8", buf.y8), ("dx8", buf.dx8), ("G", buf.G), ("Gq", buf.gq)):
            np.testing.assert_array_equal(host(t), want[name], err_msg=f"step {k}: {name}")
        np.testing.assert_array_equal(host(Wt), want["W_new"], err_msg=f"step {k}: W")
        mx = host(buf.maxima()).astype(np.int64) & 0xFFFFFFFF
        assert mx.tolist() == [oracle.absmax(want["Y32"]), oracle.absmax(want["dX32"]),
                               oracle.absmax(want["G"])], k
        sc = host(buf.scal)
        assert sc[3:7].tolist() == [want["s_y"], want["s_dx"], want["s"], want["ws"]], k
        Wt0 = want["W_new"]


@pytest.mark.parametrize("one_pass", [True, False])
@pytest.mark.parametrize("relu", [0, 1])
@pytest.mark.parametrize("tb", [1, 2, 5, 7, 12, 31])
def test_conv_fwd_requant_target_bits_relu(tb, relu, one_pass):
    """Any target_bits (s = 0 at 31: the sums are returned clamped; above 7
    the one-pass request runs two passes) and the Conv2D layer's ReLU, on a
    ragged 9x7 image pair."""
    N, H, W = 2, 9, 7
    desc = ops.conv_desc(N, H, W, 64, 64)
    ws = torch.empty(ops.int_conv_requant_workspace_bytes(desc), dtype=torch.uint8, device=dev()) \
        if one_pass else None
    d = ionn_synth.conv3x3(N=N, H=H, W=W, Cin=64, Cout=64, seed=tb + 10 * relu)
    Y = oracle.conv_fwd(d["X"], d["W"])
    y8, s = oracle.niti_requant(Y, tb, bool(relu))
    out = torch.empty(N, H, W, 64, dtype=torch.int8, device=dev())
    scal = torch.zeros(2, dtype=torch.int32, device=dev())
    ops.int_conv_fwd_requant(to_dev(d["X"]), to_dev(d["W"]), out, desc, tb, relu,
                             scal[0:1], shift_out=scal[1:2], workspace=ws)
    np.testing.assert_array_equal(host(out), y8)
    assert host(scal).tolist() == [oracle.absmax(Y), s]
    # delta propagation through the same path
    dX = oracle.conv_dgrad(d["dY"], d["W"], d["X"].shape)
    dx8, sd = oracle.niti_requant(dX, tb)
    out2 = torch.empty(N, H, W, 64, dtype=torch.int8, device=dev())
    scal.zero_()
    ops.int_conv_dgrad_requant(to_dev(d["dY"]), to_dev(d["W"]), out2, desc, tb,
                               scal[0:1], shift_out=scal[1:2], workspace=ws)
    np.testing.assert_array_equal(host(out2), dx8)
    assert host(scal).tolist() == [oracle.absmax(dX), sd]


@pytest.mark.parametrize("case", ["zeros", "one_hot", "small", "large"])
def test_conv_requant_one_pass_edge_values(case):
    """The one-pass path where the block shifts differ from the tensor's:
    all-zero images (every shift 0), a single non-zero pixel (one block at
    the tensor's shift, every other block far below it), values that never
    need a shift, and the largest sums the int8 ranges allow."""
    N, H, W = 2, 17, 15
    rng = np.random.default_rng({"zeros": 1, "one_hot": 2, "small": 3, "large": 4}[case])
    Wt = np.clip(np.round(rng.normal(0, 15, (64, 3, 3, 64))), -128, 127).astype(np.int8)
    X = np.zeros((N, H, W, 64), np.int8)
    if case == "one_hot":
        X[1, 8, 7, :] = 127
    elif case == "small":
        X = rng.integers(-1, 2, (N, H, W, 64)).astype(np.int8)
        Wt = rng.integers(-1, 2, (64, 3, 3, 64)).astype(np.int8)
    elif case == "large":
        X[:] = -128
        X[0, ::2, ::3, :] = 127
        Wt[:] = -128
    desc = ops.conv_desc(N, H, W, 64, 64)
    ws = torch.empty(ops.int_conv_requant_workspace_bytes(desc), dtype=torch.uint8, device=dev())
    ws.fill_(0xA5)   # stale workspace contents must not matter
    for relu in (0, 1):
        Y = oracle.conv_fwd(X, Wt)
        y8, s = oracle.niti_requant(Y, 7, bool(relu))
        out = torch.full((N, H, W, 64), 99, dtype=torch.int8, device=dev())
        scal = torch.zeros(2, dtype=torch.int32, device=dev())
        ops.int_conv_fwd_requant(to_dev(X), to_dev(Wt), out, desc, 7, relu, scal[0:1], shift_out=scal[1:2],
                                 workspace=ws)
        np.testing.assert_array_equal(host(out), y8, err_msg=f"{case} relu={relu}")
        assert host(scal).tolist() == [oracle.absmax(Y), s]


def test_conv_requant_refusals_and_empty():
    from integer_only_nn_amd._lib import IonnError
    # width 1: the halo of a 256-pixel tile does not fit, no fused path
    x1 = torch.zeros(3, 5, 1, 64, dtype=torch.int8, device=dev())
    w1 = torch.zeros(64, 3, 3, 64, dtype=torch.int8, device=dev())
    o1 = torch.zeros(3, 5, 1, 64, dtype=torch.int8, device=dev())
    s1 = torch.zeros(2, dtype=torch.int32, device=dev())
    with pytest.raises(IonnError) as e:
        ops.int_conv_fwd_requant(x1, w1, o1, ops.conv_desc(3, 5, 1, 64, 64), 7, 0, s1[0:1])
    assert e.value.status == 5
    x = torch.zeros(1, 4, 4, 32, dtype=torch.int8, device=dev())
    w = torch.zeros(64, 3, 3, 32, dtype=torch.int8, device=dev())
    o = torch.zeros(1, 4, 4, 64, dtype=torch.int8, device=dev())
    scal = torch.zeros(2, dtype=torch.int32, device=dev())
    with pytest.raises(IonnError) as e:   # 32 input channels: no fused path
        ops.int_conv_fwd_requant(x, w, o, ops.conv_desc(1, 4, 4, 32, 64), 7, 0, scal[0:1])
    assert e.value.status == 5
    x64 = torch.zeros(1, 4, 4, 64, dtype=torch.int8, device=dev())
    w64 = torch.zeros(64, 3, 3, 64, dtype=torch.int8, device=dev())
    with pytest.raises(IonnError) as e:
        ops.int_conv_fwd_requant(x64, w64, o, ops.conv_desc(1, 4, 4, 64, 64), 0, 0, scal[0:1])
    assert e.value.status == 3
    # a workspace smaller than the one-pass path needs is refused
    d4 = ops.conv_desc(1, 4, 4, 64, 64)
    small = torch.empty(ops.int_conv_requant_workspace_bytes(d4) - 16, dtype=torch.uint8, device=dev())
    with pytest.raises(IonnError) as e:
        ops.int_conv_fwd_requant(x64, w64, o, d4, 7, 0, scal[0:1], workspace=small)
    assert e.value.status == 7
    # no pixels: nothing to contract, s = 0 is written
    scal.fill_(9)
    scal[0] = 0
    ops.int_conv_fwd_requant(x64, w64, o, ops.conv_desc(0, 4, 4, 64, 64), 7, 0, scal[0:1], shift_out=scal[1:2])
    assert host(scal).tolist() == [0, 0]


def test_conv_fused_workload_full():
    """128x56x56x64 -> 64 through the fused path: y8, dx8 and their shifts
    against the oracle (float64-product variant), and the same bytes as the
    int32-then-requantise path."""
    say("generating conv inputs")
    d = ionn_synth.conv3x3()
    X, W, dY = d["X"], d["W"], d["dY"]
    N, H, Wd, C = X.shape
    Wt = to_dev(W)
    buf = steps.ConvStepBuffers.make(N, H, Wd, C, 64, dev())
    steps.conv_step_fused(to_dev(X), Wt, to_dev(dY), buf)
    sc = host(buf.scal).astype(np.int64) & 0xFFFFFFFF
    say("oracle: forward")
    Yo = fast.conv_fwd(X, W)
    y8, s_y = oracle.niti_requant(Yo, 7)
    np.testing.assert_array_equal(host(buf.y8), y8)
    assert (sc[0], sc[3]) == (oracle.absmax(Yo), s_y)
    del Yo, y8
    say("oracle: dgrad")
    dXo = fast.conv_dgrad(dY, W, X.shape)
    dx8, s_dx = oracle.niti_requant(dXo, 7)
    np.testing.assert_array_equal(host(buf.dx8), dx8)
    assert (sc[1], sc[4]) == (oracle.absmax(dXo), s_dx)
    # the two-pass path gives the same bytes at full size
    buf2 = steps.ConvStepBuffers.make(N, H, Wd, C, 64, dev(), one_pass=False)
    steps.conv_step_fused(to_dev(X), to_dev(W), to_dev(dY), buf2)
    np.testing.assert_array_equal(host(buf2.y8), host(buf.y8))
    np.testing.assert_array_equal(host(buf2.dx8), host(buf.dx8))
    assert host(buf2.scal)[[0, 1, 3, 4]].tolist() == host(buf.scal)[[0, 1, 3, 4]].tolist()


def test_conv_step_fused_replayed_from_graph():
    """The fused conv step captured in one HIP graph and replayed three
    times (ragged 13x11 images), with eager work between replays: the maxima
    restart from the fill kernel each time, the requantising passes read the
    finished maxima, and every replay matches the oracle's step on the
    weights the previous one left."""
    N, H, W = 3, 13, 11
    d = ionn_synth.conv3x3(N=N, H=H, W=W, Cin=64, Cout=64, seed=77)
    X, Wt0, dY = d["X"], d["W"], d["dY"]
    Wt = to_dev(Wt0)
    Xd, dYd = to_dev(X), to_dev(dY)
    buf = steps.ConvStepBuffers.make(N, H, W, 64, 64, dev(), with_gq=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        steps.conv_step_fused(Xd, Wt, dYd, buf, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        say("conv fused graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        want = osteps.conv_step(X, Wt0, dY)
        for k, t in (("y8", buf.y8), ("dx8", buf.dx8), ("Gq", buf.gq)):
            np.testing.assert_array_equal(host(t), want[k], err_msg=f"replay {rep}: {k}")
        np.testing.assert_array_equal(host(Wt), want["W_new"], err_msg=f"replay {rep}: W")
        sc = host(buf.scal).astype(np.int64) & 0xFFFFFFFF
        assert sc[3:7].tolist() == [want["s_y"], want["s_dx"], want["s"], want["ws"]], (rep, sc)
        Wt0 = want["W_new"]
        torch.zeros(1000, device=dev()).add_(1.0)   # unrelated eager work between replays
