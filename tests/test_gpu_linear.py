"""GPU parity: int8 Linear contractions (fwd / dgrad / wgrad on the matrix
cores) and whole single-layer NITI steps against the oracle, bit-exact,
including every max-abs and shift value.  Shapes span several 64- and
256-wide tiles with ragged tails, the degenerate sizes, and the large-linear
workload (8192 x 4096 x 4096) checked on sampled outputs plus properties that
hold at any size."""
import numpy as np
import pytest
import torch

import ionn_synth
import oracle
from oracle import fast
from oracle import steps as osteps
from integer_only_nn_amd import ops, steps
from gpu_helpers import dev, host, say, to_dev, u32

pytestmark = pytest.mark.gpu


def _contract(X, W, dY, act=None):
    B, IN = X.shape
    OUT = W.shape[0]
    Xd, Wd, dYd = to_dev(X), to_dev(W), to_dev(dY)
    Y = torch.empty(B, OUT, dtype=torch.int32, device=dev())
    dX = torch.empty(B, IN, dtype=torch.int32, device=dev())
    G = torch.empty(OUT, IN, dtype=torch.int32, device=dev())
    am = torch.zeros(3, dtype=torch.int32, device=dev())
    ops.int_linear_fwd(Xd, Wd, Y, absmax_Y=am[0:1])
    ops.int_linear_dgrad(dYd, Wd, dX, relu_act=None if act is None else to_dev(act), absmax_dX=am[1:2])
    ops.int_linear_wgrad(dYd, Xd, G, absmax_G=am[2:3])
    a = host(am).astype(np.int64) & 0xFFFFFFFF
    return host(Y), host(dX), host(G), a.tolist()


SHAPES = [(1, 1, 1), (3, 5, 7), (16, 64, 32), (17, 33, 10), (256, 784, 10), (256, 10, 128),
          (65, 127, 129), (129, 257, 300), (300, 200, 100), (1024, 1024, 512), (1100, 1030, 1050),
          (2048, 256, 1024)]


@pytest.mark.parametrize("B,IN,OUT", SHAPES)
def test_contractions_vs_oracle(B, IN, OUT):
    say("shape", B, IN, OUT)
    d = ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=B + IN + OUT)
    X, W, dY = d["X"], d["W"], d["dY"]
    Y, dX, G, am = _contract(X, W, dY)
    Yo, dXo, Go = oracle.linear_fwd(X, W), oracle.linear_dgrad(dY, W), oracle.linear_wgrad(dY, X)
    np.testing.assert_array_equal(Y, Yo)
    np.testing.assert_array_equal(dX, dXo)
    np.testing.assert_array_equal(G, Go)
    assert am == [oracle.absmax(Yo), oracle.absmax(dXo), oracle.absmax(Go)]


# a long batch through narrow layers (N, K <= 160): the row-run staging
# path of fwd and dgrad (rows of any byte length, fragments built with
# v_alignbyte, bytes past K masked), ragged last stages, single columns
SKINNY = [(65536, 147, 160), (65536, 160, 2), (65536, 2, 160), (4096, 160, 147), (4112, 147, 160),
          (4096, 1, 1), (8192, 160, 160), (4096, 33, 31), (4128, 64, 96), (6000, 100, 5),
          # a last block of brows rows whose brows N values end inside a word
          # (masked dgrad N = 147, fwd N = 7 and N = 2), and ragged rows with N
          # a multiple of 4 (dgrad N = 160 under the mask, fwd N = 32)
          (4099, 147, 160), (4101, 32, 7), (4101, 32, 2), (4099, 160, 32)]


@pytest.mark.parametrize("B,IN,OUT", SKINNY)
def test_skinny_contractions_vs_oracle(B, IN, OUT):
    say("skinny", B, IN, OUT)
    d = ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=B + 3 * IN + OUT)
    X, W, dY = d["X"], d["W"], d["dY"]
    act = ionn_synth.uniform_int(B + IN, 20, (B, IN), -128, 127)
    Y, dX, G, am = _contract(X, W, dY, act=act)
    Yo = oracle.linear_fwd(X, W)
    dXo = oracle.relu_mask(oracle.linear_dgrad(dY, W), act)
    Go = oracle.linear_wgrad(dY, X)
    np.testing.assert_array_equal(Y, Yo)
    np.testing.assert_array_equal(dX, dXo)
    np.testing.assert_array_equal(G, Go)
    assert am == [oracle.absmax(Yo), oracle.absmax(dXo), oracle.absmax(Go)]


# small G over a long batch: the LDS row-copy path (byte and dword copies,
# rows of 2 and 3 bytes whose dwords span two rows, one to 32 blocks of
# 32 x 32, ragged batch tails) and, past 32 blocks or with 1-byte rows, the
# generic split
LONG_WGRAD = [(65536, 147, 160), (65536, 160, 2), (5000, 33, 7), (4097, 256, 128), (9000, 250, 130),
              (20000, 64, 96), (4096, 1, 1), (5000, 1, 7), (4500, 3, 1), (4099, 2, 5)]


@pytest.mark.parametrize("B,IN,OUT", LONG_WGRAD)
def test_wgrad_long_batch(B, IN, OUT):
    say("wgrad long", B, IN, OUT)
    d = ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=B + 3 * IN + OUT)
    X, dY = d["X"], d["dY"]
    G = torch.empty(OUT, IN, dtype=torch.int32, device=dev())
    am = torch.zeros(1, dtype=torch.int32, device=dev())
    ops.int_linear_wgrad(to_dev(dY), to_dev(X), G, absmax_G=am)
    want = fast.linear_wgrad(dY, X)
    np.testing.assert_array_equal(host(G), want)
    assert u32(am) == oracle.absmax(want)


@pytest.mark.parametrize("B,IN,OUT", [(65536, 147, 160), (65536, 160, 2), (5000, 33, 7), (4097, 256, 128),
                                   (5000, 2, 7), (4500, 3, 2)])
def test_wgrad_long_batch_workspace(B, IN, OUT):
    # the partial-sums form gives the same G and max as the oracle; called
    # twice in a row (the workspace is overwritten, never cleared)
    say("wgrad long ws", B, IN, OUT)
    ws = torch.empty(ops.int_linear_wgrad_workspace_bytes(B, IN, OUT), dtype=torch.uint8, device=dev())
    assert ws.numel() > 0
    for seed in (1, 2):
        d = ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=seed * 7 + B + IN)
        X, dY = d["X"], d["dY"]
        G = torch.full((OUT, IN), 99, dtype=torch.int32, device=dev())
        am = torch.zeros(1, dtype=torch.int32, device=dev())
        ops.int_linear_wgrad_ws(to_dev(dY), to_dev(X), G, ws, absmax_G=am)
        want = fast.linear_wgrad(dY, X)
        np.testing.assert_array_equal(host(G), want)
        assert u32(am) == oracle.absmax(want)


def test_wgrad_long_batch_workspace_4byte_aligned():
    # a workspace 4 bytes past a 16-byte boundary: the partials go in rows of
    # G instead of the 32 x 32 blocks (whose 16-byte stores need alignment)
    B, IN, OUT = 65536, 147, 160
    say("wgrad long ws misaligned", B, IN, OUT)
    need = ops.int_linear_wgrad_workspace_bytes(B, IN, OUT)
    ws = torch.empty(need + 16, dtype=torch.uint8, device=dev())[4:]
    d = ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=11)
    X, dY = d["X"], d["dY"]
    G = torch.full((OUT, IN), 99, dtype=torch.int32, device=dev())
    am = torch.zeros(1, dtype=torch.int32, device=dev())
    ops.int_linear_wgrad_ws(to_dev(dY), to_dev(X), G, ws, absmax_G=am)
    want = fast.linear_wgrad(dY, X)
    np.testing.assert_array_equal(host(G), want)
    assert u32(am) == oracle.absmax(want)


def test_wgrad_long_batch_extremes():
    # every product 16384 or -16256: the largest sums the long path meets
    B, IN, OUT = 8192, 40, 24
    X = np.full((B, IN), -128, np.int8)
    X[:, ::3] = 127
    dY = np.full((B, OUT), -128, np.int8)
    G = torch.empty(OUT, IN, dtype=torch.int32, device=dev())
    ops.int_linear_wgrad(to_dev(dY), to_dev(X), G)
    np.testing.assert_array_equal(host(G), fast.linear_wgrad(dY, X))


@pytest.mark.parametrize("B,IN,OUT", [(16, 64, 32), (256, 256, 128), (33, 100, 17), (1024, 1024, 256)])
def test_dgrad_relu_mask(B, IN, OUT):
    d = ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=7)
    act = ionn_synth.uniform_int(7, 20, (B, IN), -128, 127)
    _, dX, _, am = _contract(d["X"], d["W"], d["dY"], act=act)
    want = oracle.relu_mask(oracle.linear_dgrad(d["dY"], d["W"]), act)
    np.testing.assert_array_equal(dX, want)
    assert am[1] == oracle.absmax(want)


def test_empty_reduction_gives_zero():
    X = np.zeros((8, 0), np.int8)
    W = np.zeros((4, 0), np.int8)
    Y = torch.full((8, 4), 7, dtype=torch.int32, device=dev())
    am = torch.zeros(1, dtype=torch.int32, device=dev())
    ops.int_linear_fwd(to_dev(X), to_dev(W), Y, absmax_Y=am)
    assert not host(Y).any() and u32(am) == 0


def test_single_linear_step_config():
    """16x64 -> 32 layer, one NITI step: W', delta, every shift."""
    d = ionn_synth.single_linear()
    want = osteps.linear_step(d["X"], d["W"], d["dY"])
    W = to_dev(d["W"])
    buf = steps.LinearStepBuffers.make(16, 64, 32, dev(), with_gq=True)
    steps.linear_step(to_dev(d["X"]), W, to_dev(d["dY"]), buf)
    np.testing.assert_array_equal(host(buf.Y), want["Y32"])
    np.testing.assert_array_equal(host(buf.dX), want["dX32"])
    np.testing.assert_array_equal(host(buf.delta), want["delta"])
    np.testing.assert_array_equal(host(buf.G), want["G"])
    np.testing.assert_array_equal(host(buf.gq), want["Gq"])
    np.testing.assert_array_equal(host(W), want["W_new"])
    sc = host(buf.scal).tolist()
    assert sc[3] == want["s_d"] and (sc[4], sc[5]) == (want["s"], want["ws"])
    assert (host(W) != d["W"]).any()


def test_deterministic_repeat():
    d = ionn_synth.single_linear(B=1024, IN=1024, OUT=512, seed=9)
    r1 = _contract(d["X"], d["W"], d["dY"])
    r2 = _contract(d["X"], d["W"], d["dY"])
    for a, b in zip(r1[:3], r2[:3]):
        np.testing.assert_array_equal(a, b)


def test_large_linear_step_full():
    """The 8192x4096x4096 step as the benchmark runs it, every element and
    every shift against the oracle (float64-product variant, pinned to the C
    loops by tests/test_oracle_fast.py)."""
    say("generating the large-linear inputs")
    d = ionn_synth.large_linear()
    X, W, dY = d["X"], d["W"], d["dY"]
    T, IN, OUT = 8192, 4096, 4096
    Wd = to_dev(W)
    buf = steps.LinearStepBuffers.make(T, IN, OUT, dev(), with_gq=True)
    say("running the step")
    steps.linear_step(to_dev(X), Wd, to_dev(dY), buf)
    sc = host(buf.scal).astype(np.int64) & 0xFFFFFFFF
    say("oracle: forward")
    Yo = fast.linear_fwd(X, W)
    np.testing.assert_array_equal(host(buf.Y), Yo)
    assert sc[0] == oracle.absmax(Yo)
    del Yo
    say("oracle: dgrad")
    dXo = fast.linear_dgrad(dY, W)
    np.testing.assert_array_equal(host(buf.dX), dXo)
    assert sc[1] == oracle.absmax(dXo)
    delta, s_d = oracle.niti_requant(dXo, 7)
    np.testing.assert_array_equal(host(buf.delta), delta)
    assert sc[3] == s_d
    del dXo, delta
    say("oracle: wgrad + update")
    Go = fast.linear_wgrad(dY, X)
    np.testing.assert_array_equal(host(buf.G), Go)
    assert sc[2] == oracle.absmax(Go)
    Wo, gqo, s, ws = oracle.niti_update(Go, W, 8, 2)
    assert (sc[4], sc[5]) == (s, ws)
    np.testing.assert_array_equal(host(buf.gq), gqo)
    np.testing.assert_array_equal(host(Wd), Wo)


def test_linear_step_replayed_from_graph():
    """The training step (fill, fwd, dgrad, delta, wgrad, update) captured in
    one HIP graph and replayed three times at a ragged size, with eager work
    between replays: the fill kernel resets the maxima on every replay and
    each replay matches the oracle's step on the weights it left."""
    d = ionn_synth.single_linear(B=300, IN=520, OUT=264, seed=21)
    X, W, dY = d["X"], d["W"], d["dY"]
    Wd = to_dev(W)
    Xd, dYd = to_dev(X), to_dev(dY)
    buf = steps.LinearStepBuffers.make(300, 520, 264, dev(), with_gq=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        steps.linear_step(Xd, Wd, dYd, buf, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        say("linear step graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        want = osteps.linear_step(X, W, dY)
        np.testing.assert_array_equal(host(buf.delta), want["delta"], err_msg=f"replay {rep}: delta")
        np.testing.assert_array_equal(host(buf.gq), want["Gq"], err_msg=f"replay {rep}: Gq")
        np.testing.assert_array_equal(host(Wd), want["W_new"], err_msg=f"replay {rep}: W")
        sc = host(buf.scal).tolist()
        assert sc[3] == want["s_d"] and (sc[4], sc[5]) == (want["s"], want["ws"]), (rep, sc)
        W = want["W_new"]
        torch.zeros(1000, device=dev()).add_(1.0)   # unrelated eager work between replays


@pytest.mark.parametrize("B,IN,OUT", [(300, 520, 264), (256, 256, 256), (16, 64, 32)])
def test_linear_steps_alternating_scalar_sets(B, IN, OUT):
    """Steps whose update clears the next step's max-combined scalars
    (niti_quantize_update_clear) instead of a fill before each step: five
    consecutive steps against the oracle's, every maximum and shift."""
    d = ionn_synth.single_linear(B=B, IN=IN, OUT=OUT, seed=B + IN)
    X, W, dY = d["X"], d["W"], d["dY"]
    Wd, Xd, dYd = to_dev(W), to_dev(X), to_dev(dY)
    buf = steps.LinearStepBuffers.make(B, IN, OUT, dev(), with_gq=True, alternate=True)
    buf.scal[8:15].fill_(12345)    # stale values: the first step's set must not be used unless cleared
    buf.scal[8:11].zero_()
    for t in range(5):
        steps.linear_step(Xd, Wd, dYd, buf)
        want = osteps.linear_step(X, W, dY)
        np.testing.assert_array_equal(host(buf.gq), want["Gq"], err_msg=f"step {t}: Gq")
        np.testing.assert_array_equal(host(Wd), want["W_new"], err_msg=f"step {t}: W")
        m = host(buf.maxima()).astype(np.int64) & 0xFFFFFFFF
        assert m.tolist() == [oracle.absmax(want["Y32"]), oracle.absmax(want["dX32"]), oracle.absmax(want["G"])], t
        sc = host(buf.scal).tolist()
        assert sc[3] == want["s_d"] and (sc[4], sc[5]) == (want["s"], want["ws"]), (t, sc)
        W = want["W_new"]


def test_linear_steps_alternating_replayed_from_graph():
    """Two alternating steps captured in one HIP graph, replayed three times
    with eager work between replays: each replay is two oracle steps."""
    d = ionn_synth.single_linear(B=300, IN=520, OUT=264, seed=33)
    X, W, dY = d["X"], d["W"], d["dY"]
    Wd, Xd, dYd = to_dev(W), to_dev(X), to_dev(dY)
    buf = steps.LinearStepBuffers.make(300, 520, 264, dev(), with_gq=True, alternate=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        steps.linear_step(Xd, Wd, dYd, buf, stream=s.cuda_stream)
        steps.linear_step(Xd, Wd, dYd, buf, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        say("alternating linear steps graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        want = osteps.linear_step(X, W, dY)
        want = osteps.linear_step(X, want["W_new"], dY)
        np.testing.assert_array_equal(host(Wd), want["W_new"], err_msg=f"replay {rep}: W")
        np.testing.assert_array_equal(host(buf.gq), want["Gq"], err_msg=f"replay {rep}: Gq")
        m = host(buf.scal[12:15]).astype(np.int64) & 0xFFFFFFFF   # the second step's set
        assert m.tolist() == [oracle.absmax(want["Y32"]), oracle.absmax(want["dX32"]), oracle.absmax(want["G"])]
        W = want["W_new"]
        torch.zeros(1000, device=dev()).add_(1.0)
