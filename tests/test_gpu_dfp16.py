"""GPU parity: DFP-16 chunked contractions (int8-split on the matrix cores),
down-conversion with its exponents, and Gavg against the oracle, bit-exact
(Gavg as an IEEE double)."""
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


def _exp(v):
    return torch.tensor([v], dtype=torch.int32, device=dev())


def _run(d, M, K, N):
    buf = steps.DfpStepBuffers.make(M, K, N, dev())
    steps.dfp16_step(to_dev(d["X"]), _exp(d["eX"]), to_dev(d["W"]), _exp(d["eW"]), to_dev(d["dY"]),
                     _exp(d["edY"]), buf)
    return buf


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 64, 5), (17, 40, 9), (128, 128, 128), (200, 256, 136),
                                   (128, 64, 128), (640, 128, 384), (1024, 384, 128),
                                   (256, 320, 1024), (1000, 64, 48), (4096, 256, 256),
                                   (2304, 128, 2048),
                                   # more output tiles than compute units, a last round
                                   # that leaves most workgroups idle: fwd (456 tiles of
                                   # 3 chunks), dgrad (456 tiles of 3 chunks, 272 of 2)
                                   (3072, 192, 2432), (3072, 2432, 192), (2176, 2048, 128)])
def test_dfp16_step_vs_oracle(M, K, N):
    say("dfp16", M, K, N)
    d = ionn_synth.dfp16_gemm(M=M, K=K, N=N, seed=M + K)
    want = osteps.dfp16_step(d["X"], d["eX"], d["W"], d["eW"], d["dY"], d["edY"])
    buf = _run(d, M, K, N)
    np.testing.assert_array_equal(host(buf.Y), want["Y"])
    np.testing.assert_array_equal(host(buf.dX), want["dX"])
    np.testing.assert_array_equal(host(buf.G), want["G"])
    e = host(buf.exps).tolist()
    assert e[:3] == [want["eY"], want["edX"], want["eG"]] and e[3:6] == [0, 0, 0]
    assert float(host(buf.gavg)[0]) == want["gavg"]


def test_dfp16_golden_chunk_case():
    c = dict(X=np.zeros((2, 128), np.int16), W=np.zeros((1, 128), np.int16))
    c["X"][0, :] = 1000
    c["X"][1, 0] = 7
    c["W"][0, :64] = 3
    c["W"][0, 64:] = -1
    Y = torch.empty(2, 1, dtype=torch.int16, device=dev())
    eY = _exp(0)
    ws = torch.empty(ops.dfp16_workspace_bytes(2, 128, 1, 0), dtype=torch.uint8, device=dev())
    ops.dfp16_gemm_fwd(to_dev(c["X"]), _exp(-10), to_dev(c["W"]), _exp(-12), Y, eY, ws)
    assert host(Y)[:, 0].tolist() == [32000, 6] and int(host(eY)[0]) == -20


@pytest.mark.parametrize("M,K,N", [(64, 192, 32), (256, 128, 128)])
def test_dfp16_extreme_mantissas(M, K, N):
    """Values at +-32767 / -32768 exercise the high-digit range of the split
    (the second shape takes the tile-aligned 32x32x32 path in all three
    contractions, the first the general one)."""
    rng = np.random.default_rng(3)
    pick = np.array([-32768, -32767, 32767, 32640, 32639, -129, -128, 127, 128, 0, 1, -1], np.int16)
    X = pick[rng.integers(0, len(pick), (M, K))]
    W = pick[rng.integers(0, len(pick), (N, K))]
    dY = pick[rng.integers(0, len(pick), (M, N))]
    d = dict(X=X, W=W, dY=dY, eX=-30, eW=-30, edY=-30)
    want = osteps.dfp16_step(X, -30, W, -30, dY, -30)
    buf = _run(d, M, K, N)
    np.testing.assert_array_equal(host(buf.Y), want["Y"])
    np.testing.assert_array_equal(host(buf.dX), want["dX"])
    np.testing.assert_array_equal(host(buf.G), want["G"])


@pytest.mark.parametrize("M,K,N", [(256, 256, 128), (512, 128, 256), (4352, 128, 1024)])
def test_dfp16_blocks_far_below_the_tensor_shift(M, K, N):
    """Row blocks of X and dY at scales from zero to full range.  Without K
    splits the contractions store every 32-row block at its own shift, and
    the in-place pass then moves each block by d = Rs - s_b: from 0 for the
    full-range blocks past 16 for the all-zero ones (full-range products
    wrap their chunks, so the tensor's maximum nears 2^31)."""
    rng = np.random.default_rng(11)
    scales = [0, 1, 3, 40, 300, 3000, 32767, 32767]

    def rows(n, k):
        a = np.zeros((n, k), np.int16)
        for b in range(0, n, 32):
            sc = scales[(b // 32) % len(scales)]
            if sc:
                a[b:b + 32] = rng.integers(-sc, sc + 1, (min(32, n - b), k))
        return a

    X, dY = rows(M, K), rows(M, N)
    W = rng.integers(-32768, 32768, (N, K)).astype(np.int16)
    d = dict(X=X, W=W, dY=dY, eX=-20, eW=-20, edY=-20)
    want = osteps.dfp16_step(X, -20, W, -20, dY, -20)
    buf = _run(d, M, K, N)
    np.testing.assert_array_equal(host(buf.Y), want["Y"])
    np.testing.assert_array_equal(host(buf.dX), want["dX"])
    np.testing.assert_array_equal(host(buf.G), want["G"])
    e = host(buf.exps).tolist()
    assert e[:3] == [want["eY"], want["edX"], want["eG"]]


def test_dfp16_exponent_overflow_flagged():
    X = np.full((16, 64), 30000, np.int16)
    W = np.full((16, 64), 30000, np.int16)
    Y = torch.empty(16, 16, dtype=torch.int16, device=dev())
    eY, st = _exp(0), _exp(0)
    ws = torch.empty(ops.dfp16_workspace_bytes(16, 64, 16, 0), dtype=torch.uint8, device=dev())
    ops.dfp16_gemm_fwd(to_dev(X), _exp(120), to_dev(W), _exp(10), Y, eY, ws, status_out=st)
    assert int(host(st)[0]) == 1


def test_dfp16_workload_full():
    """M=25088, K=256, N=1024: every output, exponent and Gavg against the
    oracle (float64-product variant of the chunked contraction)."""
    M, K, N = 25088, 256, 1024
    say("generating DFP-16 inputs")
    d = ionn_synth.dfp16_gemm()
    buf = _run(d, M, K, N)
    e = host(buf.exps).tolist()
    assert e[3:6] == [0, 0, 0]
    say("oracle: forward")
    Yo, eY, _ = fast.dfp16_fwd(d["X"], d["eX"], d["W"], d["eW"])
    np.testing.assert_array_equal(host(buf.Y), Yo)
    say("oracle: dgrad")
    dXo, edX, _ = fast.dfp16_dgrad(d["dY"], d["edY"], d["W"], d["eW"])
    np.testing.assert_array_equal(host(buf.dX), dXo)
    say("oracle: wgrad")
    Go, eG, _ = fast.dfp16_wgrad(d["dY"], d["edY"], d["X"], d["eX"])
    np.testing.assert_array_equal(host(buf.G), Go)
    assert e[:3] == [eY, edX, eG]
    assert float(host(buf.gavg)[0]) == oracle.gavg(Go, eG, d["eW"])


@pytest.mark.parametrize("M,K,N", [(640, 128, 384), (256, 320, 1024)])
def test_dfp16_step_replayed_from_graph(M, K, N):
    """The DFP-16 step (three contractions with their K splits and
    reductions, the down-conversions, Gavg) captured in one HIP graph and
    replayed three times; the outputs are overwritten between replays, so
    each replay has to rebuild every value, exponent and status."""
    d = ionn_synth.dfp16_gemm(M=M, K=K, N=N, seed=M + 3 * K)
    want = osteps.dfp16_step(d["X"], d["eX"], d["W"], d["eW"], d["dY"], d["edY"])
    buf = steps.DfpStepBuffers.make(M, K, N, dev())
    args = (to_dev(d["X"]), _exp(d["eX"]), to_dev(d["W"]), _exp(d["eW"]), to_dev(d["dY"]), _exp(d["edY"]))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        steps.dfp16_step(*args, buf, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        say("dfp16 graph replay", rep, M, K, N)
        for t, v in ((buf.Y, 123), (buf.dX, -5), (buf.G, 77), (buf.exps, -7), (buf.gavg, -1.0)):
            t.fill_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(buf.Y), want["Y"], err_msg=f"replay {rep}: Y")
        np.testing.assert_array_equal(host(buf.dX), want["dX"], err_msg=f"replay {rep}: dX")
        np.testing.assert_array_equal(host(buf.G), want["G"], err_msg=f"replay {rep}: G")
        e = host(buf.exps).tolist()
        assert e[:3] == [want["eY"], want["edX"], want["eG"]] and e[3:6] == [0, 0, 0], (rep, e)
        assert float(host(buf.gavg)[0]) == want["gavg"]
