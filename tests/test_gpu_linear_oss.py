"""GPU parity: a Linear layer's forward with its offsets and the static OSS
requantisation ("Integer On-Device Training: Overview", sections 7 and 8),
against the oracle's contraction followed by its OSS chain, bit-exact.  The
tile-aligned shapes run the contraction with the chain in its epilogue; the
others go through an int32 workspace."""
import numpy as np
import pytest
import torch

import ionn_synth
import oracle
from oracle import fast
from integer_only_nn_amd import ops
from integer_only_nn_amd._lib import IonnError
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu

IONN_ERR_WORKSPACE = 7


def _params(OUT, seed, k_lo, k_hi):
    rng = np.random.default_rng(seed)
    off = rng.integers(-2**18, 2**18, OUT, dtype=np.int64).astype(np.int32)
    mult = rng.integers(1, 2**11, OUT, dtype=np.int64).astype(np.int32)
    mult[::7] *= -1
    k = rng.integers(k_lo, k_hi, OUT).astype(np.int8)
    return off, mult, k


def _run(X, W, off, mult, k, relu, workspace=True, misalign_y=False):
    B, IN = X.shape
    OUT = W.shape[0]
    if misalign_y:
        buf = torch.empty(B * OUT + 1, dtype=torch.int8, device=dev())
        Y = buf[1:].view(B, OUT)
    else:
        Y = torch.empty(B, OUT, dtype=torch.int8, device=dev())
    ws = None
    nb = ops.int_linear_fwd_oss_workspace_bytes(B, IN, OUT)
    if workspace:
        ws = torch.empty(max(nb, B * OUT * 4, 16), dtype=torch.uint8, device=dev())
    ops.int_linear_fwd_oss(to_dev(X), to_dev(W), to_dev(off), to_dev(mult), to_dev(k), Y, relu=relu,
                           workspace=ws)
    return host(Y)


SHAPES = [(256, 256, 256), (512, 768, 1024), (1, 1, 1), (100, 70, 33), (256, 256, 100), (300, 512, 256),
          (256, 100, 256)]


@pytest.mark.parametrize("B,IN,OUT", SHAPES)
@pytest.mark.parametrize("relu", [False, True])
def test_fwd_oss_vs_oracle(B, IN, OUT, relu):
    say("fwd_oss", B, IN, OUT, relu)
    rng = np.random.default_rng(B + IN + OUT)
    X = rng.integers(-128, 128, (B, IN), dtype=np.int64).astype(np.int8)
    W = rng.integers(-128, 128, (OUT, IN), dtype=np.int64).astype(np.int8)
    off, mult, k = _params(OUT, seed=OUT, k_lo=8, k_hi=20)
    want = oracle.oss_requant(oracle.linear_fwd(X, W), off, mult, k, relu=relu)
    tile = B % 256 == 0 and IN % 256 == 0 and OUT % 256 == 0
    assert (ops.int_linear_fwd_oss_workspace_bytes(B, IN, OUT) == 0) == tile
    got = _run(X, W, off, mult, k, relu, workspace=not tile)
    np.testing.assert_array_equal(got, want)


def test_fwd_oss_workspace_rules():
    rng = np.random.default_rng(3)
    B, IN, OUT = 256, 256, 256
    X = rng.integers(-128, 128, (B, IN), dtype=np.int64).astype(np.int8)
    W = rng.integers(-128, 128, (OUT, IN), dtype=np.int64).astype(np.int8)
    off, mult, k = _params(OUT, seed=4, k_lo=10, k_hi=14)
    want = oracle.oss_requant(oracle.linear_fwd(X, W), off, mult, k)
    # a misaligned output leaves the fused kernel: without a workspace the call
    # is refused, with one it is exact
    with pytest.raises(IonnError) as e:
        _run(X, W, off, mult, k, False, workspace=False, misalign_y=True)
    assert e.value.status == IONN_ERR_WORKSPACE
    np.testing.assert_array_equal(_run(X, W, off, mult, k, False, workspace=True, misalign_y=True), want)
    # an untiled shape without a workspace is refused too
    with pytest.raises(IonnError):
        _run(X[:100], W, off, mult, k, False, workspace=False)


def test_fwd_oss_large_linear_full():
    """The 8192 x 4096 x 4096 forward of the benchmark's workload, every
    element against the oracle (float64-product contraction, pinned to the C
    loops by tests/test_oracle_fast.py, then the OSS chain)."""
    d = ionn_synth.large_linear()
    X, W = d["X"], d["W"]
    off, mult, k = _params(4096, seed=11, k_lo=16, k_hi=22)
    for relu in (False, True):
        say("fwd_oss full", relu)
        got = _run(X, W, off, mult, k, relu, workspace=False)
        Yo = fast.linear_fwd(X, W)
        want = oracle.oss_requant(Yo, off, mult, k, relu=relu)
        np.testing.assert_array_equal(got, want)
        lo = 0 if relu else -128
        assert (want == 127).any() and (want == lo).any() and ((want > lo) & (want < 127)).mean() > 0.1
