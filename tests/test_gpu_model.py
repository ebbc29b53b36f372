"""GPU parity: the model-level driver (ionn_model_forward / backward, the
INT_LAYERS forward and backward of the TI "Integer On-Device Training:
Overview" page, sections 7 and 8) against the oracle's model step, bit-exact:
the page's arc-fault example network (Conv 16x2 valid + ReLU, Linear 160 +
ReLU, Linear 2, batch 8) over ten steps, a large batch of it, and a model of
3x3 convolutions that exercises the conv dgrad mask."""
import numpy as np
import pytest
import torch

import ionn_synth
import oracle
from oracle import steps as osteps
from integer_only_nn_amd import steps
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def _check_step(m, layers, X, labels, tmc, tmw, step_no):
    new, rec = osteps.model_step(layers, X, labels, tmc, tmw)
    m.step(to_dev(X), to_dev(labels), to_dev(tmc), to_dev(tmw))
    L = len(layers)
    np.testing.assert_array_equal(host(m.out), rec["acts"][-1].reshape(X.shape[0], -1),
                                  err_msg=f"step {step_no}: output")
    for l in range(L):
        np.testing.assert_array_equal(host(m.dev[l]["weight"]), new[l]["weight"], err_msg=f"step {step_no} W{l}")
        np.testing.assert_array_equal(host(m.dev[l]["offset"]), new[l]["offset"], err_msg=f"step {step_no} b{l}")
    sh = host(m.shifts).tolist()
    assert sh[0] == rec["s_err"]
    for l in range(L):
        want = [rec["s_dgrad"].get(l, -1), *rec["s_w"][l], *rec["s_b"][l]]
        assert sh[1 + 5 * l:6 + 5 * l] == want, (step_no, l, sh, want)
    return new


def test_arc_fault_network_ten_steps():
    d = ionn_synth.arc_fault()
    layers = osteps.arc_fault_layers(d)
    m = steps.Model(layers, 8, dev())
    for i in range(10):
        say("arc-fault step", i)
        layers = _check_step(m, layers, d["X"], d["labels"], d["tmc"], d["tmw"], i)


def test_arc_fault_network_large_batch():
    B = 4096
    d = ionn_synth.arc_fault(B=B, seed=3)
    layers = osteps.arc_fault_layers(d)
    m = steps.Model(layers, B, dev())
    for i in range(3):
        say("arc-fault B=4096 step", i)
        layers = _check_step(m, layers, d["X"], d["labels"], d["tmc"], d["tmw"], i)


def test_arc_fault_network_bench_batch():
    """The batch the benchmark times (65536): the narrow-layer contractions
    over 512 stages on one workgroup per compute unit, the long-batch
    weight gradients over 256 batch ranges, the full-row-window conv
    kernels; two steps, every weight, offset, shift and output."""
    B = 65536
    d = ionn_synth.arc_fault(B=B, seed=5)
    layers = osteps.arc_fault_layers(d)
    m = steps.Model(layers, B, dev())
    for i in range(2):
        say("arc-fault B=65536 step", i)
        layers = _check_step(m, layers, d["X"], d["labels"], d["tmc"], d["tmw"], i)


def _conv_layer(rng, H, W, Cin, Cout, K, pad, relu):
    return dict(kind="conv", relu=relu, H=H, W=W, Cin=Cin, Cout=Cout, KH=K, KW=K, pad=pad,
                weight=np.clip(np.round(rng.normal(0, 12, (Cout, K, K, Cin))), -128, 127).astype(np.int8),
                offset=rng.integers(-200, 200, Cout).astype(np.int32),
                mult=rng.integers(1, 4, Cout).astype(np.int32),
                k=rng.integers(9, 11, Cout).astype(np.int8))


def test_conv_stack_model():
    """3x3 / pad 1 convolutions of 16 channels (matrix-core path) after a 3x3
    conv from 3 channels (direct path), then a Linear: every dgrad of a conv
    is masked by the previous conv's ReLU."""
    rng = np.random.default_rng(9)
    B, H, W = 6, 10, 9
    layers = [_conv_layer(rng, H, W, 3, 16, 3, 1, True), _conv_layer(rng, H, W, 16, 16, 3, 1, True),
              _conv_layer(rng, H, W, 16, 16, 3, 1, True),
              dict(kind="linear", relu=False, IN=H * W * 16, OUT=5,
                   weight=np.clip(np.round(rng.normal(0, 10, (5, H * W * 16))), -128, 127).astype(np.int8),
                   offset=rng.integers(-200, 200, 5).astype(np.int32),
                   mult=rng.integers(1, 4, 5).astype(np.int32), k=rng.integers(10, 12, 5).astype(np.int8))]
    X = rng.integers(-100, 100, (B, H, W, 3)).astype(np.int8)
    labels = rng.integers(0, 5, B).astype(np.int32)
    tmc, tmw = np.full(5, 80, np.int8), np.full(5, -50, np.int8)
    m = steps.Model(layers, B, dev())
    for i in range(3):
        say("conv stack step", i)
        layers = _check_step(m, layers, X, labels, tmc, tmw, i)


@pytest.mark.parametrize("B", [1, 3, 33, 100])
def test_arc_fault_network_batches(B):
    """Batches on both sides of the one-workgroup path's size limit (about
    4M multiply-adds per step: B = 1, 3, 33 take it, B = 100 the
    multi-kernel driver)."""
    d = ionn_synth.arc_fault(B=B, seed=B)
    layers = osteps.arc_fault_layers(d)
    m = steps.Model(layers, B, dev())
    for i in range(3):
        say("arc-fault B", B, "step", i)
        layers = _check_step(m, layers, d["X"], d["labels"], d["tmc"], d["tmw"], i)


def test_conv_stack_model_small():
    """The 3x3 conv stack at a size the one-workgroup path takes: padded
    convolutions, the masked conv dgrad and a flattening Linear."""
    rng = np.random.default_rng(11)
    B, H, W = 2, 6, 5
    layers = [_conv_layer(rng, H, W, 3, 16, 3, 1, True), _conv_layer(rng, H, W, 16, 16, 3, 1, True),
              _conv_layer(rng, H, W, 16, 16, 3, 1, False),
              dict(kind="linear", relu=True, IN=H * W * 16, OUT=7,
                   weight=np.clip(np.round(rng.normal(0, 10, (7, H * W * 16))), -128, 127).astype(np.int8),
                   offset=rng.integers(-200, 200, 7).astype(np.int32),
                   mult=rng.integers(1, 4, 7).astype(np.int32), k=rng.integers(10, 12, 7).astype(np.int8))]
    X = rng.integers(-100, 100, (B, H, W, 3)).astype(np.int8)
    labels = np.array([2, 9], np.int32)   # 9 matches no class
    tmc, tmw = np.full(7, 70, np.int8), np.full(7, -40, np.int8)
    m = steps.Model(layers, B, dev())
    for i in range(3):
        say("small conv stack step", i)
        layers = _check_step(m, layers, X, labels, tmc, tmw, i)


def _mlp(rng, dims, relus):
    layers = []
    for i in range(len(dims) - 1):
        n_in, n_out = dims[i], dims[i + 1]
        layers.append(dict(kind="linear", relu=relus[i], IN=n_in, OUT=n_out,
                           weight=np.clip(np.round(rng.normal(0, 25, (n_out, n_in))), -128, 127).astype(np.int8),
                           offset=rng.integers(-300, 300, n_out).astype(np.int32),
                           mult=rng.integers(1, 5, n_out).astype(np.int32),
                           k=rng.integers(6, 10, n_out).astype(np.int8)))
    return layers


@pytest.mark.parametrize("L", [8, 9])
def test_deep_mlp_layer_limit(L):
    """Ragged widths, ReLU on some layers only: eight layers run in one
    workgroup, nine on the multi-kernel path; both bit-exact, every shift."""
    rng = np.random.default_rng(40 + L)
    dims = [37, 23, 64, 5, 17, 33, 9, 40, 3, 11][:L + 1]
    relus = [True, False, True, True, False, True, True, False, True][:L]
    layers = _mlp(rng, dims, relus)
    B = 4
    X = rng.integers(-128, 128, (B, dims[0])).astype(np.int8)
    C = dims[-1]
    labels = np.array([0, C - 1, 1, C + 3], np.int32)   # the last matches no class
    tmc, tmw = np.full(C, 90, np.int8), np.full(C, -20, np.int8)
    m = steps.Model(layers, B, dev())
    for i in range(3):
        say(f"deep MLP L={L} step", i)
        layers = _check_step(m, layers, X, labels, tmc, tmw, i)


@pytest.mark.parametrize("B", [8, 100])
def test_model_step_replayed_from_graph(B):
    """A whole training step captured in one HIP graph and replayed three
    times, with eager work and synchronisations between the replays: each
    replay matches the oracle's next step (B = 8: the one-workgroup kernels;
    B = 100: the multi-kernel driver)."""
    d = ionn_synth.arc_fault(B=B, seed=50 + B)
    layers = osteps.arc_fault_layers(d)
    m = steps.Model(layers, B, dev())
    X, lab, tmc, tmw = (to_dev(d[k]) for k in ("X", "labels", "tmc", "tmw"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        m.step(X, lab, tmc, tmw, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        say("graph replay", rep, "B", B)
        g.replay()
        torch.cuda.synchronize()
        new, rec = osteps.model_step(layers, d["X"], d["labels"], d["tmc"], d["tmw"])
        np.testing.assert_array_equal(host(m.out), rec["acts"][-1].reshape(B, -1), err_msg=f"replay {rep}: output")
        for l in range(len(layers)):
            np.testing.assert_array_equal(host(m.dev[l]["weight"]), new[l]["weight"], err_msg=f"replay {rep} W{l}")
            np.testing.assert_array_equal(host(m.dev[l]["offset"]), new[l]["offset"], err_msg=f"replay {rep} b{l}")
        assert host(m.shifts).tolist()[0] == rec["s_err"]
        layers = new
        torch.zeros(1000, device=dev()).add_(1.0)   # unrelated eager work between replays


@pytest.mark.parametrize("B", [2, 40, 64])
def test_rectangular_padded_conv_model(B):
    """Rectangular kernels with and without padding (1x3 pad 1 grows the
    height by two rows, 2x2 valid shrinks both), odd channel counts, both
    paths (B = 2 and 40 one workgroup; B = 64 multi-kernel: the second
    layer's 64*7*4*5 input gradients exceed the 8192 kept in LDS)."""
    rng = np.random.default_rng(90 + B)
    H, W = 5, 4

    def conv(H, W, Cin, Cout, KH, KW, pad, relu):
        return dict(kind="conv", relu=relu, H=H, W=W, Cin=Cin, Cout=Cout, KH=KH, KW=KW, pad=pad,
                    weight=np.clip(np.round(rng.normal(0, 20, (Cout, KH, KW, Cin))), -128, 127).astype(np.int8),
                    offset=rng.integers(-200, 200, Cout).astype(np.int32),
                    mult=rng.integers(1, 4, Cout).astype(np.int32), k=rng.integers(6, 9, Cout).astype(np.int8))

    l0 = conv(H, W, 3, 5, 1, 3, 1, True)            # -> (H + 2) x W x 5
    l1 = conv(H + 2, W, 5, 4, 2, 2, 0, True)        # -> (H + 1) x (W - 1) x 4
    n_in = (H + 1) * (W - 1) * 4
    l2 = dict(kind="linear", relu=False, IN=n_in, OUT=6,
              weight=np.clip(np.round(rng.normal(0, 15, (6, n_in))), -128, 127).astype(np.int8),
              offset=rng.integers(-200, 200, 6).astype(np.int32),
              mult=rng.integers(1, 4, 6).astype(np.int32), k=rng.integers(6, 9, 6).astype(np.int8))
    layers = [l0, l1, l2]
    X = rng.integers(-128, 128, (B, H, W, 3)).astype(np.int8)
    labels = rng.integers(0, 7, B).astype(np.int32)   # 6 matches no class
    tmc, tmw = np.full(6, 100, np.int8), np.full(6, -30, np.int8)
    m = steps.Model(layers, B, dev())
    for i in range(3):
        say("rectangular conv model B", B, "step", i)
        layers = _check_step(m, layers, X, labels, tmc, tmw, i)
