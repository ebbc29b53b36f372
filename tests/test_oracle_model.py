"""Pins for the oracle's model-level driver (the INT_LAYERS forward and
backward of the TI "Integer On-Device Training: Overview" page, sections 7
and 8) and its per-class target error.  Each check compares the driver with
something other than itself: hand-derived errors, an int64 numpy forward of
the example network followed by the OSS chain in float64, reductions to the
already pinned single-layer pieces, a 1x1 convolution against the linear
layer over pixels, and the zero-error fixed point."""
import json
import os

import numpy as np
import pytest

import ionn_synth
import oracle
from oracle import steps

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_mse_grad_golden():
    c = json.load(open(os.path.join(GOLD, "oss_cases.json")))["targets"][0]
    g = oracle.mse_grad_targets(np.array(c["out"], np.int8), np.array(c["labels"], np.int32),
                                np.array(c["tmc"], np.int8), np.array(c["tmw"], np.int8))
    assert g.tolist() == c["g"]


def test_mse_grad_is_the_negated_single_target_error():
    # with tmc = 127 and tmw = 0 it is -(onehot*127 - out), the pinned output error negated
    rng = np.random.default_rng(1)
    out = rng.integers(-128, 128, (33, 7)).astype(np.int8)
    labels = rng.integers(0, 7, 33).astype(np.int32)
    g = oracle.mse_grad_targets(out, labels, np.full(7, 127, np.int8), np.zeros(7, np.int8))
    np.testing.assert_array_equal(g, -oracle.output_error(out, labels, 127))


def _np_conv_valid(X, W):
    # int64 sliding-window correlation, stride 1, no padding
    N, H, Wd, Cin = X.shape
    Cout, KH, KW, _ = W.shape
    Ho, Wo = H - KH + 1, Wd - KW + 1
    Y = np.zeros((N, Ho, Wo, Cout), np.int64)
    for kh in range(KH):
        for kw in range(KW):
            Y += np.einsum("nhwc,oc->nhwo", X[:, kh:kh + Ho, kw:kw + Wo, :].astype(np.int64),
                           W[:, kh, kw, :].astype(np.int64))
    return Y


def _oss_f64(z, L):
    t = z.astype(np.float64) + L["offset"].astype(np.float64)
    y = np.floor(t * L["mult"].astype(np.float64) * np.exp2(-L["k"].astype(np.float64)))
    return np.clip(y, 0.0 if L["relu"] else -128.0, 127.0).astype(np.int8)


def test_forward_of_example_network_independent():
    d = ionn_synth.arc_fault()
    layers = steps.arc_fault_layers(d)
    acts = steps.model_forward(layers, d["X"])
    a1 = _oss_f64(_np_conv_valid(d["X"], layers[0]["weight"]), layers[0])
    np.testing.assert_array_equal(acts[1], a1)
    a2 = _oss_f64(a1.reshape(8, -1).astype(np.int64) @ layers[1]["weight"].astype(np.int64).T, layers[1])
    np.testing.assert_array_equal(acts[2], a2)
    a3 = _oss_f64(a2.astype(np.int64) @ layers[2]["weight"].astype(np.int64).T, layers[2])
    np.testing.assert_array_equal(acts[3], a3)
    assert acts[1].shape == (8, 49, 1, 3) and acts[3].shape == (8, 2)


def _linear_layer(rng, IN, OUT, relu):
    return dict(kind="linear", relu=relu, IN=IN, OUT=OUT,
                weight=rng.integers(-128, 128, (OUT, IN)).astype(np.int8),
                offset=rng.integers(-300, 300, OUT).astype(np.int32),
                mult=rng.integers(1, 5, OUT).astype(np.int32),
                k=rng.integers(6, 9, OUT).astype(np.int8))


def test_single_linear_model_is_the_layer_step():
    rng = np.random.default_rng(2)
    L = _linear_layer(rng, 40, 6, relu=False)
    X = rng.integers(-128, 128, (12, 40)).astype(np.int8)
    labels = rng.integers(0, 6, 12).astype(np.int32)
    tmc, tmw = np.full(6, 90, np.int8), np.full(6, -70, np.int8)
    new, rec = steps.model_step([L], X, labels, tmc, tmw)
    out = oracle.oss_requant(oracle.linear_fwd(X, L["weight"]), L["offset"], L["mult"], L["k"])
    g = oracle.mse_grad_targets(out, labels, tmc, tmw)
    delta, _ = oracle.niti_requant(g, 7)
    W_new, *_ = oracle.niti_update(oracle.linear_wgrad(delta, X), L["weight"], 8, 2)
    off_new, *_ = oracle.niti_update_i32(delta.astype(np.int64).sum(0).astype(np.int32), L["offset"], 8, 2)
    np.testing.assert_array_equal(new[0]["weight"], W_new)
    np.testing.assert_array_equal(new[0]["offset"], off_new)


def test_1x1_conv_model_equals_linear_model_over_pixels():
    rng = np.random.default_rng(3)
    Lin = _linear_layer(rng, 5, 4, relu=False)
    Lc = dict(Lin, kind="conv", H=3, W=2, Cin=5, Cout=4, KH=1, KW=1, pad=0,
              weight=Lin["weight"].reshape(4, 1, 1, 5))
    X = rng.integers(-128, 128, (2, 3, 2, 5)).astype(np.int8)
    acts_c = steps.model_forward([Lc], X)
    acts_l = steps.model_forward([Lin], X.reshape(-1, 5))
    np.testing.assert_array_equal(acts_c[1].reshape(-1, 4), acts_l[1])


def test_zero_error_is_a_fixed_point():
    d = ionn_synth.arc_fault(B=1, seed=5)
    layers = steps.arc_fault_layers(d)
    out = steps.model_forward(layers, d["X"])[-1]
    lab = np.array([0], np.int32)
    tmc = np.array([out[0, 0], 0], np.int8)
    tmw = np.array([0, out[0, 1]], np.int8)
    new, rec = steps.model_step(layers, d["X"], lab, tmc, tmw)
    assert not rec["e32"].any()
    for a, b in zip(new, layers):
        np.testing.assert_array_equal(a["weight"], b["weight"])
        np.testing.assert_array_equal(a["offset"], b["offset"])


def test_example_network_trains():
    """Ten steps on one fixed batch move the logits toward the targets."""
    d = ionn_synth.arc_fault()
    layers = steps.arc_fault_layers(d)
    tgt = np.where(np.arange(2)[None, :] == d["labels"][:, None], d["tmc"][None, :], d["tmw"][None, :])
    err0 = np.abs(steps.model_forward(layers, d["X"])[-1].astype(int) - tgt).mean()
    for _ in range(10):
        layers, _ = steps.model_step(layers, d["X"], d["labels"], d["tmc"], d["tmw"])
    err1 = np.abs(steps.model_forward(layers, d["X"])[-1].astype(int) - tgt).mean()
    assert err1 < err0
