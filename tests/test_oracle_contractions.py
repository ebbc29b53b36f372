"""Pins for the oracle's contractions (linear and conv) and composed steps.

Independent references: hand-derived cases (tests/golden/contraction_cases.json),
numpy float64 matrix products and torch float64 conv2d and its gradients (exact
here: every partial sum is an integer far below 2^53), the adjoint identity
<Y,dY> = <X,dX> = <W,G>, and thread-count invariance.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import ionn_synth
from oracle import steps

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _i8(a):
    return np.ascontiguousarray(np.array(a, dtype=np.int8))


def _f64mm(a, b):
    return (a.astype(np.float64) @ b.astype(np.float64)).astype(np.int64)


# ---- linear --------------------------------------------------------------

def test_lin1_golden():
    c = _load("contraction_cases.json")["LIN-1"]
    X, W, dY = _i8(c["X"]), _i8(c["W"]), _i8(c["dY"])
    Y, dX, G = oracle.linear_fwd(X, W), oracle.linear_dgrad(dY, W), oracle.linear_wgrad(dY, X)
    assert Y.tolist() == c["Y"] and dX.tolist() == c["dX"] and G.tolist() == c["G"]
    ip = c["inner_product"]
    assert int((Y.astype(np.int64) * dY).sum()) == ip
    assert int((X.astype(np.int64) * dX).sum()) == ip
    assert int((W.astype(np.int64) * G).sum()) == ip


@pytest.mark.parametrize("B,IN,OUT", [(1, 1, 1), (3, 5, 7), (16, 64, 32), (17, 33, 10),
                                      (64, 784, 10), (5, 130, 257)])
def test_linear_vs_float64(B, IN, OUT):
    rng = np.random.default_rng(B * 1000 + IN)
    X = rng.integers(-128, 128, (B, IN)).astype(np.int8)
    W = rng.integers(-128, 128, (OUT, IN)).astype(np.int8)
    dY = rng.integers(-128, 128, (B, OUT)).astype(np.int8)
    Y, wy = oracle.linear_fwd(X, W, return_wraps=True)
    dX, wd = oracle.linear_dgrad(dY, W, return_wraps=True)
    G, wg = oracle.linear_wgrad(dY, X, return_wraps=True)
    np.testing.assert_array_equal(Y, _f64mm(X, W.T))
    np.testing.assert_array_equal(dX, _f64mm(dY, W))
    np.testing.assert_array_equal(G, _f64mm(dY.T, X))
    assert wy == wd == wg == 0
    # sampled single outputs agree with the full tensors
    for _ in range(10):
        b, o, i = rng.integers(B), rng.integers(OUT), rng.integers(IN)
        assert oracle.linear_fwd_at(X, W, b, o) == Y[b, o]
        assert oracle.linear_dgrad_at(dY, W, b, i) == dX[b, i]
        assert oracle.linear_wgrad_at(dY, X, o, i) == G[o, i]


def test_linear_adjoint_identity():
    d = ionn_synth.single_linear(B=40, IN=96, OUT=48, seed=3)
    X, W, dY = d["X"], d["W"], d["dY"]
    Y, dX, G = oracle.linear_fwd(X, W), oracle.linear_dgrad(dY, W), oracle.linear_wgrad(dY, X)
    a = int((Y.astype(np.int64) * dY).sum())
    assert a == int((X.astype(np.int64) * dX).sum()) == int((W.astype(np.int64) * G).sum())


def test_wraps_are_modular_and_counted():
    # 2^18 products of 127*127 = 16129 overflow int32: the result is the sum mod 2^32.
    K = 1 << 18
    X = np.full((1, K), 127, np.int8)
    W = np.full((1, K), 127, np.int8)
    Y, wraps = oracle.linear_fwd(X, W, return_wraps=True)
    exact = K * 16129
    want = ((exact + 2**31) % 2**32) - 2**31
    assert wraps == 1 and int(Y[0, 0]) == want


def test_thread_count_invariance():
    d = ionn_synth.single_linear(B=64, IN=256, OUT=96, seed=5)
    old = oracle.get_threads()
    try:
        oracle.set_threads(1)
        r1 = [oracle.linear_fwd(d["X"], d["W"]), oracle.linear_wgrad(d["dY"], d["X"])]
        oracle.set_threads(max(2, os.cpu_count() or 2))
        rn = [oracle.linear_fwd(d["X"], d["W"]), oracle.linear_wgrad(d["dY"], d["X"])]
    finally:
        oracle.set_threads(old)
    for a, b in zip(r1, rn):
        np.testing.assert_array_equal(a, b)


def test_relu_mask_and_output_error():
    d = np.array([[5, -3, 7], [1, 2, -9]], np.int32)
    act = np.array([[1, 0, -4], [127, 3, 2]], np.int8)
    assert oracle.relu_mask(d, act).tolist() == [[5, 0, 0], [1, 2, -9]]
    out = np.array([[10, -5, 127], [0, -128, 3]], np.int8)
    lab = np.array([2, 1], np.int32)
    assert oracle.output_error(out, lab, 127).tolist() == [[-10, 5, 0], [0, 255, -3]]


# ---- conv ----------------------------------------------------------------

def test_conv1_golden():
    c = _load("contraction_cases.json")["CONV-1"]
    X = _i8(c["X"]).reshape(1, 3, 3, 1)
    ones = np.ones((1, 3, 3, 1), np.int8)
    tap = np.zeros((1, 3, 3, 1), np.int8)
    tap[0, 0, 0, 0] = 1
    assert oracle.conv_fwd(X, ones).reshape(3, 3).tolist() == c["Y_ones"]
    assert oracle.conv_fwd(X, tap).reshape(3, 3).tolist() == c["Y_tap00"]
    assert oracle.conv_dgrad(X, tap, X.shape).reshape(3, 3).tolist() == c["dX_tap00_dY_eq_X"]
    imp = np.zeros((1, 3, 3, 1), np.int8)
    imp[0, 1, 1, 0] = 1
    np.testing.assert_array_equal(oracle.conv_wgrad(imp, X).reshape(3, 3), X.reshape(3, 3))


def _torch_conv_refs(X, W, dY, P):
    # NHWC -> NCHW, OHWI -> OIHW; float64 is exact for these integer sums.
    Xt = torch.from_numpy(X.astype(np.float64)).permute(0, 3, 1, 2).contiguous()
    Wt = torch.from_numpy(W.astype(np.float64)).permute(0, 3, 1, 2).contiguous()
    dYt = torch.from_numpy(dY.astype(np.float64)).permute(0, 3, 1, 2).contiguous()
    Y = torch.nn.functional.conv2d(Xt, Wt, padding=P)
    dX = torch.nn.grad.conv2d_input(Xt.shape, Wt, dYt, padding=P)
    G = torch.nn.grad.conv2d_weight(Xt, Wt.shape, dYt, padding=P)
    back = lambda t, perm: t.permute(*perm).contiguous().numpy().astype(np.int64)
    return back(Y, (0, 2, 3, 1)), back(dX, (0, 2, 3, 1)), back(G, (0, 2, 3, 1))


@pytest.mark.parametrize("N,H,Wd,Cin,Cout,K,P", [(1, 3, 3, 1, 1, 3, 1), (2, 5, 7, 3, 4, 3, 1),
                                                 (2, 6, 6, 8, 16, 3, 1), (1, 4, 5, 2, 3, 1, 0),
                                                 (1, 6, 5, 3, 2, 3, 0), (1, 7, 7, 2, 2, 5, 2)])
def test_conv_vs_torch_float64(N, H, Wd, Cin, Cout, K, P):
    rng = np.random.default_rng(N * 100 + H * 10 + Cin)
    X = rng.integers(-128, 128, (N, H, Wd, Cin)).astype(np.int8)
    W = rng.integers(-128, 128, (Cout, K, K, Cin)).astype(np.int8)
    Ho, Wo = H + 2 * P - K + 1, Wd + 2 * P - K + 1
    dY = rng.integers(-128, 128, (N, Ho, Wo, Cout)).astype(np.int8)
    Yr, dXr, Gr = _torch_conv_refs(X, W, dY, P)
    Y = oracle.conv_fwd(X, W, P)
    dX = oracle.conv_dgrad(dY, W, X.shape, P)
    G = oracle.conv_wgrad(dY, X, K, K, P)
    np.testing.assert_array_equal(Y, Yr)
    np.testing.assert_array_equal(dX, dXr)
    np.testing.assert_array_equal(G, Gr)
    for _ in range(5):
        n, h, w, c = rng.integers(N), rng.integers(Ho), rng.integers(Wo), rng.integers(Cout)
        assert oracle.conv_fwd_at(X, W, P, n, h, w, c) == Y[n, h, w, c]
        hh, ww, ci = rng.integers(H), rng.integers(Wd), rng.integers(Cin)
        assert oracle.conv_dgrad_at(dY, W, X.shape, P, n, hh, ww, ci) == dX[n, hh, ww, ci]
        co, kh, kw = rng.integers(Cout), rng.integers(K), rng.integers(K)
        assert oracle.conv_wgrad_at(dY, X, K, K, P, co, kh, kw, ci) == G[co, kh, kw, ci]


def _torch_conv_refs_rect(X, W, dY, P):
    Xt = torch.from_numpy(X.astype(np.float64)).permute(0, 3, 1, 2).contiguous()
    Wt = torch.from_numpy(W.astype(np.float64)).permute(0, 3, 1, 2).contiguous()
    dYt = torch.from_numpy(dY.astype(np.float64)).permute(0, 3, 1, 2).contiguous()
    Y = torch.nn.functional.conv2d(Xt, Wt, padding=P)
    dX = torch.nn.grad.conv2d_input(Xt.shape, Wt, dYt, padding=P)
    G = torch.nn.grad.conv2d_weight(Xt, Wt.shape, dYt, padding=P)
    back = lambda t: t.permute(0, 2, 3, 1).contiguous().numpy().astype(np.int64)
    return back(Y), back(dX), back(G)


# rectangular kernels, including the 16 x 2 "valid" filter bank of the TI
# page's arc-fault example network (input 64 x 2 x 1, 3 filters -> 49 x 1 x 3)
@pytest.mark.parametrize("N,H,Wd,Cin,Cout,KH,KW,P", [(8, 64, 2, 1, 3, 16, 2, 0), (2, 5, 4, 3, 2, 1, 3, 1),
                                                     (1, 9, 6, 2, 5, 4, 2, 1), (3, 7, 7, 4, 3, 5, 1, 0)])
def test_conv_rectangular_vs_torch_float64(N, H, Wd, Cin, Cout, KH, KW, P):
    rng = np.random.default_rng(H * 31 + KH * 7 + KW)
    X = rng.integers(-128, 128, (N, H, Wd, Cin)).astype(np.int8)
    W = rng.integers(-128, 128, (Cout, KH, KW, Cin)).astype(np.int8)
    Ho, Wo = H + 2 * P - KH + 1, Wd + 2 * P - KW + 1
    dY = rng.integers(-128, 128, (N, Ho, Wo, Cout)).astype(np.int8)
    Yr, dXr, Gr = _torch_conv_refs_rect(X, W, dY, P)
    np.testing.assert_array_equal(oracle.conv_fwd(X, W, P), Yr)
    np.testing.assert_array_equal(oracle.conv_dgrad(dY, W, X.shape, P), dXr)
    np.testing.assert_array_equal(oracle.conv_wgrad(dY, X, KH, KW, P), Gr)


def test_conv_adjoint_and_1x1_equals_linear():
    d = ionn_synth.conv3x3(N=2, H=9, W=7, Cin=16, Cout=8, seed=4)
    X, W, dY = d["X"], d["W"], d["dY"][..., :8]
    dY = np.ascontiguousarray(dY)
    Y, dX, G = oracle.conv_fwd(X, W), oracle.conv_dgrad(dY, W, X.shape), oracle.conv_wgrad(dY, X)
    a = int((Y.astype(np.int64) * dY).sum())
    assert a == int((X.astype(np.int64) * dX).sum()) == int((W.astype(np.int64) * G).sum())
    # I9: a 1x1 conv over N*H*W pixels is the linear layer over those rows
    W1 = np.ascontiguousarray(W[:, 1:2, 1:2, :])
    Y1 = oracle.conv_fwd(X, W1, 0)
    Xr = X.reshape(-1, 16)
    np.testing.assert_array_equal(Y1.reshape(-1, 8), oracle.linear_fwd(Xr, W1.reshape(8, 16)))
    G1 = oracle.conv_wgrad(dY, X, 1, 1, 0)
    np.testing.assert_array_equal(G1.reshape(8, 16), oracle.linear_wgrad(dY.reshape(-1, 8), Xr))


# ---- composed steps ------------------------------------------------------

def test_mlp_step_hand_case():
    """Two-layer MLP, batch 1, derived by hand (see the derivation below).

    Forward: z1 = [5,-2] -> a1 = ReLU = [5,0]; z2 = [10,5] = a2.  Error
    [117,-5] (7 bits, shift 0).  Layer 2: dgrad with the pre-update W2,
    117*[2,-1] - 5*[1,1] = [229,-122], masked by a1>0 -> [229,0], 8 bits ->
    shift 1 -> delta1 = [115,0]; G2 = [[585,0],[-25,0]], shift 2, ws 0,
    Gq = [146,0,-6,0] -> W2' = [[-128,-1],[7,1]].  Layer 1: dgrad
    115*[1,2] = [115,230] -> shift 1 -> delta0 = [58,115]; G1 = [[345,115],
    [0,0]], shift 1, ws 0, Gq = [173,58,0,0] -> W1' = [[-128,-56],[-1,1]].
    """
    X = _i8([[3, 1]])
    W1 = _i8([[1, 2], [-1, 1]])
    W2 = _i8([[2, -1], [1, 1]])
    lab = np.array([0], np.int32)
    (W1n, W2n), rec = steps.mlp_step(X, lab, [W1, W2])
    assert rec["acts"][1].tolist() == [[5, 0]] and rec["acts"][2].tolist() == [[10, 5]]
    assert rec["s_fwd"] == [0, 0] and rec["s_err"] == 0
    assert rec["deltas"][2].tolist() == [[117, -5]]
    assert rec["deltas"][1].tolist() == [[115, 0]] and rec["deltas"][0].tolist() == [[58, 115]]
    assert rec["s_dgrad"] == [1, 1]
    assert rec["s_upd"] == [(1, 0), (2, 0)]
    assert W2n.tolist() == [[-128, -1], [7, 1]]
    assert W1n.tolist() == [[-128, -56], [-1, 1]]


def test_mlp_train_invariants_small():
    d = ionn_synth.mlp(B=32, sizes=(40, 24, 16, 10), seed=0)
    Ws, recs = steps.mlp_train(d["X"], d["labels"], d["Ws"], steps=3)
    assert len(recs) == 3
    for rec in recs:
        for a in rec["acts"][1:3]:
            assert a.min() >= 0                         # ReLU on hidden layers
        for l, dl in enumerate(rec["deltas"][:-1]):
            assert dl.min() >= -128 and dl.max() <= 127
            if 1 <= l <= 2:
                assert not dl[rec["acts"][l] <= 0].any()  # masked where the unit was off
    for W0, W1 in zip(d["Ws"], Ws):
        assert W0.shape == W1.shape and W1.dtype == np.int8


def test_linear_step_config1_properties():
    d = ionn_synth.single_linear()
    r = steps.linear_step(d["X"], d["W"], d["dY"])
    np.testing.assert_array_equal(r["Y32"], _f64mm(d["X"], d["W"].T))
    np.testing.assert_array_equal(r["G"], _f64mm(d["dY"].T, d["X"]))
    assert r["s"] == oracle.niti_shift(oracle.absmax(r["G"]), 8)
    assert r["ws"] == max(0, r["s"] - 2)
    assert r["s_d"] == oracle.niti_shift(oracle.absmax(r["dX32"]), 7)
    assert (r["W_new"] != d["W"]).any()   # the small config moves the weights


@pytest.mark.parametrize("case", ["STEP-1", "STEP-2"])
def test_conv_step_golden(case):
    """The oracle's whole conv step (forward + requantisation, dgrad +
    requantisation, wgrad + NITI update) on hand-worked cases."""
    from oracle import steps as osteps
    with open(os.path.join(GOLD, "conv_step_cases.json")) as f:
        c = json.load(f)[case]
    img = lambda k: np.array(c[k], np.int8).reshape(1, 3, 3, 1)
    W = np.array(c["W"], np.int8).reshape(1, 3, 3, 1)
    r = osteps.conv_step(img("X"), W, img("dY"))
    np.testing.assert_array_equal(r["y8"].reshape(3, 3), c["y8"])
    np.testing.assert_array_equal(r["dx8"].reshape(3, 3), c["dx8"])
    np.testing.assert_array_equal(r["G"].reshape(3, 3), c["G"])
    np.testing.assert_array_equal(r["Gq"].reshape(3, 3), c["Gq"])
    np.testing.assert_array_equal(r["W_new"].reshape(3, 3), c["W_new"])
    assert (r["s_y"], r["s_dx"], r["s"], r["ws"]) == (c["s_y"], c["s_dx"], c["s"], c["ws"])
