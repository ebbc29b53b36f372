"""GPU parity: NITI max-abs, requantiser, update and output error against the
oracle ("Integer On-Device Training: Overview", section 3), bit-exact,
including every shift value."""
import json
import os

import numpy as np
import pytest
import torch

import ionn_synth
import oracle
from integer_only_nn_amd import ops
from gpu_helpers import dev, host, say, to_dev, u32

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gpu_absmax(G):
    am = torch.zeros(1, dtype=torch.int32, device=dev())
    ops.ionn_absmax_i32(G, am)
    return am


def _gpu_update(G, W, tb, mu):
    Gd, Wd = to_dev(G), to_dev(W)
    am = _gpu_absmax(Gd)
    sh = torch.zeros(2, dtype=torch.int32, device=dev())
    gq = torch.empty_like(Gd)
    ops.niti_quantize_update(Gd, am, tb, mu, Wd, shifts_out=sh, gq_out=gq)
    return host(Wd), host(gq), host(sh).tolist(), u32(am)


def _gpu_requant(acc, tb, relu=False):
    a = to_dev(acc)
    am = _gpu_absmax(a)
    out = torch.empty(a.shape, dtype=torch.int8, device=dev())
    sh = torch.zeros(1, dtype=torch.int32, device=dev())
    ops.niti_quantize(a, am, tb, relu, out, shift_out=sh)
    return host(out), int(host(sh)[0]), u32(am)


def test_golden_cases_on_gpu():
    cases = json.load(open(os.path.join(GOLD, "niti_cases.json")))
    for c in cases["update"]:
        say("update", c["name"])
        W, gq, (s, ws), m = _gpu_update(np.array(c["G"], np.int32), np.array(c["W"], np.int8),
                                        c["target_bits"], c["mu_weight"])
        assert (m, s, ws) == (c["max"], c["shift"], c["weight_shift"])
        assert gq.tolist() == c["Gq"] and W.tolist() == c["W_new"]
    for c in cases["requant"]:
        say("requant", c["name"])
        out, s, _ = _gpu_requant(np.array(c["acc"], np.int32), c["target_bits"], c.get("relu", False))
        assert s == c["shift"] and out.tolist() == c["out"]


SIZES = [0, 1, 3, 15, 16, 17, 255, 4096, 4097, 65536 + 5, (1 << 20) + 3]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("scale", [100, 1 << 20, 1 << 31])
def test_requant_and_update_random(n, scale):
    say("n", n, "scale", scale)
    acc = ionn_synth.uniform_int(n + scale % 97, 11, (n,), -scale, scale - 1, dtype=np.int64).astype(np.int32)
    W = ionn_synth.uniform_int(n, 12, (n,), -128, 127)
    for tb, relu in ((7, False), (7, True), (8, False)):
        out, s, m = _gpu_requant(acc, tb, relu)
        want, ws = oracle.niti_requant(acc, tb, relu)
        assert m == oracle.absmax(acc) and s == ws
        np.testing.assert_array_equal(out, want)
    Wg, gq, (s, ws), _ = _gpu_update(acc, W, 8, 2)
    Wo, gqo, so, wso = oracle.niti_update(acc, W, 8, 2)
    assert (s, ws) == (so, wso)
    np.testing.assert_array_equal(gq, gqo)
    np.testing.assert_array_equal(Wg, Wo)


def test_unaligned_views_take_the_scalar_path():
    n = 1000
    acc = ionn_synth.uniform_int(3, 13, (n + 1,), -70000, 70000, dtype=np.int32)
    W = ionn_synth.uniform_int(3, 14, (n + 1,), -128, 127)
    a = to_dev(acc)[1:]
    w = to_dev(W)[1:]
    assert a.data_ptr() % 16 != 0
    am = _gpu_absmax(a)
    out = torch.empty(n + 1, dtype=torch.int8, device=dev())[1:]
    ops.niti_quantize(a, am, 7, False, out)
    np.testing.assert_array_equal(host(out), oracle.niti_requant(acc[1:].copy(), 7)[0])
    ops.niti_quantize_update(a, am, 8, 2, w)
    np.testing.assert_array_equal(host(w), oracle.niti_update(acc[1:].copy(), W[1:].copy(), 8, 2)[0])


def test_extremes_int32_min_and_max():
    acc = np.array([-2**31, 2**31 - 1, 5, -5, 0], np.int32)
    for tb in (1, 7, 8, 31):
        out, s, m = _gpu_requant(acc, tb)
        want, ws = oracle.niti_requant(acc, tb)
        assert m == 2**31 and s == ws
        np.testing.assert_array_equal(out, want)
    for mu in (0, 2, 31):
        Wg, gq, (s, ws), _ = _gpu_update(acc, np.array([127, -128, 0, 1, -1], np.int8), 8, mu)
        Wo, gqo, so, wso = oracle.niti_update(acc, np.array([127, -128, 0, 1, -1], np.int8), 8, mu)
        assert (s, ws) == (so, wso)
        np.testing.assert_array_equal(gq, gqo)
        np.testing.assert_array_equal(Wg, Wo)


def test_update_at_large_linear_size():
    """16.8M weights (the large-linear workload), G spanning ~2^20."""
    n = 4096 * 4096
    say("generating", n)
    G = ionn_synth.uniform_int(0, 15, (n,), -(1 << 20), (1 << 20) - 1, dtype=np.int32)
    W = ionn_synth.large_linear(T=1, IN=4096, OUT=4096)["W"].reshape(-1)
    Wg, gq, (s, ws), m = _gpu_update(G, W, 8, 2)
    Wo, gqo, so, wso = oracle.niti_update(G, W, 8, 2)
    assert (s, ws, m) == (so, wso, oracle.absmax(G))
    np.testing.assert_array_equal(gq, gqo)
    np.testing.assert_array_equal(Wg, Wo)


def test_output_error():
    d = ionn_synth.mlp(B=37, sizes=(8, 10))
    out = ionn_synth.uniform_int(1, 16, (37, 10), -128, 127)
    lab = d["labels"]
    e = torch.empty(37, 10, dtype=torch.int32, device=dev())
    am = torch.zeros(1, dtype=torch.int32, device=dev())
    ops.int_output_error(to_dev(out), to_dev(lab), 127, e, absmax_e=am)
    want = oracle.output_error(out, lab, 127)
    np.testing.assert_array_equal(host(e), want)
    assert u32(am) == oracle.absmax(want)
