"""Pins for the oracle's offset (bias) path: the static OSS requantisation,
the offset gradient and the NITI update of int32 offsets.

Each check compares the oracle with something other than itself:
hand-derived values (tests/golden/oss_cases.json, from the TI "Integer
On-Device Training: Overview" page, sections 7 and 8 for the OSS chain and the
offsets, section 3 for the update), the chain evaluated step by step in
float64 where that is exact, numpy's exact int64 sums, and the already pinned
int8 NITI update on inputs where the two must agree.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "oss_cases.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _gold()["oss"], ids=lambda c: c["name"])
def test_oss_golden(case):
    out = oracle.oss_requant(np.array(case["acc"], np.int32), np.array(case["offset"], np.int32),
                             np.array(case["mult"], np.int32), np.array(case["k"], np.int8),
                             relu=case["relu"])
    np.testing.assert_array_equal(out, np.array(case["out"], np.int8))


def _onnx_chain_f64(acc, offset, mult, k, relu):
    """The page's chain as float64 nodes: Add, Mul(mult), Mul(2^-k), Floor,
    Clip.  Exact when no int32 wrap happens and |t * mult| < 2^53."""
    t = acc.astype(np.float64) + offset.astype(np.float64)[None, :]
    y = t * mult.astype(np.float64)[None, :]
    y = y * np.exp2(-k.astype(np.float64))[None, :]
    y = np.floor(y)
    return np.clip(y, 0.0 if relu else -128.0, 127.0).astype(np.int8)


@pytest.mark.parametrize("relu", [False, True])
def test_oss_matches_float64_chain(relu):
    rng = np.random.default_rng(7)
    M, C = 37, 29
    acc = rng.integers(-2**24, 2**24, (M, C), dtype=np.int64).astype(np.int32)
    offset = rng.integers(-2**20, 2**20, C, dtype=np.int64).astype(np.int32)
    mult = rng.integers(-2**20, 2**20, C, dtype=np.int64).astype(np.int32)
    k = rng.integers(0, 40, C).astype(np.int8)
    got = oracle.oss_requant(acc, offset, mult, k, relu=relu)
    np.testing.assert_array_equal(got, _onnx_chain_f64(acc, offset, mult, k, relu))
    # the clip range is reached on both sides, and values in between occur
    assert (got == 127).any() and (got == (0 if relu else -128)).any()
    assert ((got > (0 if relu else -128)) & (got < 127)).any()


def test_oss_identity_and_shift_only():
    rng = np.random.default_rng(8)
    acc = rng.integers(-300, 300, (11, 5), dtype=np.int64).astype(np.int32)
    z = np.zeros(5, np.int32)
    # mult 1, k 0, no offset: saturation to int8 only
    out = oracle.oss_requant(acc, z, np.ones(5, np.int32), np.zeros(5, np.int8))
    np.testing.assert_array_equal(out, np.clip(acc, -128, 127).astype(np.int8))
    # mult 2^j, k j: the offset add and the clip only
    off = np.array([3, -3, 0, 100, -100], np.int32)
    out = oracle.oss_requant(acc, off, np.full(5, 8, np.int32), np.full(5, 3, np.int8))
    np.testing.assert_array_equal(out, np.clip(acc.astype(np.int64) + off, -128, 127).astype(np.int8))


@pytest.mark.parametrize("case", _gold()["bias_grad"], ids=lambda c: c["name"])
def test_bias_grad_golden(case):
    np.testing.assert_array_equal(oracle.bias_grad(np.array(case["d"], np.int8)),
                                  np.array(case["gb"], np.int32))


def test_bias_grad_exact_sums():
    rng = np.random.default_rng(9)
    d = rng.integers(-128, 128, (513, 70), dtype=np.int64).astype(np.int8)
    gb = oracle.bias_grad(d)
    want = d.astype(np.int64).sum(axis=0)
    np.testing.assert_array_equal(gb.astype(np.int64), want)
    assert int(gb.astype(np.int64).sum()) == int(d.astype(np.int64).sum())
    # a single row is its own gradient; zero rows give zeros
    np.testing.assert_array_equal(oracle.bias_grad(d[:1]), d[0].astype(np.int32))
    np.testing.assert_array_equal(oracle.bias_grad(np.zeros((0, 70), np.int8)), np.zeros(70, np.int32))


@pytest.mark.parametrize("case", _gold()["update_i32"], ids=lambda c: c["name"])
def test_update_i32_golden(case):
    Pn, gq, s, ws = oracle.niti_update_i32(np.array(case["G"], np.int32), np.array(case["P"], np.int32),
                                           case["target_bits"], case["mu"])
    assert (s, ws) == (case["shift"], case["weight_shift"])
    np.testing.assert_array_equal(gq, np.array(case["Gq"], np.int32))
    np.testing.assert_array_equal(Pn, np.array(case["P_new"], np.int32))


def test_update_i32_small_gradient_is_plain_subtraction():
    # max |G| < 2^tb: shift 0, weight shift 0, d = G, so P - G exactly
    rng = np.random.default_rng(10)
    G = rng.integers(-255, 256, 1000, dtype=np.int64).astype(np.int32)
    P = rng.integers(-2**30, 2**30, 1000, dtype=np.int64).astype(np.int32)
    Pn, gq, s, ws = oracle.niti_update_i32(G, P, 8, 2)
    assert (s, ws) == (0, 0)
    np.testing.assert_array_equal(gq, G)
    np.testing.assert_array_equal(Pn.astype(np.int64), P.astype(np.int64) - G.astype(np.int64))


def test_update_i32_agrees_with_int8_update_inside_int8_range():
    # P in the int8 range and steps small enough that neither clamp acts:
    # the int32 update must equal the int8 NITI update
    rng = np.random.default_rng(11)
    G = rng.integers(-2**20, 2**20, 4096, dtype=np.int64).astype(np.int32)
    W = rng.integers(-60, 61, 4096, dtype=np.int64).astype(np.int8)
    Wn, gq8, s8, ws8 = oracle.niti_update(G, W, 8, 2)
    Pn, gq, s, ws = oracle.niti_update_i32(G, W.astype(np.int32), 8, 2)
    assert (s, ws) == (s8, ws8)
    np.testing.assert_array_equal(gq, gq8)
    assert np.all(np.abs(Pn.astype(np.int64)) <= 127), "steps chosen to stay inside int8"
    np.testing.assert_array_equal(Pn, Wn.astype(np.int32))
