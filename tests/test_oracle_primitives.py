"""Pins for the oracle's primitives and the NITI quantiser / update.

Each check compares the oracle with something other than itself: hand-derived
values (tests/golden/niti_cases.json, derived from the NITI steps of the TI
"Integer On-Device Training: Overview" page, section 3), Python's exact big
integers, or invariants that the NITI definition implies.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rhu_py(x, s):
    # Python's >> on ints is floor division by 2^s, exact for any size.
    return x if s == 0 else (x + (1 << (s - 1))) >> s


# ---- rhu / floor shift ---------------------------------------------------

def test_rhu_exhaustive_int16_all_shifts():
    x = np.arange(-32768, 32768, dtype=np.int32)
    x64 = x.astype(np.int64)
    for s in range(32):
        want = x64 if s == 0 else (x64 + (1 << (s - 1))) >> s   # numpy >> on int64 floors
        got = oracle.rhu_array(x, s)
        np.testing.assert_array_equal(got, want.astype(np.int32), err_msg=f"s={s}")


def test_rhu_random_int32_and_edges():
    rng = np.random.default_rng(1)
    x = rng.integers(-2**31, 2**31, size=1_000_000, dtype=np.int64).astype(np.int32)
    edges = np.array([-2**31, -2**31 + 1, -1, 0, 1, 2**31 - 2, 2**31 - 1], np.int32)
    x = np.concatenate([x, edges])
    for s in (1, 2, 7, 13, 24, 25, 31):
        want = ((x.astype(np.int64) + (1 << (s - 1))) >> s).astype(np.int32)
        np.testing.assert_array_equal(oracle.rhu_array(x, s), want, err_msg=f"s={s}")
    for v in edges.tolist():
        for s in range(32):
            assert oracle.rhu(v, s) == _rhu_py(v, s)


def test_rhu_ties_go_toward_plus_infinity():
    # "round-half-up": -0.5 -> 0, -1.5 -> -1, 0.5 -> 1, 1.5 -> 2
    assert [oracle.rhu(v, 1) for v in (-1, -3, 1, 3)] == [0, -1, 1, 2]


def test_floor_shift_matches_python():
    for v in (-2**31, -7, -1, 0, 1, 7, 2**31 - 1):
        for s in range(32):
            assert oracle.floor_shift(v, s) == v >> s


# ---- bitlen / shift ------------------------------------------------------

def test_bitlen_matches_int_bit_length():
    vals = list(range(0, 4097)) + [2**k + d for k in range(1, 32) for d in (-1, 0, 1)]
    vals += np.random.default_rng(2).integers(0, 2**32, 10000, dtype=np.uint64).tolist()
    for m in vals:
        m = int(m) & 0xFFFFFFFF
        assert oracle.bitlen(m) == m.bit_length()
        # bits_needed = ceil(log2(m + 1)) exactly: least b with m < 2^b
        assert (m < (1 << oracle.bitlen(m))) and (m == 0 or m >= (1 << (oracle.bitlen(m) - 1)))


def test_abs_of_int32_min_is_2_pow_31():
    assert oracle.abs_u32(-2**31) == 2**31
    assert oracle.absmax(np.array([-2**31, 5], np.int32)) == 2**31
    assert oracle.absmax(np.zeros(0, np.int32)) == 0


@pytest.mark.parametrize("tb", [1, 7, 8, 15, 31])
def test_shift_zero_iff_max_fits(tb):
    # I1: s = 0  <=>  m <= 2^tb - 1
    for m in [0, 1, (1 << tb) - 1, 1 << tb, (1 << tb) + 1, 2**32 - 1]:
        m &= 0xFFFFFFFF
        s = oracle.niti_shift(m, tb)
        assert (s == 0) == (m <= (1 << tb) - 1)
        assert s == max(0, m.bit_length() - tb)


def test_sat():
    assert [oracle.sat8(v) for v in (-1000, -129, -128, 0, 127, 128, 999)] == \
        [-128, -128, -128, 0, 127, 127, 127]
    assert [oracle.sat16(v) for v in (-40000, -32768, 32767, 32768)] == [-32768, -32768, 32767, 32767]


def test_ceil_log2():
    for n in range(0, 2000):
        want = 0 if n <= 1 else (n - 1).bit_length()
        assert oracle.ceil_log2(n) == want


# ---- NITI golden cases ---------------------------------------------------

@pytest.mark.parametrize("case", _load("niti_cases.json")["update"], ids=lambda c: c["name"])
def test_niti_update_golden(case):
    G = np.array(case["G"], np.int32)
    W = np.array(case["W"], np.int8)
    assert oracle.absmax(G) == case["max"]
    assert oracle.bitlen(case["max"]) == case["bits_needed"]
    Wn, Gq, s, ws = oracle.niti_update(G, W, case["target_bits"], case["mu_weight"])
    assert (s, ws) == (case["shift"], case["weight_shift"])
    assert Gq.tolist() == case["Gq"]
    assert oracle.rhu_array(Gq, ws).tolist() == case["delta"]
    assert Wn.tolist() == case["W_new"]
    assert W.tolist() == case["W"]  # input untouched


@pytest.mark.parametrize("case", _load("niti_cases.json")["requant"], ids=lambda c: c["name"])
def test_niti_requant_golden(case):
    acc = np.array(case["acc"], np.int32)
    out, s = oracle.niti_requant(acc, case["target_bits"], relu=case.get("relu", False))
    assert s == case["shift"]
    assert oracle.rhu_array(acc, s).tolist() == case["pre_clamp"]
    assert out.tolist() == case["out"]


def test_two_roundings_differ_from_one():
    # NITI-B's last element: the step-3 and step-4 roundings are sequential.
    assert oracle.rhu(oracle.rhu(4208, 5), 3) == 17
    assert oracle.rhu(4208, 8) == 16


# ---- invariants (random) -------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_requant_invariants(seed):
    rng = np.random.default_rng(seed)
    scale = [1, 100, 2**12, 2**20, 2**30, 2**31][seed]
    acc = rng.integers(-scale, scale, size=5000, dtype=np.int64).astype(np.int32)
    for tb in (7, 8):
        out, s = oracle.niti_requant(acc, tb)
        m = oracle.absmax(acc)
        pre = oracle.rhu_array(acc, s)
        assert out.min() >= -128 and out.max() <= 127                  # I3
        if s == 0:
            assert m <= (1 << tb) - 1                                   # I1
            np.testing.assert_array_equal(pre, acc)
        else:
            mx = int(np.abs(pre.astype(np.int64)).max())
            assert (1 << (tb - 1)) <= mx <= (1 << tb)                   # I2
        if tb == 7:
            assert np.abs(pre.astype(np.int64)).max() <= 128            # deltas within 7 bits
        np.testing.assert_array_equal(out, np.clip(pre, -128, 127))
        outr, sr = oracle.niti_requant(acc, tb, relu=True)
        assert sr == s
        np.testing.assert_array_equal(outr, np.maximum(out, 0))


@pytest.mark.parametrize("seed", range(4))
def test_update_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    G = rng.integers(-(1 << (8 + 3 * seed)), 1 << (8 + 3 * seed), 4000).astype(np.int32)
    W = rng.integers(-128, 128, 4000).astype(np.int8)
    Wn, Gq, s, ws = oracle.niti_update(G, W, 8, 2)
    assert 0 <= ws <= s and (s > 2 or ws == 0)                          # I5
    d = oracle.rhu_array(Gq, ws)
    np.testing.assert_array_equal(Wn, np.clip(W.astype(np.int64) - d, -128, 127))
    if ws >= 8 + 2:
        assert not d.any() and (Wn == W).all()                           # I5: d == 0 once ws >= tb+2
    Wz, _, sz, wsz = oracle.niti_update(np.zeros_like(G), W, 8, 2)
    assert (sz, wsz) == (0, 0) and (Wz == W).all()                       # I4
