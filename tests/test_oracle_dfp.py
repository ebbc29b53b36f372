"""Pins for the oracle's DFP-16 contraction, down-conversion and Gavg.

Sources: "Mixed Precision Training of Convolutional Neural Networks using
Integer Operations" (summary), sections 3, 3.1 and 4; "Adaptive Precision
Training for Resource Constrained Devices" (Gavg, Equation 4).  References
used: hand-derived cases (tests/golden/dfp_cases.json); exact int64 sums from
numpy (the chunked result must stay within the rounding bound of the exact
sum); the single-chunk case, where the contraction is the plain matrix product;
and invariants of the down-conversion.
"""
import json
import os

import numpy as np
import pytest

import ionn_synth
import oracle
from oracle import steps

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load():
    with open(os.path.join(GOLD, "dfp_cases.json")) as f:
        return json.load(f)


def test_dfp1_dfp2_golden():
    c = _load()
    K = c["DFP-1"]["K"]
    X = np.zeros((2, K), np.int16)
    X[0, :] = 1000
    X[1, 0] = 7
    W = np.zeros((1, K), np.int16)
    W[0, :64] = 3
    W[0, 64:] = -1
    assert oracle.dfp_chunk_shift(K, 64) == c["DFP-1"]["r"]
    Y, eY, acc = oracle.dfp16_fwd(X, -10, W, -12, 64)
    assert acc[:, 0].tolist() == [c["DFP-1"]["acc"], c["DFP-2"]["acc"]]
    assert Y[:, 0].tolist() == [c["DFP-1"]["out"], c["DFP-2"]["out"]]
    assert eY == -10 - 12 + c["DFP-1"]["exp_offset"]
    # DFP-1 is exact: 32000 * 2^2 = 128000 = 1000*(64*3 - 64*1)
    assert int(Y[0, 0]) * 4 == 1000 * (64 * 3 - 64)
    assert abs(int(Y[1, 0]) * 4 - c["DFP-2"]["exact"]) <= c["DFP-2"]["error_bound"]


def test_gavg_golden_and_exact():
    g = _load()["GAVG-1"]
    assert oracle.gavg(np.array(g["g"], np.int16), g["e_g"], g["e_w"]) == g["gavg"]
    # exact in double: sum < 2^53 and the scaling is a power of two
    rng = np.random.default_rng(0)
    G = rng.integers(-32768, 32768, 1 << 18).astype(np.int16)
    s = int(np.abs(G.astype(np.int64)).sum())
    assert oracle.gavg(G, -17, -9) == (s / (1 << 18)) * 2.0 ** -8
    assert oracle.gavg(np.array([-32768], np.int16), 0, 0) == 32768.0


def test_int32_chain_claim():
    c = _load()["int32_chain"]
    v = c["max_int16_magnitude"]
    assert 2 * v * v == c["two_products"] < c["int32_max"] < 3 * v * v == c["three_products"]
    assert 2 * 32768 * 32768 > c["int32_max"]


def test_chunk_shift_values():
    # r = ceil(log2(number of chunks)); the three roles of the DFP workload
    assert [oracle.dfp_chunk_shift(L, 64) for L in (1, 64, 65, 128, 256, 1024, 25088)] == \
        [0, 0, 1, 1, 2, 4, 9]


@pytest.mark.parametrize("M,K,N", [(3, 64, 5), (17, 40, 9), (1, 1, 1)])
def test_single_chunk_is_plain_product(M, K, N):
    rng = np.random.default_rng(M + K + N)
    X = rng.integers(-32768, 32768, (M, K)).astype(np.int16) // 4   # no wrap within 64 terms
    W = rng.integers(-32768, 32768, (N, K)).astype(np.int16) // 4
    acc = oracle.dfp_contract(X, K, 1, W, 1, K, M, N, K, 64)
    np.testing.assert_array_equal(acc, X.astype(np.int64) @ W.astype(np.int64).T)


def _bound(L, rs, chunk=64):
    nc = -(-L // chunk)
    r = oracle.dfp_chunk_shift(L, chunk)
    return (nc * (1 << (r - 1)) if r > 0 else 0) + ((1 << (r + rs - 1)) if r + rs > 0 else 0)


@pytest.mark.parametrize("M,K,N", [(40, 256, 24), (30, 200, 70), (9, 1000, 5)])
def test_roles_within_rounding_bound_of_exact(M, K, N):
    """I11: |out * 2^(r+Rs) - exact| <= n_c 2^(r-1) + 2^(r+Rs-1) in units of
    2^(Ea+Eb), for all three roles (exact sums from int64 numpy)."""
    d = ionn_synth.dfp16_gemm(M=M, K=K, N=N, seed=1)
    X, W, dY = d["X"], d["W"], d["dY"]
    X64, W64, dY64 = (a.astype(np.int64) for a in (X, W, dY))
    cases = [
        (oracle.dfp16_fwd(X, d["eX"], W, d["eW"]), X64 @ W64.T, K, d["eX"] + d["eW"]),
        (oracle.dfp16_dgrad(dY, d["edY"], W, d["eW"]), dY64 @ W64, N, d["edY"] + d["eW"]),
        (oracle.dfp16_wgrad(dY, d["edY"], X, d["eX"]), dY64.T @ X64, M, d["edY"] + d["eX"]),
    ]
    for (out, e, acc), exact, L, e_in in cases:
        r = oracle.dfp_chunk_shift(L, 64)
        rs = e - e_in - r
        assert rs >= 0
        assert out.shape == exact.shape
        err = np.abs(out.astype(np.int64) * (1 << (r + rs)) - exact)
        assert err.max() <= _bound(L, rs), (L, r, rs, err.max())
        # I10: mantissas in range; Rs > 0 means the largest lands in [2^14, 2^15]
        m = np.abs(out.astype(np.int64)).max()
        if rs > 0:
            assert (1 << 14) <= m <= (1 << 15)
        # down-conversion of the returned accumulator reproduces the output
        out2, rs2 = oracle.dfp_downconvert(acc)
        np.testing.assert_array_equal(out2, out)
        assert rs2 == rs


def test_dfp_exponent_range_checked():
    X = np.full((1, 64), 30000, np.int16)
    W = np.full((1, 64), 30000, np.int16)
    with pytest.raises(OverflowError):
        oracle.dfp16_fwd(X, 120, W, 10)


def test_dfp16_step_small():
    d = ionn_synth.dfp16_gemm(M=128, K=64, N=96, seed=2)
    r = steps.dfp16_step(d["X"], d["eX"], d["W"], d["eW"], d["dY"], d["edY"])
    assert r["Y"].shape == (128, 96) and r["dX"].shape == (128, 64) and r["G"].shape == (96, 64)
    g = np.abs(r["G"].astype(np.int64)).mean() * 2.0 ** (r["eG"] - d["eW"])
    assert r["gavg"] == g
