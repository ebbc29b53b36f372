"""Pins of the oracle's adaptive-precision steps ("Adaptive Precision Training
for Resource Constrained Devices": the k-bit grid and its resolution eps,
Equations 1-3; Gavg, Equation 4; Algorithms 1 and 2), checked against
exact rational arithmetic, exhaustive enumeration, hand-worked cases and
the closed-form behaviour the page describes for its Figure 1."""
import math
from fractions import Fraction

import numpy as np
import pytest

import ionn_synth
import oracle
from oracle import apt


def _sat(v, k):
    return max(-(1 << (k - 1)), min((1 << (k - 1)) - 1, v))


def _exact_update(m, g, k, e_w, e_g, lam):
    """W - lr * g in exact rationals: the real value, divided by eps, rounded
    to the nearest grid point with ties toward -inf (so the change rounds
    half-up), saturated to k bits."""
    w = Fraction(m) * Fraction(2) ** e_w
    x = (w - Fraction(2) ** (-lam) * Fraction(g) * Fraction(2) ** e_g) / Fraction(2) ** e_w
    return _sat(math.ceil(x - Fraction(1, 2)), k)


def test_hand_worked_update_and_gavg():
    # k = 4 (grid -8..7), eps = 2^-4, g = G * 2^-8, lr = 1: each change is
    # G / 16 weight steps: 1, -1, 0.5 -> 1 (half rounds up), -2.5 -> -2.
    W = np.array([5, -3, 0, 7], np.int16)
    G = np.array([16, -16, 8, -40], np.int16)
    Wn, under = oracle.apt_update(W, 4, -4, G, -8, 0)
    assert Wn.tolist() == [4, -2, -1, 7]   # 7 - (-2) = 9 saturates to 7
    assert under == 0
    # Gavg = mean(16, 16, 8, 40) * 2^-8 / 2^-4 = 20 / 16
    assert oracle.gavg(G, -8, -4) == 1.25
    # the same gradient with lr = 2^-3: changes 1/8, -1/8, 1/16, -5/16 all round to 0
    Wn, under = oracle.apt_update(W, 4, -4, G, -8, 3)
    assert Wn.tolist() == W.tolist() and under == 4


@pytest.mark.parametrize("seed", range(6))
def test_update_matches_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        k = int(rng.integers(2, 17))
        e_w = int(rng.integers(-30, 10))
        e_g = int(rng.integers(-40, 10))
        lam = int(rng.integers(0, 30))
        n = 64
        lim = 1 << (k - 1)
        W = rng.integers(-lim, lim, n).astype(np.int16)
        G = rng.integers(-32768, 32768, n).astype(np.int16)
        G[:4] = [0, -32768, 32767, 1]
        Wn, under = oracle.apt_update(W, k, e_w, G, e_g, lam)
        want = [_exact_update(int(m), int(g), k, e_w, e_g, lam) for m, g in zip(W, G)]
        assert Wn.tolist() == want, (k, e_w, e_g, lam)
        unchanged = sum(1 for m, g, v in zip(W, G, want) if g != 0 and
                        math.ceil(Fraction(int(m)) - Fraction(int(g)) * Fraction(2) ** (e_g - lam - e_w)
                                  - Fraction(1, 2)) == m)
        assert under == unchanged


def test_update_sigma_edges():
    # sigma = e_w + lr_shift - e_g at 0 (the change is g itself), at the
    # half-step ties, and far out on both sides
    W = np.array([0, 0, 0, 0, 100, -100], np.int16)
    G = np.array([3, -3, 1, -1, 32767, -32768], np.int16)
    Wn, _ = oracle.apt_update(W, 16, 0, G, 0, 0)
    assert Wn.tolist() == [-3, 3, -1, 1, 100 - 32767, -100 + 32768]
    # sigma = 1: +1/2 rounds up to a change of 1, -1/2 rounds up to 0
    Wn, under = oracle.apt_update(np.zeros(2, np.int16), 8, 1, np.array([1, -1], np.int16), 0, 0)
    assert Wn.tolist() == [-1, 0] and under == 1
    # sigma = 200: every change underflows
    Wn, under = oracle.apt_update(W, 16, 100, G, -100, 0)
    assert Wn.tolist() == W.tolist() and under == 6
    # sigma = -200: every nonzero change saturates on the side opposite to g
    Wn, _ = oracle.apt_update(W, 8, -100, G, 100, 0)
    assert Wn.tolist() == [-128, 127, -128, 127, -128, 127]
    Wn, _ = oracle.apt_update(W, 8, -100, np.zeros(6, np.int16), 100, 0)
    assert Wn.tolist() == [0, 0, 0, 0, 100, -100]


def test_update_saturates_to_k_bits():
    for k in range(2, 17):
        lim = 1 << (k - 1)
        W = np.array([lim - 1, -lim, 0], np.int16)
        G = np.array([-1, 1, 0], np.int16)
        Wn, _ = oracle.apt_update(W, k, 0, G, 0, 0)
        assert Wn.tolist() == [lim - 1, -lim, 0]
        # a weight outside the k-bit range is brought into it
        Wn, _ = oracle.apt_update(np.array([32767, -32768], np.int16), k, 0,
                                  np.zeros(2, np.int16), 0, 0)
        assert Wn.tolist() == [lim - 1, -lim]


def test_underflow_grows_as_precision_falls():
    # the same gradient against coarser and coarser grids (larger eps):
    # more of its changes are lost
    G = ionn_synth.apt_grad(7, 4096, 300.0)
    W = np.zeros(4096, np.int16)
    counts = [oracle.apt_update(W, 16, e_w, G, 0, 0)[1] for e_w in range(0, 14)]
    assert all(a <= b for a, b in zip(counts, counts[1:]))
    assert counts[0] == 0 and counts[-1] == int(np.count_nonzero(G))


def test_rescale_exhaustive():
    for k in range(2, 16):  # one bit more: same value, exact
        lim = 1 << (k - 1)
        m = np.arange(-lim, lim, dtype=np.int16)
        up = oracle.apt_rescale(m, k, +1)
        assert (up.astype(np.int64) == 2 * m.astype(np.int64)).all()  # 2m * 2^(e-1) == m * 2^e
        assert up.min() >= -(1 << k) and up.max() <= (1 << k) - 1
        back = oracle.apt_rescale(up, k + 1, -1)
        assert (back == m).all()
    for k in range(3, 17):  # one bit less: within one old step, even m exact
        lim = 1 << (k - 1)
        m = np.arange(-lim, lim, dtype=np.int64)
        dn = oracle.apt_rescale(m.astype(np.int16), k, -1).astype(np.int64)
        assert dn.min() >= -(lim >> 1) and dn.max() <= (lim >> 1) - 1
        err = 2 * dn - m
        assert np.abs(err).max() <= 1
        assert (err[m % 2 == 0] == 0).all()
        # odd values round half up except where that leaves the range
        odd = (m % 2 != 0) & (m != lim - 1)
        assert (2 * dn[odd] == m[odd] + 1).all()
        assert dn[m == lim - 1][0] == (lim >> 1) - 1
    z = np.array([1, -2, 3], np.int16)
    assert oracle.apt_rescale(z, 8, 0).tolist() == z.tolist()


def test_decide_truth_table():
    d = oracle.apt_decide
    inf = float("inf")
    assert d(0.5, 1, 6, 1.0, inf, 2, 16) == 1          # below T_min: one bit more
    assert d(3.0, 3, 6, 1.0, inf, 2, 16) == 0          # mean 1.0 is not below 1.0
    assert d(2.9, 3, 6, 1.0, inf, 2, 16) == 1          # mean 0.966..
    assert d(0.5, 1, 16, 1.0, inf, 2, 16) == 0         # already at k_max
    assert d(50.0, 1, 6, 1.0, 10.0, 2, 16) == -1       # above T_max: one bit less
    assert d(20.0, 2, 6, 1.0, 10.0, 2, 16) == 0        # mean 10.0 is not above 10.0
    assert d(50.0, 1, 2, 1.0, 10.0, 2, 16) == 0        # already at k_min
    assert d(1e300, 1, 6, 1.0, inf, 2, 16) == 0        # T_max = inf never lowers
    assert d(0.0, 0, 6, 1.0, inf, 2, 16) == 0          # no samples: no change
    assert d(5.0, 1, 6, 1.0, 10.0, 2, 16) == 0         # inside the band


def test_gavg_doubles_per_added_bit():
    G = ionn_synth.apt_grad(3, 1000, 50.0)
    base = oracle.gavg(G, -10, -5)
    for b in range(1, 8):
        assert oracle.gavg(G, -10, -5 - b) == base * 2 ** b


def _const_grads(Gs, egs):
    return lambda ep, st, l, state: (Gs[l], egs[l])


def test_workflow_closed_form_raises_and_lowers():
    """A layer whose gradient stays the same: each added bit doubles Gavg,
    so from Gavg_0 < T_min the precision rises by one bit per epoch until
    Gavg_0 * 2^r >= T_min (the behaviour the page describes for its layer A
    with T_max = inf); a layer above T_max falls by one bit per epoch until
    it is no longer above, or reaches k_min."""
    n = 512
    Gs = [ionn_synth.apt_grad(100 + l, n, s) for l, s in enumerate((20.0, 4000.0, 600.0))]
    egs = [-14, -6, -10]
    Ws, _ = ionn_synth.apt_weights([n] * 3, k0=6, seed=2)
    es = [-6, -6, -6]
    g0 = [oracle.gavg(G, eg, e) for G, eg, e in zip(Gs, egs, es)]
    t_min, t_max, k_min, k_max = 1.0, 64.0, 3, 16
    assert g0[0] < t_min and g0[1] > t_max and t_min <= g0[2] <= t_max
    r_up = 0
    while g0[0] * 2 ** r_up < t_min:
        r_up += 1
    r_dn = 0
    while g0[1] / 2 ** r_dn > t_max and 6 - r_dn > k_min:
        r_dn += 1
    state = apt.new_state(Ws, [6, 6, 6], es)
    epochs = max(r_up, r_dn) + 2
    hist = apt.run(state, _const_grads(Gs, egs), epochs, steps=4, eval_every=2, lr_shift=12,
                   t_min=t_min, t_max=t_max, k_min=k_min, k_max=k_max)
    for ep, h in enumerate(hist):
        assert h["counts"] == [2, 2, 2]
        assert h["k"][0] == 6 + min(ep + 1, r_up)
        assert h["k"][1] == 6 - min(ep + 1, r_dn)
        assert h["k"][2] == 6
        assert h["e_w"] == [es[0] - (h["k"][0] - 6), es[1] - (h["k"][1] - 6), es[2]]
    assert r_up >= 2 and r_dn >= 2


def test_workflow_weights_stay_in_k_bits():
    sizes = ionn_synth.RESNET20_SIZES[:4]
    Ws, es = ionn_synth.apt_weights(sizes, k0=6, seed=1)
    state = apt.new_state(Ws, [6] * 4, es)
    sig = [30.0, 300.0, 3000.0, 30000.0]

    def grads(ep, st, l, s):
        return ionn_synth.apt_grad((ep * 8 + st) * 4 + l, sizes[l], sig[l]), -16

    hist = apt.run(state, grads, epochs=4, steps=3, eval_every=1, lr_shift=2,
                   t_min=1.0, t_max=200.0, k_min=2, k_max=16)
    for s in state:
        lim = 1 << (s["k"] - 1)
        assert s["W"].min() >= -lim and s["W"].max() <= lim - 1
    assert any(d != 0 for h in hist for d in h["dk"])
