"""GPU parity: the 784-256-128-10 int8 MLP trained for 10 NITI steps (batch
256) against the oracle; every forward, error, dgrad and update shift of every
step and the final weights must match bit for bit."""
import numpy as np
import pytest

import ionn_synth
from oracle import steps as osteps
from integer_only_nn_amd import steps
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,sizes,nsteps,moves", [(256, (784, 256, 128, 10), 10, False),
                                                  (37, (50, 33, 20, 10), 4, True),
                                                  (8, (64, 16, 10), 3, True)])
def test_mlp_training_matches_oracle(B, sizes, nsteps, moves):
    d = ionn_synth.mlp(B=B, sizes=sizes, seed=0)
    Wo, recs = osteps.mlp_train(d["X"], d["labels"], d["Ws"], nsteps)
    m = steps.MLP.make([to_dev(w) for w in d["Ws"]], B, with_gq=True)
    X, lab = to_dev(d["X"]), to_dev(d["labels"])
    for t in range(nsteps):
        m.step(X, lab)
        got = m.shift_record()
        want = {k: recs[t][k] for k in ("s_fwd", "s_err", "s_dgrad", "s_upd")}
        say("step", t, got)
        assert got == want, f"step {t}"
        # every layer's weight gradient and its quantised form, every step:
        # at full size the weights cannot move (each weight shift >= 9), so
        # the update is checked through G and Gq
        for l in range(len(sizes) - 1):
            np.testing.assert_array_equal(host(m.G[l]), recs[t]["G"][l], err_msg=f"step {t} G{l}")
            np.testing.assert_array_equal(host(m.Gq[l]), recs[t]["Gq"][l], err_msg=f"step {t} Gq{l}")
        if t == nsteps - 1:
            for l in range(len(sizes) - 1):
                np.testing.assert_array_equal(host(m.acts[l + 1]), recs[t]["acts"][l + 1])
            for l in range(len(sizes)):
                np.testing.assert_array_equal(host(m.deltas[l]), recs[t]["deltas"][l])
    for l, w in enumerate(Wo):
        np.testing.assert_array_equal(host(m.Ws[l]), w)
    # With the full-size MLP every weight shift is >= 9, so the NITI deltas
    # round to 0 and the weights stay put (the oracle agrees); the small
    # MLPs move their weights.
    moved = any((host(m.Ws[l]) != d["Ws"][l]).any() for l in range(len(Wo)))
    assert moved == moves
