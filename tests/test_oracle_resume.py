"""Resuming training from saved weights ("Integer On-Device Training:
Overview", section 9: trained weights live in RAM and are not kept across a
power cycle, so a device that must resume stores and reloads its weight and
offset arrays).  Training 5 steps, writing the state to a file, reading it
back and training 5 more must give the bits of 10 straight steps: the step
is a function of the weights, offsets and the batch alone."""
import numpy as np

import ionn_synth
from oracle import steps as osteps


def _save_load(path, arrays):
    np.savez(path, *arrays)
    with np.load(path, allow_pickle=False) as z:
        return [z[f"arr_{i}"] for i in range(len(arrays))]


def test_mlp_resume_is_bit_identical(tmp_path):
    d = ionn_synth.mlp(B=37, sizes=(50, 33, 20, 10), seed=0)
    W10, _ = osteps.mlp_train(d["X"], d["labels"], d["Ws"], 10)
    W5, _ = osteps.mlp_train(d["X"], d["labels"], d["Ws"], 5)
    back = _save_load(tmp_path / "mlp.npz", W5)
    Wr, _ = osteps.mlp_train(d["X"], d["labels"], back, 5)
    for a, b, w0 in zip(Wr, W10, d["Ws"]):
        np.testing.assert_array_equal(a, b)
    assert any((a != w0).any() for a, w0 in zip(W10, d["Ws"]))   # the weights did move


def test_model_resume_is_bit_identical(tmp_path):
    a = ionn_synth.arc_fault(B=64)
    layers = osteps.arc_fault_layers(a)
    step = lambda ls: osteps.model_step(ls, a["X"], a["labels"], a["tmc"], a["tmw"])[0]
    full = layers
    for _ in range(10):
        full = step(full)
    half = layers
    for _ in range(5):
        half = step(half)
    saved = _save_load(tmp_path / "model.npz", [L["weight"] for L in half] + [L["offset"] for L in half])
    n = len(half)
    resumed = [dict(L, weight=saved[l], offset=saved[n + l]) for l, L in enumerate(layers)]
    for _ in range(5):
        resumed = step(resumed)
    for x, y in zip(resumed, full):
        np.testing.assert_array_equal(x["weight"], y["weight"])
        np.testing.assert_array_equal(x["offset"], y["offset"])
    assert any((x["offset"] != L["offset"]).any() for x, L in zip(full, layers))
