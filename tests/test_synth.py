"""The seeded input generators: determinism, published SplitMix64 output,
shapes and value ranges of the five workloads."""
import numpy as np

import ionn_synth


def test_splitmix64_reference_value():
    # SplitMix64 seeded with 0: the first output is 0xE220A8397B1DCDAF
    # (the published sequence of Steele, Lea and Flood's generator).
    assert int(ionn_synth.splitmix64(0, 0, 1)[0]) == 0xE220A8397B1DCDAF


def test_counter_property():
    a = ionn_synth.splitmix64(3, 7, 100)
    b = ionn_synth.splitmix64(3, 7, 60, start=40)
    np.testing.assert_array_equal(a[40:], b)
    assert not np.array_equal(a, ionn_synth.splitmix64(3, 8, 100))


def test_workload_shapes_and_ranges():
    d = ionn_synth.single_linear()
    assert d["X"].shape == (16, 64) and d["W"].shape == (32, 64) and d["dY"].shape == (16, 32)
    assert d["dY"].min() >= -64 and d["dY"].max() <= 63
    m = ionn_synth.mlp(B=64)
    assert [w.shape for w in m["Ws"]] == [(256, 784), (128, 256), (10, 128)]
    assert m["X"].min() >= 0 and m["labels"].max() <= 9 and m["labels"].dtype == np.int32
    c = ionn_synth.conv3x3(N=2)
    assert c["X"].shape == (2, 56, 56, 64) and c["W"].shape == (64, 3, 3, 64)
    f = ionn_synth.dfp16_gemm(M=64, K=32, N=16)
    assert f["X"].dtype == np.int16 and -20 <= f["eX"] <= -8


def test_normal_statistics():
    v = ionn_synth.normal_int(0, 2, (200000,), 20.0, -128, 127).astype(np.float64)
    assert abs(v.mean()) < 0.3 and abs(v.std() - 20.0) < 0.3
    v = ionn_synth.normal_int(0, 2, (200000,), 4000.0, -32768, 32767, dtype=np.int16)
    assert abs(v.astype(np.float64).std() - 4000.0) < 40


def test_deterministic():
    a = ionn_synth.large_linear(T=64, IN=32, OUT=16)
    b = ionn_synth.large_linear(T=64, IN=32, OUT=16)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
