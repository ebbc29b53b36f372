"""GPU parity: per-channel offsets (bias) and the static OSS requantisation
("Integer On-Device Training: Overview", sections 7 and 8; the update by the
NITI steps of section 3) against the oracle, bit-exact."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from integer_only_nn_amd import ops
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "oss_cases.json")) as f:
        return json.load(f)


def _gpu_oss(acc, off, mult, k, relu, misalign=False):
    M, C = acc.shape
    if misalign:  # same values one element into a larger buffer: the unaligned path
        buf = torch.empty(M * C + 1, dtype=torch.int32, device=dev())
        buf[1:] = to_dev(acc).reshape(-1)
        a = buf[1:].view(M, C)
    else:
        a = to_dev(acc)
    out = torch.empty((M, C), dtype=torch.int8, device=dev())
    ops.ionn_oss_requant(a, to_dev(off), to_dev(mult), to_dev(k), out, relu=relu)
    return host(out)


def _gpu_bias_grad(d, misalign=False):
    M, C = d.shape
    if misalign:
        buf = torch.empty(M * C + 3, dtype=torch.int8, device=dev())
        buf[3:] = to_dev(d).reshape(-1)
        dd = buf[3:].view(M, C)
    else:
        dd = to_dev(d)
    gb = torch.full((C,), 12345, dtype=torch.int32, device=dev())  # overwritten
    ws = torch.empty(max(ops.ionn_bias_grad_workspace_bytes(M, C), 4), dtype=torch.uint8, device=dev())
    ops.ionn_bias_grad(dd, gb, ws)
    return host(gb)


def _gpu_update_i32(G, P, tb, mu):
    Gd, Pd = to_dev(G), to_dev(P)
    am = torch.zeros(1, dtype=torch.int32, device=dev())
    ops.ionn_absmax_i32(Gd, am)
    sh = torch.zeros(2, dtype=torch.int32, device=dev())
    gq = torch.empty_like(Gd)
    ops.niti_quantize_update_i32(Gd, am, tb, mu, Pd, shifts_out=sh, gq_out=gq)
    return host(Pd), host(gq), host(sh).tolist()


def test_golden_cases_on_gpu():
    g = _gold()
    for c in g["oss"]:
        say("oss", c["name"])
        out = _gpu_oss(np.array(c["acc"], np.int32), np.array(c["offset"], np.int32),
                       np.array(c["mult"], np.int32), np.array(c["k"], np.int8), c["relu"])
        assert out.tolist() == c["out"]
    for c in g["bias_grad"]:
        say("bias_grad", c["name"])
        assert _gpu_bias_grad(np.array(c["d"], np.int8)).tolist() == c["gb"]
    for c in g["update_i32"]:
        say("update_i32", c["name"])
        P, gq, (s, ws) = _gpu_update_i32(np.array(c["G"], np.int32), np.array(c["P"], np.int32),
                                         c["target_bits"], c["mu"])
        assert (s, ws) == (c["shift"], c["weight_shift"])
        assert gq.tolist() == c["Gq"] and P.tolist() == c["P_new"]


def _oss_inputs(M, C, seed, full_range):
    rng = np.random.default_rng(seed)
    acc = rng.integers(-2**31, 2**31, (M, C), dtype=np.int64).astype(np.int32)
    if full_range:
        off = rng.integers(-2**31, 2**31, C, dtype=np.int64).astype(np.int32)
        mult = rng.integers(-2**31, 2**31, C, dtype=np.int64).astype(np.int32)
        k = rng.integers(0, 63, C).astype(np.int8)
    else:  # a layer-like mix: a middle band of outputs plus both clip ends
        acc = (acc >> 12).astype(np.int32)
        off = rng.integers(-2**16, 2**16, C, dtype=np.int64).astype(np.int32)
        mult = rng.integers(1, 2**10, C, dtype=np.int64).astype(np.int32)
        k = rng.integers(14, 26, C).astype(np.int8)
    return acc, off, mult, k


OSS_SHAPES = [(1, 1), (3, 5), (257, 19), (1000, 12), (33, 4096), (8192, 4096)]


@pytest.mark.parametrize("M,C", OSS_SHAPES)
@pytest.mark.parametrize("relu", [False, True])
def test_oss_parity(M, C, relu):
    for full in (False, True):
        say("oss", M, C, relu, full)
        acc, off, mult, k = _oss_inputs(M, C, seed=M * 7 + C + int(relu), full_range=full)
        want = oracle.oss_requant(acc, off, mult, k, relu=relu)
        got = _gpu_oss(acc, off, mult, k, relu)
        np.testing.assert_array_equal(got, want)
        if not full and M * C >= 4096:
            lo = 0 if relu else -128
            assert (want == 127).any() and (want == lo).any() and ((want > lo) & (want < 127)).any()


def test_oss_unaligned_and_edges():
    acc, off, mult, k = _oss_inputs(129, 64, seed=5, full_range=True)
    k[:4] = [0, 62, 1, 61]
    mult[:2] = [-2**31, 2**31 - 1]
    acc[0, :2] = [2**31 - 1, -2**31]
    off[:2] = [1, -1]
    for relu in (False, True):
        want = oracle.oss_requant(acc, off, mult, k, relu=relu)
        np.testing.assert_array_equal(_gpu_oss(acc, off, mult, k, relu, misalign=True), want)
        np.testing.assert_array_equal(_gpu_oss(acc, off, mult, k, relu), want)
    # empty tensors are a no-op
    e = torch.empty((0, 8), dtype=torch.int32, device=dev())
    ops.ionn_oss_requant(e, to_dev(off[:8]), to_dev(mult[:8]), to_dev(k[:8]),
                         torch.empty((0, 8), dtype=torch.int8, device=dev()))


BG_SHAPES = [(0, 5), (1, 1), (7, 33), (129, 64), (1000, 4096 + 16), (8192, 4096),
             # narrow rows (C < 64, not a multiple of 16): the flat-array path,
             # with n mod 4 tail bytes, odd C and C sharing factors with 1024
             (65537, 3), (65536, 2), (20000, 17), (6000, 48), (3211264, 3)]


@pytest.mark.parametrize("M,C", BG_SHAPES)
def test_bias_grad_parity(M, C):
    say("bias_grad", M, C)
    rng = np.random.default_rng(M + 3 * C)
    d = rng.integers(-128, 128, (M, C), dtype=np.int64).astype(np.int8)
    want = oracle.bias_grad(d)
    np.testing.assert_array_equal(_gpu_bias_grad(d), want)
    if M * C:
        np.testing.assert_array_equal(_gpu_bias_grad(d, misalign=True), want)


def test_bias_grad_needs_workspace():
    from integer_only_nn_amd._lib import IonnError
    d = torch.zeros((100, 64), dtype=torch.int8, device=dev())
    gb = torch.empty(64, dtype=torch.int32, device=dev())
    with pytest.raises(IonnError):
        ops.ionn_bias_grad(d, gb, None)
    n = ops.ionn_bias_grad_workspace_bytes(100, 64)
    assert n >= 64 * 4
    with pytest.raises(IonnError):
        ops.ionn_bias_grad(d, gb, torch.empty(n - 4, dtype=torch.uint8, device=dev()))


def test_bias_grad_extreme_columns():
    # every value -128 or 127 in whole columns: the largest sums of the shape
    M, C = 4099, 48
    d = np.full((M, C), 127, np.int8)
    d[:, 1::2] = -128
    np.testing.assert_array_equal(_gpu_bias_grad(d), oracle.bias_grad(d))


@pytest.mark.parametrize("n", [0, 1, 17, 4096, 65536 + 3])
@pytest.mark.parametrize("tb,mu", [(8, 2), (4, 1), (16, 0)])
def test_update_i32_parity(n, tb, mu):
    say("update_i32", n, tb, mu)
    rng = np.random.default_rng(n + tb)
    G = rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    P = rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    if n >= 4:
        P[:2] = [-2**31, 2**31 - 1]  # at the clamps
        G[:2] = [2**30, -2**30]
    Pn, gq, s, ws = oracle.niti_update_i32(G, P, tb, mu)
    gP, ggq, (gs, gws) = _gpu_update_i32(G, P, tb, mu)
    assert (gs, gws) == (s, ws)
    np.testing.assert_array_equal(ggq, gq)
    np.testing.assert_array_equal(gP, Pn)


def test_offset_backward_chain():
    """Offset gradient -> its max -> the int32 update, as one step on the
    device, against the same chain in the oracle (8192 x 4096 error rows)."""
    rng = np.random.default_rng(21)
    M, C = 8192, 4096
    d = rng.integers(-64, 64, (M, C), dtype=np.int64).astype(np.int8)
    P = rng.integers(-2**20, 2**20, C, dtype=np.int64).astype(np.int32)
    gb = oracle.bias_grad(d)
    Pn, gq, s, ws = oracle.niti_update_i32(gb, P, 8, 2)
    dd, Pd = to_dev(d), to_dev(P)
    gbd = torch.empty(C, dtype=torch.int32, device=dev())
    gws = torch.empty(ops.ionn_bias_grad_workspace_bytes(M, C), dtype=torch.uint8, device=dev())
    ops.ionn_bias_grad(dd, gbd, gws)
    am = torch.zeros(1, dtype=torch.int32, device=dev())
    ops.ionn_absmax_i32(gbd, am)
    sh = torch.zeros(2, dtype=torch.int32, device=dev())
    ops.niti_quantize_update_i32(gbd, am, 8, 2, Pd, shifts_out=sh)
    np.testing.assert_array_equal(host(gbd), gb)
    assert host(sh).tolist() == [s, ws]
    np.testing.assert_array_equal(host(Pd), Pn)
