"""GPU parity: DFP as the DFP page runs it ("Mixed Precision Training of
Convolutional Neural Networks using Integer Operations": 3.1 conversions,
4 FP32 chunk partials with the one-bit input shift, 3 Blocked-DFP, the FP32
weight update) against the oracle, bit for bit: every int16 mantissa and
exponent, and every FP32 output (the reduction order is part of the
definition, so the same order gives the same bits)."""
import numpy as np
import pytest
import torch

import ionn_synth
import oracle
from integer_only_nn_amd import ops
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu

FWD, DGRAD, WGRAD = 0, 1, 2


def _e(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=dev())


def _cws():
    return torch.empty(ops.dfp_convert_workspace_bytes(), dtype=torch.uint8, device=dev())


def _same_f32(got, want, msg=""):
    """Bitwise equality of float32 arrays (so -0.0, inf and every rounding count)."""
    g = np.ascontiguousarray(got, np.float32).view(np.uint32)
    w = np.ascontiguousarray(want, np.float32).view(np.uint32)
    bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
    assert bad.size == 0, f"{msg}: {bad.size} differ, first at {bad[:5]}: {got.reshape(-1)[bad[:5]]} vs {want.reshape(-1)[bad[:5]]}"


# ---- conversions ------------------------------------------------------------

def _gpu_from_f32(x, P):
    xd = to_dev(x.astype(np.float32))
    out = torch.empty(x.size, dtype=torch.int16, device=dev())
    e, st = _e(12345), _e(77)
    ops.dfp_from_f32(xd, out, e, _cws(), P=P, status_out=st)
    return host(out).reshape(x.shape), int(host(e)[0]), int(host(st)[0])


@pytest.mark.parametrize("n", [1, 3, 4, 1003, 1 << 20])
@pytest.mark.parametrize("P", [2, 8, 15, 16])
def test_from_f32_parity(n, P):
    rng = np.random.default_rng(n + P)
    for scale in (1.0, 3e-3, 1e30, 1e-40):
        say("from_f32", n, P, scale)
        x = (rng.standard_normal(n) * scale).astype(np.float32)
        I, e, st = oracle.dfp_from_f32(x, P)
        gI, ge, gst = _gpu_from_f32(x, P)
        assert (ge, gst) == (e, st)
        np.testing.assert_array_equal(gI, I)


def test_from_f32_edges():
    # ties to even, the saturating maximum, zeros, lone subnormals
    x = np.array([1.0, 2.5 * 2 ** -14, -2.5 * 2 ** -14, 3.5 * 2 ** -14, 0.0, -0.0], np.float32)
    assert _gpu_from_f32(x, 16)[0].tolist() == oracle.dfp_from_f32(x, 16)[0].tolist() == [16384, 2, -2, 4, 0, 0]
    x = np.array([np.float32(2.0) - np.float32(2 ** -23), -1.0], np.float32)
    assert _gpu_from_f32(x, 16)[0].tolist() == [32767, -16384]
    I, e, st = _gpu_from_f32(np.zeros(9, np.float32), 16)
    assert I.tolist() == [0] * 9 and (e, st) == (0, 0)
    s = np.array([2 ** -149, -3 * 2 ** -149, 0.0], np.float32)
    I, e, st = oracle.dfp_from_f32(s, 16)
    gI, ge, gst = _gpu_from_f32(s, 16)
    assert gI.tolist() == I.tolist() and (ge, gst) == (e, st) and st == 1
    for bad in (np.inf, np.nan):
        assert _gpu_from_f32(np.array([1.0, bad, 2.0, 3.0], np.float32), 16)[2] == 2


def test_to_f32_parity():
    rng = np.random.default_rng(2)
    I = rng.integers(-32768, 32768, 5000).astype(np.int16)
    I[:3] = [0, -32768, 32767]
    for e in (-14, 0, 20, -140, -160, 100, 120, -1100, 1100):
        out = torch.empty(I.size, dtype=torch.float32, device=dev())
        ops.dfp_to_f32(to_dev(I), _e(e), out)
        _same_f32(host(out), oracle.dfp_to_f32(I, e), f"e={e}")


@pytest.mark.parametrize("rows,K,B", [(1, 1, 64), (7, 64, 64), (33, 1000, 64), (5, 300, 100), (256, 4096, 64),
                                      (3, 50, 7)])
def test_from_f32_blocked_parity(rows, K, B):
    rng = np.random.default_rng(rows * K + B)
    x = (rng.standard_normal((rows, K)) * 10.0 ** rng.integers(-6, 6, (rows, 1))).astype(np.float32)
    if K >= 2 * B:
        x[0, B:2 * B] *= 1e5
    I, E, st = oracle.dfp_from_f32_blocked(x, B=B)
    out = torch.empty((rows, K), dtype=torch.int16, device=dev())
    nb = (K + B - 1) // B
    eo = torch.empty(rows * nb, dtype=torch.int32, device=dev())
    sto = _e(5)
    ops.dfp_from_f32_blocked(to_dev(x), out, eo, B=B, status_out=sto)
    np.testing.assert_array_equal(host(out), I)
    np.testing.assert_array_equal(host(eo).reshape(rows, nb), E)
    assert int(host(sto)[0]) == st


# ---- FP32-partial contractions -------------------------------------------------

def _gpu_f32(which, A, eA, B, eB, M, K, N, shift, nsplit, misalign=False):
    def put(a):
        if not misalign:
            return to_dev(a)
        buf = torch.empty(a.size + 1, dtype=torch.int16, device=dev())
        buf[1:] = to_dev(a).reshape(-1)
        return buf[1:].view(a.shape)
    Ad, Bd = put(A), put(B)
    shape = {FWD: (M, N), DGRAD: (M, K), WGRAD: (N, K)}[which]
    out = torch.full(shape, float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(ops.dfp16_f32_workspace_bytes(M, K, N, which, nsplit), dtype=torch.uint8, device=dev())
    fn = {FWD: ops.dfp16_gemm_fwd_f32, DGRAD: ops.dfp16_gemm_dgrad_f32, WGRAD: ops.dfp16_gemm_wgrad_f32}[which]
    fn(Ad, _e(eA), Bd, _e(eB), out, ws, input_shift=shift, nsplit=nsplit)
    return host(out)


def _default_S(M, K, N, which):
    """The default FP32 range count, from the oracle's statement of the rule;
    the library must use the same one."""
    S = oracle.dfp16_default_splits(M, K, N, {FWD: "fwd", DGRAD: "dgrad", WGRAD: "wgrad"}[which])
    assert ops.dfp16_f32_splits(M, K, N, which) == S, (M, K, N, which)
    return S


def _ora_f32(which, A, eA, B, eB, S, shift):
    fn = {FWD: oracle.dfp16_fwd_f32, DGRAD: oracle.dfp16_dgrad_f32, WGRAD: oracle.dfp16_wgrad_f32}[which]
    return fn(A, eA, B, eB, S=S, input_shift=shift)[0]


def _operands(which, M, K, N, seed, sigma=4000.0):
    d = ionn_synth.dfp16_gemm(M=M, K=K, N=N, seed=seed)
    if sigma != 4000.0:
        rng = np.random.default_rng(seed)
        for key, shp in (("X", (M, K)), ("W", (N, K)), ("dY", (M, N))):
            d[key] = np.clip(np.round(rng.standard_normal(shp) * sigma), -32768, 32767).astype(np.int16)
    if which == FWD:
        return d["X"], d["eX"], d["W"], d["eW"]
    if which == DGRAD:
        return d["dY"], d["edY"], d["W"], d["eW"]
    return d["dY"], d["edY"], d["X"], d["eX"]


F32_SHAPES = [(128, 64, 128), (256, 512, 384), (1, 1, 1), (100, 130, 70), (257, 200, 129), (640, 1024, 128),
              (64, 4096, 64)]


@pytest.mark.parametrize("M,K,N", F32_SHAPES)
@pytest.mark.parametrize("which", [FWD, DGRAD, WGRAD])
def test_f32_contraction_parity(M, K, N, which):
    A, eA, B, eB = _operands(which, M, K, N, seed=M + K + N + which)
    L = {FWD: K, DGRAD: N, WGRAD: M}[which]
    nch = (L + 63) // 64
    default = _default_S(M, K, N, which)
    for shift, nsplit in ((1, 0), (0, 0), (1, 1), (1, nch), (1, min(3, nch))):
        S = nsplit or default
        say("f32", which, M, K, N, shift, nsplit, S)
        want = _ora_f32(which, A, eA, B, eB, S, shift)
        _same_f32(_gpu_f32(which, A, eA, B, eB, M, K, N, shift, nsplit), want, f"which={which} S={S}")


@pytest.mark.parametrize("which", [FWD, DGRAD, WGRAD])
def test_f32_contraction_unaligned_operands(which):
    M, K, N = 256, 256, 128
    A, eA, B, eB = _operands(which, M, K, N, seed=9 + which)
    S = _default_S(M, K, N, which)
    _same_f32(_gpu_f32(which, A, eA, B, eB, M, K, N, 1, 0, misalign=True), _ora_f32(which, A, eA, B, eB, S, 1))


def test_f32_contraction_extreme_exponents():
    """Scalings into the subnormal range and past the largest single."""
    M, K, N = 128, 128, 128
    A, _, B, _ = _operands(FWD, M, K, N, seed=4)
    for eA, eB in ((-100, -100), (-70, -90), (60, 60), (127, 127), (-128, -128)):
        _same_f32(_gpu_f32(FWD, A, eA, B, eB, M, K, N, 1, 0), _ora_f32(FWD, A, eA, B, eB, 1, 1), f"{eA},{eB}")


@pytest.mark.parametrize("which", [FWD, DGRAD, WGRAD])
def test_f32_contraction_full_size_sampled(which):
    """The DFP-16 layer M=25088, K=256, N=1024 in the launch the benchmark
    times: 4096 sampled outputs (and whole rows) against the oracle."""
    M, K, N = 25088, 256, 1024
    A, eA, B, eB = _operands(which, M, K, N, seed=0)
    S = _default_S(M, K, N, which)
    got = _gpu_f32(which, A, eA, B, eB, M, K, N, 1, 0)
    R, C = got.shape
    rng = np.random.default_rng(which)
    idx = [(int(r), int(c)) for r, c in zip(rng.integers(0, R, 4096), rng.integers(0, C, 4096))]
    idx += [(R - 1, c) for c in range(0, C, max(1, C // 64))] + [(0, C - 1)]
    role = {FWD: "fwd", DGRAD: "dgrad", WGRAD: "wgrad"}[which]
    want = np.array([oracle.dfp16_f32_at(role, A, eA, B, eB, r, c, S=S) for r, c in idx], np.float32)
    _same_f32(np.array([got[r, c] for r, c in idx], np.float32), want, role)
    assert np.isfinite(got).all()


# ---- FP32 weight update ---------------------------------------------------------

@pytest.mark.parametrize("n", [1, 7, 4096, (1 << 20) + 3])
def test_sgd_update_parity(n):
    rng = np.random.default_rng(n)
    W = (rng.standard_normal(n) * 0.05).astype(np.float32)
    G = (rng.standard_normal(n) * 3.0).astype(np.float32)
    for lr in (0.1, 2.0 ** -7, 0.0123):
        W2, W16, eW, st = oracle.dfp16_sgd(W, G, lr)
        Wd, Gd = to_dev(W), to_dev(G)
        w16 = torch.empty(n, dtype=torch.int16, device=dev())
        e, s = _e(0), _e(9)
        ops.dfp16_sgd_update(Wd, Gd, lr, w16, e, _cws(), status_out=s)
        _same_f32(host(Wd), W2, f"lr={lr}")
        np.testing.assert_array_equal(host(w16), W16)
        assert (int(host(e)[0]), int(host(s)[0])) == (eW, st)


def test_paper_step_chain():
    """One training step of a DFP layer as the page runs it: FP32 weights
    and input converted to DFP-16, the three FP32-partial contractions, the
    output re-quantised for the next layer, and the FP32 weight update with
    its DFP-16 copy; every intermediate against the oracle."""
    M, K, N = 384, 256, 256
    rng = np.random.default_rng(12)
    X32 = (rng.standard_normal((M, K)) * 2.0).astype(np.float32)
    W32 = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    dY32 = (rng.standard_normal((M, N)) * 1e-3).astype(np.float32)
    Xo, eX, _ = oracle.dfp_from_f32(X32)
    Wo, eW, _ = oracle.dfp_from_f32(W32)
    dYo, edY, _ = oracle.dfp_from_f32(dY32)
    Y = oracle.dfp16_fwd_f32(Xo, eX, Wo, eW, S=_default_S(M, K, N, FWD))[0]
    Yo, eY, _ = oracle.dfp_from_f32(Y)
    dX = oracle.dfp16_dgrad_f32(dYo, edY, Wo, eW, S=_default_S(M, K, N, DGRAD))[0]
    G = oracle.dfp16_wgrad_f32(dYo, edY, Xo, eX, S=_default_S(M, K, N, WGRAD))[0]
    W2, W16, eW2, _ = oracle.dfp16_sgd(W32, G, 0.01)

    cws = _cws()
    conv = lambda t: (torch.empty(t.shape, dtype=torch.int16, device=dev()), _e(0))
    Xd, eXd = conv(X32)
    ops.dfp_from_f32(to_dev(X32), Xd, eXd, cws)
    Wd32 = to_dev(W32)
    Wd, eWd = conv(W32)
    ops.dfp_from_f32(Wd32, Wd, eWd, cws)
    dYd, edYd = conv(dY32)
    ops.dfp_from_f32(to_dev(dY32), dYd, edYd, cws)
    ws = lambda w: torch.empty(ops.dfp16_f32_workspace_bytes(M, K, N, w), dtype=torch.uint8, device=dev())
    Yd = torch.empty((M, N), dtype=torch.float32, device=dev())
    ops.dfp16_gemm_fwd_f32(Xd, eXd, Wd, eWd, Yd, ws(FWD))
    Y16, eY16 = conv(Y)
    ops.dfp_from_f32(Yd, Y16, eY16, cws)
    dXd = torch.empty((M, K), dtype=torch.float32, device=dev())
    ops.dfp16_gemm_dgrad_f32(dYd, edYd, Wd, eWd, dXd, ws(DGRAD))
    Gd = torch.empty((N, K), dtype=torch.float32, device=dev())
    ops.dfp16_gemm_wgrad_f32(dYd, edYd, Xd, eXd, Gd, ws(WGRAD))
    ops.dfp16_sgd_update(Wd32, Gd, 0.01, Wd, eWd, cws)
    _same_f32(host(Yd), Y, "Y")
    np.testing.assert_array_equal(host(Y16), Yo)
    assert int(host(eY16)[0]) == eY
    _same_f32(host(dXd), dX, "dX")
    _same_f32(host(Gd), G, "G")
    _same_f32(host(Wd32), W2, "W32")
    np.testing.assert_array_equal(host(Wd), W16)
    assert int(host(eWd)[0]) == eW2


# ---- Blocked-DFP forward -------------------------------------------------------

@pytest.mark.parametrize("M,K,N", [(128, 256, 128), (256, 1024, 384), (100, 130, 70), (1, 64, 1), (640, 256, 256),
                                   (128, 4096, 128)])
def test_blocked_fwd_parity(M, K, N):
    """Float tensors with rows of very different scales, converted to
    Blocked-DFP (64-value blocks), then the blocked forward contraction."""
    rng = np.random.default_rng(M + K + N)
    X32 = (rng.standard_normal((M, K)) * 10.0 ** rng.integers(-3, 3, (M, 1))).astype(np.float32)
    W32 = (rng.standard_normal((N, K)) * 10.0 ** rng.integers(-3, 1, (1, K))).astype(np.float32)
    Xb, eX, _ = oracle.dfp_from_f32_blocked(X32)
    Wb, eW, _ = oracle.dfp_from_f32_blocked(W32)
    nch = (K + 63) // 64
    default = _default_S(M, K, N, FWD)
    for shift, nsplit in ((1, 0), (0, 1), (1, min(3, nch))):
        S = nsplit or default
        say("blocked", M, K, N, shift, S)
        want, _ = oracle.dfp16_fwd_f32_blocked(Xb, eX, Wb, eW, S=S, input_shift=shift)
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev())
        ws = torch.empty(ops.dfp16_f32_workspace_bytes(M, K, N, FWD, nsplit), dtype=torch.uint8, device=dev())
        ops.dfp16_gemm_fwd_f32_blocked(to_dev(Xb), to_dev(eX), to_dev(Wb), to_dev(eW), Y, ws,
                                       input_shift=shift, nsplit=nsplit)
        _same_f32(host(Y), want, f"S={S} shift={shift}")


def test_blocked_fwd_from_device_conversion_and_subnormal_terms():
    """The blocked conversion on the device feeding the blocked forward;
    block exponents low enough that chunk terms land in the subnormal range
    (where v_ldexp_f32 rounds them once, as the oracle does)."""
    M, K, N = 256, 512, 128
    rng = np.random.default_rng(77)
    X32 = (rng.standard_normal((M, K)) * 1e-20).astype(np.float32)
    W32 = (rng.standard_normal((N, K)) * 1e-19).astype(np.float32)
    X32[: M // 2, 64:128] *= 1e15   # half the rows keep only tiny blocks
    Xd = torch.empty((M, K), dtype=torch.int16, device=dev())
    Wd = torch.empty((N, K), dtype=torch.int16, device=dev())
    eXd = torch.empty(M * (K // 64), dtype=torch.int32, device=dev())
    eWd = torch.empty(N * (K // 64), dtype=torch.int32, device=dev())
    ops.dfp_from_f32_blocked(to_dev(X32), Xd, eXd)
    ops.dfp_from_f32_blocked(to_dev(W32), Wd, eWd)
    Xb, eX, _ = oracle.dfp_from_f32_blocked(X32)
    Wb, eW, _ = oracle.dfp_from_f32_blocked(W32)
    np.testing.assert_array_equal(host(Xd), Xb)
    np.testing.assert_array_equal(host(eXd).reshape(eX.shape), eX)
    assert (eX.astype(np.int64)[:, :, None] + eW.astype(np.int64).T[None] + 1).min() < -150   # subnormal terms occur
    want, _ = oracle.dfp16_fwd_f32_blocked(Xb, eX, Wb, eW, S=_default_S(M, K, N, FWD))
    Y = torch.empty((M, N), dtype=torch.float32, device=dev())
    ws = torch.empty(ops.dfp16_f32_workspace_bytes(M, K, N, FWD), dtype=torch.uint8, device=dev())
    ops.dfp16_gemm_fwd_f32_blocked(Xd, eXd, Wd, eWd, Y, ws)
    _same_f32(host(Y), want, "blocked subnormal")
    assert (np.abs(want) < 2.0 ** -126).any() and (want != 0).any()
