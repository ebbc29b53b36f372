"""GPU parity: adaptive per-layer precision ("Adaptive Precision Training for
Resource Constrained Devices": the k-bit update on the 2^e grid, Gavg
sampling, Algorithm 1's one-bit moves between epochs as Algorithm 2 lays
them out) against the oracle, bit-exact for every weight, precision and
exponent and bitwise for the double Gavg sums."""
import numpy as np
import pytest
import torch

import ionn_synth
import oracle
from oracle import apt as oapt
from integer_only_nn_amd import ops
from integer_only_nn_amd.steps import AptLayers
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def _i32(v):
    return torch.tensor(list(v), dtype=torch.int32, device=dev())


def _layers(sizes, seed, kmax=16):
    rng = np.random.default_rng(seed)
    ks = [int(rng.integers(2, kmax + 1)) for _ in sizes]
    Ws = []
    for l, (n, k) in enumerate(zip(sizes, ks)):
        lim = 1 << (k - 1)
        Ws.append(rng.integers(-lim, lim, n).astype(np.int16))
    return Ws, ks


def _grads(sizes, seed, sigma=2000.0):
    return [ionn_synth.apt_grad(seed * 1000 + l, n, sigma, seed=seed) for l, n in enumerate(sizes)]


UPDATE_SIZES = [
    [1], [7], [8], [9], [4097], [8192], [8193],
    [8192 * 3 + 5, 3, 100, 65536 + 8],
    ionn_synth.RESNET20_SIZES,
]


@pytest.mark.parametrize("sizes", UPDATE_SIZES, ids=lambda s: f"L{len(s)}_n{sum(s)}")
@pytest.mark.parametrize("sample", [False, True])
def test_update_parity(sizes, sample):
    say("apt_update", len(sizes), sum(sizes), sample)
    seed = len(sizes) * 7 + sum(sizes) % 97
    Ws, ks = _layers(sizes, seed)
    Gs = _grads(sizes, seed)
    rng = np.random.default_rng(seed + 1)
    e_w = [int(x) for x in rng.integers(-20, 0, len(sizes))]
    e_g = [int(x) for x in rng.integers(-30, -5, len(sizes))]
    lr = 4
    st = AptLayers(Ws, ks, e_w, dev())
    eg = _i32(e_g)
    Gd = [to_dev(g) for g in Gs]
    st.step(Gd, eg, lr, sample=sample)
    for l in range(len(sizes)):
        want, _ = oracle.apt_update(Ws[l], ks[l], e_w[l], Gs[l], e_g[l], lr)
        np.testing.assert_array_equal(host(st.W[l]), want, err_msg=f"layer {l}")
    if sample:
        want = [0.0 + oracle.gavg(Gs[l], e_g[l], e_w[l]) for l in range(len(sizes))]
        assert host(st.gsum).tolist() == want
        assert host(st.gcnt).tolist() == [1] * len(sizes)
    else:
        assert host(st.gcnt).tolist() == [0] * len(sizes)


@pytest.mark.parametrize("sigma", [-40, -17, -16, -15, -1, 0, 1, 2, 15, 16, 17, 20, 21, 60])
def test_update_sigma_range(sigma):
    """sigma = e_w + lr_shift - e_g across both branches and the clamps of
    the shifts, with extreme mantissas and every k."""
    n = 4096 + 3
    rng = np.random.default_rng(100 + sigma)
    G = rng.integers(-32768, 32768, n).astype(np.int16)
    G[:6] = [-32768, 32767, 0, 1, -1, 2]
    for k in (2, 8, 15, 16):
        lim = 1 << (k - 1)
        W = rng.integers(-lim, lim, n).astype(np.int16)
        W[:2] = [lim - 1, -lim]
        lr = 3
        e_g = -10
        e_w = sigma + e_g - lr
        st = AptLayers([W], [k], [e_w], dev())
        st.step([to_dev(G)], _i32([e_g]), lr, sample=True)
        want, _ = oracle.apt_update(W, k, e_w, G, e_g, lr)
        np.testing.assert_array_equal(host(st.W[0]), want, err_msg=f"k={k}")
        assert host(st.gsum).tolist() == [0.0 + oracle.gavg(G, e_g, e_w)]


def test_update_unaligned_and_mixed():
    """2-byte aligned tensors take the element path; a model may mix
    aligned and unaligned layers in one launch."""
    sizes = [1000, 8192 + 17, 3]
    Ws, ks = _layers(sizes, 5)
    Gs = _grads(sizes, 5)
    e_w, e_g = [-8, -9, -10], [-20, -21, -22]
    Wd, Gd = [], []
    for l, (w, g) in enumerate(zip(Ws, Gs)):
        off = l % 2  # layer 1 is shifted by one element
        bw = torch.empty(w.size + off, dtype=torch.int16, device=dev())
        bg = torch.empty(g.size + 1, dtype=torch.int16, device=dev())
        bw[off:] = to_dev(w)
        bg[1:] = to_dev(g)
        Wd.append(bw[off:])
        Gd.append(bg[1:])
    gsum = torch.zeros(3, dtype=torch.float64, device=dev())
    gcnt = torch.zeros(3, dtype=torch.int32, device=dev())
    ws = torch.empty(ops.apt_workspace_bytes(sizes), dtype=torch.uint8, device=dev())
    ops.apt_update(Wd, Gd, _i32(ks), _i32(e_w), _i32(e_g), 2, gsum, gcnt, ws)
    for l in range(3):
        want, _ = oracle.apt_update(Ws[l], ks[l], e_w[l], Gs[l], e_g[l], 2)
        np.testing.assert_array_equal(host(Wd[l]), want)
    assert host(gsum).tolist() == [0.0 + oracle.gavg(Gs[l], e_g[l], e_w[l]) for l in range(3)]


def test_update_full_size_layer():
    """One 4096 x 4096 layer (16.8 M weights) in the launch shape the
    benchmark times, every weight checked."""
    n = 4096 * 4096
    W, _ = ionn_synth.apt_weights([n], k0=12, seed=3)
    W = W[0]
    G = ionn_synth.apt_grad(9, n, 3000.0, seed=3)
    st = AptLayers([W], [12], [-10], dev())
    st.step([to_dev(G)], _i32([-22]), 6, sample=True)
    want, _ = oracle.apt_update(W, 12, -10, G, -22, 6)
    np.testing.assert_array_equal(host(st.W[0]), want)
    assert host(st.gsum).tolist() == [0.0 + oracle.gavg(G, -22, -10)]


def test_sampling_accumulates_in_step_order():
    sizes = [3000, 20000]
    Ws, ks = _layers(sizes, 8)
    e_w = [-6, -7]
    st = AptLayers(Ws, ks, e_w, dev())
    want = [0.0, 0.0]
    for s in range(5):
        Gs = _grads(sizes, 20 + s, sigma=100.0 * (s + 1))
        e_g = [-12 - s, -9 + s]
        st.step([to_dev(g) for g in Gs], _i32(e_g), 5, sample=True)
        for l in range(2):
            want[l] = want[l] + oracle.gavg(Gs[l], e_g[l], e_w[l])
    assert host(st.gsum).tolist() == want
    assert host(st.gcnt).tolist() == [5, 5]


def test_adjust_parity():
    """Every branch of the decision: below T_min (raise, or held at k_max),
    above T_max (lower, or held at k_min), inside the band, no samples."""
    sizes = [500, 8192 * 2 + 1, 64, 9000, 7, 33000, 1]
    ks = [6, 16, 5, 2, 9, 12, 3]
    sums = [0.5, 0.1, 300.0, 300.0, 5.0, 0.0, 0.9]
    cnts = [2, 1, 3, 1, 1, 0, 1]
    rng = np.random.default_rng(4)
    Ws = [rng.integers(-(1 << (k - 1)), 1 << (k - 1), n).astype(np.int16) for n, k in zip(sizes, ks)]
    e_w = [-5, -9, -3, -1, -7, -12, -2]
    t_min, t_max, k_min, k_max = 1.0, 50.0, 2, 16
    st = AptLayers(Ws, ks, e_w, dev())
    st.gsum.copy_(torch.tensor(sums, dtype=torch.float64))
    st.gcnt.copy_(torch.tensor(cnts, dtype=torch.int32))
    st.end_epoch(t_min, t_max, k_min, k_max)
    dks = [oracle.apt_decide(s, c, k, t_min, t_max, k_min, k_max) for s, c, k in zip(sums, cnts, ks)]
    assert dks == [1, 0, -1, 0, 0, 0, 1]
    assert host(st.dk).tolist() == dks
    assert host(st.k).tolist() == [k + d for k, d in zip(ks, dks)]
    assert host(st.e_w).tolist() == [e - d for e, d in zip(e_w, dks)]
    for l in range(len(sizes)):
        np.testing.assert_array_equal(host(st.W[l]), oracle.apt_rescale(Ws[l], ks[l], dks[l]))
    assert host(st.gsum).tolist() == [0.0] * 7 and host(st.gcnt).tolist() == [0] * 7


def test_workflow_parity_resnet20():
    """Algorithm 2 over the 20 weight layers of a ResNet-20, starting at 6
    bits: 4 epochs of 4 steps, Gavg sampled on every other step, precision
    moved between epochs; every layer's weights, k and exponent compared
    after each epoch, and the epoch's sums before the move."""
    sizes = ionn_synth.RESNET20_SIZES
    L = len(sizes)
    Ws, es = ionn_synth.apt_weights(sizes, k0=6, seed=0)
    sig = [40.0 * (1 + (l % 5) ** 3) for l in range(L)]
    egs = [-14 - (l % 3) for l in range(L)]

    def grad(ep, st, l, state=None):
        return ionn_synth.apt_grad((ep * 16 + st) * L + l, sizes[l], sig[l]), egs[l]

    epochs, steps, every, lr = 4, 4, 2, 3
    t_min, t_max = 1.0, 40.0
    ostate = oapt.new_state(Ws, [6] * L, es)
    dstate = AptLayers(Ws, [6] * L, es, dev())
    eg = _i32(egs)
    moved = 0
    for ep in range(epochs):
        sums, counts = [0.0] * L, [0] * L
        for st in range(steps):
            grads = [grad(ep, st, l) for l in range(L)]
            sample = st % every == 0
            oapt.step(ostate, grads, lr, sums if sample else None, counts if sample else None)
            dstate.step([to_dev(g) for g, _ in grads], eg, lr, sample=sample)
        say("epoch", ep)
        assert host(dstate.gsum).tolist() == sums
        assert host(dstate.gcnt).tolist() == counts
        dks = oapt.adjust(ostate, sums, counts, t_min, t_max, 2, 16)
        dstate.end_epoch(t_min, t_max, 2, 16)
        assert host(dstate.dk).tolist() == dks
        assert host(dstate.k).tolist() == [s["k"] for s in ostate]
        assert host(dstate.e_w).tolist() == [s["e_w"] for s in ostate]
        for l in range(L):
            np.testing.assert_array_equal(host(dstate.W[l]), ostate[l]["W"], err_msg=f"epoch {ep} layer {l}")
        moved += sum(1 for d in dks if d)
    assert moved > 0


def test_dfp16_wgrad_then_update():
    """A DFP-16 layer's weight gradient (dfp16_gemm_wgrad) feeding the k-bit
    update: the whole chain against the oracle's."""
    d = ionn_synth.dfp16_gemm(M=1000, K=96, N=80, seed=11)
    k, e_w = 10, d["eW"] + 6
    Wk = np.clip(d["W"] >> 6, -(1 << (k - 1)), (1 << (k - 1)) - 1).astype(np.int16)
    G, eG, _ = oracle.dfp16_wgrad(d["dY"], d["edY"], d["X"], d["eX"])
    Gd = torch.empty((80, 96), dtype=torch.int16, device=dev())
    eGd = torch.zeros(1, dtype=torch.int32, device=dev())
    ws = torch.empty(ops.dfp16_workspace_bytes(1000, 96, 80, 2), dtype=torch.uint8, device=dev())
    ops.dfp16_gemm_wgrad(to_dev(d["dY"]), _i32([d["edY"]]), to_dev(d["X"]), _i32([d["eX"]]), Gd, eGd, ws)
    np.testing.assert_array_equal(host(Gd), G)
    assert int(host(eGd)[0]) == eG
    st = AptLayers([Wk.reshape(-1)], [k], [e_w], dev())
    st.step([Gd.view(-1)], eGd, 2, sample=True)
    want, _ = oracle.apt_update(Wk.reshape(-1), k, e_w, G.reshape(-1), eG, 2)
    np.testing.assert_array_equal(host(st.W[0]), want)
    assert host(st.gsum).tolist() == [0.0 + oracle.gavg(G.reshape(-1), eG, e_w)]


def test_k_outside_range_reads_as_bound():
    n = 100
    W = np.arange(-50, 50, dtype=np.int16)
    G = np.full(n, -64, np.int16)
    st = AptLayers([W, W], [1, 40], [0, 0], dev())
    st.step([to_dev(G), to_dev(G)], _i32([0, 0]), 0)
    np.testing.assert_array_equal(host(st.W[0]), oracle.apt_update(W, 2, 0, G, 0, 0)[0])
    np.testing.assert_array_equal(host(st.W[1]), oracle.apt_update(W, 16, 0, G, 0, 0)[0])


def test_update_replayed_from_graph():
    """A sampling step captured in a HIP graph and replayed three times,
    with eager work and synchronisations between the replays: every replay
    matches the oracle applying the same step again."""
    sizes = [5000, 300, 20000]
    Ws, ks = _layers(sizes, 31)
    Gs = _grads(sizes, 31)
    e_w, e_g = [-9, -8, -10], [-18, -17, -19]
    st = AptLayers(Ws, ks, e_w, dev())
    st.bind_grads([to_dev(g) for g in Gs])
    eg = _i32(e_g)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st.step(None, eg, 1, sample=True, stream=s.cuda_stream)
    torch.cuda.synchronize()
    ostate = oapt.new_state(Ws, ks, e_w)
    sums, counts = [0.0] * 3, [0] * 3
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        oapt.step(ostate, list(zip(Gs, e_g)), 1, sums, counts)
        for l in range(3):
            np.testing.assert_array_equal(host(st.W[l]), ostate[l]["W"], err_msg=f"replay {rep} layer {l}")
        assert host(st.gsum).tolist() == sums and host(st.gcnt).tolist() == counts
        torch.zeros(1000, device=dev()).add_(1.0)   # unrelated eager work between replays


# ---- layers held in int8 (k <= 8): half the memory, the same arithmetic ----

@pytest.mark.parametrize("sample", [False, True])
def test_int8_storage_update_parity(sample):
    """Layers of every size class held in int8 (odd sizes, ragged tails, a
    1-byte misaligned tensor on the element path) mixed with int16 layers in
    one launch: every weight equals the oracle's int16 result."""
    sizes = [1, 7, 8, 4097, 8193, 65536 + 5, 3000]
    seed = 17
    Ws, ks = _layers(sizes, seed, kmax=8)
    Gs = _grads(sizes, seed)
    rng = np.random.default_rng(seed + 1)
    e_w = [int(x) for x in rng.integers(-20, 0, len(sizes))]
    e_g = [int(x) for x in rng.integers(-30, -5, len(sizes))]
    i8 = (0, 1, 3, 5, 6)
    st = AptLayers(Ws, ks, e_w, dev(), int8_layers=i8)
    assert [w.element_size() for w in st.W] == [1 if l in i8 else 2 for l in range(len(sizes))]
    # layer 6 held one byte off its allocation's alignment (element path)
    buf = torch.empty(sizes[6] + 1, dtype=torch.int8, device=dev())
    buf[1:] = st.W[6]
    W6 = buf[1:]
    Wd = st.W[:6] + [W6]
    gsum = torch.zeros(len(sizes), dtype=torch.float64, device=dev())
    gcnt = torch.zeros(len(sizes), dtype=torch.int32, device=dev())
    ws = torch.empty(ops.apt_workspace_bytes(sizes), dtype=torch.uint8, device=dev())
    ops.apt_update_mixed(Wd, [to_dev(g) for g in Gs], _i32(ks), _i32(e_w), _i32(e_g), 4,
                         gsum if sample else None, gcnt if sample else None, ws if sample else None)
    for l in range(len(sizes)):
        want, _ = oracle.apt_update(Ws[l], ks[l], e_w[l], Gs[l], e_g[l], 4)
        np.testing.assert_array_equal(host(Wd[l]).astype(np.int16), want, err_msg=f"layer {l}")
    if sample:
        assert host(gsum).tolist() == [0.0 + oracle.gavg(Gs[l], e_g[l], e_w[l]) for l in range(len(sizes))]


def test_int8_storage_k_reads_and_stays_within_8():
    """An int8 layer reads a k above 8 as 8, and the epoch policy never
    raises it past 8 (it still lowers it); an int16 layer beside it rises."""
    n = 5000
    rng = np.random.default_rng(3)
    W8 = rng.integers(-128, 128, n).astype(np.int16)
    W16 = rng.integers(-128, 128, n).astype(np.int16)
    G = ionn_synth.apt_grad(5, n, 500.0)
    st = AptLayers([W8, W16], [8, 8], [-6, -6], dev(), int8_layers=(0,))
    st.k.copy_(torch.tensor([12, 8], dtype=torch.int32))       # read as 8 for the int8 layer
    st.step([to_dev(G), to_dev(G)], _i32([-12, -12]), 2)
    want, _ = oracle.apt_update(W8, 8, -6, G, -12, 2)
    np.testing.assert_array_equal(host(st.W[0]).astype(np.int16), want)
    # a mean below T_min: the int16 layer gains a bit, the int8 one is held
    st.k.copy_(torch.tensor([8, 8], dtype=torch.int32))
    st.gsum.copy_(torch.tensor([0.01, 0.01], dtype=torch.float64))
    st.gcnt.copy_(torch.tensor([1, 1], dtype=torch.int32))
    before = [host(w).astype(np.int16) for w in st.W]
    st.end_epoch(1.0, 50.0, 2, 16)
    assert host(st.dk).tolist() == [0, 1] and host(st.k).tolist() == [8, 9]
    np.testing.assert_array_equal(host(st.W[0]).astype(np.int16), before[0])
    np.testing.assert_array_equal(host(st.W[1]), oracle.apt_rescale(before[1], 8, 1))
    # a mean above T_max: the int8 layer loses a bit like any other
    st.gsum.copy_(torch.tensor([500.0, 0.5], dtype=torch.float64))
    st.gcnt.copy_(torch.tensor([1, 1], dtype=torch.int32))
    st.end_epoch(1.0, 50.0, 2, 16)
    assert host(st.dk).tolist()[0] == -1 and int(host(st.k)[0]) == 7
    np.testing.assert_array_equal(host(st.W[0]).astype(np.int16), oracle.apt_rescale(before[0], 8, -1))


def test_int8_storage_workflow_parity_resnet20():
    """Algorithm 2 over a ResNet-20's 20 layers held in int8 (k from 6,
    k_max 8): 3 epochs of 4 steps against the oracle run with k_max = 8; the
    weights take half the bytes of the int16 layers."""
    sizes = ionn_synth.RESNET20_SIZES
    L = len(sizes)
    Ws, es = ionn_synth.apt_weights(sizes, k0=6, seed=1)
    sig = [30.0 * (1 + (l % 4) ** 3) for l in range(L)]
    egs = [-13 - (l % 3) for l in range(L)]
    ostate = oapt.new_state(Ws, [6] * L, es)
    dstate = AptLayers(Ws, [6] * L, es, dev(), int8_layers=tuple(range(L)))
    assert sum(w.numel() * w.element_size() for w in dstate.W) == sum(sizes)
    eg = _i32(egs)
    moved = 0
    for ep in range(3):
        sums, counts = [0.0] * L, [0] * L
        for s in range(4):
            grads = [(ionn_synth.apt_grad((ep * 8 + s) * L + l, sizes[l], sig[l]), egs[l]) for l in range(L)]
            sample = s % 2 == 0
            oapt.step(ostate, grads, 3, sums if sample else None, counts if sample else None)
            dstate.step([to_dev(g) for g, _ in grads], eg, 3, sample=sample)
        dks = oapt.adjust(ostate, sums, counts, 1.0, 30.0, 2, 8)
        dstate.end_epoch(1.0, 30.0, 2, 16)   # the int8 layers stop at 8 by themselves
        assert host(dstate.dk).tolist() == dks
        assert host(dstate.k).tolist() == [s["k"] for s in ostate]
        for l in range(L):
            np.testing.assert_array_equal(host(dstate.W[l]).astype(np.int16), ostate[l]["W"],
                                          err_msg=f"epoch {ep} layer {l}")
        moved += sum(1 for d in dks if d)
    assert moved > 0
