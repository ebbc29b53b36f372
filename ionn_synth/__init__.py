"""Seeded synthetic inputs for the integer training step.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the GPU library's tests/benchmarks and the CPU oracle consume
the arrays it returns, so the two sides always see identical bytes.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: element i of stream
(seed, sid) is mix64(base + (i + 1) * GAMMA) with base = (seed << 32) | sid.
Uniform integers: lo + (u mod (hi - lo + 1)).  Normals: Box-Muller on
consecutive pairs, u1 = ((x0 >> 11) + 1) * 2^-53 in (0, 1],
u2 = (x1 >> 11) * 2^-53, then sigma * z rounded half away from zero and
clipped.  Stream ids: X=1, W=2, dY=3, labels=4, W1..W3=5..7, exponents of
X/W/dY = 8..10; per layer l of a model, offsets / multipliers / shifts =
20 + 3 l, 21 + 3 l, 22 + 3 l; target magnitudes = 40, 41.
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

SID_X, SID_W, SID_DY, SID_LABELS, SID_W1, SID_W2, SID_W3, SID_EX, SID_EW, SID_EDY = range(1, 11)


def _mix64(z):
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, sid: int, n: int, start: int = 0) -> np.ndarray:
    """n raw 64-bit outputs of stream (seed, sid), starting at counter `start`."""
    base = np.uint64(((int(seed) & 0xFFFFFFFF) << 32) | (int(sid) & 0xFFFFFFFF))
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(base + i * GAMMA)


def uniform_int(seed, sid, shape, lo, hi, dtype=np.int8):
    n = int(np.prod(shape))
    rng = np.uint64(hi - lo + 1)
    out = np.empty(n, dtype)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        u = splitmix64(seed, sid, m, s)
        out[s:s + m] = (np.int64(lo) + (u % rng).astype(np.int64)).astype(dtype)
    return out.reshape(shape)


def normal_int(seed, sid, shape, sigma, lo, hi, dtype=np.int8):
    """round_half_away(sigma * N(0,1)) clipped to [lo, hi]."""
    n = int(np.prod(shape))
    npairs = (n + 1) // 2
    out = np.empty(2 * npairs, dtype)
    for p0 in range(0, npairs, _CHUNK):
        pm = min(_CHUNK, npairs - p0)
        u = splitmix64(seed, sid, 2 * pm, 2 * p0)
        u1 = ((u[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
        u2 = (u[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        r = np.sqrt(-2.0 * np.log(u1))
        t = 2.0 * np.pi * u2
        z = np.empty(2 * pm, np.float64)
        z[0::2] = r * np.cos(t)
        z[1::2] = r * np.sin(t)
        v = sigma * z
        v = np.sign(v) * np.floor(np.abs(v) + 0.5)
        out[2 * p0:2 * (p0 + pm)] = np.clip(v, lo, hi).astype(dtype)
    return out[:n].reshape(shape)


# ---------------------------------------------------------------------------
# The five workloads.  Size arguments default to the full configuration;
# parity tests pass smaller sizes with the same value distributions.
# ---------------------------------------------------------------------------

def single_linear(B=16, IN=64, OUT=32, seed=0):
    """Single int8 linear layer: X ~ U[-128,127], W ~ round(N(0,30)),
    incoming deltas ~ U[-64,63]."""
    return dict(
        X=uniform_int(seed, SID_X, (B, IN), -128, 127),
        W=normal_int(seed, SID_W, (OUT, IN), 30.0, -128, 127),
        dY=uniform_int(seed, SID_DY, (B, OUT), -64, 63),
    )


def mlp(B=256, sizes=(784, 256, 128, 10), seed=0):
    """Int8 MLP: inputs ~ U[0,127], labels ~ U{0..C-1}, W_l ~ round(N(0,25))."""
    Ws = []
    for l in range(len(sizes) - 1):
        Ws.append(normal_int(seed, SID_W1 + l, (sizes[l + 1], sizes[l]), 25.0, -128, 127))
    return dict(
        X=uniform_int(seed, SID_X, (B, sizes[0]), 0, 127),
        labels=uniform_int(seed, SID_LABELS, (B,), 0, sizes[-1] - 1, dtype=np.int32),
        Ws=Ws,
    )


def large_linear(T=8192, IN=4096, OUT=4096, seed=0):
    """Large int8 linear layer: X ~ round(N(0,40)), W ~ round(N(0,20)),
    deltas ~ U[-64,63]."""
    return dict(
        X=normal_int(seed, SID_X, (T, IN), 40.0, -128, 127),
        W=normal_int(seed, SID_W, (OUT, IN), 20.0, -128, 127),
        dY=uniform_int(seed, SID_DY, (T, OUT), -64, 63),
    )


def conv3x3(N=128, H=56, W=56, Cin=64, Cout=64, seed=0):
    """Int8 3x3 conv layer (NHWC / OHWI): X ~ U[0,127], W ~ round(N(0,15)),
    deltas ~ U[-64,63] shaped like the output."""
    return dict(
        X=uniform_int(seed, SID_X, (N, H, W, Cin), 0, 127),
        W=normal_int(seed, SID_W, (Cout, 3, 3, Cin), 15.0, -128, 127),
        dY=uniform_int(seed, SID_DY, (N, H, W, Cout), -64, 63),
    )


def dfp16_gemm(M=25088, K=256, N=1024, seed=0):
    """DFP-16 1x1-conv GEMM: int16 mantissas round(N(0,4000)) clipped to the
    int16 range, one shared exponent per tensor ~ U{-20..-8}."""
    e = lambda sid: int(uniform_int(seed, sid, (1,), -20, -8, dtype=np.int32)[0])
    return dict(
        X=normal_int(seed, SID_X, (M, K), 4000.0, -32768, 32767, dtype=np.int16),
        W=normal_int(seed, SID_W, (N, K), 4000.0, -32768, 32767, dtype=np.int16),
        dY=normal_int(seed, SID_DY, (M, N), 4000.0, -32768, 32767, dtype=np.int16),
        eX=e(SID_EX), eW=e(SID_EW), edY=e(SID_EDY),
    )


def arc_fault(B=8, seed=0):
    """The example network of the TI on-device training page (arc-fault
    detection): input 64 x 2 x 1 int8, Conv 3 filters 16 x 2 valid + ReLU
    (-> 49 x 1 x 3 = 147), Linear 160 + ReLU, Linear 2; batch 8.  Weights
    ~ round(N(0, 25)) (conv) and round(N(0, 20)) (linear); int32 offsets
    ~ U[-256, 255]; multipliers ~ U[1, 4]; per-filter right shifts
    ~ U{8..10}; inputs ~ round(N(0, 40)); labels ~ U{0, 1}; per-class target
    magnitudes ~ U[60, 100] (true class) and U[-100, -60] (other class)."""
    shapes = [(3, 16, 2, 1), (160, 147), (2, 160)]
    sigma = [25.0, 20.0, 20.0]
    layers = []
    for l, shp in enumerate(shapes):
        C = shp[0]
        layers.append(dict(
            W=normal_int(seed, SID_W1 + l, shp, sigma[l], -128, 127),
            offset=uniform_int(seed, 20 + 3 * l, (C,), -256, 255, dtype=np.int32),
            mult=uniform_int(seed, 21 + 3 * l, (C,), 1, 4, dtype=np.int32),
            k=uniform_int(seed, 22 + 3 * l, (C,), 8, 10, dtype=np.int8),
        ))
    return dict(
        X=normal_int(seed, SID_X, (B, 64, 2, 1), 40.0, -128, 127),
        labels=uniform_int(seed, SID_LABELS, (B,), 0, 1, dtype=np.int32),
        layers=layers,
        tmc=uniform_int(seed, 40, (2,), 60, 100),
        tmw=uniform_int(seed, 41, (2,), -100, -60),
    )


# Adaptive-precision workload: the weight-layer sizes of a CIFAR ResNet-20
# (the network the adaptive precision page trains): a 3x3 conv 3 -> 16, six
# 3x3 convs 16 -> 16, one 16 -> 32 and five 32 -> 32, one 32 -> 64 and five
# 64 -> 64, and the 64 -> 10 classifier: 20 layers, 268,336 weights.
RESNET20_SIZES = ([16 * 3 * 9] + [16 * 16 * 9] * 6 + [32 * 16 * 9] + [32 * 32 * 9] * 5
                  + [64 * 32 * 9] + [64 * 64 * 9] * 5 + [10 * 64])
SID_APT_W = 50          # + layer
SID_APT_E = 120         # + layer: initial weight exponents
SID_APT_G = 1 << 16     # + running gradient index


def apt_weights(sizes=RESNET20_SIZES, k0=6, seed=0):
    """Initial k0-bit weight mantissas per layer, round(N(0, 2^(k0-1) / 3))
    clipped to the k0-bit range, and an exponent per layer ~ U{-12..-6}."""
    lim = 1 << (k0 - 1)
    Ws = [normal_int(seed, SID_APT_W + l, (n,), lim / 3.0, -lim, lim - 1, dtype=np.int16)
          for l, n in enumerate(sizes)]
    es = [int(uniform_int(seed, SID_APT_E + l, (1,), -12, -6, dtype=np.int32)[0])
          for l in range(len(sizes))]
    return Ws, es


def apt_grad(index, n, sigma, seed=0):
    """int16 gradient mantissas round(N(0, sigma)) clipped to the int16 range;
    `index` numbers the draw (step and layer)."""
    return normal_int(seed, SID_APT_G + int(index), (n,), float(sigma), -32768, 32767, dtype=np.int16)
