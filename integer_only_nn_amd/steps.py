"""Training steps as sequences of libionn calls on one stream.

Nothing here computes: each function allocates device buffers (PyTorch is
the allocator) and enqueues the library's kernels in the order the method
gives.  Shift values stay on the device; they are read back only when a
caller asks for them.

Order of a step ("Integer On-Device Training: Overview", sections 3, 4, 6.2):
forward (activations requantised with a dynamic NITI shift), the user loss
writes the output delta, then the backward pass per layer from the last:
delta propagation with the pre-update weights (ReLU mask, requantised to
target_bits = 7) and the weight gradient followed by the NITI update.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import ops

TB_WEIGHT = 8
MU_WEIGHT = 2
TB_DELTA = 7


def _i32(*shape, device):
    return torch.empty(shape, dtype=torch.int32, device=device)


def _i8(*shape, device):
    return torch.empty(shape, dtype=torch.int8, device=device)


# ---------------------------------------------------------------------------
# Single linear layer.
# ---------------------------------------------------------------------------

@dataclass
class LinearStepBuffers:
    """Device buffers of one linear-layer step (allocated once, reused).

    scal, int32[16]: [0:3] the max |Y|, |dX|, |G| of the last step, [3] the
    delta's shift, [4:6] the update's s, ws; [8:11] and [12:15] the two sets
    the maxima are max-combined into when steps alternate (alternate=True):
    each step's update clears the set the next step uses, so no fill kernel
    runs per step; the maxima of the step just taken are then in set
    `maxima()`."""
    Y: torch.Tensor
    dX: torch.Tensor
    G: torch.Tensor
    delta: torch.Tensor
    scal: torch.Tensor
    gq: Optional[torch.Tensor] = None
    alternate: bool = False
    phase: int = 0

    @staticmethod
    def make(B, IN, OUT, device, with_gq=False, alternate=False):
        return LinearStepBuffers(_i32(B, OUT, device=device), _i32(B, IN, device=device),
                                 _i32(OUT, IN, device=device), _i8(B, IN, device=device),
                                 torch.zeros(16, dtype=torch.int32, device=device),
                                 _i32(OUT, IN, device=device) if with_gq else None, alternate)

    def maxima(self):
        """The max |Y|, |dX|, |G| scalars of the last step (device view)."""
        if not self.alternate:
            return self.scal[0:3]
        o = 8 if self.phase == 1 else 12
        return self.scal[o:o + 3]


def linear_step(X, W, dY, buf: LinearStepBuffers, requant_delta=True, tb_w=TB_WEIGHT,
                mu=MU_WEIGHT, tb_d=TB_DELTA, stream=None):
    """fwd (int32 Y + max) -> dgrad (int32 dX + max) [-> delta, 7 bits] ->
    wgrad (int32 G + max) -> NITI update of W in place.  With
    buf.alternate the maxima go to one of two scalar sets and the update
    clears the other, instead of a fill before the step (a captured HIP
    graph must then hold an even number of steps)."""
    s = buf.scal
    if buf.alternate:
        m = s[8:11] if buf.phase == 0 else s[12:15]
        nxt = s[12:15] if buf.phase == 0 else s[8:11]
        buf.phase ^= 1
    else:
        m, nxt = s[0:3], None
        ops.ionn_fill_u32(m, 0, stream=stream)
    ops.int_linear_fwd(X, W, buf.Y, absmax_Y=m[0:1], stream=stream)
    ops.int_linear_dgrad(dY, W, buf.dX, absmax_dX=m[1:2], stream=stream)
    if requant_delta:
        ops.niti_quantize(buf.dX, m[1:2], tb_d, False, buf.delta, shift_out=s[3:4], stream=stream)
    ops.int_linear_wgrad(dY, X, buf.G, absmax_G=m[2:3], stream=stream)
    if nxt is None:
        ops.niti_quantize_update(buf.G, m[2:3], tb_w, mu, W, shifts_out=s[4:6], gq_out=buf.gq,
                                 stream=stream)
    else:
        ops.niti_quantize_update_clear(buf.G, m[2:3], tb_w, mu, W, nxt, shifts_out=s[4:6], gq_out=buf.gq,
                                       stream=stream)


def linear_step_small(X, W, dY, buf: LinearStepBuffers, tb_w=TB_WEIGHT, mu=MU_WEIGHT, tb_d=TB_DELTA,
                      stream=None):
    """The same step as linear_step (with the delta requantised) in one
    launch, for layers that int_linear_step_small_fits takes: the maxima go
    to buf.scal[0:3] (written, not combined) and the shifts s_d, s, ws to
    buf.scal[3:6]."""
    s = buf.scal
    ops.int_linear_step_small(X, W, dY, tb_w, mu, tb_d, buf.Y, buf.dX, buf.delta, buf.G, s[0:3], s[3:6],
                              gq=buf.gq, stream=stream)


# ---------------------------------------------------------------------------
# Multi-layer perceptron (all layers trainable).
# ---------------------------------------------------------------------------

@dataclass
class MLP:
    Ws: List[torch.Tensor]
    relu: List[bool]
    B: int
    acts: List[torch.Tensor] = field(default_factory=list)
    z32: List[torch.Tensor] = field(default_factory=list)
    d32: List[torch.Tensor] = field(default_factory=list)
    deltas: List[torch.Tensor] = field(default_factory=list)
    G: List[torch.Tensor] = field(default_factory=list)
    Gq: Optional[List[torch.Tensor]] = None   # with_gq: each layer's Gq of the last step
    e32: Optional[torch.Tensor] = None
    # per step: [fwd max x L | err max | dgrad max x L | G max x L] (uint32)
    # and shifts [fwd s x L | err s | dgrad s x L | (s, ws) x L]
    maxes: Optional[torch.Tensor] = None
    shifts: Optional[torch.Tensor] = None

    @staticmethod
    def make(Ws, B, relu=None, with_gq=False):
        L = len(Ws)
        dev = Ws[0].device
        m = MLP(list(Ws), relu if relu is not None else [l < L - 1 for l in range(L)], B)
        if with_gq:
            m.Gq = [_i32(*w.shape, device=dev) for w in Ws]
        sizes = [Ws[0].shape[1]] + [w.shape[0] for w in Ws]
        m.acts = [None] + [_i8(B, sizes[l + 1], device=dev) for l in range(L)]
        m.z32 = [_i32(B, sizes[l + 1], device=dev) for l in range(L)]
        m.d32 = [_i32(B, sizes[l], device=dev) for l in range(L)]
        m.deltas = [_i8(B, sizes[l], device=dev) for l in range(L + 1)]
        m.G = [_i32(*w.shape, device=dev) for w in Ws]
        m.e32 = _i32(B, sizes[-1], device=dev)
        m.maxes = torch.zeros(3 * L + 1, dtype=torch.int32, device=dev)
        m.shifts = torch.zeros(4 * L + 1, dtype=torch.int32, device=dev)
        return m

    def step(self, X, labels, target_mag=127, tb_w=TB_WEIGHT, mu=MU_WEIGHT, tb_a=TB_DELTA,
             tb_d=TB_DELTA, stream=None):
        L = len(self.Ws)
        mx, sh = self.maxes, self.shifts
        ops.ionn_fill_u32(mx, 0, stream=stream)
        self.acts[0] = X
        for l in range(L):
            ops.int_linear_fwd(self.acts[l], self.Ws[l], self.z32[l], absmax_Y=mx[l:l + 1],
                               stream=stream)
            ops.niti_quantize(self.z32[l], mx[l:l + 1], tb_a, self.relu[l], self.acts[l + 1],
                              shift_out=sh[l:l + 1], stream=stream)
        ops.int_output_error(self.acts[L], labels, target_mag, self.e32, absmax_e=mx[L:L + 1],
                             stream=stream)
        ops.niti_quantize(self.e32, mx[L:L + 1], tb_d, False, self.deltas[L],
                          shift_out=sh[L:L + 1], stream=stream)
        for l in range(L - 1, -1, -1):
            mask = self.acts[l] if (l >= 1 and self.relu[l - 1]) else None
            dm = mx[L + 1 + l:L + 2 + l]
            ops.int_linear_dgrad(self.deltas[l + 1], self.Ws[l], self.d32[l], relu_act=mask,
                                 absmax_dX=dm, stream=stream)
            ops.niti_quantize(self.d32[l], dm, tb_d, False, self.deltas[l],
                              shift_out=sh[L + 1 + l:L + 2 + l], stream=stream)
            gm = mx[2 * L + 1 + l:2 * L + 2 + l]
            ops.int_linear_wgrad(self.deltas[l + 1], self.acts[l], self.G[l], absmax_G=gm,
                                 stream=stream)
            ops.niti_quantize_update(self.G[l], gm, tb_w, mu, self.Ws[l],
                                     shifts_out=sh[2 * L + 1 + 2 * l:2 * L + 3 + 2 * l],
                                     gq_out=self.Gq[l] if self.Gq is not None else None,
                                     stream=stream)

    def shift_record(self):
        """Host copy of the last step's shifts in the oracle's record layout."""
        L = len(self.Ws)
        s = self.shifts.cpu().tolist()
        return dict(s_fwd=s[:L], s_err=s[L], s_dgrad=s[L + 1:2 * L + 1],
                    s_upd=[(s[2 * L + 1 + 2 * l], s[2 * L + 2 + 2 * l]) for l in range(L)])


# ---------------------------------------------------------------------------
# 3x3 conv layer.
# ---------------------------------------------------------------------------

@dataclass
class ConvStepBuffers:
    """Device buffers of one 3x3 conv step.

    scal, int32[16]: [0:3] the max |Y|, |dX|, |G|, [3] s_y, [4] s_dx,
    [5:7] the update's s, ws; [8:11] and [12:15] the two sets the maxima are
    max-combined into when steps alternate (alternate=True): each step's
    update clears the set the next step uses, so no fill kernel runs per
    step; the maxima of the step just taken are then in set `maxima()`."""
    Y: torch.Tensor
    y8: torch.Tensor
    dX: torch.Tensor
    dx8: torch.Tensor
    G: torch.Tensor
    scal: torch.Tensor
    gq: Optional[torch.Tensor] = None
    ws: Optional[torch.Tensor] = None   # weight-gradient workspace (None: no fast path)
    rws: Optional[torch.Tensor] = None  # one-pass requantisation workspace (None: two passes)
    alternate: bool = False
    phase: int = 0

    @staticmethod
    def make(N, H, W, Cin, Cout, device, with_gq=False, one_pass=True, alternate=False):
        d = ops.conv_desc(N, H, W, Cin, Cout)
        wsb = ops.int_conv_wgrad_workspace_bytes(d)
        rwb = ops.int_conv_requant_workspace_bytes(d) if one_pass else 0
        return ConvStepBuffers(_i32(N, H, W, Cout, device=device), _i8(N, H, W, Cout, device=device),
                               _i32(N, H, W, Cin, device=device), _i8(N, H, W, Cin, device=device),
                               _i32(Cout, 3, 3, Cin, device=device),
                               torch.zeros(16, dtype=torch.int32, device=device),
                               _i32(Cout, 3, 3, Cin, device=device) if with_gq else None,
                               torch.empty(wsb, dtype=torch.uint8, device=device) if wsb else None,
                               torch.empty(rwb, dtype=torch.uint8, device=device) if rwb else None,
                               alternate)

    def maxima(self):
        """The max |Y|, |dX|, |G| scalars of the last step (device view)."""
        if not self.alternate:
            return self.scal[0:3]
        o = 8 if self.phase == 1 else 12
        return self.scal[o:o + 3]

    def _sets(self, stream):
        """The maxima of this step and the set the update clears (None: a
        fill kernel cleared this step's set)."""
        s = self.scal
        if not self.alternate:
            ops.ionn_fill_u32(s[0:3], 0, stream=stream)
            return s[0:3], None
        m = s[8:11] if self.phase == 0 else s[12:15]
        nxt = s[12:15] if self.phase == 0 else s[8:11]
        self.phase ^= 1
        return m, nxt


def _conv_update(buf, m, nxt, tb_w, mu, Wt, stream):
    s = buf.scal
    if nxt is None:
        ops.niti_quantize_update(buf.G, m[2:3], tb_w, mu, Wt, shifts_out=s[5:7], gq_out=buf.gq, stream=stream)
    else:
        ops.niti_quantize_update_clear(buf.G, m[2:3], tb_w, mu, Wt, nxt, shifts_out=s[5:7], gq_out=buf.gq,
                                       stream=stream)


def conv_step(X, Wt, dY, buf: ConvStepBuffers, tb_a=TB_DELTA, tb_d=TB_DELTA, tb_w=TB_WEIGHT,
              mu=MU_WEIGHT, stream=None):
    N, H, W_, Cin = X.shape
    Cout = Wt.shape[0]
    d = ops.conv_desc(N, H, W_, Cin, Cout)
    s = buf.scal
    m, nxt = buf._sets(stream)
    ops.int_conv_fwd(X, Wt, buf.Y, d, absmax_Y=m[0:1], stream=stream)
    ops.niti_quantize(buf.Y, m[0:1], tb_a, False, buf.y8, shift_out=s[3:4], stream=stream)
    ops.int_conv_dgrad(dY, Wt, buf.dX, d, absmax_dX=m[1:2], stream=stream)
    ops.niti_quantize(buf.dX, m[1:2], tb_d, False, buf.dx8, shift_out=s[4:5], stream=stream)
    ops.int_conv_wgrad(dY, X, buf.G, d, absmax_G=m[2:3], workspace=buf.ws, stream=stream)
    _conv_update(buf, m, nxt, tb_w, mu, Wt, stream)


def conv_step_fused(X, Wt, dY, buf: ConvStepBuffers, tb_a=TB_DELTA, tb_d=TB_DELTA, tb_w=TB_WEIGHT,
                    mu=MU_WEIGHT, stream=None):
    """The same step with the requantisation fused into the contractions
    (64 -> 64 channels): y8, dx8, G, the update and every shift as in
    conv_step; buf.Y and buf.dX are not written (the int32 sums are never
    stored).  With buf.rws each requantising contraction is one pass plus a
    streaming pass over its int8 output, else two contraction passes.  With
    buf.alternate no fill kernel runs (a captured HIP graph must then hold
    an even number of steps)."""
    N, H, W_, Cin = X.shape
    Cout = Wt.shape[0]
    d = ops.conv_desc(N, H, W_, Cin, Cout)
    s = buf.scal
    m, nxt = buf._sets(stream)
    ops.int_conv_fwd_requant(X, Wt, buf.y8, d, tb_a, False, m[0:1], shift_out=s[3:4], workspace=buf.rws,
                             stream=stream)
    ops.int_conv_dgrad_requant(dY, Wt, buf.dx8, d, tb_d, m[1:2], shift_out=s[4:5], workspace=buf.rws,
                               stream=stream)
    ops.int_conv_wgrad(dY, X, buf.G, d, absmax_G=m[2:3], workspace=buf.ws, stream=stream)
    _conv_update(buf, m, nxt, tb_w, mu, Wt, stream)


# ---------------------------------------------------------------------------
# DFP-16 layer.
# ---------------------------------------------------------------------------

@dataclass
class DfpStepBuffers:
    Y: torch.Tensor
    dX: torch.Tensor
    G: torch.Tensor
    ws: torch.Tensor          # one workspace, reused by the three contractions
    exps: torch.Tensor        # int32[8]: eY, edX, eG, status x3
    gavg: torch.Tensor        # float64[1]

    @staticmethod
    def make(M, K, N, device):
        wsb = max(ops.dfp16_workspace_bytes(M, K, N, w) for w in range(3))
        return DfpStepBuffers(torch.empty(M, N, dtype=torch.int16, device=device),
                              torch.empty(M, K, dtype=torch.int16, device=device),
                              torch.empty(N, K, dtype=torch.int16, device=device),
                              torch.empty(wsb, dtype=torch.uint8, device=device),
                              torch.zeros(8, dtype=torch.int32, device=device),
                              torch.zeros(1, dtype=torch.float64, device=device))


def dfp16_step(X, eX, W, eW, dY, edY, buf: DfpStepBuffers, stream=None):
    """eX, eW, edY: device int32[1] exponents."""
    e = buf.exps
    ops.dfp16_gemm_fwd(X, eX, W, eW, buf.Y, e[0:1], buf.ws, status_out=e[3:4], stream=stream)
    ops.dfp16_gemm_dgrad(dY, edY, W, eW, buf.dX, e[1:2], buf.ws, status_out=e[4:5], stream=stream)
    ops.dfp16_gemm_wgrad(dY, edY, X, eX, buf.G, e[2:3], buf.ws, status_out=e[5:6], stream=stream)
    ops.dfp16_gavg(buf.G, e[2:3], eW, buf.gavg, stream=stream)


# ---------------------------------------------------------------------------
# Model-level driver (ionn_model_forward / ionn_model_backward).
# ---------------------------------------------------------------------------

class Model:
    """Device copy of a layer list and the driver's workspace.  Layers are
    dicts: kind "conv" or "linear", relu, geometry (conv: H, W, Cin, Cout, KH,
    KW, pad; linear: IN, OUT) and host arrays weight, offset, mult, k."""

    def __init__(self, layers, B, device):
        self.B = B
        self.dev = []
        for L in layers:
            conv = L["kind"] == "conv"
            t = (0 if conv else 2) + (1 if L["relu"] else 0)
            geo = dict(H=L["H"], W=L["W"], Cin=L["Cin"], Cout=L["Cout"], KH=L["KH"], KW=L["KW"], pad=L["pad"]) \
                if conv else dict(H=1, W=1, Cin=L["IN"], Cout=L["OUT"])
            self.dev.append(dict(type=t, **geo,
                                 weight=torch.from_numpy(L["weight"].copy()).to(device),
                                 offset=torch.from_numpy(L["offset"].copy()).to(device),
                                 mult=torch.from_numpy(L["mult"].copy()).to(device),
                                 k=torch.from_numpy(L["k"].copy()).to(device)))
        self.larr = ops.layer_array(self.dev)
        n = ops.ionn_model_workspace_bytes(self.larr, B)
        self.ws = torch.empty(n, dtype=torch.uint8, device=device)
        self.shifts = torch.zeros(1 + 5 * len(layers), dtype=torch.int32, device=device)
        last = self.dev[-1]
        n_out = last["Cout"]
        if last["type"] < 2:
            n_out *= (last["H"] + 2 * last["pad"] - last["KH"] + 1) * (last["W"] + 2 * last["pad"] - last["KW"] + 1)
        self.out = torch.empty(B, n_out, dtype=torch.int8, device=device)

    def forward(self, X, stream=None):
        ops.ionn_model_forward(self.larr, X, self.ws, out=self.out, stream=stream)

    def backward(self, X, labels, tmc, tmw, stream=None):
        ops.ionn_model_backward(self.larr, X, labels, tmc, tmw, self.ws, shifts_out=self.shifts, stream=stream)

    def step(self, X, labels, tmc, tmw, stream=None):
        self.forward(X, stream=stream)
        self.backward(X, labels, tmc, tmw, stream=stream)


# ---------------------------------------------------------------------------
# Adaptive per-layer precision (apt_update / apt_adjust).
# ---------------------------------------------------------------------------

class AptLayers:
    """Device state of adaptive per-layer precision over L int16 weight
    tensors: their precisions k, weight exponents e_w and the epoch's Gavg
    sums and counts, plus the workspace a sampling step needs.  The host
    never reads the state back unless asked to.  The ctypes argument arrays
    are built once (bind_grads for the gradient buffers), so a step costs
    one library call."""

    def __init__(self, Ws, ks, es, device, int8_layers=()):
        """int8_layers: indices of layers held in int8 (their k must be at
        most 8 and stays there: half the memory of int16)."""
        self.W = []
        for l, w in enumerate(Ws):
            if l in int8_layers:
                if int(ks[l]) > 8 or w.min(initial=0) < -128 or w.max(initial=0) > 127:
                    raise ValueError(f"layer {l}: int8 storage needs k <= 8 and mantissas in [-128, 127]")
                w = w.astype(np.int8)
            self.W.append(torch.from_numpy(np.ascontiguousarray(w).copy()).to(device))
        L = len(self.W)
        self._mixed = bool(int8_layers)
        self.k = torch.tensor(list(ks), dtype=torch.int32, device=device)
        self.e_w = torch.tensor(list(es), dtype=torch.int32, device=device)
        self.gsum = torch.zeros(L, dtype=torch.float64, device=device)
        self.gcnt = torch.zeros(L, dtype=torch.int32, device=device)
        self.dk = torch.zeros(L, dtype=torch.int32, device=device)
        self.ws = torch.empty(max(ops.apt_workspace_bytes([w.numel() for w in self.W]), 8),
                              dtype=torch.uint8, device=device)
        self._Wp = ops._ptr_array(self.W, None, "W")
        self._wb = ops._wbytes(self.W)
        self._n = ops._sizes(self.W)
        self._G = None

    def bind_grads(self, Gs):
        """Fix the gradient buffers (int16 device tensors, one per layer) that
        step() reads when it is given none."""
        if len(Gs) != len(self.W) or any(g.numel() != w.numel() for g, w in zip(Gs, self.W)):
            raise ValueError("one gradient per layer, of the layer's size")
        self._G = (list(Gs), ops._ptr_array(Gs, torch.int16, "G"))

    def step(self, Gs, e_g, lr_shift, sample=False, stream=None):
        """One update of every layer with gradients Gs (int16 device tensors;
        None: the bound buffers) and their exponents e_g (int32 device [L])."""
        if Gs is not None:
            self.bind_grads(Gs)
        if self._G is None:
            raise ValueError("no gradient buffers")
        L = len(self.W)
        args = (self._G[1], self._n, ops._p(self.k), ops._p(self.e_w), ops._p(e_g, torch.int32, L, "e_g"),
                int(lr_shift), ops._p(self.gsum) if sample else None, ops._p(self.gcnt) if sample else None,
                ops._p(self.ws) if sample else None, self.ws.numel() if sample else 0, ops._stream(stream))
        if self._mixed:
            ops.check(ops.lib().apt_update_mixed(L, self._Wp, self._wb, *args), "apt_update_mixed")
        else:
            ops.check(ops.lib().apt_update(L, self._Wp, *args), "apt_update")

    def end_epoch(self, t_min, t_max, k_min=2, k_max=16, stream=None):
        L = len(self.W)
        args = (self._n, ops._p(self.k), ops._p(self.e_w), ops._p(self.gsum), ops._p(self.gcnt), float(t_min),
                float(t_max), int(k_min), int(k_max), ops._p(self.dk), ops._stream(stream))
        if self._mixed:
            ops.check(ops.lib().apt_adjust_mixed(L, self._Wp, self._wb, *args), "apt_adjust_mixed")
        else:
            ops.check(ops.lib().apt_adjust(L, self._Wp, *args), "apt_adjust")
