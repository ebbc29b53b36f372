"""Whole training steps composed from the oracle's C primitives.

TEST INFRASTRUCTURE ONLY.  Each function is the sequence of operations that a
step performs, in the order the method gives; every arithmetic operation runs
in ``ionn_oracle.c``.

Sources: "Integer On-Device Training: Overview" (TI), section 3 "The NITI
Algorithm" (update rule, delta propagation with target_bits = 7), section 4
(forward fills the activation buffer and ReLU mask; the backward pass reads the
loss delta and updates the weights) and section 6.2 (device training loop:
forward, user loss, backward); "Mixed Precision Training of CNNs using Integer
Operations", sections 3.1 and 4 (DFP primitives, chunked accumulation);
"Adaptive Precision Training for Resource Constrained Devices" (Gavg).
"""
import numpy as np

from . import (bias_grad, conv_dgrad, conv_fwd, conv_wgrad, dfp16_dgrad, dfp16_fwd, dfp16_wgrad,
               gavg, linear_dgrad, linear_fwd, linear_wgrad, niti_requant, niti_update,
               niti_update_i32, oss_requant, output_error, mse_grad_targets, relu_mask)

# Readings: weight-update target_bits = 8 and mu_weight = 2 for every layer
# (U8); propagated deltas and requantised activations use target_bits = 7.
TB_WEIGHT = 8
MU_WEIGHT = 2
TB_DELTA = 7


def linear_step(X, W, dY, tb_w=TB_WEIGHT, mu=MU_WEIGHT, tb_d=TB_DELTA):
    """One NITI step of a single linear layer given its incoming delta dY.

    Returns a dict with the int32 forward output, the int32 dgrad, the
    propagated int8 delta and its shift, the int32 weight gradient, Gq, the
    updated weights and the two update shifts.
    """
    Y32 = linear_fwd(X, W)
    dX32 = linear_dgrad(dY, W)          # with the pre-update weights
    delta, s_d = niti_requant(dX32, tb_d)
    G = linear_wgrad(dY, X)
    W_new, Gq, s, ws = niti_update(G, W, tb_w, mu)
    return dict(Y32=Y32, dX32=dX32, delta=delta, s_d=s_d, G=G, Gq=Gq, W_new=W_new, s=s, ws=ws)


def mlp_step(X, labels, Ws, relu_layers=None, target_mag=127, tb_w=TB_WEIGHT, mu=MU_WEIGHT,
             tb_a=TB_DELTA, tb_d=TB_DELTA):
    """One training step of an L-layer int8 MLP (all layers trainable).

    Forward: a_l = requant(a_{l-1} W_l^T, tb_a) with ReLU on every layer but
    the logits layer (reading U10).  Error: e = onehot*target_mag - a_L,
    requantised to tb_d bits.  Backward, l = L..1: dgrad with the pre-update
    W_l, masked by a_{l-1} > 0 when layer l-1 has a ReLU, requantised to
    tb_d bits (delta_0 of the input too, reading U11); wgrad
    G_l = delta_l^T a_{l-1}; NITI update of W_l.

    Returns (new weights list, record dict of every shift and tensor).
    """
    L = len(Ws)
    if relu_layers is None:
        relu_layers = [l < L - 1 for l in range(L)]
    acts = [X]
    s_fwd = []
    for l in range(L):
        z = linear_fwd(acts[-1], Ws[l])
        a, s = niti_requant(z, tb_a, relu=relu_layers[l])
        acts.append(a)
        s_fwd.append(s)
    e32 = output_error(acts[-1], labels, target_mag)
    delta, s_err = niti_requant(e32, tb_d)
    new_W = list(Ws)
    s_dgrad = [None] * L
    s_upd = [None] * L
    Gs = [None] * L
    Gqs = [None] * L
    deltas = [None] * (L + 1)
    deltas[L] = delta
    for l in range(L - 1, -1, -1):
        d32 = linear_dgrad(deltas[l + 1], Ws[l])
        if l >= 1 and relu_layers[l - 1]:
            d32 = relu_mask(d32, acts[l])
        deltas[l], s_dgrad[l] = niti_requant(d32, tb_d)
        Gs[l] = linear_wgrad(deltas[l + 1], acts[l])
        new_W[l], Gqs[l], s, ws = niti_update(Gs[l], Ws[l], tb_w, mu)
        s_upd[l] = (s, ws)
    rec = dict(acts=acts, s_fwd=s_fwd, e32=e32, s_err=s_err, deltas=deltas, s_dgrad=s_dgrad,
               s_upd=s_upd, G=Gs, Gq=Gqs)
    return new_W, rec


def mlp_train(X, labels, Ws, steps, **kw):
    """`steps` MLP steps on one fixed batch (reading U15); returns the final
    weights and the list of per-step records."""
    recs = []
    for _ in range(steps):
        Ws, rec = mlp_step(X, labels, Ws, **kw)
        recs.append(rec)
    return Ws, recs


def conv_step(X, W, dY, P=1, tb_a=TB_DELTA, tb_d=TB_DELTA, tb_w=TB_WEIGHT, mu=MU_WEIGHT):
    """One NITI step of a stride-1 conv layer: forward with requantised output
    activations, dgrad with a requantised propagated delta, wgrad and update."""
    Y32 = conv_fwd(X, W, P)
    y8, s_y = niti_requant(Y32, tb_a)
    dX32 = conv_dgrad(dY, W, X.shape, P)
    dx8, s_dx = niti_requant(dX32, tb_d)
    G = conv_wgrad(dY, X, W.shape[1], W.shape[2], P)
    W_new, Gq, s, ws = niti_update(G, W, tb_w, mu)
    return dict(Y32=Y32, y8=y8, s_y=s_y, dX32=dX32, dx8=dx8, s_dx=s_dx, G=G, Gq=Gq, W_new=W_new,
                s=s, ws=ws)


def dfp16_step(X, eX, W, eW, dY, edY, chunk=64):
    """One DFP-16 layer step: forward, dgrad and wgrad contractions with
    chunked overflow management and down-conversion, then Gavg of the weight
    gradient against the weights' resolution."""
    Y, eY, accY = dfp16_fwd(X, eX, W, eW, chunk)
    dX, edX, accdX = dfp16_dgrad(dY, edY, W, eW, chunk)
    G, eG, accG = dfp16_wgrad(dY, edY, X, eX, chunk)
    return dict(Y=Y, eY=eY, accY=accY, dX=dX, edX=edX, accdX=accdX, G=G, eG=eG, accG=accG,
                gavg=gavg(G, eG, eW))


# ---------------------------------------------------------------------------
# Model-level driver: the INT_LAYERS forward and backward of the TI page
# (section 7: layer types Conv2D, Conv2D+ReLU, Linear, Linear+ReLU with int8
# weights, int32 offsets and OSS shifts/multipliers; section 8: the OSS chain
# and the per-class TARGET_MAG loss; section 3: NITI updates).  A layer is a
# dict: kind "conv" or "linear", relu, for conv KH, KW, pad and the input
# geometry H, W, Cin, Cout; for linear IN, OUT; and the parameters weight
# (int8), offset (int32), mult (int32), k (int8).
# Readings U26-U28 of the design notes.
# ---------------------------------------------------------------------------

def _as_rows(a, L):
    """Activation a of a layer's input, as the layer reads it."""
    if L["kind"] == "conv":
        return a.reshape(-1, L["H"], L["W"], L["Cin"])
    return a.reshape(a.shape[0], -1)


def model_forward(layers, X):
    """a_l = OSS(contraction(a_{l-1}, W_l); offset_l, mult_l, k_l, relu_l).
    Returns the activations [X, a_1, ..., a_L] (int8, conv outputs NHWC)."""
    acts = [X]
    for L in layers:
        a = _as_rows(acts[-1], L)
        if L["kind"] == "conv":
            z = conv_fwd(a, L["weight"], L["pad"])
        else:
            z = linear_fwd(a, L["weight"])
        C = z.shape[-1]
        y = oss_requant(z.reshape(-1, C), L["offset"], L["mult"], L["k"], relu=L["relu"])
        acts.append(y.reshape(z.shape))
    return acts


def model_step(layers, X, labels, tmc, tmw, tb_d=TB_DELTA, tb_w=TB_WEIGHT, mu=MU_WEIGHT):
    """One training step of the model (forward, the MSE gradient against the
    per-class targets, backward with updates of every layer's W and offsets).

    Backward, l = L..1, with delta_L = requant(out - target, tb_d):
      gb_l = column sums of delta_l (rows: batch, times pixels for conv);
      G_l = wgrad(delta_l, a_{l-1});
      for l > 1: d = dgrad(delta_l, W_l) with the pre-update W_l, masked by
        a_{l-1} > 0 when layer l-1 has a ReLU, delta_{l-1} = requant(d, tb_d);
      W_l = NITI update(G_l), offset_l = NITI int32 update(gb_l).
    The first layer's input gradient is not formed: nothing consumes it.
    Returns (new layers, record of tensors and shifts)."""
    acts = model_forward(layers, X)
    e32 = mse_grad_targets(acts[-1].reshape(acts[-1].shape[0], -1), labels, tmc, tmw)
    delta, s_err = niti_requant(e32, tb_d)
    new = [dict(L) for L in layers]
    rec = dict(acts=acts, e32=e32, s_err=s_err, deltas={len(layers): delta}, s_dgrad={}, s_w={},
               s_b={}, G={}, gb={})
    for l in range(len(layers) - 1, -1, -1):
        L = layers[l]
        a_in = _as_rows(acts[l], L)
        if L["kind"] == "conv":
            Ho = L["H"] + 2 * L["pad"] - L["KH"] + 1
            Wo = L["W"] + 2 * L["pad"] - L["KW"] + 1
            d_out = delta.reshape(-1, Ho, Wo, L["Cout"])
            G = conv_wgrad(d_out, a_in, L["KH"], L["KW"], L["pad"])
        else:
            d_out = delta.reshape(delta.shape[0], -1)
            G = linear_wgrad(d_out, a_in)
        gb = bias_grad(d_out.reshape(-1, d_out.shape[-1]))
        rec["G"][l], rec["gb"][l] = G, gb
        if l > 0:
            if L["kind"] == "conv":
                d32 = conv_dgrad(d_out, L["weight"], a_in.shape, L["pad"])
            else:
                d32 = linear_dgrad(d_out, L["weight"])
            if layers[l - 1]["relu"]:
                d32 = relu_mask(d32, a_in)
            delta, rec["s_dgrad"][l] = niti_requant(d32, tb_d)
            rec["deltas"][l] = delta
        new[l]["weight"], _, s, ws = niti_update(G, L["weight"], tb_w, mu)
        rec["s_w"][l] = (s, ws)
        new[l]["offset"], _, s, ws = niti_update_i32(gb, L["offset"], tb_w, mu)
        rec["s_b"][l] = (s, ws)
    return new, rec


def arc_fault_layers(d):
    """The arc-fault example network (ionn_synth.arc_fault) as model layers."""
    prm = [dict(weight=q["W"], offset=q["offset"], mult=q["mult"], k=q["k"]) for q in d["layers"]]
    return [
        dict(kind="conv", relu=True, H=64, W=2, Cin=1, Cout=3, KH=16, KW=2, pad=0, **prm[0]),
        dict(kind="linear", relu=True, IN=147, OUT=160, **prm[1]),
        dict(kind="linear", relu=False, IN=160, OUT=2, **prm[2]),
    ]
