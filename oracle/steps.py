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

from . import (conv_dgrad, conv_fwd, conv_wgrad, dfp16_dgrad, dfp16_fwd, dfp16_wgrad, gavg,
               linear_dgrad, linear_fwd, linear_wgrad, niti_requant, niti_update, output_error,
               relu_mask)

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
    deltas = [None] * (L + 1)
    deltas[L] = delta
    for l in range(L - 1, -1, -1):
        d32 = linear_dgrad(deltas[l + 1], Ws[l])
        if l >= 1 and relu_layers[l - 1]:
            d32 = relu_mask(d32, acts[l])
        deltas[l], s_dgrad[l] = niti_requant(d32, tb_d)
        G = linear_wgrad(deltas[l + 1], acts[l])
        new_W[l], _, s, ws = niti_update(G, Ws[l], tb_w, mu)
        s_upd[l] = (s, ws)
    rec = dict(acts=acts, s_fwd=s_fwd, e32=e32, s_err=s_err, deltas=deltas, s_dgrad=s_dgrad,
               s_upd=s_upd)
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
