"""Adaptive precision training workflow ("Adaptive Precision Training for
Resource Constrained Devices", Algorithm 2 around Algorithm 1) over the
oracle's per-layer steps -- TEST INFRASTRUCTURE ONLY.

Every layer holds k-bit weight mantissas W (int16 storage), its precision k
and its weight exponent e_w (one grid step eps = 2^e_w).  Within an epoch
each step updates every layer with its gradient (reading U30), and on the
sampling steps the layer's Gavg (Equation 4) is added to the epoch's sum.
Between epochs Algorithm 1 moves each layer's k by at most one bit on the
mean of those samples and rescales the weights to the new grid (U33).
"""
from . import apt_decide, apt_rescale, apt_update, gavg


def new_state(Ws, ks, es):
    return [dict(W=W.copy(), k=int(k), e_w=int(e)) for W, k, e in zip(Ws, ks, es)]


def step(state, grads, lr_shift, sums=None, counts=None):
    """One training step's updates.  grads[l] = (G int16, e_g).  When `sums`
    is given the step is a sampling step: Gavg of every layer is added to
    sums[l] (one double addition, in step order) and counts[l] grows by 1.
    Returns the underflow count per layer."""
    under = []
    for l, (s, (G, e_g)) in enumerate(zip(state, grads)):
        if sums is not None:
            sums[l] = sums[l] + gavg(G, e_g, s["e_w"])
            counts[l] += 1
        s["W"], u = apt_update(s["W"], s["k"], s["e_w"], G, e_g, lr_shift)
        under.append(u)
    return under


def adjust(state, sums, counts, t_min, t_max, k_min, k_max):
    """Algorithm 1 for every layer, then the rescale; resets the sums.
    Returns the per-layer change of k."""
    dks = []
    for l, s in enumerate(state):
        dk = apt_decide(sums[l], counts[l], s["k"], t_min, t_max, k_min, k_max)
        if dk:
            s["W"] = apt_rescale(s["W"], s["k"], dk)
            s["k"] += dk
            s["e_w"] -= dk
        dks.append(dk)
        sums[l] = 0.0
        counts[l] = 0
    return dks


def run(state, grad_fn, epochs, steps, eval_every, lr_shift, t_min, t_max, k_min=2, k_max=16):
    """Algorithm 2: `epochs` epochs of `steps` steps; the steps with
    step % eval_every == 0 sample Gavg; the precision moves between epochs.
    grad_fn(epoch, step, l, state) -> (G, e_g).  Returns a per-epoch history
    of (k, e_w, dk, sums, counts)."""
    L = len(state)
    hist = []
    for ep in range(epochs):
        sums, counts = [0.0] * L, [0] * L
        for st in range(steps):
            grads = [grad_fn(ep, st, l, state) for l in range(L)]
            sample = st % eval_every == 0
            step(state, grads, lr_shift, sums if sample else None, counts if sample else None)
        rec = dict(sums=list(sums), counts=list(counts))
        rec["dk"] = adjust(state, sums, counts, t_min, t_max, k_min, k_max)
        rec["k"] = [s["k"] for s in state]
        rec["e_w"] = [s["e_w"] for s in state]
        hist.append(rec)
    return hist
