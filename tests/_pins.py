"""Pins that tie the CPU oracle to things other than itself.

Each ``pin_*`` takes an oracle-like module (``forward``, ``backward``,
``dense_kl_loss``) and raises AssertionError when the module disagrees with
a closed form, a library routine, finite differences or an invariant of the
mathematics. ``tests/test_oracle_pins.py`` runs them on the real oracle and on
mutated copies of it (each mutant must fail at least one pin).
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special as sps
import scipy.stats as sst
import torch
import torch.nn.functional as F


def _rand_problem(rng, N, d, V, K, scale=1.0):
    H = rng.standard_normal((N, d)) * scale
    W = rng.standard_normal((V, d)) / math.sqrt(d)
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(N)])
    logits = rng.standard_normal((N, K)) * 1.7
    return H, W, ids, logits


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    tol = atol + rtol * (np.max(np.abs(b)) if b.size else 0.0)
    assert err <= tol, f"{what}: max|diff|={err:.3e} > tol={tol:.3e}"


# --- closed forms ----------------------------------------------------------

def pin_two_token_softplus(o):
    """V = 2, K = 1: KL_i = softplus((z_other - z_id) / T), written with
    explicit dot products; gradient from the derivative of softplus."""
    rng = np.random.default_rng(11)
    N, d, T, g = 4, 3, 1.7, 0.9
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((2, d))
    ids = np.array([[0], [1], [1], [0]])
    logits = rng.standard_normal((N, 1))
    kl = []
    dH = np.zeros((N, d))
    dW = np.zeros((2, d))
    for i in range(N):
        a = ids[i, 0]
        b = 1 - a
        za = sum(H[i, j] * W[a, j] for j in range(d))
        zb = sum(H[i, j] * W[b, j] for j in range(d))
        u = (zb - za) / T
        kl.append(math.log1p(math.exp(u)))
        sig = 1.0 / (1.0 + math.exp(-u))  # d softplus / du
        c = g / N * sig / T
        for j in range(d):
            dH[i, j] = c * (W[b, j] - W[a, j])
            dW[b, j] += c * H[i, j]
            dW[a, j] -= c * H[i, j]
    out = o.forward(H, W, ids, logits, T)
    _close(out["loss"], sum(kl) / N, 1e-13, what="two-token loss")
    _close(out["row_kl"], kl, 1e-13, what="two-token row_kl")
    gdH, gdW = o.backward(H, W, ids, logits, T, g)
    _close(gdH, dH, 1e-12, what="two-token dH")
    _close(gdW, dW, 1e-12, what="two-token dW")


def pin_uniform_student(o):
    """W = 0 makes the student uniform: KL_i = log V - entropy(p_i) with the
    entropy from scipy.stats; dH = 0 and dW_v = g/(N T) sum_i (1/V - P_iv) H_i."""
    rng = np.random.default_rng(12)
    N, d, V, K, T, g = 5, 4, 9, 3, 2.0, 1.3
    H, _, ids, logits = _rand_problem(rng, N, d, V, K)
    W = np.zeros((V, d))
    out = o.forward(H, W, ids, logits, T)
    ent = np.array([sst.entropy(np.exp(logits[i] / T)) for i in range(N)])
    _close(out["row_kl"], math.log(V) - ent, 1e-12, what="uniform row_kl")
    _close(out["row_lse"], np.full(N, math.log(V)), 1e-13, what="uniform lse")
    dH, dW = o.backward(H, W, ids, logits, T, g)
    assert np.all(dH == 0.0), "uniform student: dH must vanish when W = 0"
    P = np.zeros((N, V))
    for i in range(N):
        pi = sps.softmax(logits[i] / T)
        for k in range(K):
            P[i, ids[i, k]] += pi[k]
    ref = np.zeros((V, d))
    for v in range(V):
        for i in range(N):
            ref[v] += g / (N * T) * (1.0 / V - P[i, v]) * H[i]
    _close(dW, ref, 1e-12, what="uniform dW")


def pin_cross_entropy(o):
    """K = 1: the teacher is one-hot, so the loss is torch's cross-entropy of
    Z / T; gradients from torch autograd through that library routine."""
    rng = np.random.default_rng(13)
    N, d, V, T, g = 6, 5, 17, 1.5, 0.8
    H, W, ids, logits = _rand_problem(rng, N, d, V, 1)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    ce = F.cross_entropy(Ht @ Wt.T / T, torch.tensor(ids[:, 0]))
    (g * ce).backward()
    out = o.forward(H, W, ids, logits, T)
    _close(out["loss"], ce.item(), 1e-13, what="K=1 loss vs cross_entropy")
    dH, dW = o.backward(H, W, ids, logits, T, g)
    _close(dH, Ht.grad.numpy(), 1e-12, what="K=1 dH")
    _close(dW, Wt.grad.numpy(), 1e-12, what="K=1 dW")


def pin_dense_grid_libraries(o):
    """The pages' dense baseline (full teacher grid, zeros off the top-K)
    evaluated with library routines: scipy rel_entr and torch kl_div."""
    rng = np.random.default_rng(14)
    N, d, V, K, T = 5, 4, 13, 4, 1.5
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    P = np.zeros((N, V))
    for i in range(N):
        P[i, ids[i]] = sps.softmax(logits[i] / T)
    logQ = sps.log_softmax(H @ W.T / T, axis=1)
    ref1 = sps.rel_entr(P, np.exp(logQ)).sum() / N
    ref2 = F.kl_div(torch.tensor(logQ), torch.tensor(P), reduction="sum").item() / N
    _close(ref1, ref2, 1e-12, what="library cross-check")
    _close(o.forward(H, W, ids, logits, T)["loss"], ref1, 1e-12, what="loss vs rel_entr")
    _close(o.dense_kl_loss(H, W, ids, logits, T), ref1, 1e-12, what="dense grid vs rel_entr")


def pin_equality_case(o):
    """K = V and teacher logits equal to the student logits: KL = 0 and all
    gradients vanish, for any T."""
    rng = np.random.default_rng(15)
    N, d, V, T = 4, 3, 7, 1.7
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    ids = np.stack([rng.permutation(V) for _ in range(N)])
    Z = H @ W.T
    logits = np.take_along_axis(Z, ids, axis=1)
    out = o.forward(H, W, ids, logits, T)
    assert abs(out["loss"]) < 1e-13 and np.all(np.abs(out["row_kl"]) < 1e-13), out
    dH, dW = o.backward(H, W, ids, logits, T, 1.0)
    assert np.max(np.abs(dH)) < 1e-14 and np.max(np.abs(dW)) < 1e-14


# --- finite differences ----------------------------------------------------

def pin_finite_differences(o):
    """Central differences of g * loss (fp64, h = 1e-6) for every entry of H
    and W agree with the oracle's dH and dW to rel 1e-6."""
    rng = np.random.default_rng(16)
    N, d, V, K, T, g = 3, 5, 11, 3, 1.3, 0.7
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    dH, dW = o.backward(H, W, ids, logits, T, g)
    h = 1e-6

    def L(Hx, Wx):
        return g * o.forward(Hx, Wx, ids, logits, T)["loss"]

    fH = np.zeros_like(H)
    for idx in np.ndindex(H.shape):
        Hp = H.copy(); Hp[idx] += h
        Hm = H.copy(); Hm[idx] -= h
        fH[idx] = (L(Hp, W) - L(Hm, W)) / (2 * h)
    fW = np.zeros_like(W)
    for idx in np.ndindex(W.shape):
        Wp = W.copy(); Wp[idx] += h
        Wm = W.copy(); Wm[idx] -= h
        fW[idx] = (L(H, Wp) - L(H, Wm)) / (2 * h)
    _close(dH, fH, 1e-6, what="finite differences dH")
    _close(dW, fW, 1e-6, what="finite differences dW")


# --- invariants --------------------------------------------------------------

def pin_invariants(o):
    rng = np.random.default_rng(17)
    N, d, V, K, T, g = 9, 6, 23, 5, 1.4, 1.1
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    base = o.forward(H, W, ids, logits, T)
    dH, dW = o.backward(H, W, ids, logits, T, g)
    # KL >= 0 per row
    assert np.all(base["row_kl"] >= -1e-15), base["row_kl"]
    # permuting the K (id, logit) pairs changes nothing
    perm = rng.permutation(K)
    p2 = o.forward(H, W, ids[:, perm], logits[:, perm], T)
    _close(p2["row_kl"], base["row_kl"], 1e-13, what="K-permutation row_kl")
    dH2, dW2 = o.backward(H, W, ids[:, perm], logits[:, perm], T, g)
    _close(dH2, dH, 1e-13, what="K-permutation dH")
    _close(dW2, dW, 1e-13, what="K-permutation dW")
    # permuting rows permutes row outputs and dH, keeps loss and dW
    rp = rng.permutation(N)
    r2 = o.forward(H[rp], W, ids[rp], logits[rp], T)
    _close(r2["loss"], base["loss"], 1e-13, what="row-permutation loss")
    _close(r2["row_lse"], base["row_lse"][rp], 1e-13, what="row-permutation lse")
    dH3, dW3 = o.backward(H[rp], W, ids[rp], logits[rp], T, g)
    _close(dH3, dH[rp], 1e-13, what="row-permutation dH")
    _close(dW3, dW, 1e-12, what="row-permutation dW")
    # block (chunk) size does not change the result
    for blk in (1, 4, N):
        _close(o.forward(H, W, ids, logits, T, block=blk)["loss"], base["loss"], 1e-13,
               what=f"block {blk} loss")
        dHb, dWb = o.backward(H, W, ids, logits, T, g, block=blk)
        _close(dHb, dH, 1e-13, what=f"block {blk} dH")
        _close(dWb, dW, 1e-12, what=f"block {blk} dW")
    # linear in the upstream gradient
    dH4, dW4 = o.backward(H, W, ids, logits, T, 2.5 * g)
    _close(dH4, 2.5 * dH, 1e-13, what="linearity dH")
    _close(dW4, 2.5 * dW, 1e-13, what="linearity dW")
    # each dZ row sums to zero, so the columns of dW sum to zero
    _close(dW.sum(axis=0), np.zeros(d), 0.0, atol=1e-14 * max(1.0, np.abs(dW).max() * V),
           what="column sums of dW")
    # shifting every row of W by one vector leaves the softmax, hence loss,
    # dH and dW, unchanged
    c = rng.standard_normal(d)
    s = o.forward(H, W + c[None, :], ids, logits, T)
    _close(s["row_kl"], base["row_kl"], 1e-11, what="W-shift row_kl")
    dH5, dW5 = o.backward(H, W + c[None, :], ids, logits, T, g)
    _close(dH5, dH, 1e-10, what="W-shift dH")
    _close(dW5, dW, 1e-10, what="W-shift dW")
    # temperature identity: loss(H, W, l, T) = loss(H/T, W, l/T, 1);
    # dH_T = dH_1(H/T) / T and dW_T = dW_1(H/T)
    t1 = o.forward(H / T, W, ids, logits / T, 1.0)
    _close(t1["loss"], base["loss"], 1e-13, what="temperature identity loss")
    dH6, dW6 = o.backward(H / T, W, ids, logits / T, 1.0, g)
    # backward at T scales dZ by 1/(N T); at T = 1 by 1/N, hence the 1/T
    _close(dH6 / T, dH, 1e-12, what="temperature identity dH")
    _close(dW6, dW, 1e-12, what="temperature identity dW")


def pin_row_functions(o):
    """The one-row-at-a-time helpers used at full size agree with the full
    forward/backward (themselves pinned by finite differences above)."""
    if not hasattr(o, "sampled_rows"):
        return
    rng = np.random.default_rng(18)
    N, d, V, K, T, g = 12, 5, 31, 4, 1.6, 0.9
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    f = o.forward(H, W, ids, logits, T)
    dH, dW = o.backward(H, W, ids, logits, T, g)
    rows = [0, 5, 11]
    sr = o.sampled_rows(H, W, ids, logits, T, rows, N, g)
    _close(sr["row_lse"], f["row_lse"][rows], 1e-13, what="sampled lse")
    _close(sr["row_kl"], f["row_kl"][rows], 1e-13, what="sampled kl")
    _close(sr["dH_rows"], dH[rows], 1e-13, what="sampled dH rows")
    vrows = [0, 7, int(ids[3, 1]), 30]
    _close(o.dw_rows(H, W, ids, logits, T, vrows, f["row_lse"], g), dW[vrows], 1e-12,
           what="sampled dW rows")


def pin_fused_brute_force_dropped_and_repeated_ids(o):
    """Pure-Python loops (math module only) on a tiny problem whose teacher
    ids break the pages' setting: ids outside [0, V) (7, 6, -2, -5 with V = 6)
    keep their share of the teacher's normalisation but gather nothing and
    scatter nothing, and a repeated id is gathered per entry and scatters
    the sum of its masses. Written as KL = sum p log p - sum_valid p s[id] +
    lse (the oracle uses sum p (log p - log q[id])); the loss is checked
    against central finite differences too, and the dense grid (repeated ids
    merged into one cell, no cell for the others) against a loop over the
    grid."""
    rng = np.random.default_rng(28)
    N, d, V, K, T, g = 4, 3, 6, 3, 1.9, 0.8
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    ids = np.array([[0, 5, 2], [7, 1, -2], [3, 3, 4], [6, -5, 0]])
    logits = rng.standard_normal((N, K))
    kl, lses, dz = [], [], np.zeros((N, V))
    for i in range(N):
        a = [logits[i, k] / T for k in range(K)]
        ma = max(a)
        za = sum(math.exp(x - ma) for x in a)
        p = [math.exp(x - ma) / za for x in a]
        s = [sum(H[i, j] * W[v, j] for j in range(d)) / T for v in range(V)]
        ms = max(s)
        lse = ms + math.log(sum(math.exp(x - ms) for x in s))
        val = sum(p[k] * math.log(p[k]) for k in range(K)) + lse
        for k in range(K):
            if 0 <= ids[i, k] < V:
                val -= p[k] * s[ids[i, k]]
        kl.append(val)
        lses.append(lse)
        for v in range(V):
            mass = sum(p[k] for k in range(K) if ids[i, k] == v)
            dz[i, v] = g / (N * T) * (math.exp(s[v] - lse) - mass)
    dH = [[sum(dz[i, v] * W[v, j] for v in range(V)) for j in range(d)] for i in range(N)]
    dW = [[sum(dz[i, v] * H[i, j] for i in range(N)) for j in range(d)] for v in range(V)]
    out = o.forward(H, W, ids, logits, T)
    _close(out["row_kl"], kl, 1e-13, what="bad ids: row_kl")
    _close(out["row_lse"], lses, 1e-13, what="bad ids: row_lse")
    _close(out["loss"], sum(kl) / N, 1e-13, what="bad ids: loss")
    gdH, gdW = o.backward(H, W, ids, logits, T, g)
    _close(gdH, dH, 1e-13, what="bad ids: dH")
    _close(gdW, dW, 1e-13, what="bad ids: dW")
    sr = o.sampled_rows(H, W, ids, logits, T, [1, 2, 3], N, g)
    _close(sr["row_kl"], [kl[1], kl[2], kl[3]], 1e-13, what="bad ids: sampled kl")
    _close(sr["dH_rows"], [dH[1], dH[2], dH[3]], 1e-13, what="bad ids: sampled dH")
    _close(o.dw_rows(H, W, ids, logits, T, [0, 3, 5], out["row_lse"], g), [dW[0], dW[3], dW[5]], 1e-12,
           what="bad ids: dW rows")
    # the gradient is the exact gradient of this loss: central differences
    h = 1e-6
    fH = np.zeros_like(H)
    for idx in np.ndindex(H.shape):
        Hp = H.copy(); Hp[idx] += h
        Hm = H.copy(); Hm[idx] -= h
        fH[idx] = g * (o.forward(Hp, W, ids, logits, T)["loss"] - o.forward(Hm, W, ids, logits, T)["loss"]) / (2 * h)
    _close(gdH, fH, 1e-6, what="bad ids: finite differences dH")
    # the dense grid: one cell per vocabulary entry
    grid = 0.0
    for i in range(N):
        a = [logits[i, k] / T for k in range(K)]
        ma = max(a)
        za = sum(math.exp(x - ma) for x in a)
        for v in range(V):
            P = sum(math.exp(a[k] - ma) / za for k in range(K) if ids[i, k] == v)
            if P > 0:
                s = [sum(H[i, j] * W[u, j] for j in range(d)) / T for u in range(V)]
                grid += P * (math.log(P) - (s[v] - lses[i]))
    _close(o.dense_kl_loss(H, W, ids, logits, T), grid / N, 1e-13, what="bad ids: dense grid")
    # the forward-chunked functions on Z = H W^T give the same loss and, by
    # the chain rule, the same gradients
    if hasattr(o, "logits_forward"):
        Z = H @ W.T
        _close(o.logits_forward(Z, ids, logits, T)["row_kl"], kl, 1e-13, what="bad ids: logits row_kl")
        dZ = o.logits_backward(Z, ids, logits, T, g)
        _close(dZ @ W, dH, 1e-13, what="bad ids: chain rule dH")
        _close(dZ.T @ H, dW, 1e-13, what="bad ids: chain rule dW")


# --- forward-chunked KL (the student's logit grid is given) ------------------

def _rand_logits_problem(rng, N, V, K, scale=1.0):
    Z = rng.standard_normal((N, V)) * scale
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(N)])
    logits = rng.standard_normal((N, K)) * 1.7
    return Z, ids, logits


def pin_logits_cross_entropy(o):
    """K = 1 (one-hot teacher): torch's cross-entropy of Z / T, and its
    autograd gradient with respect to Z."""
    if not hasattr(o, "logits_forward"):
        return
    rng = np.random.default_rng(21)
    N, V, T, g = 7, 19, 1.7, 0.6
    Z, ids, logits = _rand_logits_problem(rng, N, V, 1)
    Zt = torch.tensor(Z, requires_grad=True)
    ce = F.cross_entropy(Zt / T, torch.tensor(ids[:, 0]))
    (g * ce).backward()
    out = o.logits_forward(Z, ids, logits, T)
    _close(out["loss"], ce.item(), 1e-13, what="logits K=1 loss vs cross_entropy")
    _close(out["row_lse"], sps.logsumexp(Z / T, axis=1), 1e-13, what="logits lse vs scipy")
    _close(o.logits_backward(Z, ids, logits, T, g), Zt.grad.numpy(), 1e-12, what="logits K=1 dZ")


def pin_logits_dense_libraries(o):
    """General K: the dense teacher grid against softmax(Z/T) through scipy's
    rel_entr and torch's kl_div (loss), and torch autograd through kl_div
    (gradient)."""
    if not hasattr(o, "logits_forward"):
        return
    rng = np.random.default_rng(22)
    N, V, K, T, g = 6, 15, 5, 1.3, 1.4
    Z, ids, logits = _rand_logits_problem(rng, N, V, K)
    P = np.zeros((N, V))
    for i in range(N):
        P[i, ids[i]] = sps.softmax(logits[i] / T)
    ref = sps.rel_entr(P, sps.softmax(Z / T, axis=1)).sum(axis=1)
    out = o.logits_forward(Z, ids, logits, T)
    _close(out["row_kl"], ref, 1e-12, what="logits row_kl vs rel_entr")
    Zt = torch.tensor(Z, requires_grad=True)
    kl = F.kl_div(torch.log_softmax(Zt / T, dim=1), torch.tensor(P), reduction="sum") / N
    (g * kl).backward()
    _close(out["loss"], kl.item(), 1e-12, what="logits loss vs kl_div")
    _close(o.logits_backward(Z, ids, logits, T, g), Zt.grad.numpy(), 1e-12, what="logits dZ vs autograd")


def pin_logits_finite_differences(o):
    """Central differences of g * loss (h = 1e-6) for every entry of Z."""
    if not hasattr(o, "logits_forward"):
        return
    rng = np.random.default_rng(23)
    N, V, K, T, g = 3, 9, 4, 0.8, 1.2
    Z, ids, logits = _rand_logits_problem(rng, N, V, K)
    dZ = o.logits_backward(Z, ids, logits, T, g)
    h = 1e-6
    fd = np.zeros_like(Z)
    for idx in np.ndindex(Z.shape):
        Zp = Z.copy(); Zp[idx] += h
        Zm = Z.copy(); Zm[idx] -= h
        fd[idx] = g * (o.logits_forward(Zp, ids, logits, T)["loss"]
                       - o.logits_forward(Zm, ids, logits, T)["loss"]) / (2 * h)
    _close(dZ, fd, 1e-6, what="logits finite differences")


def pin_logits_brute_force_dropped_ids(o):
    """Pure-Python loops (math module only) on a tiny grid where some ids are
    outside [0, V): those entries keep their share of the teacher's
    normalisation but add nothing to the gathered logit or to the gradient."""
    if not hasattr(o, "logits_forward"):
        return
    rng = np.random.default_rng(24)
    N, V, K, T, g = 4, 6, 3, 1.9, 0.8
    Z = rng.standard_normal((N, V))
    ids = np.array([[0, 5, 2], [7, 1, -1], [3, 3, 4], [6, 2, 0]])  # 7, -1, 6 dropped; row 2 repeats 3
    logits = rng.standard_normal((N, K))
    kl, dz = [], np.zeros((N, V))
    for i in range(N):
        a = [logits[i, k] / T for k in range(K)]
        ma = max(a)
        za = sum(math.exp(x - ma) for x in a)
        p = [math.exp(x - ma) / za for x in a]
        s = [Z[i, v] / T for v in range(V)]
        ms = max(s)
        lse = ms + math.log(sum(math.exp(x - ms) for x in s))
        val = sum(p[k] * math.log(p[k]) for k in range(K))
        for k in range(K):
            if 0 <= ids[i, k] < V:
                val -= p[k] * s[ids[i, k]]
        kl.append(val + lse)
        for v in range(V):
            mass = sum(p[k] for k in range(K) if ids[i, k] == v)
            dz[i, v] = g / (N * T) * (math.exp(s[v] - lse) - mass)
    out = o.logits_forward(Z, ids, logits, T)
    _close(out["row_kl"], kl, 1e-13, what="brute-force row_kl")
    _close(o.logits_backward(Z, ids, logits, T, g), dz, 1e-13, what="brute-force dZ")


def pin_logits_closed_forms_and_invariants(o):
    if not hasattr(o, "logits_forward"):
        return
    rng = np.random.default_rng(25)
    N, V, K, T, g = 8, 21, 5, 1.6, 0.9
    Z, ids, logits = _rand_logits_problem(rng, N, V, K)
    base = o.logits_forward(Z, ids, logits, T)
    dZ = o.logits_backward(Z, ids, logits, T, g)
    # constant rows: the student is uniform, KL = log V - entropy(p) (scipy)
    c = rng.standard_normal((N, 1))
    u = o.logits_forward(np.repeat(c, V, axis=1), ids, logits, T)
    ent = np.array([sst.entropy(sps.softmax(logits[i] / T)) for i in range(N)])
    _close(u["row_kl"], math.log(V) - ent, 1e-12, what="uniform logits row_kl")
    _close(u["row_lse"], c[:, 0] / T + math.log(V), 1e-13, what="uniform logits lse")
    # adding a constant to a row changes lse by c/T and nothing else
    sh = o.logits_forward(Z + c, ids, logits, T)
    _close(sh["row_kl"], base["row_kl"], 1e-12, what="row-shift row_kl")
    _close(sh["row_lse"], base["row_lse"] + c[:, 0] / T, 1e-12, what="row-shift lse")
    _close(o.logits_backward(Z + c, ids, logits, T, g), dZ, 1e-12, what="row-shift dZ")
    # every dZ row sums to zero; only the K teacher entries can be negative
    _close(dZ.sum(axis=1), np.zeros(N), 0.0, atol=1e-15, what="dZ row sums")
    mask = np.ones_like(dZ, dtype=bool)
    np.put_along_axis(mask, ids, False, axis=1)
    assert np.all(dZ[mask] > 0.0)
    # KL >= 0; K-pair permutation; block size; linearity in g
    assert np.all(base["row_kl"] >= -1e-15)
    perm = rng.permutation(K)
    _close(o.logits_forward(Z, ids[:, perm], logits[:, perm], T)["row_kl"], base["row_kl"], 1e-13,
           what="logits K-permutation")
    for blk in (1, 3):
        _close(o.logits_forward(Z, ids, logits, T, block=blk)["loss"], base["loss"], 1e-13,
               what=f"logits block {blk}")
        _close(o.logits_backward(Z, ids, logits, T, g, block=blk), dZ, 1e-13, what=f"logits dZ block {blk}")
    _close(o.logits_backward(Z, ids, logits, T, 3.0 * g), 3.0 * dZ, 1e-13, what="logits dZ linear in g")
    # temperature identity: (Z, l, T) is (Z/T, l/T, 1), dZ_T = dZ_1(Z/T) / T
    t1 = o.logits_forward(Z / T, ids, logits / T, 1.0)
    _close(t1["loss"], base["loss"], 1e-13, what="logits temperature identity")
    _close(o.logits_backward(Z / T, ids, logits / T, 1.0, g) / T, dZ, 1e-12,
           what="logits temperature identity dZ")


def pin_logits_matches_fused(o):
    """With Z = H W^T the forward-chunked functions give the fused loss, and
    the output layer's chain rule (dH = dZ W, dW = dZ^T H) gives the fused
    gradients; the two are written in different arrangements."""
    if not hasattr(o, "logits_forward"):
        return
    rng = np.random.default_rng(26)
    N, d, V, K, T, g = 6, 5, 17, 4, 1.2, 0.7
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    f = o.forward(H, W, ids, logits, T)
    lf = o.logits_forward(H @ W.T, ids, logits, T)
    _close(lf["row_kl"], f["row_kl"], 1e-12, what="logits vs fused row_kl")
    _close(lf["row_lse"], f["row_lse"], 1e-13, what="logits vs fused lse")
    dH, dW = o.backward(H, W, ids, logits, T, g)
    dZ = o.logits_backward(H @ W.T, ids, logits, T, g)
    _close(dZ @ W, dH, 1e-12, what="chain rule dH")
    _close(dZ.T @ H, dW, 1e-12, what="chain rule dW")
    sr = o.logits_sampled_rows(H @ W.T, ids, logits, T, [0, 4], N, g)
    _close(sr["dZ_rows"], dZ[[0, 4]], 1e-13, what="logits sampled dZ rows")
    _close(sr["row_kl"], lf["row_kl"][[0, 4]], 1e-13, what="logits sampled kl")


# --- ignored positions (first teacher id -1) -----------------------------------

def pin_ignored_positions(o):
    """Ignoring a position is deleting it: loss, dW and the kept rows' outputs
    equal those of the problem without it (computed by the unmasked paths,
    pinned above), its KL and gradient row are zero, its other teacher
    entries are never used; with nothing kept the loss is NaN and every
    gradient is zero. For the fused and the forward-chunked functions, the
    dense-grid baseline and the one-row helpers."""
    if not hasattr(o, "kept_positions"):
        return
    rng = np.random.default_rng(27)
    N, d, V, K, T, g = 10, 5, 19, 4, 1.3, 0.8
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    ign = np.array([1, 4, 5, 9])
    keep = np.setdiff1d(np.arange(N), ign)
    ids_m = ids.copy()
    ids_m[ign, 0] = -1
    ids_m[ign[0], 1:] = 10 ** 9  # never used
    assert np.array_equal(o.kept_positions(ids_m), np.isin(np.arange(N), keep))
    f = o.forward(H, W, ids_m, logits, T)
    fr = o.forward(H[keep], W, ids[keep], logits[keep], T)
    _close(f["loss"], fr["loss"], 1e-13, what="ignored: loss")
    assert np.all(f["row_kl"][ign] == 0.0)
    _close(f["row_kl"][keep], fr["row_kl"], 1e-13, what="ignored: kept row_kl")
    _close(f["row_lse"], o.forward(H, W, ids, logits, T)["row_lse"], 1e-13, what="ignored: lse")
    dH, dW = o.backward(H, W, ids_m, logits, T, g)
    dHr, dWr = o.backward(H[keep], W, ids[keep], logits[keep], T, g)
    assert np.all(dH[ign] == 0.0)
    _close(dH[keep], dHr, 1e-13, what="ignored: kept dH")
    _close(dW, dWr, 1e-13, what="ignored: dW")
    _close(o.dense_kl_loss(H, W, ids_m, logits, T), fr["loss"], 1e-12, what="ignored: dense grid")
    sr = o.sampled_rows(H, W, ids_m, logits, T, [0, 1, 6], len(keep), g)
    _close(sr["dH_rows"], dH[[0, 1, 6]], 1e-13, what="ignored: sampled dH")
    _close(sr["row_kl"], f["row_kl"][[0, 1, 6]], 1e-13, what="ignored: sampled kl")
    _close(o.dw_rows(H, W, ids_m, logits, T, [0, 3, 18], f["row_lse"], g), dW[[0, 3, 18]], 1e-12,
           what="ignored: dW rows")
    Z = H @ W.T
    lf = o.logits_forward(Z, ids_m, logits, T)
    lfr = o.logits_forward(Z[keep], ids[keep], logits[keep], T)
    _close(lf["loss"], lfr["loss"], 1e-13, what="ignored: logits loss")
    assert np.all(lf["row_kl"][ign] == 0.0)
    dZ = o.logits_backward(Z, ids_m, logits, T, g)
    assert np.all(dZ[ign] == 0.0)
    _close(dZ[keep], o.logits_backward(Z[keep], ids[keep], logits[keep], T, g), 1e-13,
           what="ignored: logits dZ")
    ls = o.logits_sampled_rows(Z, ids_m, logits, T, [1, 2], len(keep), g)
    _close(ls["dZ_rows"], dZ[[1, 2]], 1e-13, what="ignored: logits sampled dZ")
    # only -1 marks a position; another negative first id is an out-of-range
    # id whose mass is dropped, and the position still counts
    ids_n = ids.copy()
    ids_n[2, 0] = -5
    assert o.kept_positions(ids_n)[2]
    ln = o.logits_forward(Z, ids_n, logits, T)
    assert ln["row_kl"][2] != 0.0
    _close(ln["loss"], math.fsum(ln["row_kl"].tolist()) / N, 1e-13, what="out-of-range first id counts")
    # nothing kept
    ids_all = ids.copy()
    ids_all[:, 0] = -1
    assert math.isnan(o.forward(H, W, ids_all, logits, T)["loss"])
    dH0, dW0 = o.backward(H, W, ids_all, logits, T, g)
    assert not dH0.any() and not dW0.any()
    assert math.isnan(o.logits_forward(Z, ids_all, logits, T)["loss"])
    assert not o.logits_backward(Z, ids_all, logits, T, g).any()


# --- the alternative loss: generalised Jensen-Shannon divergence ---------------

def pin_jsd_scipy_jensenshannon(o):
    """beta = 1/2: per row, scipy's Jensen-Shannon distance squared between
    the teacher's top-K distribution on the vocabulary and softmax(Z / T)."""
    if not hasattr(o, "jsd_forward"):
        return
    from scipy.spatial.distance import jensenshannon
    rng = np.random.default_rng(31)
    N, d, V, K, T = 6, 5, 19, 5, 1.3
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    q = sps.softmax(H @ W.T / T, axis=1)
    ref = []
    for i in range(N):
        P = np.zeros(V)
        P[ids[i]] = sps.softmax(logits[i] / T)
        ref.append(jensenshannon(P, q[i]) ** 2)
    out = o.jsd_forward(H, W, ids, logits, T, 0.5)
    _close(out["row_kl"], ref, 1e-12, what="JSD 1/2 vs scipy jensenshannon")
    _close(out["loss"], np.mean(ref), 1e-12, what="JSD 1/2 loss")
    assert np.all(out["row_kl"] >= 0.0) and np.all(out["row_kl"] <= math.log(2.0))


def pin_jsd_small_beta_is_forward_kl(o):
    """JSD_beta / beta tends to the forward KL (pinned above) as beta -> 0,
    loss and gradients, with an O(beta) remainder."""
    if not hasattr(o, "jsd_forward"):
        return
    rng = np.random.default_rng(32)
    N, d, V, K, T, g, beta = 5, 4, 17, 4, 1.4, 0.9, 1e-7
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    f = o.forward(H, W, ids, logits, T)
    j = o.jsd_forward(H, W, ids, logits, T, beta)
    _close(j["row_kl"] / beta, f["row_kl"], 1e-5, what="JSD/beta vs KL")
    _close(j["row_lse"], f["row_lse"], 1e-14, what="JSD lse")
    dH, dW = o.backward(H, W, ids, logits, T, g)
    jH, jW = o.jsd_backward(H, W, ids, logits, T, beta, g)
    _close(jH / beta, dH, 1e-5, what="JSD/beta dH vs KL dH")
    _close(jW / beta, dW, 1e-5, what="JSD/beta dW vs KL dW")


def pin_jsd_torch_autograd(o):
    """General beta: the loss through torch's kl_div (KL(P || M) and
    KL(q || M) with M = beta P + (1 - beta) q, P with zeros off the top-K)
    and its gradients by torch autograd."""
    if not hasattr(o, "jsd_forward"):
        return
    rng = np.random.default_rng(33)
    N, d, V, K, T, g, beta = 5, 4, 15, 4, 0.8, 1.3, 0.3
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    P = np.zeros((N, V))
    for i in range(N):
        P[i, ids[i]] = sps.softmax(logits[i] / T)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    Pt = torch.tensor(P)
    q = torch.softmax(Ht @ Wt.T / T, dim=1)
    logM = torch.log(beta * Pt + (1 - beta) * q)
    jsd = (beta * F.kl_div(logM, Pt, reduction="sum") + (1 - beta) * F.kl_div(logM, q, reduction="sum")) / N
    (g * jsd).backward()
    out = o.jsd_forward(H, W, ids, logits, T, beta)
    _close(out["loss"], jsd.item(), 1e-12, what="JSD loss vs kl_div")
    jH, jW = o.jsd_backward(H, W, ids, logits, T, beta, g)
    _close(jH, Ht.grad.numpy(), 1e-11, what="JSD dH vs autograd")
    _close(jW, Wt.grad.numpy(), 1e-11, what="JSD dW vs autograd")


def pin_jsd_brute_force_and_finite_differences(o):
    """Pure-Python loops (math module only) with ids outside [0, V) and a
    repeated id, written over the teacher's support only (the off-support
    entries contribute -(1 - beta) log(1 - beta) times the student's mass
    there); central differences of the loss for every entry of H and W."""
    if not hasattr(o, "jsd_forward"):
        return
    rng = np.random.default_rng(34)
    N, d, V, K, T, g, beta = 4, 3, 6, 3, 1.6, 0.7, 0.35
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    ids = np.array([[0, 5, 2], [7, 1, -2], [3, 3, 4], [6, -5, 0]])
    logits = rng.standard_normal((N, K))
    ref = []
    for i in range(N):
        a = [logits[i, k] / T for k in range(K)]
        ma = max(a)
        za = sum(math.exp(x - ma) for x in a)
        p = [math.exp(x - ma) / za for x in a]
        s = [sum(H[i, j] * W[v, j] for j in range(d)) / T for v in range(V)]
        ms = max(s)
        lse = ms + math.log(sum(math.exp(x - ms) for x in s))
        support = sorted({int(v) for v in ids[i] if 0 <= v < V})
        val, qs = 0.0, 0.0
        for v in support:
            Pv = sum(p[k] for k in range(K) if ids[i, k] == v)
            qv = math.exp(s[v] - lse)
            Mv = beta * Pv + (1 - beta) * qv
            val += beta * Pv * math.log(Pv / Mv) + (1 - beta) * qv * math.log(qv / Mv)
            qs += qv
        val += -(1 - beta) * math.log(1 - beta) * (1 - qs)
        ref.append(val)
    out = o.jsd_forward(H, W, ids, logits, T, beta)
    _close(out["row_kl"], ref, 1e-13, what="JSD brute force")
    dH, dW = o.jsd_backward(H, W, ids, logits, T, beta, g)
    h = 1e-6

    def L(Hx, Wx):
        return g * o.jsd_forward(Hx, Wx, ids, logits, T, beta)["loss"]

    for X, dX, name in ((H, dH, "dH"), (W, dW, "dW")):
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp = X.copy(); Xp[idx] += h
            Xm = X.copy(); Xm[idx] -= h
            fd[idx] = (L(Xp, W) - L(Xm, W)) / (2 * h) if X is H else (L(H, Xp) - L(H, Xm)) / (2 * h)
        _close(dX, fd, 1e-6, what=f"JSD finite differences {name}")


def pin_jsd_invariants(o):
    if not hasattr(o, "jsd_forward"):
        return
    rng = np.random.default_rng(35)
    N, d, V, K, T, g, beta = 8, 5, 21, 5, 1.5, 1.1, 0.4
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    base = o.jsd_forward(H, W, ids, logits, T, beta)
    dH, dW = o.jsd_backward(H, W, ids, logits, T, beta, g)
    assert np.all(base["row_kl"] >= 0.0)
    # teacher equal to the student over the whole vocabulary: zero loss, zero gradients
    ide = np.stack([rng.permutation(V) for _ in range(N)])
    eq = np.take_along_axis(H @ W.T, ide, axis=1)
    e = o.jsd_forward(H, W, ide, eq, T, beta)
    assert np.max(np.abs(e["row_kl"])) < 1e-13
    eH, eW = o.jsd_backward(H, W, ide, eq, T, beta, g)
    assert np.max(np.abs(eH)) < 1e-13 and np.max(np.abs(eW)) < 1e-13
    # K-pair permutation, block size, linearity in g, W row shift
    perm = rng.permutation(K)
    _close(o.jsd_forward(H, W, ids[:, perm], logits[:, perm], T, beta)["row_kl"], base["row_kl"], 1e-13,
           what="JSD K-permutation")
    for blk in (1, 3):
        _close(o.jsd_forward(H, W, ids, logits, T, beta, block=blk)["loss"], base["loss"], 1e-13,
               what=f"JSD block {blk}")
        bH, bW = o.jsd_backward(H, W, ids, logits, T, beta, g, block=blk)
        _close(bH, dH, 1e-13, what=f"JSD block {blk} dH")
        _close(bW, dW, 1e-12, what=f"JSD block {blk} dW")
    lH, lW = o.jsd_backward(H, W, ids, logits, T, beta, 2.5 * g)
    _close(lH, 2.5 * dH, 1e-13, what="JSD linear in g")
    c = rng.standard_normal(d)
    _close(o.jsd_forward(H, W + c, ids, logits, T, beta)["row_kl"], base["row_kl"], 1e-11, what="JSD W shift")
    # every dZ row sums to zero: the columns of dW sum to zero
    _close(dW.sum(axis=0), np.zeros(d), 0.0, atol=1e-14 * max(1.0, np.abs(dW).max() * V),
           what="JSD column sums of dW")
    # temperature identity
    t1 = o.jsd_forward(H / T, W, ids, logits / T, 1.0, beta)
    _close(t1["loss"], base["loss"], 1e-13, what="JSD temperature identity")
    tH, tW = o.jsd_backward(H / T, W, ids, logits / T, 1.0, beta, g)
    _close(tH / T, dH, 1e-12, what="JSD temperature identity dH")
    _close(tW, dW, 1e-12, what="JSD temperature identity dW")
    # ignoring a position is deleting it
    ign = np.array([2, 5])
    keep = np.setdiff1d(np.arange(N), ign)
    ids_m = ids.copy()
    ids_m[ign, 0] = -1
    m = o.jsd_forward(H, W, ids_m, logits, T, beta)
    _close(m["loss"], o.jsd_forward(H[keep], W, ids[keep], logits[keep], T, beta)["loss"], 1e-13,
           what="JSD ignored: loss")
    assert np.all(m["row_kl"][ign] == 0.0)
    mH, mW = o.jsd_backward(H, W, ids_m, logits, T, beta, g)
    rH, rW = o.jsd_backward(H[keep], W, ids[keep], logits[keep], T, beta, g)
    assert np.all(mH[ign] == 0.0)
    _close(mH[keep], rH, 1e-13, what="JSD ignored: dH")
    _close(mW, rW, 1e-13, what="JSD ignored: dW")


# --- the skew KL and skew reverse KL ----------------------------------------

def pin_skl_alpha_zero_is_forward_kl(o):
    """The skew KL at alpha = 0 is the forward KL pinned above (rows with
    distinct in-range ids), loss, rows and gradients; near alpha = 1 the
    mixture is the teacher itself and the loss vanishes."""
    if not hasattr(o, "alt_forward"):
        return
    rng = np.random.default_rng(41)
    N, d, V, K, T, g = 6, 5, 23, 5, 1.2, 0.8
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    f = o.forward(H, W, ids, logits, T)
    s = o.alt_forward(H, W, ids, logits, T, "skl", 0.0)
    _close(s["row_kl"], f["row_kl"], 1e-12, what="SKL(0) rows vs KL")
    _close(s["loss"], f["loss"], 1e-12, what="SKL(0) loss vs KL")
    _close(s["row_lse"], f["row_lse"], 1e-14, what="SKL lse")
    dH, dW = o.backward(H, W, ids, logits, T, g)
    sH, sW = o.alt_backward(H, W, ids, logits, T, "skl", 0.0, g)
    _close(sH, dH, 1e-12, what="SKL(0) dH vs KL dH")
    _close(sW, dW, 1e-12, what="SKL(0) dW vs KL dW")
    near = o.alt_forward(H, W, ids, logits, T, "skl", 1.0 - 1e-9)
    assert np.max(np.abs(near["row_kl"])) < 1e-7, near["row_kl"]


def pin_skew_losses_torch_autograd(o):
    """Both losses through torch (kl_div on the dense grid, P with zeros off
    the top-K) and their gradients by autograd."""
    if not hasattr(o, "alt_forward"):
        return
    rng = np.random.default_rng(42)
    N, d, V, K, T, g = 5, 4, 15, 4, 0.9, 1.2
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    P = np.zeros((N, V))
    for i in range(N):
        P[i, ids[i]] = sps.softmax(logits[i] / T)
    for loss, a in (("skl", 0.3), ("srkl", 0.2)):
        Ht = torch.tensor(H, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        Pt = torch.tensor(P)
        q = torch.softmax(Ht @ Wt.T / T, dim=1)
        if loss == "skl":
            val = F.kl_div(torch.log(a * Pt + (1 - a) * q), Pt, reduction="sum") / N
        else:
            val = F.kl_div(torch.log(a * q + (1 - a) * Pt), q, reduction="sum") / N
        (g * val).backward()
        out = o.alt_forward(H, W, ids, logits, T, loss, a)
        _close(out["loss"], val.item(), 1e-12, what=f"{loss} loss vs kl_div")
        aH, aW = o.alt_backward(H, W, ids, logits, T, loss, a, g)
        _close(aH, Ht.grad.numpy(), 1e-11, what=f"{loss} dH vs autograd")
        _close(aW, Wt.grad.numpy(), 1e-11, what=f"{loss} dW vs autograd")


def pin_skew_losses_brute_force_and_finite_differences(o):
    """Pure-Python loops (math module only) with ids outside [0, V) and a
    repeated id, over the teacher's support (for the skew reverse KL the
    entries off it add -log(alpha) times the student's mass there); central
    differences of the loss for every entry of H and W."""
    if not hasattr(o, "alt_forward"):
        return
    rng = np.random.default_rng(43)
    N, d, V, K, T, g = 4, 3, 6, 3, 1.4, 0.6
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    ids = np.array([[0, 5, 2], [7, 1, -2], [3, 3, 4], [6, -5, 0]])
    logits = rng.standard_normal((N, K))
    for loss, a in (("skl", 0.25), ("srkl", 0.15)):
        ref = []
        for i in range(N):
            t = [logits[i, k] / T for k in range(K)]
            mt = max(t)
            zt = sum(math.exp(x - mt) for x in t)
            p = [math.exp(x - mt) / zt for x in t]
            s = [sum(H[i, j] * W[v, j] for j in range(d)) / T for v in range(V)]
            ms = max(s)
            lse = ms + math.log(sum(math.exp(x - ms) for x in s))
            support = sorted({int(v) for v in ids[i] if 0 <= v < V})
            val, qs = 0.0, 0.0
            for v in support:
                Pv = sum(p[k] for k in range(K) if ids[i, k] == v)
                qv = math.exp(s[v] - lse)
                if loss == "skl":
                    val += Pv * math.log(Pv / (a * Pv + (1 - a) * qv))
                else:
                    val += qv * math.log(qv / (a * qv + (1 - a) * Pv))
                qs += qv
            if loss == "srkl":
                val += -math.log(a) * (1 - qs)
            ref.append(val)
        out = o.alt_forward(H, W, ids, logits, T, loss, a)
        _close(out["row_kl"], ref, 1e-13, what=f"{loss} brute force")
        dH, dW = o.alt_backward(H, W, ids, logits, T, loss, a, g)
        h = 1e-6

        def L(Hx, Wx):
            return g * o.alt_forward(Hx, Wx, ids, logits, T, loss, a)["loss"]

        for X, dX, name in ((H, dH, "dH"), (W, dW, "dW")):
            fd = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                Xp = X.copy(); Xp[idx] += h
                Xm = X.copy(); Xm[idx] -= h
                fd[idx] = (L(Xp, W) - L(Xm, W)) / (2 * h) if X is H else (L(H, Xp) - L(H, Xm)) / (2 * h)
            _close(dX, fd, 1e-6, what=f"{loss} finite differences {name}")


def pin_skew_losses_bounds_and_limits(o):
    """0 <= value <= -log(alpha) per position (distinct in-range ids); the
    skew reverse KL equals -log(alpha) when the student puts no mass on the
    teacher's support, and tends to scipy's reverse KL(q || P) as alpha -> 0
    when the teacher covers the vocabulary (K = V)."""
    if not hasattr(o, "alt_forward"):
        return
    rng = np.random.default_rng(44)
    N, d, V, K, T = 7, 5, 19, 6, 1.1
    H, W, ids, logits = _rand_problem(rng, N, d, V, K, scale=2.0)
    for loss, a in (("skl", 0.1), ("skl", 0.6), ("srkl", 0.1), ("srkl", 0.6)):
        r = o.alt_forward(H, W, ids, logits, T, loss, a)["row_kl"]
        assert np.all(r >= -1e-15) and np.all(r <= -math.log(a) + 1e-15), (loss, a, r)
    # the student's mass off the teacher's support: one hidden unit, the
    # support's logits 60 below the rest
    a = 0.3
    H1 = np.ones((3, 1))
    ids1 = np.array([[1, 4], [0, 2], [5, 3]])
    lg1 = rng.standard_normal((3, 2))
    for i in range(3):
        W1 = np.zeros((V, 1))
        W1[ids1[i]] = -60.0
        r = o.alt_forward(H1[i:i + 1], W1, ids1[i:i + 1], lg1[i:i + 1], 1.0, "srkl", a)["row_kl"]
        _close(r, [-math.log(a)], 1e-12, what="SRKL, student off the support")
    # K = V: reverse KL as alpha -> 0
    ids2 = np.stack([rng.permutation(V) for _ in range(N)])
    lg2 = rng.standard_normal((N, V))
    q = sps.softmax(H @ W.T / T, axis=1)
    P = np.zeros((N, V))
    for i in range(N):
        P[i, ids2[i]] = sps.softmax(lg2[i] / T)
    rkl = sps.rel_entr(q, P).sum(axis=1)
    r = o.alt_forward(H, W, ids2, lg2, T, "srkl", 1e-9)["row_kl"]
    _close(r, rkl, 1e-6, what="SRKL(alpha -> 0) vs scipy rel_entr(q, P)")


def pin_skew_losses_invariants(o):
    if not hasattr(o, "alt_forward"):
        return
    rng = np.random.default_rng(45)
    N, d, V, K, T, g = 8, 5, 21, 5, 1.5, 1.1
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    for loss, a in (("skl", 0.2), ("srkl", 0.3)):
        base = o.alt_forward(H, W, ids, logits, T, loss, a)
        dH, dW = o.alt_backward(H, W, ids, logits, T, loss, a, g)
        # teacher equal to the student over the whole vocabulary
        ide = np.stack([rng.permutation(V) for _ in range(N)])
        eq = np.take_along_axis(H @ W.T, ide, axis=1)
        e = o.alt_forward(H, W, ide, eq, T, loss, a)
        assert np.max(np.abs(e["row_kl"])) < 1e-13, (loss, e["row_kl"])
        eH, eW = o.alt_backward(H, W, ide, eq, T, loss, a, g)
        assert np.max(np.abs(eH)) < 1e-13 and np.max(np.abs(eW)) < 1e-13
        perm = rng.permutation(K)
        _close(o.alt_forward(H, W, ids[:, perm], logits[:, perm], T, loss, a)["row_kl"], base["row_kl"],
               1e-13, what=f"{loss} K-permutation")
        for blk in (1, 3):
            _close(o.alt_forward(H, W, ids, logits, T, loss, a, block=blk)["loss"], base["loss"], 1e-13,
                   what=f"{loss} block {blk}")
            bH, bW = o.alt_backward(H, W, ids, logits, T, loss, a, g, block=blk)
            _close(bH, dH, 1e-13, what=f"{loss} block {blk} dH")
            _close(bW, dW, 1e-12, what=f"{loss} block {blk} dW")
        lH, lW = o.alt_backward(H, W, ids, logits, T, loss, a, 2.5 * g)
        _close(lH, 2.5 * dH, 1e-13, what=f"{loss} linear in g")
        c = rng.standard_normal(d)
        _close(o.alt_forward(H, W + c, ids, logits, T, loss, a)["row_kl"], base["row_kl"], 1e-11,
               what=f"{loss} W shift")
        _close(dW.sum(axis=0), np.zeros(d), 0.0, atol=1e-14 * max(1.0, np.abs(dW).max() * V),
               what=f"{loss} column sums of dW")
        t1 = o.alt_forward(H / T, W, ids, logits / T, 1.0, loss, a)
        _close(t1["loss"], base["loss"], 1e-13, what=f"{loss} temperature identity")
        tH, tW = o.alt_backward(H / T, W, ids, logits / T, 1.0, loss, a, g)
        _close(tH / T, dH, 1e-12, what=f"{loss} temperature identity dH")
        _close(tW, dW, 1e-12, what=f"{loss} temperature identity dW")
        ign = np.array([1, 6])
        keep = np.setdiff1d(np.arange(N), ign)
        ids_m = ids.copy()
        ids_m[ign, 0] = -1
        m = o.alt_forward(H, W, ids_m, logits, T, loss, a)
        _close(m["loss"], o.alt_forward(H[keep], W, ids[keep], logits[keep], T, loss, a)["loss"], 1e-13,
               what=f"{loss} ignored: loss")
        assert np.all(m["row_kl"][ign] == 0.0)
        mH, mW = o.alt_backward(H, W, ids_m, logits, T, loss, a, g)
        rH, rW = o.alt_backward(H[keep], W, ids[keep], logits[keep], T, loss, a, g)
        assert np.all(mH[ign] == 0.0)
        _close(mH[keep], rH, 1e-13, what=f"{loss} ignored: dH")
        _close(mW, rW, 1e-13, what=f"{loss} ignored: dW")
    for loss, bad in (("skl", 1.0), ("skl", -0.1), ("srkl", 0.0), ("srkl", 1.5), ("jsd", 1.0)):
        try:
            o.alt_forward(H, W, ids, logits, T, loss, bad)
        except ValueError:
            continue
        raise AssertionError(f"{loss} accepted parameter {bad}")


# --- reverse KL over the teacher's top-K support -----------------------------

def _support_problem(rng, N, d, V, K, T):
    """Random problem with distinct in-range ids; the student's tempered
    logits at them and the teacher's probabilities, per row."""
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    s_at = np.stack([(W[ids[i]] @ H[i]) / T for i in range(N)])
    p = np.stack([sps.softmax(logits[i] / T) for i in range(N)])
    return H, W, ids, logits, s_at, p


def pin_topk_rkl_scipy_entropy(o):
    """With distinct in-range ids, each position's loss is scipy's relative
    entropy of the student's softmax over the teacher's ids against the
    teacher's probabilities (scipy normalises its first argument)."""
    if not hasattr(o, "topk_rkl_forward"):
        return
    rng = np.random.default_rng(61)
    for T in (1.0, 1.8):
        N, d, V, K = 6, 5, 23, 7
        H, W, ids, logits, s_at, p = _support_problem(rng, N, d, V, K, T)
        ref = np.array([sst.entropy(np.exp(s_at[i] - s_at[i].max()), p[i]) for i in range(N)])
        out = o.topk_rkl_forward(H, W, ids, logits, T)
        _close(out["row_kl"], ref, 1e-12, what=f"TRKL rows vs scipy entropy, T={T}")
        _close(out["loss"], ref.mean(), 1e-12, what=f"TRKL loss vs scipy entropy, T={T}")
        lse = np.array([sps.logsumexp(s_at[i]) for i in range(N)])
        _close(out["row_lse"], lse, 1e-12, what="logsumexp over the support")


def pin_topk_rkl_torch_autograd(o):
    """The loss through torch (log-softmax over the gathered student logits,
    kl_div with log targets) and its gradients by autograd."""
    if not hasattr(o, "topk_rkl_backward"):
        return
    rng = np.random.default_rng(62)
    N, d, V, K, T, g = 5, 4, 17, 5, 1.3, 0.8
    H, W, ids, logits = _rand_problem(rng, N, d, V, K)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    idt = torch.tensor(ids)
    s = Ht @ Wt.T / T
    log_qt = torch.log_softmax(torch.gather(s, 1, idt), dim=1)
    log_p = torch.log_softmax(torch.tensor(logits) / T, dim=1)
    val = F.kl_div(log_p, log_qt, reduction="sum", log_target=True) / N
    (g * val).backward()
    out = o.topk_rkl_forward(H, W, ids, logits, T)
    _close(out["loss"], val.item(), 1e-12, what="TRKL loss vs kl_div")
    dH, dW = o.topk_rkl_backward(H, W, ids, logits, T, g)
    _close(dH, Ht.grad.numpy(), 1e-11, what="TRKL dH vs autograd")
    _close(dW, Wt.grad.numpy(), 1e-11, what="TRKL dW vs autograd")


def pin_topk_rkl_brute_force_and_finite_differences(o):
    """Pure-Python loops (math module only) with ids outside [0, V), a
    repeated id (its masses add) and an ignored position; central
    differences of the loss for every entry of H and W."""
    if not hasattr(o, "topk_rkl_backward"):
        return
    rng = np.random.default_rng(63)
    N, d, V, K, T, g = 5, 3, 7, 4, 1.6, 0.7
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    ids = np.array([[0, 6, 2, 9], [7, 1, -2, 4], [3, 3, 5, 1], [-1, 2, 0, 4], [6, -5, 0, 6]])
    logits = rng.standard_normal((N, K))
    vals = []
    for i in range(N):
        if ids[i, 0] == -1:
            vals.append(0.0)
            continue
        t = [logits[i, k] / T for k in range(K)]
        mt = max(t)
        zt = sum(math.exp(x - mt) for x in t)
        p = [math.exp(x - mt) / zt for x in t]
        sup = sorted({int(v) for v in ids[i] if 0 <= v < V})
        s = {v: sum(H[i, j] * W[v, j] for j in range(d)) / T for v in sup}
        ms = max(s.values())
        lse = ms + math.log(sum(math.exp(s[v] - ms) for v in sup))
        val = 0.0
        for v in sup:
            Pv = sum(p[k] for k in range(K) if ids[i, k] == v)
            qv = math.exp(s[v] - lse)
            val += qv * math.log(qv / Pv)
        vals.append(val)
    out = o.topk_rkl_forward(H, W, ids, logits, T)
    _close(out["row_kl"], vals, 1e-12, what="TRKL rows vs brute force")
    _close(out["loss"], sum(vals) / 4, 1e-12, what="TRKL mean over the kept positions")
    dH, dW = o.topk_rkl_backward(H, W, ids, logits, T, g)
    eps = 1e-6

    def loss_at(Hx, Wx):
        return g * o.topk_rkl_forward(Hx, Wx, ids, logits, T)["loss"]

    fdH = np.zeros_like(H)
    for i in range(N):
        for j in range(d):
            Hp, Hm = H.copy(), H.copy()
            Hp[i, j] += eps
            Hm[i, j] -= eps
            fdH[i, j] = (loss_at(Hp, W) - loss_at(Hm, W)) / (2 * eps)
    fdW = np.zeros_like(W)
    for v in range(V):
        for j in range(d):
            Wp, Wm = W.copy(), W.copy()
            Wp[v, j] += eps
            Wm[v, j] -= eps
            fdW[v, j] = (loss_at(H, Wp) - loss_at(H, Wm)) / (2 * eps)
    _close(dH, fdH, 1e-7, what="TRKL dH vs central differences")
    _close(dW, fdW, 1e-7, what="TRKL dW vs central differences")


def pin_topk_rkl_closed_forms_and_invariants(o):
    """Zero at the teacher (student logits log P + c at the support), zero
    for a single support entry, the two-entry closed form with the logistic
    function, independence of the student's logits off the support (no
    gradient there either), shift invariance, and non-negativity."""
    if not hasattr(o, "topk_rkl_backward"):
        return
    rng = np.random.default_rng(64)
    # zero at the teacher: W rows at the ids are unit vectors, H_i = T (log p + c)
    K, V, T = 4, 9, 1.5
    ids = np.array([[2, 7, 0, 5]])
    logits = rng.standard_normal((1, K))
    logp = np.log(sps.softmax(logits[0] / T))
    W = rng.standard_normal((V, K))
    W[ids[0]] = np.eye(K)
    H = (T * (logp + 0.7))[None, :]
    out = o.topk_rkl_forward(H, W, ids, logits, T)
    _close(out["loss"], 0.0, 0.0, atol=1e-14, what="TRKL at the teacher")
    dH, dW = o.topk_rkl_backward(H, W, ids, logits, T)
    _close(dH, 0.0, 0.0, atol=1e-14, what="TRKL gradient at the teacher")
    _close(dW, 0.0, 0.0, atol=1e-14, what="TRKL gradient at the teacher")
    # one support entry: qt = P = 1
    H1, W1, ids1, lg1 = _rand_problem(rng, 3, 4, 8, 1)
    _close(o.topk_rkl_forward(H1, W1, ids1, lg1, 1.2)["loss"], 0.0, 0.0, atol=1e-15, what="K = 1")
    _close(o.topk_rkl_backward(H1, W1, ids1, lg1, 1.2)[0], 0.0, 0.0, atol=1e-15, what="K = 1 gradient")
    # two entries: qt_1 = expit(s_1 - s_2)
    N, d, V, T = 4, 3, 6, 0.8
    H2, W2, ids2, lg2 = _rand_problem(rng, N, d, V, 2)
    ref = []
    for i in range(N):
        s1, s2 = (W2[ids2[i]] @ H2[i]) / T
        q1, q2 = sps.expit(s1 - s2), sps.expit(s2 - s1)
        p1, p2 = sps.expit((lg2[i, 0] - lg2[i, 1]) / T), sps.expit((lg2[i, 1] - lg2[i, 0]) / T)
        ref.append(q1 * math.log(q1 / p1) + q2 * math.log(q2 / p2))
    _close(o.topk_rkl_forward(H2, W2, ids2, lg2, T)["row_kl"], ref, 1e-12, what="two-entry closed form")
    # off the support: other vocabulary rows change nothing and get no gradient
    N, d, V, K, T = 5, 4, 20, 3, 1.1
    H3, W3, ids3, lg3 = _rand_problem(rng, N, d, V, K)
    off = np.setdiff1d(np.arange(V), ids3.reshape(-1))
    W3b = W3.copy()
    W3b[off] = rng.standard_normal((off.size, d)) * 25.0
    a = o.topk_rkl_forward(H3, W3, ids3, lg3, T)
    b = o.topk_rkl_forward(H3, W3b, ids3, lg3, T)
    _close(b["row_kl"], a["row_kl"], 1e-12, what="TRKL independent of off-support logits")
    _, dW3 = o.topk_rkl_backward(H3, W3b, ids3, lg3, T)
    assert np.all(dW3[off] == 0.0), "TRKL gradient off the support"
    assert np.all(a["row_kl"] >= -1e-15), "TRKL is a divergence"
    # shift: one more hidden unit adding the same constant to every logit
    H4 = np.concatenate([H3, np.ones((N, 1))], axis=1)
    W4 = np.concatenate([W3, np.full((V, 1), 3.7)], axis=1)
    _close(o.topk_rkl_forward(H4, W4, ids3, lg3, T)["row_kl"], a["row_kl"], 1e-12, what="shift invariance")


ALL_PINS = [
    pin_two_token_softplus,
    pin_uniform_student,
    pin_cross_entropy,
    pin_dense_grid_libraries,
    pin_equality_case,
    pin_finite_differences,
    pin_invariants,
    pin_row_functions,
    pin_fused_brute_force_dropped_and_repeated_ids,
    pin_logits_cross_entropy,
    pin_logits_dense_libraries,
    pin_logits_finite_differences,
    pin_logits_brute_force_dropped_ids,
    pin_logits_closed_forms_and_invariants,
    pin_logits_matches_fused,
    pin_ignored_positions,
    pin_jsd_scipy_jensenshannon,
    pin_jsd_small_beta_is_forward_kl,
    pin_jsd_torch_autograd,
    pin_jsd_brute_force_and_finite_differences,
    pin_jsd_invariants,
    pin_skl_alpha_zero_is_forward_kl,
    pin_skew_losses_torch_autograd,
    pin_skew_losses_brute_force_and_finite_differences,
    pin_skew_losses_bounds_and_limits,
    pin_skew_losses_invariants,
    pin_topk_rkl_scipy_entropy,
    pin_topk_rkl_torch_autograd,
    pin_topk_rkl_brute_force_and_finite_differences,
    pin_topk_rkl_closed_forms_and_invariants,
]
