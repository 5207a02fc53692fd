"""Plain fp64 CPU oracle of the fused chunked KL loss (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module. It shares no code with the GPU path.

What it computes
----------------
The pages describe three ways to compute one and the same distillation loss
and call them mathematically equivalent; the textbook dense KL is their
correctness baseline [P1 "Making knowledge distillation cheap enough to run at
scale", section "Two system changes", the three bullets]. The oracle is that
definition written out in fp64:

* student logits ``z_i = W . H_i`` over the full vocabulary (the output
  projection that the fused loss folds into the loss, same section, fused
  chunked KL bullet); tempered ``s_i = z_i / T``;
  ``log q_i = s_i - logsumexp(s_i)`` (full-vocabulary log-softmax);
* teacher: the cached top-K (id, logit) pairs of each position [same page,
  "Two system changes", offline distillation paragraph]; probability mass is
  zero outside the top-K and the K logits are renormalised with a softmax at
  temperature T: ``p_i = softmax(l_i / T)``;
* per-position forward KL ``KL_i = sum_k p_ik (log p_ik - log q_i[id_ik])``;
* ``loss = (1/N) sum_i KL_i`` (mean over positions).

Ignored positions (reading; the pages only mention ablations on sequence
packing [P1, section "The resulting student model", last paragraphs]): a
position whose first teacher id is ``IGNORE_ID`` (-1) has no teacher target,
as at padding or packing boundaries. It contributes nothing: KL_i = 0, a zero
gradient row, and the mean runs over the positions that are kept (N is their
number below; with none kept the loss is NaN and every gradient is zero). The
other entries of an ignored row are never used.

Teacher ids that break the pages' setting of K distinct in-vocabulary ids per
position (readings; the pages only describe a cache of the teacher's top 100
tokens per position [P1, "Two system changes", offline distillation
paragraph]):

* an id outside [0, V) keeps its share of the teacher's softmax over K, but
  the student has no entry for it: its gathered student logit reads as 0 and
  it is not part of the student's normalisation, so its term is
  ``p_k (log p_k + lse_i)``, and it adds nothing to the gradient's scatter;
* a repeated id is gathered once per entry (the loss is read entry by entry:
  ``sum_k p_k (log p_k - log q_i[id_k])``) and the scatter adds its masses.

The dense-grid baseline (``dense_kl_loss``) cannot hold either case the same
way: its grid merges repeated ids into one probability ``P_v`` and has no
cell for an id outside [0, V), so it computes ``sum_v P_v (log P_v - log
q_v)`` over the grid. The two agree whenever a position's ids are distinct and
in range; the gradients agree always.

Gradient (derived here; the pages say a closed form exists but do not print
it [P1, section "The resulting student model", last paragraph]): with
upstream scalar ``g``,
``dZ_i = g / (N T) * (softmax(s_i) - scatter_add(ids_i, p_i))``,
``dH = dZ W`` and ``dW = dZ^T H``.

Readings where the pages are silent (temperature on both sides with no T**2
factor, forward KL direction, mean reduction, duplicate ids add their mass)
are listed with the rest of the design notes.

Alternative losses on the same distributions (readings: the pages report
ablations on the choice of loss without naming them [P1, section "The
resulting student model", last paragraphs]): the generalised Jensen-Shannon
divergence, the skew KL and the skew reverse KL, in their own section below.

Rows are processed in blocks only to bound memory; rows are independent, so
the block size does not enter the result except through summation order.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Tuple

import numpy as np

__all__ = [
    "teacher_distribution",
    "student_log_softmax",
    "forward",
    "backward",
    "loss_and_grads",
    "dense_kl_loss",
    "sampled_rows",
    "dw_rows",
    "logits_forward",
    "logits_backward",
    "logits_sampled_rows",
    "kept_positions",
    "IGNORE_ID",
    "jsd_forward",
    "jsd_backward",
    "jsd_loss_and_grads",
    "ALT_LOSSES",
    "alt_forward",
    "alt_backward",
    "alt_loss_and_grads",
    "topk_rkl_forward",
    "topk_rkl_backward",
    "topk_rkl_loss_and_grads",
    "topk_rkl_sampled",
]


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (fp32/bf16) or array to fp64 numpy."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _ids(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


IGNORE_ID = -1


def kept_positions(ids) -> np.ndarray:
    """Boolean [N]: positions whose first teacher id is not IGNORE_ID."""
    ids = _ids(ids)
    return ids[:, 0] != IGNORE_ID if ids.shape[0] else np.zeros(0, dtype=bool)


def _usable_ids(ids: np.ndarray, kept: np.ndarray) -> np.ndarray:
    # ignored rows may hold anything; give them harmless indices (their
    # results are discarded)
    return np.where(kept[:, None], ids, 0)


def _in_vocab(ids_rows: np.ndarray, V: int) -> np.ndarray:
    """Boolean mask of the ids that name a vocabulary entry."""
    return (ids_rows >= 0) & (ids_rows < V)


def _logq_at(logq: np.ndarray, lse: np.ndarray, ids_rows: np.ndarray) -> np.ndarray:
    """log q_i[id_ik] for each teacher entry; an id outside [0, V) has no
    student entry, its tempered logit reads as 0, so its value is -lse_i."""
    ok = _in_vocab(ids_rows, logq.shape[1])
    at = np.take_along_axis(logq, np.where(ok, ids_rows, 0), axis=1)
    return np.where(ok, at, -lse[:, None])


def _logsumexp_rows(a: np.ndarray) -> np.ndarray:
    m = a.max(axis=1, keepdims=True)
    return m[:, 0] + np.log(np.exp(a - m).sum(axis=1))


def teacher_distribution(topk_logits, T: float) -> Tuple[np.ndarray, np.ndarray]:
    """Teacher top-K renormalised at temperature T: returns (p, log p), [N, K].

    The cache keeps the teacher's top-K tokens per position [P1, "Two system
    changes", offline distillation paragraph]; outside them the teacher mass
    is taken as zero and the K logits are renormalised with a softmax.
    """
    a = _f64(topk_logits) / float(T)
    logp = a - _logsumexp_rows(a)[:, None]
    return np.exp(logp), logp


def student_log_softmax(H_rows, W, T: float) -> Tuple[np.ndarray, np.ndarray]:
    """Full-vocabulary student log-softmax of ``z = H W^T`` at temperature T.

    Returns (log q [rows, V], lse [rows]) with ``lse = logsumexp(z / T)``.
    """
    s = (_f64(H_rows) @ _f64(W).T) / float(T)
    lse = _logsumexp_rows(s)
    return s - lse[:, None], lse


def forward(H, W, ids, logits, T: float, block: int = 256) -> Dict[str, object]:
    """Loss, per-row logsumexp of z/T and per-row KL.

    Returns dict(loss=float, row_lse=[N], row_kl=[N]) in fp64.
    """
    H = _f64(H)
    W = _f64(W)
    ids = _ids(ids)
    n_rows = H.shape[0]
    kept = kept_positions(ids)
    ids = _usable_ids(ids, kept)
    row_lse = np.empty(n_rows)
    row_kl = np.empty(n_rows)
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        logq, lse = student_log_softmax(H[r0:r1], W, T)
        p, logp = teacher_distribution(logits[r0:r1], T)
        logq_at = _logq_at(logq, lse, ids[r0:r1])
        row_kl[r0:r1] = (p * (logp - logq_at)).sum(axis=1)
        row_lse[r0:r1] = lse
    row_kl[~kept] = 0.0
    N = int(kept.sum())  # the mean runs over the kept positions
    loss = math.fsum(row_kl.tolist()) / N if N else float("nan")
    return {"loss": loss, "row_lse": row_lse, "row_kl": row_kl}


def _dz_rows(H_rows, W, ids_rows, logits_rows, T, coef):
    logq, _ = student_log_softmax(H_rows, W, T)
    q = np.exp(logq)
    p, _ = teacher_distribution(logits_rows, T)
    target = np.zeros_like(q)
    # scatter-add of the teacher mass onto the ids that name a vocabulary
    # entry (repeated ids add up; an id outside [0, V) adds nothing)
    rows = np.repeat(np.arange(q.shape[0]), p.shape[1])
    ok = _in_vocab(ids_rows, q.shape[1]).reshape(-1)
    np.add.at(target, (rows[ok], ids_rows.reshape(-1)[ok]), p.reshape(-1)[ok])
    return coef * (q - target)


def backward(H, W, ids, logits, T: float, g: float = 1.0,
             block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients (dH [N, d], dW [V, d]) of ``g * loss`` in fp64."""
    H = _f64(H)
    W = _f64(W)
    ids = _ids(ids)
    n_rows = H.shape[0]
    kept = kept_positions(ids)
    ids = _usable_ids(ids, kept)
    N = int(kept.sum())  # the mean runs over the kept positions
    coef = float(g) / (N * float(T)) if N else 0.0
    dH = np.empty_like(H)
    dW = np.zeros_like(W)
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        dZ = _dz_rows(H[r0:r1], W, ids[r0:r1], logits[r0:r1], T, coef)
        dZ[~kept[r0:r1]] = 0.0
        dH[r0:r1] = dZ @ W
        dW += dZ.T @ H[r0:r1]
    return dH, dW


def loss_and_grads(H, W, ids, logits, T: float, g: float = 1.0,
                   block: int = 256) -> Dict[str, object]:
    out = forward(H, W, ids, logits, T, block)
    out["dH"], out["dW"] = backward(H, W, ids, logits, T, g, block)
    return out


def dense_kl_loss(H, W, ids, logits, T: float) -> float:
    """The pages' dense baseline on a tiny problem: build the full teacher
    probability grid (zeros off the top-K) and the full student log-prob grid,
    then sum ``P (log P - log Q)`` over the grid where P > 0, divided by N
    [P1, "Two system changes", dense KL bullet]. Repeated ids share one grid
    cell (their masses add); ids outside [0, V) have no cell."""
    H = _f64(H)
    W = _f64(W)
    ids = _ids(ids)
    N, K = ids.shape
    V = W.shape[0]
    kept = kept_positions(ids)
    a = _f64(logits) / float(T)
    P = np.zeros((N, V))
    for i in range(N):
        if not kept[i]:
            continue
        e = np.exp(a[i] - a[i].max())
        for k in range(K):
            if 0 <= ids[i, k] < V:  # the grid has no cell for other ids
                P[i, ids[i, k]] += e[k] / e.sum()
    Z = H @ W.T / float(T)
    logQ = np.empty_like(Z)
    for i in range(N):
        m = Z[i].max()
        logQ[i] = Z[i] - (m + math.log(np.exp(Z[i] - m).sum()))
    total = 0.0
    for i in range(N):
        for v in range(V):
            if P[i, v] > 0:
                total += P[i, v] * (math.log(P[i, v]) - logQ[i, v])
    n_kept = int(kept.sum())
    return total / n_kept if n_kept else float("nan")


def sampled_rows(H, W, ids, logits, T: float, rows: Iterable[int],
                 N_total: int, g: float = 1.0) -> Dict[str, np.ndarray]:
    """Per-row results for a few rows of a large problem, one row at a time.

    Returns dict(rows, row_lse, row_kl, dH_rows) where ``dH_rows`` are the rows
    of the gradient of ``g * loss`` for a problem of ``N_total`` kept
    positions.
    """
    rows = np.asarray(list(rows), dtype=np.int64)
    Wf = _f64(W)
    coef = float(g) / (N_total * float(T)) if N_total else 0.0
    lse_out = np.empty(rows.size)
    kl_out = np.empty(rows.size)
    dh_out = np.empty((rows.size, Wf.shape[1]))
    for j, r in enumerate(rows.tolist()):
        Hr = _f64(H[r:r + 1])
        idr = _ids(ids[r:r + 1])
        lgr = _f64(logits[r:r + 1])
        logq, lse = student_log_softmax(Hr, Wf, T)
        lse_out[j] = lse[0]
        if not kept_positions(idr)[0]:
            kl_out[j] = 0.0
            dh_out[j] = 0.0
            continue
        p, logp = teacher_distribution(lgr, T)
        kl_out[j] = (p * (logp - _logq_at(logq, lse, idr))).sum()
        dz = _dz_rows(Hr, Wf, idr, lgr, T, coef)
        dh_out[j] = (dz @ Wf)[0]
    return {"rows": rows, "row_lse": lse_out, "row_kl": kl_out, "dH_rows": dh_out}


def dw_rows(H, W, ids, logits, T: float, vrows: Iterable[int], row_lse,
            g: float = 1.0) -> np.ndarray:
    """Rows ``vrows`` of dW for the whole problem, given every position's
    logsumexp of z/T (``row_lse``, as written by ``forward``):
    ``dW_v = sum_n dZ_nv H_n`` with ``dZ_nv = g/(N T) (exp(z_nv/T - lse_n)
    - P_nv)`` and ``P_nv`` the teacher mass on id v (same definition as
    ``backward``, evaluated one vocabulary row at a time)."""
    Hf = _f64(H)
    ids_ = _ids(ids)
    kept = kept_positions(ids_)
    vrows = np.asarray(list(vrows), dtype=np.int64)
    N = int(kept.sum())  # the mean runs over the kept positions
    coef = float(g) / (N * float(T)) if N else 0.0
    Wv = _f64(W[vrows])  # [nv, d]
    p, _ = teacher_distribution(logits, T)
    lse = np.asarray(row_lse, dtype=np.float64)
    out = np.zeros((vrows.size, Hf.shape[1]))
    for j, v in enumerate(vrows.tolist()):
        z = Hf @ Wv[j] / float(T)
        P = (p * (ids_ == v)).sum(axis=1)
        dz = coef * (np.exp(z - lse) - P)
        dz[~kept] = 0.0
        out[j] = dz @ Hf
    return out


# ---------------------------------------------------------------------------
# Forward-chunked KL: the student's logit grid is given.
# ---------------------------------------------------------------------------
# The pages' middle variant keeps the teacher sparse (its cached top-K per
# position, never expanded to the dense grid) and computes the loss slice by
# slice over positions, while the student's own logits are computed in full
# by the output layer and kept for the backward pass [P1 "Making knowledge
# distillation cheap enough to run at scale", section "Two system changes",
# forward-chunked KL bullet]. The loss is the same one as above, with
# ``z_i = Z_i`` read from the given grid instead of ``W . H_i``; the caller's
# output layer turns dZ into its own gradients.
#
# Written here in the arrangement ``KL_i = e_i - gamma_i + lse_i`` with
# ``e_i = sum_k p_ik log p_ik`` and ``gamma_i = sum_k p_ik s_i[id_ik]``
# (equal to ``sum_k p_ik (log p_ik - log q_i[id_ik])`` because the p_ik sum
# to one), which is independent of the arithmetic of ``forward`` above.
# An id outside [0, V) contributes nothing to gamma_i or to the scatter of
# the gradient (its teacher mass is dropped), the convention of the library.


def _valid_ids(ids_rows: np.ndarray, V: int) -> np.ndarray:
    return (ids_rows >= 0) & (ids_rows < V)


def logits_forward(Z, ids, logits, T: float, block: int = 256) -> Dict[str, object]:
    """Loss, per-row logsumexp of Z/T and per-row KL from the logit grid
    ``Z [N, V]``; returns dict(loss, row_lse, row_kl) in fp64."""
    Z = _f64(Z)
    ids = _ids(ids)
    n_rows, V = Z.shape
    kept = kept_positions(ids)
    ids = _usable_ids(ids, kept)
    row_lse = np.empty(n_rows)
    row_kl = np.empty(n_rows)
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        s = Z[r0:r1] / float(T)
        lse = _logsumexp_rows(s)
        p, logp = teacher_distribution(logits[r0:r1], T)
        idr = ids[r0:r1]
        ok = _valid_ids(idr, V)
        s_at = np.take_along_axis(s, np.where(ok, idr, 0), axis=1)
        e = (p * logp).sum(axis=1)
        gamma = (p * np.where(ok, s_at, 0.0)).sum(axis=1)
        row_kl[r0:r1] = e - gamma + lse
        row_lse[r0:r1] = lse
    row_kl[~kept] = 0.0
    N = int(kept.sum())  # the mean runs over the kept positions
    loss = math.fsum(row_kl.tolist()) / N if N else float("nan")
    return {"loss": loss, "row_lse": row_lse, "row_kl": row_kl}


def logits_backward(Z, ids, logits, T: float, g: float = 1.0, block: int = 256) -> np.ndarray:
    """Gradient ``dZ [N, V]`` of ``g * loss`` with respect to the logit grid:
    ``dZ_i = g / (N T) * (softmax(Z_i / T) - scatter_add(ids_i, p_i))``."""
    Z = _f64(Z)
    ids = _ids(ids)
    n_rows, V = Z.shape
    kept = kept_positions(ids)
    ids = _usable_ids(ids, kept)
    N = int(kept.sum())  # the mean runs over the kept positions
    scale = float(g) / (N * float(T)) if N else 0.0
    dZ = np.empty_like(Z)
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        s = Z[r0:r1] / float(T)
        q = np.exp(s - _logsumexp_rows(s)[:, None])
        p, _ = teacher_distribution(logits[r0:r1], T)
        idr = ids[r0:r1]
        ok = _valid_ids(idr, V)
        P = np.zeros_like(q)
        rr, kk = np.nonzero(ok)
        np.add.at(P, (rr, idr[rr, kk]), p[rr, kk])
        dZ[r0:r1] = scale * (q - P)
        dZ[r0:r1][~kept[r0:r1]] = 0.0
    return dZ


def logits_sampled_rows(Z, ids, logits, T: float, rows: Iterable[int], N_total: int,
                        g: float = 1.0) -> Dict[str, np.ndarray]:
    """``logits_forward`` / ``logits_backward`` restricted to a few rows of a
    large grid (one row at a time); dZ rows are those of a problem with
    ``N_total`` kept positions."""
    rows = [int(r) for r in rows]
    out_lse, out_kl, out_dz = [], [], []
    for r in rows:
        Zr = _f64(Z[r:r + 1])
        f = logits_forward(Zr, ids[r:r + 1], logits[r:r + 1], T)
        dz = logits_backward(Zr, ids[r:r + 1], logits[r:r + 1], T, g)
        out_lse.append(f["row_lse"][0])
        out_kl.append(f["row_kl"][0])
        out_dz.append(dz[0] / N_total if N_total else 0.0 * dz[0])  # logits_backward divided by N = 1
    return {"rows": np.asarray(rows), "row_lse": np.asarray(out_lse),
            "row_kl": np.asarray(out_kl), "dZ_rows": np.stack(out_dz) if out_dz else np.zeros((0, 0))}


# ---------------------------------------------------------------------------
# An alternative loss on the same inputs: the generalised Jensen-Shannon
# divergence between the teacher's top-K distribution and the student.
# ---------------------------------------------------------------------------
# The pages report ablations on the choice of loss function for the
# distilled student without naming the losses [P1 "Making knowledge
# distillation cheap enough to run at scale", section "The resulting student
# model"]. The loss taken here (a reading) is the generalised Jensen-Shannon
# divergence with weight beta in (0, 1), with the same teacher and student
# distributions as the KL above:
#
#   P_i  = the teacher's top-K probabilities softmax(l_i / T) placed on the
#          vocabulary (repeated ids add their mass; ids outside [0, V) have
#          no vocabulary entry and their mass is left out),
#   q_i  = softmax(z_i / T) over the full vocabulary,
#   M_i  = beta P_i + (1 - beta) q_i,
#   JSD_i = beta KL(P_i || M_i) + (1 - beta) KL(q_i || M_i),
#
# beta = 1/2 being the symmetric Jensen-Shannon divergence; for small beta,
# JSD_i / beta tends to the forward KL above. The loss is the mean over the
# kept positions, and ignored positions (first id IGNORE_ID) are treated as
# above. Gradient (derived here): with g_v = (1 - beta) log(q_v / M_v) and
# gbar = sum_v q_v g_v, d JSD_i / d s_v = q_v (g_v - gbar), hence
# dZ_i = g / (N T) * q_i * (g_i - gbar_i), dH = dZ W, dW = dZ^T H.


def _teacher_grid(ids_rows: np.ndarray, logits_rows, T: float, V: int) -> np.ndarray:
    """Teacher probabilities on the vocabulary, [rows, V]."""
    p, _ = teacher_distribution(logits_rows, T)
    P = np.zeros((ids_rows.shape[0], V))
    ok = _in_vocab(ids_rows, V)
    rr, kk = np.nonzero(ok)
    np.add.at(P, (rr, ids_rows[rr, kk]), p[rr, kk])
    return P


def _jsd_parts(logq: np.ndarray, P: np.ndarray, beta: float):
    """Per row: (JSD, q, g) with log M formed in the log domain (exact zeros
    of P stay out of the teacher term)."""
    with np.errstate(divide="ignore"):
        logP = np.log(P)
    logM = np.logaddexp(math.log(beta) + logP, math.log1p(-beta) + logq)
    q = np.exp(logq)
    on = P > 0
    kl_p = np.where(on, P * (np.where(on, logP, 0.0) - logM), 0.0).sum(axis=1)
    g = (1.0 - beta) * (logq - logM)
    kl_q = (q * (logq - logM)).sum(axis=1)
    return beta * kl_p + (1.0 - beta) * kl_q, q, g


def _check_beta(beta: float) -> float:
    beta = float(beta)
    if not 0.0 < beta < 1.0:
        raise ValueError("beta must lie in (0, 1)")
    return beta


# ---------------------------------------------------------------------------
# Two more alternative losses of the same kind: the skew KL and the skew
# reverse KL divergences between the teacher's top-K distribution and the
# student (readings like the JSD above: the pages name no loss).
# ---------------------------------------------------------------------------
# With P_i and q_i as above and a parameter alpha:
#
#   SKL_i  = KL(P_i || alpha P_i + (1 - alpha) q_i),        0 <= alpha < 1,
#   SRKL_i = KL(q_i || alpha q_i + (1 - alpha) P_i),        0 < alpha <= 1.
#
# The skew KL at alpha = 0 is the forward KL above (for rows whose teacher
# ids are all in range). The skew reverse KL stays finite although P_i is
# zero off the top-K (there its mixture is alpha q_i), and tends to the
# reverse KL(q_i || P_i) as alpha -> 0 where P_i covers the vocabulary.
# Since each mixture is at least alpha times the distribution in front,
# both are at most -log(alpha) per position. The loss is the mean over the
# kept positions, ignored positions as above. Gradient (derived here), of the
# JSD's form: d L_i / d s_v = q_v (g_v - gbar_i), gbar_i = sum_v q_v g_v, with
# g_v the derivative of L_i in q_v:
#
#   SKL:  g_v = -(1 - alpha) P_v / M_v                  (0 where P_v = 0),
#   SRKL: g_v = log(q_v / M_v) + 1 - alpha q_v / M_v    (-log alpha where P_v = 0).


def _skl_parts(logq: np.ndarray, P: np.ndarray, alpha: float):
    """Per row: (SKL, q, g), M = alpha P + (1 - alpha) q in the log domain."""
    with np.errstate(divide="ignore"):
        logP = np.log(P)
    la = math.log(alpha) if alpha > 0.0 else -math.inf
    logM = np.logaddexp(la + logP, math.log1p(-alpha) + logq)
    on = P > 0
    lp = np.where(on, logP, 0.0)
    loss = np.where(on, P * (lp - logM), 0.0).sum(axis=1)
    g = np.where(on, -(1.0 - alpha) * np.exp(lp - logM), 0.0)
    return loss, np.exp(logq), g


def _srkl_parts(logq: np.ndarray, P: np.ndarray, alpha: float):
    """Per row: (SRKL, q, g), M = alpha q + (1 - alpha) P in the log domain
    (M >= alpha q > 0, so log(q / M) is finite everywhere)."""
    with np.errstate(divide="ignore"):
        logP = np.log(P)
    lb = math.log1p(-alpha) if alpha < 1.0 else -math.inf
    logM = np.logaddexp(math.log(alpha) + logq, lb + logP)
    q = np.exp(logq)
    r = logq - logM  # log(q / M)
    loss = (q * r).sum(axis=1)
    g = r + 1.0 - alpha * np.exp(r)
    return loss, q, g


# loss name -> (per-row parts, admissible parameter range as a predicate)
ALT_LOSSES = {
    "jsd": (_jsd_parts, lambda a: 0.0 < a < 1.0),
    "skl": (_skl_parts, lambda a: 0.0 <= a < 1.0),
    "srkl": (_srkl_parts, lambda a: 0.0 < a <= 1.0),
}


def _check_alt(loss: str, a: float):
    if loss not in ALT_LOSSES:
        raise ValueError(f"unknown loss {loss!r}")
    parts, ok = ALT_LOSSES[loss]
    a = float(a)
    if not ok(a):
        raise ValueError(f"parameter {a} out of range for {loss}")
    return parts, a


def alt_forward(H, W, ids, logits, T: float, loss: str, a: float, block: int = 256) -> Dict[str, object]:
    """Loss, per-row logsumexp of z/T and per-row value of an alternative
    loss ("jsd": weight beta = a; "skl", "srkl": alpha = a); fp64."""
    parts, a = _check_alt(loss, a)
    H = _f64(H)
    W = _f64(W)
    ids = _ids(ids)
    lg = _f64(logits)
    n_rows, V = H.shape[0], W.shape[0]
    kept = kept_positions(ids)
    ids = _usable_ids(ids, kept)
    row_lse = np.empty(n_rows)
    row_kl = np.empty(n_rows)
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        logq, lse = student_log_softmax(H[r0:r1], W, T)
        P = _teacher_grid(ids[r0:r1], lg[r0:r1], T, V)
        row_kl[r0:r1], _, _ = parts(logq, P, a)
        row_lse[r0:r1] = lse
    row_kl[~kept] = 0.0
    N = int(kept.sum())  # the mean runs over the kept positions
    loss_v = math.fsum(row_kl.tolist()) / N if N else float("nan")
    return {"loss": loss_v, "row_lse": row_lse, "row_kl": row_kl}


def alt_backward(H, W, ids, logits, T: float, loss: str, a: float, g: float = 1.0,
                 block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients (dH [N, d], dW [V, d]) of ``g * loss`` for an alternative
    loss; fp64."""
    parts, a = _check_alt(loss, a)
    H = _f64(H)
    W = _f64(W)
    ids = _ids(ids)
    lg = _f64(logits)
    n_rows, V = H.shape[0], W.shape[0]
    kept = kept_positions(ids)
    ids = _usable_ids(ids, kept)
    N = int(kept.sum())
    coef = float(g) / (N * float(T)) if N else 0.0
    dH = np.empty_like(H)
    dW = np.zeros_like(W)
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        logq, _ = student_log_softmax(H[r0:r1], W, T)
        P = _teacher_grid(ids[r0:r1], lg[r0:r1], T, V)
        _, q, gv = parts(logq, P, a)
        gbar = (q * gv).sum(axis=1)
        dZ = coef * q * (gv - gbar[:, None])
        dZ[~kept[r0:r1]] = 0.0
        dH[r0:r1] = dZ @ W
        dW += dZ.T @ H[r0:r1]
    return dH, dW


def alt_loss_and_grads(H, W, ids, logits, T: float, loss: str, a: float, g: float = 1.0,
                       block: int = 256) -> Dict[str, object]:
    out = alt_forward(H, W, ids, logits, T, loss, a, block)
    out["dH"], out["dW"] = alt_backward(H, W, ids, logits, T, loss, a, g, block)
    return out


def jsd_forward(H, W, ids, logits, T: float, beta: float = 0.5, block: int = 256) -> Dict[str, object]:
    """Loss, per-row logsumexp of z/T and per-row JSD_beta; fp64."""
    return alt_forward(H, W, ids, logits, T, "jsd", _check_beta(beta), block)


def jsd_backward(H, W, ids, logits, T: float, beta: float = 0.5, g: float = 1.0,
                 block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients (dH [N, d], dW [V, d]) of ``g * loss`` for JSD_beta; fp64."""
    return alt_backward(H, W, ids, logits, T, "jsd", _check_beta(beta), g, block)


def jsd_loss_and_grads(H, W, ids, logits, T: float, beta: float = 0.5, g: float = 1.0,
                       block: int = 256) -> Dict[str, object]:
    return alt_loss_and_grads(H, W, ids, logits, T, "jsd", beta, g, block)


# ---------------------------------------------------------------------------
# Reverse KL over the teacher's top-K support (a reading: the pages report
# ablations on the choice of loss without naming the losses [P1 "Making
# knowledge distillation cheap enough to run at scale", section "The
# resulting student model"]).
# ---------------------------------------------------------------------------
# The reverse KL(q || P) is infinite wherever the student puts mass off the
# teacher's top-K, so it is taken over the support: with P_i the teacher's
# probabilities on the vocabulary as above (repeated ids add their mass, ids
# outside [0, V) have none) and S_i = {v : P_iv > 0}, the student's
# distribution is restricted to S_i and renormalised there,
#
#   qt_iv = exp(s_iv) / sum_{u in S_i} exp(s_iu)       (v in S_i),
#   TRKL_i = KL(qt_i || P_i) = sum_{v in S_i} qt_iv (log qt_iv - log P_iv),
#
# and 0 for a position whose support is empty. It depends on the student's
# logits at S_i only. The loss is the mean over the kept positions (ignored
# positions as above). Gradient (derived here): with r_v = log(qt_v / P_v),
# d TRKL_i / d s_v = qt_v (r_v - TRKL_i) on S_i and 0 off it, so
# dZ_i = g / (N T) * that, dH = dZ W, dW = dZ^T H.


def _topk_rkl_parts(s: np.ndarray, P: np.ndarray):
    """Per row: (TRKL, logsumexp of s over the support, dTRKL/ds) from the
    tempered student logits ``s`` and the teacher grid ``P`` ([rows, V])."""
    on = P > 0
    has = on.any(axis=1)
    s_on = np.where(on, s, -np.inf)
    m = np.where(has, s_on.max(axis=1), 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(has, m + np.log(np.exp(s_on - m[:, None]).sum(axis=1)), -np.inf)
        logP = np.where(on, np.log(np.where(on, P, 1.0)), 0.0)
    log_qt = np.where(on, s - np.where(has, lse, 0.0)[:, None], 0.0)
    qt = np.where(on, np.exp(log_qt), 0.0)
    r = np.where(on, log_qt - logP, 0.0)
    loss = (qt * r).sum(axis=1)
    grad = qt * (r - loss[:, None])
    return loss, lse, grad


def topk_rkl_forward(H, W, ids, logits, T: float, block: int = 256) -> Dict[str, object]:
    """Loss, per-row logsumexp of s = z/T over the teacher's support, and
    per-row TRKL; fp64 (the student logits formed in full, then restricted)."""
    H = _f64(H)
    W = _f64(W)
    ids = _ids(ids)
    lg = _f64(logits)
    n_rows, V = H.shape[0], W.shape[0]
    kept = kept_positions(ids)
    ids = _usable_ids(ids, kept)
    row_lse = np.empty(n_rows)
    row_kl = np.empty(n_rows)
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        s = (H[r0:r1] @ W.T) / float(T)
        P = _teacher_grid(ids[r0:r1], lg[r0:r1], T, V)
        row_kl[r0:r1], row_lse[r0:r1], _ = _topk_rkl_parts(s, P)
    row_kl[~kept] = 0.0
    N = int(kept.sum())  # the mean runs over the kept positions
    loss_v = math.fsum(row_kl.tolist()) / N if N else float("nan")
    return {"loss": loss_v, "row_lse": row_lse, "row_kl": row_kl}


def topk_rkl_backward(H, W, ids, logits, T: float, g: float = 1.0,
                      block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients (dH [N, d], dW [V, d]) of ``g * loss`` for TRKL; fp64."""
    H = _f64(H)
    W = _f64(W)
    ids = _ids(ids)
    lg = _f64(logits)
    n_rows, V = H.shape[0], W.shape[0]
    kept = kept_positions(ids)
    ids = _usable_ids(ids, kept)
    N = int(kept.sum())
    coef = float(g) / (N * float(T)) if N else 0.0
    dH = np.empty_like(H)
    dW = np.zeros_like(W)
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        s = (H[r0:r1] @ W.T) / float(T)
        P = _teacher_grid(ids[r0:r1], lg[r0:r1], T, V)
        _, _, grad = _topk_rkl_parts(s, P)
        dZ = coef * grad
        dZ[~kept[r0:r1]] = 0.0
        dH[r0:r1] = dZ @ W
        dW += dZ.T @ H[r0:r1]
    return dH, dW


def topk_rkl_loss_and_grads(H, W, ids, logits, T: float, g: float = 1.0,
                            block: int = 256) -> Dict[str, object]:
    out = topk_rkl_forward(H, W, ids, logits, T, block)
    out["dH"], out["dW"] = topk_rkl_backward(H, W, ids, logits, T, g, block)
    return out


def topk_rkl_sampled(H, W, ids, logits, T: float, rows: Iterable[int], vrows: Iterable[int],
                     g: float = 1.0) -> Dict[str, np.ndarray]:
    """TRKL results for a few rows of a large problem, and rows ``vrows`` of
    dW. The loss depends on the student's logits at the support only, so
    each needed position's logits are formed at its own ids (the same
    values as the full row, without the rest of it): per sampled position
    its logsumexp over the support, TRKL and dH row; each dW row sums the
    positions whose support holds it. The gradient scale counts every kept
    position of the problem."""
    Wf = _f64(W)
    ids_all = _ids(ids)
    lg_all = _f64(logits)
    kept = kept_positions(ids_all)
    N = int(kept.sum())
    coef = float(g) / (N * float(T)) if N else 0.0
    V = Wf.shape[0]

    def row_parts(r):
        idr = ids_all[r]
        if not kept[r]:
            return None
        p, _ = teacher_distribution(lg_all[r:r + 1], T)
        sup = sorted({int(v) for v in idr if 0 <= v < V})
        Pv = np.array([p[0][idr == v].sum() for v in sup])
        on = Pv > 0
        sup = [v for v, o in zip(sup, on) if o]
        Pv = Pv[on]
        if not sup:
            return sup, np.zeros(0), -np.inf, 0.0
        s = (Wf[sup] @ _f64(H[r:r + 1])[0]) / float(T)
        m = s.max()
        lse = m + math.log(np.exp(s - m).sum())
        qt = np.exp(s - lse)
        rv = (s - lse) - np.log(Pv)
        L = float((qt * rv).sum())
        return sup, coef * qt * (rv - L), lse, L

    rows = np.asarray(list(rows), dtype=np.int64)
    lse_out = np.empty(rows.size)
    kl_out = np.zeros(rows.size)
    dh_out = np.zeros((rows.size, Wf.shape[1]))
    for j, r in enumerate(rows.tolist()):
        parts = row_parts(r)
        if parts is None:
            lse_out[j] = np.nan  # not written for an ignored position
            continue
        sup, dz, lse_out[j], kl_out[j] = parts
        if sup:
            dh_out[j] = dz @ Wf[sup]
    vrows = np.asarray(list(vrows), dtype=np.int64)
    dw_out = np.zeros((vrows.size, Wf.shape[1]))
    for j, v in enumerate(vrows.tolist()):
        for r in np.nonzero((ids_all == v).any(axis=1) & kept)[0].tolist():
            sup, dz, _, _ = row_parts(r)
            if v in sup:
                dw_out[j] += dz[sup.index(v)] * _f64(H[r:r + 1])[0]
    return {"rows": rows, "row_lse": lse_out, "row_kl": kl_out, "dH_rows": dh_out, "dW_rows": dw_out}
