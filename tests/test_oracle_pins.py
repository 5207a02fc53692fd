"""The CPU oracle, pinned to closed forms, library routines, finite
differences and invariants; plus mutation checks showing that plausible
mistakes in the oracle (a dropped term, a wrong sign, a misplaced temperature,
a misaligned gather) fail at least one pin."""
import importlib.util
import os
import sys
import types

import numpy as np
import pytest

from oracle import kl as oracle_kl
from tests import _pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_kl)


# (name, original text, replacement) applied to oracle/kl.py's source
MUTANTS = [
    ("drop_teacher_entropy", "(p * (logp - logq_at))", "(p * (-logq_at))"),
    ("kl_sign_flipped", "(p * (logp - logq_at))", "(p * (logq_at - logp))"),
    ("teacher_no_temperature", "a = _f64(topk_logits) / float(T)", "a = _f64(topk_logits)"),
    ("student_no_temperature", "s = (_f64(H_rows) @ _f64(W).T) / float(T)",
     "s = (_f64(H_rows) @ _f64(W).T)"),
    ("teacher_not_renormalised", "logp = a - _logsumexp_rows(a)[:, None]", "logp = a - a.max()"),
    ("grad_missing_T", "coef = float(g) / (N * float(T))", "coef = float(g) / N"),
    ("gather_sorted_ids", "np.add.at(target, (rows[ok], ids_rows.reshape(-1)[ok]), p.reshape(-1)[ok])",
     "np.add.at(target, (rows[ok], np.sort(ids_rows, axis=1).reshape(-1)[ok]), p.reshape(-1)[ok])"),
    ("dW_wrong_operand", "dW += dZ.T @ H[r0:r1]", "dW += dZ.T @ (H[r0:r1] * 0.5)"),
    ("sum_not_mean", "loss = math.fsum(row_kl.tolist()) / N if N",
     "loss = math.fsum(row_kl.tolist()) if N"),
    # teacher ids outside [0, V) and repeated ids (fused functions)
    ("fused_gather_wraps_ids",
     "at = np.take_along_axis(logq, np.where(ok, ids_rows, 0), axis=1)\n    return np.where(ok, at, -lse[:, None])",
     "return np.take_along_axis(logq, ids_rows % logq.shape[1], axis=1)"),
    ("fused_dropped_entry_without_lse", "return np.where(ok, at, -lse[:, None])", "return np.where(ok, at, 0.0)"),
    ("fused_scatter_clips_ids",
     "np.add.at(target, (rows[ok], ids_rows.reshape(-1)[ok]), p.reshape(-1)[ok])",
     "np.add.at(target, (rows, np.clip(ids_rows, 0, q.shape[1] - 1).reshape(-1)), p.reshape(-1))"),
    ("dense_grid_wraps_negative_ids", "if 0 <= ids[i, k] < V:  # the grid", "if ids[i, k] < V:  # the grid"),
    # forward-chunked KL (logit grid given)
    ("logits_drop_entropy", "row_kl[r0:r1] = e - gamma + lse", "row_kl[r0:r1] = -gamma + lse"),
    ("logits_gamma_sign", "row_kl[r0:r1] = e - gamma + lse", "row_kl[r0:r1] = e + gamma + lse"),
    ("logits_gather_no_T", "s_at = np.take_along_axis(s, np.where(ok, idr, 0), axis=1)",
     "s_at = np.take_along_axis(Z[r0:r1], np.where(ok, idr, 0), axis=1)"),
    ("logits_keep_dropped_ids", "gamma = (p * np.where(ok, s_at, 0.0)).sum(axis=1)",
     "gamma = (p * s_at).sum(axis=1)"),
    ("logits_grad_no_T", "scale = float(g) / (N * float(T))", "scale = float(g) / N"),
    ("logits_grad_no_teacher", "dZ[r0:r1] = scale * (q - P)", "dZ[r0:r1] = scale * q"),
    ("logits_scatter_first_id_only", "rr, kk = np.nonzero(ok)", "rr, kk = np.nonzero(ok[:, :1])"),
    # the alternative loss (generalised Jensen-Shannon divergence)
    ("jsd_beta_swapped", "return beta * kl_p + (1.0 - beta) * kl_q", "return (1.0 - beta) * kl_p + beta * kl_q"),
    ("jsd_mixture_ignores_beta", "logM = np.logaddexp(math.log(beta) + logP, math.log1p(-beta) + logq)",
     "logM = np.logaddexp(math.log(0.5) + logP, math.log(0.5) + logq)"),
    ("jsd_gradient_without_mean", "dZ = coef * q * (gv - gbar[:, None])", "dZ = coef * q * gv"),
    ("jsd_gradient_without_weight", "g = (1.0 - beta) * (logq - logM)", "g = (logq - logM)"),
    ("jsd_grid_wraps_negative_ids", "    ok = _in_vocab(ids_rows, V)\n    rr, kk", "    ok = ids_rows < V\n    rr, kk"),
    ("jsd_teacher_term_sign", "kl_p = np.where(on, P * (np.where(on, logP, 0.0) - logM), 0.0)",
     "kl_p = np.where(on, P * (logM - np.where(on, logP, 0.0)), 0.0)"),
    # the skew KL and skew reverse KL
    ("skl_gradient_sign", "g = np.where(on, -(1.0 - alpha) * np.exp(lp - logM), 0.0)",
     "g = np.where(on, (1.0 - alpha) * np.exp(lp - logM), 0.0)"),
    ("skl_gradient_without_weight", "g = np.where(on, -(1.0 - alpha) * np.exp(lp - logM), 0.0)",
     "g = np.where(on, -np.exp(lp - logM), 0.0)"),
    ("skl_mixture_swapped", "logM = np.logaddexp(la + logP, math.log1p(-alpha) + logq)",
     "logM = np.logaddexp(la + logq, math.log1p(-alpha) + logP)"),
    ("skl_loss_sign", "loss = np.where(on, P * (lp - logM), 0.0).sum(axis=1)",
     "loss = np.where(on, P * (logM - lp), 0.0).sum(axis=1)"),
    ("srkl_gradient_without_alpha", "g = r + 1.0 - alpha * np.exp(r)", "g = r + 1.0 - np.exp(r)"),
    ("srkl_mixture_ignores_alpha", "logM = np.logaddexp(math.log(alpha) + logq, lb + logP)",
     "logM = np.logaddexp(math.log(0.5) + logq, math.log(0.5) + logP)"),
    ("srkl_loss_sign", "loss = (q * r).sum(axis=1)", "loss = (q * -r).sum(axis=1)"),
    # the reverse KL over the teacher's top-K support
    ("trkl_full_vocabulary_normaliser", "    s_on = np.where(on, s, -np.inf)\n", "    s_on = s\n"),
    ("trkl_gradient_without_mean", "grad = qt * (r - loss[:, None])", "grad = qt * r"),
    ("trkl_teacher_log_sign", "r = np.where(on, log_qt - logP, 0.0)", "r = np.where(on, log_qt + logP, 0.0)"),
    ("trkl_student_no_temperature", "        s = (H[r0:r1] @ W.T) / float(T)\n        P = _teacher_grid(ids[r0:r1], lg[r0:r1], T, V)\n        row_kl[r0:r1], row_lse[r0:r1], _ = _topk_rkl_parts(s, P)",
     "        s = (H[r0:r1] @ W.T)\n        P = _teacher_grid(ids[r0:r1], lg[r0:r1], T, V)\n        row_kl[r0:r1], row_lse[r0:r1], _ = _topk_rkl_parts(s, P)"),
    ("trkl_gradient_dense_off_support", "grad = qt * (r - loss[:, None])",
     "grad = np.where(on, qt * (r - loss[:, None]), -np.exp(s - np.where(has, lse, 0.0)[:, None]) * 1e-3)"),
    # ignored positions
    ("ignored_counted_in_mean", "N = int(kept.sum())  # the mean runs over the kept positions",
     "N = kept.size  # the mean runs over the kept positions"),
    ("ignored_row_kl_kept", "row_kl[~kept] = 0.0", "pass"),
    ("ignored_grad_row_kept", "dZ[~kept[r0:r1]] = 0.0", "pass"),
    ("ignored_logits_grad_row_kept", "dZ[r0:r1][~kept[r0:r1]] = 0.0", "pass"),
    ("ignore_marker_any_negative", "return ids[:, 0] != IGNORE_ID if", "return ids[:, 0] >= 0 if"),
]


def _mutant(orig, new):
    src = open(os.path.join(ROOT, "oracle", "kl.py")).read()
    assert src.count(orig) >= 1, f"mutation anchor not found: {orig}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(orig, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, new):
    mod = _mutant(orig, new)
    failed = []
    for pin in _pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):  # a wrong value or an invalid index
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
