"""GPU parity of the dense baseline (full student log-probability and teacher
probability grids, kept for the backward) against the CPU oracle, through the
C-ABI. The dense path computes the same loss and gradients as the fused one,
so the oracle's loss and gradients are the reference; on a tiny problem also
the oracle's grid-wide dense function."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import TOL, assert_parity, maxrel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run_dense(x, T, g=None, accumulate_dW=False, dW_init=None):
    import chunked_kl_loss_amd as kd

    H, W, ids, lg = (x[k].to(DEV) for k in ("H", "W", "ids", "logits"))
    loss, lse, kl, saved = kd.dense_forward(H, W, ids, lg, T)
    gt = None if g is None else torch.tensor([g], dtype=torch.float32, device=DEV)
    dW = None if dW_init is None else dW_init.clone().to(DEV)
    dH, dW = kd.dense_backward(H, W, ids, lg, T, saved, gt, dW=dW, accumulate_dW=accumulate_dW)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "row_lse": lse.double().cpu().numpy(),
            "row_kl": kl.double().cpu().numpy(), "dH": dH.double().cpu().numpy(),
            "dW": dW.double().cpu().numpy()}


CASES = [
    ("dense_tiny_fp32", "tiny_fp32", dict(N=70, d=72, V=1000, K=7, T=0.7), 41),
    ("dense_bf16_ragged", "small_bf16", dict(N=300, d=576, V=3001, K=20, T=1.3), 42),
    ("dense_bf16_tile256", "small_bf16", dict(N=257, d=256, V=4096, K=100, T=1.0), 43),
    # large enough for 384-row vocabulary tiles on the projection
    ("dense_bf16_vtile384", "small_bf16", dict(N=2048, d=128, V=11905, K=16, T=1.2), 45),
]


@pytest.mark.parametrize("case,name,over,seed", CASES, ids=[c[0] for c in CASES])
def test_dense_parity_vs_oracle(case, name, over, seed):
    w = wl.get_config(name).with_(**over)
    x = wl.generate(w, seed=seed)
    print(f"case {case}: N={w.N} d={w.d} V={w.V} K={w.K} T={w.T} {w.dtype}", flush=True)
    got = _run_dense(x, w.T, g=0.8)
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, g=0.8)
    assert_parity(got, ref, w.dtype, case)
    assert maxrel(got["row_kl"], ref["row_kl"]) <= TOL[w.dtype]["loss"] * 10


def test_dense_matches_grid_baseline_and_ignores_positions():
    w = wl.get_config("tiny_fp32").with_(N=24, d=16, V=300, K=5, T=1.2)
    x = wl.generate(w, seed=44)
    ids = x["ids"].clone()
    ids[[3, 10], 0] = -1
    x = dict(x, ids=ids)
    print("case dense tiny grid baseline with ignored rows", flush=True)
    got = _run_dense(x, w.T)
    ref = oracle.dense_kl_loss(x["H"], x["W"], x["ids"], x["logits"], w.T)
    assert abs(got["loss"] - ref) <= 1e-5 * abs(ref)
    assert got["row_kl"][3] == 0.0 and not np.any(got["dH"][[3, 10]])
    assert_parity(got, oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T), "fp32",
                  "dense ignored")


def test_dense_accumulate_and_agrees_with_fused():
    import chunked_kl_loss_amd as kd

    w = wl.get_config("small_bf16").with_(N=200, d=320, V=2500, K=30, chunk=64)
    x = wl.generate(w, seed=45)
    print("case dense accumulate / fused agreement", flush=True)
    init = torch.randn(w.V, w.d, generator=torch.Generator().manual_seed(1))
    got = _run_dense(x, w.T, accumulate_dW=True, dW_init=init)
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T)
    err = np.abs(got["dW"] - (init.double().numpy() + ref["dW"])).max()
    assert err <= TOL["bf16"]["grad"] * np.abs(ref["dW"]).max() + 1e-6 * np.abs(init.numpy()).max()
    H, W, ids, lg = (x[k].to(DEV) for k in ("H", "W", "ids", "logits"))
    lf, lse_f, _ = kd.kdkl_forward(H, W, ids, lg, w.T, w.chunk)
    ld, lse_d, _, _ = kd.dense_forward(H, W, ids, lg, w.T)
    torch.cuda.synchronize()
    # the dense path stores its logit grid in the storage dtype (bf16, as a
    # bf16 output layer would); the fused path keeps the fp32 accumulators, so
    # the two agree to the bf16 tolerance
    assert abs(lf.item() - ld.item()) <= TOL["bf16"]["loss"] * abs(lf.item())
    assert maxrel(lse_d.double().cpu().numpy(), lse_f.double().cpu().numpy()) <= TOL["bf16"]["loss"]


def test_dense_empty_input():
    import chunked_kl_loss_amd as kd

    print("case dense N=0", flush=True)
    H = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    W = torch.randn(500, 64, device=DEV).to(torch.bfloat16)
    ids = torch.empty(0, 4, dtype=torch.int32, device=DEV)
    lg = torch.empty(0, 4, device=DEV)
    loss, lse, kl, saved = kd.dense_forward(H, W, ids, lg, 1.0)
    dH, dW = kd.dense_backward(H, W, ids, lg, 1.0, saved)
    torch.cuda.synchronize()
    assert math.isnan(loss.item()) and not torch.any(dW).item()
