"""GPU parity of the skew KL and skew reverse KL (kdkl_options.loss =
KDKL_LOSS_SKL / KDKL_LOSS_SRKL, alpha in kdkl_options.beta) against the CPU
oracle's alt functions, element by element, through the C-ABI: both storage
types, several alpha and T, ragged tiles and chunks, backward groups over
vocabulary slices, the workloads' geometries, K = 1024, ids outside [0, V),
repeated ids, ignored positions, the limits alpha = 0 (skew KL = KL) and
alpha = 1 (skew reverse KL = 0)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import TOL, assert_parity, maxrel, run_gpu

pytestmark = pytest.mark.gpu

LOSSES = {"skl": 2, "srkl": 3}  # kdkl_loss values

CASES = [
    ("skl_fp32_ragged", "skl", "tiny_fp32", dict(N=70, d=72, V=4000, K=7, chunk=48, T=0.7), 91, 0.1),
    ("srkl_fp32_ragged", "srkl", "tiny_fp32", dict(N=70, d=72, V=4000, K=7, chunk=48, T=0.7), 92, 0.1),
    ("skl_fp32_alpha0", "skl", "tiny_fp32", dict(N=100, chunk=32, T=1.5), 93, 0.0),
    ("srkl_fp32_alpha07", "srkl", "tiny_fp32", dict(N=100, chunk=32, T=1.5), 94, 0.7),
    ("skl_bf16_ragged_zipf", "skl", "small_bf16", dict(N=300, d=200, V=5000, K=20, chunk=128, T=2.0), 95, 0.1),
    ("srkl_bf16_ragged_zipf", "srkl", "small_bf16", dict(N=300, d=200, V=5000, K=20, chunk=128, T=2.0), 96, 0.1),
    ("skl_bf16_groups4", "skl", "small_bf16", dict(N=148, d=64, V=262001, K=12, chunk=32, T=0.8), 97, 0.3),
    ("srkl_bf16_groups4", "srkl", "small_bf16", dict(N=148, d=64, V=262001, K=12, chunk=32, T=0.8), 98, 0.3),
    ("skl_gptoss_geometry", "skl", "gptoss20b_32k", dict(N=80, chunk=32), 99, 0.1),
    ("srkl_longctx_geometry_T2", "srkl", "longctx_256k", dict(N=64, chunk=24), 100, 0.1),
    ("srkl_bf16_max_K", "srkl", "small_bf16", dict(N=100, d=128, V=6000, K=1024, chunk=64, T=1.0), 101, 0.2),
    ("skl_bf16_max_K", "skl", "small_bf16", dict(N=100, d=128, V=6000, K=1024, chunk=64, T=1.0), 102, 0.2),
]


def _case(name, over, seed):
    w = wl.get_config(name).with_(**over)
    return w, wl.generate(w, seed=seed)


@pytest.mark.parametrize("case,loss,name,over,seed,alpha", CASES, ids=[c[0] for c in CASES])
def test_skew_parity_vs_oracle(case, loss, name, over, seed, alpha):
    w, x = _case(name, over, seed)
    opts = {"loss": LOSSES[loss], "beta": alpha}
    print(f"case {case}: N={w.N} d={w.d} V={w.V} K={w.K} chunk={w.chunk} T={w.T} alpha={alpha} {w.dtype}",
          flush=True)
    got = run_gpu(x, w.T, w.chunk, g=0.8, options=opts)
    ref = oracle.alt_loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, loss, alpha, g=0.8)
    assert_parity(got, ref, w.dtype, case)
    assert maxrel(got["row_kl"], ref["row_kl"]) <= TOL[w.dtype]["loss"] * 10


def test_skl_alpha0_matches_kl_path():
    """The skew KL at alpha = 0 through its own epilogue against the KL's
    kernels on the same inputs (distinct in-range ids)."""
    w, x = _case("small_bf16", dict(N=300, d=576, V=3001, K=20, chunk=128, T=1.3), 103)
    print("case skl alpha 0 vs kl", flush=True)
    s = run_gpu(x, w.T, w.chunk, g=1.1, options={"loss": LOSSES["skl"], "beta": 0.0})
    k = run_gpu(x, w.T, w.chunk, g=1.1)
    assert abs(s["loss"] - k["loss"]) <= 1e-5 * abs(k["loss"])
    assert maxrel(s["dH"], k["dH"]) <= 1e-2 and maxrel(s["dW"], k["dW"]) <= 1e-2


def test_srkl_alpha1_is_zero():
    w, x = _case("tiny_fp32", dict(N=60, V=1000, K=6, chunk=16, T=1.1), 104)
    print("case srkl alpha 1", flush=True)
    got = run_gpu(x, w.T, w.chunk, options={"loss": LOSSES["srkl"], "beta": 1.0})
    assert abs(got["loss"]) <= 1e-6
    assert np.max(np.abs(got["dH"])) <= 1e-7 and np.max(np.abs(got["dW"])) <= 1e-7


@pytest.mark.parametrize("loss,alpha", [("skl", 0.2), ("srkl", 0.25)])
@pytest.mark.parametrize("name,over,seed", [
    ("tiny_fp32", dict(N=60, V=1000, K=6, chunk=16, T=1.1), 105),
    ("small_bf16", dict(N=300, d=576, V=3001, K=20, chunk=128, T=1.3), 106),
])
def test_skew_bad_ids_and_ignored_positions(loss, alpha, name, over, seed):
    w, x = _case(name, over, seed)
    ids = x["ids"].clone()
    N = ids.shape[0]
    bad = torch.tensor([-5, w.V, w.V + 3, 2 ** 30, -2, -(2 ** 31)], dtype=torch.int32)
    ids[::2, 0] = bad.repeat(N // len(bad) + 1)[: (N + 1) // 2]
    ids[::3, 2] = ids[::3, 1]                      # repeated ids
    ids[[4, 17], 0] = -1                           # ignored positions
    ids[9, :] = torch.tensor([w.V + 1] * w.K)      # a position with no vocabulary entry at all
    x2 = dict(x, ids=ids)
    opts = {"loss": LOSSES[loss], "beta": alpha}
    print(f"case {loss} bad ids {name}: N={w.N} V={w.V} K={w.K}", flush=True)
    got = run_gpu(x2, w.T, w.chunk, g=1.2, options=opts)
    ref = oracle.alt_loss_and_grads(x2["H"], x2["W"], x2["ids"], x2["logits"], w.T, loss, alpha, g=1.2)
    assert_parity(got, ref, w.dtype, f"{loss} bad ids {name}")
    assert np.all(got["row_kl"][[4, 17]] == 0.0) and np.all(got["dH"][[4, 17]] == 0.0)
    # no support: the skew KL is 0, the skew reverse KL -log(alpha)
    want = 0.0 if loss == "skl" else -math.log(alpha)
    assert abs(got["row_kl"][9] - want) <= 1e-5


@pytest.mark.parametrize("loss", ["skl", "srkl"])
def test_skew_bitwise_determinism_and_autograd(loss):
    import chunked_kl_loss_amd as kd

    w, x = _case("small_bf16", dict(N=512, V=8000, chunk=200), 107)
    opts = {"loss": LOSSES[loss], "beta": 0.1}
    print(f"case {loss} determinism and autograd", flush=True)
    a = run_gpu(x, w.T, w.chunk, options=opts)
    b = run_gpu(x, w.T, w.chunk, options=opts)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["dH"], b["dH"]) and np.array_equal(a["dW"], b["dW"])
    dev = "cuda:0"
    H = x["H"].to(dev).requires_grad_(True)
    W = x["W"].to(dev).requires_grad_(True)
    out = kd.fused_kl_loss(H, W, x["ids"].to(dev), x["logits"].to(dev), w.T, w.chunk, options=opts)
    (2.0 * out).backward()
    ref = oracle.alt_loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, loss, 0.1, g=2.0)
    assert abs(out.item() - ref["loss"]) <= 1e-3 * abs(ref["loss"])
    assert maxrel(H.grad.double().cpu().numpy(), ref["dH"]) <= 2e-2
    assert maxrel(W.grad.double().cpu().numpy(), ref["dW"]) <= 2e-2
