"""GPU parity of the alternative loss (generalised Jensen-Shannon divergence,
kdkl_options.loss = KDKL_LOSS_JSD) against the CPU oracle's jsd functions,
element by element, through the C-ABI: both storage types, several beta and
T, ragged tiles and chunks, backward groups over vocabulary slices, ids
outside [0, V), repeated ids and ignored positions."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import TOL, assert_parity, maxrel, run_gpu

pytestmark = pytest.mark.gpu

CASES = [
    ("jsd_fp32_ragged", "tiny_fp32", dict(N=70, d=72, V=4000, K=7, chunk=48, T=0.7), 71, 0.5),
    ("jsd_fp32_beta01", "tiny_fp32", dict(N=100, chunk=32, T=1.5), 72, 0.1),
    ("jsd_bf16_ragged_zipf", "small_bf16", dict(N=300, d=200, V=5000, K=20, chunk=128, T=2.0), 73, 0.5),
    ("jsd_bf16_beta09", "small_bf16", dict(N=300, d=576, V=3001, K=20, chunk=128, T=1.3), 74, 0.9),
    ("jsd_bf16_groups4", "small_bf16", dict(N=148, d=64, V=262001, K=12, chunk=32, T=0.8), 75, 0.3),
    ("jsd_gptoss_geometry", "gptoss20b_32k", dict(N=80, chunk=32), 76, 0.5),
    ("jsd_longctx_geometry_T2", "longctx_256k", dict(N=64, chunk=24), 77, 0.5),
    ("jsd_bf16_max_K", "small_bf16", dict(N=100, d=128, V=6000, K=1024, chunk=64, T=1.0), 78, 0.5),
]


def _jsd_case(name, over, seed):
    w = wl.get_config(name).with_(**over)
    return w, wl.generate(w, seed=seed)


@pytest.mark.parametrize("case,name,over,seed,beta", CASES, ids=[c[0] for c in CASES])
def test_jsd_parity_vs_oracle(case, name, over, seed, beta):
    import chunked_kl_loss_amd as kd

    w, x = _jsd_case(name, over, seed)
    opts = {"loss": kd.KDKL_LOSS_JSD, "beta": beta}
    print(f"case {case}: N={w.N} d={w.d} V={w.V} K={w.K} chunk={w.chunk} T={w.T} beta={beta} {w.dtype}",
          flush=True)
    got = run_gpu(x, w.T, w.chunk, g=0.8, options=opts)
    ref = oracle.jsd_loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, beta, g=0.8)
    assert_parity(got, ref, w.dtype, case)
    assert maxrel(got["row_kl"], ref["row_kl"]) <= TOL[w.dtype]["loss"] * 10


@pytest.mark.parametrize("name,over,seed", [
    ("tiny_fp32", dict(N=60, V=1000, K=6, chunk=16, T=1.1), 79),
    ("small_bf16", dict(N=300, d=576, V=3001, K=20, chunk=128, T=1.3), 80),
])
def test_jsd_bad_ids_and_ignored_positions(name, over, seed):
    import chunked_kl_loss_amd as kd

    w, x = _jsd_case(name, over, seed)
    ids = x["ids"].clone()
    N = ids.shape[0]
    bad = torch.tensor([-5, w.V, w.V + 3, 2 ** 30, -2, -(2 ** 31)], dtype=torch.int32)
    ids[::2, 0] = bad.repeat(N // len(bad) + 1)[: (N + 1) // 2]
    ids[::3, 2] = ids[::3, 1]                      # repeated ids
    ids[[4, 17], 0] = -1                           # ignored positions
    ids[9, :] = torch.tensor([w.V + 1] * w.K)      # a position with no vocabulary entry at all
    x2 = dict(x, ids=ids)
    opts = {"loss": kd.KDKL_LOSS_JSD, "beta": 0.4}
    print(f"case jsd bad ids {name}: N={w.N} V={w.V} K={w.K}", flush=True)
    got = run_gpu(x2, w.T, w.chunk, g=1.2, options=opts)
    ref = oracle.jsd_loss_and_grads(x2["H"], x2["W"], x2["ids"], x2["logits"], w.T, 0.4, g=1.2)
    assert_parity(got, ref, w.dtype, f"jsd bad ids {name}")
    assert np.all(got["row_kl"][[4, 17]] == 0.0) and np.all(got["dH"][[4, 17]] == 0.0)
    # no support: JSD = (1 - beta) log(1 / (1 - beta))
    assert abs(got["row_kl"][9] + 0.6 * math.log(0.6)) <= 1e-5


def test_jsd_bitwise_determinism_and_autograd():
    import chunked_kl_loss_amd as kd

    w, x = _jsd_case("small_bf16", dict(N=512, V=8000, chunk=200), 81)
    opts = {"loss": kd.KDKL_LOSS_JSD, "beta": 0.5}
    a = run_gpu(x, w.T, w.chunk, options=opts)
    b = run_gpu(x, w.T, w.chunk, options=opts)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["dH"], b["dH"]) and np.array_equal(a["dW"], b["dW"])
    dev = "cuda:0"
    H = x["H"].to(dev).requires_grad_(True)
    W = x["W"].to(dev).requires_grad_(True)
    loss = kd.fused_kl_loss(H, W, x["ids"].to(dev), x["logits"].to(dev), w.T, w.chunk, options=opts)
    (2.0 * loss).backward()
    ref = oracle.jsd_loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, 0.5, g=2.0)
    assert abs(loss.item() - ref["loss"]) <= 1e-3 * abs(ref["loss"])
    assert maxrel(H.grad.double().cpu().numpy(), ref["dH"]) <= 2e-2
    assert maxrel(W.grad.double().cpu().numpy(), ref["dW"]) <= 2e-2
