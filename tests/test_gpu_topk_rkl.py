"""GPU parity of the reverse KL over the teacher's top-K support
(kdkl_options.loss = KDKL_LOSS_TRKL) against the CPU oracle's topk_rkl
functions, element by element, through the C-ABI: both storage types, the
generic and the bf16 main loops, ragged tiles and chunks, backward groups over
vocabulary slices, the workloads' geometries, K = 1024, ids outside [0, V),
repeated ids, an empty support, ignored positions; the allocation-free
forward; determinism and autograd; and the 32K workload at full size."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import TOL, maxrel, run_gpu

pytestmark = pytest.mark.gpu

TRKL = {"loss": 4}  # KDKL_LOSS_TRKL

CASES = [
    ("fp32_ragged", "tiny_fp32", dict(N=70, d=72, V=4000, K=7, chunk=48, T=0.7), 121, None),
    ("bf16_generic_ragged_zipf", "small_bf16", dict(N=300, d=200, V=5000, K=20, chunk=128, T=2.0), 122, None),
    ("bf16_groups", "small_bf16", dict(N=148, d=64, V=262001, K=12, chunk=32, T=0.8), 123, None),
    ("bf16_groups4_slices3", "small_bf16", dict(N=148, d=64, V=262001, K=12, chunk=32, T=0.8), 124,
     {"chunks_per_group": 4, "vocab_slices": 3}),
    ("gptoss_geometry", "gptoss20b_32k", dict(N=80, chunk=32), 125, None),
    ("longctx_geometry_T2", "longctx_256k", dict(N=64, chunk=24), 126, None),
    ("bf16_max_K", "small_bf16", dict(N=100, d=128, V=6000, K=1024, chunk=64, T=1.0), 127, None),
    # the backward holds rows of up to 6 vectors per lane in registers
    # (d <= 3072 in bf16, 1536 in fp32); wider rows take two passes
    ("bf16_rows_at_register_limit", "small_bf16", dict(N=90, d=3072, V=5000, K=20, chunk=32, T=1.0), 134, None),
    ("bf16_wide_rows_two_pass", "small_bf16", dict(N=90, d=3080, V=5000, K=20, chunk=32, T=1.0), 135, None),
    ("fp32_wide_rows_two_pass", "tiny_fp32", dict(N=50, d=1540, V=3000, K=9, chunk=32, T=1.0), 136, None),
]


def _case(name, over, seed):
    w = wl.get_config(name).with_(**over)
    return w, wl.generate(w, seed=seed)


def _check(got, ref, x, dtype, what):
    """Loss, per-row loss, logsumexp over the support (kept rows; -inf where
    the support is empty) and both gradients, at the storage type's
    tolerances."""
    tol = TOL[dtype]
    kept = oracle.kept_positions(x["ids"])
    rl = abs(got["loss"] - ref["loss"]) / abs(ref["loss"])
    ek = maxrel(got["row_kl"], ref["row_kl"])
    lg, lr = got["row_lse"][kept], ref["row_lse"][kept]
    fin = np.isfinite(lr)
    assert np.array_equal(np.isfinite(lg), fin) and np.all(lg[~fin] == -np.inf), f"{what}: empty supports"
    el = maxrel(lg[fin], lr[fin]) if fin.any() else 0.0
    eh = maxrel(got["dH"], ref["dH"])
    ew = maxrel(got["dW"], ref["dW"])
    msg = (f"{what}: loss {got['loss']:.7g} vs {ref['loss']:.7g} rel {rl:.2e}; row_kl {ek:.2e}; "
           f"lse {el:.2e}; dH {eh:.2e}; dW {ew:.2e} (tol {tol})")
    print(msg, flush=True)
    assert rl <= tol["loss"] and el <= tol["loss"] and ek <= 10 * tol["loss"], msg
    assert eh <= tol["grad"] and ew <= tol["grad"], msg


@pytest.mark.parametrize("case,name,over,seed,blocking", CASES, ids=[c[0] for c in CASES])
def test_topk_rkl_parity_vs_oracle(case, name, over, seed, blocking):
    w, x = _case(name, over, seed)
    opts = dict(TRKL, **(blocking or {}))
    print(f"case {case}: N={w.N} d={w.d} V={w.V} K={w.K} chunk={w.chunk} T={w.T} {w.dtype} {opts}", flush=True)
    got = run_gpu(x, w.T, w.chunk, g=0.8, options=opts)
    ref = oracle.topk_rkl_loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, g=0.8)
    _check(got, ref, x, w.dtype, case)


@pytest.mark.parametrize("name,over,seed", [
    ("tiny_fp32", dict(N=40, d=64, V=500, K=1, chunk=16, T=1.0), 137),
    ("small_bf16", dict(N=70, d=128, V=800, K=1, chunk=32, T=2.0), 138),
])
def test_topk_rkl_single_entry_support(name, over, seed):
    """K = 1: the renormalised student and teacher both put all their mass on
    the one id, so the loss, every per-row value and both gradients are
    exactly zero; the logsumexp over the support is that id's logit (against
    the oracle)."""
    w, x = _case(name, over, seed)
    print(f"case trkl K=1 {name}", flush=True)
    got = run_gpu(x, w.T, w.chunk, options=TRKL)
    ref = oracle.topk_rkl_loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T)
    assert got["loss"] == 0.0 and np.all(got["row_kl"] == 0.0)
    assert np.all(got["dH"] == 0.0) and np.all(got["dW"] == 0.0)
    kept = oracle.kept_positions(x["ids"])
    e = maxrel(got["row_lse"][kept], ref["row_lse"][kept])
    print(f"lse {e:.2e}", flush=True)
    assert e <= TOL[w.dtype]["loss"]


@pytest.mark.parametrize("name,over,seed", [
    ("tiny_fp32", dict(N=60, V=1000, K=6, chunk=16, T=1.1), 128),
    ("small_bf16", dict(N=300, d=576, V=3001, K=20, chunk=128, T=1.3), 129),
])
def test_topk_rkl_bad_ids_and_ignored_positions(name, over, seed):
    w, x = _case(name, over, seed)
    ids = x["ids"].clone()
    N = ids.shape[0]
    bad = torch.tensor([-5, w.V, w.V + 3, 2 ** 30, -2, -(2 ** 31)], dtype=torch.int32)
    ids[::2, 0] = bad.repeat(N // len(bad) + 1)[: (N + 1) // 2]
    ids[::3, 2] = ids[::3, 1]                      # repeated ids: the masses add
    ids[[4, 17], 0] = -1                           # ignored positions
    ids[9, :] = torch.tensor([w.V + 1] * w.K)      # a kept position with an empty support
    x2 = dict(x, ids=ids)
    print(f"case trkl bad ids {name}: N={w.N} V={w.V} K={w.K}", flush=True)
    got = run_gpu(x2, w.T, w.chunk, g=1.2, options=TRKL)
    ref = oracle.topk_rkl_loss_and_grads(x2["H"], x2["W"], x2["ids"], x2["logits"], w.T, g=1.2)
    _check(got, ref, x2, w.dtype, f"trkl bad ids {name}")
    assert np.all(got["row_kl"][[4, 17]] == 0.0) and np.all(got["dH"][[4, 17]] == 0.0)
    assert got["row_kl"][9] == 0.0 and got["row_lse"][9] == -np.inf and np.all(got["dH"][9] == 0.0)


def test_topk_rkl_gradient_only_on_the_support_and_accumulate():
    """dW rows of ids in no position's support are exactly zero (overwritten,
    also over NaNs, or left as they were with accumulate_dW)."""
    w, x = _case("small_bf16", dict(N=200, d=256, V=7000, K=16, chunk=64, T=1.0), 130)
    print("case trkl support-only dW and accumulate", flush=True)
    got = run_gpu(x, w.T, w.chunk, options=TRKL)
    used = np.zeros(w.V, dtype=bool)
    used[x["ids"].numpy().reshape(-1)] = True
    assert np.all(got["dW"][~used] == 0.0)
    # without accumulate_dW every row is written, whatever dW held
    poisoned = run_gpu(x, w.T, w.chunk, options=TRKL, dW_init=torch.full((w.V, w.d), float("nan")))
    assert np.array_equal(poisoned["dW"], got["dW"])
    init = torch.randn(w.V, w.d) * 1e-2  # (the sum's fp32 rounding stays far below the tolerance)
    acc = run_gpu(x, w.T, w.chunk, options=TRKL, accumulate_dW=True, dW_init=init)
    base = init.double().numpy()
    assert np.array_equal(acc["dW"][~used], base[~used])
    assert maxrel(acc["dW"][used] - base[used], got["dW"][used]) <= 1e-5


def test_topk_rkl_hot_id_over_several_runs():
    """One id at every one of 3000 positions (the head of a Zipf-like id
    distribution): its dW row is summed by several workgroups, one per run of
    1024 entries, and their partial rows in order; bitwise reproducible."""
    w, x = _case("small_bf16", dict(N=3000, d=128, V=2000, K=8, chunk=512, T=1.0), 133)
    ids = x["ids"].clone()
    hot = 7
    ids[~(ids == hot).any(dim=1), 0] = hot
    x2 = dict(x, ids=ids)
    print("case trkl hot id over several runs", flush=True)
    got = run_gpu(x2, w.T, w.chunk, g=0.9, options=TRKL)
    ref = oracle.topk_rkl_loss_and_grads(x2["H"], x2["W"], x2["ids"], x2["logits"], w.T, g=0.9)
    _check(got, ref, x2, w.dtype, "trkl hot id")
    assert maxrel(got["dW"][hot], ref["dW"][hot]) <= 1e-2
    again = run_gpu(x2, w.T, w.chunk, g=0.9, options=TRKL)
    assert np.array_equal(got["dW"], again["dW"]) and np.array_equal(got["dH"], again["dH"])


def test_topk_rkl_noalloc_forward_and_determinism():
    import chunked_kl_loss_amd as kd

    w, x = _case("small_bf16", dict(N=512, V=8000, chunk=200), 131)
    print("case trkl no-alloc forward and determinism", flush=True)
    a = run_gpu(x, w.T, w.chunk, options=TRKL)
    b = run_gpu(x, w.T, w.chunk, options=TRKL)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["dH"], b["dH"]) and np.array_equal(a["dW"], b["dW"])
    dev = "cuda:0"
    d = {k: v.to(dev) for k, v in x.items()}
    loss = torch.empty(1, device=dev)
    lse = torch.empty(kd.saved_shape(w.N, TRKL), device=dev)
    kl = torch.empty(w.N, device=dev)
    kd.kdkl_forward_noalloc(d["H"], d["W"], d["ids"], d["logits"], w.T, w.chunk, loss=loss, row_lse=lse,
                            row_kl=kl, options=TRKL)
    torch.cuda.synchronize()
    assert loss.item() == a["loss"]
    assert torch.equal(lse, a["_dev"]["row_lse"])


def test_topk_rkl_autograd():
    import chunked_kl_loss_amd as kd

    w, x = _case("small_bf16", dict(N=256, V=6000, chunk=128), 132)
    print("case trkl autograd", flush=True)
    dev = "cuda:0"
    H = x["H"].to(dev).requires_grad_(True)
    W = x["W"].to(dev).requires_grad_(True)
    out = kd.fused_kl_loss(H, W, x["ids"].to(dev), x["logits"].to(dev), w.T, w.chunk, options=TRKL)
    (2.0 * out).backward()
    ref = oracle.topk_rkl_loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, g=2.0)
    assert abs(out.item() - ref["loss"]) <= 1e-3 * abs(ref["loss"])
    assert maxrel(H.grad.double().cpu().numpy(), ref["dH"]) <= 2e-2
    assert maxrel(W.grad.double().cpu().numpy(), ref["dW"]) <= 2e-2


@pytest.mark.parametrize("name", ["gptoss20b_32k", "longctx_256k"])
def test_topk_rkl_full_size(name):
    """The 32K gpt-oss-like workload (Zipf-like ids, one group) and the 256K
    one (uniform ids, T = 2, eight groups: dW written by the first, added to
    by the others) in the bench's launch configuration: sampled positions
    (loss, logsumexp over the support, dH rows) and dW rows of rarely used
    ids and of the most used one (at 32K summed over several runs) against
    the oracle, unused ids' dW rows exactly zero, the loss as the mean of the
    per-row values, and <W, dW> = <H, dH>."""
    import chunked_kl_loss_amd as kd

    w = wl.get_config(name)
    x = wl.generate(w)
    dev = "cuda:0"
    print(f"case trkl full size {w.name}", flush=True)
    H, W, ids, lg = (x[k].to(dev) for k in ("H", "W", "ids", "logits"))
    loss, row_lse, row_kl = kd.kdkl_forward(H, W, ids, lg, w.T, w.chunk, options=TRKL)
    dH, dW = kd.kdkl_backward(H, W, ids, lg, w.T, w.chunk, row_lse, options=TRKL)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = sorted({0, 1, w.chunk, w.N - 1} | set(rng.choice(w.N, 8, replace=False).tolist()))
    counts = np.bincount(x["ids"].numpy().reshape(-1), minlength=w.V)
    rare = np.nonzero((counts >= 1) & (counts <= max(40, int(np.percentile(counts, 5)))))[0]
    vrows = sorted(rng.choice(rare, 4, replace=False).tolist()) + [int(np.argmax(counts))]  # and the most used id
    ref = oracle.topk_rkl_sampled(x["H"], x["W"], x["ids"], x["logits"], w.T, rows, vrows)
    lse = row_lse[0].double().cpu().numpy()
    kl = row_kl.double().cpu().numpy()
    e_lse = maxrel(lse[rows], ref["row_lse"])
    e_kl = maxrel(kl[rows], ref["row_kl"])
    e_dh = maxrel(dH[rows].double().cpu().numpy(), ref["dH_rows"])
    e_dw = maxrel(dW[vrows].double().cpu().numpy(), ref["dW_rows"])
    print(f"trkl full size: lse {e_lse:.2e} kl {e_kl:.2e} dH {e_dh:.2e} dW {e_dw:.2e}", flush=True)
    assert e_lse <= 1e-3 and e_kl <= 1e-2 and e_dh <= 2e-2 and e_dw <= 2e-2
    unused = np.nonzero(counts == 0)[0]
    assert unused.size or w.N * w.K > 50 * w.V  # (uniform ids at 256K leave no id unused)
    assert not torch.any(dW[torch.from_numpy(unused[:4096]).to(dev)] != 0)
    assert abs(loss.item() - float(kl.mean())) <= 1e-5 * abs(float(kl.mean()))
    wd = float((W.double() * dW.double()).sum())
    hd = float((H.double() * dH.double()).sum())
    scale = float((H.double() * dH.double()).abs().sum())
    print(f"<W,dW> {wd:.6e} <H,dH> {hd:.6e} scale {scale:.3e}", flush=True)
    assert abs(wd - hd) <= 1e-3 * scale
