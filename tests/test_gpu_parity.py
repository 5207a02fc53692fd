"""GPU parity: the HIP path through the C-ABI against the CPU oracle, element
by element, on seeded inputs that span several tiles and ragged tails, plus
the method's degenerate cases and invariants."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import TOL, assert_parity, maxrel, run_gpu

pytestmark = pytest.mark.gpu

# (case id, workload, overrides, seed) — sizes the oracle finishes in seconds.
CASES = [
    ("tiny_fp32_full", "tiny_fp32", {}, None),
    ("fp32_ragged_all", "tiny_fp32", dict(N=70, d=72, V=4000, K=7, chunk=48, T=0.7), 7),
    ("fp32_chunk_ragged_T", "tiny_fp32", dict(N=100, chunk=32, T=1.5), 8),
    ("bf16_ragged_zipf", "small_bf16", dict(N=300, d=200, V=5000, K=20, chunk=128, T=2.0), 9),
    ("small_bf16_full", "small_bf16", {}, None),
    ("llama3b_geometry", "llama3b_8k", dict(N=96, chunk=40), None),
    ("gptoss20b_geometry", "gptoss20b_32k", dict(N=80, chunk=32), None),
    ("longctx_geometry_T2", "longctx_256k", dict(N=64, chunk=24), None),
    # hidden sizes whose dH / dW products use 320-wide tiles: one exact, one
    # with a partial last tile, both with ragged vocabulary and chunk tails
    ("bf16_d_tile320_exact", "small_bf16", dict(N=130, d=960, V=2500, K=12, chunk=64, T=1.0), 11),
    ("bf16_d_tile320_ragged", "small_bf16", dict(N=200, d=576, V=3001, K=30, chunk=96, T=1.3), 10),
    # bf16 main loop with a vocabulary smaller than one tile
    ("bf16_fast_small_V", "small_bf16", dict(N=90, d=128, V=300, K=10, chunk=64, T=1.0), 12),
    # launches large enough for 384-row vocabulary tiles on the forward / dZ
    # products (one workgroup round of 384-row tiles against two of 256):
    # an exact multiple of 384, and a last tile holding a single row with a
    # ragged second chunk
    ("bf16_vtile384_exact", "small_bf16", dict(N=2048, d=128, V=12288, K=16, chunk=2048, T=1.1), 13),
    ("bf16_vtile384_one_row", "small_bf16", dict(N=2100, d=192, V=11905, K=8, chunk=2048, T=0.9), 14),
    # vocabularies large enough for the dW product to fill its rounds of
    # workgroups, so that both calls take several chunks at a time (over the
    # whole vocabulary, a partial last tile): three chunks (groups of two: a
    # full group, then one partial chunk), five (a full group of four, then
    # one partial chunk), nine (a group of eight, then one partial chunk),
    # seventeen (a group of sixteen, then five rows)
    ("bf16_backward_groups2", "small_bf16", dict(N=150, d=64, V=131001, K=16, chunk=64, T=1.2), 15),
    ("bf16_backward_groups4", "small_bf16", dict(N=148, d=64, V=262001, K=12, chunk=32, T=0.8), 16),
    ("bf16_backward_groups8", "small_bf16", dict(N=133, d=64, V=524001, K=20, chunk=16, T=1.1), 21),
    ("bf16_backward_groups16", "small_bf16", dict(N=261, d=64, V=524001, K=20, chunk=16, T=1.1), 29),
    # the largest teacher top-K the boundary takes, over a small vocabulary:
    # dozens of teacher entries per column in every vocabulary tile
    ("bf16_max_K", "small_bf16", dict(N=100, d=128, V=6000, K=1024, chunk=64, T=1.0), 17),
    ("fp32_max_K", "tiny_fp32", dict(N=40, d=64, V=1500, K=1024, chunk=16, T=0.9), 18),
    # a single position (one partial token tile)
    ("bf16_one_position", "small_bf16", dict(N=1, d=128, V=3000, K=10, chunk=64, T=1.0), 19),
    ("fp32_one_position", "tiny_fp32", dict(N=1, d=64, V=700, K=5, chunk=8, T=1.0), 20),
]


def _inputs(name, over, seed):
    w = wl.get_config(name).with_(**over)
    x = wl.generate(w, seed=seed)
    return w, x


@pytest.mark.parametrize("case,name,over,seed", CASES, ids=[c[0] for c in CASES])
def test_parity_vs_oracle(case, name, over, seed):
    w, x = _inputs(name, over, seed)
    print(f"case {case}: N={w.N} d={w.d} V={w.V} K={w.K} chunk={w.chunk} T={w.T} {w.dtype}",
          flush=True)
    got = run_gpu(x, w.T, w.chunk)
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T)
    assert_parity(got, ref, w.dtype, case)
    # per-row KL as well
    assert maxrel(got["row_kl"], ref["row_kl"]) <= TOL[w.dtype]["loss"] * 10


@pytest.mark.parametrize("name,over", [
    ("gptoss20b_32k", dict(N=80, chunk=32)),  # 320-wide hidden-size tiles, backward groups
    ("llama3b_8k", dict(N=96, chunk=40)),     # 256-wide hidden-size tiles
], ids=["d_tile320", "d_tile256"])
@pytest.mark.parametrize("in_place", [1, 2])
def test_dh_reading_w_in_place(name, over, in_place):
    # the dH product reading W through the LDS transpose read (1) or a W^T
    # copy (2), whichever the plan would pick for these sizes
    w, x = _inputs(name, over, None)
    opts = {"dh_w_in_place": in_place}
    import chunked_kl_loss_amd as kd
    assert kd.plan_info(w.N, w.d, w.V, w.K, w.chunk, w.torch_dtype, opts)["dh_w_in_place"] == (in_place == 1)
    print(f"case dh_w_in_place={in_place} {name}: N={w.N} d={w.d} V={w.V} chunk={w.chunk}", flush=True)
    got = run_gpu(x, w.T, w.chunk, options=opts)
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T)
    assert_parity(got, ref, w.dtype, f"{name} dH reading W in place")


# Vocabulary slices apart from the chunks per group (the backward's dZ
# buffer holds group rows x V/slices columns): more slices than chunks, fewer,
# one chunk over several slices, and the generic (fp32) main loop in slices;
# each case has a ragged last slice and a ragged last group.
SLICE_CASES = [
    ("bf16_groups4_slices16", "small_bf16", dict(N=148, d=64, V=262001, K=12, chunk=32, T=0.8), 16,
     dict(chunks_per_group=4, vocab_slices=16)),
    ("bf16_groups4_slices3", "small_bf16", dict(N=148, d=64, V=262001, K=12, chunk=32, T=0.8), 16,
     dict(chunks_per_group=4, vocab_slices=3)),
    ("bf16_one_chunk_slices5", "small_bf16", dict(N=300, d=576, V=30001, K=20, chunk=128, T=1.3), 51,
     dict(chunks_per_group=1, vocab_slices=5)),
    ("bf16_d320_groups2_slices7", "gptoss20b_32k", dict(N=80, V=40000, chunk=32), 52,
     dict(chunks_per_group=2, vocab_slices=7)),
    ("fp32_slices3", "tiny_fp32", dict(N=70, d=72, V=4000, K=7, chunk=48, T=0.7), 53,
     dict(vocab_slices=3)),
]


@pytest.mark.parametrize("case,name,over,seed,opts", SLICE_CASES, ids=[c[0] for c in SLICE_CASES])
def test_vocabulary_slices(case, name, over, seed, opts):
    import chunked_kl_loss_amd as kd

    w, x = _inputs(name, over, seed)
    plan = kd.plan_info(w.N, w.d, w.V, w.K, w.chunk, w.torch_dtype, opts)
    print(f"case {case}: N={w.N} d={w.d} V={w.V} chunk={w.chunk} plan {plan}", flush=True)
    assert plan["vocab_slices"] == opts["vocab_slices"]
    got = run_gpu(x, w.T, w.chunk, g=0.6, options=opts)
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, g=0.6)
    assert_parity(got, ref, w.dtype, case)


def test_chunk_size_independence():
    w, x = _inputs("tiny_fp32", dict(N=64, V=1000, K=5), 21)
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T)
    outs = []
    for chunk in (1, 7, 32, 64, 1000):
        got = run_gpu(x, w.T, chunk)
        assert_parity(got, ref, "fp32", f"chunk={chunk}")
        outs.append(got)
    for o in outs[1:]:
        assert abs(o["loss"] - outs[0]["loss"]) <= 1e-6 * abs(outs[0]["loss"])


def test_upstream_gradient_and_accumulate():
    w, x = _inputs("tiny_fp32", dict(N=50, V=3000, K=6, chunk=16, T=1.3), 22)
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, g=0.37)
    got = run_gpu(x, w.T, w.chunk, g=0.37)
    assert_parity(got, ref, "fp32", "g=0.37")
    # accumulate: dW starts from a given tensor and adds
    init = torch.randn(w.V, w.d, dtype=torch.float32)
    acc = run_gpu(x, w.T, w.chunk, g=0.37, accumulate_dW=True, dW_init=init)
    # fp32 addition into an O(1) tensor: one rounding of the sum per element
    expect = init.double().numpy() + ref["dW"]
    err = np.abs(acc["dW"] - expect).max()
    assert err <= 2 * np.finfo(np.float32).eps * np.abs(expect).max() + 1e-5 * np.abs(ref["dW"]).max()


def test_upstream_gradient_and_accumulate_in_backward_groups():
    # the bf16 path taking its chunks in groups over vocabulary slices: each
    # group's dW read-modify-write adds to the caller's dW, and the upstream
    # gradient scales both products
    w, x = _inputs("small_bf16", dict(N=150, d=64, V=131001, K=16, chunk=64, T=1.2), 15)
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, g=0.37)
    scale = float(np.abs(ref["dW"]).max())
    init = torch.randn(w.V, w.d, dtype=torch.float32) * scale
    got = run_gpu(x, w.T, w.chunk, g=0.37, accumulate_dW=True, dW_init=init)
    eh = maxrel(got["dH"], ref["dH"])
    ew = maxrel(got["dW"] - init.double().numpy(), ref["dW"])
    print(f"groups g=0.37 accumulate: dH {eh:.2e} dW {ew:.2e}", flush=True)
    assert eh <= TOL["bf16"]["grad"] and ew <= TOL["bf16"]["grad"]


def test_bitwise_determinism():
    w, x = _inputs("small_bf16", dict(N=512, V=8000, chunk=200), 23)
    a = run_gpu(x, w.T, w.chunk)
    b = run_gpu(x, w.T, w.chunk)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["row_lse"], b["row_lse"])
    assert np.array_equal(a["dH"], b["dH"])
    assert np.array_equal(a["dW"], b["dW"])


def test_k_equals_one_is_cross_entropy():
    w, x = _inputs("tiny_fp32", dict(N=40, V=700, K=1, chunk=16, T=1.0), 24)
    got = run_gpu(x, w.T, w.chunk)
    Z = x["H"].double() @ x["W"].double().T
    ce = torch.nn.functional.cross_entropy(Z, x["ids"][:, 0].long()).item()
    assert abs(got["loss"] - ce) <= 1e-5 * abs(ce)


def test_k_equals_v_and_matching_teacher_gives_zero():
    # teacher logits equal to the student's logits over the whole vocabulary
    w, x = _inputs("tiny_fp32", dict(N=20, V=64, K=64, chunk=8, T=1.7), 25)
    ids = torch.stack([torch.randperm(64, generator=torch.Generator().manual_seed(i))
                       for i in range(20)]).to(torch.int32)
    Z = (x["H"].double() @ x["W"].double().T)
    x["ids"] = ids
    x["logits"] = torch.gather(Z, 1, ids.long()).float()
    got = run_gpu(x, w.T, w.chunk)
    assert abs(got["loss"]) < 1e-5
    assert np.abs(got["dH"]).max() < 1e-6 and np.abs(got["dW"]).max() < 1e-6


def test_uniform_student_closed_form():
    # W = 0: KL_i = log V - entropy of the teacher's renormalised top-K
    w, x = _inputs("small_bf16", dict(N=33, V=1234 * 8, K=50, chunk=16, T=2.0), 26)
    x["W"] = torch.zeros_like(x["W"])
    got = run_gpu(x, w.T, w.chunk)
    import scipy.stats as sst
    lg = x["logits"].double().numpy()
    ent = np.array([sst.entropy(np.exp(lg[i] / w.T)) for i in range(w.N)])
    ref = np.mean(math.log(w.V) - ent)
    assert abs(got["loss"] - ref) <= 1e-4 * abs(ref)
    assert np.abs(got["dH"]).max() == 0.0


@pytest.mark.parametrize("options", [None, {"loss": 1, "beta": 0.5}, {"loss": 4}], ids=["kl", "jsd", "trkl"])
def test_empty_input(options):
    """No positions: the loss is NaN (a mean over none), dW is zeroed, or
    left as it was with accumulate_dW; for the KL, the generalised JSD and the
    reverse KL over the top-K support."""
    import chunked_kl_loss_amd as kd

    dev = "cuda:0"
    print(f"case empty input, options {options}", flush=True)
    H = torch.zeros(0, 64, dtype=torch.bfloat16, device=dev)
    W = torch.randn(300, 64, device=dev).to(torch.bfloat16)
    ids = torch.zeros(0, 4, dtype=torch.int32, device=dev)
    lg = torch.zeros(0, 4, device=dev)
    loss, lse, kl = kd.kdkl_forward(H, W, ids, lg, 1.0, 16, options=options)
    dW0 = torch.full((300, 64), 5.0, device=dev)
    dH, dW = kd.kdkl_backward(H, W, ids, lg, 1.0, 16, lse, dW=dW0.clone(), options=options)
    torch.cuda.synchronize()
    assert math.isnan(loss.item())
    assert torch.count_nonzero(dW).item() == 0
    _, dWa = kd.kdkl_backward(H, W, ids, lg, 1.0, 16, lse, dW=dW0.clone(), accumulate_dW=True, options=options)
    assert torch.equal(dWa, dW0)


@pytest.mark.parametrize("name,over,seed", [
    ("tiny_fp32", dict(N=30, V=1000, K=6, chunk=8), 27),
    ("small_bf16", dict(N=300, d=576, V=3001, K=20, chunk=128, T=1.3), 34),
    ("gptoss20b_32k", dict(N=80, V=40000, chunk=32), 35),  # backward groups, 320-wide hidden tiles
])
def test_out_of_range_and_repeated_ids(name, over, seed):
    # ids outside [0, V) and repeated ids break the pages' setting of K
    # distinct in-vocabulary ids per position; the library never faults and
    # computes the documented reading, which the oracle defines: an id
    # outside [0, V) keeps its share of the teacher's softmax but gathers a
    # zero logit outside the student's normalisation and scatters nothing; a
    # repeated id is gathered per entry and its masses add. Compared element
    # by element, with ignored positions (first id -1) mixed in.
    w, x = _inputs(name, over, seed)
    ids = x["ids"].clone()
    N = ids.shape[0]
    bad = torch.tensor([-5, w.V, w.V + 3, 2 ** 30, -2, -(2 ** 31)], dtype=torch.int32)
    ids[:, 0] = bad.repeat(N // len(bad) + 1)[:N]
    ids[::3, 2] = ids[::3, 1]                      # a repeated id in every third row
    ids[1::7, w.K - 1] = w.V - 1                   # the last vocabulary row, sometimes twice
    ids[[4, 17], 0] = -1                           # ignored positions
    x2 = dict(x, ids=ids)
    print(f"case bad ids {name}: N={w.N} d={w.d} V={w.V} K={w.K} chunk={w.chunk}", flush=True)
    got = run_gpu(x2, w.T, w.chunk, g=0.7)
    ref = oracle.loss_and_grads(x2["H"], x2["W"], x2["ids"], x2["logits"], w.T, g=0.7)
    assert_parity(got, ref, w.dtype, f"bad ids {name}")
    assert maxrel(got["row_kl"], ref["row_kl"]) <= TOL[w.dtype]["loss"] * 10


def test_autograd_function_matches_direct_calls():
    import chunked_kl_loss_amd as kd

    w, x = _inputs("small_bf16", dict(N=256, V=4096, K=32, chunk=100), 28)
    dev = "cuda:0"
    H = x["H"].to(dev).requires_grad_(True)
    W = x["W"].to(dev).requires_grad_(True)
    loss = kd.fused_kl_loss(H, W, x["ids"].to(dev), x["logits"].to(dev), w.T, w.chunk)
    (2.0 * loss).backward()
    ref = oracle.loss_and_grads(x["H"], x["W"], x["ids"], x["logits"], w.T, g=2.0)
    assert abs(loss.item() - ref["loss"]) <= 1e-3 * abs(ref["loss"])
    assert maxrel(H.grad.double().cpu().numpy(), ref["dH"]) <= 2e-2
    assert maxrel(W.grad.double().cpu().numpy(), ref["dW"]) <= 2e-2


@pytest.mark.parametrize("name,over,seed", [
    ("small_bf16", dict(N=128, V=6000, K=40, chunk=64, T=2.0), 29),
    ("longctx_256k", dict(N=96, V=40000, chunk=32), 30),  # the 256K workload's geometry and T
])
def test_temperature_identity_exact_for_T2(name, over, seed):
    # loss(H, W, l, 2) == loss(H/2, W, l/2, 1), dH_2 = dH_1 / 2 and
    # dW_2 = dW_1. Halving is exact in binary floating point, and every
    # rounding of the T = 2 run sees exactly half (or, for dW's products
    # dZ_2 H = (dZ_1 / 2)(2 H / 2), the same) of the T = 1 run's operands:
    # 1/T and the gradient scale g / (N T) are exact halves, and each
    # product with them is rounded once. So the two runs agree bit for bit.
    w, x = _inputs(name, over, seed)
    a = run_gpu(x, 2.0, w.chunk)
    x1 = dict(x, H=(x["H"].float() / 2).to(x["H"].dtype), logits=x["logits"] / 2)
    b = run_gpu(x1, 1.0, w.chunk)
    print(f"T=2 identity {name}: loss {a['loss']!r} vs {b['loss']!r}; "
          f"lse max diff {np.abs(a['row_lse'] - b['row_lse']).max():.3e}; "
          f"dH max diff {np.abs(a['dH'] - b['dH'] / 2).max():.3e}; "
          f"dW max diff {np.abs(a['dW'] - b['dW']).max():.3e}", flush=True)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["row_lse"], b["row_lse"])
    assert np.array_equal(a["row_kl"], b["row_kl"])
    assert np.array_equal(a["dH"], b["dH"] / 2.0)
    assert np.array_equal(a["dW"], b["dW"])


def _mark_ignored(x, rows):
    """First id -1 marks an ignored position; the rest of such a row is
    garbage that must never be used."""
    ids = x["ids"].clone()
    lg = x["logits"].clone()
    ids[rows, 0] = -1
    ids[rows[0], 1:] = 10 ** 9
    lg[rows[1]] = float("nan")
    return dict(x, ids=ids, logits=lg)


@pytest.mark.parametrize("name,over,seed", [
    ("tiny_fp32", dict(N=90, chunk=32), 31),
    ("small_bf16", dict(N=300, d=576, V=3001, K=20, chunk=128, T=1.3), 32),
])
def test_ignored_positions(name, over, seed):
    w, x = _inputs(name, over, seed)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(w.N, size=w.N // 4, replace=False))
    xm = _mark_ignored(x, rows)
    print(f"case ignored positions {name}: N={w.N} ignored={len(rows)}", flush=True)
    got = run_gpu(xm, w.T, w.chunk, g=0.9)
    ref = oracle.loss_and_grads(xm["H"], xm["W"], xm["ids"], xm["logits"], w.T, g=0.9)
    assert np.all(got["row_kl"][rows] == 0.0) and np.all(got["dH"][rows] == 0.0)
    assert_parity(got, ref, w.dtype, f"ignored {name}")


def test_all_positions_ignored():
    w, x = _inputs("small_bf16", dict(N=64, d=256, V=2000, K=8, chunk=32), 33)
    xm = _mark_ignored(x, np.arange(w.N))
    print("case all positions ignored", flush=True)
    got = run_gpu(xm, w.T, w.chunk)
    assert math.isnan(got["loss"])
    assert not np.any(got["dH"]) and not np.any(got["dW"])
