"""GPU parity of the forward-chunked KL path (the student's logit grid Z is
given) against the CPU oracle, element by element, through the C-ABI.

Z is drawn on the host as the product of the workload's seeded H and W
(rounded to the storage dtype), so both sides read identical bytes. Row
lengths with a row start off a 16-byte boundary exercise the scalar head and
tail of each row."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import TOL, maxrel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _problem(dtype, N, V, K, seed, T=1.0):
    rng = np.random.default_rng(seed)
    d = 64
    H = torch.from_numpy(rng.standard_normal((N, d)).astype(np.float32))
    W = torch.from_numpy((rng.standard_normal((V, d)) / math.sqrt(d)).astype(np.float32))
    Z = (H @ W.T).to(dtype)
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(N)]) if N else np.zeros((0, K))
    ids = torch.from_numpy(ids.astype(np.int32))
    lg = torch.from_numpy(np.sort(rng.standard_normal((N, K)) * math.sqrt(2.0), axis=1)[:, ::-1]
                          .astype(np.float32).copy())
    return Z, ids, lg


def _run(Z, ids, lg, T, g=None, inplace=False):
    import chunked_kl_loss_amd as kd

    Zd, idd, lgd = Z.to(DEV), ids.to(DEV), lg.to(DEV)
    loss, lse, kl = kd.logits_forward(Zd, idd, lgd, T)
    gt = None if g is None else torch.tensor([g], dtype=torch.float32, device=DEV)
    dZ = kd.logits_backward(Zd, idd, lgd, T, lse, gt, dZ=Zd if inplace else None)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "row_lse": lse.double().cpu().numpy(),
            "row_kl": kl.double().cpu().numpy(), "dZ": dZ.double().cpu().numpy()}


def _check(got, Z, ids, lg, T, g, kind, what):
    ref_f = oracle.logits_forward(Z, ids, lg, T)
    ref_dz = oracle.logits_backward(Z, ids, lg, T, g)
    tol = TOL[kind]
    rl = abs(got["loss"] - ref_f["loss"]) / max(abs(ref_f["loss"]), 1e-30)
    el = maxrel(got["row_lse"], ref_f["row_lse"])
    ek = maxrel(got["row_kl"], ref_f["row_kl"])
    ed = maxrel(got["dZ"], ref_dz)
    msg = f"{what}: loss rel {rl:.2e} lse {el:.2e} kl {ek:.2e} dZ {ed:.2e} (tol {tol})"
    print(msg, flush=True)
    assert rl <= tol["loss"] and el <= tol["loss"] and ek <= tol["loss"], msg
    assert ed <= tol["grad"], msg


@pytest.mark.parametrize("dtype,kind,N,V,K,T,g", [
    (torch.float32, "fp32", 130, 1001, 16, 1.0, None),    # fp32 rows start 4 bytes apart
    (torch.float32, "fp32", 64, 4096, 100, 2.0, 0.7),     # aligned rows, T = 2
    (torch.bfloat16, "bf16", 257, 5003, 100, 1.0, None),  # bf16, ragged row starts
    (torch.bfloat16, "bf16", 96, 32000, 100, 1.0, 1.3),   # configuration-sized vocabulary
    (torch.bfloat16, "bf16", 33, 7, 3, 1.5, None),        # V smaller than one vector
    (torch.bfloat16, "bf16", 40, 3000, 300, 1.0, None),   # K > 256 (16 slots per lane)
])
def test_logits_parity_vs_oracle(dtype, kind, N, V, K, T, g):
    print(f"case logits {kind} N={N} V={V} K={K} T={T} g={g}", flush=True)
    Z, ids, lg = _problem(dtype, N, V, K, seed=N + V + K)
    got = _run(Z, ids, lg, T, g)
    _check(got, Z, ids, lg, T, 1.0 if g is None else g, kind, f"{kind} N={N} V={V} K={K}")


@pytest.mark.parametrize("dtype,kind,N,V,K,T", [
    (torch.bfloat16, "bf16", 24, 150000, 100, 1.0),  # two pieces per row
    (torch.float32, "fp32", 12, 70000, 300, 1.5),    # fp32, two teacher entries per thread
    (torch.bfloat16, "bf16", 8, 16384, 1024, 1.0),   # one piece per row, K = 1024
    (torch.bfloat16, "bf16", 10, 16376, 100, 1.0),   # a vector short of the piece path
])
def test_logits_long_rows(dtype, kind, N, V, K, T):
    """Rows of whole 16-byte vectors long enough for the backward's
    workgroup-per-piece layout (and one just short of it): repeated and
    dropped ids, an id on each side of a piece boundary, an ignored row, and
    the in-place gradient equal to the out-of-place one."""
    print(f"case logits long rows {kind} N={N} V={V} K={K}", flush=True)
    Z, ids, lg = _problem(dtype, N, V, K, seed=N + V + K)
    es = 2 if dtype == torch.bfloat16 else 4
    nvec = V * es // 16
    pieces = -(-nvec // 16384)
    edge = -(-nvec // pieces) * (16 // es)  # first column of the second piece
    ids[0, 1] = ids[0, 0]                      # repeated: the masses add
    ids[1, 2], ids[1, 3] = V, -3               # outside [0, V): dropped
    ids[2, 0] = -1                             # ignored position
    ids[3, 4], ids[3, 5] = edge - 1, min(edge, V - 1)
    ids[4, 6], ids[4, 7] = 0, V - 1
    g = 0.9
    got = _run(Z, ids, lg, T, g)
    inp = _run(Z, ids, lg, T, g, inplace=True)
    assert np.array_equal(got["dZ"], inp["dZ"])
    assert np.all(got["dZ"][2] == 0.0) and got["row_kl"][2] == 0.0
    _check(got, Z, ids, lg, T, g, kind, f"long rows {kind} N={N} V={V} K={K}")


def test_logits_k1_cross_entropy_and_single_entry_vocab():
    import torch.nn.functional as F

    print("case logits K=1 and V=1", flush=True)
    Z, ids, lg = _problem(torch.float32, 50, 333, 1, seed=3)
    got = _run(Z, ids, lg, 1.0)
    ce = F.cross_entropy(Z.double(), ids[:, 0].long()).item()
    assert abs(got["loss"] - ce) <= 1e-5 * abs(ce)
    Z1 = torch.randn(9, 1)
    got = _run(Z1, torch.zeros(9, 1, dtype=torch.int32), torch.randn(9, 1), 1.0)
    assert abs(got["loss"]) <= 1e-6 and np.all(np.abs(got["dZ"]) <= 1e-6)


def test_logits_duplicate_and_out_of_range_ids():
    print("case logits duplicate and out-of-range ids", flush=True)
    Z, ids, lg = _problem(torch.float32, 24, 500, 6, seed=4)
    ids[:, 1] = ids[:, 0]                                   # duplicates add their mass
    ids[:, 5] = torch.tensor([-1, 500, 503, 2 ** 30] * 6)  # dropped, never read
    got = _run(Z, ids, lg, 1.0)
    assert np.isfinite(got["dZ"]).all()
    _check(got, Z, ids, lg, 1.0, 1.0, "fp32", "dup/out-of-range")


def test_logits_masked_vocabulary_entries():
    # -inf logits (vocabulary entries masked out by the caller) take no
    # probability and get a zero gradient
    print("case logits -inf entries", flush=True)
    Z, ids, lg = _problem(torch.float32, 20, 700, 8, seed=5)
    Z[:, 600:] = -float("inf")
    ids = ids % 600
    got = _run(Z, ids, lg, 1.0)
    assert np.all(got["dZ"][:, 600:] == 0.0)
    Zc = Z[:, :600].contiguous()
    ref = oracle.logits_forward(Zc, ids, lg, 1.0)
    assert maxrel(got["row_lse"], ref["row_lse"]) <= 1e-5
    assert maxrel(got["dZ"][:, :600], oracle.logits_backward(Zc, ids, lg, 1.0)) <= 1e-5


def test_logits_empty_input():
    import chunked_kl_loss_amd as kd

    print("case logits N=0", flush=True)
    Z = torch.empty(0, 100, dtype=torch.bfloat16, device=DEV)
    ids = torch.empty(0, 4, dtype=torch.int32, device=DEV)
    lg = torch.empty(0, 4, device=DEV)
    loss, lse, kl = kd.logits_forward(Z, ids, lg, 1.0)
    dZ = kd.logits_backward(Z, ids, lg, 1.0, lse)
    torch.cuda.synchronize()
    assert math.isnan(loss.item()) and dZ.numel() == 0


def test_logits_in_place_and_determinism():
    print("case logits in-place and determinism", flush=True)
    Z, ids, lg = _problem(torch.bfloat16, 200, 4099, 100, seed=6)
    a = _run(Z, ids, lg, 1.0)
    b = _run(Z, ids, lg, 1.0)
    c = _run(Z, ids, lg, 1.0, inplace=True)
    assert a["loss"] == b["loss"] and np.array_equal(a["row_lse"], b["row_lse"])
    assert np.array_equal(a["dZ"], b["dZ"]) and np.array_equal(a["dZ"], c["dZ"])


def test_logits_autograd_function():
    import chunked_kl_loss_amd as kd

    print("case logits autograd", flush=True)
    Z, ids, lg = _problem(torch.bfloat16, 128, 2048, 32, seed=7)
    Zd = Z.to(DEV).requires_grad_(True)
    loss = kd.forward_chunked_kl_loss(Zd, ids.to(DEV), lg.to(DEV), 1.5)
    (2.0 * loss).backward()
    ref = oracle.logits_backward(Z, ids, lg, 1.5, 2.0)
    assert maxrel(Zd.grad.double().cpu().numpy(), ref) <= TOL["bf16"]["grad"]
    assert abs(loss.item() - oracle.logits_forward(Z, ids, lg, 1.5)["loss"]) <= 1e-4


def test_logits_ignored_positions():
    print("case logits ignored positions", flush=True)
    Z, ids, lg = _problem(torch.bfloat16, 150, 3003, 50, seed=8)
    rows = np.arange(0, 150, 4)
    ids[rows, 0] = -1
    ids[rows[0], 1:] = 10 ** 9  # never used
    lg[rows[1]] = float("nan")  # never used
    got = _run(Z, ids, lg, 1.2, 0.8)
    assert np.all(got["row_kl"][rows] == 0.0) and np.all(got["dZ"][rows] == 0.0)
    _check(got, Z, ids, lg, 1.2, 0.8, "bf16", "logits ignored positions")
    ids_all = ids.clone()
    ids_all[:, 0] = -1
    got = _run(Z, ids_all, lg, 1.0)
    assert math.isnan(got["loss"]) and not np.any(got["dZ"])


def test_logits_full_size_gptoss20b_32k():
    """The 32K-position gpt-oss-like workload (N=32768, V=201088, K=100, bf16)
    with Z = H W^T computed on the device: sampled rows against the oracle and
    properties that hold at any size."""
    import chunked_kl_loss_amd as kd

    w = wl.get_config("gptoss20b_32k")
    print(f"case logits full size {w.name}", flush=True)
    x = wl.generate(w)
    Hd, Wd = x["H"].to(DEV), x["W"].to(DEV)
    Z = torch.matmul(Hd, Wd.T.contiguous())  # bf16 [N, V]
    del Hd, Wd
    ids, lg = x["ids"].to(DEV), x["logits"].to(DEV)
    loss, lse, kl = kd.logits_forward(Z, ids, lg, w.T)
    dZ = kd.logits_backward(Z, ids, lg, w.T, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = sorted({0, 1, 4095, w.N // 2, w.N - 1} | set(rng.choice(w.N, 8, replace=False).tolist()))
    Zr = Z[rows].cpu()
    ref = oracle.logits_sampled_rows(Zr, x["ids"][rows], x["logits"][rows], w.T, range(len(rows)), w.N)
    got_dz = dZ[rows].double().cpu().numpy()
    e_lse = maxrel(lse[rows].double().cpu().numpy(), ref["row_lse"])
    e_kl = maxrel(kl[rows].double().cpu().numpy(), ref["row_kl"])
    e_dz = maxrel(got_dz, ref["dZ_rows"])
    print(f"full size sampled rows {len(rows)}: lse {e_lse:.2e} kl {e_kl:.2e} dZ {e_dz:.2e}", flush=True)
    assert e_lse <= 1e-4 and e_kl <= 1e-4 and e_dz <= TOL["bf16"]["grad"]
    # loss is the mean of the per-row KL; each dZ row sums to ~0
    mean_kl = float(kl.double().mean().item())
    assert abs(loss.item() - mean_kl) <= 1e-5 * abs(mean_kl)
    rs, ra = 0.0, float("inf")
    for r0 in range(0, w.N, 4096):
        blk = dZ[r0:r0 + 4096].double()
        rs = max(rs, blk.sum(1).abs().max().item())
        ra = min(ra, blk.abs().sum(1).min().item())
        del blk
    assert rs <= 1e-2 * ra, (rs, ra)
    # the in-place gradient equals the out-of-place one
    dZ2 = kd.logits_backward(Z, ids, lg, w.T, lse, dZ=Z)
    torch.cuda.synchronize()
    assert torch.equal(dZ2, dZ)
