"""GPU parity at full workload sizes, in the launch configuration bench.py
times (same workload, chunk and dtype): sampled outputs that the CPU oracle
computes one row at a time, plus properties that hold at any size."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(w, x):
    import chunked_kl_loss_amd as kd

    dev = "cuda:0"
    H, W, ids, lg = (x[k].to(dev) for k in ("H", "W", "ids", "logits"))
    loss, row_lse, row_kl = kd.kdkl_forward(H, W, ids, lg, w.T, w.chunk)
    dH, dW = kd.kdkl_backward(H, W, ids, lg, w.T, w.chunk, row_lse)
    torch.cuda.synchronize()
    out = {"loss": loss.item(), "row_lse": row_lse.double().cpu().numpy(),
           "row_kl": row_kl.double().cpu().numpy(), "dH": dH.cpu(), "dW": dW.cpu()}
    del H, W, ids, lg, dH, dW
    torch.cuda.empty_cache()
    return out


def _sample_rows(w, rng, n=12):
    fixed = {0, 1, w.chunk - 1, w.chunk, w.N // 2, w.N - 1}
    rnd = set(rng.choice(w.N, size=n, replace=False).tolist())
    return sorted(fixed | rnd)


def _check_rows(w, x, got, rows):
    ref = oracle.sampled_rows(x["H"], x["W"], x["ids"], x["logits"], w.T, rows, w.N)
    e_lse = np.abs(got["row_lse"][rows] - ref["row_lse"]).max() / np.abs(ref["row_lse"]).max()
    e_kl = np.abs(got["row_kl"][rows] - ref["row_kl"]).max() / np.abs(ref["row_kl"]).max()
    dh = got["dH"][rows].double().numpy()
    e_dh = np.abs(dh - ref["dH_rows"]).max() / np.abs(ref["dH_rows"]).max()
    print(f"{w.name} sampled rows {len(rows)}: lse {e_lse:.2e} kl {e_kl:.2e} dH {e_dh:.2e}", flush=True)
    assert e_lse <= 1e-3 and e_kl <= 1e-3 and e_dh <= 2e-2


def _check_properties(w, x, got):
    # loss is the mean of the per-row KL the same call wrote
    mean_kl = float(np.mean(got["row_kl"]))
    assert abs(got["loss"] - mean_kl) <= 1e-5 * abs(mean_kl)
    # every dZ row sums to zero, so each column of dW sums to ~0
    dW = got["dW"]
    cs = dW.double().sum(0).abs()
    ca = dW.double().abs().sum(0)
    assert float((cs / ca).max()) <= 1e-2, float((cs / ca).max())
    # <W, dW> = <H, dH>: both equal sum over (n, v) of dZ_nv z_nv
    wd = float((x["W"].double() * dW.double()).sum())
    hd = 0.0
    scale = 0.0
    for r0 in range(0, w.N, 16384):
        h = x["H"][r0:r0 + 16384].double()
        g = got["dH"][r0:r0 + 16384].double()
        hd += float((h * g).sum())
        scale += float((h * g).abs().sum())
    print(f"{w.name}: <W,dW> {wd:.6e} <H,dH> {hd:.6e} scale {scale:.3e}", flush=True)
    assert abs(wd - hd) <= 1e-3 * scale


def _check_against_stored_oracle(w, x, got, rng):
    """Every row's lse and KL and the loss against the oracle's stored
    per-row results (written by tests/golden/make_fullsize_oracle.py, which
    calls only the oracle), and sampled rows of dW, which need every row's
    lse (the stored oracle values)."""
    g = np.load(os.path.join(GOLDEN, f"oracle_{w.name}_rows.npz"))
    assert int(g["seed"]) == wl.seed_for(w)
    assert g["row_lse"].shape == (w.N,)
    rel = abs(got["loss"] - float(g["loss"])) / abs(float(g["loss"]))
    e_lse = np.abs(got["row_lse"] - g["row_lse"]).max() / np.abs(g["row_lse"]).max()
    e_kl = np.abs(got["row_kl"] - g["row_kl"]).max() / np.abs(g["row_kl"]).max()
    print(f"{w.name} full rows: loss {got['loss']:.9g} vs {float(g['loss']):.9g} rel {rel:.2e}; "
          f"lse {e_lse:.2e} kl {e_kl:.2e}", flush=True)
    assert rel <= 1e-3 and e_lse <= 1e-3 and e_kl <= 1e-3
    ids = x["ids"].numpy()
    vrows = sorted({0, 1, 5, 255, 256, int(ids[0, 0]), int(ids[123, 7]), w.V - 129, w.V - 1}
                   | set(rng.choice(w.V, size=8, replace=False).tolist()))
    ref = oracle.dw_rows(x["H"], x["W"], x["ids"], x["logits"], w.T, vrows, g["row_lse"])
    dw = got["dW"][vrows].double().numpy()
    e_dw = np.abs(dw - ref).max() / np.abs(ref).max()
    print(f"{w.name} sampled dW rows {len(vrows)}: {e_dw:.2e}", flush=True)
    assert e_dw <= 2e-2


def test_gptoss20b_32k_full_size():
    w = wl.get_config("gptoss20b_32k")
    x = wl.generate(w)
    got = _run(w, x)
    rng = np.random.default_rng(7)
    _check_against_stored_oracle(w, x, got, rng)
    _check_rows(w, x, got, _sample_rows(w, rng))
    _check_properties(w, x, got)


def test_longctx_256k_full_size():
    # the launch configuration the default bench times (T = 2, chunks of 4096
    # in groups of eight over vocabulary quarters, W^T copy)
    w = wl.get_config("longctx_256k")
    x = wl.generate(w)
    got = _run(w, x)
    rng = np.random.default_rng(8)
    _check_against_stored_oracle(w, x, got, rng)
    _check_rows(w, x, got, _sample_rows(w, rng, n=6))
    _check_properties(w, x, got)


def test_llama3b_8k_full_size():
    # all eight chunks in one group over the whole vocabulary, W read in place
    w = wl.get_config("llama3b_8k")
    x = wl.generate(w)
    got = _run(w, x)
    rng = np.random.default_rng(9)
    _check_against_stored_oracle(w, x, got, rng)
    _check_rows(w, x, got, _sample_rows(w, rng))
    _check_properties(w, x, got)
