"""GPU parity of the alternative losses (generalised Jensen-Shannon
divergence, skew KL, skew reverse KL) at the full 32K gpt-oss-like workload,
in the launch configuration bench.py times for it (one group of sixteen
chunks over vocabulary quarters): sampled rows that the CPU oracle computes
on their own (rows are independent; the gradient's scale g / (N T) is the
whole problem's), plus properties that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

LOSSES = [("jsd", 1, 0.5), ("skl", 2, 0.1), ("srkl", 3, 0.1)]  # (oracle name, kdkl_loss, parameter)


@pytest.fixture(scope="module")
def workload():
    w = wl.get_config("gptoss20b_32k")
    return w, wl.generate(w)


@pytest.mark.parametrize("loss,code,a", LOSSES, ids=[l[0] for l in LOSSES])
def test_alt_loss_full_size(workload, loss, code, a):
    import chunked_kl_loss_amd as kd

    w, x = workload
    opts = {"loss": code, "beta": a}
    plan = kd.plan_info(w.N, w.d, w.V, w.K, w.chunk, w.torch_dtype, opts)
    print(f"case {loss} full size {w.name}: N={w.N} plan {plan}", flush=True)
    dev = "cuda:0"
    H, W, ids, lg = (x[k].to(dev) for k in ("H", "W", "ids", "logits"))
    out, row_lse, row_kl = kd.kdkl_forward(H, W, ids, lg, w.T, w.chunk, options=opts)
    g = 0.7
    dH, dW = kd.kdkl_backward(H, W, ids, lg, w.T, w.chunk, row_lse,
                              torch.tensor([g], dtype=torch.float32, device=dev), options=opts)
    torch.cuda.synchronize()
    got_loss = out.item()
    lse = row_lse[0].double().cpu().numpy()
    rk = row_kl.double().cpu().numpy()
    dH, dW = dH.cpu(), dW.cpu()
    del H, W, ids, lg
    torch.cuda.empty_cache()

    # the loss is the mean of the rows' values (every position is kept)
    assert abs(got_loss - rk.mean()) <= 1e-5 * abs(rk.mean())
    rng = np.random.default_rng(11 + code)
    rows = sorted({0, 1, w.chunk - 1, w.chunk, w.N // 2, w.N - 1} |
                  set(rng.choice(w.N, size=10, replace=False).tolist()))
    sub = {k: x[k][rows] for k in ("H", "ids", "logits")}
    ref = oracle.alt_forward(sub["H"], x["W"], sub["ids"], sub["logits"], w.T, loss, a)
    e_lse = np.abs(lse[rows] - ref["row_lse"]).max() / np.abs(ref["row_lse"]).max()
    e_kl = np.abs(rk[rows] - ref["row_kl"]).max() / np.abs(ref["row_kl"]).max()
    rH, _ = oracle.alt_backward(sub["H"], x["W"], sub["ids"], sub["logits"], w.T, loss, a, g)
    rH *= len(rows) / w.N  # the whole problem's scale g / (N T)
    e_dh = float(np.abs(dH[rows].double().numpy() - rH).max() / np.abs(rH).max())
    print(f"{loss} {w.name} sampled rows {len(rows)}: lse {e_lse:.2e} value {e_kl:.2e} dH {e_dh:.2e}", flush=True)
    assert e_lse <= 1e-5 and e_kl <= 1e-3 and e_dh <= 2e-2
    # every dZ row sums to zero: dW's columns sum to (nearly) zero
    cs = dW.double().sum(0).abs()
    ca = dW.double().abs().sum(0)
    assert float((cs / ca).max()) <= 1e-2
    # <W, dW> = <H, dH>: both are the sum over (n, v) of dZ_nv z_nv
    wd = float((x["W"].double() * dW.double()).sum())
    hd, scale = 0.0, 0.0
    for r0 in range(0, w.N, 16384):
        h = x["H"][r0:r0 + 16384].double()
        gh = dH[r0:r0 + 16384].double()
        hd += float((h * gh).sum())
        scale += float((h * gh).abs().sum())
    print(f"{loss}: <W,dW> {wd:.6e} <H,dH> {hd:.6e} scale {scale:.3e}", flush=True)
    assert abs(wd - hd) <= 1e-3 * scale
