"""Helpers for the GPU tests: run the HIP path through the C-ABI binding and
compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances: loss relative error; gradients max-norm-relative error
# (||gpu - ref||_inf / ||ref||_inf over the whole tensor).
TOL = {
    "fp32": {"loss": 1e-5, "grad": 1e-5},
    "bf16": {"loss": 1e-3, "grad": 2e-2},
}


def to_dev(x, dev="cuda:0"):
    return {k: v.to(dev) for k, v in x.items()}


def run_gpu(x, T, chunk, g=None, accumulate_dW=False, dW_init=None, stream=None, options=None):
    """Forward + backward on cuda:0; returns numpy fp64 results."""
    import chunked_kl_loss_amd as kd

    d = to_dev(x)
    loss, row_lse, row_kl = kd.kdkl_forward(d["H"], d["W"], d["ids"], d["logits"], T, chunk,
                                            stream=stream, options=options)
    gt = None if g is None else torch.tensor([g], dtype=torch.float32, device="cuda:0")
    dW = None if dW_init is None else dW_init.clone().to("cuda:0")
    dH, dW = kd.kdkl_backward(d["H"], d["W"], d["ids"], d["logits"], T, chunk, row_lse, gt,
                              dW=dW, accumulate_dW=accumulate_dW, stream=stream, options=options)
    torch.cuda.synchronize()
    lse = row_lse[0] if row_lse.dim() == 2 else row_lse  # the JSD saves [lse; gbar]
    return {
        "loss": float(loss.item()),
        "row_lse": lse.double().cpu().numpy(),
        "row_kl": row_kl.double().cpu().numpy(),
        "dH": dH.double().cpu().numpy(),
        "dW": dW.double().cpu().numpy(),
        "_dev": {"loss": loss, "row_lse": row_lse, "dH": dH, "dW": dW},
    }


def maxrel(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a - b).max())


def assert_parity(got, ref, dtype, what=""):
    tol = TOL[dtype]
    rl = abs(got["loss"] - ref["loss"]) / abs(ref["loss"])
    eh = maxrel(got["dH"], ref["dH"])
    ew = maxrel(got["dW"], ref["dW"])
    lse = np.abs(got["row_lse"] - ref["row_lse"]).max() / np.abs(ref["row_lse"]).max()
    msg = (f"{what}: loss {got['loss']:.7g} vs {ref['loss']:.7g} rel {rl:.2e}; "
           f"row_lse {lse:.2e}; dH {eh:.2e}; dW {ew:.2e} (tol {tol})")
    print(msg, flush=True)
    assert rl <= tol["loss"], msg
    assert lse <= tol["loss"], msg
    assert eh <= tol["grad"], msg
    assert ew <= tol["grad"], msg
