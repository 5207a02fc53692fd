"""The allocation-free forward (kdkl_forward_noalloc, static device scratch)
against kdkl_forward (caller's workspace) through the C-ABI: two calls in a
row, the second with a smaller input, each equal bit for bit (the blocking
never changes per-row arithmetic) and within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _both(w, x, options=None):
    import chunked_kl_loss_amd as kd

    dev = torch.device(DEV)
    H, W, ids, lg = (x[k].to(dev) for k in ("H", "W", "ids", "logits"))
    ref_loss, ref_lse, ref_kl = kd.kdkl_forward(H, W, ids, lg, w.T, w.chunk, options=options)
    loss = torch.full((1,), float("nan"), device=dev)
    lse = torch.full(kd.saved_shape(w.N, options), float("nan"), device=dev)
    kl = torch.full((w.N,), float("nan"), device=dev)
    torch.cuda.synchronize(dev)
    before = torch.cuda.memory_allocated(dev)
    kd.kdkl_forward_noalloc(H, W, ids, lg, w.T, w.chunk, loss=loss, row_lse=lse, row_kl=kl, options=options)
    torch.cuda.synchronize(dev)
    assert torch.cuda.memory_allocated(dev) == before
    return (ref_loss.item(), ref_lse.cpu().numpy(), ref_kl.cpu().numpy()), \
        (loss.item(), lse.cpu().numpy(), kl.cpu().numpy())


def test_forward_noalloc_matches_forward_twice():
    import chunked_kl_loss_amd as kd

    # gpt-oss-like head, 8192 positions in chunks of 2048: the library's
    # forward takes all four chunks per launch (84 MB of workspace), the
    # allocation-free one two (42 MB of its 64 MiB array)
    w1 = wl.get_config("gptoss20b_32k").with_(N=8192)
    p1 = kd.plan_info(w1.N, w1.d, w1.V, w1.K, w1.chunk, w1.torch_dtype)
    assert p1["chunks_per_group"] == 4 and p1["fwd_bytes"] > (64 << 20)
    # then a smaller input: 3000 positions (a full chunk and a ragged one) of
    # another seed, with ignored positions and ids outside [0, V)
    w2 = w1.with_(N=3000)
    for w, seed in ((w1, 61), (w2, 62)):
        x = wl.generate(w, seed=seed)
        if w is w2:
            ids = x["ids"].clone()
            ids[[5, 2100], 0] = -1
            ids[7, 3] = w.V + 11
            x = dict(x, ids=ids)
        print(f"case noalloc N={w.N} d={w.d} V={w.V} chunk={w.chunk} seed={seed}", flush=True)
        ref, got = _both(w, x)
        assert got[0] == ref[0], (got[0], ref[0])
        assert np.array_equal(got[1], ref[1]) and np.array_equal(got[2], ref[2])
        rows = [0, 1, w.chunk - 1, w.chunk, w.N - 1]
        o = oracle.sampled_rows(x["H"], x["W"], x["ids"], x["logits"], w.T, rows, w.N)
        e_lse = np.abs(got[1][rows] - o["row_lse"]).max() / np.abs(o["row_lse"]).max()
        e_kl = np.abs(got[2][rows] - o["row_kl"]).max() / np.abs(o["row_kl"]).max()
        print(f"noalloc N={w.N}: loss {got[0]:.7g}; oracle rows lse {e_lse:.2e} kl {e_kl:.2e}", flush=True)
        assert e_lse <= 1e-3 and e_kl <= 1e-3


def test_forward_noalloc_alternative_loss():
    """An alternative loss (the skew reverse KL) through the allocation-free
    forward: its extra per-group buffer of student logits at the teacher
    entries also lives in the static array; results equal kdkl_forward's bit
    for bit, both saved rows (logsumexp and gbar) included."""
    import chunked_kl_loss_amd as kd

    w = wl.get_config("gptoss20b_32k").with_(N=8192)
    opts = {"loss": kd.KDKL_LOSS_SRKL, "beta": 0.1}
    x = wl.generate(w, seed=63)
    print(f"case noalloc srkl N={w.N} chunk={w.chunk}", flush=True)
    ref, got = _both(w, x, opts)
    assert got[0] == ref[0], (got[0], ref[0])
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[2], ref[2])
    rows = [0, w.chunk, w.N - 1]
    sub = {k: x[k][rows] for k in ("H", "ids", "logits")}
    o = oracle.alt_forward(sub["H"], x["W"], sub["ids"], sub["logits"], w.T, "srkl", 0.1)
    e_kl = np.abs(got[2][rows] - o["row_kl"]).max() / np.abs(o["row_kl"]).max()
    assert e_kl <= 1e-3, e_kl
