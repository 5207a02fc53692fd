"""The fused forward + backward (the KL and two of the alternative losses)
captured once into a HIP graph (torch's CUDA graph API on ROCm) and
replayed: each replay, run after eager work and a synchronisation, must
equal the eager result bit for bit (the path launches only its own kernels
on the caller's stream and records no memset nodes). Also the
forward-chunked path."""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


# the KL, the generalised JSD and the reverse KL over the top-K support
# (whose sparse dW counts entries with integer atomics and must still give
# the same bits on every replay)
LOSSES = [("kl", None), ("jsd", {"loss": 1, "beta": 0.5}), ("trkl", {"loss": 4})]


@pytest.mark.parametrize("name,options", LOSSES, ids=[c[0] for c in LOSSES])
def test_fused_step_graph_replays_match_eager(name, options):
    import chunked_kl_loss_amd as kd

    w = wl.get_config("small_bf16").with_(N=640, d=576, V=5000, K=32, chunk=256)
    print(f"case graph capture fused step, loss {name}", flush=True)
    inputs = [wl.generate(w, seed=s) for s in (51, 52, 53)]
    dev = torch.device(DEV)
    H = inputs[0]["H"].to(dev)
    W = inputs[0]["W"].to(dev)
    ids = inputs[0]["ids"].to(dev)
    lg = inputs[0]["logits"].to(dev)
    fb, bb = kd.workspace_size(w.N, w.d, w.V, w.K, w.chunk, H.dtype, options=options)
    ws_f = torch.empty(fb, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bb, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(kd.saved_shape(w.N, options), dtype=torch.float32, device=dev)
    kl = torch.empty(w.N, dtype=torch.float32, device=dev)
    g = torch.tensor([0.7], dtype=torch.float32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty((w.V, w.d), dtype=torch.float32, device=dev)

    def step(stream):
        kd.kdkl_forward(H, W, ids, lg, w.T, w.chunk, loss=loss, row_lse=lse, row_kl=kl,
                        workspace=ws_f, stream=stream, options=options)
        kd.kdkl_backward(H, W, ids, lg, w.T, w.chunk, lse, g, dH=dH, dW=dW, workspace=ws_b,
                         stream=stream, options=options)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step(side)  # warm up outside the capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize(dev)

    for rep in range(3):
        x = inputs[rep % len(inputs)]
        H.copy_(x["H"])
        W.copy_(x["W"])
        ids.copy_(x["ids"])
        lg.copy_(x["logits"])
        torch.cuda.synchronize(dev)
        graph.replay()
        torch.cuda.synchronize(dev)
        got = [t.clone() for t in (loss, lse, kl, dH, dW)]
        # some unrelated eager work between replays
        _ = (torch.randn(1000, 1000, device=dev) @ torch.randn(1000, 1000, device=dev)).sum().item()
        step(torch.cuda.current_stream(dev))
        torch.cuda.synchronize(dev)
        ref = (loss, lse, kl, dH, dW)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
        print(f"replay {rep}: loss {got[0].item():.6f} equals eager", flush=True)
        assert np.isfinite(got[0].item())


def test_logits_step_graph_replays_match_eager():
    import chunked_kl_loss_amd as kd

    print("case graph capture forward-chunked step", flush=True)
    dev = torch.device(DEV)
    gen = torch.Generator(device=dev).manual_seed(54)
    N, V, K = 300, 7001, 50
    Z = torch.randn(N, V, generator=gen, device=dev).to(torch.bfloat16)
    ids = torch.randint(0, V, (N, K), generator=gen, device=dev, dtype=torch.int32)
    ids[::7, 0] = -1  # some ignored positions
    lg = torch.randn(N, K, generator=gen, device=dev)
    loss = torch.empty(1, device=dev)
    lse = torch.empty(N, device=dev)
    kl = torch.empty(N, device=dev)
    dZ = torch.empty_like(Z)
    ws = torch.empty(kd.LOGITS_BWD_WORKSPACE, dtype=torch.uint8, device=dev)

    def step(stream):
        kd.logits_forward(Z, ids, lg, 1.3, loss=loss, row_lse=lse, row_kl=kl, stream=stream)
        kd.logits_backward(Z, ids, lg, 1.3, lse, None, dZ=dZ, workspace=ws, stream=stream)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    for rep in range(3):
        Z.copy_(torch.randn(N, V, generator=gen, device=dev).to(torch.bfloat16))
        torch.cuda.synchronize(dev)
        graph.replay()
        torch.cuda.synchronize(dev)
        got = [t.clone() for t in (loss, lse, kl, dZ)]
        step(torch.cuda.current_stream(dev))
        torch.cuda.synchronize(dev)
        for a, b in zip(got, (loss, lse, kl, dZ)):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
