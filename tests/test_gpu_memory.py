"""Peak device memory of one fused forward + backward is linear in the number
of positions, with the slope of the per-position tensors alone.

The pages' long-context benchmark shows the fused chunked loss keeping memory
flat where the dense loss runs out [P1 "Making knowledge distillation cheap
enough to run at scale", section "Two system changes", the isolated benchmark
at 256K positions]. Here that claim is checked at the 256K workload's
geometry (d=2880, V=201088, K=100, chunk 4096, T=2): the peak over the call
must be a + b * N with b the bytes each position owns (H and dH in bf16, the
teacher ids and logits, the saved row logsumexp and the per-row KL), so that
nothing the path allocates grows with N beyond them.

Values do not enter a memory measurement; inputs are drawn on the device from
a seeded generator with the workload's distributions (H ~ N(0, 1),
W ~ N(0, 1/d), logits ~ N(0, 2), ids uniform on [0, V)).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

D, V, K, CHUNK, T = 2880, 201088, 100, 4096, 2.0
PER_POSITION = 2 * D + 2 * D + 4 * K + 4 * K + 4 + 4  # H, dH, ids, logits, row_lse, row_kl


def _peak_bytes(N: int, W: torch.Tensor, seed: int) -> int:
    import chunked_kl_loss_amd as kd

    dev = W.device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    H = torch.randn(N, D, generator=g, device=dev).to(torch.bfloat16)
    lg = (torch.randn(N, K, generator=g, device=dev) * 2.0 ** 0.5).sort(dim=1, descending=True).values
    ids = torch.randint(0, V, (N, K), generator=g, device=dev, dtype=torch.int32)
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    loss, row_lse, row_kl = kd.kdkl_forward(H, W, ids, lg, T, CHUNK)
    dH, dW = kd.kdkl_backward(H, W, ids, lg, T, CHUNK, row_lse)
    torch.cuda.synchronize(dev)
    peak = torch.cuda.max_memory_allocated(dev)
    assert torch.isfinite(loss).item()
    del H, lg, ids, loss, row_lse, row_kl, dH, dW
    torch.cuda.empty_cache()
    return peak


def test_peak_memory_linear_in_positions():
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    W = (torch.randn(V, D, generator=g, device=dev) * D ** -0.5).to(torch.bfloat16)
    Ns = [32768, 65536, 131072, 262144]
    peaks = []
    for i, N in enumerate(Ns):
        print(f"peak memory case N={N}", flush=True)
        peaks.append(_peak_bytes(N, W, 100 + i))
    x = np.array(Ns, dtype=np.float64)
    y = np.array(peaks, dtype=np.float64)
    b, a = np.polyfit(x, y, 1)
    r2 = 1.0 - ((y - (a + b * x)) ** 2).sum() / ((y - y.mean()) ** 2).sum()
    print(f"peaks GiB {[round(p / 2**30, 3) for p in peaks]} slope {b:.1f} B/position "
          f"(per-position tensors {PER_POSITION}) intercept {a / 2**30:.3f} GiB r2 {r2:.6f}", flush=True)
    assert r2 > 0.999
    assert abs(b - PER_POSITION) <= 0.1 * PER_POSITION
