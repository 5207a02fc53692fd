"""GPU test of the optional teacher-id validation (kdkl_check_ids) against
counts taken with numpy on planted cases: ids outside [0, V) and repeated
ids in kept positions are counted; ignored positions (first id -1) are not,
whatever the rest of their row holds."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _reference(ids: np.ndarray, V: int):
    kept = ids[:, 0] != -1
    k = ids[kept]
    bad = int(((k < 0) | (k >= V)).sum())
    dup = int(sum(len(np.unique(r)) < len(r) for r in k))
    return bad, dup


def _distinct_rows(rng, N, K, V):
    return np.stack([rng.choice(V, size=K, replace=False) for _ in range(N)]).astype(np.int32)


@pytest.mark.parametrize("N,K,V", [(3000, 100, 50000), (257, 1, 7), (40, 1024, 5000), (1, 3, 3)])
def test_check_ids_counts(N, K, V):
    import chunked_kl_loss_amd as kd

    print(f"case check_ids N={N} K={K} V={V}", flush=True)
    rng = np.random.default_rng(N + K)
    ids = _distinct_rows(rng, N, K, V)
    assert kd.check_ids(torch.from_numpy(ids).to(DEV), V) == (0, 0)
    rows = rng.choice(N, size=max(1, N // 7), replace=False)
    for i, r in enumerate(rows):
        kind = i % 4
        if kind == 0:
            ids[r, rng.integers(K)] = [V, V + 7, -3, 2 ** 31 - 1][i % 4 if K > 1 else 0]
        elif kind == 1 and K > 1:
            ids[r, K - 1] = ids[r, 0]          # a repeated id
        elif kind == 2 and K > 1:
            ids[r, 1] = -1                     # -1 after the first position is out of range
        else:
            ids[r, 0] = -1                     # ignored position, garbage after it
            ids[r, 1:] = V + 1
    got = kd.check_ids(torch.from_numpy(ids).to(DEV), V)
    ref = _reference(ids, V)
    print(f"counts {got} reference {ref}", flush=True)
    assert got == ref


def test_check_ids_empty():
    import chunked_kl_loss_amd as kd

    print("case check_ids N=0", flush=True)
    assert kd.check_ids(torch.empty(0, 5, dtype=torch.int32, device=DEV), 10) == (0, 0)
