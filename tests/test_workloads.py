"""Seeded synthetic inputs: shapes, ranges, distinctness, sortedness,
determinism, and the sizes the pages fix."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def test_page_figures_fix_the_workload_sizes():
    g = json.load(open(GOLDEN))
    assert wl.CONFIGS["gptoss20b_32k"].V == g["gpt_oss_vocab"]["value"]
    assert wl.CONFIGS["longctx_256k"].V == g["gpt_oss_vocab"]["value"]
    for name in ("small_bf16", "llama3b_8k", "gptoss20b_32k", "longctx_256k"):
        assert wl.CONFIGS[name].K == g["teacher_topk_cached"]["value"]
    t = g["teacher_tensor_example"]
    nbytes = t["batch"] * t["vocab"] * t["seq"] * t["bytes_per_elem"]
    assert abs(nbytes / 1e9 - t["approx_GB"]) / t["approx_GB"] < 0.1


@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16"])
def test_generated_inputs_are_valid(name):
    w = wl.get_config(name)
    x = wl.generate(w)
    assert x["H"].shape == (w.N, w.d) and x["H"].dtype == w.torch_dtype
    assert x["W"].shape == (w.V, w.d) and x["W"].dtype == w.torch_dtype
    ids = x["ids"].numpy()
    assert ids.shape == (w.N, w.K) and ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < w.V
    s = np.sort(ids, axis=1)
    assert np.all(s[:, 1:] != s[:, :-1]), "ids must be distinct per row"
    lg = x["logits"].numpy()
    assert lg.dtype == np.float32 and np.all(lg[:, 1:] <= lg[:, :-1])
    # variance of the logits and of W rows
    assert abs(lg.var() / w.logit_var - 1) < 0.1
    wv = x["W"].float().var().item() * w.d
    assert abs(wv - 1) < 0.05


def test_determinism_and_seed():
    w = wl.get_config("C1")
    a = wl.generate(w)
    b = wl.generate(w)
    for k in a:
        assert torch.equal(a[k], b[k])
    c = wl.generate(w, seed=5)
    assert not torch.equal(a["H"], c["H"])


def test_zipf_rank_frequencies():
    # first-draw frequency of id 0 under Zipf(1.1) over V ids is 1 / H_{V,1.1}
    w = wl.get_config("small_bf16")
    x = wl.generate(w, N=4000)
    ids = x["ids"].numpy()
    r = np.arange(1, w.V + 1, dtype=np.float64) ** -1.1
    p0 = 1.0 / r.sum()
    first = np.mean(ids[:, 0] == 0)
    assert abs(first - p0) < 4 * np.sqrt(p0 * (1 - p0) / ids.shape[0])
    # id 0 is present in nearly every row (100 distinct draws)
    assert np.mean((ids == 0).any(axis=1)) > 0.99


def test_uniform_ids_cover_vocab():
    w = wl.get_config("tiny_fp32")
    ids = wl.generate(w, N=2000)["ids"].numpy().ravel()
    h = np.bincount(ids, minlength=w.V)
    expect = ids.size / w.V
    assert abs(h.mean() - expect) < 1e-9
    assert h.std() < 3 * np.sqrt(expect)
