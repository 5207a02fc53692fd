#!/usr/bin/env python3
"""Benchmark of the fused chunked KL loss (forward + backward) on one MI355X.

One step = kdkl_forward + kdkl_backward over one batch of synthetic inputs
already resident in HBM (every kernel of the path). Prints ONE JSON line.

Default workload: the long-context case, the gpt-oss-20b-like head at 256K
tokens (N=262144, d=2880, V=201088, K=100, chunk=4096, bf16, T=2), the
largest single-GPU configuration; --config gptoss20b_32k times the same head
at 32K tokens (chunk 2048, T=1).

--path logits measures the forward-chunked variant instead: one step =
kdkl_logits_forward + kdkl_logits_backward on the logit grid Z = H W^T of the
same workload (computed on the device before timing, as the caller's output
layer would); that path is bound by HBM bandwidth. --path dense measures the
dense baseline (full grids kept for the backward).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused KL fwd+bwd tokens/s; MFMA util % of bf16 peak; peak HBM GiB"
# MI355X published dense peaks (TFLOP/s) by arithmetic type.
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kdkl_kernels.hip", "kdkl_logits.hip", "kdkl_jsd.hip", "kdkl_api.hip", "kdkl_internal.h"):
        with open(os.path.join(ROOT, "chunked_kl_loss_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/traffic_<kernel>_<workload>.txt, lines "key: value"),
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device copy of known size, profiled with the same rocprofv3
    counters as the kernels to scale FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch

    n = 1 << 28  # 2^28 fp32 = 1 GiB each way
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def cpu_baseline(w, x, rows: int, loss: str = "kl", beta: float = 0.5):
    """The CPU oracle, as it stands, on the first `rows` positions of the same
    workload (full vocabulary and hidden size)."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    H, ids, lg = x["H"][:rows], x["ids"][:rows], x["logits"][:rows]
    t0 = time.perf_counter()
    if loss == "trkl":
        oracle.topk_rkl_forward(H, x["W"], ids, lg, w.T)
        oracle.topk_rkl_backward(H, x["W"], ids, lg, w.T)
    elif loss != "kl":
        oracle.alt_forward(H, x["W"], ids, lg, w.T, loss, beta)
        oracle.alt_backward(H, x["W"], ids, lg, w.T, loss, beta)
    else:
        oracle.forward(H, x["W"], ids, lg, w.T)
        oracle.backward(H, x["W"], ids, lg, w.T)
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows} of {w.N} positions of {w.name} (full V={w.V}, d={w.d}); "
                      f"fp64 numpy forward+backward, {dt:.1f} s"}


def cpu_baseline_logits(w, Z_rows, x, rows: int):
    """The CPU oracle of the forward-chunked path on the first `rows` rows of
    the logit grid (full vocabulary)."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    ids, lg = x["ids"][:rows], x["logits"][:rows]
    t0 = time.perf_counter()
    oracle.logits_forward(Z_rows, ids, lg, w.T)
    oracle.logits_backward(Z_rows, ids, lg, w.T)
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows} of {w.N} rows of the {w.name} logit grid (full V={w.V}); "
                      f"fp64 numpy forward+backward, {dt:.1f} s"}


class PowerSampler:
    """Socket power and gfx clock of the device, sampled in a thread (amdsmi,
    no HIP) while the timed steps run. The sensor reports a running average
    that trails the load by about a second, so samples from the first
    `settle` seconds are dropped."""

    def __init__(self, interval=0.02, settle=1.0):
        self.interval, self.settle = interval, settle
        self.samples, self.error, self._stop, self.limit = [], None, None, None

    def _handle(self, amdsmi, dev):
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) == 1:
            return handles[0]
        props = torch.cuda.get_device_properties(dev)
        bus = getattr(props, "pci_bus_id", None)
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
            if bus is not None and int(bdf.split(":")[1], 16) == bus:
                return h
        raise RuntimeError(f"cannot match the device among {len(handles)} amdsmi handles")

    def start(self, dev):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = self._handle(amdsmi, dev)
        except Exception as e:  # no sensor access: report why, time as usual
            self.error = repr(e)
            return
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    info = amdsmi.amdsmi_get_power_info(h)
                    pw = info["current_socket_power"]
                    self.limit = info.get("power_limit")
                    clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"]
                    self.samples.append((time.time(), float(pw), float(clk)))
                except Exception as e:
                    self.error = repr(e)
                    return
                time.sleep(self.interval)

        self._t0 = time.time()
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        self._amdsmi = amdsmi

    def stop(self, ms_per_step, t_end=None):
        """Summary of the samples from `settle` seconds after start to t_end."""
        if self._stop is None:
            return {"error": self.error}
        self._stop.set()
        self._thread.join()
        self._amdsmi.amdsmi_shut_down()
        t_end = t_end if t_end is not None else time.time()
        kept = [s for s in self.samples if self._t0 + self.settle <= s[0] <= t_end]
        if not kept:
            return {"error": self.error or "no samples after the settling time (time more steps)"}
        avg_w = sum(s[1] for s in kept) / len(kept)
        return {"avg_w": round(avg_w, 1), "max_w": max(s[1] for s in kept),
                "gfx_mhz": round(sum(s[2] for s in kept) / len(kept), 1),
                "joules_per_step": round(avg_w * ms_per_step / 1e3, 2), "samples": len(kept),
                "settle_s": self.settle,
                # amdsmi reports the limit in microwatts
                "power_limit_w": (round(self.limit / 1e6, 1) if isinstance(self.limit, (int, float)) and self.limit > 1e5
                                  else self.limit)}


def kernel_table(kstats, steps):
    kernels = {}
    for name, s in kstats.items():
        kernels[name] = {
            "launches_per_step": s["launches"] / steps,
            "avg_ms": s["total_ms"] / max(1, s["launches"]),
            "ms_per_step": s["total_ms"] / steps,
            "tflops": (s["flops"] / (s["total_ms"] / 1e3) / 1e12) if s["total_ms"] > 0 else 0.0,
            "gbs": (s["bytes"] / (s["total_ms"] / 1e3) / 1e9) if s["total_ms"] > 0 else 0.0,
        }
    return kernels


def bench_logits(args, w, x):
    import torch

    import chunked_kl_loss_amd as kd

    dev = torch.device("cuda:0")
    Hd, Wd = x["H"].to(dev), x["W"].to(dev)
    Z = torch.matmul(Hd, Wd.T.contiguous())  # the output layer's logit grid [N, V]
    del Hd, Wd
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    ids, lg = x["ids"].to(dev), x["logits"].to(dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    row_lse = torch.empty(w.N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(w.N, dtype=torch.float32, device=dev)
    dZ = Z if args.inplace else torch.empty_like(Z)
    ws = torch.empty(kd.LOGITS_BWD_WORKSPACE, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        kd.logits_forward(Z, ids, lg, w.T, loss=loss, row_lse=row_lse, row_kl=row_kl, stream=stream)
        kd.logits_backward(Z, ids, lg, w.T, row_lse, None, dZ=dZ, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    log(f"bench: warmup done, loss={loss.item():.6f}")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    kd.profile_begin()
    torch.cuda.synchronize(dev)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    kstats = kd.profile_end()
    ms = ev0.elapsed_time(ev1) / args.steps
    peak_gib = torch.cuda.max_memory_allocated(dev) / 2**30
    log(f"bench: {ms:.3f} ms/step")
    dtype = "bf16" if w.dtype == "bf16" else "fp32"
    es = 2 if dtype == "bf16" else 4
    bytes_step = 3.0 * w.N * w.V * es + 2.0 * w.N * w.K * 8.0 + 12.0 * w.N
    dom = max(kstats, key=lambda k: kstats[k]["total_ms"])
    ds = kstats[dom]
    achieved = ds["bytes"] / (ds["total_ms"] / 1e3) / 1e9
    out = {
        "metric": "forward-chunked KL fwd+bwd tokens/s (student logit grid given); HBM GB/s; peak HBM GiB",
        "value": round(w.N / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; logit grid = H W^T of the workload's H and W)",
        "config": {"workload": w.name, "path": "forward-chunked (logit grid given)", "N": w.N,
                   "V": w.V, "K": w.K, "T": w.T, "dZ_in_place": bool(args.inplace),
                   "parallelism": "single GPU"},
        "hbm_gbs_step": round(bytes_step / (ms / 1e3) / 1e9, 1),
        "bytes_per_step": bytes_step,
        "peak_hbm_gib": round(peak_gib, 3),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(dom, w.name),
                     "avg_launch_ms": round(ds["total_ms"] / ds["launches"], 4),
                     "bytes_per_launch": ds["bytes"] / ds["launches"]},
        "kernels": kernel_table(kstats, args.steps),
    }
    if not args.no_cpu_baseline:
        rows = min(args.cpu_rows, w.N)
        log(f"bench: timing the CPU oracle on {rows} rows")
        out["cpu_baseline"] = cpu_baseline_logits(w, Z[:rows].cpu(), x, rows)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_dense(args, w, x):
    """The pages' dense baseline: full student and teacher grids kept for the
    backward pass (no recompute: 6 N V d flop per step)."""
    import torch

    import chunked_kl_loss_amd as kd

    dev = torch.device("cuda:0")
    torch.cuda.reset_peak_memory_stats(dev)
    H, W, ids, lg = (x[k].to(dev) for k in ("H", "W", "ids", "logits"))
    fb, sb, bb = kd.dense_sizes(w.N, w.d, w.V, w.K, H.dtype)
    saved = torch.empty(sb, dtype=torch.uint8, device=dev)
    ws_f = torch.empty(fb, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    row_lse = torch.empty(w.N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(w.N, dtype=torch.float32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty((w.V, w.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        # the forward's logit-grid workspace is released before the backward's
        # is taken, as an autograd framework would
        wf = torch.empty(fb, dtype=torch.uint8, device=dev)
        kd.dense_forward(H, W, ids, lg, w.T, saved=saved, loss=loss, row_lse=row_lse, row_kl=row_kl,
                         workspace=wf, stream=stream)
        del wf
        wb = torch.empty(bb, dtype=torch.uint8, device=dev)
        kd.dense_backward(H, W, ids, lg, w.T, saved, None, dH=dH, dW=dW, workspace=wb, stream=stream)
        del wb

    del ws_f
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    log(f"bench: warmup done, loss={loss.item():.6f}")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    kd.profile_begin()
    torch.cuda.synchronize(dev)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    kstats = kd.profile_end()
    ms = ev0.elapsed_time(ev1) / args.steps
    peak_gib = torch.cuda.max_memory_allocated(dev) / 2**30
    log(f"bench: {ms:.2f} ms/step, peak {peak_gib:.2f} GiB")
    dtype = "bf16" if w.dtype == "bf16" else "fp32"
    flops_step = 6.0 * w.N * w.V * w.d
    peak = PEAK_TFLOPS[dtype]
    dom = max(kstats, key=lambda k: kstats[k]["total_ms"])
    ds = kstats[dom]
    t = ds["total_ms"] / 1e3
    if ds["flops"] > 0:
        roof = {"bound": "mfma", "achieved": round(ds["flops"] / t / 1e12, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ds["flops"] / t / 1e12 / peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(ds["bytes"] / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ds["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4)}
    roof.update({"kernel": dom, "traffic": load_traffic(dom, w.name),
                 "avg_launch_ms": round(ds["total_ms"] / ds["launches"], 4)})
    out = {
        "metric": "dense KL (full grids) fwd+bwd tokens/s; MFMA util % of bf16 peak; peak HBM GiB",
        "value": round(w.N / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": w.name, "path": "dense (full grids kept)", "N": w.N, "d": w.d, "V": w.V,
                   "K": w.K, "T": w.T, "parallelism": "single GPU"},
        "mfma_util_pct": round(100.0 * flops_step / (ms / 1e3) / (peak * 1e12), 2),
        "flop_per_step": flops_step,
        "peak_hbm_gib": round(peak_gib, 3),
        "saved_grids_gib": round(sb / 2**30, 3),
        "roofline": roof,
        "kernels": kernel_table(kstats, args.steps),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="longctx_256k")
    ap.add_argument("--N", type=int, default=None, help="override the number of positions")
    ap.add_argument("--chunk", type=int, default=None, help="override the chunk size")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=("fused", "logits", "dense"), default="fused",
                    help="fused: the fused chunked loss (default); logits: the forward-chunked "
                         "loss on a given logit grid; dense: the dense baseline (full grids)")
    ap.add_argument("--inplace", action="store_true",
                    help="logits path: write dZ over the logit grid")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the synthetic inputs (default: the workload's own, 1000 + its number)")
    ap.add_argument("--gen-reading", choices=("1based", "0based"), default="1based",
                    help="reading of the workload list's cross-references for the teacher "
                         "generator of the 8K and 256K workloads (1based: uniform ids, N(0, 2))")
    ap.add_argument("--loss", choices=("kl", "jsd", "skl", "srkl", "trkl"), default="kl",
                    help="kl: the pages' forward KL (default); jsd: the generalised Jensen-Shannon "
                         "divergence; skl / srkl: the skew KL / skew reverse KL; trkl: the reverse KL "
                         "over the teacher's top-K support (kdkl_options.loss)")
    ap.add_argument("--beta", type=float, default=0.5, help="the JSD's weight beta")
    ap.add_argument("--alpha", type=float, default=0.1, help="the skew losses' alpha")
    ap.add_argument("--chunks-per-group", type=int, default=0,
                    help="kdkl_options.chunks_per_group (0: the library's choice)")
    ap.add_argument("--vocab-slices", type=int, default=0,
                    help="kdkl_options.vocab_slices (0: as many as chunks per group)")
    ap.add_argument("--dh-w-in-place", type=int, default=0, choices=(0, 1, 2),
                    help="kdkl_options.dh_w_in_place (0: the library's choice, 1: in place, 2: W^T copy)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured into a HIP graph")
    ap.add_argument("--no-power", action="store_true",
                    help="do not sample socket power and the gfx clock (amdsmi) over the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is described, not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import chunked_kl_loss_amd as kd
    import workloads as wl

    w = wl.get_config(args.config)
    if args.N is not None:
        w = w.with_(N=args.N)
    if args.chunk is not None:
        w = w.with_(chunk=args.chunk)
    if args.gen_reading == "0based":
        w = wl.other_reading(w)
    dev = torch.device("cuda:0")
    log(f"bench: generating {w.name} N={w.N} d={w.d} V={w.V} K={w.K} chunk={w.chunk} T={w.T}")
    t0 = time.time()
    x = wl.generate(w, seed=args.seed)
    log(f"bench: inputs generated in {time.time() - t0:.1f} s")
    torch.cuda.set_device(dev)
    if args.path == "logits":
        torch.zeros(1, device=dev)
        bench_logits(args, w, x)
        return
    if args.path == "dense":
        torch.zeros(1, device=dev)
        bench_dense(args, w, x)
        return
    torch.zeros(1, device=dev)  # initialise the device before reading memory stats
    torch.cuda.reset_peak_memory_stats(dev)
    H, W, ids, lg = (x[k].to(dev) for k in ("H", "W", "ids", "logits"))
    opts = {"chunks_per_group": args.chunks_per_group, "vocab_slices": args.vocab_slices,
            "dh_w_in_place": args.dh_w_in_place}
    loss_param = args.beta if args.loss == "jsd" else args.alpha
    if args.loss != "kl":
        codes = {"jsd": kd.KDKL_LOSS_JSD, "skl": kd.KDKL_LOSS_SKL, "srkl": kd.KDKL_LOSS_SRKL,
                 "trkl": kd.KDKL_LOSS_TRKL}
        opts.update(loss=codes[args.loss], beta=loss_param)
    plan = kd.plan_info(w.N, w.d, w.V, w.K, w.chunk, H.dtype, opts)
    log(f"bench: plan {plan}")
    fb, bb = kd.workspace_size(w.N, w.d, w.V, w.K, w.chunk, H.dtype, opts)
    ws_f = torch.empty(fb, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bb, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    row_lse = torch.empty(kd.saved_shape(w.N, opts), dtype=torch.float32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty((w.V, w.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        kd.kdkl_forward(H, W, ids, lg, w.T, w.chunk, loss=loss, row_lse=row_lse,
                        workspace=ws_f, stream=stream, want_row_kl=False, options=opts)
        kd.kdkl_backward(H, W, ids, lg, w.T, w.chunk, row_lse, None, dH=dH, dW=dW,
                         workspace=ws_b, stream=stream, options=opts)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    log(f"bench: warmup done, loss={loss.item():.6f}")

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    sampler = None if args.no_power else PowerSampler()
    samples_end = None
    if args.graph:
        # one step captured into a HIP graph and replayed (the library
        # launches only its own kernels on the given stream, no memset
        # nodes); the per-kernel table comes from eager steps afterwards
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        stream = side
        with torch.cuda.graph(graph, stream=side):
            step()
        torch.cuda.synchronize(dev)
        stream = torch.cuda.current_stream(dev)  # replay() runs on the current stream
        graph.replay()
        torch.cuda.synchronize(dev)
        if sampler:
            sampler.start(dev)
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize(dev)
        samples_end = time.time()
        kd.profile_begin()
        for _ in range(min(args.steps, 3)):
            step()
        torch.cuda.synchronize(dev)
        kstats = kd.profile_end()
        ksteps = min(args.steps, 3)
    else:
        kd.profile_begin()
        torch.cuda.synchronize(dev)
        if sampler:
            sampler.start(dev)
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize(dev)
        samples_end = time.time()
        kstats = kd.profile_end()
        ksteps = args.steps
    ms = ev0.elapsed_time(ev1) / args.steps
    power = sampler.stop(ms, samples_end) if sampler else None
    peak_gib = torch.cuda.max_memory_allocated(dev) / 2**30
    log(f"bench: {ms:.2f} ms/step")

    dtype = "bf16" if w.dtype == "bf16" else "fp32"
    # the matrix work of a step: four vocabulary-wide products (forward,
    # recompute, dH, dW); the reverse KL over the top-K support has none, only
    # its support's dot products (forward and backward), dH and dW over the
    # support (2 N K d flop each, on the vector units)
    trkl = args.loss == "trkl"
    flops_step = 8.0 * w.N * w.K * w.d if trkl else 8.0 * w.N * w.V * w.d
    peak = PEAK_TFLOPS[dtype]
    tok_s = w.N / (ms / 1e3)
    mfma_pct = 100.0 * flops_step / (ms / 1e3) / (peak * 1e12)

    kernels = kernel_table(kstats, ksteps)
    dom = max(kstats, key=lambda k: kstats[k]["total_ms"])
    ds = kstats[dom]
    achieved = ds["flops"] / (ds["total_ms"] / 1e3) / 1e12
    traffic = load_traffic(dom, w.name)
    if trkl:  # gathers of W and H rows: bound by HBM
        achieved_gbs = ds["bytes"] / (ds["total_ms"] / 1e3) / 1e9
        if dom == "topk_rkl":  # its forward and backward launches alternate: their mean
            tf, tb = load_traffic("topk_rkl_fwd", w.name), load_traffic("topk_rkl_bwd", w.name)
            traffic = (tf + tb) / 2 if tf is not None and tb is not None else None
        else:  # (the counters cover dW's summing kernel, not the whole sort)
            traffic = None
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "avg_launch_ms": round(ds["total_ms"] / ds["launches"], 4),
                    "bytes_per_launch": ds["bytes"] / ds["launches"]}
    else:
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": traffic,
                    "avg_launch_ms": round(ds["total_ms"] / ds["launches"], 4),
                    "flop_per_launch": ds["flops"] / ds["launches"]}

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": w.name, "N": w.N, "d": w.d, "V": w.V, "K": w.K, "chunk": w.chunk,
                   "T": w.T, "teacher_ids": w.id_dist, "teacher_logit_var": w.logit_var,
                   "gen_reading": args.gen_reading,
                   "seed": args.seed if args.seed is not None else wl.seed_for(w),
                   "loss": (args.loss if args.loss in ("kl", "trkl") else
                            f"jsd(beta={args.beta})" if args.loss == "jsd" else f"{args.loss}(alpha={args.alpha})"),
                   "plan": plan,
                   "parallelism": "single GPU"},
        "mfma_util_pct": None if trkl else round(mfma_pct, 2),
        # the same time against the 6 N V d flop of forward + dH + dW alone
        # (the recompute is part of the method and counted above)
        "mfma_util_pct_without_recompute": None if trkl else round(mfma_pct * 0.75, 2),
        "flop_per_step": flops_step,
        "peak_hbm_gib": round(peak_gib, 3),
        "workspace_gib": {"forward": round(fb / 2**30, 3), "backward": round(bb / 2**30, 3)},
        "roofline": roofline,
        "kernels": kernels,
    }
    if power is not None:
        out["power"] = power
    if not args.no_cpu_baseline:
        rows = min(args.cpu_rows, w.N)
        log(f"bench: timing the CPU oracle on {rows} positions")
        out["cpu_baseline"] = cpu_baseline(w, x, rows, args.loss, loss_param)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
