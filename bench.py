"""Benchmark of the fused CE + TVD loss on one MI355X.

One step = the whole hot path over one batch already resident in HBM: the
per-row forward outputs (lse_s, lse_t, ce, tvd, sigma), the mean of ce and tvd
over the valid rows, and the gradient of mean ce + mean tvd w.r.t. the student
logits.  Two paths compute that step and both are timed:
  fused    : count valid rows (1/n_valid on the device) -> one forward+backward
             pass over the logits -> mean (the headline when a teacher is given);
  separate : forward -> mean (and 1/n_valid) -> backward.
The headline workload is the training batch: 8192 rows x 151936 classes, bf16
logits, LM-like synthetic logits (N(0, 1.5^2) plus 32 N(8, 2^2) spikes per row,
independent teacher).  The other workloads (pr: 1024 rows, the PR page's own
shape; ties: 16384 rows with identical / uniform / ignored rows; hugev: 64 x
262144) and CE-only mode get lines of their own under "configs".

Timing: every timed rep is preceded, outside the timed region, by a 1 GiB
write that flushes the L2 caches and the Infinity Cache, and is bracketed by
HIP events on the stream the kernels run on; ms_per_step is the mean over the
timed reps.  The practical ceilings are the library's own reference streams
(read-only, and two reads + one write), measured the same way.  Prints one
JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]
                    [--no-linear] [--no-vocab-parallel] [--no-ex] [--no-ceiling]
    python bench.py --only-linear [--steps K] [--warmup W]    (the lm_head leg alone)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "fwd+bwd tokens/s and achieved HBM GB/s (% of peak), BT=8192 V=151936 bf16"
FLUSH_BYTES = 1 << 30
# sources of the kernels whose HBM counters are committed (profiles/pmc_traffic.json)
KERNEL_SOURCES = ["common.hpp", "ids.hpp", "launch.hpp", "forward.hip", "forward_cluster.hip", "backward.hip"]
II = -100


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "cross_entropy_tv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- timing

class Timer:
    """Per-rep HIP-event timing of a sequence of calls, with a cache flush before
    every rep (outside the timed region)."""

    def __init__(self, dev):
        import torch
        self.torch = torch
        self.flush_buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)

    def flush(self):
        self.flush_buf.add_(1)

    def run(self, calls, steps, warmup):
        """calls: list of zero-argument callables forming one step.  Returns
        (mean ms of each call, mean ms of the step, wall seconds of the timed loop)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            self.flush()
            for c in calls:
                c()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
        t0 = time.perf_counter()
        for k in range(steps):
            self.flush()
            for i, c in enumerate(calls):
                evs[k][i].record(stream)
                c()
            evs[k][-1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i in range(len(calls))]
        step = sum(e[0].elapsed_time(e[-1]) for e in evs) / steps
        return per, step, wall


def roofline(alg_bytes, ms, kernel):
    gbs = alg_bytes / ms / 1e6
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": kernel, "alg_bytes_per_launch": int(alg_bytes),
            "avg_launch_ms": round(ms, 4)}


def algorithmic_bytes(BT, V, es, n_valid, teacher):
    """Unique bytes each kernel must move: logits read once per pass that needs
    them, the gradient written once, plus the per-row state (see the design notes)."""
    n_ign = BT - n_valid
    streams = 2 if teacher else 1
    fwd = n_valid * streams * V * es + BT * 8 + BT * 4 * (5 if teacher else 2)
    bwd = n_valid * (streams + 1) * V * es + n_ign * V * es + BT * 8 + BT * 4 * (3 if teacher else 1) + 4
    red = BT * (4 * (2 if teacher else 1) + 8) + 16
    fused = n_valid * (streams + 1) * V * es + n_ign * V * es + BT * 8 + BT * 4 * (5 if teacher else 2) + 4
    return {"forward": fwd, "reduce": red, "backward": bwd, "forward_backward": fused}


# ---------------------------------------------------------------- the two paths

def measure(timer, w, zs, us, tg, n_valid, steps, warmup, teacher):
    """Both paths on one device-resident batch; returns their timings and rooflines."""
    import torch
    import cross_entropy_tv_amd as lx

    BT, V = w.BT, w.V
    dev = zs.device
    f = lambda: torch.empty(BT, dtype=torch.float32, device=dev)  # noqa: E731
    ce, lse_s = f(), f()
    tvd, lse_t, sigma = (f(), f(), f()) if teacher else (None, None, None)
    u = us if teacher else None
    mean = torch.empty(2, dtype=torch.float32, device=dev)
    inv = torch.empty(1, dtype=torch.float32, device=dev)
    grad = torch.empty_like(zs)
    dt = lx.LX_BF16 if w.dtype == "bf16" else lx.LX_F32
    nws = max(lx.lx_ce_tvd_workspace_bytes(BT, V, dt, teacher),
              lx.lx_ce_tvd_forward_backward_workspace_bytes(BT, V, dt, teacher))
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream()
    ab = algorithmic_bytes(BT, V, w.esize, n_valid, teacher)

    sep_calls = [lambda: lx.lx_ce_tvd_forward(zs, u, tg, II, ce, tvd, lse_s, lse_t, sigma, ws, s),
                 lambda: lx.lx_ce_tvd_reduce_mean(ce, tvd, tg, II, mean, None, inv, s),
                 lambda: lx.lx_ce_tvd_backward(grad, zs, u, tg, II, lse_s, lse_t, sigma, 1.0, 1.0, inv, s)]
    (fwd_ms, red_ms, bwd_ms), sep_ms, _ = timer.run(sep_calls, steps, warmup)
    sep_mean = mean.cpu().tolist()
    one_calls = [lambda: lx.lx_ce_tvd_count_valid(tg, II, None, inv, s),
                 lambda: lx.lx_ce_tvd_forward_backward(zs, u, tg, II, ce, tvd, lse_s, lse_t, sigma, grad, 1.0, 1.0,
                                                       inv, ws, s),
                 lambda: lx.lx_ce_tvd_reduce_mean(ce, tvd, tg, II, mean, None, None, s)]
    (cnt_ms, fb_ms, red2_ms), one_ms, wall = timer.run(one_calls, steps, warmup)
    del grad, ws
    r = lambda x: round(x, 4)  # noqa: E731
    return {
        "workload": f"{w.name} {BT}x{V} {w.dtype}", "mode": "ce_tvd" if teacher else "ce_only",
        "n_valid_rows": n_valid,
        "one_pass": {"ms_per_step": r(one_ms), "tokens_per_s": round(BT / one_ms * 1e3, 1), "count_ms": r(cnt_ms),
                     "forward_backward_ms": r(fb_ms), "reduce_ms": r(red2_ms),
                     "roofline": roofline(ab["forward_backward"], fb_ms, "forward_backward"),
                     "mean": mean.cpu().tolist(), "wall_s_timed_loop": round(wall, 4)},
        "separate": {"ms_per_step": r(sep_ms), "tokens_per_s": round(BT / sep_ms * 1e3, 1), "forward_ms": r(fwd_ms),
                     "reduce_ms": r(red_ms), "backward_ms": r(bwd_ms),
                     "forward_roofline": roofline(ab["forward"], fwd_ms, "forward"),
                     "backward_roofline": roofline(ab["backward"], bwd_ms, "backward"), "mean": sep_mean},
    }


def run_vocab_parallel(timer, w, zs, us, tg, n_valid, steps, warmup, n_shards=8):
    """The per-device passes of an n_shards-way vocabulary-parallel layout at its real
    shape: one device's column shard (BT, V / n_shards) of the same logits.  One step =
    step-1 partials -> merge of the n_shards gathered partials -> step-2 partials ->
    merge -> backward of the shard (the exchanges between devices are not run here)."""
    import torch
    import cross_entropy_tv_amd as lx

    BT, V = w.BT, w.V
    Vs = V // n_shards
    dev = zs.device
    zsh, ush = zs[:, :Vs].contiguous(), us[:, :Vs].contiguous()
    stats = torch.empty((n_shards, BT, 5), dtype=torch.float32, device=dev)
    tv = torch.empty((n_shards, BT, 2), dtype=torch.float32, device=dev)
    f = lambda: torch.empty(BT, dtype=torch.float32, device=dev)  # noqa: E731
    ce, lse_s, lse_t, tvd, sigma = f(), f(), f(), f(), f()
    inv = torch.empty(1, dtype=torch.float32, device=dev)
    grad = torch.empty_like(zsh)
    s = torch.cuda.current_stream()
    lx.lx_ce_tvd_count_valid(tg, II, None, inv, s)
    for n in range(n_shards):  # stand-ins for the other devices' partials
        lx.lx_ce_tvd_vp_stats(zsh, ush, tg, 0, II, stats[n], s)
    lx.lx_ce_tvd_vp_merge_stats(stats, tg, V, II, ce, lse_s, lse_t, s)
    for n in range(n_shards):
        lx.lx_ce_tvd_vp_tv(zsh, ush, tg, II, lse_s, lse_t, tv[n], s)
    calls = [lambda: lx.lx_ce_tvd_vp_stats(zsh, ush, tg, 0, II, stats[0], s),
             lambda: lx.lx_ce_tvd_vp_merge_stats(stats, tg, V, II, ce, lse_s, lse_t, s),
             lambda: lx.lx_ce_tvd_vp_tv(zsh, ush, tg, II, lse_s, lse_t, tv[0], s),
             lambda: lx.lx_ce_tvd_vp_merge_tv(tv, tg, II, tvd, sigma, s),
             lambda: lx.lx_ce_tvd_backward_shard(grad, zsh, ush, tg, 0, V, II, lse_s, lse_t, sigma, 1.0, 1.0, inv, s)]
    ms, step_ms, _ = timer.run(calls, steps, warmup)
    n_ign = BT - n_valid
    es = w.esize
    alg = {"stats": n_valid * 2 * Vs * es + BT * 8 + BT * 20,
           "merge_stats": BT * (8 + n_shards * 20 + 12),
           "tv": n_valid * 2 * Vs * es + BT * (8 + 8 + 8),
           "merge_tv": BT * (8 + n_shards * 8 + 8),
           "backward": n_valid * 3 * Vs * es + n_ign * Vs * es + BT * (8 + 12) + 4}
    out = {"shard": f"{BT}x{Vs} {w.dtype} (1 of {n_shards} column shards)"}
    for (name, b), t in zip(alg.items(), ms):
        out[f"{name}_ms"] = round(t, 4)
        out[f"{name}_GBs"] = round(b / t / 1e6, 1)
        if name in ("stats", "tv", "backward"):
            out[f"{name}_pct_peak"] = round(100.0 * b / t / 1e6 / HBM_PEAK_GBS, 2)
    out["device_step_ms"] = round(step_ms, 4)
    return out


def run_ex(timer, w, zs, us, tg, n_valid, steps, warmup, pad=128):
    """The one-pass forward + backward of the ABI-breadth entry points on the same batch:
    binary16 copies of the logits; the logits inside arrays padded to V + pad columns
    (row strides, e.g. a vocabulary rounded up to a multiple of 256); per-row upstream
    gradients (an unreduced loss).  Each is timed alone, with its algorithmic bytes
    those of the one pass (read student and teacher once, write the gradient once)."""
    import torch
    import cross_entropy_tv_amd as lx

    BT, V = w.BT, w.V
    dev = zs.device
    f = lambda: torch.empty(BT, dtype=torch.float32, device=dev)  # noqa: E731
    ce, lse_s, tvd, lse_t, sigma = f(), f(), f(), f(), f()
    s = torch.cuda.current_stream()
    alg = algorithmic_bytes(BT, V, w.esize, n_valid, True)["forward_backward"]
    inv = torch.empty(1, dtype=torch.float32, device=dev)
    lx.lx_ce_tvd_count_valid(tg, II, None, inv, s)
    nws = lx.lx_ce_tvd_forward_backward_workspace_bytes(BT, V, lx.LX_BF16, True)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    out = {}

    def record(name, fn, extra=None):
        (ms,), _, _ = timer.run([fn], steps, warmup)
        out[name] = {"ms": round(ms, 4), "GBs": round(alg / ms / 1e6, 1),
                     "pct_peak": round(100.0 * alg / ms / 1e6 / HBM_PEAK_GBS, 2), **(extra or {})}

    g = torch.empty_like(zs)
    plain = lambda: lx.lx_ce_tvd_forward_backward(zs, us, tg, II, ce, tvd, lse_s, lse_t, sigma, g, 1.0, 1.0, inv,  # noqa: E731
                                                   ws, s)
    record("reference", plain)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261202)
    wce = torch.rand(BT, generator=gen, device=dev) + 0.5
    wtv = torch.rand(BT, generator=gen, device=dev) + 0.5
    record("row_factors", lambda: lx.lx_ce_tvd_forward_backward_ex(
        zs, us, tg, II, ce, tvd, lse_s, lse_t, sigma, g, 1.0, 1.0, wce, wtv, inv, ws, s))
    z16, u16 = zs.to(torch.float16), us.to(torch.float16)
    g16 = torch.empty_like(z16)
    record("f16", lambda: lx.lx_ce_tvd_forward_backward(z16, u16, tg, II, ce, tvd, lse_s, lse_t, sigma, g16, 1.0, 1.0,
                                                        inv, ws, s), {"logits": "f16"})
    del z16, u16, g16
    zbig = torch.empty((BT, V + pad), dtype=zs.dtype, device=dev)
    ubig = torch.empty((BT, V + pad), dtype=us.dtype, device=dev)
    zbig[:, :V] = zs
    ubig[:, :V] = us
    zv, uv = zbig[:, :V], ubig[:, :V]
    gbig = torch.empty_like(zbig)
    gv = gbig[:, :V]
    record("strided", lambda: lx.lx_ce_tvd_forward_backward_ex(
        zv, uv, tg, II, ce, tvd, lse_s, lse_t, sigma, gv, 1.0, 1.0, g_scale=inv, workspace=ws, stream=s),
        {"row_stride": V + pad})
    del zbig, ubig, gbig
    return out


def run_linear(timer, steps, warmup, BT=8192, V=151936, H=4096, chunk_rows=8192, vendor_reference=True):
    """The lm_head products + CE + TVD in one call (student and teacher lm_heads of
    hidden size H over the vocabulary, seeded synthetic hidden states and weights),
    timed with HIP events; FLOP/s against the dense bf16 matrix-core peak."""
    import numpy as np
    import torch
    import cross_entropy_tv_amd as lx
    import workloads as W

    dev = torch.device("cuda:0")
    x_s, w_s, x_t, w_t, t = W.linear_inputs(BT, V, H, H, seed=77)

    def d(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    X, Wd, Xt, Wt, tg = d(x_s), d(w_s), d(x_t), d(w_t), torch.from_numpy(t).to(dev)
    del x_s, w_s, x_t, w_t
    f = lambda: torch.empty(BT, dtype=torch.float32, device=dev)  # noqa: E731
    ce, tvd, lse_s, lse_t, sigma = f(), f(), f(), f(), f()
    gx = torch.empty((BT, H), dtype=torch.float32, device=dev)
    gw = torch.empty((V, H), dtype=torch.float32, device=dev)
    inv = torch.empty(1, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()
    lx.lx_ce_tvd_count_valid(tg, II, None, inv, s)
    wsb = lx.lx_ce_tvd_linear_workspace_bytes(BT, V, H, True, chunk_rows)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    (ms,), _, _ = timer.run([lambda: lx.lx_ce_tvd_linear_forward_backward(
        X, Wd, Xt, Wt, tg, II, ce, tvd, lse_s, lse_t, sigma, gx, gw, 1.0, 1.0, inv, chunk_rows, ws, s)],
        max(3, steps // 4), max(1, warmup // 2))
    flops = 2.0 * BT * V * H * 4  # student and teacher logits, grad of x, grad of w
    # the kernels run 6 products of that size: each of the two loss passes recomputes
    # the logits of both heads, since no logit is stored
    flops_run = 2.0 * BT * V * H * 6
    out = {"shape": f"BT={BT} V={V} H_s=H_t={H} chunk_rows={chunk_rows}", "workspace_bytes": int(wsb),
           "workspace_bytes_per_chunk_logit": round(wsb / (min(chunk_rows, BT) * V), 2),
           "ms": round(ms, 3), "tokens_per_s": round(BT / ms * 1e3, 1), "TFLOPs": round(flops / ms / 1e9, 1),
           "pct_mfma_peak": round(100.0 * flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
           "TFLOPs_executed": round(flops_run / ms / 1e9, 1),
           "pct_mfma_peak_executed": round(100.0 * flops_run / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2)}
    del ws, gx, gw
    if vendor_reference:
        # the vendor library's product at the logits shape, same operands, as a reference
        # for the library's own product kernel (context only: nothing above uses it)
        C = torch.empty((BT, V), dtype=torch.bfloat16, device=dev)
        (vm,), _, _ = timer.run([lambda: torch.matmul(X, Wd.t(), out=C)], max(3, steps // 4), max(1, warmup // 2))
        out["vendor_logits_product_ms"] = round(vm, 3)
        out["vendor_logits_product_pct_mfma_peak"] = round(
            100.0 * 2.0 * BT * V * H / vm / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2)
        del C
    return out


def stream_ceilings(timer, dev, steps, warmup, nbytes=2 << 30):
    """Achieved GB/s of the library's reference streams: read-only over 2 * nbytes,
    and two reads + one write of nbytes each (3 * nbytes moved)."""
    import torch
    import cross_entropy_tv_amd as lx

    a = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.full((nbytes // 4,), 3, dtype=torch.int32, device=dev)
    o = torch.empty_like(a)
    big = torch.cat([a, b])
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    (rd,), _, _ = timer.run([lambda: lx.lx_stream_read(big, sink, s)], steps, warmup)
    (rw,), _, _ = timer.run([lambda: lx.lx_stream_read2_write(a, b, o, s)], steps, warmup)
    del a, b, o, big
    return {"read_GBs": round(2 * nbytes / rd / 1e6, 1), "read2_write_GBs": round(3 * nbytes / rw / 1e6, 1),
            "read_bytes": 2 * nbytes, "read2_write_bytes": 3 * nbytes}


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters,
    if they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = d.get("kernels", {}).get(kernel_key)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- CPU baseline (the oracle as it stands)

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, seconds_per_worker=1.5, batch=4, workers=None, one_core_seconds=6.0):
    """The float64 oracle, as it stands, timed on the host cores over a bounded sample of
    the same workload's rows (forward + backward per row).  Each worker process takes
    its own rows in batches and stops once its timed oracle work passes
    ``seconds_per_worker``; the rate is the sum of the workers' rates (they run
    concurrently).  A single process alone gives the 1-core figure."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    workers = workers or min(cores, 16)
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        res = pool.map(_cpu_worker, [(w.name, i, workers, batch, seconds_per_worker) for i in range(workers)])
    with ctx.Pool(1) as pool:
        one = pool.map(_cpu_worker, [(w.name, 0, 1, batch, one_core_seconds)])[0]
    rate = sum(r[0] / r[1] for r in res)
    nrows = sum(r[0] for r in res)
    cpu_s = sum(r[1] for r in res)
    return {"value": round(rate, 1), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "one_core_value": round(one[0] / one[1], 1), "cpu_model": cpu_model(), "host_cores_available": cores,
            "sample": f"{nrows} rows of the {w.name} workload ({w.BT}x{w.V} {w.dtype}), float64 numpy oracle "
                      f"forward+backward per row, {workers} single-threaded processes, {cpu_s:.1f} s of timed "
                      f"CPU work in total; 1-core figure: {one[0]} rows in {one[1]:.1f} s in one process"}


def _cpu_worker(arg):
    name, wid, nworkers, batch, budget = arg
    os.environ["OMP_NUM_THREADS"] = "1"
    import oracle
    import workloads as W
    w = W.get(name)
    tg = W.targets(w)
    done, spent, k = 0, 0.0, 0
    while spent < budget and done < 256:
        rows = [(wid + nworkers * (k * batch + j)) % w.BT for j in range(batch)]
        k += 1
        z, u = W.rows(w, rows)
        t = tg[rows]
        t0 = time.perf_counter()
        oracle.forward(z, u, t, W.IGNORE_INDEX)
        oracle.backward(z, u, t, W.IGNORE_INDEX, 1.0 / w.BT, 1.0 / w.BT)
        spent += time.perf_counter() - t0
        done += len(rows)
    return done, spent


# ---------------------------------------------------------------- main

def load_workload(name, dev):
    import numpy as np
    import torch
    import workloads as W

    w = W.get(name)
    t0 = time.perf_counter()
    z, u, t = W.full(w)
    print(f"[bench] generated {w.name} {w.BT}x{w.V} {w.dtype} in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)

    def dev_copy(raw):
        if raw.dtype == np.uint16:
            return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(raw).to(dev)

    zs, us, tg = dev_copy(z), dev_copy(u), dev_copy(t)
    return w, zs, us, tg, int((t != W.IGNORE_INDEX).sum())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload lines other than train")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-vocab-parallel", action="store_true")
    ap.add_argument("--no-ex", action="store_true", help="skip the binary16 / strided / per-row one-pass legs")
    ap.add_argument("--no-linear", action="store_true", help="skip the lm_head product + loss leg")
    ap.add_argument("--only-linear", action="store_true",
                    help="run only the lm_head product + loss leg and print its JSON object (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (rows shard across GPUs "
              "with no exchange except a 3-scalar loss reduction, which this single-GPU build does not run)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import cross_entropy_tv_amd as lx  # noqa: F401  (fails loudly if the HIP library is missing)

    dev = torch.device("cuda:0")
    timer = Timer(dev)
    K, Wm = args.steps, args.warmup
    if args.only_linear:
        print(json.dumps({"linear": run_linear(timer, K, Wm)}), flush=True)
        return
    w, zs, us, tg, n_valid = load_workload("train", dev)
    head = measure(timer, w, zs, us, tg, n_valid, K, Wm, True)
    print(f"[bench] train ce_tvd: one pass {head['one_pass']['ms_per_step']:.4f} ms/step, separate "
          f"{head['separate']['ms_per_step']:.4f}", file=sys.stderr, flush=True)
    extra = {"configs": {}}
    extra["configs"]["train_ce_only"] = measure(timer, w, zs, us, tg, n_valid, K, Wm, False)
    if not args.no_vocab_parallel:
        extra["vocab_parallel"] = run_vocab_parallel(timer, w, zs, us, tg, n_valid, K, Wm)
    if not args.no_ex:
        extra["one_pass_ex"] = run_ex(timer, w, zs, us, tg, n_valid, K, Wm)
    del zs, us, tg
    torch.cuda.empty_cache()
    if not args.no_configs:
        for name in ("pr", "ties", "hugev"):
            wc, zc, uc, tc, nc = load_workload(name, dev)
            extra["configs"][name] = measure(timer, wc, zc, uc, tc, nc, K, Wm, True)
            if name == "hugev":
                extra["configs"]["hugev_ce_only"] = measure(timer, wc, zc, uc, tc, nc, K, Wm, False)
            del zc, uc, tc
            torch.cuda.empty_cache()
    if not args.no_linear:
        extra["linear"] = run_linear(timer, K, Wm)
        torch.cuda.empty_cache()
        # the same call in chunks of 2048 rows: a quarter of the per-chunk workspace
        small = run_linear(timer, K, Wm, chunk_rows=2048, vendor_reference=False)
        extra["linear"]["chunk_rows_2048"] = {k: small[k] for k in ("workspace_bytes", "ms", "tokens_per_s",
                                                                   "pct_mfma_peak", "pct_mfma_peak_executed")}
        torch.cuda.empty_cache()
    if not args.no_ceiling:
        c = stream_ceilings(timer, dev, K, Wm)
        fwd = head["separate"]["forward_roofline"]["achieved"]
        fb = head["one_pass"]["roofline"]["achieved"]
        bwd = head["separate"]["backward_roofline"]["achieved"]
        c["read_ceiling_covers_forward"] = c["read_GBs"] >= fwd
        c["read2_write_ceiling_covers_one_pass_and_backward"] = c["read2_write_GBs"] >= max(fb, bwd)
        extra["ceilings"] = c

    one, sep = head["one_pass"], head["separate"]
    rl = dict(one["roofline"])
    rl["traffic"] = traffic_from_profiles("forward_backward_ce_tvd_train")
    line = {
        "metric": METRIC,
        "value": one["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": one["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "train", "BT": w.BT, "V": w.V, "logits": w.dtype, "mode": "ce_tvd",
                   "path": "one pass (count -> forward_backward -> mean)", "global_batch": w.BT,
                   "parallelism": "none (1 GPU)", "timing": "per rep, HIP events, 1 GiB cache flush before each rep"},
        "roofline": rl,
        "separate_step": {"tokens_per_s": sep["tokens_per_s"], "ms_per_step": sep["ms_per_step"]},
        "passes": {"forward_ms": sep["forward_ms"], "reduce_ms": sep["reduce_ms"], "backward_ms": sep["backward_ms"],
                   "forward_GBs": sep["forward_roofline"]["achieved"],
                   "backward_GBs": sep["backward_roofline"]["achieved"],
                   "forward_pct_peak": round(100 * sep["forward_roofline"]["frac"], 2),
                   "backward_pct_peak": round(100 * sep["backward_roofline"]["frac"], 2),
                   "one_pass_ms": one["forward_backward_ms"], "one_pass_pct_peak": round(100 * one["roofline"]["frac"], 2)},
        "mean_loss": one["mean"],
        "wall_s_timed_loop_incl_flush": one["wall_s_timed_loop"],
        **extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
