"""Benchmark of the fused CE + TVD loss on one MI355X.

One step = the whole hot path over one batch already resident in HBM: the
per-row forward outputs (lse_s, lse_t, ce, tvd, sigma), the mean of ce and tvd
over the valid rows, and the gradient of mean ce + mean tvd w.r.t. the student
logits.  Two paths compute that step and both are timed:
  fused    : count valid rows (1/n_valid on the device) -> one forward+backward
             pass over the logits -> mean (the headline when a teacher is given);
  separate : forward -> mean (and 1/n_valid) -> backward.
The default workload is the training batch: 8192 rows x 151936 classes, bf16
logits, LM-like synthetic logits (N(0, 1.5^2) plus 32 N(8, 2^2) spikes per row,
independent teacher).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train]
                    [--mode ce_tvd|ce] [--no-cpu-baseline] [--no-ce-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "fwd+bwd tokens/s and achieved HBM GB/s (% of peak), BT=8192 V=151936 bf16"
# sources of the kernels whose HBM counters are committed (profiles/pmc_traffic.json)
KERNEL_SOURCES = ["common.hpp", "ids.hpp", "launch.hpp", "forward.hip", "forward_cluster.hip", "backward.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "cross_entropy_tv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(BT, V, es, n_valid, teacher):
    """Unique bytes each kernel must move (see the design notes, 'algorithmic bytes')."""
    n_ign = BT - n_valid
    streams = 2 if teacher else 1
    fwd = n_valid * streams * V * es + BT * 8 + BT * 4 * (5 if teacher else 2)
    bwd = n_valid * (streams + 1) * V * es + n_ign * V * es + BT * 8 + BT * 4 * (3 if teacher else 1) + 4
    red = BT * (4 * (2 if teacher else 1) + 8) + 16
    return {"forward": fwd, "reduce": red, "backward": bwd}


def run_mode(w, zs, us, tg, n_valid, steps, warmup, teacher):
    import torch
    import cross_entropy_tv_amd as lx

    BT, V = w.BT, w.V
    dev = zs.device
    f = lambda: torch.empty(BT, dtype=torch.float32, device=dev)  # noqa: E731
    ce, lse_s = f(), f()
    tvd, lse_t, sigma = (f(), f(), f()) if teacher else (None, None, None)
    mean = torch.empty(2, dtype=torch.float32, device=dev)
    inv = torch.empty(1, dtype=torch.float32, device=dev)
    grad = torch.empty_like(zs)
    dt = lx.LX_BF16 if w.dtype == "bf16" else lx.LX_F32
    nws = lx.lx_ce_tvd_workspace_bytes(BT, V, dt, teacher)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    u = us if teacher else None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        lx.lx_ce_tvd_forward(zs, u, tg, -100, ce, tvd, lse_s, lse_t, sigma, ws, stream)
        if ev is not None:
            ev[1].record(stream)
        lx.lx_ce_tvd_reduce_mean(ce, tvd, tg, -100, mean, None, inv, stream)
        if ev is not None:
            ev[2].record(stream)
        lx.lx_ce_tvd_backward(grad, zs, u, tg, -100, lse_s, lse_t, sigma, 1.0, 1.0, inv, stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    red_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    bwd_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    ab = algorithmic_bytes(BT, V, w.esize, n_valid, teacher)
    res = {
        "ms_per_step": wall * 1e3 / steps,
        "tokens_per_s": BT * steps / wall,
        "forward_ms": fwd_ms, "reduce_ms": red_ms, "backward_ms": bwd_ms,
        "forward_GBs": ab["forward"] / fwd_ms / 1e6, "backward_GBs": ab["backward"] / bwd_ms / 1e6,
        "alg_bytes": ab,
        "mean": mean.cpu().tolist(),
    }
    res["forward_pct_peak"] = 100.0 * res["forward_GBs"] / HBM_PEAK_GBS
    res["backward_pct_peak"] = 100.0 * res["backward_GBs"] / HBM_PEAK_GBS
    return res


def run_fused(w, zs, us, tg, n_valid, steps, warmup, teacher=True):
    """One step = count the valid rows (1/n_valid on the device) -> one fused forward +
    backward pass -> mean of the per-row losses."""
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
    nws = lx.lx_ce_tvd_forward_backward_workspace_bytes(BT, V, dt, teacher)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        lx.lx_ce_tvd_count_valid(tg, -100, None, inv, stream)
        if ev is not None:
            ev[1].record(stream)
        lx.lx_ce_tvd_forward_backward(zs, u, tg, -100, ce, tvd, lse_s, lse_t, sigma, grad, 1.0, 1.0, inv, ws,
                                      stream)
        if ev is not None:
            ev[2].record(stream)
        lx.lx_ce_tvd_reduce_mean(ce, tvd, tg, -100, mean, None, None, stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cnt_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    fb_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    red_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    n_ign = BT - n_valid
    streams = 2 if teacher else 1
    alg = n_valid * (streams + 1) * V * w.esize + n_ign * V * w.esize + BT * 8 + BT * 4 * (5 if teacher else 2) + 4
    return {"ms_per_step": wall * 1e3 / steps, "tokens_per_s": BT * steps / wall, "count_ms": cnt_ms,
            "fused_ms": fb_ms, "reduce_ms": red_ms, "fused_GBs": alg / fb_ms / 1e6,
            "fused_pct_peak": 100.0 * alg / fb_ms / 1e6 / HBM_PEAK_GBS, "alg_bytes": alg,
            "mean": mean.cpu().tolist()}


def run_vocab_parallel(w, zs, us, tg, n_valid, steps, warmup, n_shards=8):
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
    stream = torch.cuda.current_stream()
    lx.lx_ce_tvd_count_valid(tg, -100, None, inv, stream)
    for n in range(n_shards):  # stand-ins for the other devices' partials
        lx.lx_ce_tvd_vp_stats(zsh, ush, tg, 0, -100, stats[n], stream)
    lx.lx_ce_tvd_vp_merge_stats(stats, tg, V, -100, ce, lse_s, lse_t, stream)
    for n in range(n_shards):
        lx.lx_ce_tvd_vp_tv(zsh, ush, tg, -100, lse_s, lse_t, tv[n], stream)

    def step(ev=None):
        calls = (lambda: lx.lx_ce_tvd_vp_stats(zsh, ush, tg, 0, -100, stats[0], stream),
                 lambda: lx.lx_ce_tvd_vp_merge_stats(stats, tg, V, -100, ce, lse_s, lse_t, stream),
                 lambda: lx.lx_ce_tvd_vp_tv(zsh, ush, tg, -100, lse_s, lse_t, tv[0], stream),
                 lambda: lx.lx_ce_tvd_vp_merge_tv(tv, tg, -100, tvd, sigma, stream),
                 lambda: lx.lx_ce_tvd_backward_shard(grad, zsh, ush, tg, 0, V, -100, lse_s, lse_t, sigma, 1.0,
                                                     1.0, inv, stream))
        for k, c in enumerate(calls):
            if ev is not None:
                ev[k].record(stream)
            c()
        if ev is not None:
            ev[len(calls)].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    ms = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i in range(5)]
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
    out["device_step_ms"] = round(sum(ms), 4)
    return out


def _time_call(fn, steps, warmup):
    """Average HIP-event time (ms) of fn() on the current stream."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps


def run_ex(w, zs, us, tg, n_valid, steps, warmup, pad=128):
    """The one-pass forward + backward of the ABI-breadth entry points on the same batch:
    binary16 copies of the logits; the logits inside arrays padded to V + pad columns
    (row strides, e.g. a vocabulary rounded up to a multiple of 256), gradient in
    place; per-row upstream gradients (an unreduced loss).  Each is timed alone, with
    its algorithmic bytes those of the one pass (read student and teacher once, write
    the gradient once)."""
    import torch
    import cross_entropy_tv_amd as lx

    BT, V = w.BT, w.V
    dev = zs.device
    f = lambda: torch.empty(BT, dtype=torch.float32, device=dev)  # noqa: E731
    ce, lse_s, tvd, lse_t, sigma = f(), f(), f(), f(), f()
    stream = torch.cuda.current_stream()
    n_ign = BT - n_valid
    alg = n_valid * 3 * V * w.esize + n_ign * V * w.esize + BT * 8 + BT * 4 * 5 + 4
    inv = torch.empty(1, dtype=torch.float32, device=dev)
    lx.lx_ce_tvd_count_valid(tg, -100, None, inv, stream)
    nws = lx.lx_ce_tvd_forward_backward_workspace_bytes(BT, V, lx.LX_BF16, True)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    out = {}

    def record(name, ms, extra=None):
        out[name] = {"ms": round(ms, 4), "GBs": round(alg / ms / 1e6, 1),
                     "pct_peak": round(100.0 * alg / ms / 1e6 / HBM_PEAK_GBS, 2), **(extra or {})}

    g = torch.empty_like(zs)

    def plain():
        lx.lx_ce_tvd_forward_backward(zs, us, tg, -100, ce, tvd, lse_s, lse_t, sigma, g, 1.0, 1.0, inv, ws, stream)

    # the headline call again, for reference next to the variants (same process, same memory state)
    record("reference", _time_call(plain, steps, warmup))
    # per-row upstream gradients of an unreduced loss (factors ~ U(0.5, 1.5))
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261202)
    wce = torch.rand(BT, generator=gen, device=dev) + 0.5
    wtv = torch.rand(BT, generator=gen, device=dev) + 0.5
    record("row_factors", _time_call(lambda: lx.lx_ce_tvd_forward_backward_ex(
        zs, us, tg, -100, ce, tvd, lse_s, lse_t, sigma, g, 1.0, 1.0, wce, wtv, inv, ws, stream), steps, warmup))
    # binary16 logits: the bf16 batch rounded to binary16
    z16, u16 = zs.to(torch.float16), us.to(torch.float16)
    g16 = torch.empty_like(z16)
    record("f16", _time_call(lambda: lx.lx_ce_tvd_forward_backward(
        z16, u16, tg, -100, ce, tvd, lse_s, lse_t, sigma, g16, 1.0, 1.0, inv, ws, stream), steps, warmup),
        {"logits": "f16"})
    del z16, u16, g16
    # row strides: views into arrays of V + pad columns, gradient in place over a scratch copy
    zbig = torch.empty((BT, V + pad), dtype=zs.dtype, device=dev)
    ubig = torch.empty((BT, V + pad), dtype=us.dtype, device=dev)
    zbig[:, :V] = zs
    ubig[:, :V] = us
    zv, uv = zbig[:, :V], ubig[:, :V]
    gbig = torch.empty_like(zbig)
    gv = gbig[:, :V]
    record("strided", _time_call(lambda: lx.lx_ce_tvd_forward_backward_ex(
        zv, uv, tg, -100, ce, tvd, lse_s, lse_t, sigma, gv, 1.0, 1.0, g_scale=inv, workspace=ws, stream=stream),
        steps, warmup), {"row_stride": V + pad})
    del zbig, ubig, gbig
    record("reference_after", _time_call(plain, steps, warmup))
    return out


def run_linear(steps, warmup, BT=8192, V=151936, H=4096, chunk_rows=8192):
    """The lm_head products + CE + TVD in one call (student and teacher lm_heads of
    hidden size H over the vocabulary, seeded synthetic hidden states and weights):
    the whole call, and each bf16 matrix product alone at the call's shapes, timed
    with HIP events; FLOP/s against the dense bf16 matrix-core peak.  The whole
    batch is one chunk (a workspace of ~10 B per logit, 12.4 GB here): chunks of
    4096 rows cost 2.4% more time, of 2048 rows 8%."""
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
    stream = torch.cuda.current_stream()
    lx.lx_ce_tvd_count_valid(tg, -100, None, inv, stream)
    ws = torch.empty(lx.lx_ce_tvd_linear_workspace_bytes(BT, V, True, chunk_rows), dtype=torch.uint8, device=dev)
    ms = _time_call(lambda: lx.lx_ce_tvd_linear_forward_backward(
        X, Wd, Xt, Wt, tg, -100, ce, tvd, lse_s, lse_t, sigma, gx, gw, 1.0, 1.0, inv, chunk_rows, ws, stream),
        steps, warmup)
    flops = 2.0 * BT * V * H * 4  # student and teacher logits, grad of x, grad of w
    out = {"shape": f"BT={BT} V={V} H_s=H_t={H} chunk_rows={chunk_rows}", "ms": round(ms, 3),
           "tokens_per_s": round(BT / ms * 1e3, 1), "TFLOPs": round(flops / ms / 1e9, 1),
           "pct_mfma_peak": round(100.0 * flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2)}
    # each product alone, at the shapes of one chunk
    R = chunk_rows
    z = torch.empty((R, V), dtype=torch.float32, device=dev)
    # G with gradient-like values: an all-zero operand lets the matrix cores
    # draw less power, and the products on it ran 14-28% faster than on the
    # gradient the call itself produces
    gen = torch.Generator(device=dev)
    gen.manual_seed(78)
    G = (torch.randn((R, V), generator=gen, device=dev) * 1e-5).to(torch.bfloat16)
    Gt, Xt = G.t().contiguous(), X[:R].t().contiguous()
    gemms = {
        "logits_XWt": (lambda: lx.lx_gemm_bf16(X[:R], True, Wd, True, z, R, V, H, False, stream), R, V, H),
        "grad_x_GW": (lambda: lx.lx_gemm_bf16(G, True, Wd, False, gx[:R], R, H, V, False, stream), R, H, V),
        # as the call forms it: from the transposed copies of G and x (both K-contiguous)
        "grad_w_GtX": (lambda: lx.lx_gemm_bf16(Gt, True, Xt, True, gw, V, H, R, True, stream), V, H, R),
    }
    for name, (fn, M, N, K) in gemms.items():
        t_ms = _time_call(fn, steps, warmup)
        fl = 2.0 * M * N * K
        out[name] = {"M": M, "N": N, "K": K, "ms": round(t_ms, 4), "TFLOPs": round(fl / t_ms / 1e9, 1),
                     "pct_mfma_peak": round(100.0 * fl / t_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2)}
    del z, G, Gt, Xt, ws, gx, gw
    return out


def copy_ceiling(dev, nbytes=2 << 30, reps=10):
    """Achieved GB/s of a plain device copy (read + write), the practical streaming ceiling."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    a.fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    return 2 * nbytes / ms / 1e6


def traffic_from_profiles(kernel_key, launches_bytes):
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


def cpu_baseline(w, seconds_per_worker=1.5, batch=4, workers=None):
    """The float64 oracle, as it stands, timed on the host cores over a bounded sample of
    the same workload's rows (forward + backward per row).  Each worker process takes
    its own rows in batches and stops once its timed oracle work passes
    ``seconds_per_worker``; the rate is the sum of the workers' rates (they run
    concurrently)."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    workers = workers or min(cores, 16)
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        res = pool.map(_cpu_worker, [(w.name, i, workers, batch, seconds_per_worker) for i in range(workers)])
    rate = sum(r[0] / r[1] for r in res)
    nrows = sum(r[0] for r in res)
    cpu_s = sum(r[1] for r in res)
    return {"value": round(rate, 1), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{nrows} rows of the {w.name} workload ({w.BT}x{w.V} {w.dtype}), float64 numpy oracle "
                      f"forward+backward per row, {workers} single-threaded processes, {cpu_s:.1f} s of timed "
                      f"CPU work in total"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train")
    ap.add_argument("--mode", default="ce_tvd", choices=["ce_tvd", "ce"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ce-only", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-vocab-parallel", action="store_true")
    ap.add_argument("--no-ex", action="store_true", help="skip the binary16 / strided / per-row one-pass legs")
    ap.add_argument("--no-linear", action="store_true", help="skip the lm_head product + loss leg")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (rows shard across GPUs "
              "with no exchange except a 3-scalar loss reduction, which this single-GPU build does not run)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import cross_entropy_tv_amd as lx  # noqa: F401  (fails loudly if the HIP library is missing)
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.get(args.workload)
    t_gen = time.perf_counter()
    z, u, t = W.full(w)
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] generated {w.name} {w.BT}x{w.V} {w.dtype} in {gen_s:.1f} s", file=sys.stderr, flush=True)

    def dev_copy(raw):
        if raw.dtype == np.uint16:
            return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(raw).to(dev)

    zs, us, tg = dev_copy(z), dev_copy(u), dev_copy(t)
    del z, u
    n_valid = int((t != W.IGNORE_INDEX).sum())
    teacher = args.mode == "ce_tvd"
    main_res = run_mode(w, zs, us, tg, n_valid, args.steps, args.warmup, teacher)
    print(f"[bench] {args.mode}: {main_res['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
    extra = {}
    if teacher and not args.no_ce_only:
        ce_res = run_mode(w, zs, us, tg, n_valid, args.steps, args.warmup, False)
        extra["ce_only"] = {k: ce_res[k] for k in ("tokens_per_s", "ms_per_step", "forward_ms", "backward_ms",
                                                    "forward_GBs", "backward_GBs", "forward_pct_peak",
                                                    "backward_pct_peak")}
        if not args.no_fused:
            cf = run_fused(w, zs, us, tg, n_valid, args.steps, args.warmup, teacher=False)
            extra["ce_only"]["fused"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in cf.items()
                                         if k != "mean"}
    if teacher and not args.no_fused:
        fu = run_fused(w, zs, us, tg, n_valid, args.steps, args.warmup)
        extra["fused"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in fu.items()}
    if teacher and not args.no_vocab_parallel and w.V % 8 == 0:
        extra["vocab_parallel"] = run_vocab_parallel(w, zs, us, tg, n_valid, args.steps, args.warmup)
    if teacher and not args.no_ex and w.dtype == "bf16":
        extra["one_pass_ex"] = run_ex(w, zs, us, tg, n_valid, args.steps, args.warmup)
    if teacher and not args.no_linear:
        extra["linear"] = run_linear(args.steps, args.warmup)
    if not args.no_ceiling:
        extra["copy_ceiling_GBs"] = copy_ceiling(dev)

    # Headline: the fused path when it ran (forward and backward in one pass over the
    # logits, then the mean), else the separate passes.  Both are reported.
    if "fused" in extra:
        fu = extra["fused"]
        path = "fused"
        value, ms_step = fu["tokens_per_s"], fu["ms_per_step"]
        kname, kms, kbytes = "forward_backward", fu["fused_ms"], fu["alg_bytes"]
    else:
        path = "separate"
        value, ms_step = main_res["tokens_per_s"], main_res["ms_per_step"]
        # dominant kernel: the pass with the larger share of the step
        kname = "backward" if main_res["backward_ms"] >= main_res["forward_ms"] else "forward"
        kms, kbytes = main_res[f"{kname}_ms"], main_res["alg_bytes"][kname]
    achieved = kbytes / kms / 1e6
    traffic = traffic_from_profiles(f"{kname}_{args.mode}_{w.name}", kbytes)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kname,
                "alg_bytes_per_launch": kbytes, "avg_launch_ms": round(kms, 4)}
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "BT": w.BT, "V": w.V, "logits": w.dtype, "mode": args.mode,
                   "path": path, "global_batch": w.BT, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "separate_step": {"tokens_per_s": round(main_res["tokens_per_s"], 1),
                          "ms_per_step": round(main_res["ms_per_step"], 4)},
        "passes": {"forward_ms": round(main_res["forward_ms"], 4), "reduce_ms": round(main_res["reduce_ms"], 4),
                   "backward_ms": round(main_res["backward_ms"], 4),
                   "forward_GBs": round(main_res["forward_GBs"], 1),
                   "backward_GBs": round(main_res["backward_GBs"], 1),
                   "forward_pct_peak": round(main_res["forward_pct_peak"], 2),
                   "backward_pct_peak": round(main_res["backward_pct_peak"], 2)},
        "mean_loss": main_res["mean"],
        **extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
