"""Comparison of the HIP path against the float64 oracle.

Tolerances (the loss's stated accuracy targets):
  * ce, lse_s, lse_t: 1e-4 absolute;
  * tvd, sigma: 1e-5 absolute;
  * gradient: 2^-8 * |ref| + 1e-6 absolute (2^-8 is the half-ulp of a bf16
    store relative to the value, so fp32 math rounded once to bf16 fits);
  * ignored rows: bit-exact +0.0 everywhere.

Near ties.  sign(p - q) is discontinuous.  An element v with
|p_v - q_v| < 1e-7, or within 2^-16 * max(p_v, q_v) (about 4x the fp32
rounding of p and q), is exempt from sign agreement: its gradient may follow
any of the three sign branches, which moves it by at most |g_tvd| * p_v.
sigma integrates those signs, so a row's sigma may move by up to
slack = 2 * sum of p over its exempt elements, which in turn moves every
gradient element of the row by at most 0.5 * |g_tvd| * p_v * slack.  On the
seeded workloads the exempt sets are empty or tiny, so these widenings do not
weaken the checks.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"
TOL_CE = 1e-4
TOL_TV = 1e-5
TIE_REL = 2.0 ** -16
TIE_ABS = 1e-7
G_REL = 2.0 ** -8
G_ABS = 1e-6


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(raw: np.ndarray) -> torch.Tensor:
    if raw.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(raw)).to(DEV)


def bits32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def grad_to_host(g: torch.Tensor) -> np.ndarray:
    return g.float().cpu().numpy().astype(np.float64)


def grad_bits(g: torch.Tensor) -> np.ndarray:
    if g.dtype in (torch.bfloat16, torch.float16):
        return g.view(torch.int16).cpu().numpy().view(np.uint16)
    return g.view(torch.int32).cpu().numpy().view(np.uint32)


def tie_info(z_raw, u_raw, valid):
    """(oracle p, exempt mask, per-row sigma slack) for the valid rows."""
    zv = oracle.decode(z_raw)[valid]
    uv = oracle.decode(u_raw)[valid]
    p = oracle.probs_rows(zv, oracle.logsumexp_rows(zv))
    q = oracle.probs_rows(uv, oracle.logsumexp_rows(uv))
    d = np.abs(p - q)
    mask = (d < TIE_ABS) | (d <= TIE_REL * np.maximum(p, q))
    slack = 2.0 * np.sum(np.where(mask, p, 0.0), axis=1)
    return p, mask, slack


def check_forward(out: dict, z_raw, u_raw, target, ignore_index, label=""):
    """out: dict of float32 numpy arrays (ce, lse_s and, with a teacher, tvd, lse_t, sigma)."""
    target = np.asarray(target)
    ref = oracle.forward(z_raw, u_raw, target, ignore_index)
    valid = target != ignore_index
    keys = ("ce", "lse_s") if u_raw is None else ("ce", "tvd", "lse_s", "lse_t", "sigma")
    for k in keys:
        assert np.all(bits32(out[k][~valid]) == 0), f"{label}: ignored rows of {k} are not +0.0"
    for k in ("ce", "lse_s") + (() if u_raw is None else ("lse_t",)):
        err = np.abs(out[k][valid].astype(np.float64) - ref[k][valid])
        assert np.all(err <= TOL_CE), f"{label}: {k} max err {err.max()} at row {np.argmax(err)}"
    if u_raw is None or not valid.any():
        return ref
    err = np.abs(out["tvd"][valid].astype(np.float64) - ref["tvd"][valid])
    assert np.all(err <= TOL_TV), f"{label}: tvd max err {err.max()}"
    _, _, slack = tie_info(z_raw, u_raw, valid)
    err = np.abs(out["sigma"][valid].astype(np.float64) - ref["sigma"][valid])
    assert np.all(err <= TOL_TV + slack), f"{label}: sigma max err {err.max()} (slack {slack[np.argmax(err)]})"
    return ref


def check_grad(g_gpu: np.ndarray, g_bits: np.ndarray, z_raw, u_raw, target, ignore_index, g_ce, g_tvd, label=""):
    """g_gpu: float64 view of the device gradient; g_bits: its raw bits.  g_ce and
    g_tvd are scalars or per-row arrays (the upstream gradient of each row)."""
    target = np.asarray(target)
    valid = target != ignore_index
    assert np.all(g_bits[~valid] == 0), f"{label}: ignored gradient rows are not +0.0"
    ref = oracle.backward(z_raw, u_raw, target, ignore_index, g_ce, g_tvd)
    tol = G_REL * np.abs(ref) + G_ABS
    if u_raw is not None and valid.any():
        p, mask, slack = tie_info(z_raw, u_raw, valid)
        gt = np.abs(np.broadcast_to(np.asarray(g_tvd, dtype=np.float64), target.shape))[valid][:, None]
        extra = gt * p * (1 + G_REL) * (mask + 0.5 * slack[:, None])
        tol[valid] += extra
    err = np.abs(g_gpu - ref)
    bad = err > tol
    if bad.any():
        r, v = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {bad.sum()} gradient elements out of tolerance; first at row {r} v {v}: "
                             f"gpu {g_gpu[r, v]!r} ref {ref[r, v]!r} tol {tol[r, v]!r}")
    if u_raw is None and z_raw.shape[1] >= 2 and np.ndim(g_ce) == 0 and g_ce > 0:
        # CE-only: exactly one negative entry per valid row, at its target
        neg = g_gpu[valid] < 0
        assert np.all(neg.sum(1) == 1) and np.all(neg[np.arange(neg.shape[0]), target[valid]]), \
            f"{label}: target handling"
    return ref
