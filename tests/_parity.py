"""Comparison of the HIP path against the float64 oracle.

Tolerances (the loss's stated accuracy targets):
  * ce, lse_s, lse_t: 1e-4 absolute;
  * tvd, sigma: 1e-5 absolute;
  * gradient: 2^-8 * |ref| + 1e-6 absolute (2^-8 is the unit roundoff of a
    bf16 store, so fp32 math rounded once to bf16 fits);
  * ignored rows: bit-exact +0.0 everywhere.

The gradient is also held to the same bound with its absolute term scaled by
the row's upstream gradient, M = |g_ce| + |g_tvd| (as applied to the row),
when M < 1: rel * |ref| + 1e-6 * min(1, M).  A mean over n rows scales every
gradient by 1/n, and an unscaled 1e-6 would then exceed nearly every element
(at n = 8192 the bulk of a row is ~1e-10), checking little beyond the target.
rel is 2^-8 for kernels that form p in fp32; the one-pass kernels keep
2^15 * p as binary16 (relative error 2^-11) where the gradient's scale allows,
and are held to their own bound, rel = 2^-8 + 2^-10.  binary16 gradients add
2^-25 (half the spacing of binary16 subnormals) to the absolute term.

Near ties.  sign(p - q) is discontinuous, and |p - q| has a subgradient of
every sign at p = q.  Two sets of elements are distinguished:
  * relative near ties, |p - q| <= 2^-16 * max(p, q): fp32 cannot order p
    and q reliably there (the kernels' lse carries a few fp32 ulps), exact ties
    included (p = q in float64 from different logits, e.g. V = 1, still rounds
    apart in fp32; only identical student and teacher rows give equal fp32
    arguments, and their exact zeros are asserted on their own);
  * the exemption of the accuracy targets, |p - q| < 1e-7, or a relative
    near tie.
Gradients: at exempt elements the kernel may take any of the three sign
branches.  The branch it took is read back from its gradient where the gap
between branches, |g_tvd| / 2 * p, is at least 4x the gradient tolerance, and
the gradient is then compared, with the plain tolerances, against the oracle's
result for exactly those signs (``oracle.backward(signs=...)``).  Exempt
elements whose branch cannot be read back (gap below 4x the tolerance) may
differ by up to the gap.  sigma: a kernel's sigma is held to 1e-5 against the
oracle's sigma for the signs read back from the same kernel's gradient where
that is available, else to 1e-5 plus the slack 2 * sum of p over the relative
near ties of the row (the mass whose signs fp32 cannot order).  Every check
returns its statistics (worst error/tolerance ratios, branch flips, slack
used) so the tests can print and cap them.
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
G_REL_P16 = 2.0 ** -8 + 2.0 ** -10   # one-pass kernels: binary16 copy of 2^15 * p
F16_FLOOR = 2.0 ** -25               # binary16 gradients: half the subnormal spacing


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


def probs(z_raw, u_raw, valid):
    """(p, q) of the valid rows, from the oracle's building blocks."""
    zv = oracle.decode(z_raw)[valid]
    uv = oracle.decode(u_raw)[valid]
    return (oracle.probs_rows(zv, oracle.logsumexp_rows(zv)),
            oracle.probs_rows(uv, oracle.logsumexp_rows(uv)))


def near_ties(p, q):
    """(relative near ties, exempt set) as boolean masks (see the module notes)."""
    d = np.abs(p - q)
    rel = d <= TIE_REL * np.maximum(p, q)
    return rel, rel | (d < TIE_ABS)


def tie_info(z_raw, u_raw, valid):
    """(p, exempt mask, per-row sigma slack over the relative near ties) for the valid rows."""
    p, q = probs(z_raw, u_raw, valid)
    rel, exempt = near_ties(p, q)
    return p, exempt, 2.0 * np.sum(np.where(rel, p, 0.0), axis=1)


def merge_stats(acc: dict, st: dict) -> dict:
    """Running maxima / sums of the statistics of several checks."""
    for k, v in st.items():
        if k.startswith("n_"):
            acc[k] = acc.get(k, 0) + v
        else:
            acc[k] = max(acc.get(k, 0.0), v)
    return acc


def format_stats(st: dict) -> str:
    return ", ".join(f"{k} {v:.3g}" if isinstance(v, float) else f"{k} {v}" for k, v in sorted(st.items()))


# ---------------------------------------------------------------- forward

def check_forward_ref(out: dict, ref: dict, valid, teacher: bool, slack=None, label="", sigma_branch=None):
    """Forward outputs against precomputed oracle outputs.

    out: float32 arrays; ref: the oracle's float64 arrays for the same rows;
    slack: per-row sigma slack (length = number of valid rows) or None;
    sigma_branch: optional float64 [R] oracle sigma for the signs the kernel
    took (rows where it is not NaN are held to 1e-5 against it, no slack).
    Returns statistics."""
    st = {}
    keys = ("ce", "tvd", "lse_s", "lse_t", "sigma") if teacher else ("ce", "lse_s")
    for k in keys:
        assert np.all(bits32(out[k][~valid]) == 0), f"{label}: ignored rows of {k} are not +0.0"
    if not valid.any():
        return st
    for k in ("ce", "lse_s") + (("lse_t",) if teacher else ()):
        err = np.abs(out[k][valid].astype(np.float64) - ref[k][valid])
        st[f"{k}_err/tol"] = float(err.max() / TOL_CE)
        assert np.all(err <= TOL_CE), f"{label}: {k} max err {err.max()} at valid row {np.argmax(err)}"
    if not teacher:
        return st
    err = np.abs(out["tvd"][valid].astype(np.float64) - ref["tvd"][valid])
    st["tvd_err/tol"] = float(err.max() / TOL_TV)
    assert np.all(err <= TOL_TV), f"{label}: tvd max err {err.max()} at valid row {np.argmax(err)}"
    sg = out["sigma"][valid].astype(np.float64)
    err = np.abs(sg - ref["sigma"][valid])
    slack = np.zeros_like(err) if slack is None else np.asarray(slack, dtype=np.float64)
    used = np.maximum(err - TOL_TV, 0.0)
    st["sigma_err/tol"] = float(err.max() / TOL_TV)
    st["sigma_slack_used"] = float(used.max())
    st["sigma_slack_allowed_max"] = float(slack.max()) if slack.size else 0.0
    st["n_rows_using_sigma_slack"] = int(np.count_nonzero(used > 0))
    bad = err > TOL_TV + slack
    assert not bad.any(), (f"{label}: sigma err {err[bad].max()} beyond 1e-5 + slack "
                           f"{slack[bad][np.argmax(err[bad])]} (valid row {np.nonzero(bad)[0][0]})")
    if sigma_branch is not None:
        sb = np.asarray(sigma_branch, dtype=np.float64)[valid]
        have = ~np.isnan(sb)
        if have.any():
            eb = np.abs(sg[have] - sb[have])
            st["sigma_branch_err/tol"] = float(eb.max() / TOL_TV)
            assert np.all(eb <= TOL_TV), f"{label}: sigma {eb.max()} from the sigma of the branch its gradient took"
    return st


def check_forward(out: dict, z_raw, u_raw, target, ignore_index, label="", stats=None):
    """out: dict of float32 numpy arrays (ce, lse_s and, with a teacher, tvd, lse_t, sigma)."""
    target = np.asarray(target)
    ref = oracle.forward(z_raw, u_raw, target, ignore_index)
    valid = target != ignore_index
    slack = None
    if u_raw is not None and valid.any():
        _, _, slack = tie_info(z_raw, u_raw, valid)
    st = check_forward_ref(out, ref, valid, u_raw is not None, slack, label)
    if stats is not None:
        merge_stats(stats, st)
    return ref


# ---------------------------------------------------------------- gradient

def _row_vec(g, R):
    return np.broadcast_to(np.asarray(g, dtype=np.float64), (R,)).copy()


def check_grad(g_gpu: np.ndarray, g_bits: np.ndarray, z_raw, u_raw, target, ignore_index, g_ce, g_tvd, label="",
               rel=G_REL, fmt="bf16", sigma_gpu=None, stats=None, ref=None, pq=None, sigma_ref=None,
               stated_rel=G_REL):
    """g_gpu: float64 view of the device gradient; g_bits: its raw bits.  g_ce and
    g_tvd are the upstream gradients of each row as applied (scalars or per-row
    arrays).  rel: the relative part of the scaled bound (G_REL_P16 for the
    one-pass kernels).  stated_rel: the relative part of the stated bound (2^-8;
    the lm_head path's G, an intermediate of its products formed from binary16
    p, is held to G_REL_P16 there too).  fmt: the gradient's storage type ("f16"
    adds F16_FLOOR).
    sigma_gpu: the sigma [R] the same kernel computed (optional): then it is held
    to 1e-5 against the oracle's sigma for the branch the gradient took.
    ref, pq, sigma_ref: the oracle gradient of these rows, their (p, q) and the
    oracle's sigma, when the caller already has them.  Returns the oracle gradient for the branch taken."""
    target = np.asarray(target)
    R, V = z_raw.shape
    valid = target != ignore_index
    assert np.all(g_bits[~valid] == 0), f"{label}: ignored gradient rows are not +0.0"
    if ref is None:
        ref = oracle.backward(z_raw, u_raw, target, ignore_index, g_ce, g_tvd)
    gce, gtv = _row_vec(g_ce, R), _row_vec(g_tvd, R)
    M = np.abs(gce) + (0.0 if u_raw is None else np.abs(gtv))
    floor = G_ABS * np.minimum(1.0, M)[:, None] + (F16_FLOOR if fmt == "f16" else 0.0)
    st = {}
    widen = np.zeros((R, V))
    if u_raw is not None and valid.any():
        p, q = probs(z_raw, u_raw, valid) if pq is None else pq
        rel_set, exempt = near_ties(p, q)
        vi = np.nonzero(valid)[0]
        beta = 0.5 * gtv[vi][:, None]
        gap = np.abs(beta) * p
        # The branch is read where the gap between branches is 4x the kernel's own
        # error: its relative rounding plus 2^-38 * M, the binary16 subnormal spacing
        # of 2^15 * p (scaled), not the tolerance's absolute floor, which is far
        # above the gradient of a row whose mean scale is 1/n.
        noise = rel * np.abs(ref[vi]) + 2.0 ** -38 * M[vi][:, None]
        ident = exempt & (gap > 4.0 * noise)
        s_ref = np.sign(p - q)
        s_gpu = s_ref.copy()
        with np.errstate(divide="ignore", invalid="ignore"):
            k = np.rint((g_gpu[vi] - ref[vi]) / (beta * p))
        s_gpu[ident] = np.clip(s_ref[ident] + k[ident], -1.0, 1.0)
        flips = ident & (s_gpu != s_ref)
        unident = exempt & ~ident
        st["n_exempt"] = int(exempt.sum())
        st["n_rel_near_ties"] = int(rel_set.sum())
        st["n_branch_flips"] = int(flips.sum())
        st["n_flips_outside_rel_near_ties"] = int((flips & ~rel_set).sum())
        st["n_exempt_unreadable"] = int(unident.sum())
        # any branch at exempt elements whose branch cannot be read back
        widen[vi] = np.where(unident, 2.0 * gap * (1 + G_REL), 0.0)
        sigma_branch = np.full(R, np.nan)
        if sigma_ref is not None:
            sigma_branch[vi] = np.asarray(sigma_ref, dtype=np.float64)[vi]
        fr = np.nonzero(flips.any(axis=1))[0]
        if fr.size:
            s_alt = np.zeros((R, V))
            s_alt[vi] = s_gpu
            rows = vi[fr]
            alt = oracle.backward(z_raw[rows], u_raw[rows], target[rows], ignore_index, gce[rows], gtv[rows],
                                  signs=s_alt[rows])
            ref = ref.copy()
            ref[rows] = alt
            fw_alt = oracle.forward(z_raw[rows], u_raw[rows], target[rows], ignore_index, signs=s_alt[rows])
            if sigma_ref is None:
                sigma_branch[rows] = oracle.forward(z_raw[rows], u_raw[rows], target[rows], ignore_index)["sigma"]
            st["sigma_branch_shift"] = float(np.max(np.abs(fw_alt["sigma"] - sigma_branch[rows])))
            sigma_branch[rows] = fw_alt["sigma"]
        # the mass whose branch is not known: relative near ties that could not be read
        unknown = 2.0 * np.sum(np.where(unident & rel_set, p, 0.0), axis=1)
        st["sigma_unread_mass"] = float(unknown.max())
        if sigma_gpu is not None:
            sg = np.asarray(sigma_gpu, dtype=np.float64)[vi]
            if np.isnan(sigma_branch[vi]).any():
                miss = vi[np.isnan(sigma_branch[vi])]
                sigma_branch[miss] = oracle.forward(z_raw[miss], u_raw[miss], target[miss], ignore_index)["sigma"]
            sb = sigma_branch[vi]
            eb = np.abs(sg - sb)
            st["sigma_branch_err/tol"] = float(np.max(eb / (TOL_TV + unknown)))
            assert np.all(eb <= TOL_TV + unknown), (
                f"{label}: sigma off by {eb.max()} from the sigma of the sign branch its own gradient took "
                f"(unread near-tie mass {unknown[np.argmax(eb)]})")
            ds = eb
        else:
            ds = TOL_TV + 2.0 * np.sum(np.where(rel_set, p, 0.0), axis=1)
        # sigma's error reaches every element of the row through beta * p * (sigma - sigma_branch)
        widen[vi] += np.abs(beta) * p * ds[:, None]
    err = np.abs(g_gpu - ref)
    tol_ns = stated_rel * np.abs(ref) + G_ABS + widen
    tol_u = rel * np.abs(ref) + floor + widen
    st["grad_err/tol"] = float(np.max(err / np.maximum(tol_ns, 1e-300))) if err.size else 0.0
    st["grad_err/tol_scaled"] = float(np.max(err / np.maximum(tol_u, 1e-300))) if err.size else 0.0
    for name, tol in (("stated", tol_ns), ("scaled", tol_u)):
        bad = err > tol
        if bad.any():
            r, v = np.argwhere(bad)[0]
            raise AssertionError(f"{label}: {bad.sum()} gradient elements outside the {name} tolerance; first at "
                                 f"row {r} v {v}: gpu {g_gpu[r, v]!r} ref {ref[r, v]!r} tol {tol[r, v]!r}")
    if u_raw is None and V >= 2 and valid.any():
        # CE-only: exactly one negative entry per valid row, at its target, where g_ce > 0
        pos = gce > 0
        if pos.any():
            neg = g_gpu[valid & pos] < 0
            assert np.all(neg.sum(1) == 1) and np.all(neg[np.arange(neg.shape[0]), target[valid & pos]]), \
                f"{label}: target handling"
    if stats is not None:
        merge_stats(stats, st)
    return ref
