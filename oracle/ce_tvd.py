"""Float64 CPU oracle for the fused cross-entropy + total-variation-distance loss.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The product path
(the HIP library and its Python binding) never routes through it, and this
module shares no code with that path.

What is computed, and where the definitions come from.  The subject is the
"Liger-Kernel PR #1384 analysis" page (blog.secrett2633.cloud, the analysis of
the merged Liger-Kernel pull request "add fused CE + TV distance kernel").  Per
token row with student logits z (length V), teacher logits u and target t:

* page section "Forward Pass", step 1: the log-sum-exp of each row,
  lse = max + log(sum exp(x - max)), for student and teacher;
* page section "Forward Pass", step 2: with p = softmax(z), q = softmax(u)
  obtained from those log-sum-exps, the total variation
  tvd = 0.5 * sum_v |p_v - q_v| and sigma = sum_v p_v * sign(p_v - q_v);
  the cross-entropy is ce = lse_s - z[t];
* page section "Backward Pass": the gradient with respect to z is
  g_ce * (p_v - [v == t]) + g_tvd * 0.5 * p_v * (sign(p_v - q_v) - sigma),
  with sign(0) = 0 at ties and ignore-index rows contributing nothing;
* page section "Core idea" ("핵심 아이디어"): only O(BT) per-row state
  (ce, tvd, lse_s, lse_t, sigma) is kept between the two passes.

The method is exact (the aibars.net Liger-Kernel page, "Technical
implementation": no approximation), so the oracle is the plain definition,
written with whole-row float64 numpy operations: no blocking, no online
rescaling, no fusion.  The online max/sum-exp streaming of the page is only a
faster route to the same log-sum-exp and is not reproduced here.

Readings where the page is silent (each listed in the design notes):

* an ignored row (target == ignore_index, tested first) has ce = tvd = lse_s =
  lse_t = sigma = +0.0 and an all-+0.0 gradient row;
* a target outside [0, V) that is not the ignore index is a precondition
  violation: the oracle raises ValueError;
* logits must be finite, except that -inf entries are allowed in a row with at
  least one finite entry (those entries get p = 0);
* CE-only mode (no teacher): ce and lse_s only; gradient g_ce * (p - onehot);
* the mean reduction divides the sums over valid rows by the number of valid
  rows (0/0 = NaN when every row is ignored).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- decoding

def decode(raw: np.ndarray) -> np.ndarray:
    """Logits as float64.  uint16 arrays are bf16 bit patterns; float16/float32/float64 are values.

    bf16 is the upper half of an IEEE binary32 word, so widening the bits by 16
    and reinterpreting gives the exact value; binary16 and binary32 values
    widen to float64 exactly.
    """
    raw = np.asarray(raw)
    if raw.dtype == np.uint16:
        return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if raw.dtype in (np.float16, np.float32, np.float64):
        return raw.astype(np.float64)
    raise TypeError(f"unsupported logits dtype {raw.dtype}")


def _check_rows(x: np.ndarray, name: str) -> None:
    if np.isnan(x).any() or np.isposinf(x).any():
        raise ValueError(f"{name}: NaN or +inf logits are outside the oracle's domain")
    if (~np.isfinite(x)).all(axis=-1).any():
        raise ValueError(f"{name}: a row has no finite logit")


def _valid_mask(target: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    target = np.asarray(target, dtype=np.int64)
    ignored = target == ignore_index
    bad = (~ignored) & ((target < 0) | (target >= V))
    if bad.any():
        raise ValueError(f"target out of [0, {V}) at rows {np.nonzero(bad)[0][:8].tolist()}")
    return ~ignored


# ---------------------------------------------------------------- building blocks

def logsumexp_rows(x: np.ndarray) -> np.ndarray:
    """lse of every row: row max plus the log of the summed exponentials of (x - max).

    "Forward Pass", step 1 of the PR #1384 analysis page.
    """
    m = np.max(x, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True)))[..., 0]


def probs_rows(x: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """softmax of every row, formed from the stored lse: exp(x - lse)."""
    return np.exp(x - lse[..., None])


# ---------------------------------------------------------------- forward

def _branch_signs(signs, valid: np.ndarray, shape) -> np.ndarray:
    """The caller's sign vector for the valid rows (values -1, 0 or +1)."""
    s = np.broadcast_to(np.asarray(signs, dtype=np.float64), shape)[valid]
    if not np.all((s == -1.0) | (s == 0.0) | (s == 1.0)):
        raise ValueError("signs must hold -1, 0 or +1")
    return s


def forward(z_raw, u_raw, target, ignore_index: int = -100, signs=None) -> dict:
    """Per-row forward outputs (float64 arrays of shape [R]).

    Returns dict(ce, tvd, lse_s, lse_t, sigma).  ``u_raw=None`` selects CE-only
    mode, where tvd, lse_t and sigma are returned as None.

    ``signs`` (optional, shape [R, V], values -1, 0, +1) replaces sign(p - q) in
    sigma.  |p - q| has a subgradient of every sign where p = q, and where p
    and q agree to within the rounding of the arithmetic at hand any sign
    branch is a correct answer; the page's tie rule (0 at ties) is the
    default.  With explicit signs the result is the one for that branch, so a
    kernel's output can be compared with the branch it took.  tvd does not
    depend on the signs.
    """
    z = decode(z_raw)
    R, V = z.shape
    valid = _valid_mask(target, V, ignore_index)
    t = np.where(valid, np.asarray(target, dtype=np.int64), 0)
    out = {k: np.zeros(R, dtype=np.float64) for k in ("ce", "tvd", "lse_s", "lse_t", "sigma")}
    if u_raw is None:
        out["tvd"] = out["lse_t"] = out["sigma"] = None
    if not valid.any():
        return out
    zv = z[valid]
    _check_rows(zv, "student")
    lse_s = logsumexp_rows(zv)
    out["lse_s"][valid] = lse_s
    out["ce"][valid] = lse_s - zv[np.arange(zv.shape[0]), t[valid]]
    if u_raw is None:
        return out
    uv = decode(u_raw)[valid]
    _check_rows(uv, "teacher")
    lse_t = logsumexp_rows(uv)
    p = probs_rows(zv, lse_s)
    q = probs_rows(uv, lse_t)
    d = p - q
    s = np.sign(d) if signs is None else _branch_signs(signs, valid, z.shape)
    out["lse_t"][valid] = lse_t
    out["tvd"][valid] = 0.5 * np.sum(np.abs(d), axis=-1)
    out["sigma"][valid] = np.sum(p * s, axis=-1)
    return out


# ---------------------------------------------------------------- backward

def backward(z_raw, u_raw, target, ignore_index: int = -100,
             g_ce=1.0, g_tvd=1.0, signs=None) -> np.ndarray:
    """d(sum_r g_ce[r] * ce[r] + g_tvd[r] * tvd[r])/dz for every row, float64 [R, V].

    "Backward Pass" of the PR #1384 analysis page: the cross-entropy part is
    p - onehot(t); the total-variation part is the softmax Jacobian applied to
    0.5 * sign(p - q), i.e. 0.5 * p * (sign(p - q) - sigma).  The oracle
    recomputes lse, p, q and sigma itself from the logits.  Ignored rows are
    all +0.0.  ``u_raw=None`` is CE-only mode.  g_ce and g_tvd are the
    upstream gradients of each row's ce and tvd: scalars (the page's case)
    or arrays of R per-row values (an unreduced loss).  ``signs`` is as in
    ``forward``: the gradient of the branch with those signs (sigma formed
    from them too).
    """
    z = decode(z_raw)
    R, V = z.shape
    valid = _valid_mask(target, V, ignore_index)
    grad = np.zeros((R, V), dtype=np.float64)
    if not valid.any():
        return grad
    g_ce = np.broadcast_to(np.asarray(g_ce, dtype=np.float64), (R,))[valid][:, None]
    g_tvd = np.broadcast_to(np.asarray(g_tvd, dtype=np.float64), (R,))[valid][:, None]
    zv = z[valid]
    _check_rows(zv, "student")
    rows = np.arange(zv.shape[0])
    t = np.asarray(target, dtype=np.int64)[valid]
    p = probs_rows(zv, logsumexp_rows(zv))
    onehot = np.zeros_like(p)
    onehot[rows, t] = 1.0
    gv = g_ce * (p - onehot)
    if u_raw is not None:
        uv = decode(u_raw)[valid]
        _check_rows(uv, "teacher")
        q = probs_rows(uv, logsumexp_rows(uv))
        s = np.sign(p - q) if signs is None else _branch_signs(signs, valid, z.shape)
        sigma = np.sum(p * s, axis=-1, keepdims=True)
        gv = gv + g_tvd * 0.5 * p * (s - sigma)
    grad[valid] = gv
    return grad


# ---------------------------------------------------------------- reduction

def reduce_mean(ce, tvd, target, ignore_index: int = -100):
    """(mean ce, mean tvd or None, n_valid) over the rows whose target is not ignore_index."""
    target = np.asarray(target, dtype=np.int64)
    valid = target != ignore_index
    n = int(valid.sum())
    with np.errstate(invalid="ignore", divide="ignore"):
        mce = np.float64(np.sum(np.asarray(ce, dtype=np.float64)[valid])) / np.float64(n)
        mtv = None if tvd is None else np.float64(np.sum(np.asarray(tvd, dtype=np.float64)[valid])) / np.float64(n)
    return mce, mtv, n


# ---------------------------------------------------------------- lm_head product + loss

def linear_forward_backward(x_s_raw, w_s_raw, x_t_raw, w_t_raw, target, ignore_index: int = -100,
                            g_ce=1.0, g_tvd=1.0) -> dict:
    """The loss over the logits of student and teacher lm_heads, with the gradients
    of the student's hidden states and weight.

    The aibars.net Liger-Kernel page's fused linear cross-entropy: the logits are
    the lm_head product z = x_s w_s^T (u = x_t w_t^T for the teacher), computed
    here exactly in float64 (a matrix product of the decoded inputs); the loss
    and G = d(g_ce ce + g_tvd tvd)/dz are ``forward`` and ``backward`` above;
    by the chain rule through z = x w^T, dL/dx_s = G w_s and dL/dw_s = G^T x_s.
    ``x_t_raw=None`` is CE-only mode.  Returns the forward dict plus ``grad``
    (G), ``grad_x_s`` and ``grad_w_s``.
    """
    xs, ws = decode(x_s_raw), decode(w_s_raw)
    z = xs @ ws.T
    u = None if x_t_raw is None else decode(x_t_raw) @ decode(w_t_raw).T
    out = forward(z, u, target, ignore_index)
    g = backward(z, u, target, ignore_index, g_ce, g_tvd)
    out["grad"] = g
    out["grad_x_s"] = g @ ws
    out["grad_w_s"] = g.T @ xs
    out["z"], out["u"] = z, u
    return out
