"""Pins of the float64 oracle to things other than itself.

Each check takes an oracle module (``forward``, ``backward``, ``reduce_mean``)
and raises AssertionError when it disagrees with an independent source:

* ``brute_force_decimal``: 50-digit ``decimal`` arithmetic on tiny rows, the
  loss straight from its definition (no max shift, no stored lse) and the
  gradient by central differences of that loss;
* ``closed_forms``: uniform rows (ce = log V), V = 1, V = 2 (sigmoid/tanh
  forms), identical rows, disjoint spikes;
* ``library``: CE-only against torch.nn.functional.cross_entropy and
  scipy.special.logsumexp; TVD against scipy's softmax and cityblock distance;
  the full gradient against torch float64 autograd of
  g_ce*CE + g_tvd*0.5*|softmax(z) - softmax(u)|_1 (autograd of abs uses 0 at 0);
* ``invariants``: bounds, TVD = 1 - sum min(p, q), symmetry, zero gradient row
  sums, shift invariance, permutation equivariance, linearity in the upstream
  gradients;
* ``ignore_rules``: ignored rows all +0.0, precedence of the ignore index,
  out-of-range targets raise; mean reduction including the all-ignored case;
* ``row_weights``: per-row upstream gradients (an unreduced loss) against
  torch float64 autograd of sum_r w_ce[r] * CE_r + w_tvd[r] * TVD_r;
* ``sign_branches``: results for an explicit sign vector (a near-tie branch)
  against torch float64 autograd of the loss with |p - q| replaced by
  s * (p - q), sigma recovered from that gradient;
* ``linear_chain_rule``: the lm_head variant against torch float64 autograd
  through x @ w.T and central differences on single entries of x and w;
* ``decoding``: every finite bf16 and binary16 bit pattern decodes to the value
  its sign, exponent and fraction fields define (IEEE 754 binary16; bf16 as
  the upper half of binary32), built here with math.ldexp.

The mutation test plants mistakes in copies of the oracle and checks that at
least one of these fails for each.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np

TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert a.shape == b.shape and err <= tol, f"{what}: max abs err {err} > {tol}"


# ------------------------------------------------------------ brute force in Decimal

def _dec_loss_parts(z, u, t):
    """(ce, tvd, sigma, lse_s, lse_t) of one row straight from the definitions."""
    ez = [x.exp() for x in z]
    eu = [x.exp() for x in u]
    sz, su = sum(ez), sum(eu)
    p = [e / sz for e in ez]
    q = [e / su for e in eu]
    lse_s, lse_t = sz.ln(), su.ln()
    ce = lse_s - z[t]
    tvd = sum(abs(a - b) for a, b in zip(p, q)) / 2
    sigma = Decimal(0)
    for a, b in zip(p, q):
        if a > b:
            sigma += a
        elif a < b:
            sigma -= a
    return ce, tvd, sigma, lse_s, lse_t


def brute_force_decimal(orc, seed=7):
    getcontext().prec = 50
    rng = np.random.default_rng(seed)
    h = Decimal("1e-22")
    for V in (1, 2, 3, 5, 8):
        R = 3
        z = rng.normal(0, 2.0, size=(R, V))
        u = rng.normal(0, 2.0, size=(R, V))
        t = rng.integers(0, V, size=R)
        g_ce, g_tvd = 0.375, 1.25
        fw = orc.forward(z, u, t, -100)
        gr = orc.backward(z, u, t, -100, g_ce, g_tvd)
        for r in range(R):
            zd = [Decimal(float(x)) for x in z[r]]
            ud = [Decimal(float(x)) for x in u[r]]
            ce, tvd, sig, ls, lt = _dec_loss_parts(zd, ud, int(t[r]))
            for k, ref in (("ce", ce), ("tvd", tvd), ("sigma", sig), ("lse_s", ls), ("lse_t", lt)):
                _close(fw[k][r], float(ref), what=f"decimal {k} V={V} row {r}")
            for v in range(V):
                zp = list(zd); zp[v] += h
                zm = list(zd); zm[v] -= h
                cp, tp, *_ = _dec_loss_parts(zp, ud, int(t[r]))
                cm, tm, *_ = _dec_loss_parts(zm, ud, int(t[r]))
                fd = (Decimal(g_ce) * (cp - cm) + Decimal(g_tvd) * (tp - tm)) / (2 * h)
                _close(gr[r, v], float(fd), tol=1e-12, what=f"decimal grad V={V} row {r} v {v}")


# ------------------------------------------------------------ closed forms

def closed_forms(orc):
    # uniform student row: ce = log V, lse = c + log V, for any target
    for V, c in ((1, 0.0), (7, -3.25), (1024, 2.5), (151936, 0.875)):
        z = np.full((1, V), c)
        u = np.zeros((1, V))
        fw = orc.forward(z, u, [V - 1], -100)
        _close(fw["ce"], [math.log(V)], tol=1e-9, what="uniform ce")
        _close(fw["lse_s"], [c + math.log(V)], tol=1e-9, what="uniform lse")
        # teacher uniform too: both softmaxes are 1/V, no total variation
        _close(fw["tvd"], [0.0], tol=1e-12, what="uniform tvd")
    # V = 1: softmax is 1, every loss and gradient is 0
    z = np.array([[3.0], [-7.0]])
    u = np.array([[1.0], [5.0]])
    fw = orc.forward(z, u, [0, 0], -100)
    for k in ("ce", "tvd", "sigma"):
        _close(fw[k], [0.0, 0.0], what=f"V=1 {k}")
    _close(orc.backward(z, u, [0, 0], -100, 0.7, 1.3), np.zeros((2, 1)), what="V=1 grad")
    # V = 2: p1 = expit(z1 - z0); tvd = |expit(dz) - expit(du)|;
    # sigma = sign(p1 - q1) * (p1 - p0) = sign(p1 - q1) * tanh(dz / 2)
    rng = np.random.default_rng(3)
    z = rng.normal(0, 3, size=(64, 2))
    u = rng.normal(0, 3, size=(64, 2))
    fw = orc.forward(z, u, np.zeros(64, dtype=np.int64), -100)
    dz, du = z[:, 1] - z[:, 0], u[:, 1] - u[:, 0]
    p1 = 1.0 / (1.0 + np.exp(-dz))
    q1 = 1.0 / (1.0 + np.exp(-du))
    _close(fw["tvd"], np.abs(p1 - q1), what="V=2 tvd")
    _close(fw["sigma"], np.sign(p1 - q1) * np.tanh(dz / 2), what="V=2 sigma")
    _close(fw["ce"], np.log1p(np.exp(dz)), tol=1e-9, what="V=2 ce (target 0)")
    # identical rows: tvd = sigma = 0 and the total-variation gradient vanishes exactly
    z = rng.normal(0, 3, size=(4, 33))
    fw = orc.forward(z, z.copy(), [0, 5, 9, 32], -100)
    assert np.all(fw["tvd"] == 0.0) and np.all(fw["sigma"] == 0.0), "identical rows: tvd/sigma not exactly 0"
    g = orc.backward(z, z.copy(), [0, 5, 9, 32], -100, 0.0, 1.0)
    assert np.all(g == 0.0), "identical rows: tvd gradient not exactly 0"
    # disjoint spikes: p and q put almost all mass on different classes
    V = 50
    z = np.zeros((1, V)); z[0, 3] = 60.0
    u = np.zeros((1, V)); u[0, 17] = 60.0
    fw = orc.forward(z, u, [3], -100)
    assert fw["tvd"][0] > 1.0 - 1e-12, "disjoint spikes: tvd should be ~1"
    assert fw["sigma"][0] > 1.0 - 1e-12, "disjoint spikes: sigma should be ~1"


# ------------------------------------------------------------ libraries

def library(orc):
    import scipy.special as sp
    from scipy.spatial.distance import cityblock
    import torch

    rng = np.random.default_rng(11)
    R, V = 6, 37
    z = rng.normal(0, 2.5, size=(R, V))
    u = rng.normal(0, 2.5, size=(R, V))
    t = rng.integers(0, V, size=R)
    t[2] = -100
    # CE-only forward vs torch's cross_entropy and scipy's logsumexp
    fw = orc.forward(z, None, t, -100)
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(z), torch.from_numpy(t),
                                            reduction="none", ignore_index=-100).numpy()
    _close(fw["ce"], ref, what="ce vs torch cross_entropy")
    valid = t != -100
    _close(fw["lse_s"][valid], sp.logsumexp(z[valid], axis=1), what="lse vs scipy logsumexp")
    # TVD vs half the L1 (cityblock) distance of scipy softmaxes
    fw2 = orc.forward(z, u, t, -100)
    for r in np.nonzero(valid)[0]:
        _close(fw2["tvd"][r], 0.5 * cityblock(sp.softmax(z[r]), sp.softmax(u[r])), what="tvd vs scipy")
        _close(fw2["lse_t"][r], sp.logsumexp(u[r]), what="lse_t vs scipy")
    # gradients vs torch float64 autograd
    for g_ce, g_tvd in ((1.0, 1.0), (0.25, -2.0), (0.0, 1.0), (1.0, 0.0)):
        zt = torch.from_numpy(z).requires_grad_(True)
        ut = torch.from_numpy(u)
        tt = torch.from_numpy(t)
        ce = torch.nn.functional.cross_entropy(zt, tt, reduction="none", ignore_index=-100)
        tv = 0.5 * (torch.softmax(zt, -1) - torch.softmax(ut, -1)).abs().sum(-1)
        loss = (g_ce * ce + g_tvd * tv * torch.from_numpy(valid)).sum()
        loss.backward()
        _close(orc.backward(z, u, t, -100, g_ce, g_tvd), zt.grad.numpy(), what=f"grad vs autograd {g_ce},{g_tvd}")
        zt2 = torch.from_numpy(z).requires_grad_(True)
        (g_ce * torch.nn.functional.cross_entropy(zt2, tt, reduction="sum", ignore_index=-100)).backward()
        _close(orc.backward(z, None, t, -100, g_ce, g_tvd), zt2.grad.numpy(), what="CE-only grad vs autograd")


# ------------------------------------------------------------ invariants

def invariants(orc):
    rng = np.random.default_rng(5)
    for V, scale in ((2, 1.0), (9, 4.0), (100, 2.0), (4096, 3.0)):
        R = 8
        z = rng.normal(0, scale, size=(R, V))
        u = rng.normal(0, scale, size=(R, V))
        t = rng.integers(0, V, size=R)
        fw = orc.forward(z, u, t, -100)
        assert np.all(fw["ce"] >= 0), "ce >= 0"
        assert np.all((fw["tvd"] >= 0) & (fw["tvd"] <= 1)), "0 <= tvd <= 1"
        assert np.all(np.abs(fw["sigma"]) <= 1 + 1e-12), "|sigma| <= 1"
        mz = z.max(1)
        assert np.all(mz <= fw["lse_s"] + 1e-12) and np.all(fw["lse_s"] <= mz + math.log(V) + 1e-12), "lse bounds"
        # tvd = 1 - sum min(p, q) = sum max(p - q, 0), from softmaxes computed here
        p = np.exp(z - z.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
        q = np.exp(u - u.max(1, keepdims=True)); q /= q.sum(1, keepdims=True)
        _close(fw["tvd"], 1 - np.minimum(p, q).sum(1), tol=1e-12, what="tvd = 1 - sum min")
        _close(fw["tvd"], np.maximum(p - q, 0).sum(1), tol=1e-12, what="tvd = sum (p-q)+")
        # sigma = sum_{p>q} p - sum_{p<q} p
        _close(fw["sigma"], np.where(p > q, p, 0).sum(1) - np.where(p < q, p, 0).sum(1), what="sigma split")
        # symmetry of tvd
        _close(orc.forward(u, z, t, -100)["tvd"], fw["tvd"], what="tvd symmetric")
        # gradient rows sum to zero
        g = orc.backward(z, u, t, -100, 0.8, 1.7)
        assert np.max(np.abs(g.sum(1))) < 1e-12, "grad row sum"
        # shift invariance (z + c, u + c'): lse shifts, ce/tvd/sigma/grad unchanged
        c1, c2 = 3.5, -11.0
        fs = orc.forward(z + c1, u + c2, t, -100)
        _close(fs["lse_s"], fw["lse_s"] + c1, tol=1e-11, what="lse shift")
        for k in ("ce", "tvd", "sigma"):
            _close(fs[k], fw[k], tol=1e-11, what=f"{k} shift invariance")
        _close(orc.backward(z + c1, u + c2, t, -100, 0.8, 1.7), g, tol=1e-12, what="grad shift invariance")
        # permutation equivariance of the vocabulary (target remapped)
        perm = rng.permutation(V)
        inv = np.argsort(perm)
        fp = orc.forward(z[:, perm], u[:, perm], inv[t], -100)
        for k in ("ce", "tvd", "sigma", "lse_s", "lse_t"):
            _close(fp[k], fw[k], tol=1e-11, what=f"{k} permutation")
        _close(orc.backward(z[:, perm], u[:, perm], inv[t], -100, 0.8, 1.7), g[:, perm], what="grad permutation")
        # linearity in (g_ce, g_tvd)
        a = orc.backward(z, u, t, -100, 1.0, 0.0)
        b = orc.backward(z, u, t, -100, 0.0, 1.0)
        _close(g, 0.8 * a + 1.7 * b, what="grad linearity")
        # CE part of the gradient: exactly one negative entry per row, at the target
        neg = a < 0
        assert np.all(neg.sum(1) == 1) and np.all(neg[np.arange(R), t]), "ce grad sign pattern"


# ------------------------------------------------------------ ignore index and reduction

def ignore_rules(orc):
    rng = np.random.default_rng(9)
    R, V = 5, 16
    z = rng.normal(0, 2, size=(R, V))
    u = rng.normal(0, 2, size=(R, V))
    t = np.array([3, -100, 15, -100, 0])
    fw = orc.forward(z, u, t, -100)
    for k in ("ce", "tvd", "lse_s", "lse_t", "sigma"):
        assert np.all(fw[k][[1, 3]] == 0.0) and not np.any(np.signbit(fw[k][[1, 3]])), f"ignored {k} must be +0.0"
    g = orc.backward(z, u, t, -100, 1.0, 1.0)
    assert np.all(g[[1, 3]] == 0.0) and not np.any(np.signbit(g[[1, 3]])), "ignored grad rows must be +0.0"
    # an ignore index inside [0, V) takes precedence over the class with that id
    t2 = np.array([3, 3, 5, 7, 3])
    fw2 = orc.forward(z, u, t2, 3)
    assert np.all(fw2["ce"][[0, 1, 4]] == 0.0) and np.all(fw2["ce"][[2, 3]] > 0), "ignore precedence"
    # out-of-range targets are a precondition violation
    for bad in (V, -1, 10**12):
        try:
            orc.forward(z, u, np.array([0, 1, bad, 2, 3]), -100)
        except ValueError:
            pass
        else:
            raise AssertionError(f"target {bad} should raise")
    # mean over valid rows
    mce, mtv, n = orc.reduce_mean(fw["ce"], fw["tvd"], t, -100)
    assert n == 3
    _close(mce, fw["ce"][[0, 2, 4]].mean(), what="mean ce")
    _close(mtv, fw["tvd"][[0, 2, 4]].mean(), what="mean tvd")
    mce, mtv, n = orc.reduce_mean(np.zeros(3), np.zeros(3), np.full(3, -100), -100)
    assert n == 0 and math.isnan(mce) and math.isnan(mtv), "all-ignored mean is NaN"
    # -inf logits present in both rows at the same classes: same result as dropping those classes
    zi, ui = z.copy(), u.copy()
    keep = np.ones(V, dtype=bool); keep[[2, 9, 11]] = False
    zi[:, ~keep] = -np.inf
    ui[:, ~keep] = -np.inf
    tt = np.array([0, 1, 3, 4, 5])
    remap = np.cumsum(keep) - 1
    fi = orc.forward(zi, ui, tt, -100)
    fr = orc.forward(z[:, keep], u[:, keep], remap[tt], -100)
    for k in ("ce", "tvd", "sigma", "lse_s", "lse_t"):
        _close(fi[k], fr[k], what=f"-inf classes {k}")
    gi = orc.backward(zi, ui, tt, -100, 1.0, 1.0)
    assert np.all(gi[:, ~keep] == 0.0)
    _close(gi[:, keep], orc.backward(z[:, keep], u[:, keep], remap[tt], -100, 1.0, 1.0), what="-inf classes grad")


# ------------------------------------------------------------ per-row upstream gradients

def row_weights(orc):
    import torch

    rng = np.random.default_rng(13)
    R, V = 7, 29
    z = rng.normal(0, 2.5, size=(R, V))
    u = rng.normal(0, 2.5, size=(R, V))
    t = rng.integers(0, V, size=R)
    t[4] = -100
    valid = t != -100
    w_ce = rng.normal(0, 1.0, size=R)
    w_tvd = rng.normal(0, 1.0, size=R)
    zt = torch.from_numpy(z).requires_grad_(True)
    tt = torch.from_numpy(t)
    ce = torch.nn.functional.cross_entropy(zt, tt, reduction="none", ignore_index=-100)
    tv = 0.5 * (torch.softmax(zt, -1) - torch.softmax(torch.from_numpy(u), -1)).abs().sum(-1)
    m = torch.from_numpy(valid.astype(np.float64))
    ((torch.from_numpy(w_ce) * ce + torch.from_numpy(w_tvd) * tv * m).sum()).backward()
    _close(orc.backward(z, u, t, -100, w_ce, w_tvd), zt.grad.numpy(), what="per-row weights vs autograd")
    zt2 = torch.from_numpy(z).requires_grad_(True)
    ce2 = torch.nn.functional.cross_entropy(zt2, tt, reduction="none", ignore_index=-100)
    (torch.from_numpy(w_ce) * ce2).sum().backward()
    _close(orc.backward(z, None, t, -100, w_ce, w_tvd), zt2.grad.numpy(), what="CE-only per-row weights")
    # equal per-row weights are the scalar case
    _close(orc.backward(z, u, t, -100, np.full(R, 0.3), np.full(R, -1.1)),
           orc.backward(z, u, t, -100, 0.3, -1.1), what="constant row weights")


# ------------------------------------------------------------ explicit sign branches

def sign_branches(orc):
    """Results for a given sign vector s (the branch of |p - q| a kernel took at
    near ties): the loss g_ce*CE + g_tvd*0.5*sum_v s_v (p_v - q_v) has the
    gradient the oracle gives for that branch (torch float64 autograd; s is a
    constant), sigma of the branch follows from that gradient (with g_ce = 0 and
    g_tvd = 1 every element is 0.5 p_v (s_v - sigma)), tvd does not move, and
    the true signs reproduce the default results."""
    import torch

    rng = np.random.default_rng(17)
    R, V = 5, 13
    z = rng.normal(0, 2.0, size=(R, V))
    u = rng.normal(0, 2.0, size=(R, V))
    t = rng.integers(0, V, size=R)
    t[3] = -100
    valid = t != -100
    s = rng.integers(-1, 2, size=(R, V)).astype(np.float64)
    for g_ce, g_tvd in ((0.6, 1.4), (0.0, 1.0)):
        zt = torch.from_numpy(z).requires_grad_(True)
        ce = torch.nn.functional.cross_entropy(zt, torch.from_numpy(t), reduction="none", ignore_index=-100)
        tv = 0.5 * (torch.from_numpy(s) * (torch.softmax(zt, -1) - torch.softmax(torch.from_numpy(u), -1))).sum(-1)
        (g_ce * ce + g_tvd * tv * torch.from_numpy(valid.astype(np.float64))).sum().backward()
        g = orc.backward(z, u, t, -100, g_ce, g_tvd, signs=s)
        _close(g, zt.grad.numpy(), what=f"branch gradient vs autograd {g_ce},{g_tvd}")
    # sigma of the branch from the autograd gradient of the total-variation part alone
    pz = np.exp(z - z.max(1, keepdims=True))
    pz /= pz.sum(1, keepdims=True)
    gt = zt.grad.numpy()
    fw = orc.forward(z, u, t, -100, signs=s)
    for r in np.nonzero(valid)[0]:
        v = int(np.argmax(pz[r]))
        _close(fw["sigma"][r], s[r, v] - 2.0 * gt[r, v] / pz[r, v], tol=1e-10, what="branch sigma from gradient")
    _close(fw["tvd"], orc.forward(z, u, t, -100)["tvd"], what="tvd independent of the branch")
    # the true signs (softmaxes computed here) give the default results
    pu = np.exp(u - u.max(1, keepdims=True))
    pu /= pu.sum(1, keepdims=True)
    st = np.sign(pz - pu)
    _close(orc.forward(z, u, t, -100, signs=st)["sigma"], orc.forward(z, u, t, -100)["sigma"], what="true signs")
    _close(orc.backward(z, u, t, -100, 0.3, 0.9, signs=st), orc.backward(z, u, t, -100, 0.3, 0.9),
           what="true-sign gradient")


# ------------------------------------------------------------ logits decoding

def _ieee_value(bits: int, exp_bits: int, frac_bits: int) -> float:
    """Value of a finite IEEE-style bit pattern from its fields."""
    sign = -1.0 if bits >> (exp_bits + frac_bits) else 1.0
    e = (bits >> frac_bits) & ((1 << exp_bits) - 1)
    f = bits & ((1 << frac_bits) - 1)
    bias = (1 << (exp_bits - 1)) - 1
    if e == 0:
        return sign * math.ldexp(f, 1 - bias - frac_bits)
    return sign * math.ldexp((1 << frac_bits) + f, e - bias - frac_bits)


def decoding(orc):
    pats = np.arange(1 << 16, dtype=np.uint32)
    for name, exp_bits, frac_bits, raw in (
            ("bf16", 8, 7, pats.astype(np.uint16)),
            ("binary16", 5, 10, pats.astype(np.uint16).view(np.float16))):
        finite = ((pats >> frac_bits) & ((1 << exp_bits) - 1)) != (1 << exp_bits) - 1
        got = orc.decode(raw[finite])
        ref = np.array([_ieee_value(int(b), exp_bits, frac_bits) for b in pats[finite]])
        assert got.dtype == np.float64 and np.array_equal(got, ref), f"{name} decoding"


# ------------------------------------------------------------ lm_head product + loss

def linear_chain_rule(orc):
    """The loss over lm_head logits and its gradients w.r.t. the student's hidden
    states and weight, against torch float64 autograd through x @ w.T, and
    central differences of the float64 loss on single entries."""
    import torch

    rng = np.random.default_rng(21)
    BT, Hs, Ht, V = 6, 5, 7, 11
    xs, ws = rng.normal(0, 1.5, (BT, Hs)), rng.normal(0, 1.0, (V, Hs))
    xt, wt = rng.normal(0, 1.5, (BT, Ht)), rng.normal(0, 1.0, (V, Ht))
    t = rng.integers(0, V, BT)
    t[2] = -100
    valid = torch.from_numpy((t != -100).astype(np.float64))
    tt = torch.from_numpy(t)
    for teacher in (True, False):
        g_ce, g_tvd = 0.7, -1.3
        out = orc.linear_forward_backward(xs, ws, xt if teacher else None, wt if teacher else None, t, -100,
                                          g_ce, g_tvd)
        X = torch.from_numpy(xs).requires_grad_(True)
        W = torch.from_numpy(ws).requires_grad_(True)
        z = X @ W.T
        ce = torch.nn.functional.cross_entropy(z, tt, reduction="none", ignore_index=-100)
        loss = g_ce * ce.sum()
        if teacher:
            u = torch.from_numpy(xt) @ torch.from_numpy(wt).T
            tv = 0.5 * (torch.softmax(z, -1) - torch.softmax(u, -1)).abs().sum(-1) * valid
            loss = loss + g_tvd * tv.sum()
            _close(out["tvd"], tv.detach().numpy(), what="linear tvd vs autograd forward")
        loss.backward()
        _close(out["ce"], ce.detach().numpy(), what="linear ce vs torch")
        _close(out["grad_x_s"], X.grad.numpy(), what=f"grad_x_s vs autograd (teacher {teacher})")
        _close(out["grad_w_s"], W.grad.numpy(), what=f"grad_w_s vs autograd (teacher {teacher})")

    # central differences of the loss on a few single entries of x_s and w_s
    def loss_of(xs_, ws_):
        fw = orc.forward(xs_ @ ws_.T, xt @ wt.T, t, -100)
        return 0.7 * fw["ce"].sum() + 1.1 * fw["tvd"].sum()

    out = orc.linear_forward_backward(xs, ws, xt, wt, t, -100, 0.7, 1.1)
    h = 1e-6
    for (b, k) in ((0, 0), (3, 4), (5, 2)):
        xp, xm = xs.copy(), xs.copy()
        xp[b, k] += h
        xm[b, k] -= h
        _close(out["grad_x_s"][b, k], (loss_of(xp, ws) - loss_of(xm, ws)) / (2 * h), tol=1e-6,
               what=f"grad_x_s[{b},{k}] central difference")
    for (v, k) in ((0, 1), (7, 3), (10, 4)):
        wp, wm = ws.copy(), ws.copy()
        wp[v, k] += h
        wm[v, k] -= h
        _close(out["grad_w_s"][v, k], (loss_of(xs, wp) - loss_of(xs, wm)) / (2 * h), tol=1e-6,
               what=f"grad_w_s[{v},{k}] central difference")


ALL_PINS = (brute_force_decimal, closed_forms, library, invariants, ignore_rules, row_weights, sign_branches,
            decoding, linear_chain_rule)
