"""Parity of the fused forward + backward entry point (and the valid-row count it
relies on) with the float64 oracle, on the GPU, through the C ABI.

Shapes that take the one-pass kernel (bf16 with a teacher, V % 8 == 0,
16-byte aligned) are compared element by element on small cases that span
several member chunks, ragged last members and the special rows; the other
shapes run the forward and the backward back to back and are checked the same
way.  The full-size workloads are in test_gpu_fullsize.py.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _parity import (DEV, G_REL, G_REL_P16, TOL_TV, announce, bits32, check_forward, check_grad, grad_bits,
                     grad_to_host, tie_info, to_dev)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cross_entropy_tv_amd as lx  # noqa: E402

II = W.IGNORE_INDEX
SENTINEL = 12345.0


def outputs(BT, teacher=True):
    keys = ("ce", "tvd", "lse_s", "lse_t", "sigma") if teacher else ("ce", "lse_s")
    return {k: torch.full((BT,), SENTINEL, dtype=torch.float32, device=DEV) for k in keys}


def run_fused(zs, us, tg, g_ce, g_tvd, grad=None, g_scale=None, ii=II):
    out = outputs(zs.shape[0], us is not None)
    if grad is None:
        grad = torch.full_like(zs, SENTINEL)
    lx.lx_ce_tvd_forward_backward(zs, us, tg, ii, out["ce"], out.get("tvd"), out["lse_s"], out.get("lse_t"),
                                  out.get("sigma"), grad, g_ce, g_tvd, g_scale)
    return out, grad


def host(out):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def one_pass(BT, V, dtype="bf16", teacher=True):
    """True when the shape takes the one-pass kernel (bf16 rows of at least 2048
    classes, V % 8 == 0; it needs a workspace)."""
    dt = lx.LX_BF16 if dtype == "bf16" else lx.LX_F32
    return dtype == "bf16" and V % 8 == 0 and V >= 2048 and \
        lx.lx_ce_tvd_forward_backward_workspace_bytes(BT, V, dt, teacher) > 0


def fused_case(label, z, u, t, g_ce=0.5, g_tvd=1.5, in_place=False):
    announce(f"fused {label}: shape {z.shape} dtype {z.dtype} teacher {u is not None} in_place {in_place}")
    zs, tg = to_dev(z), to_dev(t)
    us = None if u is None else to_dev(u)
    out, g = run_fused(zs, us, tg, g_ce, g_tvd, grad=zs if in_place else None)
    o = host(out)
    check_forward(o, z, u, t, II, label)
    dtype = "bf16" if z.dtype == np.uint16 else "f32"
    rel = G_REL_P16 if (u is not None and one_pass(*z.shape, dtype)) else G_REL
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, g_ce, g_tvd, label, rel=rel, sigma_gpu=o.get("sigma"))
    return o, g


@pytest.mark.parametrize("teacher", [True, False], ids=["ce_tvd", "ce_only"])
@pytest.mark.parametrize("in_place", [False, True], ids=["out_of_place", "in_place"])
@pytest.mark.parametrize("BT,V", [(520, 8200), (600, 20000), (3, 65536), (40, 151936)],
                         ids=["520x8200", "600x20000", "3x65536", "40x151936"])
def test_one_pass_shapes(BT, V, in_place, teacher):
    """One-pass kernel: ragged last member, ignored / identical / uniform rows and rows
    whose logits span far more than the exponent range of fp32 from one reference."""
    assert one_pass(BT, V, teacher=teacher)
    ign = [0, BT - 1] if BT > 4 else [1]
    ident = [2] if BT > 4 else []
    unif = [3] if BT > 4 else []
    z, u, t = W.custom(BT, V, "bf16", seed=BT * 3 + V, scale=3.0, teacher_noise=0.5, ignore_rows=ign,
                       identical_rows=ident, uniform_rows=unif)
    if BT > 8:
        hi = W.bf16_bits_rne(np.array([150.0, 120.0], dtype=np.float32))
        z[5, V // 3] = hi[0]
        u[6, V - 5] = hi[1]
        z[8, 1], u[8, 2] = hi[0], hi[1]
    o, _ = fused_case(f"one-pass {BT}x{V}", z, u if teacher else None, t, in_place=in_place)
    if ident and teacher:
        assert o["tvd"][2] == 0.0 and o["sigma"][2] == 0.0
    if unif:
        assert abs(o["ce"][3] - math.log(V)) <= 1e-4


def reference_trap_rows(BT, V, period, lo, hi, seed):
    """bf16 rows whose groups of 8 columns hold lo where (group mod period) < 256
    and hi elsewhere: with 256 threads a thread's first group is then a lo group
    and its others hi ones, so every thread's sum against its first group's
    maximum is about n e^(hi - lo) (n its hi elements) -- each below fp32's
    limit, their sum over the workgroup far above it unless the kernels redo such
    sums against the true maximum."""
    g = np.arange(V) // 8
    row = np.where(g % period < 256, lo, hi).astype(np.float32)
    rng = np.random.default_rng(seed)
    z = np.repeat(row[None, :], BT, axis=0) + rng.integers(0, 4, (BT, V)).astype(np.float32) * 0.125
    return W.bf16_bits_rne(z)


def test_reference_sums_near_the_fp32_limit():
    """One pass and read-once forward on 128 x 151936 (K = 4 members of 4748 groups):
    each thread's sum against its first group is ~1e37 (82 between lo and hi), the
    sum over a workgroup would overflow fp32; the redo against the true maximum
    keeps every output finite and within tolerance."""
    BT, V = 128, 151936
    z = reference_trap_rows(BT, V, 4748, -57.0, 25.0, seed=3)
    u = reference_trap_rows(BT, V, 4748, -50.0, 24.0, seed=4)
    t = np.random.default_rng(5).integers(0, V, BT).astype(np.int64)
    t[7] = II
    assert one_pass(BT, V)
    fused_case("reference sums near the fp32 limit", z, u, t)
    announce("forward on the same rows")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    out = outputs(BT)
    lx.lx_ce_tvd_forward(zs, us, tg, II, out["ce"], out["tvd"], out["lse_s"], out["lse_t"], out["sigma"])
    check_forward(host(out), z, u, t, II, "forward, reference sums near the fp32 limit")


@pytest.mark.parametrize("V", [38400, 72000], ids=["K1_V38400", "K2_V72000"])
def test_lds_part_of_the_chunk(V):
    """2048 rows make each row a single-digit number of members whose chunks are longer
    than the registers hold, so their tails live in LDS; in place, with special rows,
    compared with the oracle on sampled rows (and row properties on all of them)."""
    BT = 2048
    special = {"ignore_rows": [0, 9, BT - 1], "identical_rows": [2, 10], "uniform_rows": [3]}
    z, u, t = W.custom(BT, V, "bf16", seed=V, scale=3.0, teacher_noise=0.5, **special)
    hi = W.bf16_bits_rne(np.array([150.0, 120.0], dtype=np.float32))
    z[5, V - 7] = hi[0]   # in the LDS part of the last member: far above the thread's reference
    u[6, V - 100] = hi[1]
    rows = np.array(sorted({0, 2, 3, 5, 6, 9, 10, 11, 777, 1500, BT - 2, BT - 1}))
    zr, ur = z[rows].copy(), u[rows].copy()
    announce(f"fused LDS part {BT}x{V} in place")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    out, g = run_fused(zs, us, tg, 0.5, 1.5, grad=zs)
    o = host(out)
    assert o["tvd"][2] == 0.0 and o["sigma"][2] == 0.0 and o["tvd"][10] == 0.0
    assert abs(o["ce"][3] - math.log(V)) <= 1e-4
    valid = t != II
    gs = g.float()
    rs, ra = gs.sum(1).abs().cpu().numpy(), gs.abs().sum(1).cpu().numpy()
    del gs
    assert np.all(rs[valid] <= 2.0 ** -8 * ra[valid] + V * 1e-6 + 1e-9)
    sel = torch.from_numpy(rows).to(DEV)
    check_forward({k: v[rows] for k, v in o.items()}, zr, ur, t[rows], II, f"LDS part {V}")
    check_grad(grad_to_host(g[sel]), grad_bits(g[sel]), zr, ur, t[rows], II, 0.5, 1.5, f"LDS part {V}",
               rel=G_REL_P16, sigma_gpu=o["sigma"][rows])


def test_gradient_precision_at_large_upstream_gradients():
    """Upstream gradients in the thousands lift the bulk of the gradient (|g| ~ p * 3000)
    far above the 1e-6 absolute floor, so the 2^-8 relative bound is what is checked,
    element by element (alpha + beta * s stays far from 0 for these g_ce, g_tvd).  Rows
    whose target holds nearly all the mass check that the target element keeps
    k * g_ce * (p_t - 1) through the cancellation: its bound adds the fp32 error of
    p_t (lse near 24 carries ~1e-6, so 2^-16 relative is ample) times terms of size
    k * g_ce, about 0.06 here, where p_t taken from the fp16 copy would be off by ~1.5."""
    BT, V = 600, 20000
    z, u, t = W.custom(BT, V, "bf16", seed=77, scale=3.0, teacher_noise=0.5, ignore_rows=[4])
    assert one_pass(BT, V)
    peak = W.bf16_bits_rne(np.array([24.0, 17.0], dtype=np.float32))
    for r in range(10, 30):
        z[r, t[r]] = peak[0] if r % 2 else peak[1]
        if r % 3 == 0:
            u[r, t[r]] = peak[1]
    g_ce, g_tvd = 3000.0, 1000.0
    announce("fused, g_ce = 3000, g_tvd = 1000, peaked target rows")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    out, g = run_fused(zs, us, tg, g_ce, g_tvd)
    check_forward(host(out), z, u, t, II, "large upstream gradients")
    ref = oracle.backward(z, u, t, II, g_ce, g_tvd)
    gh = grad_to_host(g)
    valid = t != II
    p, mask, slack = tie_info(z, u, valid)
    tol = 2.0 ** -8 * np.abs(ref) + 1e-6
    tol[valid] += g_tvd * p * (1 + 2.0 ** -8) * (mask + 0.5 * slack[:, None])
    rows = np.nonzero(valid)[0]
    pt = p[np.arange(len(rows)), t[rows]]
    tol[rows, t[rows]] += (2.0 ** -16 * pt + 8 * 2.0 ** -24) * (g_ce + g_tvd)
    err = np.abs(gh - ref)
    tgt = np.zeros((BT, V), dtype=bool)
    tgt[rows, t[rows]] = True
    print(f"worst err/tol: bulk {np.max(err[~tgt] / tol[~tgt]):.3f}, target {np.max(err[tgt] / tol[tgt]):.3f}")
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} elements out of tolerance, first at {np.argwhere(bad)[0]}"
    # the bulk really is above the floor: most elements are held to the relative bound
    assert np.mean(np.abs(ref[valid]) > 2.0 ** 8 * 1e-6) > 0.5
    assert np.all(gh[~valid] == 0)


@pytest.mark.parametrize("k,g_ce,g_tvd,in_place", [(2.0 ** -12, 1.0, -1.0, False), (2.0 ** -12, 1.0, -1.0, True),
                                                   (1.0e-3, 1.0, 1.0, False), (1.0e-3, 0.25, -1.75, True)],
                         ids=["M2e-11", "M2e-11_in_place", "M2e-3", "M2e-3_in_place"])
def test_fp16_p_path_relative_precision(k, g_ce, g_tvd, in_place):
    """With M = k * (|g_ce| + |g_tvd|) <= 2.08e-3 the one-pass kernel forms the gradient
    from an fp16 copy of 2^15 * p.  Checked against the stated bound (2^-8 relative +
    1e-6) and against its own: bf16 rounding plus fp16 rounding, (2^-8 + 2^-10) |g|,
    on a floor of 2^-38 * M (the spacing of fp16 subnormals, scaled) plus the fp32
    rounding of alpha + beta * s and sigma's error, which the 1e-6 floor would
    otherwise hide.  Rows with a few dominant non-target logits put p
    near 1/2 and 1/3 on elements that take the fp16 route (|g| up to ~M/2)."""
    BT, V = 600, 20000
    z, u, t = W.custom(BT, V, "bf16", seed=91, scale=3.0, teacher_noise=0.5, ignore_rows=[4])
    peak = W.bf16_bits_rne(np.array([24.0], dtype=np.float32))[0]
    for r in range(10, 20):
        z[r, t[r]] = peak
    for r in range(20, 40):
        for c in range(2 + r % 2):
            z[r, (t[r] + 1 + 977 * c) % V] = peak
    assert one_pass(BT, V)
    M = k * (abs(g_ce) + abs(g_tvd))
    assert M <= 2.08e-3
    announce(f"fused, fp16-p path: k = {k}, g_ce = {g_ce}, g_tvd = {g_tvd}, in place {in_place}")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    ks = torch.full((1,), k, dtype=torch.float32, device=DEV)
    out, g = run_fused(zs, us, tg, g_ce, g_tvd, grad=zs if in_place else None, g_scale=ks)
    check_forward(host(out), z, u, t, II, "fp16-p path")
    gh, gb = grad_to_host(g), grad_bits(g)
    ref = check_grad(gh, gb, z, u, t, II, k * g_ce, k * g_tvd, "fp16-p path", rel=G_REL_P16)
    valid = t != II
    p, mask, slack = tie_info(z, u, valid)
    tol = (2.0 ** -8 + 2.0 ** -10) * np.abs(ref) + 2.0 ** -38 * M
    # + fp32 rounding of alpha + beta * s, absolute (it may cancel): p * 2^-22 * M, and
    # sigma's own error (its tolerance) carried by beta = k * g_tvd / 2 into every element
    tol[valid] += abs(k * g_tvd) * p * (1 + 2.0 ** -8) * (mask + 0.5 * slack[:, None]) + p * 2.0 ** -22 * M \
        + 0.5 * abs(k * g_tvd) * p * TOL_TV
    rows = np.nonzero(valid)[0]
    tol[rows, t[rows]] += (2.0 ** -16 * p[np.arange(len(rows)), t[rows]] + 8 * 2.0 ** -24) * M
    err = np.abs(gh - ref)
    print(f"worst err/tol {np.max(err / tol):.3f}; largest |g| {np.max(np.abs(ref)):.3g}")
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} elements out of tolerance, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("BT,V,dtype,teacher", [(520, 4099, "bf16", True), (520, 3000, "f32", True),
                                                (6, 50001, "bf16", True), (520, 4099, "bf16", False),
                                                (7, 1024, "f32", False), (515, 1024, "bf16", True)],
                         ids=["bf16_V_not_8", "f32", "split_bf16", "ce_only_V_not_8", "tiny_f32_ce_only",
                              "short_rows"])
def test_two_pass_fallback_shapes(BT, V, dtype, teacher):
    assert not one_pass(BT, V, dtype, teacher)
    ign = [1, BT - 1] if BT > 4 else [1]
    z, u, t = W.custom(BT, V, dtype, seed=BT + 5 * V, scale=3.0, teacher_noise=0.5, ignore_rows=ign)
    fused_case(f"fallback {BT}x{V} {dtype}", z, u if teacher else None, t, g_ce=0.75, g_tvd=-0.5)


def test_unaligned_gradient_takes_the_two_pass_path():
    z, u, t = W.custom(520, 8200, "bf16", seed=3, scale=2.0, teacher_noise=0.5, ignore_rows=[4])
    announce("fused with a gradient 2 bytes off a 16-byte boundary")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    base = torch.zeros(520 * 8200 + 16, dtype=torch.bfloat16, device=DEV)
    g = base[1:1 + 520 * 8200].view(520, 8200)
    out, g = run_fused(zs, us, tg, 0.5, 1.5, grad=g)
    check_forward(host(out), z, u, t, II, "unaligned grad")
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, 0.5, 1.5, "unaligned grad", rel=G_REL)


def test_identical_rows_give_exactly_zero_total_variation():
    z, _, t = W.custom(530, 16384, "bf16", seed=21, scale=3.0, ignore_rows=[7])
    announce("fused, teacher == student: tvd, sigma and the tvd gradient exactly 0")
    zs, tg = to_dev(z), to_dev(t)
    out, g = run_fused(zs, zs.clone(), tg, 0.0, 1.0)
    o = host(out)
    assert np.all(o["tvd"] == 0.0) and np.all(o["sigma"] == 0.0)
    assert torch.count_nonzero(g.view(torch.int16)) == 0


def test_out_of_range_target_poisons_its_row_only():
    z, u, t = W.custom(520, 8200, "bf16", seed=8, scale=2.0, teacher_noise=0.5)
    t[5], t[9] = 8200, -3
    announce("fused, targets out of range on rows 5 and 9")
    out, g = run_fused(to_dev(z), to_dev(u), to_dev(t), 0.5, 0.5)
    o = host(out)
    assert np.isnan(o["ce"][5]) and np.isnan(o["ce"][9])
    gf = g.float()
    assert bool(torch.isnan(gf[5]).all()) and bool(torch.isnan(gf[9]).all())
    ok = np.ones(520, bool)
    ok[[5, 9]] = False
    assert np.all(np.isfinite(o["ce"][ok])) and bool(torch.isfinite(gf[torch.from_numpy(ok).to(DEV)]).all())
    for k in ("tvd", "lse_s", "lse_t", "sigma"):
        assert np.all(np.isfinite(o[k])), k


def test_deterministic_and_close_to_the_two_pass_result():
    z, u, t = W.custom(600, 20000, "bf16", seed=44, scale=2.5, teacher_noise=0.5, ignore_rows=[3])
    announce("fused: 3 repeats bitwise; vs forward + backward within the tolerances")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    runs = []
    for _ in range(3):
        out, g = run_fused(zs, us, tg, 0.5, 1.5)
        runs.append((host(out), g.view(torch.int16).cpu()))
    for o, gb in runs[1:]:
        for k in o:
            assert np.array_equal(bits32(o[k]), bits32(runs[0][0][k])), k
        assert torch.equal(gb, runs[0][1])
    sep = outputs(600)
    lx.lx_ce_tvd_forward(zs, us, tg, II, sep["ce"], sep["tvd"], sep["lse_s"], sep["lse_t"], sep["sigma"])
    g2 = torch.empty_like(zs)
    lx.lx_ce_tvd_backward(g2, zs, us, tg, II, sep["lse_s"], sep["lse_t"], sep["sigma"], 0.5, 1.5)
    s = host(sep)
    for k, tol in (("ce", 2e-4), ("lse_s", 2e-4), ("lse_t", 2e-4), ("tvd", 2e-5), ("sigma", 2e-5)):
        assert np.max(np.abs(s[k] - runs[0][0][k])) <= tol, k
    # gradients: both passes round once to bf16; elements at a near tie of p and q may
    # take different sign branches in the two kernels (each is exempt against the
    # oracle), which moves them by up to |g_tvd| * p
    g1 = runs[0][1].view(torch.bfloat16).float().numpy().astype(np.float64)
    d = np.abs(g2.float().cpu().numpy() - g1)
    valid = t != II
    p, mask, slack = tie_info(z, u, valid)
    tol = 2.0 ** -7 * np.abs(g1) + 2e-6
    tol[valid] += 1.5 * p * (1 + 2.0 ** -7) * (mask + slack[:, None])
    assert np.all(d <= tol), f"{np.sum(d > tol)} gradient elements differ"


def test_count_valid():
    t = np.full(1000, II, dtype=np.int64)
    t[::3] = 5
    tg = to_dev(t)
    n = torch.zeros(1, dtype=torch.int64, device=DEV)
    inv = torch.zeros(1, dtype=torch.float32, device=DEV)
    lx.lx_ce_tvd_count_valid(tg, II, n, inv)
    assert int(n.item()) == 334 and inv.item() == np.float32(1.0 / 334)
    lx.lx_ce_tvd_count_valid(torch.full((10,), II, dtype=torch.int64, device=DEV), II, n, inv)
    assert int(n.item()) == 0 and inv.item() == 0.0
