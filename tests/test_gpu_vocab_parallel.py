"""Parity of the vocabulary-parallel entry points with the float64 oracle, on the GPU,
through the C ABI.

The vocabulary of every row is cut into column shards, as a sharded lm_head
would leave it, each shard a contiguous (BT, V_shard) array.  Every shard runs
its step-1 partials (lx_ce_tvd_vp_stats); the partials are gathered in shard
order and merged (lx_ce_tvd_vp_merge_stats) into ce, lse_s and lse_t; every
shard then runs its step-2 partials (lx_ce_tvd_vp_tv) from the merged lse; a
second merge (lx_ce_tvd_vp_merge_tv) gives tvd and sigma; and every shard runs
its backward (lx_ce_tvd_backward_shard).  The merged outputs and the gradient
columns put back together are compared with the oracle on the whole rows, to the
same tolerances as the single-device entry points.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads as W
from _parity import DEV, announce, bits32, check_forward, check_grad, grad_bits, grad_to_host, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cross_entropy_tv_amd as lx  # noqa: E402

II = W.IGNORE_INDEX


def shard_bounds(V, widths):
    assert sum(widths) == V
    b = np.concatenate([[0], np.cumsum(widths)])
    return [(int(b[i]), int(b[i + 1])) for i in range(len(widths))]


def run_vp(z, u, t, bounds, g_ce, g_tvd, in_place=False, g_scale=None):
    """The whole vocabulary-parallel protocol on one device.  Returns (outputs, grad)."""
    BT, V = z.shape
    teacher = u is not None
    tg = to_dev(t)
    P = lx.lx_vp_stats_floats(teacher)
    zs = [to_dev(np.ascontiguousarray(z[:, a:b])) for a, b in bounds]
    us = [to_dev(np.ascontiguousarray(u[:, a:b])) for a, b in bounds] if teacher else [None] * len(bounds)
    stats = torch.full((len(bounds), BT, P), 777.0, dtype=torch.float32, device=DEV)
    for n, (a, _) in enumerate(bounds):
        lx.lx_ce_tvd_vp_stats(zs[n], us[n], tg, a, II, stats[n])
    f = lambda: torch.full((BT,), 12345.0, dtype=torch.float32, device=DEV)
    out = {"ce": f(), "lse_s": f()}
    if teacher:
        out.update(lse_t=f(), tvd=f(), sigma=f())
    lx.lx_ce_tvd_vp_merge_stats(stats, tg, V, II, out["ce"], out["lse_s"], out.get("lse_t"))
    if teacher:
        tv = torch.full((len(bounds), BT, 2), 777.0, dtype=torch.float32, device=DEV)
        for n in range(len(bounds)):
            lx.lx_ce_tvd_vp_tv(zs[n], us[n], tg, II, out["lse_s"], out["lse_t"], tv[n])
        lx.lx_ce_tvd_vp_merge_tv(tv, tg, II, out["tvd"], out["sigma"])
    grads = []
    for n, (a, _) in enumerate(bounds):
        g = zs[n] if in_place else torch.full_like(zs[n], 3.0)
        lx.lx_ce_tvd_backward_shard(g, zs[n], us[n], tg, a, V, II, out["lse_s"], out.get("lse_t"),
                                    out.get("sigma"), g_ce, g_tvd, g_scale)
        grads.append(g)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, torch.cat(grads, dim=1)


CASES = [
    # (BT, V, shard widths, dtype, teacher)
    (520, 8200, [2050, 2050, 2050, 2050], "bf16", True),      # widths not a multiple of 8
    (520, 8200, [4096, 4104], "bf16", True),
    (300, 30000, [3750] * 8, "bf16", True),
    (64, 10007, [1, 5000, 5006], "bf16", True),                # a one-column shard
    (260, 6000, [1999, 2001, 2000], "f32", True),
    (520, 8200, [2050, 2050, 2050, 2050], "bf16", False),
    (260, 6000, [2999, 3001], "f32", False),
    (8, 1024, [1024], "f32", True),                            # one shard: the plain loss
    (64, 50000, [24996, 25004], "bf16", True),                 # shards over one pass of held units (2560 x 8)
    (32, 31000, [31000], "f32", True),                         # fp32: 10240 logits per pass, 4 passes
]


@pytest.mark.parametrize("in_place", [False, True], ids=["out_of_place", "in_place"])
@pytest.mark.parametrize("BT,V,widths,dtype,teacher", CASES,
                         ids=[f"{c[0]}x{c[1]}_{len(c[2])}shards_{c[3]}_{'tvd' if c[4] else 'ce'}" for c in CASES])
def test_vocab_parallel_matches_the_oracle(BT, V, widths, dtype, teacher, in_place):
    bounds = shard_bounds(V, widths)
    ign = [0, BT - 1] if BT > 4 else [3]
    special = {"identical_rows": [2], "uniform_rows": [1]} if BT > 4 else {}
    z, u, t = W.custom(BT, V, dtype, seed=BT + 7 * V + len(widths), scale=3.0, teacher_noise=0.5,
                       ignore_rows=ign, **special)
    # targets on the first and last column of every shard, and in the one-column shard
    for k, (a, b) in enumerate(bounds):
        for j, c in enumerate((a, b - 1)):
            r = 4 + 2 * k + j
            if r < BT and r not in ign:
                t[r] = c
    announce(f"vocab-parallel {BT}x{V} shards {widths} {dtype} teacher={teacher} in_place={in_place}")
    o, g = run_vp(z, u if teacher else None, t, bounds, 0.5, 1.5, in_place=in_place)
    check_forward(o, z, u if teacher else None, t, II, "vocab-parallel")
    check_grad(grad_to_host(g), grad_bits(g), z, u if teacher else None, t, II, 0.5, 1.5, "vocab-parallel")
    if teacher and BT > 4:
        assert o["tvd"][2] == 0.0 and o["sigma"][2] == 0.0          # identical rows: exact zero
    if BT > 4:
        assert abs(o["ce"][1] - math.log(V)) <= 1e-4                 # uniform row


def test_vocab_parallel_is_deterministic_and_close_to_the_whole_rows():
    BT, V = 400, 20000
    z, u, t = W.custom(BT, V, "bf16", seed=5, scale=2.5, teacher_noise=0.5, ignore_rows=[7])
    bounds = shard_bounds(V, [2500] * 8)
    announce("vocab-parallel: bitwise repeatable; against lx_ce_tvd_forward on whole rows")
    runs = [run_vp(z, u, t, bounds, 0.5, 1.5) for _ in range(2)]
    for k in runs[0][0]:
        assert np.array_equal(bits32(runs[0][0][k]), bits32(runs[1][0][k])), k
    assert torch.equal(runs[0][1].view(torch.int16), runs[1][1].view(torch.int16))
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    f = lambda: torch.empty(BT, dtype=torch.float32, device=DEV)
    whole = {k: f() for k in ("ce", "tvd", "lse_s", "lse_t", "sigma")}
    lx.lx_ce_tvd_forward(zs, us, tg, II, whole["ce"], whole["tvd"], whole["lse_s"], whole["lse_t"], whole["sigma"])
    torch.cuda.synchronize()
    for k, tol in (("ce", 2e-4), ("lse_s", 2e-4), ("lse_t", 2e-4), ("tvd", 2e-5), ("sigma", 1e-4)):
        d = np.abs(whole[k].cpu().numpy() - runs[0][0][k])
        assert np.max(d) <= tol, (k, float(np.max(d)))


def test_out_of_range_target_poisons_the_row_in_every_shard():
    BT, V = 64, 9000
    z, u, t = W.custom(BT, V, "bf16", seed=9, scale=2.0, teacher_noise=0.5)
    t[3], t[5] = V, -2
    bounds = shard_bounds(V, [3000, 3000, 3000])
    announce("vocab-parallel: targets out of range on rows 3 and 5")
    o, g = run_vp(z, u, t, bounds, 1.0, 1.0)
    assert np.isnan(o["ce"][3]) and np.isnan(o["ce"][5])
    gf = g.float()
    assert bool(torch.isnan(gf[3]).all()) and bool(torch.isnan(gf[5]).all())
    ok = torch.ones(BT, dtype=torch.bool)
    ok[[3, 5]] = False
    assert bool(torch.isfinite(gf[ok.to(DEV)]).all())
    assert np.all(np.isfinite(o["ce"][ok.numpy()]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_negative_infinity_columns_in_shards(dtype):
    """-inf logits (masked columns): scattered columns, and for some rows a whole shard
    (every unit a thread holds there is -inf)."""
    BT, V = 64, 6000
    z, u, t = W.custom(BT, V, dtype, seed=23, scale=2.0, teacher_noise=0.5)
    ninf = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    cols = [0, 7, 1999, 2000, 3333]
    z[:, cols] = ninf
    u[:, cols] = ninf
    z[:10, 4000:] = ninf
    u[:10, 4000:] = ninf
    bad = np.isin(t, cols) | ((np.arange(BT) < 10) & (t >= 4000))
    t[bad] = 50
    announce(f"vocab-parallel: -inf columns and a masked shard, {dtype}")
    o, g = run_vp(z, u, t, shard_bounds(V, [2000, 2000, 2000]), 0.5, 1.5)
    check_forward(o, z, u, t, II, "vocab-parallel -inf")
    gh = grad_to_host(g)
    check_grad(gh, grad_bits(g), z, u, t, II, 0.5, 1.5, "vocab-parallel -inf")
    assert np.all(gh[:, cols] == 0.0) and np.all(gh[:10, 4000:] == 0.0)


def _offset_copy(raw: np.ndarray, elems: int) -> torch.Tensor:
    """Device copy of raw starting `elems` elements past an aligned allocation."""
    BT, V = raw.shape
    base = torch.zeros(BT * V + 64, dtype=torch.bfloat16 if raw.dtype == np.uint16 else torch.float32, device=DEV)
    view = base[elems:elems + BT * V].view(BT, V)
    view.copy_(to_dev(raw))
    return view


@pytest.mark.parametrize("zoff,uoff", [(1, 1), (3, 5)], ids=["both+1", "mismatched"])
def test_unaligned_shards(zoff, uoff):
    """Shard arrays off the 16-byte grid: with equal offsets the rows keep a scalar
    head and tail around 16-byte units; with different ones every element is read
    singly.  The partials and merges against the oracle on whole rows."""
    BT, V = 48, 9000
    z, u, t = W.custom(BT, V, "bf16", seed=31 + zoff + 7 * uoff, scale=2.5, teacher_noise=0.5, ignore_rows=[4])
    bounds = shard_bounds(V, [2999, 3001, 3000])
    announce(f"vocab-parallel: shards at element offsets z+{zoff} u+{uoff}")
    tg = to_dev(t)
    stats = torch.full((3, BT, 5), 777.0, dtype=torch.float32, device=DEV)
    tv = torch.full((3, BT, 2), 777.0, dtype=torch.float32, device=DEV)
    zs = [_offset_copy(np.ascontiguousarray(z[:, a:b]), zoff) for a, b in bounds]
    us = [_offset_copy(np.ascontiguousarray(u[:, a:b]), uoff) for a, b in bounds]
    for n, (a, _) in enumerate(bounds):
        lx.lx_ce_tvd_vp_stats(zs[n], us[n], tg, a, II, stats[n])
    f = lambda: torch.full((BT,), 12345.0, dtype=torch.float32, device=DEV)
    out = {k: f() for k in ("ce", "lse_s", "lse_t", "tvd", "sigma")}
    lx.lx_ce_tvd_vp_merge_stats(stats, tg, V, II, out["ce"], out["lse_s"], out["lse_t"])
    for n in range(3):
        lx.lx_ce_tvd_vp_tv(zs[n], us[n], tg, II, out["lse_s"], out["lse_t"], tv[n])
    lx.lx_ce_tvd_vp_merge_tv(tv, tg, II, out["tvd"], out["sigma"])
    torch.cuda.synchronize()
    check_forward({k: v.cpu().numpy() for k, v in out.items()}, z, u, t, II, "vocab-parallel unaligned")


def test_shard_sums_near_the_fp32_limit():
    """8 shards of 18992 columns (2374 16-byte units each): in every shard the first
    256 units (one per thread, the thread's reference) hold lo and the rest hi, 82
    above, so each thread's sum against its reference is ~1e37 and the sum over a
    workgroup would overflow fp32 unless the thread redoes it against its true
    maximum."""
    BT, V = 64, 151936
    Vs = V // 8
    col = np.arange(V) % Vs
    row = np.where(col // 8 < 256, -57.0, 25.0).astype(np.float32)
    rng = np.random.default_rng(11)
    z = W.bf16_bits_rne(row[None, :] + rng.integers(0, 4, (BT, V)).astype(np.float32) * 0.125)
    u = W.bf16_bits_rne(row[None, :] - 1.0 + rng.integers(0, 4, (BT, V)).astype(np.float32) * 0.125)
    t = rng.integers(0, V, BT).astype(np.int64)
    announce("vocab-parallel: per-thread sums near the fp32 limit, 8 shards of 18992")
    o, g = run_vp(z, u, t, shard_bounds(V, [Vs] * 8), 0.5, 1.5)
    check_forward(o, z, u, t, II, "vocab-parallel sums near the fp32 limit")
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, 0.5, 1.5, "vocab-parallel sums near the fp32 limit")


def test_train_workload_in_eight_shards():
    """The training batch (8192 x 151936 bf16) cut into 8 shards of 18992 columns, the
    shape each device of an 8-way vocabulary-parallel layout holds; mean-reduced
    (g_scale = 1/n_valid); sampled rows against the oracle, properties on all rows."""
    w = W.get("train")
    announce(f"vocab-parallel train {w.BT}x{w.V} in 8 shards: generating inputs")
    z, u, t = W.full(w)
    rng = np.random.default_rng(17)
    rows = np.array(sorted(set(rng.choice(w.BT, 40, replace=False).tolist()) | {0, w.BT - 1}))
    zr, ur = z[rows].copy(), u[rows].copy()
    bounds = shard_bounds(w.V, [w.V // 8] * 8)
    tg = to_dev(t)
    inv = torch.zeros(1, dtype=torch.float32, device=DEV)
    lx.lx_ce_tvd_count_valid(tg, II, None, inv)
    n_valid = int((t != II).sum())
    announce("vocab-parallel train: partials, merges, backward")
    o, g = run_vp(z, u, t, bounds, 1.0, 1.0, g_scale=inv)
    del z, u
    gs = g.float()
    rs, ra = gs.sum(1).abs().cpu().numpy(), gs.abs().sum(1).cpu().numpy()
    del gs
    assert np.all(rs <= 2.0 ** -8 * ra + w.V * 1e-6 / n_valid + 1e-9)
    assert np.all((o["tvd"] >= 0) & (o["tvd"] <= 1 + 1e-6))
    sel = torch.from_numpy(rows).to(DEV)
    announce(f"vocab-parallel train: oracle on {len(rows)} sampled rows")
    check_forward({k: v[rows] for k, v in o.items()}, zr, ur, t[rows], II, "vocab-parallel train")
    check_grad(grad_to_host(g[sel]), grad_bits(g[sel]), zr, ur, t[rows], II, 1.0 / n_valid, 1.0 / n_valid,
               "vocab-parallel train")
