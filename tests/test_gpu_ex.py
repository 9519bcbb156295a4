"""Parity with the float64 oracle, on the GPU through the C ABI, of what the
entry points with the ``_ex`` suffix add, and of binary16 logits:

* IEEE binary16 logits (and gradients) on every path: one workgroup per row,
  rows split across workgroups, the read-once forward and the one-pass
  forward + backward, the backward, the vocabulary-parallel pieces;
* row strides: student, teacher and gradient as views into wider arrays (a
  padded vocabulary), strides that keep every row on a 16-byte boundary (the
  read-once / one-pass kernels), strides that do not, and different strides
  per tensor; padding columns must stay untouched;
* per-row upstream gradients (an unreduced loss), on the backward and on the
  one-pass kernel, with row factors large enough that the one pass forms the
  large-p groups from fp32 p.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads as W
from _parity import DEV, G_REL, G_REL_P16, announce, check_forward, check_grad, grad_bits, grad_to_host, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cross_entropy_tv_amd as lx  # noqa: E402

II = W.IGNORE_INDEX
SENTINEL = 12345.0
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
LX_DT = {"bf16": lx.LX_BF16, "f16": lx.LX_F16, "f32": lx.LX_F32}


def outputs(BT, teacher=True):
    keys = ("ce", "tvd", "lse_s", "lse_t", "sigma") if teacher else ("ce", "lse_s")
    return {k: torch.full((BT,), SENTINEL, dtype=torch.float32, device=DEV) for k in keys}


def host(out):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def special_rows(BT):
    if BT <= 4:
        return {"ignore_rows": [1]}
    return {"ignore_rows": [1, BT - 1], "identical_rows": [2], "uniform_rows": [3]}


def padded(raw: np.ndarray, dtype: str, pad: int):
    """A (BT, V) view with row stride V + pad into a sentinel-filled device array."""
    BT, V = raw.shape
    big = torch.full((BT, V + pad), SENTINEL, dtype=TORCH_DT[dtype], device=DEV)
    big[:, :V] = to_dev(raw)
    return big, big[:, :V]


def pad_bits(big: torch.Tensor, V: int) -> np.ndarray:
    return grad_bits(big[:, V:].contiguous())


def sentinel_bits(dtype: str) -> int:
    return int(grad_bits(torch.full((1,), SENTINEL, dtype=TORCH_DT[dtype]))[0])


# ---------------------------------------------------------------- binary16 logits

@pytest.mark.parametrize("teacher", [True, False], ids=["ce_tvd", "ce_only"])
@pytest.mark.parametrize("BT,V", [(520, 4099), (6, 50001), (520, 8200), (40, 151936)],
                         ids=["rowpath_520x4099", "split_6x50001", "readonce_520x8200", "onepass_40x151936"])
def test_binary16_logits(BT, V, teacher):
    """Forward, backward and forward_backward (in place) with binary16 logits."""
    z, u, t = W.custom(BT, V, "f16", seed=BT + 3 * V, scale=3.0, teacher_noise=0.5, **special_rows(BT))
    if not teacher:
        u = None
    label = f"f16 {BT}x{V} {'ce_tvd' if teacher else 'ce_only'}"
    announce(label)
    zs, tg = to_dev(z), to_dev(t)
    us = None if u is None else to_dev(u)
    out = outputs(BT, teacher)
    lx.lx_ce_tvd_forward(zs, us, tg, II, out["ce"], out.get("tvd"), out["lse_s"], out.get("lse_t"), out.get("sigma"))
    o = host(out)
    check_forward(o, z, u, t, II, label + " forward")
    g = torch.full_like(zs, SENTINEL)
    lx.lx_ce_tvd_backward(g, zs, us, tg, II, out["lse_s"], out.get("lse_t"), out.get("sigma"), 0.5, 1.5)
    torch.cuda.synchronize()
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, 0.5, 1.5, label + " backward", fmt="f16")
    if teacher and BT > 4:
        assert o["tvd"][2] == 0.0 and o["sigma"][2] == 0.0, "identical rows must give exactly 0"
    if BT > 4:
        assert abs(o["ce"][3] - math.log(V)) <= 1e-4
    # one call, in place (the one-pass kernel where the shape allows)
    out2 = outputs(BT, teacher)
    lx.lx_ce_tvd_forward_backward(zs, us, tg, II, out2["ce"], out2.get("tvd"), out2["lse_s"], out2.get("lse_t"),
                                  out2.get("sigma"), zs, 0.5, 1.5)
    check_forward(host(out2), z, u, t, II, label + " forward_backward")
    check_grad(grad_to_host(zs), grad_bits(zs), z, u, t, II, 0.5, 1.5, label + " forward_backward in place",
               rel=G_REL_P16, fmt="f16")


def test_binary16_vocabulary_parallel():
    """Step-1 / step-2 partials of three uneven column shards of binary16 logits,
    merged, and the shard backwards, against the oracle on the whole rows."""
    BT, V = 64, 10007
    z, u, t = W.custom(BT, V, "f16", seed=991, scale=3.0, teacher_noise=0.5, **special_rows(BT))
    t[5], t[6] = 0, V - 1
    edges = [0, 3001, 3002, V]
    announce(f"f16 vocabulary-parallel {BT}x{V} in {len(edges) - 1} shards")
    tg = to_dev(t)
    n = len(edges) - 1
    stats = torch.empty((n, BT, 5), dtype=torch.float32, device=DEV)
    shards = []
    for i in range(n):
        zs = to_dev(np.ascontiguousarray(z[:, edges[i]:edges[i + 1]]))
        us = to_dev(np.ascontiguousarray(u[:, edges[i]:edges[i + 1]]))
        shards.append((zs, us))
        lx.lx_ce_tvd_vp_stats(zs, us, tg, edges[i], II, stats[i])
    out = outputs(BT)
    lx.lx_ce_tvd_vp_merge_stats(stats, tg, V, II, out["ce"], out["lse_s"], out["lse_t"])
    tv = torch.empty((n, BT, 2), dtype=torch.float32, device=DEV)
    for i, (zs, us) in enumerate(shards):
        lx.lx_ce_tvd_vp_tv(zs, us, tg, II, out["lse_s"], out["lse_t"], tv[i])
    lx.lx_ce_tvd_vp_merge_tv(tv, tg, II, out["tvd"], out["sigma"])
    check_forward(host(out), z, u, t, II, "f16 vocabulary-parallel")
    parts = []
    for i, (zs, us) in enumerate(shards):
        g = torch.full_like(zs, SENTINEL)
        lx.lx_ce_tvd_backward_shard(g, zs, us, tg, edges[i], V, II, out["lse_s"], out["lse_t"], out["sigma"],
                                    0.5, 1.5)
        parts.append(g)
    g = torch.cat(parts, dim=1)
    torch.cuda.synchronize()
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, 0.5, 1.5, "f16 vocabulary-parallel backward", fmt="f16")


# ---------------------------------------------------------------- row strides

# (student pad, teacher pad, grad pad) in elements
STRIDES = {
    "aligned": (8, 24, 8),    # 2-byte rows stay on 16-byte boundaries: read-once / one-pass kernels
    "odd": (3, 3, 3),          # rows drift across 16-byte boundaries together: vector path with per-row heads
    "mixed": (3, 5, 1),        # rows of the three tensors drift apart: element-wise path
}


@pytest.mark.parametrize("teacher", [True, False], ids=["ce_tvd", "ce_only"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("stride", sorted(STRIDES))
@pytest.mark.parametrize("BT,V", [(520, 8200), (6, 20000)], ids=["520x8200", "split_6x20000"])
def test_strided_rows(BT, V, stride, dtype, teacher):
    """forward_ex, backward_ex and forward_backward_ex on row-strided views; the
    columns past V of every row (the padding) are never written."""
    ps, pt, pg = STRIDES[stride]
    z, u, t = W.custom(BT, V, dtype, seed=BT + V + ps + pt, scale=3.0, teacher_noise=0.5, **special_rows(BT))
    if not teacher:
        u = None
    label = f"strided {stride} {BT}x{V} {dtype} {'ce_tvd' if teacher else 'ce_only'}"
    announce(label)
    zbig, zs = padded(z, dtype, ps)
    us = None
    if teacher:
        ubig, us = padded(u, dtype, pt)
    tg = to_dev(t)
    sent = sentinel_bits(dtype)
    out = outputs(BT, teacher)
    lx.lx_ce_tvd_forward_ex(zs, us, tg, II, out["ce"], out.get("tvd"), out["lse_s"], out.get("lse_t"),
                            out.get("sigma"))
    check_forward(host(out), z, u, t, II, label + " forward_ex")
    gbig = torch.full((BT, V + pg), SENTINEL, dtype=TORCH_DT[dtype], device=DEV)
    g = gbig[:, :V]
    lx.lx_ce_tvd_backward_ex(g, zs, us, tg, II, out["lse_s"], out.get("lse_t"), out.get("sigma"), 0.5, 1.5)
    torch.cuda.synchronize()
    gc = g.contiguous()
    check_grad(grad_to_host(gc), grad_bits(gc), z, u, t, II, 0.5, 1.5, label + " backward_ex", fmt=dtype)
    assert np.all(pad_bits(gbig, V) == sent), f"{label}: backward_ex wrote into the padding"
    # one call, out of place, then in place into the student's own view
    gbig.fill_(SENTINEL)
    out2 = outputs(BT, teacher)
    lx.lx_ce_tvd_forward_backward_ex(zs, us, tg, II, out2["ce"], out2.get("tvd"), out2["lse_s"], out2.get("lse_t"),
                                     out2.get("sigma"), g, 0.5, 1.5)
    check_forward(host(out2), z, u, t, II, label + " forward_backward_ex")
    gc = g.contiguous()
    check_grad(grad_to_host(gc), grad_bits(gc), z, u, t, II, 0.5, 1.5, label + " forward_backward_ex",
               rel=G_REL_P16, fmt=dtype)
    assert np.all(pad_bits(gbig, V) == sent), f"{label}: forward_backward_ex wrote into the padding"
    lx.lx_ce_tvd_forward_backward_ex(zs, us, tg, II, out2["ce"], out2.get("tvd"), out2["lse_s"], out2.get("lse_t"),
                                     out2.get("sigma"), zs, 0.5, 1.5)
    torch.cuda.synchronize()
    zc = zs.contiguous()
    check_grad(grad_to_host(zc), grad_bits(zc), z, u, t, II, 0.5, 1.5, label + " forward_backward_ex in place",
               rel=G_REL_P16, fmt=dtype)
    assert np.all(pad_bits(zbig, V) == sent), f"{label}: in-place gradient wrote into the padding"


def test_strided_training_batch_sampled():
    """The training batch (8192 x 151936 bf16) inside arrays padded to 152064 columns
    (a vocabulary rounded up to a multiple of 256), one pass in place, mean-reduced:
    sampled rows against the oracle, zero row sums everywhere, padding untouched."""
    w = W.get("train")
    BT, V, pad = w.BT, w.V, 128
    announce(f"strided training batch {BT}x{V} (row stride {V + pad}) one pass in place")
    rows = np.array(sorted({0, 1, 2, 777, 4095, 4096, 6000, BT - 2, BT - 1}))
    zr, ur = W.rows(w, rows)
    t = W.targets(w)
    z, u, _ = W.full(w)
    zbig = torch.full((BT, V + pad), SENTINEL, dtype=torch.bfloat16, device=DEV)
    ubig = torch.full((BT, V + pad), SENTINEL, dtype=torch.bfloat16, device=DEV)
    zbig[:, :V] = to_dev(z)
    ubig[:, :V] = to_dev(u)
    del z, u
    zs, us, tg = zbig[:, :V], ubig[:, :V], to_dev(t)
    inv = torch.empty(1, dtype=torch.float32, device=DEV)
    lx.lx_ce_tvd_count_valid(tg, II, None, inv)
    out = outputs(BT)
    lx.lx_ce_tvd_forward_backward_ex(zs, us, tg, II, out["ce"], out["tvd"], out["lse_s"], out["lse_t"],
                                     out["sigma"], zs, 1.0, 1.0, g_scale=inv)
    o = host(out)
    k = 1.0 / BT
    sel = torch.from_numpy(rows).to(DEV)
    gsel = zs[sel].contiguous()
    check_forward({kk: v[rows] for kk, v in o.items()}, zr, ur, t[rows], II, "strided train")
    check_grad(grad_to_host(gsel), grad_bits(gsel), zr, ur, t[rows], II, k, k, "strided train", rel=G_REL_P16,
               sigma_gpu=o["sigma"][rows])
    gs = zs.float()
    rs, ra = gs.sum(1).abs().cpu().numpy(), gs.abs().sum(1).cpu().numpy()
    del gs
    assert np.all(rs <= 2.0 ** -8 * ra + V * 1e-6 + 1e-9)
    assert np.all(pad_bits(zbig, V) == sentinel_bits("bf16")), "padding written"


# ---------------------------------------------------------------- per-row upstream gradients

def row_factors(BT, seed):
    rng = np.random.default_rng(seed)
    w_ce = rng.normal(0, 1.0, BT).astype(np.float32)
    w_tvd = rng.normal(0, 1.0, BT).astype(np.float32)
    w_ce[::7] = 0.0                     # rows with no CE gradient
    w_tvd[::5] = 0.0
    w_ce[3::11] *= 2000.0               # large upstream gradients: the one pass takes fp32 p for large p
    w_tvd[4::13] *= -3000.0
    return w_ce, w_tvd


@pytest.mark.parametrize("entry", ["backward_ex", "forward_backward_ex"])
@pytest.mark.parametrize("teacher", [True, False], ids=["ce_tvd", "ce_only"])
@pytest.mark.parametrize("dtype,BT,V", [("bf16", 520, 8200), ("f16", 520, 8200), ("bf16", 64, 151936),
                                        ("f32", 515, 1031)],
                         ids=["bf16_520x8200", "f16_520x8200", "bf16_64x151936", "f32_515x1031"])
def test_per_row_upstream_gradients(entry, teacher, dtype, BT, V):
    """grad row r = k * (g_ce * w_ce[r] * (p - onehot) + g_tvd * w_tvd[r] * 0.5 * p * (s - sigma))."""
    z, u, t = W.custom(BT, V, dtype, seed=5 * BT + V, scale=3.0, teacher_noise=0.5, **special_rows(BT))
    if not teacher:
        u = None
    w_ce, w_tvd = row_factors(BT, BT + V)
    g_ce, g_tvd, k = 0.75, -1.25, 0.5
    label = f"row factors {entry} {dtype} {BT}x{V} {'ce_tvd' if teacher else 'ce_only'}"
    announce(label)
    zs, tg = to_dev(z), to_dev(t)
    us = None if u is None else to_dev(u)
    wc, wt = to_dev(w_ce), to_dev(w_tvd)
    scale = torch.full((1,), k, dtype=torch.float32, device=DEV)
    out = outputs(BT, teacher)
    g = torch.full_like(zs, SENTINEL)
    if entry == "backward_ex":
        lx.lx_ce_tvd_forward(zs, us, tg, II, out["ce"], out.get("tvd"), out["lse_s"], out.get("lse_t"),
                             out.get("sigma"))
        lx.lx_ce_tvd_backward_ex(g, zs, us, tg, II, out["lse_s"], out.get("lse_t"), out.get("sigma"), g_ce, g_tvd,
                                 wc, wt, scale)
    else:
        lx.lx_ce_tvd_forward_backward_ex(zs, us, tg, II, out["ce"], out.get("tvd"), out["lse_s"], out.get("lse_t"),
                                         out.get("sigma"), g, g_ce, g_tvd, wc, wt, scale)
    check_forward(host(out), z, u, t, II, label)
    eff_ce = k * g_ce * w_ce.astype(np.float64)
    eff_tvd = k * g_tvd * w_tvd.astype(np.float64)
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, eff_ce, eff_tvd, label,
               rel=G_REL_P16 if entry == "forward_backward_ex" else G_REL, fmt=dtype)
    # rows whose factors are both 0 have an exactly zero gradient
    both0 = (w_ce == 0) & ((w_tvd == 0) | (u is None))
    assert np.all(grad_to_host(g)[both0] == 0.0)


def test_row_factors_of_one_match_the_scalar_entry_points():
    """All-ones row factors give bit-identical results to the scalar entry points."""
    BT, V = 520, 8200
    z, u, t = W.custom(BT, V, "bf16", seed=4242, scale=3.0, teacher_noise=0.5, **special_rows(BT))
    announce("row factors of one vs scalar, bitwise")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    ones = torch.ones(BT, dtype=torch.float32, device=DEV)
    o1, o2 = outputs(BT), outputs(BT)
    g1, g2 = torch.empty_like(zs), torch.empty_like(zs)
    lx.lx_ce_tvd_forward_backward(zs, us, tg, II, o1["ce"], o1["tvd"], o1["lse_s"], o1["lse_t"], o1["sigma"], g1,
                                  0.5, 1.5)
    lx.lx_ce_tvd_forward_backward_ex(zs, us, tg, II, o2["ce"], o2["tvd"], o2["lse_s"], o2["lse_t"], o2["sigma"], g2,
                                     0.5, 1.5, ones, ones)
    torch.cuda.synchronize()
    assert torch.equal(g1.view(torch.int16), g2.view(torch.int16))
    for key in o1:
        assert torch.equal(o1[key].view(torch.int32), o2[key].view(torch.int32)), key
    g3 = torch.empty_like(zs)
    lx.lx_ce_tvd_backward(g3, zs, us, tg, II, o1["lse_s"], o1["lse_t"], o1["sigma"], 0.5, 1.5)
    g4 = torch.empty_like(zs)
    lx.lx_ce_tvd_backward_ex(g4, zs, us, tg, II, o1["lse_s"], o1["lse_t"], o1["sigma"], 0.5, 1.5, ones, ones)
    torch.cuda.synchronize()
    assert torch.equal(g3.view(torch.int16), g4.view(torch.int16))
