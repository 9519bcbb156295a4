"""Parity of the HIP path (through the C ABI) with the float64 oracle, on the GPU.

Small cases compare every output element; they span several tiles, ragged
tails, unaligned rows, every forward path (one workgroup per row, rows split
across workgroups, rows read once by cooperating workgroups) and the
degenerate cases.  The full-size workloads are in test_gpu_fullsize.py.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _parity import (DEV, announce, bits32, check_forward, check_grad, grad_bits, grad_to_host, to_dev)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

import cross_entropy_tv_amd as lx  # noqa: E402

II = W.IGNORE_INDEX
SENTINEL = 12345.0


def forward_path(BT, V, dtype, teacher):
    """Which forward kernel a contiguous, 16-byte aligned (BT, V) case takes (the
    planning rules of the library, read off its workspace queries)."""
    dt = {"bf16": lx.LX_BF16, "f16": lx.LX_F16, "f32": lx.LX_F32}[dtype]
    if lx.lx_ce_tvd_workspace_bytes(BT, V, dt, teacher) == 0:
        return "row"
    read_once = teacher and (V % (4 if dtype == "f32" else 8) == 0) and V >= (1024 if dtype == "f32" else 2048)
    return "read-once" if read_once else "split-V"


def fwd_outputs(BT, teacher=True):
    keys = ("ce", "tvd", "lse_s", "lse_t", "sigma") if teacher else ("ce", "lse_s")
    return {k: torch.full((BT,), SENTINEL, dtype=torch.float32, device=DEV) for k in keys}


def run_fwd(zs, us, tg, ii=II):
    out = fwd_outputs(zs.shape[0], us is not None)
    lx.lx_ce_tvd_forward(zs, us, tg, ii, out["ce"], out.get("tvd"), out["lse_s"], out.get("lse_t"),
                         out.get("sigma"))
    return out


def run_bwd(out, zs, us, tg, g_ce, g_tvd, ii=II, grad=None, g_scale=None):
    if grad is None:
        grad = torch.full_like(zs, SENTINEL)
    lx.lx_ce_tvd_backward(grad, zs, us, tg, ii, out["lse_s"], out.get("lse_t"), out.get("sigma"), g_ce, g_tvd,
                          g_scale)
    return grad


def host(out):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def full_case(label, z, u, t, g_ce=0.5, g_tvd=1.5, ii=II):
    """Forward + backward on every element of a small case."""
    announce(f"{label}: shape {z.shape} dtype {z.dtype} teacher {u is not None}")
    zs, tg = to_dev(z), to_dev(t)
    us = None if u is None else to_dev(u)
    out = run_fwd(zs, us, tg, ii)
    check_forward(host(out), z, u, t, ii, label)
    g = run_bwd(out, zs, us, tg, g_ce, g_tvd, ii)
    torch.cuda.synchronize()
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, ii, g_ce, g_tvd, label)
    return out, g


# ---------------------------------------------------------------- the tiny workload, end to end

def test_tiny_workload_end_to_end():
    w = W.get("tiny")  # 8 x 1024 f32, row 3 ignored, upstream gradients 1 / num_valid_rows
    z, u, t = W.full(w, threads=1)
    announce("tiny 8x1024 f32: forward, mean, backward with g_scale = 1/n_valid")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    out = run_fwd(zs, us, tg)
    mean = torch.full((2,), SENTINEL, dtype=torch.float32, device=DEV)
    nval = torch.zeros(1, dtype=torch.int64, device=DEV)
    inv = torch.zeros(1, dtype=torch.float32, device=DEV)
    lx.lx_ce_tvd_reduce_mean(out["ce"], out["tvd"], tg, II, mean, nval, inv)
    g = run_bwd(out, zs, us, tg, 1.0, 1.0, g_scale=inv)
    ref = check_forward(host(out), z, u, t, II, "tiny")
    mce, mtv, n = oracle.reduce_mean(ref["ce"], ref["tvd"], t, II)
    assert n == 7 and int(nval.item()) == 7
    assert abs(inv.item() - 1 / 7) <= 1e-7
    m = mean.cpu().numpy()
    assert abs(m[0] - mce) <= 1e-4 and abs(m[1] - mtv) <= 1e-5
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, 1 / 7, 1 / 7, "tiny")
    # host scalars instead of the device scale give the same result
    g2 = run_bwd(out, zs, us, tg, 1 / 7, 1 / 7)
    check_grad(grad_to_host(g2), grad_bits(g2), z, u, t, II, 1 / 7, 1 / 7, "tiny host g")


# ---------------------------------------------------------------- both forward paths, ragged shapes

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("teacher", [True, False], ids=["ce_tvd", "ce_only"])
@pytest.mark.parametrize("BT,V", [(520, 4099), (515, 1031), (6, 50001), (3, 40000), (64, 8200)],
                         ids=["520x4099", "515x1031", "6x50001", "3x40000", "64x8200"])
def test_ragged_shapes(BT, V, dtype, teacher):
    ign = [1, BT - 1] if BT > 4 else [1]
    ident = [2] if BT > 4 else []
    unif = [3] if BT > 4 else []
    z, u, t = W.custom(BT, V, dtype, seed=BT * 7 + V, scale=3.0, teacher_noise=0.5, ignore_rows=ign,
                       identical_rows=ident, uniform_rows=unif)
    label = f"{forward_path(BT, V, dtype, teacher)} {BT}x{V} {dtype} {'ce_tvd' if teacher else 'ce_only'}"
    out, g = full_case(label, z, u if teacher else None, t)
    if teacher and ident:
        o = host(out)
        assert o["tvd"][2] == 0.0 and o["sigma"][2] == 0.0, "identical rows must give exactly 0"
    if unif:
        assert abs(host(out)["ce"][3] - math.log(V)) <= 1e-4


@pytest.mark.parametrize("BT,V", [(520, 8200), (600, 20000), (512, 24576)],
                         ids=["cluster_520x8200", "cluster_600x20000", "cluster_512x24576"])
def test_cluster_path_shapes(BT, V):
    """Read-once forward (rows split across cooperating workgroups): ragged last member,
    ignored / identical / uniform rows, and rows whose logits span more than the
    per-thread exponent range (the overflow fallback)."""
    z, u, t = W.custom(BT, V, "bf16", seed=BT + V, scale=3.0, teacher_noise=0.5,
                       ignore_rows=[0, 7, BT - 1], identical_rows=[2, 9], uniform_rows=[3])
    hi = W.bf16_bits_rne(np.array([150.0, 120.0], dtype=np.float32))
    z[5, V // 3] = hi[0]          # far above every thread's first-group reference
    u[6, V - 5] = hi[1]
    z[8, 1], u[8, 2] = hi[0], hi[1]
    out, g = full_case(f"cluster {BT}x{V}", z, u, t, g_ce=0.5, g_tvd=1.5)
    o = host(out)
    assert o["tvd"][2] == 0.0 and o["sigma"][2] == 0.0 and o["tvd"][9] == 0.0
    assert abs(o["ce"][3] - math.log(V)) <= 1e-4


@pytest.mark.parametrize("V", [38400, 72000], ids=["K1_V38400", "K2_V72000"])
def test_cluster_path_lds_part(V):
    """Rows whose member chunks are longer than the registers hold (tails in LDS),
    forward outputs on sampled rows against the oracle."""
    BT = 2048
    z, u, t = W.custom(BT, V, "bf16", seed=V + 1, scale=3.0, teacher_noise=0.5, ignore_rows=[0, BT - 1],
                       identical_rows=[2], uniform_rows=[3])
    hi = W.bf16_bits_rne(np.array([150.0], dtype=np.float32))
    z[5, V - 7] = hi[0]
    announce(f"read-once forward, LDS part {BT}x{V}")
    o = host(run_fwd(to_dev(z), to_dev(u), to_dev(t)))
    rows = np.array([0, 1, 2, 3, 4, 5, 6, 999, BT - 2, BT - 1])
    check_forward({k: v[rows] for k, v in o.items()}, z[rows], u[rows], t[rows], II, f"LDS part {V}")
    assert o["tvd"][2] == 0.0 and abs(o["ce"][3] - math.log(V)) <= 1e-4


def test_cluster_path_deterministic_and_matches_row_path():
    z, u, t = W.custom(530, 16384, "bf16", seed=77, scale=2.0, offset_range=10.0, ignore_rows=[4])
    announce("cluster path: 3 repeats bitwise, and vs the two-stream row path on unaligned copies")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    runs = [host(run_fwd(zs, us, tg)) for _ in range(3)]
    for o in runs[1:]:
        for k in o:
            assert np.array_equal(bits32(o[k]), bits32(runs[0][k])), k
    # an unaligned copy takes the two-stream row path: same results within the tolerances
    zo, uo = _offset_view(z, 1), _offset_view(u, 1)
    o2 = host(run_fwd(zo, uo, tg))
    for k, tol in (("ce", 1e-4), ("lse_s", 1e-4), ("lse_t", 1e-4), ("tvd", 2e-5), ("sigma", 2e-5)):
        assert np.max(np.abs(o2[k] - runs[0][k])) <= tol, k


def test_independent_teacher_and_offsets():
    z, u, t = W.custom(40, 70001, "bf16", seed=5, scale=2.0, offset_range=20.0)
    full_case("split 40x70001 bf16 offsets", z, u, t, g_ce=1.0, g_tvd=-0.75)
    z, u, t = W.custom(600, 3001, "bf16", seed=6, scale=1.5, offset_range=20.0)
    full_case("row 600x3001 bf16 offsets", z, u, t, g_ce=0.25, g_tvd=2.0)


# ---------------------------------------------------------------- layouts: unaligned, mismatched alignment, in place

def _offset_view(raw: np.ndarray, elems: int) -> torch.Tensor:
    """Device copy of raw living `elems` elements past a 256-byte-aligned allocation."""
    BT, V = raw.shape
    base = torch.zeros(BT * V + 64, dtype=torch.bfloat16 if raw.dtype == np.uint16 else torch.float32, device=DEV)
    view = base[elems:elems + BT * V].view(BT, V)
    view.copy_(to_dev(raw))
    return view


@pytest.mark.parametrize("zoff,uoff,goff", [(1, 1, 1), (3, 3, 3), (1, 2, 1), (0, 0, 5)],
                         ids=["both+1", "both+3", "mismatched", "grad_mismatched"])
@pytest.mark.parametrize("BT,V", [(520, 1000), (5, 30000)], ids=["row", "split"])
def test_unaligned_pointers(zoff, uoff, goff, BT, V):
    z, u, t = W.custom(BT, V, "bf16", seed=11 + zoff + 3 * uoff, scale=2.0, teacher_noise=0.5, ignore_rows=[0])
    announce(f"unaligned z+{zoff} u+{uoff} g+{goff} {BT}x{V}")
    zs, us, tg = _offset_view(z, zoff), _offset_view(u, uoff), to_dev(t)
    out = run_fwd(zs, us, tg)
    check_forward(host(out), z, u, t, II, "unaligned")
    g = _offset_view(np.zeros_like(z), goff)
    run_bwd(out, zs, us, tg, 0.5, 1.5, grad=g)
    torch.cuda.synchronize()
    check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, 0.5, 1.5, "unaligned")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_in_place_backward_matches_out_of_place(dtype):
    z, u, t = W.custom(530, 5003, dtype, seed=21, scale=3.0, teacher_noise=0.5, ignore_rows=[7, 8])
    announce(f"in place 530x5003 {dtype}")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    out = run_fwd(zs, us, tg)
    g_out = run_bwd(out, zs, us, tg, 0.3, 0.7)
    zin = zs.clone()
    run_bwd(out, zin, us, tg, 0.3, 0.7, grad=zin)
    torch.cuda.synchronize()
    assert torch.equal(grad_bits_t(zin), grad_bits_t(g_out)), "in-place gradient differs from out-of-place"
    check_grad(grad_to_host(zin), grad_bits(zin), z, u, t, II, 0.3, 0.7, "in place")


def grad_bits_t(g):
    return g.view(torch.int16) if g.dtype == torch.bfloat16 else g.view(torch.int32)


# ---------------------------------------------------------------- degenerate cases

@pytest.mark.parametrize("V", [1, 2, 3, 7, 8, 9, 15, 17])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tiny_vocabularies(V, dtype):
    z, u, t = W.custom(9, V, dtype, seed=V, scale=2.0, ignore_rows=[4])
    full_case(f"V={V} {dtype}", z, u, t)
    full_case(f"V={V} {dtype} ce-only", z, None, t)


def test_zero_rows_is_a_noop():
    announce("BT = 0")
    e = torch.empty(0, 100, dtype=torch.bfloat16, device=DEV)
    t = torch.empty(0, dtype=torch.int64, device=DEV)
    f = torch.empty(0, dtype=torch.float32, device=DEV)
    lx.lx_ce_tvd_forward(e, e, t, II, f, f, f, f, f)
    lx.lx_ce_tvd_backward(e, e, e, t, II, f, f, f, 1.0, 1.0)
    mean = torch.full((2,), SENTINEL, device=DEV)
    n = torch.full((1,), 5, dtype=torch.int64, device=DEV)
    inv = torch.full((1,), SENTINEL, device=DEV)
    # an empty tensor's data_ptr() is NULL, which means "no tvd"; pass real (unread) buffers
    ce1, tvd1 = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    lx.lx_ce_tvd_reduce_mean(ce1, tvd1, t, II, mean, n, inv)
    torch.cuda.synchronize()
    assert torch.isnan(mean).all() and n.item() == 0 and inv.item() == 0.0


def test_out_of_range_target_poisons_its_row_only():
    z, u, t = W.custom(6, 3000, "bf16", seed=31, scale=2.0)
    t_bad = t.copy()
    t_bad[2] = 3000
    t_bad[4] = -5
    announce("out-of-range targets")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t_bad)
    out = run_fwd(zs, us, tg)
    o = host(out)
    assert np.isnan(o["ce"][2]) and np.isnan(o["ce"][4])
    good = [0, 1, 3, 5]
    ref = oracle.forward(z[good], u[good], t[good], II)
    assert np.all(np.abs(o["ce"][good] - ref["ce"]) <= 1e-4)
    # tvd / lse / sigma do not depend on the target and are still computed
    assert np.all(np.isfinite(o["tvd"])) and np.all(np.isfinite(o["lse_s"]))
    g = run_bwd(out, zs, us, tg, 1.0, 1.0)
    gh = grad_to_host(g)
    assert np.all(np.isnan(gh[[2, 4]])) and np.all(np.isfinite(gh[good]))


def test_ignore_index_inside_vocabulary_takes_precedence():
    z, u, t = W.custom(8, 2000, "bf16", seed=41, scale=2.0)
    t[[1, 5]] = 17
    full_case("ignore_index=17", z, u, t, ii=17)


def test_all_rows_ignored():
    z, u, _ = W.custom(5, 1000, "bf16", seed=43)
    t = np.full(5, II, dtype=np.int64)
    out, g = full_case("all ignored", z, u, t)
    mean = torch.zeros(2, device=DEV)
    n = torch.full((1,), 9, dtype=torch.int64, device=DEV)
    inv = torch.full((1,), SENTINEL, device=DEV)
    lx.lx_ce_tvd_reduce_mean(out["ce"], out["tvd"], to_dev(t), II, mean, n, inv)
    torch.cuda.synchronize()
    assert torch.isnan(mean).all() and n.item() == 0 and inv.item() == 0.0


def test_negative_infinity_logits():
    z, u, t = W.custom(520, 1500, "f32", seed=47, scale=2.0)
    mask_cols = [0, 7, 100, 1499]
    z[:, mask_cols] = -np.inf
    u[:, mask_cols] = -np.inf
    t[t == 7] = 8
    t[np.isin(t, mask_cols)] = 50
    out, g = full_case("-inf columns f32", z, u, t)
    assert np.all(grad_to_host(g)[:, mask_cols] == 0.0)


def test_identical_rows_exact_zero_tvd_gradient():
    z, _, t = W.custom(520, 7001, "bf16", seed=53, scale=3.0, ignore_rows=[9])
    announce("identical rows: tvd, sigma, tvd-gradient exactly 0")
    zs, tg = to_dev(z), to_dev(t)
    out = run_fwd(zs, zs, tg)
    o = host(out)
    assert np.all(o["tvd"] == 0.0) and np.all(o["sigma"] == 0.0)
    assert np.array_equal(bits32(o["lse_s"]), bits32(o["lse_t"]))
    g = run_bwd(out, zs, zs, tg, 0.0, 1.0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(grad_bits_t(g)) == 0


def test_deterministic_bitwise():
    z, u, t = W.custom(520, 9001, "bf16", seed=59, scale=2.5, teacher_noise=0.5, ignore_rows=[3])
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    announce("determinism: row path and split path, 3 repeats")
    for BTs in (520, 7):
        runs = []
        for _ in range(3):
            out = run_fwd(zs[:BTs].contiguous(), us[:BTs].contiguous(), tg[:BTs].contiguous())
            g = run_bwd(out, zs[:BTs].contiguous(), us[:BTs].contiguous(), tg[:BTs].contiguous(), 0.5, 0.5)
            torch.cuda.synchronize()
            runs.append((host(out), grad_bits_t(g).cpu()))
        for o, gb in runs[1:]:
            for k in o:
                assert np.array_equal(bits32(o[k]), bits32(runs[0][0][k])), k
            assert torch.equal(gb, runs[0][1])
