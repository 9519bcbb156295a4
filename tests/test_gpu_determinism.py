"""Bitwise determinism over many repeats (GPU) of the paths whose partial
results are merged across workgroups: the split-V forward (partials of
(max, sum-exp) and of (sum |p - q|, sum p sign) per (row, split), merged in
split order by a later stage), and the read-once forward and one pass (K
member workgroups per row exchanging partials through device-coherent slots,
merged in member order).  Each path runs 128 times on the same inputs; every
output and the gradient must equal the first run bit for bit.  Arrival order
of the members changes from run to run, so any order dependence in a merge
would show here.  The lm_head path (per-tile partials merged in a fixed
order, split-K partials of grad_x added in split order, grad_w accumulated
chunk by chunk) is repeated 16 times the same way.
"""
from __future__ import annotations

import pytest
import torch

import workloads as W
from _parity import DEV, announce, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import cross_entropy_tv_amd as lx  # noqa: E402

II = -100
REPEATS = 128


def _outputs(BT, teacher):
    f = lambda: torch.empty(BT, dtype=torch.float32, device=DEV)  # noqa: E731
    return {"ce": f(), "tvd": f() if teacher else None, "lse_s": f(), "lse_t": f() if teacher else None,
            "sigma": f() if teacher else None}


def _bits(out, g):
    res = [v.view(torch.int32).clone() for v in out.values() if v is not None]
    if g is not None:
        res.append(g.view(torch.int16).clone())
    return res


def _repeat(label, step):
    first = step()
    torch.cuda.synchronize()
    bad = 0
    for _ in range(REPEATS - 1):
        cur = step()
        bad += sum(int(not torch.equal(a, b)) for a, b in zip(first, cur))
    torch.cuda.synchronize()
    print(f"{label}: {REPEATS} runs, {bad} differing arrays", flush=True)
    assert bad == 0


def _forward_backward_separate(zs, us, tg, teacher):
    BT = zs.shape[0]

    def step():
        out = _outputs(BT, teacher)
        lx.lx_ce_tvd_forward(zs, us if teacher else None, tg, II, out["ce"], out["tvd"], out["lse_s"],
                             out["lse_t"], out["sigma"])
        g = torch.empty_like(zs)
        lx.lx_ce_tvd_backward(g, zs, us if teacher else None, tg, II, out["lse_s"], out["lse_t"], out["sigma"],
                              0.5, 1.5 if teacher else 0.0)
        return _bits(out, g)
    return step


def _one_pass(zs, us, tg, teacher):
    BT = zs.shape[0]

    def step():
        out = _outputs(BT, teacher)
        g = torch.empty_like(zs)
        lx.lx_ce_tvd_forward_backward(zs, us if teacher else None, tg, II, out["ce"], out["tvd"], out["lse_s"],
                                      out["lse_t"], out["sigma"], g, 0.5, 1.5 if teacher else 0.0)
        return _bits(out, g)
    return step


def test_split_v_forward_and_backward_128_repeats():
    # V % 8 != 0 and few rows: the split-V stages (workspace of partials)
    z, u, t = W.custom(7, 50001, "bf16", seed=71, scale=2.5, teacher_noise=0.5, ignore_rows=[2])
    assert lx.lx_ce_tvd_workspace_bytes(7, 50001, lx.LX_BF16, True) > 0, "expected the split-V forward"
    announce("determinism: split-V forward + backward, 7x50001 bf16, 128 runs")
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    _repeat("split-V 7x50001", _forward_backward_separate(zs, us, tg, True))


@pytest.mark.parametrize("BT,V", [(40, 151936), (64, 262144)], ids=["40x151936_13_members", "64x262144_8_members"])
def test_read_once_exchange_128_repeats(BT, V):
    z, u, t = W.custom(BT, V, "bf16", seed=72, scale=2.5, teacher_noise=0.5, ignore_rows=[1])
    assert lx.lx_ce_tvd_forward_backward_workspace_bytes(BT, V, lx.LX_BF16, True) > 0, "expected the read-once path"
    zs, us, tg = to_dev(z), to_dev(u), to_dev(t)
    announce(f"determinism: read-once forward + backward, {BT}x{V} bf16, 128 runs")
    _repeat(f"read-once forward + backward {BT}x{V}", _forward_backward_separate(zs, us, tg, True))
    announce(f"determinism: one pass CE+TVD, {BT}x{V} bf16, 128 runs")
    _repeat(f"one pass CE+TVD {BT}x{V}", _one_pass(zs, us, tg, True))
    announce(f"determinism: one pass CE-only, {BT}x{V} bf16, 128 runs")
    _repeat(f"one pass CE-only {BT}x{V}", _one_pass(zs, us, tg, False))


@pytest.mark.parametrize("BT,V,H,chunk", [(300, 8200, 136, 128), (64, 151936, 64, 64)],
                         ids=["300x8200_chunks_128_split_k", "64x151936_one_chunk"])
def test_linear_16_repeats(BT, V, H, chunk):
    x_s, w_s, x_t, w_t, t = W.linear_inputs(BT, V, H, H + 8, seed=73)
    d = lambda b: to_dev(b)  # noqa: E731
    X, Wd, Xt, Wt, tg = d(x_s), d(w_s), d(x_t), d(w_t), d(t)
    announce(f"determinism: lm_head {BT}x{V} H {H} chunk {chunk}, 16 runs")

    def step():
        f = lambda: torch.empty(BT, dtype=torch.float32, device=DEV)  # noqa: E731
        out = {"ce": f(), "tvd": f(), "lse_s": f(), "lse_t": f(), "sigma": f()}
        gx = torch.empty((BT, H), dtype=torch.float32, device=DEV)
        gw = torch.empty((V, H), dtype=torch.float32, device=DEV)
        lx.lx_ce_tvd_linear_forward_backward(X, Wd, Xt, Wt, tg, II, out["ce"], out["tvd"], out["lse_s"],
                                             out["lse_t"], out["sigma"], gx, gw, 0.5, 1.5, None, chunk)
        return [v.view(torch.int32).clone() for v in out.values()] + [gx.view(torch.int32).clone(),
                                                                      gw.view(torch.int32).clone()]
    first = step()
    torch.cuda.synchronize()
    bad = 0
    for _ in range(15):
        cur = step()
        bad += sum(int(not torch.equal(a, b)) for a, b in zip(first, cur))
    torch.cuda.synchronize()
    print(f"lm_head {BT}x{V}: 16 runs, {bad} differing arrays", flush=True)
    assert bad == 0
