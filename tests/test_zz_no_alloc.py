"""The allocation-free forward + backward entry point (its scratch in the
library's static device buffer) against the workspace entry point it varies,
through the C ABI on the GPU: two calls in a row on each path that needs
scratch, the second with a smaller input, so that what the first call left in
the shared buffer must not leak into the second.  Outputs and gradients must be
bit-identical to lx_ce_tvd_forward_backward's and within the tolerances of the
float64 oracle."""
from __future__ import annotations

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
DT = {"bf16": lx.LX_BF16, "f32": lx.LX_F32}

# (path, dtype, teacher, [(BT, V) of the first call, (BT, V) of the second, smaller call])
SEQUENCES = [
    ("one_pass", "bf16", True, [(600, 20000), (130, 8200)]),
    ("one_pass_ce_only", "bf16", False, [(520, 8200), (64, 4096)]),
    ("split_v_two_pass", "bf16", True, [(6, 50001), (3, 40001)]),
    ("one_pass_f32", "f32", True, [(520, 3000), (100, 1024)]),
]


def _outputs(BT, teacher):
    keys = ("ce", "tvd", "lse_s", "lse_t", "sigma") if teacher else ("ce", "lse_s")
    return {k: torch.full((BT,), 12345.0, dtype=torch.float32, device=DEV) for k in keys}


def _call(fn, zs, us, tg, **kw):
    out = _outputs(zs.shape[0], us is not None)
    g = torch.full_like(zs, 12345.0)
    fn(zs, us, tg, II, out["ce"], out.get("tvd"), out["lse_s"], out.get("lse_t"), out.get("sigma"), g, 0.5, 1.5,
       **kw)
    torch.cuda.synchronize()
    return out, g


@pytest.mark.parametrize("path,dtype,teacher,shapes", SEQUENCES, ids=[s[0] for s in SEQUENCES])
def test_noalloc_matches_the_workspace_entry_point(path, dtype, teacher, shapes):
    for i, (BT, V) in enumerate(shapes):
        z, u, t = W.custom(BT, V, dtype, seed=900 + 31 * i + V, scale=3.0, teacher_noise=0.5,
                           ignore_rows=[1, BT - 1], identical_rows=[2] if BT > 4 else [])
        if not teacher:
            u = None
        label = f"noalloc {path} call {i + 1}: {BT}x{V} {dtype}"
        announce(label)
        need = lx.lx_ce_tvd_forward_backward_workspace_bytes(BT, V, DT[dtype], teacher)
        assert 0 < need <= 8 << 20, f"{label}: the case must use scratch ({need} bytes)"
        zs, tg = to_dev(z), to_dev(t)
        us = None if u is None else to_dev(u)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        ref_out, ref_g = _call(lx.lx_ce_tvd_forward_backward, zs, us, tg, workspace=ws)
        out, g = _call(lx.lx_ce_tvd_forward_backward_noalloc, zs, us, tg)
        for k in out:
            assert torch.equal(out[k].view(torch.int32), ref_out[k].view(torch.int32)), f"{label}: {k} differs"
        gb = torch.int16 if g.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(g.view(gb), ref_g.view(gb)), f"{label}: gradient differs"
        o = {k: v.cpu().numpy() for k, v in out.items()}
        check_forward(o, z, u, t, II, label)
        rel = G_REL_P16 if (teacher and path.startswith("one_pass")) else G_REL
        check_grad(grad_to_host(g), grad_bits(g), z, u, t, II, 0.5, 1.5, label, rel=rel, sigma_gpu=o.get("sigma"))
