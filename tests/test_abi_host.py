"""The C ABI library on the host: it loads, exports every declared symbol, and its
argument validation rejects bad calls before any HIP call (CPU only: no kernel
is ever launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lx_ce_tvd.h")

lx = pytest.importorskip("cross_entropy_tv_amd", reason="HIP library not built")
L = lx.lib

# fake, never dereferenced device addresses (validation returns before any use)
A = 1 << 32


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(lx_[a-z_0-9]+)\s*\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"lx_ce_tvd_forward", "lx_ce_tvd_backward", "lx_ce_tvd_reduce_mean",
            "lx_ce_tvd_workspace_bytes", "lx_status_string"} <= set(names)
    so = ctypes.CDLL(lx.LIB_PATH)
    for n in names:
        assert hasattr(so, n), n


def test_status_strings_and_version():
    assert lx.lx_abi_version() == 1
    for code, name in ((0, "LX_OK"), (1, "LX_ERR_INVALID_ARG"), (2, "LX_ERR_UNSUPPORTED_DTYPE"),
                       (3, "LX_ERR_ALIAS"), (4, "LX_ERR_WORKSPACE"), (5, "LX_ERR_HIP")):
        assert lx.lx_status_string(code) == name


def fwd(student=A, teacher=A + (1 << 31), target=A * 3, BT=4, V=100, ii=-100, ce=A * 4, tvd=A * 4 + 64,
        lse_s=A * 4 + 128, lse_t=A * 4 + 192, sigma=A * 4 + 256, dt=1, ws=None, wsb=0):
    return L.lx_ce_tvd_forward(student, teacher, target, BT, V, ii, ce, tvd, lse_s, lse_t, sigma, dt, ws, wsb, None)


def bwd(grad=A * 5, student=A, teacher=A + (1 << 31), target=A * 3, BT=4, V=100, lse_s=A * 4 + 128,
        lse_t=A * 4 + 192, sigma=A * 4 + 256, g_scale=None, dt=1):
    return L.lx_ce_tvd_backward(grad, student, teacher, target, BT, V, -100, lse_s, lse_t, sigma, 1.0, 1.0,
                                g_scale, dt, None)


def test_forward_validation():
    assert fwd(BT=0) == lx.LX_OK                                  # no-op
    assert fwd(dt=7) == lx.LX_ERR_UNSUPPORTED_DTYPE
    assert fwd(BT=-1) == lx.LX_ERR_INVALID_ARG
    assert fwd(V=0) == lx.LX_ERR_INVALID_ARG
    assert fwd(V=2**31) == lx.LX_ERR_INVALID_ARG
    assert fwd(BT=2**62, V=2**20) == lx.LX_ERR_INVALID_ARG        # byte size overflows int64
    assert fwd(student=None) == lx.LX_ERR_INVALID_ARG
    assert fwd(target=None) == lx.LX_ERR_INVALID_ARG
    assert fwd(ce=None) == lx.LX_ERR_INVALID_ARG
    assert fwd(sigma=None) == lx.LX_ERR_INVALID_ARG               # required with a teacher
    assert fwd(student=A + 1) == lx.LX_ERR_INVALID_ARG            # not element aligned
    assert fwd(target=A * 3 + 4) == lx.LX_ERR_INVALID_ARG
    assert fwd(ce=A * 4 + 2) == lx.LX_ERR_INVALID_ARG
    assert fwd(tvd=A * 4) == lx.LX_ERR_ALIAS                      # two outputs share memory
    assert fwd(ce=A + 64) == lx.LX_ERR_ALIAS                      # output inside the student logits
    assert fwd(sigma=A * 3 + 8) == lx.LX_ERR_ALIAS                # output inside target
    # split-V shape (few rows, long rows) needs a workspace
    need = lx.lx_ce_tvd_workspace_bytes(4, 100000, 1, 1)
    assert need > 0 and lx.lx_ce_tvd_workspace_bytes(4, 100000, 1, 0) < need
    assert lx.lx_ce_tvd_workspace_bytes(8192, 151936, 1, 0) == 0   # CE-only: one stream, no exchange
    assert lx.lx_ce_tvd_workspace_bytes(8192, 151936, 0, 1) == 0   # f32 rows: one workgroup per row
    # bf16 with a teacher: the read-once path exchanges per-row partials of its K = 4
    # member workgroups (3 64-bit slots per member) and keeps a counter per row + a ticket
    slots, counters = 8192 * 4 * 3 * 8, (8192 + 1) * 4
    assert lx.lx_ce_tvd_workspace_bytes(8192, 151936, 1, 1) == (slots + counters + 255) // 256 * 256
    assert fwd(V=100000, teacher=A * 2) == lx.LX_ERR_WORKSPACE
    assert fwd(V=100000, teacher=A * 2, ws=A * 6, wsb=need - 4) == lx.LX_ERR_WORKSPACE
    assert fwd(V=100000, teacher=A * 2, ws=A * 6 + 16, wsb=need) == lx.LX_ERR_WORKSPACE  # 256-B alignment
    assert fwd(V=100000, teacher=A * 2, ws=A * 4, wsb=need) == lx.LX_ERR_ALIAS         # workspace over outputs


def test_backward_validation():
    assert bwd(BT=0) == lx.LX_OK
    assert bwd(dt=3) == lx.LX_ERR_UNSUPPORTED_DTYPE
    assert bwd(grad=None) == lx.LX_ERR_INVALID_ARG
    assert bwd(lse_s=None) == lx.LX_ERR_INVALID_ARG
    assert bwd(sigma=None) == lx.LX_ERR_INVALID_ARG
    assert bwd(grad=A + 1) == lx.LX_ERR_INVALID_ARG
    assert bwd(g_scale=A * 6 + 2) == lx.LX_ERR_INVALID_ARG
    assert bwd(grad=A + 2) == lx.LX_ERR_ALIAS                     # partial overlap with student
    assert bwd(grad=A + (1 << 31) - 100) == lx.LX_ERR_ALIAS       # overlaps teacher
    assert bwd(grad=A * 4 + 100) == lx.LX_ERR_ALIAS               # overlaps lse / sigma
    assert bwd(grad=A * 5, g_scale=A * 5 + 12) == lx.LX_ERR_ALIAS


def test_reduce_validation():
    r = L.lx_ce_tvd_reduce_mean
    assert r(A, A + 4096, A * 2, -1, -100, A * 3, None, None, None) == lx.LX_ERR_INVALID_ARG
    assert r(A, A + 4096, A * 2, 4, -100, None, None, None, None) == lx.LX_ERR_INVALID_ARG
    assert r(A, A + 4096, A * 2, 4, -100, A + 8, None, None, None) == lx.LX_ERR_ALIAS
    assert r(A, A + 4096, A * 2, 4, -100, A * 3, A * 3, None, None) == lx.LX_ERR_ALIAS
    assert r(A, A + 4096, A * 2, 4, -100, A * 3, A * 3 + 12, None, None) == lx.LX_ERR_INVALID_ARG  # n_valid align
