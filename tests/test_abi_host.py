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
    assert lx.lx_abi_version() == 7
    for code, name in ((0, "LX_OK"), (1, "LX_ERR_INVALID_ARG"), (2, "LX_ERR_UNSUPPORTED_DTYPE"),
                       (3, "LX_ERR_ALIAS"), (4, "LX_ERR_WORKSPACE"), (5, "LX_ERR_HIP"), (6, "LX_ERR_TOO_LARGE")):
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
    # f32 with a teacher: the read-once forward over quads of 4 fp32 logits, 8 members per row
    assert lx.lx_ce_tvd_workspace_bytes(8192, 151936, 0, 1) == (8192 * 8 * 24 + (8192 + 1) * 4 + 255) // 256 * 256
    # bf16 with a teacher: the read-once path exchanges per-row partials of its K >= 2
    # member workgroups (3 64-bit slots per member) and keeps a counter per row + a ticket
    ws = lx.lx_ce_tvd_workspace_bytes(8192, 151936, 1, 1)
    counters = (8192 + 1) * 4
    assert ws % 256 == 0 and any(ws == (8192 * k * 24 + counters + 255) // 256 * 256 for k in range(2, 33))
    wf = lx.lx_ce_tvd_forward_backward_workspace_bytes(8192, 151936, 1, 1)
    assert wf >= ws and any(wf == (8192 * k * 24 + counters + 255) // 256 * 256 for k in range(2, 33))
    # CE-only one pass: one exchange slot per member is used, the same layout is reserved
    assert lx.lx_ce_tvd_forward_backward_workspace_bytes(8192, 151936, 1, 0) > 0
    # f32 with a teacher: the one pass over quads of 4 fp32 logits, 8 members per row
    assert lx.lx_ce_tvd_forward_backward_workspace_bytes(8192, 151936, 0, 1) == \
        (8192 * 8 * 24 + (8192 + 1) * 4 + 255) // 256 * 256
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


def fwdbwd(student=A, teacher=A + (1 << 31), target=A * 3, BT=4, V=100, ce=A * 4, tvd=A * 4 + 64,
           lse_s=A * 4 + 128, lse_t=A * 4 + 192, sigma=A * 4 + 256, grad=A * 5, g_scale=None, dt=1, ws=None,
           wsb=0):
    return L.lx_ce_tvd_forward_backward(student, teacher, target, BT, V, -100, ce, tvd, lse_s, lse_t, sigma, grad,
                                        1.0, 1.0, g_scale, dt, ws, wsb, None)


def test_forward_backward_validation():
    assert fwdbwd(BT=0) == lx.LX_OK
    assert fwdbwd(dt=5) == lx.LX_ERR_UNSUPPORTED_DTYPE
    assert fwdbwd(grad=None) == lx.LX_ERR_INVALID_ARG
    assert fwdbwd(sigma=None) == lx.LX_ERR_INVALID_ARG
    assert fwdbwd(grad=A + 1) == lx.LX_ERR_INVALID_ARG                 # not element aligned
    assert fwdbwd(g_scale=A * 6 + 2) == lx.LX_ERR_INVALID_ARG
    assert fwdbwd(grad=A + 2) == lx.LX_ERR_ALIAS                       # partial overlap with student
    assert fwdbwd(grad=A + (1 << 31)) == lx.LX_ERR_ALIAS               # the teacher
    assert fwdbwd(grad=A * 4 + 100) == lx.LX_ERR_ALIAS                 # the forward outputs
    assert fwdbwd(ce=A * 5 + 8) == lx.LX_ERR_ALIAS                     # an output inside the gradient
    assert fwdbwd(g_scale=A * 4 + 64) == lx.LX_ERR_ALIAS               # g_scale inside an output
    need = lx.lx_ce_tvd_forward_backward_workspace_bytes(8192, 151936, 1, 1)
    big = dict(BT=8192, V=151936, teacher=A * 8, target=A * 3, ce=A * 4, tvd=A * 4 + (1 << 16),
               lse_s=A * 4 + (2 << 16), lse_t=A * 4 + (3 << 16), sigma=A * 4 + (4 << 16), grad=A * 12)
    assert fwdbwd(**big) == lx.LX_ERR_WORKSPACE
    assert fwdbwd(**big, ws=A * 16, wsb=need - 256) == lx.LX_ERR_WORKSPACE
    assert fwdbwd(**big, ws=A * 16 + 64, wsb=need) == lx.LX_ERR_WORKSPACE   # 256-B alignment
    assert fwdbwd(**big, ws=A * 12, wsb=need) == lx.LX_ERR_ALIAS          # workspace inside the gradient


def noalloc(student=A, teacher=A + (1 << 31), target=A * 3, BT=4, V=100, ce=A * 4, tvd=A * 4 + 64,
            lse_s=A * 4 + 128, lse_t=A * 4 + 192, sigma=A * 4 + 256, grad=A * 5, g_scale=None, dt=1):
    return L.lx_ce_tvd_forward_backward_noalloc(student, teacher, target, BT, V, -100, ce, tvd, lse_s, lse_t, sigma,
                                                grad, 1.0, 1.0, g_scale, dt, None)


def test_noalloc_validation():
    """The allocation-free entry point validates like lx_ce_tvd_forward_backward
    before it looks anything up, and rejects shapes beyond its static scratch."""
    assert noalloc(BT=0) == lx.LX_OK
    assert noalloc(dt=5) == lx.LX_ERR_UNSUPPORTED_DTYPE
    assert noalloc(grad=None) == lx.LX_ERR_INVALID_ARG
    assert noalloc(sigma=None) == lx.LX_ERR_INVALID_ARG
    assert noalloc(grad=A + 2) == lx.LX_ERR_ALIAS
    assert noalloc(ce=A * 5 + 8) == lx.LX_ERR_ALIAS
    limit = 8 << 20
    BT = 100000
    assert lx.lx_ce_tvd_forward_backward_workspace_bytes(BT, 151936, 1, 1) > limit
    big = dict(BT=BT, V=151936, student=A * 100, teacher=A * 200, target=A * 3, ce=A * 4, tvd=A * 4 + (1 << 20),
               lse_s=A * 4 + (2 << 20), lse_t=A * 4 + (3 << 20), sigma=A * 4 + (4 << 20), grad=A * 300)
    assert noalloc(**big) == lx.LX_ERR_TOO_LARGE


def test_reference_stream_validation():
    assert L.lx_stream_read(A, 0, A * 2, None) == lx.LX_OK
    assert L.lx_stream_read(A, 24, A * 2, None) == lx.LX_ERR_INVALID_ARG      # not a multiple of 16
    assert L.lx_stream_read(A + 8, 32, A * 2, None) == lx.LX_ERR_INVALID_ARG  # misaligned
    assert L.lx_stream_read(None, 32, A * 2, None) == lx.LX_ERR_INVALID_ARG
    assert L.lx_stream_read(A, 64, A + 16, None) == lx.LX_ERR_ALIAS          # sink inside src
    assert L.lx_stream_read2_write(A, A * 2, A * 3, 0, None) == lx.LX_OK
    assert L.lx_stream_read2_write(A, A * 2, A * 3, -16, None) == lx.LX_ERR_INVALID_ARG
    assert L.lx_stream_read2_write(A, A * 2, A + 32, 64, None) == lx.LX_ERR_ALIAS
    assert L.lx_stream_read2_write(A, None, A * 3, 64, None) == lx.LX_ERR_INVALID_ARG


def test_count_valid_validation():
    c = L.lx_ce_tvd_count_valid
    assert c(A, -1, -100, A * 2, None, None) == lx.LX_ERR_INVALID_ARG
    assert c(A, 4, -100, None, None, None) == lx.LX_ERR_INVALID_ARG       # no output
    assert c(A + 4, 4, -100, A * 2, None, None) == lx.LX_ERR_INVALID_ARG  # target alignment
    assert c(A, 4, -100, A + 8, None, None) == lx.LX_ERR_ALIAS            # n_valid inside target
    assert c(A, 4, -100, A * 2, A * 2 + 4, None) == lx.LX_ERR_ALIAS       # outputs overlap


def test_reduce_validation():
    r = L.lx_ce_tvd_reduce_mean
    assert r(A, A + 4096, A * 2, -1, -100, A * 3, None, None, None) == lx.LX_ERR_INVALID_ARG
    assert r(A, A + 4096, A * 2, 4, -100, None, None, None, None) == lx.LX_ERR_INVALID_ARG
    assert r(A, A + 4096, A * 2, 4, -100, A + 8, None, None, None) == lx.LX_ERR_ALIAS
    assert r(A, A + 4096, A * 2, 4, -100, A * 3, A * 3, None, None) == lx.LX_ERR_ALIAS
    assert r(A, A + 4096, A * 2, 4, -100, A * 3, A * 3 + 12, None, None) == lx.LX_ERR_INVALID_ARG  # n_valid align


def test_vocab_parallel_validation():
    names = set(declared_functions())
    assert {"lx_ce_tvd_vp_stats", "lx_ce_tvd_vp_merge_stats", "lx_ce_tvd_vp_tv", "lx_ce_tvd_vp_merge_tv",
            "lx_ce_tvd_backward_shard"} <= names

    def stats(student=A, teacher=A + (1 << 31), target=A * 3, BT=4, Vs=100, v0=0, dt=1, out=A * 4):
        return L.lx_ce_tvd_vp_stats(student, teacher, target, BT, Vs, v0, -100, dt, out, None)

    assert stats(BT=0) == lx.LX_OK
    assert stats(dt=5) == lx.LX_ERR_UNSUPPORTED_DTYPE
    assert stats(Vs=0) == lx.LX_ERR_INVALID_ARG
    assert stats(v0=-1) == lx.LX_ERR_INVALID_ARG
    assert stats(out=None) == lx.LX_ERR_INVALID_ARG
    assert stats(student=A + 1) == lx.LX_ERR_INVALID_ARG
    assert stats(out=A + 128) == lx.LX_ERR_ALIAS                     # inside the student shard
    assert stats(out=A * 3 + 16) == lx.LX_ERR_ALIAS                  # overlapping target

    def mstats(st=A, n=2, target=A * 3, BT=4, V=200, has_t=1, ce=A * 4, lse_s=A * 4 + 64, lse_t=A * 4 + 128):
        return L.lx_ce_tvd_vp_merge_stats(st, n, target, BT, V, -100, has_t, ce, lse_s, lse_t, None)

    assert mstats(BT=0) == lx.LX_OK
    assert mstats(n=0) == lx.LX_ERR_INVALID_ARG
    assert mstats(V=0) == lx.LX_ERR_INVALID_ARG
    assert mstats(lse_t=None) == lx.LX_ERR_INVALID_ARG              # required with a teacher
    assert mstats(ce=A + 16) == lx.LX_ERR_ALIAS                      # inside the partials
    assert mstats(lse_s=A * 4) == lx.LX_ERR_ALIAS                    # two outputs share memory

    def tv(student=A, teacher=A + (1 << 31), BT=4, Vs=100, lse_s=A * 4, lse_t=A * 4 + 64, out=A * 5):
        return L.lx_ce_tvd_vp_tv(student, teacher, A * 3, BT, Vs, -100, lse_s, lse_t, 1, out, None)

    assert tv(BT=0) == lx.LX_OK
    assert tv(teacher=None) == lx.LX_ERR_INVALID_ARG                 # step 2 needs the teacher
    assert tv(lse_t=None) == lx.LX_ERR_INVALID_ARG
    assert tv(out=A * 4 + 8) == lx.LX_ERR_ALIAS

    def mtv(t=A, n=3, BT=4, tvd=A * 4, sigma=A * 4 + 64):
        return L.lx_ce_tvd_vp_merge_tv(t, n, A * 3, BT, -100, tvd, sigma, None)

    assert mtv(BT=0) == lx.LX_OK
    assert mtv(n=0) == lx.LX_ERR_INVALID_ARG
    assert mtv(sigma=None) == lx.LX_ERR_INVALID_ARG
    assert mtv(tvd=A + 8) == lx.LX_ERR_ALIAS                         # inside the 3 x 4 x 2 partials

    def bshard(grad=A * 5, student=A, BT=4, Vs=100, v0=0, V=300):
        return L.lx_ce_tvd_backward_shard(grad, student, A + (1 << 31), A * 3, BT, Vs, v0, V, -100, A * 4 + 128,
                                          A * 4 + 192, A * 4 + 256, 1.0, 1.0, None, 1, None)

    assert bshard(BT=0) == lx.LX_OK
    assert bshard(v0=-1) == lx.LX_ERR_INVALID_ARG
    assert bshard(v0=201) == lx.LX_ERR_INVALID_ARG                   # shard runs past the row
    assert bshard(V=50) == lx.LX_ERR_INVALID_ARG
    assert bshard(grad=A + 64) == lx.LX_ERR_ALIAS                    # partial overlap with the student


def fwd_ex(student=A, lds=100, teacher=A + (1 << 31), ldt=100, target=A * 3, BT=4, V=100, ce=A * 4,
           tvd=A * 4 + 64, lse_s=A * 4 + 128, lse_t=A * 4 + 192, sigma=A * 4 + 256, dt=1):
    return L.lx_ce_tvd_forward_ex(student, lds, teacher, ldt, target, BT, V, -100, ce, tvd, lse_s, lse_t, sigma, dt,
                                  None, 0, None)


def bwd_ex(grad=A * 5, ldg=100, student=A, lds=100, teacher=A + (1 << 31), ldt=100, BT=4, V=100, gce=None,
           gtvd=None, dt=1):
    return L.lx_ce_tvd_backward_ex(grad, ldg, student, lds, teacher, ldt, A * 3, BT, V, -100, A * 4 + 128,
                                   A * 4 + 192, A * 4 + 256, 1.0, 1.0, gce, gtvd, None, dt, None)


def fwdbwd_ex(student=A, lds=100, teacher=A + (1 << 31), ldt=100, grad=A * 5, ldg=100, BT=4, V=100, gce=None,
              gtvd=None, dt=1):
    return L.lx_ce_tvd_forward_backward_ex(student, lds, teacher, ldt, A * 3, BT, V, -100, A * 4, A * 4 + 64,
                                           A * 4 + 128, A * 4 + 192, A * 4 + 256, grad, ldg, 1.0, 1.0, gce, gtvd,
                                           None, dt, None, 0, None)


def test_strided_entry_points_validation():
    for call in (fwd_ex, bwd_ex, fwdbwd_ex):
        assert call(BT=0) == lx.LX_OK                                  # no-op, strides not inspected
        assert call(dt=3) == lx.LX_ERR_UNSUPPORTED_DTYPE
        assert call(lds=99) == lx.LX_ERR_INVALID_ARG                   # row stride below V
        assert call(ldt=50) == lx.LX_ERR_INVALID_ARG
        assert call(BT=2**40, lds=2**30) == lx.LX_ERR_INVALID_ARG     # last row end not addressable
    for call in (bwd_ex, fwdbwd_ex):
        assert call(ldg=10) == lx.LX_ERR_INVALID_ARG
        assert call(gce=A * 6 + 2) == lx.LX_ERR_INVALID_ARG            # row factors float aligned
        assert call(grad=A, ldg=100, lds=120) == lx.LX_ERR_ALIAS        # in place needs the same stride
        assert call(gce=A * 5 + 64) == lx.LX_ERR_ALIAS                 # row factors inside the gradient
        assert call(gtvd=A * 5 + 600) == lx.LX_ERR_ALIAS
        # the strided span of the student covers (BT - 1) * ld + V elements (bf16: 2 bytes)
        assert call(lds=1000, grad=A + 2 * 2500) == lx.LX_ERR_ALIAS
    assert fwd_ex(lds=1000, ce=A + 2 * 2500) == lx.LX_ERR_ALIAS        # output inside the strided student
    assert fwdbwd_ex(gce=A * 4 + 64) == lx.LX_ERR_ALIAS                # row factors over an output


def test_binary16_logits_are_accepted():
    # LX_F16 (2): validation reaches the same checks as for bf16 (same element size)
    assert fwd(dt=2, tvd=A * 4) == lx.LX_ERR_ALIAS
    assert fwd(dt=2, student=A + 1) == lx.LX_ERR_INVALID_ARG
    assert bwd(dt=2, grad=A + 2) == lx.LX_ERR_ALIAS
    assert fwdbwd(dt=2, grad=A + 2) == lx.LX_ERR_ALIAS
    # the read-once / one-pass plans apply to 2-byte logits of either kind
    assert lx.lx_ce_tvd_workspace_bytes(8192, 151936, 2, 1) == lx.lx_ce_tvd_workspace_bytes(8192, 151936, 1, 1)
    assert lx.lx_ce_tvd_forward_backward_workspace_bytes(8192, 151936, 2, 0) == \
        lx.lx_ce_tvd_forward_backward_workspace_bytes(8192, 151936, 1, 0)


def test_gemm_validation():
    g = L.lx_gemm_bf16

    def call(A=A, lda=64, akc=1, B=A * 2, ldb=64, bkc=1, C=A * 3, ldc=32, M=16, N=32, K=64, acc=0):
        return g(A, lda, akc, B, ldb, bkc, C, ldc, M, N, K, acc, None)

    assert call(M=0) == lx.LX_ERR_INVALID_ARG
    assert call(K=2**31) == lx.LX_ERR_INVALID_ARG
    assert call(A=None) == lx.LX_ERR_INVALID_ARG
    assert call(K=60, lda=64, ldb=64) == lx.LX_ERR_INVALID_ARG          # K-contiguous operands need K % 8 == 0
    assert call(akc=0, M=12, lda=16) == lx.LX_ERR_INVALID_ARG           # M-contiguous A needs M % 8 == 0
    assert call(bkc=0, N=36, ldb=40, ldc=36) == lx.LX_ERR_INVALID_ARG   # N-contiguous B needs N % 8 == 0
    assert call(lda=60) == lx.LX_ERR_INVALID_ARG                         # row stride below the row
    assert call(lda=68) == lx.LX_ERR_INVALID_ARG                         # row stride not a multiple of 8
    assert call(ldc=31) == lx.LX_ERR_INVALID_ARG
    assert call(A=A + 8) == lx.LX_ERR_INVALID_ARG                        # 16-byte alignment
    assert call(C=A * 3 + 2) == lx.LX_ERR_INVALID_ARG
    assert call(C=A + 64) == lx.LX_ERR_ALIAS                             # C over A
    assert call(C=A * 2 + 1024) == lx.LX_ERR_ALIAS                       # C over B


def test_linear_validation():
    f = L.lx_ce_tvd_linear_forward_backward
    ws_need = lx.lx_ce_tvd_linear_workspace_bytes(300, 8200, 136, 1, 128)
    # per logit of a 128-row chunk: binary16 p (then G, in place: 2 B) and a tie bit; besides: per-tile
    # partials, the target logits and split-K partials of grad_x (at most 8 splits of a 128 x 136 fp32
    # block).  No logit is stored and nothing is transposed.
    per_logit = 128 * 8200
    assert per_logit * 2 <= ws_need
    assert ws_need <= (per_logit * (2 + 1 / 8) + 300 * 4 * (1 + 5 * 33) + 128 * 8 * 65 + 8 * 128 * 136 * 4 + 4096)
    assert lx.lx_ce_tvd_linear_workspace_bytes(300, 8200, 136, 0, 128) < ws_need
    ws_need = lx.lx_ce_tvd_linear_workspace_bytes(300, 8200, 64, 1, 128)  # the calls below: H = 64
    assert lx.lx_ce_tvd_linear_workspace_bytes(0, 8200, 136, 1, 128) == 0
    assert lx.lx_ce_tvd_linear_workspace_bytes(300, 8200, 136, 1, 0) == 0
    assert lx.lx_ce_tvd_linear_workspace_bytes(300, 8200, 0, 1, 128) == 0

    def call(xs=A, ws=A * 2, Hs=64, xt=A * 3, wt=A * 4, Ht=64, t=A * 5, BT=300, V=8200, ce=A * 6,
             tvd=A * 6 + 4096, lse_s=A * 6 + 8192, lse_t=A * 6 + 12288, sigma=A * 6 + 16384, gx=A * 7, gw=A * 8,
             chunk=128, wsp=A * 16, wsb=ws_need):
        return f(xs, ws, Hs, xt, wt, Ht, t, BT, V, -100, ce, tvd, lse_s, lse_t, sigma, gx, gw, 1.0, 1.0, None, chunk,
                 wsp, wsb, None)

    assert call(BT=0) == lx.LX_OK
    assert call(V=8196) == lx.LX_ERR_INVALID_ARG          # V % 8
    assert call(Hs=60) == lx.LX_ERR_INVALID_ARG           # H % 8
    assert call(Ht=0) == lx.LX_ERR_INVALID_ARG
    assert call(chunk=0) == lx.LX_ERR_INVALID_ARG
    assert call(wt=None) == lx.LX_ERR_INVALID_ARG         # teacher needs both x_t and w_t
    assert call(sigma=None) == lx.LX_ERR_INVALID_ARG
    assert call(xs=A + 8) == lx.LX_ERR_INVALID_ARG        # 16-byte alignment
    assert call(gx=A * 6 + 64) == lx.LX_ERR_ALIAS         # gradient over an output
    assert call(gw=A * 2 + 64) == lx.LX_ERR_ALIAS         # gradient over the weight
    assert call(ce=A * 16 + 64) == lx.LX_ERR_ALIAS        # output inside the workspace
    assert call(wsp=None) == lx.LX_ERR_WORKSPACE
    assert call(wsb=ws_need - 1) == lx.LX_ERR_WORKSPACE
    assert call(wsp=A * 16 + 128) == lx.LX_ERR_WORKSPACE  # 256-byte alignment
