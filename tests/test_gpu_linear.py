"""The lm_head product + CE + TVD path on the GPU, through the C ABI.

* The bf16 matrix product on the matrix cores (lx_gemm_bf16), all eight
  combinations of operand layouts and accumulation, on shapes with ragged
  tiles in M, N and K: with small-integer inputs every product and sum is
  exact in fp32, so the result must equal the integer product bit for bit
  (any indexing or layout mistake shows); with normal inputs and long K,
  within the fp32 accumulation bound.
* lx_ce_tvd_linear_forward_backward against the float64 oracle (exact
  logits, loss, G, and the chain rule through x w^T): several chunkings,
  ragged last chunks, CE+TVD and CE-only, the row and split-V forward paths.
  The gradients of x and w carry G rounded to bf16, so their bound is
  2^-8 relative to the matching product of magnitudes, |G| |w| and |G|^T |x|,
  plus the fp32 accumulation bound K 2^-23 of the same magnitudes.
* The one pass over the fp32 logits element by element: with identity hidden
  states the logits are exact and grad_w = G^T exactly, so G is checked like
  the one-pass kernels' gradient (member counts with and without an LDS part,
  a short last member, both the fp16-p and the logits-reloading step 3).
* The benchmark's configuration (8192 x 151936, hidden size 4096) on sampled
  rows, and the identity <dW, w> = <dX, x> (both equal <G, z>).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _parity import DEV, G_REL_P16, TIE_ABS, TIE_REL, announce, bits32, check_forward, check_grad, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cross_entropy_tv_amd as lx  # noqa: E402

II = W.IGNORE_INDEX
U23 = 2.0 ** -23


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(np.ascontiguousarray(bits, dtype=np.uint16))


def small_ints(rng, shape):
    vals = rng.integers(-4, 5, size=shape).astype(np.float32)
    return W.bf16_bits_rne(vals), vals.astype(np.float64)


def stored(bits_mk: np.ndarray, k_contiguous: bool, pad: int):
    """The (rows, K) logical operand stored K-contiguous (as is) or transposed, in
    an array with `pad` extra columns (a row stride larger than the row)."""
    arr = bits_mk if k_contiguous else np.ascontiguousarray(bits_mk.T)
    r, c = arr.shape
    big = np.zeros((r, c + pad), dtype=np.uint16)
    big[:, :c] = arr
    t = bf16_dev(big)
    return t[:, :c]


@pytest.mark.parametrize("accumulate", [False, True], ids=["overwrite", "accumulate"])
@pytest.mark.parametrize("a_kc,b_kc", [(True, True), (True, False), (False, True), (False, False)],
                         ids=["AK_BK", "AK_BN", "AM_BK", "AM_BN"])
@pytest.mark.parametrize("M,N,K", [(304, 520, 136), (8, 8, 8), (520, 264, 1000), (256, 256, 64)],
                         ids=["304x520x136", "8x8x8", "520x264x1000", "256x256x64"])
def test_gemm_exact_on_small_integers(M, N, K, a_kc, b_kc, accumulate):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a_bits, a = small_ints(rng, (M, K))
    b_bits, b = small_ints(rng, (N, K))
    c0 = rng.integers(-50, 51, size=(M, N)).astype(np.float32)
    ref = a @ b.T + (c0 if accumulate else 0.0)
    announce(f"gemm exact {M}x{N}x{K} a_kc {a_kc} b_kc {b_kc} acc {accumulate}")
    A = stored(a_bits, a_kc, 8)
    B = stored(b_bits, b_kc, 16)
    Cbig = torch.full((M, N + 3), 7.5, dtype=torch.float32, device=DEV)
    Cbig[:, :N] = torch.from_numpy(c0).to(DEV)
    lx.lx_gemm_bf16(A, a_kc, B, b_kc, Cbig[:, :N], M, N, K, accumulate)
    torch.cuda.synchronize()
    got = Cbig.cpu().numpy()
    assert np.array_equal(got[:, :N], ref.astype(np.float32)), \
        f"max err {np.abs(got[:, :N] - ref).max()} at {np.unravel_index(np.argmax(np.abs(got[:, :N] - ref)), ref.shape)}"
    assert np.all(got[:, N:] == 7.5), "wrote past column N"


@pytest.mark.parametrize("a_kc,b_kc", [(True, True), (True, False), (False, False)], ids=["AK_BK", "AK_BN", "AM_BN"])
def test_gemm_long_k_within_accumulation_bound(a_kc, b_kc):
    M, N, K = 264, 392, 8200
    rng = np.random.default_rng(99)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    a_bits, b_bits = W.bf16_bits_rne(a), W.bf16_bits_rne(b)
    a64, b64 = oracle.decode(a_bits), oracle.decode(b_bits)
    ref = a64 @ b64.T
    mag = np.abs(a64) @ np.abs(b64).T
    announce(f"gemm long K {M}x{N}x{K} a_kc {a_kc} b_kc {b_kc}")
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    lx.lx_gemm_bf16(stored(a_bits, a_kc, 0), a_kc, stored(b_bits, b_kc, 0), b_kc, C, M, N, K)
    torch.cuda.synchronize()
    err = np.abs(C.cpu().numpy() - ref)
    assert np.all(err <= K * U23 * mag), "outside the fp32 accumulation bound"
    assert np.max(err / mag) < 1e-5, f"typical error {np.max(err / mag)} relative to sum |a b|"


def run_linear(x_s, w_s, x_t, w_t, t, g_ce, g_tvd, chunk_rows, g_scale=None, grads=True):
    BT, H_s = x_s.shape
    V = w_s.shape[0]
    teacher = x_t is not None
    f = lambda: torch.full((BT,), 12345.0, dtype=torch.float32, device=DEV)  # noqa: E731
    out = {"ce": f(), "lse_s": f()}
    if teacher:
        out.update(tvd=f(), lse_t=f(), sigma=f())
    gx = torch.full((BT, H_s), 12345.0, dtype=torch.float32, device=DEV) if grads else None
    gw = torch.full((V, H_s), 12345.0, dtype=torch.float32, device=DEV) if grads else None
    lx.lx_ce_tvd_linear_forward_backward(bf16_dev(x_s), bf16_dev(w_s), None if x_t is None else bf16_dev(x_t),
                                         None if w_t is None else bf16_dev(w_t), to_dev(t), II, out["ce"],
                                         out.get("tvd"), out["lse_s"], out.get("lse_t"), out.get("sigma"), gx, gw,
                                         g_ce, g_tvd, g_scale, chunk_rows)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, gx, gw


def grad_bounds(ref, x_s, w_s, t, teacher, g_tvd, with_w=True):
    """Per-element bounds of grad_x_s and grad_w_s (None unless with_w) from the
    arithmetic (see the module docstring)."""
    xs, ws = oracle.decode(x_s), oracle.decode(w_s)
    G = np.abs(ref["grad"])
    if teacher:
        valid = t != II
        z, u = ref["z"][valid], ref["u"][valid]
        p = oracle.probs_rows(z, oracle.logsumexp_rows(z))
        q = oracle.probs_rows(u, oracle.logsumexp_rows(u))
        d = np.abs(p - q)
        tie = (d < TIE_ABS) | (d <= TIE_REL * np.maximum(p, q))
        slack = 2.0 * np.sum(np.where(tie, p, 0.0), axis=1)
        G[valid] += abs(g_tvd) * p * (tie + 0.5 * slack[:, None])   # any sign branch at near ties
    V, H = ws.shape
    BT = xs.shape[0]
    bx = (2.0 ** -8 + V * U23) * (G @ np.abs(ws)) + 1e-12
    bw = (2.0 ** -8 + BT * U23) * (G.T @ np.abs(xs)) + 1e-12 if with_w else None
    return bx, bw


@pytest.mark.parametrize("teacher", [True, False], ids=["ce_tvd", "ce_only"])
@pytest.mark.parametrize("BT,V,H_s,H_t,chunk", [(300, 8200, 136, 200, 300), (300, 8200, 136, 200, 128),
                                                (600, 4096, 64, 96, 600), (600, 4096, 64, 96, 1000),
                                                (37, 2056, 256, 128, 16), (12, 2056, 256, 128, 2)],
                         ids=["300x8200_one_chunk", "300x8200_chunks_128", "600x4096_rowpath",
                              "600x4096_chunk_above_rows", "37x2056_chunks_16",
                              # chunks too short for the transposed copies of G and x to fit
                              # over the logits: grad_w from G and x as they are
                              "12x2056_chunks_2"])
def test_linear_matches_the_oracle(BT, V, H_s, H_t, chunk, teacher):
    x_s, w_s, x_t, w_t, t = W.linear_inputs(BT, V, H_s, H_t if teacher else None, seed=BT + V + H_s)
    g_ce, g_tvd = 0.5, 1.5
    label = f"linear {BT}x{V} H {H_s}/{H_t} chunk {chunk} {'ce_tvd' if teacher else 'ce_only'}"
    announce(label)
    out, gx, gw = run_linear(x_s, w_s, x_t, w_t, t, g_ce, g_tvd, chunk)
    ref = oracle.linear_forward_backward(x_s, w_s, x_t, w_t, t, II, g_ce, g_tvd)
    check_forward(out, ref["z"], ref["u"], t, II, label)
    bx, bw = grad_bounds(ref, x_s, w_s, t, teacher, g_tvd)
    ex = np.abs(gx.cpu().numpy() - ref["grad_x_s"])
    ew = np.abs(gw.cpu().numpy() - ref["grad_w_s"])
    assert np.all(ex <= bx), f"{label}: grad_x_s max excess {np.max(ex / bx)} of its bound"
    assert np.all(ew <= bw), f"{label}: grad_w_s max excess {np.max(ew / bw)} of its bound"
    assert np.all(gx.cpu().numpy()[t == II] == 0.0), "ignored rows must have a zero hidden-state gradient"


@pytest.mark.parametrize("BT,V,g_ce,g_tvd", [(64, 151936, 1e-3, 1e-3), (64, 151936, 0.5, 1.5), (40, 8200, 0.5, 1.5)],
                         ids=["64x151936_fp16_p", "64x151936_reloaded_p", "40x8200_ragged_members"])
def test_linear_one_pass_gradient_elementwise(BT, V, g_ce, g_tvd):
    """Identity hidden states (H = BT) make the logits the weights' columns exactly
    and grad_w_s = G^T exactly (one product per element), so the one pass over the
    fp32 logits is checked element by element: the outputs against the oracle and G
    within the gradient tolerance; 64 x 151936 runs K = 8 members with an LDS part,
    once with the gradient scale inside the fp16-p bound and once beyond it (the
    groups with a large p formed from their logits); 40 x 8200 has a short last
    member."""
    _, w_s, _, w_t, t = W.linear_inputs(BT, V, BT, BT, seed=BT + V, logit_scale=2.5 * np.sqrt(BT))
    eye = W.bf16_bits_rne(np.eye(BT, dtype=np.float32))
    label = f"linear one pass {BT}x{V} g {g_ce}/{g_tvd}"
    announce(label)
    out, _, gw = run_linear(eye, w_s, eye, w_t, t, g_ce, g_tvd, BT)
    z = oracle.decode(w_s).T.astype(np.float32)
    u = oracle.decode(w_t).T.astype(np.float32)
    check_forward(out, z, u, t, II, label)
    G = gw.cpu().numpy().T.astype(np.float64)
    valid = t != II
    assert np.all(G[~valid] == 0.0), f"{label}: ignored rows must have a zero gradient"
    bits = np.where(valid[:, None], bits32(G.astype(np.float32)), 0)
    check_grad(G, bits, z, u, t, II, g_ce, g_tvd, label, rel=G_REL_P16, sigma_gpu=out["sigma"])


def test_linear_forward_only_and_device_scale():
    """No gradient outputs: only the loss; with g_scale = 1 / n_valid from the count."""
    BT, V, H = 300, 8200, 136
    x_s, w_s, x_t, w_t, t = W.linear_inputs(BT, V, H, H, seed=5)
    announce("linear forward only, then with g_scale")
    out, _, _ = run_linear(x_s, w_s, x_t, w_t, t, 1.0, 1.0, 128, grads=False)
    ref = oracle.linear_forward_backward(x_s, w_s, x_t, w_t, t, II, 1.0, 1.0)
    check_forward(out, ref["z"], ref["u"], t, II, "linear forward only")
    inv = torch.empty(1, dtype=torch.float32, device=DEV)
    lx.lx_ce_tvd_count_valid(to_dev(t), II, None, inv)
    n = int((t != II).sum())
    out2, gx, gw = run_linear(x_s, w_s, x_t, w_t, t, 1.0, 1.0, 128, g_scale=inv)
    ref2 = oracle.linear_forward_backward(x_s, w_s, x_t, w_t, t, II, 1.0 / n, 1.0 / n)
    bx, bw = grad_bounds(ref2, x_s, w_s, t, True, 1.0 / n)
    assert np.all(np.abs(gx.cpu().numpy() - ref2["grad_x_s"]) <= bx)
    assert np.all(np.abs(gw.cpu().numpy() - ref2["grad_w_s"]) <= bw)


def test_linear_benchmark_configuration_sampled():
    """8192 rows x 151936 classes, hidden size 4096 for student and teacher, one
    chunk of 4096 rows: sampled rows against the oracle (forward outputs and the
    hidden-state gradient), and <dW, w> = <dX, x> on the whole result."""
    BT, V, H = 8192, 151936, 4096
    x_s, w_s, x_t, w_t, t = W.linear_inputs(BT, V, H, H, seed=77)
    announce(f"linear benchmark configuration {BT}x{V} H {H}")
    inv = torch.empty(1, dtype=torch.float32, device=DEV)
    tg = to_dev(t)
    lx.lx_ce_tvd_count_valid(tg, II, None, inv)
    f = lambda: torch.empty(BT, dtype=torch.float32, device=DEV)  # noqa: E731
    out = {"ce": f(), "tvd": f(), "lse_s": f(), "lse_t": f(), "sigma": f()}
    gx = torch.empty((BT, H), dtype=torch.float32, device=DEV)
    gw = torch.empty((V, H), dtype=torch.float32, device=DEV)
    X, Wd = bf16_dev(x_s), bf16_dev(w_s)
    lx.lx_ce_tvd_linear_forward_backward(X, Wd, bf16_dev(x_t), bf16_dev(w_t), tg, II, out["ce"], out["tvd"],
                                         out["lse_s"], out["lse_t"], out["sigma"], gx, gw, 1.0, 1.0, inv,
                                         chunk_rows=4096)
    torch.cuda.synchronize()
    assert torch.isfinite(gx).all() and torch.isfinite(gw).all()
    # <dW, w> = <dX, x> = <G, z>
    lhs = float((gw.double() * Wd.double()).sum())
    rhs = float((gx.double() * X.double()).sum())
    mag = float((gw.double() * Wd.double()).abs().sum() + (gx.double() * X.double()).abs().sum())
    assert abs(lhs - rhs) <= 2.0 ** -7 * mag, (lhs, rhs, mag)
    rows = np.array([0, 1, 2, 4095, 4096, 6000, BT - 1])
    n = int((t != II).sum())
    ref = oracle.linear_forward_backward(x_s[rows], w_s, x_t[rows], w_t, t[rows], II, 1.0 / n, 1.0 / n)
    o = {k: v.cpu().numpy()[rows] for k, v in out.items()}
    check_forward(o, ref["z"], ref["u"], t[rows], II, "linear benchmark configuration")
    bx, _ = grad_bounds(ref, x_s[rows], w_s, t[rows], True, 1.0 / n, with_w=False)
    ex = np.abs(gx.cpu().numpy()[rows] - ref["grad_x_s"])
    assert np.all(ex <= bx), f"grad_x_s max excess {np.max(ex / bx)}"
