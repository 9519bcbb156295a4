"""The lm_head product + CE + TVD path on the GPU, through the C ABI.

* The bf16 matrix product on the matrix cores (lx_gemm_bf16, the library's
  own MFMA kernel), all eight combinations of operand layouts and
  accumulation, on shapes with ragged tiles in M, N and K: with small-integer
  inputs every product and sum is exact in fp32, so the result must equal the
  integer product bit for bit (any indexing or layout mistake shows); with
  normal inputs and long K, within the fp32 accumulation bound.
* lx_ce_tvd_linear_forward_backward against the float64 oracle (exact
  logits, loss, G, and the chain rule through x w^T): several chunkings,
  ragged last chunks and tiles, CE+TVD and CE-only.  The loss outputs are held
  to the loss's tolerances against the exact logits.  The gradients of x and
  w carry G, formed from binary16 p and rounded to bf16 (relative precision
  2^-8 + 2^-10), so their bound is that relative to the matching product of
  magnitudes, |G| |w| and |G|^T |x|, plus the fp32 accumulation bound K 2^-23
  of the same magnitudes; at near ties of p and q any sign branch is allowed.
* G element by element: with identity hidden states the logits are exact and
  grad_w = G^T exactly, so G is checked like the one-pass kernels' gradient
  (relative precision 2^-8 + 2^-10, sign branches read back at near ties).
* The benchmark's configuration (8192 x 151936, hidden size 4096, the batch as
  one chunk): the loss outputs and grad_x on sampled rows against the oracle
  and the identity <dW, w> = <dX, x> (both equal <G, z>) on the whole result;
  then the same launch with every row ignored but 16, so that the whole of
  grad_w (151936 x 4096) is the oracle's sum over those 16 rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _parity import DEV, G_REL_P16, announce, bits32, check_forward, check_grad, near_ties, to_dev

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
        rel, exempt = near_ties(p, q)
        slack = 2.0 * np.sum(np.where(rel, p, 0.0), axis=1)
        G[valid] += abs(g_tvd) * p * (exempt + 0.5 * slack[:, None])   # any sign branch at near ties
    V, H = ws.shape
    BT = xs.shape[0]
    bx = (G_REL_P16 + V * U23) * (G @ np.abs(ws)) + 1e-12
    bw = (G_REL_P16 + BT * U23) * (G.T @ np.abs(xs)) + 1e-12 if with_w else None
    return bx, bw


@pytest.mark.parametrize("teacher", [True, False], ids=["ce_tvd", "ce_only"])
@pytest.mark.parametrize("BT,V,H_s,H_t,chunk", [(300, 8200, 136, 200, 300), (300, 8200, 136, 200, 128),
                                                (600, 4096, 64, 96, 600), (600, 4096, 64, 96, 1000),
                                                (37, 2056, 256, 128, 16), (12, 2056, 256, 128, 2),
                                                (530, 1160, 1000, 520, 530), (5, 264, 8, 16, 5),
                                                (3, 8, 24, 8, 1)],
                         ids=["300x8200_one_chunk", "300x8200_chunks_128", "600x4096",
                              "600x4096_chunk_above_rows", "37x2056_chunks_16", "12x2056_chunks_2",
                              "530x1160_ragged_tiles", "5x264_hidden_8_16", "3x8_hidden_24_8_chunks_1"])
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
    print(f"{label}: grad_x err/bound {np.max(ex / bx):.3f}, grad_w err/bound {np.max(ew / bw):.3f}")
    assert np.all(ex <= bx), f"{label}: grad_x_s max excess {np.max(ex / bx)} of its bound"
    assert np.all(ew <= bw), f"{label}: grad_w_s max excess {np.max(ew / bw)} of its bound"
    assert np.all(gx.cpu().numpy()[t == II] == 0.0), "ignored rows must have a zero hidden-state gradient"


@pytest.mark.parametrize("BT,V,g_ce,g_tvd", [(64, 151936, 1e-3, 1e-3), (64, 151936, 0.5, 1.5), (40, 8200, 0.5, 1.5)],
                         ids=["64x151936_small_g", "64x151936_unit_g", "40x8200_ragged_tiles"])
def test_linear_one_pass_gradient_elementwise(BT, V, g_ce, g_tvd):
    """Identity hidden states (H = BT) make the logits the weights' columns exactly
    and grad_w_s = G^T exactly (one product per element), so G is checked element
    by element: the outputs against the oracle, and G, formed from binary16 p,
    within 2^-8 + 2^-10 relative (plus the scaled floor), at small and at unit
    upstream gradients; 40 x 8200 has ragged last tiles."""
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
    check_grad(G, bits, z, u, t, II, g_ce, g_tvd, label, rel=G_REL_P16, stated_rel=G_REL_P16, sigma_gpu=out["sigma"])


def test_linear_out_of_range_target_poisons_its_row_and_grad_w():
    """A target outside [0, V) that is not ignore_index: that row's ce and its
    grad_x row are NaN and, through the sum over rows, every element of grad_w;
    every other row matches the oracle run with that row ignored."""
    BT, V, H = 40, 264, 16
    x_s, w_s, x_t, w_t, t = W.linear_inputs(BT, V, H, H, seed=13)
    bad = 7
    t = t.copy()
    t[bad] = V + 5
    announce("linear: out-of-range target row 7")
    out, gx, gw = run_linear(x_s, w_s, x_t, w_t, t, 0.5, 1.5, BT)
    assert np.isnan(out["ce"][bad])
    assert np.all(np.isnan(gx.cpu().numpy()[bad]))
    assert np.all(np.isnan(gw.cpu().numpy()))
    t_ref = t.copy()
    t_ref[bad] = II
    ref = oracle.linear_forward_backward(x_s, w_s, x_t, w_t, t_ref, II, 0.5, 1.5)
    keep = np.arange(BT) != bad
    check_forward({k: v[keep] for k, v in out.items()}, ref["z"][keep], ref["u"][keep], t_ref[keep], II,
                  "linear out-of-range target, other rows")
    bx, _ = grad_bounds(ref, x_s, w_s, t_ref, True, 1.5, with_w=False)
    ex = np.abs(gx.cpu().numpy()[keep] - ref["grad_x_s"][keep])
    assert np.all(ex <= bx[keep]), f"grad_x of the other rows: max excess {np.max(ex / bx[keep])}"


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


def _full_size_call(X, Wd, Xt, Wt, t, chunk_rows):
    BT, H = X.shape
    V = Wd.shape[0]
    tg = to_dev(t)
    inv = torch.empty(1, dtype=torch.float32, device=DEV)
    lx.lx_ce_tvd_count_valid(tg, II, None, inv)
    f = lambda: torch.empty(BT, dtype=torch.float32, device=DEV)  # noqa: E731
    out = {"ce": f(), "tvd": f(), "lse_s": f(), "lse_t": f(), "sigma": f()}
    gx = torch.empty((BT, H), dtype=torch.float32, device=DEV)
    gw = torch.empty((V, H), dtype=torch.float32, device=DEV)
    lx.lx_ce_tvd_linear_forward_backward(X, Wd, Xt, Wt, tg, II, out["ce"], out["tvd"], out["lse_s"], out["lse_t"],
                                         out["sigma"], gx, gw, 1.0, 1.0, inv, chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    return out, gx, gw


@pytest.mark.timeout(900)
def test_linear_benchmark_configuration():
    """8192 rows x 151936 classes, hidden size 4096 for student and teacher, the batch
    as one chunk (the benchmark's call): sampled rows of the loss outputs and of
    grad_x against the oracle, <dW, w> = <dX, x> on the whole result; then the same
    call with all rows but 16 ignored, whose grad_w is the oracle's sum over the 16
    rows, compared on all of its 151936 x 4096 entries."""
    BT, V, H, chunk = 8192, 151936, 4096, 8192
    x_s, w_s, x_t, w_t, t = W.linear_inputs(BT, V, H, H, seed=77)
    announce(f"linear benchmark configuration {BT}x{V} H {H} chunk {chunk}")
    X, Wd, Xt, Wt = bf16_dev(x_s), bf16_dev(w_s), bf16_dev(x_t), bf16_dev(w_t)
    out, gx, gw = _full_size_call(X, Wd, Xt, Wt, t, chunk)
    assert torch.isfinite(gx).all() and torch.isfinite(gw).all()
    # <dW, w> = <dX, x> = <G, z>
    lhs = float((gw.double() * Wd.double()).sum())
    rhs = float((gx.double() * X.double()).sum())
    mag = float((gw.double() * Wd.double()).abs().sum() + (gx.double() * X.double()).abs().sum())
    assert abs(lhs - rhs) <= 2.0 ** -7 * mag, (lhs, rhs, mag)
    rows = np.array([0, 1, 2, 255, 256, 4095, 4096, 6000, BT - 1])
    n = int((t != II).sum())
    ref = oracle.linear_forward_backward(x_s[rows], w_s, x_t[rows], w_t, t[rows], II, 1.0 / n, 1.0 / n)
    o = {k: v.cpu().numpy()[rows] for k, v in out.items()}
    check_forward(o, ref["z"], ref["u"], t[rows], II, "linear benchmark configuration")
    bx, _ = grad_bounds(ref, x_s[rows], w_s, t[rows], True, 1.0 / n, with_w=False)
    ex = np.abs(gx.cpu().numpy()[rows] - ref["grad_x_s"])
    print(f"benchmark configuration: grad_x err/bound {np.max(ex / bx):.3f} on {len(rows)} rows")
    assert np.all(ex <= bx), f"grad_x_s max excess {np.max(ex / bx)}"
    del gx, gw, out
    # all rows ignored but 16: grad_w = sum over those rows of G_b^T x_b, everywhere
    keep = np.array(sorted(set(np.random.default_rng(5).choice(BT, 16, replace=False).tolist()) | {0, BT - 1}))
    keep = keep[t[keep] != II]
    t2 = np.full(BT, II, dtype=np.int64)
    t2[keep] = t[keep]
    out2, gx2, gw2 = _full_size_call(X, Wd, Xt, Wt, t2, chunk)
    k2 = 1.0 / len(keep)
    ref2 = oracle.linear_forward_backward(x_s[keep], w_s, x_t[keep], w_t, t2[keep], II, k2, k2)
    gxh = gx2.cpu().numpy()
    assert np.all(gxh[np.setdiff1d(np.arange(BT), keep)] == 0.0), "ignored rows' grad_x must be 0"
    bx2, bw2 = grad_bounds(ref2, x_s[keep], w_s, t2[keep], True, k2)
    ex2 = np.abs(gxh[keep] - ref2["grad_x_s"])
    ew2 = np.abs(gw2.cpu().numpy() - ref2["grad_w_s"])
    print(f"benchmark configuration, {len(keep)} rows kept: grad_x err/bound {np.max(ex2 / bx2):.3f}, "
          f"grad_w err/bound {np.max(ew2 / bw2):.3f} over all {V}x{H}")
    assert np.all(ex2 <= bx2), f"grad_x_s max excess {np.max(ex2 / bx2)}"
    assert np.all(ew2 <= bw2), f"grad_w_s max excess {np.max(ew2 / bw2)}"
