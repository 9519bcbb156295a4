"""Seeded synthetic logits for the fused cross-entropy + total-variation loss.

This module only draws inputs: student logits, teacher logits, targets and the
role of every row.  It holds none of the loss arithmetic, and both the float64
oracle and the HIP path take their inputs from here.

Five workloads, named by what they are (rows x vocabulary, logits dtype):

* ``tiny``  : 8 x 1024, f32, logits ~ N(0, 2^2) i.i.d.; row 3 carries the
  ignore index; upstream gradients 1/num_valid_rows.
* ``pr``    : 1024 x 151936, bf16; student ~ N(0, 3^2), teacher = student +
  N(0, 0.5^2); 5% of rows ignored (51 rows); mean-reduced, in-place gradient.
  Stands in for the workload the PR #1384 analysis page quotes its memory
  figures on (V = 151936, bf16, 1024 tokens).
* ``train`` : 8192 x 151936, bf16; N(0, 1.5^2) logits with 32 spike positions
  per row whose value is replaced by an N(8, 2^2) draw; teacher from an
  independent stream with the same law; no ignored rows.
* ``ties``  : 16384 x 151936, bf16; 10% of rows have teacher == student
  exactly, 10% have a constant student row, 5% are ignored, the rest follow
  the ``pr`` law.
* ``hugev`` : 64 x 262144, bf16; N(0, 2^2) plus a per-row offset drawn from
  U(-20, 20), independently for student and teacher.

Every row is drawn from its own counter-keyed stream
(``SeedSequence(ENTROPY, spawn_key=(workload_id, stream, row))``), so any
subset of rows can be regenerated on its own, in any order and on any number
of threads, and comes out bit-identical.  bf16 values are produced by
rounding float32 draws to nearest-even on their bit patterns; bf16 tensors
are returned as their raw uint16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ENTROPY = 20261202
IGNORE_INDEX = -100

# row roles
ROLE_NORMAL = 0
ROLE_IGNORED = 1
ROLE_IDENTICAL = 2   # teacher row == student row, bit for bit
ROLE_UNIFORM = 3     # every student logit of the row equal

# stream ids inside a workload
_S_META = 0
_S_STUDENT = 1
_S_TEACHER = 2
_S_TARGET = 3


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    BT: int
    V: int
    dtype: str          # "f32" or "bf16"
    has_teacher: bool = True

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def np_raw_dtype(self):
        return np.float32 if self.dtype == "f32" else np.uint16


WORKLOADS = {
    "tiny": Workload(1, "tiny", 8, 1024, "f32"),
    "pr": Workload(2, "pr", 1024, 151936, "bf16"),
    "train": Workload(3, "train", 8192, 151936, "bf16"),
    "ties": Workload(4, "ties", 16384, 151936, "bf16"),
    "hugev": Workload(5, "hugev", 64, 262144, "bf16"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(wid: int, stream: int, row: int | None = None) -> np.random.Generator:
    key = (wid, stream) if row is None else (wid, stream, row)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ENTROPY, spawn_key=key)))


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest, ties to even.

    Inputs are finite.  This is input preparation (how the synthetic bf16
    logits are made), not part of the loss.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (exact widening)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def roles(w: Workload) -> np.ndarray:
    """Role code of every row (int8, shape [BT])."""
    r = np.full(w.BT, ROLE_NORMAL, dtype=np.int8)
    if w.name == "tiny":
        r[3] = ROLE_IGNORED
    elif w.name == "pr":
        perm = _rng(w.wid, _S_META).permutation(w.BT)
        r[perm[: int(round(0.05 * w.BT))]] = ROLE_IGNORED
    elif w.name == "ties":
        perm = _rng(w.wid, _S_META).permutation(w.BT)
        n10, n5 = int(round(0.10 * w.BT)), int(round(0.05 * w.BT))
        r[perm[:n10]] = ROLE_IDENTICAL
        r[perm[n10:2 * n10]] = ROLE_UNIFORM
        r[perm[2 * n10:2 * n10 + n5]] = ROLE_IGNORED
    return r


def targets(w: Workload) -> np.ndarray:
    """Target class of every row (int64, shape [BT]); ignored rows carry IGNORE_INDEX."""
    rng = _rng(w.wid, _S_TARGET)
    t = rng.integers(0, w.V, size=w.BT, dtype=np.int64)
    t[roles(w) == ROLE_IGNORED] = IGNORE_INDEX
    return t


def _distinct_positions(rng: np.random.Generator, V: int, k: int) -> np.ndarray:
    """k distinct uniform positions in [0, V), in draw order."""
    out: list[int] = []
    seen: set[int] = set()
    while len(out) < k:
        for v in rng.integers(0, V, size=k + 8, dtype=np.int64).tolist():
            if v not in seen:
                seen.add(v)
                out.append(v)
                if len(out) == k:
                    break
    return np.asarray(out, dtype=np.int64)


def _row(w: Workload, r: int, role: int):
    """(student_raw, teacher_raw or None) for one row."""
    V = w.V
    gs = _rng(w.wid, _S_STUDENT, r)
    gt = _rng(w.wid, _S_TEACHER, r)
    if w.name == "tiny":
        z = gs.standard_normal(V, dtype=np.float32) * np.float32(2.0)
        u = gt.standard_normal(V, dtype=np.float32) * np.float32(2.0)
        return z, u
    if w.name == "train":
        def draw(g):
            x = g.standard_normal(V, dtype=np.float32) * np.float32(1.5)
            pos = _distinct_positions(g, V, 32)
            x[pos] = (g.standard_normal(32, dtype=np.float32) * np.float32(2.0) + np.float32(8.0))
            return bf16_bits_rne(x)
        return draw(gs), draw(gt)
    if w.name == "hugev":
        def draw(g):
            off = np.float32(g.uniform(-20.0, 20.0))
            x = g.standard_normal(V, dtype=np.float32) * np.float32(2.0) + off
            return bf16_bits_rne(x)
        return draw(gs), draw(gt)
    # "pr" and "ties": teacher = student + N(0, 0.5^2), rounded to bf16
    if role == ROLE_UNIFORM:
        c = bf16_bits_rne(np.asarray([gs.standard_normal(dtype=np.float32) * np.float32(3.0)]))[0]
        z = np.full(V, c, dtype=np.uint16)
    else:
        z = bf16_bits_rne(gs.standard_normal(V, dtype=np.float32) * np.float32(3.0))
    if role == ROLE_IDENTICAL:
        return z, z.copy()
    noise = gt.standard_normal(V, dtype=np.float32) * np.float32(0.5)
    u = bf16_bits_rne(bf16_bits_to_f32(z) + noise)
    return z, u


def rows(w: Workload, idx, role_arr: np.ndarray | None = None):
    """Student and teacher raw rows for the row indices ``idx`` (any order)."""
    idx = np.asarray(idx, dtype=np.int64).reshape(-1)
    ro = roles(w) if role_arr is None else role_arr
    zs = np.empty((idx.size, w.V), dtype=w.np_raw_dtype)
    us = np.empty((idx.size, w.V), dtype=w.np_raw_dtype)
    for k, r in enumerate(idx.tolist()):
        z, u = _row(w, r, int(ro[r]))
        zs[k] = z
        us[k] = u
    return zs, us


def full(w: Workload, threads: int | None = None, rows_limit: int | None = None):
    """All rows (or the first ``rows_limit``): (student_raw, teacher_raw, target)."""
    n = w.BT if rows_limit is None else min(rows_limit, w.BT)
    ro = roles(w)
    zs = np.empty((n, w.V), dtype=w.np_raw_dtype)
    us = np.empty((n, w.V), dtype=w.np_raw_dtype)

    def fill(lo_hi):
        lo, hi = lo_hi
        for r in range(lo, hi):
            z, u = _row(w, r, int(ro[r]))
            zs[r] = z
            us[r] = u

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    step = max(1, -(-n // (threads * 4)))
    chunks = [(lo, min(n, lo + step)) for lo in range(0, n, step)]
    if threads <= 1 or len(chunks) == 1:
        for c in chunks:
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, chunks))
    return zs, us, targets(w)[:n]


def custom(BT: int, V: int, dtype: str, seed: int, scale: float = 2.0, teacher_noise: float | None = None,
           ignore_rows=(), identical_rows=(), uniform_rows=(), offset_range: float = 0.0):
    """Seeded inputs of any shape for parity cases that are not one of the named workloads.

    Student ~ N(0, scale^2) (+ a per-row offset ~ U(-offset_range, offset_range));
    teacher independent with the same law, or student + N(0, teacher_noise^2)
    when ``teacher_noise`` is given.  Rows listed in ``identical_rows`` get a
    bit-identical teacher, rows in ``uniform_rows`` a constant student row, rows
    in ``ignore_rows`` the ignore index.  ``dtype`` is "f32", "bf16" or "f16"
    (binary16, rounded to nearest even from the float32 draws).  Returns
    (student_raw, teacher_raw, target) with bf16 as uint16 bit patterns.
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(ENTROPY, spawn_key=(1000 + seed,))))
    z = g.standard_normal((BT, V), dtype=np.float32) * np.float32(scale)
    if offset_range:
        z += g.uniform(-offset_range, offset_range, size=(BT, 1)).astype(np.float32)
    for r in uniform_rows:
        z[r] = z[r, 0]
    if teacher_noise is None:
        u = g.standard_normal((BT, V), dtype=np.float32) * np.float32(scale)
        if offset_range:
            u += g.uniform(-offset_range, offset_range, size=(BT, 1)).astype(np.float32)
    if dtype == "bf16":
        zr = bf16_bits_rne(z)
        if teacher_noise is not None:
            u = bf16_bits_to_f32(zr) + g.standard_normal((BT, V), dtype=np.float32) * np.float32(teacher_noise)
        ur = bf16_bits_rne(u)
    elif dtype == "f16":
        zr = z.astype(np.float16)  # IEEE binary16, round to nearest even
        if teacher_noise is not None:
            u = zr.astype(np.float32) + g.standard_normal((BT, V), dtype=np.float32) * np.float32(teacher_noise)
        ur = u.astype(np.float16)
    else:
        zr = z
        if teacher_noise is not None:
            u = z + g.standard_normal((BT, V), dtype=np.float32) * np.float32(teacher_noise)
        ur = u.astype(np.float32)
    for r in identical_rows:
        ur[r] = zr[r]
    t = g.integers(0, V, size=BT, dtype=np.int64)
    for r in ignore_rows:
        t[r] = IGNORE_INDEX
    return np.ascontiguousarray(zr), np.ascontiguousarray(ur), t


def linear_inputs(BT: int, V: int, H_s: int, H_t: int | None, seed: int, logit_scale: float = 2.5,
                  ignore_frac: float = 0.05):
    """Seeded inputs of the lm_head variant: hidden states x ~ N(0, 1) and weights
    w ~ N(0, (logit_scale / sqrt(H))^2), so the logits x w^T have standard deviation
    about ``logit_scale``; teacher drawn independently (``H_t=None``: no teacher);
    targets uniform, round(ignore_frac * BT) rows ignored.  bf16 bit patterns
    (uint16), rounded to nearest even.  Returns (x_s, w_s, x_t, w_t, target)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(ENTROPY, spawn_key=(2000 + seed,))))

    def draw(shape, std):
        return bf16_bits_rne(g.standard_normal(shape, dtype=np.float32) * np.float32(std))

    x_s = draw((BT, H_s), 1.0)
    w_s = draw((V, H_s), logit_scale / np.sqrt(H_s))
    x_t = w_t = None
    if H_t:
        x_t = draw((BT, H_t), 1.0)
        w_t = draw((V, H_t), logit_scale / np.sqrt(H_t))
    t = g.integers(0, V, size=BT, dtype=np.int64)
    t[g.permutation(BT)[: int(round(ignore_frac * BT))]] = IGNORE_INDEX
    return x_s, w_s, x_t, w_t, t
