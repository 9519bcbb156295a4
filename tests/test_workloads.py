"""The seeded input generator: determinism, role mix, bf16 rounding (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 10, 100000).astype(np.float32),
                        # exact halfway cases between two bf16 values, both parities
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
                        np.array([0.0, -0.0, 1.0, -2.5, 3.3895e38, 1e-40], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.bf16_bits_rne(x), ref)
    assert np.array_equal(W.bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_roles_and_targets():
    counts = {n: np.bincount(W.roles(W.get(n)), minlength=4).tolist() for n in W.WORKLOADS}
    assert counts["tiny"] == [7, 1, 0, 0] and W.roles(W.get("tiny"))[3] == W.ROLE_IGNORED
    assert counts["pr"] == [973, 51, 0, 0]
    assert counts["train"] == [8192, 0, 0, 0]
    assert counts["ties"] == [12289, 819, 1638, 1638]
    assert counts["hugev"] == [64, 0, 0, 0]
    for n in W.WORKLOADS:
        w = W.get(n)
        t = W.targets(w)
        ign = W.roles(w) == W.ROLE_IGNORED
        assert t.dtype == np.int64 and t.shape == (w.BT,)
        assert np.all(t[ign] == W.IGNORE_INDEX) and np.all((t[~ign] >= 0) & (t[~ign] < w.V))


@pytest.mark.parametrize("name", ["tiny", "pr", "ties", "train", "hugev"])
def test_rows_are_deterministic_and_order_free(name):
    w = W.get(name)
    idx = [5, 2, 3, 0]
    z1, u1 = W.rows(w, idx)
    z2, u2, _ = W.full(w, rows_limit=6, threads=3)
    assert np.array_equal(z1, z2[idx]) and np.array_equal(u1, u2[idx])
    z3, u3 = W.rows(w, idx)
    assert np.array_equal(z1, z3) and np.array_equal(u1, u3)
    assert z1.dtype == (np.float32 if w.dtype == "f32" else np.uint16)


def test_ties_rows_have_their_roles():
    w = W.get("ties")
    ro = W.roles(w)
    ident = np.nonzero(ro == W.ROLE_IDENTICAL)[0][:3]
    unif = np.nonzero(ro == W.ROLE_UNIFORM)[0][:3]
    z, u = W.rows(w, ident)
    assert np.array_equal(z, u)
    z, u = W.rows(w, unif)
    assert np.all(z == z[:, :1]) and not np.array_equal(z, u)


def test_train_rows_carry_spikes():
    w = W.get("train")
    z, u = W.rows(w, [0, 1])
    zf = W.bf16_bits_to_f32(z)
    # 32 replaced positions per row drawn from N(8, 2^2): ~27 of them above 6, while
    # N(0, 1.5^2) puts only ~5 of 151936 draws there
    n = (zf > 6.0).sum(1)
    assert np.all(n >= 15) and np.all(n <= 60), n


def test_page_memory_figures_reading():
    """The page's temporaries figures read as 6 bytes per (token, vocab) element in MiB."""
    g = json.load(open(os.path.join(HERE, "golden", "page_memory_figures.json")))
    per_token = 6 * g["V"] / 2**20
    assert round(per_token, 2) == g["temporaries_MB_per_token_unfused"]
    assert round(per_token * g["saved_MiB_at_tokens"]["tokens"]) == g["saved_MiB_at_tokens"]["MiB"]
