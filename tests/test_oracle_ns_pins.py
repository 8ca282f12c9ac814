"""Pins of the oracle's block mask inside flat query blocks (reading R21:
alpha_ns > 0), against what the pages and the mathematics fix.

[notes] key design 2: a (query block, key block) pair takes the exact online
softmax when its mask is 1 and the representative (K^c, V^c, weight = block
length) otherwise; [summary] 4 "Hyperparameters in ISA": alpha_ns, the
no-sparsity ratio.  The pins: the count's rounding; the selection against a
brute-force sort; the two limits (no exact block = the Taylor path, every
block exact = textbook attention over K_new); representatives that equal
their tokens (block-constant K, V, or b = 1) make any mask exact; the key
shift invariance of every softmax row; nested selections as alpha_ns grows.
"""

import itertools
import math

import numpy as np
import pytest

import oracle as orc
from synth import generate


def _rng(seed):
    return np.random.default_rng(seed)


def test_ns_count_rounding_and_clamp():
    assert orc.ns_count(0.0625, 320) == 20       # the pages' default at 320 kept blocks
    assert orc.ns_count(0.0, 320) == 0
    assert orc.ns_count(1.0, 320) == 320
    assert orc.ns_count(1.0 / 3.0, 3) == 1       # an integer product stays that integer
    assert orc.ns_count(0.01, 7) == 1            # any positive ratio keeps at least one block
    assert orc.ns_count(0.5, 0) == 0


def test_top_ns_brute_force_with_ties():
    rng = _rng(5)
    for trial in range(40):
        n = int(rng.integers(1, 12))
        p = rng.integers(0, 4, size=n) / 4.0     # many exact ties
        for k in range(n + 1):
            got = orc.top_ns_blocks(p, k)
            order = sorted(range(n), key=lambda u: (-p[u], u))
            assert list(got) == sorted(order[:k])
            if 0 < k < n:
                chosen = set(got.tolist())
                worst_in = min(p[u] for u in chosen)
                best_out = max(p[u] for u in range(n) if u not in chosen)
                assert worst_in >= best_out


def _mixed_inputs(seed, n_blocks=5, b=4, D=8, R=6):
    rng = _rng(seed)
    w = np.full(n_blocks, float(b))
    K_new = rng.normal(size=(n_blocks * b, D))
    V_new = rng.normal(size=(n_blocks * b, D))
    Kc = K_new.reshape(n_blocks, b, D).mean(axis=1)
    Vc = V_new.reshape(n_blocks, b, D).mean(axis=1)
    Q = rng.normal(size=(R, D)) * 1.5
    return Q, K_new, V_new, Kc, Vc, w


def test_mixed_without_exact_blocks_is_the_taylor_path():
    Q, K_new, V_new, Kc, Vc, w = _mixed_inputs(11)
    o1, l1 = orc.mixed_attention(Q, K_new, V_new, Kc, Vc, w, [])
    o2, l2 = orc.taylor_attention(Q, Kc, Vc, w)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


def test_mixed_with_every_block_exact_is_attention_over_k_new():
    Q, K_new, V_new, Kc, Vc, w = _mixed_inputs(12)
    o1, l1 = orc.mixed_attention(Q, K_new, V_new, Kc, Vc, w, np.arange(len(w)))
    o2, l2 = orc.dense_ref(Q[None, None], K_new[None, None], V_new[None, None])
    assert np.abs(o1 - o2[0, 0]).max() < 1e-12 and np.abs(l1 - l2[0, 0]).max() < 1e-12


@pytest.mark.parametrize("subset", [(), (0,), (2, 4), (0, 1, 3), (0, 1, 2, 3, 4)])
def test_mixed_block_constant_keys_values_is_exact(subset):
    rng = _rng(13)
    n_blocks, b, D = 5, 4, 8
    Kc = rng.normal(size=(n_blocks, D))
    Vc = rng.normal(size=(n_blocks, D))
    K_new = np.repeat(Kc, b, axis=0)
    V_new = np.repeat(Vc, b, axis=0)
    Q = rng.normal(size=(6, D))
    w = np.full(n_blocks, float(b))
    o1, l1 = orc.mixed_attention(Q, K_new, V_new, Kc, Vc, w, list(subset))
    o2, l2 = orc.dense_ref(Q[None, None], K_new[None, None], V_new[None, None])
    assert np.abs(o1 - o2[0, 0]).max() < 1e-12 and np.abs(l1 - l2[0, 0]).max() < 1e-12


def test_mixed_block_one_is_exact_for_any_mask():
    Q, K_new, V_new, _, _, _ = _mixed_inputs(14, n_blocks=6, b=1)
    w = np.ones(6)
    ref = orc.dense_ref(Q[None, None], K_new[None, None], V_new[None, None])
    for subset in itertools.combinations(range(6), 2):
        o, l = orc.mixed_attention(Q, K_new, V_new, K_new, V_new, w, list(subset))
        assert np.abs(o - ref[0][0, 0]).max() < 1e-12 and np.abs(l - ref[1][0, 0]).max() < 1e-12


def _small(seed, L_src=256, L_ctx=256, D=16, B=1, H=2):
    inp = generate(B, H, L_src, L_ctx, D, 64, seed=seed, variant="icl", dtype="fp32")
    return inp["q"], inp["k"], inp["v"]


def test_isa_every_flat_block_exact_is_the_exact_path():
    Q, K, V = _small(21)
    L_src = L_ctx = 256
    out = orc.isa_ref(Q, K, V, L_src, L_ctx, 64, 0.5, 0.5, alpha_ns=1.0)
    n_kv = 4 + 2
    assert out["ns"].shape == (1, 2, 4, n_kv)
    for h in range(2):
        K_new = orc.gather_concat(K[0, h], *orc.block_grid(L_src, L_ctx, 64)[:2], 4, out["sel"][0, h])
        V_new = orc.gather_concat(V[0, h], *orc.block_grid(L_src, L_ctx, 64)[:2], 4, out["sel"][0, h])
        rows = np.concatenate([np.arange(64 * i, 64 * i + 64) for i in out["flat"][0, h]])
        o, l = orc.dense_ref(Q[0, h][None, None, rows], K_new[None, None], V_new[None, None])
        assert np.abs(out["O"][0, h][rows] - o[0, 0]).max() < 1e-12
        assert np.abs(out["LSE"][0, h][rows] - l[0, 0]).max() < 1e-12


def test_isa_alpha_ns_zero_is_unchanged():
    Q, K, V = _small(22)
    a = orc.isa_ref(Q, K, V, 256, 256, 64, 0.5, 0.5)
    b = orc.isa_ref(Q, K, V, 256, 256, 64, 0.5, 0.5, alpha_ns=0.0)
    assert np.array_equal(a["O"], b["O"]) and b["ns"].shape[-1] == 0


def test_isa_mask_changes_flat_rows_only():
    Q, K, V = _small(23)
    a = orc.isa_ref(Q, K, V, 256, 256, 64, 0.5, 0.5)
    b = orc.isa_ref(Q, K, V, 256, 256, 64, 0.5, 0.5, alpha_ns=0.34)
    assert orc.ns_count(0.34, 6) == 3 and b["ns"].shape == (1, 2, 4, 3)
    for h in range(2):
        sharp_rows = np.concatenate([np.arange(64 * i, 64 * i + 64) for i in a["sharp"][0, h]])
        flat_rows = np.concatenate([np.arange(64 * i, 64 * i + 64) for i in a["flat"][0, h]])
        assert np.array_equal(a["O"][0, h][sharp_rows], b["O"][0, h][sharp_rows])
        assert np.abs(a["O"][0, h][flat_rows] - b["O"][0, h][flat_rows]).max() > 1e-6


def test_isa_ns_selection_brute_force_and_nested():
    Q, K, V = _small(24)
    starts, ends, n_src, n_ctx = orc.block_grid(256, 256, 64)
    prev = None
    for a_ns in (0.17, 0.34, 0.5, 0.84, 1.0):
        out = orc.isa_ref(Q, K, V, 256, 256, 64, 0.5, 0.5, alpha_ns=a_ns)
        for h in range(2):
            Qc = orc.pool_blocks(Q[0, h], starts, ends)
            Kc = orc.pool_blocks(K[0, h], starts, ends)
            P = orc.coarse_probs(Qc, Kc)
            kept = list(range(n_src)) + [n_src + int(j) for j in out["sel"][0, h]]
            n_ns = orc.ns_count(a_ns, len(kept))
            for f, i in enumerate(out["flat"][0, h]):
                order = sorted(range(len(kept)), key=lambda u: (-P[i, kept[u]], u))
                assert list(out["ns"][0, h, f]) == sorted(order[:n_ns])
                if prev is not None:
                    assert set(prev[h][f]) <= set(out["ns"][0, h, f].tolist())
        prev = [[out["ns"][0, h, f].tolist() for f in range(out["ns"].shape[2])] for h in range(2)]


def test_isa_with_mask_key_shift_invariance():
    Q, K, V = _small(25)
    shift = np.linspace(-1.0, 1.0, K.shape[-1])
    a = orc.isa_ref(Q, K, V, 256, 256, 64, 0.5, 0.5, alpha_ns=0.34)
    b = orc.isa_ref(Q, K + shift, V, 256, 256, 64, 0.5, 0.5, alpha_ns=0.34)
    for key in ("sel", "flat", "ns"):
        assert np.array_equal(a[key], b[key])
    assert np.abs(a["O"] - b["O"]).max() < 1e-10


def test_fixed_with_mask_matches_full_and_row_subset():
    Q, K, V = _small(26)
    out = orc.isa_ref(Q, K, V, 256, 256, 64, 0.5, 0.5, alpha_ns=0.5)
    O, L = orc.isa_ref_fixed(Q, K, V, 256, 256, 64, out["sel"], out["flat"], ns=out["ns"])
    assert np.array_equal(O, out["O"]) and np.array_equal(L, out["LSE"])
    rows = np.array([0, 63, 64, 200, 300, 511])
    Or, Lr = orc.isa_ref_fixed(Q, K, V, 256, 256, 64, out["sel"], out["flat"], rows=rows, ns=out["ns"])
    assert np.abs(Or - out["O"][:, :, rows]).max() < 1e-13
    assert np.abs(Lr - out["LSE"][:, :, rows]).max() < 1e-13
