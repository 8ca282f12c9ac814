"""Pins of the fp64 oracle to things other than itself (CPU only).

Each pin is a closed form, an invariant of the definitions, brute force on a
tiny input, a special case that reduces to a library routine (torch's
scaled_dot_product_attention / avg_pool1d / var in fp64), or a hand-worked
example (tests/golden/).  A plausible mistake in the oracle (a dropped 1/sqrt(D),
a wrong TopK or routing direction, a transposed operand, a missing block
weight) fails at least one of them; see the comment on each test.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as orc
from synth import generate, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(B, H, N, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, D)) * scale for _ in range(3)]


def _sdpa(q, k, v, mask=None):
    """Library attention in fp64 (torch math path), arrays [.., N, D]."""
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    return F.scaled_dot_product_attention(*t, attn_mask=m).numpy()


def _lse_lib(q, k):
    t = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)
    return torch.logsumexp(t / math.sqrt(q.shape[-1]), dim=-1).numpy()


# ---------------------------------------------------------------- dense ---
def test_dense_ref_matches_library_sdpa():
    # pins the 1/sqrt(D) scale, the softmax axis and the P V product order
    Q, K, V = _rand(2, 2, 96, 32, 1)
    O, LSE = orc.dense_ref(Q, K, V)
    np.testing.assert_allclose(O, _sdpa(Q, K, V), atol=1e-12, rtol=0)
    np.testing.assert_allclose(LSE, _lse_lib(Q, K), atol=1e-12, rtol=0)


def test_dense_ref_rows_subset():
    Q, K, V = _rand(1, 1, 64, 16, 2)
    rows = np.array([0, 5, 63, 17])
    O, LSE = orc.dense_ref(Q, K, V, rows=rows)
    O_all, LSE_all = orc.dense_ref(Q, K, V)
    np.testing.assert_array_equal(O[0, 0], O_all[0, 0, rows])
    np.testing.assert_array_equal(LSE[0, 0], LSE_all[0, 0, rows])


# ---------------------------------------------------------- whole ISA -----
@pytest.mark.parametrize("L_src,L_ctx,b", [(128, 128, 32), (96, 160, 32), (100, 70, 16)])
def test_isa_all_kept_all_exact_is_dense(L_src, L_ctx, b):
    # alpha_s = 1, alpha_f = 0: every context block kept, every query exact
    Q, K, V = _rand(1, 2, L_src + L_ctx, 16, 3)
    r = orc.isa_ref(Q, K, V, L_src, L_ctx, b, 1.0, 0.0)
    np.testing.assert_allclose(r["O"], _sdpa(Q, K, V), atol=1e-12, rtol=0)
    np.testing.assert_allclose(r["LSE"], _lse_lib(Q, K), atol=1e-12, rtol=0)


def test_isa_all_exact_is_masked_dense():
    # alpha_f = 0: ISA = dense attention in which the unselected context
    # blocks are masked out (a mask route, independent of the gather).
    L_src, L_ctx, b, D = 128, 192, 32, 16
    Q, K, V = _rand(1, 2, L_src + L_ctx, D, 4)
    r = orc.isa_ref(Q, K, V, L_src, L_ctx, b, 0.5, 0.0)
    for h in range(2):
        mask = np.zeros((L_src + L_ctx,))
        keep = np.zeros(L_ctx // b, dtype=bool)
        keep[r["sel"][0, h]] = True
        for j in range(L_ctx // b):
            if not keep[j]:
                mask[L_src + j * b:L_src + (j + 1) * b] = -np.inf
        ref = _sdpa(Q[0, h], K[0, h], V[0, h], np.broadcast_to(mask, (L_src + L_ctx,) * 2))
        np.testing.assert_allclose(r["O"][0, h], ref, atol=1e-12, rtol=0)


def test_isa_key_shift_invariance():
    # K -> K + 1 c^T shifts every softmax row (fine and coarse) uniformly
    L_src, L_ctx, b = 128, 128, 32
    Q, K, V = _rand(1, 2, 256, 16, 5)
    c = np.random.default_rng(9).standard_normal(16)
    r0 = orc.isa_ref(Q, K, V, L_src, L_ctx, b, 0.5, 0.5)
    r1 = orc.isa_ref(Q, K + c, V, L_src, L_ctx, b, 0.5, 0.5)
    for key in ("sel", "flat", "sharp"):
        np.testing.assert_array_equal(r0[key], r1[key])
    np.testing.assert_allclose(r0["O"], r1["O"], atol=1e-12, rtol=0)


def test_isa_value_affine_equivariance():
    # O(a V + 1 c^T) = a O(V) + 1 c^T for both paths (weights sum to one)
    Q, K, V = _rand(1, 1, 256, 16, 6)
    c = np.random.default_rng(10).standard_normal(16)
    r0 = orc.isa_ref(Q, K, V, 128, 128, 32, 0.5, 0.5)
    r1 = orc.isa_ref(Q, K, -2.5 * V + c, 128, 128, 32, 0.5, 0.5)
    np.testing.assert_allclose(r1["O"], -2.5 * r0["O"] + c, atol=1e-12, rtol=0)


def test_isa_context_block_permutation():
    # permuting whole context key/value blocks permutes the selection and
    # leaves the sharpness, the routing and the output unchanged
    L_src, L_ctx, b, D = 128, 256, 32, 16
    Q, K, V = _rand(1, 1, L_src + L_ctx, D, 7)
    n_ctx = L_ctx // b
    perm = np.random.default_rng(11).permutation(n_ctx)
    idx = np.concatenate([np.arange(L_src)] + [L_src + perm[j] * b + np.arange(b) for j in range(n_ctx)])
    K2, V2 = K[:, :, idx], V[:, :, idx]
    r0 = orc.isa_ref(Q, K, V, L_src, L_ctx, b, 0.5, 0.5)
    r1 = orc.isa_ref(Q, K2, V2, L_src, L_ctx, b, 0.5, 0.5)
    # new context block j holds old block perm[j]
    np.testing.assert_array_equal(np.sort(perm[r1["sel"][0, 0]]), r0["sel"][0, 0])
    np.testing.assert_allclose(r1["M"], r0["M"], rtol=1e-12, atol=0)
    np.testing.assert_array_equal(r1["flat"], r0["flat"])
    np.testing.assert_allclose(r1["O"], r0["O"], atol=1e-12, rtol=0)


# ------------------------------------------------------------- pooling ---
def test_pool_brute_force_and_library():
    rng = np.random.default_rng(12)
    X = rng.standard_normal((100, 8))
    starts, ends, n_src, n_ctx = orc.block_grid(60, 40, 16)
    assert (n_src, n_ctx) == (4, 3)
    assert list(starts) == [0, 16, 32, 48, 60, 76, 92] and list(ends) == [16, 32, 48, 60, 76, 92, 100]
    P = orc.pool_blocks(X, starts, ends)
    for i, (s, e) in enumerate(zip(starts, ends)):
        manual = [sum(X[t, d] for t in range(s, e)) / (e - s) for d in range(8)]
        np.testing.assert_allclose(P[i], manual, rtol=1e-14, atol=1e-15)
    # full blocks: torch's average pooling
    Xf = rng.standard_normal((128, 8))
    s, e, _, _ = orc.block_grid(64, 64, 16)
    lib = F.avg_pool1d(torch.from_numpy(Xf.T[None]), 16).numpy()[0].T
    np.testing.assert_allclose(orc.pool_blocks(Xf, s, e), lib, rtol=1e-14, atol=1e-15)


def test_pool_block_one_is_identity():
    X = np.random.default_rng(13).standard_normal((20, 4))
    s, e, _, _ = orc.block_grid(12, 8, 1)
    np.testing.assert_array_equal(orc.pool_blocks(X, s, e), X)


# -------------------------------------------------------------- coarse ---
def test_coarse_rows_sum_to_one_and_b1_is_attention_matrix():
    Q, K, _ = _rand(1, 1, 48, 8, 14)
    s, e, _, _ = orc.block_grid(24, 24, 1)
    P = orc.coarse_probs(orc.pool_blocks(Q[0, 0], s, e), orc.pool_blocks(K[0, 0], s, e))
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    # with V = identity, library attention returns the probability matrix itself
    lib = _sdpa(Q[0, 0], K[0, 0], np.eye(48))
    np.testing.assert_allclose(P, lib, atol=1e-14, rtol=0)


def test_coarse_closed_form_two_blocks():
    # q = [2,0,0,0], keys [1,0,0,0] and 0 (D = 4): logits [1, 0] -> [e, 1]/(e+1)
    P = orc.coarse_probs(np.array([[2.0, 0, 0, 0]]), np.array([[1.0, 0, 0, 0], [0, 0, 0, 0]]))
    e = math.e
    np.testing.assert_allclose(P[0], [e / (e + 1), 1 / (e + 1)], rtol=1e-15)


# ---------------------------------------------------------------- TopK ---
def test_topk_against_sorted_builtin_every_head():
    Q, K, _ = _rand(2, 3, 320, 16, 15)
    d = orc.decisions_ref(Q, K, 128, 192, 32, 0.5, 0.5)
    k = orc.select_count(0.5, 6)
    for bi in range(2):
        for h in range(3):
            c = d["c"][bi, h]
            ref = sorted(range(len(c)), key=lambda j: (-c[j], j))[:k]
            assert list(d["sel"][bi, h]) == sorted(ref)


def test_topk_brute_force_subsets_with_ties():
    c = np.array([0.3, 0.1, 0.3, 0.2, 0.1, 0.3])
    for k in range(len(c) + 1):
        best = None
        for sub in itertools.combinations(range(len(c)), k):
            # the selected set must dominate: every kept (c, -j) beats every dropped one
            rest = [j for j in range(len(c)) if j not in sub]
            if all((c[a], -a) > (c[r], -r) for a in sub for r in rest):
                assert best is None
                best = list(sub)
        assert list(orc.top_k_context(c, k)) == best


def test_topk_extremes_and_counts():
    assert orc.select_count(1.0, 7) == 7 and orc.select_count(0.0, 7) == 0
    assert orc.select_count(0.25, 256) == 64 and orc.select_count(0.125, 400) == 50
    assert orc.select_count(0.1, 30) == 3  # integer product survives double rounding
    assert orc.select_count(0.26, 10) == 3
    assert orc.flat_count(0.5, 512) == 256 and orc.flat_count(0.75, 800) == 600
    assert orc.flat_count(0.3, 10) == 3 and orc.flat_count(0.29, 10) == 2
    Q, K, _ = _rand(1, 1, 256, 8, 16)
    assert len(orc.decisions_ref(Q, K, 128, 128, 32, 1.0, 0.5)["sel"][0, 0]) == 4
    assert len(orc.decisions_ref(Q, K, 128, 128, 32, 0.0, 0.5)["sel"][0, 0]) == 0


def test_context_scores_mass_identity():
    # each coarse row sums to one: source mass + n_ctx * mean(context part)
    Q, K, _ = _rand(1, 1, 256, 8, 17)
    s, e, n_src, _ = orc.block_grid(96, 160, 32)
    P = orc.coarse_probs(orc.pool_blocks(Q[0, 0], s, e), orc.pool_blocks(K[0, 0], s, e))
    c = orc.context_scores(P, n_src)
    np.testing.assert_allclose(c.sum() + P[:n_src, :n_src].sum(axis=1).mean(), 1.0, atol=1e-14)
    assert len(c) == 5


# ----------------------------------------------------------- sharpness ---
def test_sharpness_closed_forms():
    Q, K, _ = _rand(1, 1, 256, 8, 18)
    s, e, _, _ = orc.block_grid(128, 128, 32)
    P = orc.coarse_probs(orc.pool_blocks(Q[0, 0], s, e), orc.pool_blocks(K[0, 0], s, e))
    M = orc.sharpness(P)
    N_K = P.shape[1]
    np.testing.assert_allclose(M, (P ** 2).sum(axis=1) / N_K - 1.0 / N_K ** 2, rtol=1e-9, atol=0)
    np.testing.assert_allclose(M, torch.var(torch.from_numpy(P), dim=1, unbiased=False).numpy(),
                               rtol=1e-12, atol=0)


def test_sharpness_uniform_and_one_hot_limits():
    Kc = np.random.default_rng(19).standard_normal((8, 4))
    # a zero pooled query gives a uniform row: M = 0
    assert orc.sharpness(orc.coarse_probs(np.zeros((1, 4)), Kc))[0] == 0.0
    # a huge query aligned with one key gives a one-hot row: M = (N-1)/N^2
    q = 1e4 * Kc[3:4] / np.linalg.norm(Kc[3])
    M = orc.sharpness(orc.coarse_probs(q, Kc))[0]
    np.testing.assert_allclose(M, 7 / 64, rtol=1e-12)


# ------------------------------------------------------------- routing ---
def test_routing_brute_force_and_direction():
    M = np.array([0.5, 0.1, 0.1, 0.9, 0.0, 0.3])
    flat, sharp = orc.route_queries(M, 3)
    assert list(flat) == [1, 2, 4]  # the three smallest (flattest), ties by index
    assert list(sharp) == [0, 3, 5]
    rng = np.random.default_rng(20)
    for _ in range(20):
        M = rng.integers(0, 4, size=12).astype(float)
        n = int(rng.integers(0, 13))
        ref = sorted(range(12), key=lambda i: (M[i], i))[:n]
        assert list(orc.route_queries(M, n)[0]) == sorted(ref)
    Q, K, _ = _rand(1, 1, 256, 8, 21)
    assert len(orc.decisions_ref(Q, K, 128, 128, 32, 0.5, 0.0)["flat"][0, 0]) == 0
    assert len(orc.decisions_ref(Q, K, 128, 128, 32, 0.5, 1.0)["flat"][0, 0]) == 8


def test_routing_sends_sharp_blocks_to_exact():
    # a zero query block is perfectly flat (M = 0); a block of huge queries
    # aligned with one key block is the sharpest: they must go flat / exact.
    L_src, L_ctx, b, D = 128, 128, 32, 8
    Q, K, V = _rand(1, 1, 256, D, 22, scale=0.1)
    Q[0, 0, 32:64] = 0.0
    K[0, 0, 192:224] += 3.0
    Q[0, 0, 96:128] = 50.0 * K[0, 0, 192:224].mean(axis=0)
    d = orc.decisions_ref(Q, K, L_src, L_ctx, b, 0.5, 0.25)
    assert len(d["flat"][0, 0]) == 2 and 1 in d["flat"][0, 0]
    assert 3 in d["sharp"][0, 0]
    assert d["M"][0, 0, 1] == d["M"][0, 0].min() and d["M"][0, 0, 3] == d["M"][0, 0].max()


# -------------------------------------------------------------- Taylor ---
def test_taylor_block_one_is_exact():
    # b = 1: every representative is the token itself, every weight is one
    Q, K, V = _rand(1, 2, 64, 8, 23)
    r_t = orc.isa_ref(Q, K, V, 32, 32, 1, 1.0, 1.0)
    np.testing.assert_allclose(r_t["O"], _sdpa(Q, K, V), atol=1e-12, rtol=0)
    np.testing.assert_allclose(r_t["LSE"], _lse_lib(Q, K), atol=1e-12, rtol=0)


def test_taylor_block_constant_keys_values_is_exact():
    # constant K, V inside every block: w_j e^{s_j} = sum over the block's tokens
    L_src, L_ctx, b, D = 96, 96, 32, 8
    rng = np.random.default_rng(24)
    Q = rng.standard_normal((1, 1, 192, D))
    K = np.repeat(rng.standard_normal((1, 1, 6, D)), b, axis=2)
    V = np.repeat(rng.standard_normal((1, 1, 6, D)), b, axis=2)
    r = orc.isa_ref(Q, K, V, L_src, L_ctx, b, 1.0, 1.0)
    np.testing.assert_allclose(r["O"], _sdpa(Q, K, V), atol=1e-12, rtol=0)
    np.testing.assert_allclose(r["LSE"], _lse_lib(Q, K), atol=1e-12, rtol=0)


def test_taylor_full_blocks_is_attention_over_pooled():
    # all blocks full: the weights cancel and the flat path is library
    # attention against average-pooled keys and values
    L_src, L_ctx, b, D = 128, 128, 32, 8
    Q, K, V = _rand(1, 1, 256, D, 25)
    r = orc.isa_ref(Q, K, V, L_src, L_ctx, b, 1.0, 1.0)
    pool = lambda X: F.avg_pool1d(torch.from_numpy(X[0, 0].T[None].copy()), b).numpy()[0].T
    ref = _sdpa(Q[0, 0], pool(K), pool(V))
    np.testing.assert_allclose(r["O"][0, 0], ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(r["LSE"][0, 0], _lse_lib(Q[0, 0], pool(K)) + math.log(b), atol=1e-12)


def test_taylor_partial_blocks_weighting():
    # a partial last block enters with weight = its token count: library
    # attention with the additive bias ln(w_j) on the pooled logits
    L_src, L_ctx, b, D = 80, 40, 32, 8
    Q, K, V = _rand(1, 1, 120, D, 26)
    r = orc.isa_ref(Q, K, V, L_src, L_ctx, b, 1.0, 1.0)
    s, e, _, _ = orc.block_grid(L_src, L_ctx, b)
    w = (e - s).astype(float)
    assert list(w) == [32, 32, 16, 32, 8]
    Kc = np.stack([K[0, 0, a:z].mean(0) for a, z in zip(s, e)])
    Vc = np.stack([V[0, 0, a:z].mean(0) for a, z in zip(s, e)])
    bias = np.broadcast_to(np.log(w), (120, 5))
    np.testing.assert_allclose(r["O"][0, 0], _sdpa(Q[0, 0], Kc, Vc, bias), atol=1e-12, rtol=0)


# --------------------------------------------------------- hand example ---
def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example_n8.json")))
    Q, K, V = (np.array(g[x], dtype=float)[None, None] for x in ("Q", "K", "V"))
    r = orc.isa_ref(Q, K, V, g["L_src"], g["L_ctx"], g["block"], g["alpha_s"], g["alpha_f"])
    assert list(r["sel"][0, 0]) == g["expected_sel"]
    assert list(r["flat"][0, 0]) == g["expected_flat"]
    assert list(r["sharp"][0, 0]) == g["expected_sharp"]
    e = math.e
    np.testing.assert_allclose(r["c"][0, 0], [(e / (2 * e + 2) + 0.25) / 2, (1 / (2 * e + 2) + 0.25) / 2],
                               rtol=1e-14)
    np.testing.assert_allclose(r["M"][0, 0], [((e - 1) / (2 * e + 2)) ** 2 / 4, 0.0,
                                              3 * (e * e - 1) ** 2 / (16 * (e * e + 3) ** 2), 0.0],
                               rtol=1e-12, atol=1e-18)
    Vt = V[0, 0]
    O = r["O"][0, 0]
    for t in (2, 3, 6, 7):
        np.testing.assert_allclose(O[t], [2.5, 0, 0, 1], atol=1e-14)
        np.testing.assert_allclose(r["LSE"][0, 0, t], math.log(6), atol=1e-14)
    w01 = np.array([e, e, 1, 1, e * e, 1])
    for t in (0, 1):
        np.testing.assert_allclose(O[t], w01 @ Vt[:6] / w01.sum(), atol=1e-14)
        np.testing.assert_allclose(r["LSE"][0, 0, t], math.log(2 * e + 3 + e * e), atol=1e-14)
    w45 = np.array([1, 1, e * e, e * e, 1, 1])
    for t in (4, 5):
        np.testing.assert_allclose(O[t], w45 @ Vt[:6] / w45.sum(), atol=1e-14)
        np.testing.assert_allclose(r["LSE"][0, 0, t], math.log(2 * e * e + 4), atol=1e-14)


# ----------------------------------------------------------- fixed path ---
def test_fixed_rows_subset_matches_full():
    Q, K, V = _rand(1, 2, 256, 16, 27)
    r = orc.isa_ref(Q, K, V, 128, 128, 32, 0.5, 0.5)
    rows = np.array([3, 40, 127, 128, 255, 200])
    O, LSE = orc.isa_ref_fixed(Q, K, V, 128, 128, 32, r["sel"], r["flat"], rows=rows)
    np.testing.assert_array_equal(O, r["O"][:, :, rows])
    np.testing.assert_array_equal(LSE, r["LSE"][:, :, rows])


# ---------------------------------------------------------- generator ----
def test_generator_deterministic_and_head_subset():
    a = generate(1, 3, 128, 128, 16, 64, seed=5, variant="icl")
    b = generate(1, 3, 128, 128, 16, 64, seed=5, variant="icl")
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    sub = generate(1, 3, 128, 128, 16, 64, seed=5, variant="icl", heads=[1, 2])
    np.testing.assert_array_equal(sub["k"][0], a["k"][0, 1:3])
    f = to_f64(a["q"], "bf16")
    assert f.dtype == np.float64 and np.isfinite(f).all()
