"""Pins of the fp64 backward oracle: central finite differences of the
decision-frozen forward, and torch autograd of library attention."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as orc


def _loss(Q, K, V, dO, L_src, L_ctx, b, sel, flat, ns=None):
    O, _ = orc.isa_ref_fixed(Q, K, V, L_src, L_ctx, b, sel, flat, ns=ns)
    return float((O * dO).sum())


def _check_finite_differences(Q, K, V, dO, L_src, L_ctx, b, sel, flat, ns=None):
    dQ, dK, dV = orc.isa_ref_bwd(Q, K, V, dO, L_src, L_ctx, b, sel, flat, ns)
    eps = 1e-6
    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + eps
            lp = _loss(Q, K, V, dO, L_src, L_ctx, b, sel, flat, ns)
            X[idx] = old - eps
            lm = _loss(Q, K, V, dO, L_src, L_ctx, b, sel, flat, ns)
            X[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        scale = np.abs(num).max()
        np.testing.assert_allclose(G, num, atol=1e-6 * scale, rtol=0)
    return dQ, dK, dV


@pytest.mark.parametrize("L_src,L_ctx,b,alpha_s,alpha_f", [
    (8, 8, 4, 0.5, 0.5),      # full blocks, both paths
    (10, 6, 4, 0.5, 0.5),     # partial blocks: weights 4,4,2 | 4,2
    (8, 12, 4, 0.34, 0.75),   # mostly Taylor
])
def test_isa_bwd_finite_differences(L_src, L_ctx, b, alpha_s, alpha_f):
    rng = np.random.default_rng(31)
    N, D = L_src + L_ctx, 4
    Q, K, V, dO = (rng.standard_normal((1, 1, N, D)) for _ in range(4))
    d = orc.decisions_ref(Q, K, L_src, L_ctx, b, alpha_s, alpha_f)
    assert len(d["flat"][0, 0]) > 0 and len(d["sharp"][0, 0]) > 0
    sel, flat = d["sel"], d["flat"]
    dQ, dK, dV = _check_finite_differences(Q, K, V, dO, L_src, L_ctx, b, sel, flat)
    # unselected context rows get no gradient in K and V
    s, e, n_src, n_ctx = orc.block_grid(L_src, L_ctx, b)
    for j in range(n_ctx):
        if j not in sel[0, 0]:
            assert not dK[0, 0, s[n_src + j]:e[n_src + j]].any()
            assert not dV[0, 0, s[n_src + j]:e[n_src + j]].any()


def test_dense_bwd_matches_library_autograd():
    rng = np.random.default_rng(32)
    Q, K, V, dO = (rng.standard_normal((1, 2, 40, 8)) for _ in range(4))
    t = [torch.from_numpy(x.copy()).requires_grad_(True) for x in (Q, K, V)]
    out = F.scaled_dot_product_attention(*t)
    out.backward(torch.from_numpy(dO))
    ref = orc.dense_ref_bwd(Q, K, V, dO)
    for g, x in zip(ref, t):
        np.testing.assert_allclose(g, x.grad.numpy(), atol=1e-12, rtol=0)


def test_isa_bwd_all_kept_all_exact_is_dense_bwd():
    rng = np.random.default_rng(33)
    Q, K, V, dO = (rng.standard_normal((1, 2, 64, 8)) for _ in range(4))
    d = orc.decisions_ref(Q, K, 32, 32, 16, 1.0, 0.0)
    got = orc.isa_ref_bwd(Q, K, V, dO, 32, 32, 16, d["sel"], d["flat"])
    for g, r in zip(got, orc.dense_ref_bwd(Q, K, V, dO)):
        np.testing.assert_allclose(g, r, atol=1e-12, rtol=0)


@pytest.mark.parametrize("L_src,L_ctx,b,alpha_s,alpha_f,alpha_ns", [
    (8, 16, 4, 0.5, 0.5, 0.25),     # full blocks: 2 of 4 context blocks kept, 1 of 4 exact
    (10, 10, 4, 0.67, 0.67, 0.4),   # partial blocks (weights 4,4,2 | 4,4,2), 2 of 5 exact
])
def test_isa_bwd_block_mask_finite_differences(L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns):
    """The block mask (R21): token terms of the masked-in blocks and the
    representatives of the rest in one softmax per flat row."""
    rng = np.random.default_rng(34)
    N, D = L_src + L_ctx, 4
    Q, K, V, dO = (rng.standard_normal((1, 1, N, D)) for _ in range(4))
    d = orc.decisions_ref(Q, K, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns)
    flat, ns = d["flat"], d["ns"]
    n_kv = orc.block_grid(L_src, L_ctx, b)[2] + d["sel"].shape[-1]  # N_K' = n_src + k
    assert len(flat[0, 0]) >= 2 and len(d["sharp"][0, 0]) > 0
    assert 0 < ns.shape[-1] < n_kv
    dQ, dK, dV = _check_finite_differences(Q, K, V, dO, L_src, L_ctx, b, d["sel"], flat, ns)
    # the mask changes the gradient (it is not the Taylor path's)
    tq, _, _ = orc.isa_ref_bwd(Q, K, V, dO, L_src, L_ctx, b, d["sel"], flat)
    assert np.abs(tq - dQ).max() > 1e-3 * np.abs(dQ).max()


def test_isa_bwd_mask_over_every_kept_block_is_exact():
    """n_ns = N_K': every kept block enters token by token, so a flat row's
    gradient is that of a sharp row."""
    rng = np.random.default_rng(35)
    L_src, L_ctx, b = 32, 48, 8
    Q, K, V, dO = (rng.standard_normal((1, 2, L_src + L_ctx, 8)) for _ in range(4))
    d = orc.decisions_ref(Q, K, L_src, L_ctx, b, 0.5, 0.5, 1.0)
    n_kv = L_src // b + d["sel"].shape[-1]
    assert d["ns"].shape[-1] == n_kv
    got = orc.isa_ref_bwd(Q, K, V, dO, L_src, L_ctx, b, d["sel"], d["flat"], d["ns"])
    no_flat = np.zeros((1, 2, 0), dtype=np.int64)
    ref = orc.isa_ref_bwd(Q, K, V, dO, L_src, L_ctx, b, d["sel"], no_flat)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, atol=1e-12, rtol=0)
