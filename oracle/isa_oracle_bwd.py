"""fp64 CPU oracle of the ISA backward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.

The pages train ISA end to end with hand-written forward and backward kernels
([notes] "overall framework" and "highlights": trainable sparse attention);
they print no gradient formulas.  Reading R20: the selection (TopK) and the
routing (sort by sharpness) are constants of the forward, so no gradient
passes through S_coarse.  The gradient flows through

  * the exact path over K_new, V_new (textbook attention backward), and
  * the Taylor path: pi_rj = w_j e^{s_rj} / l_r with s_rj = q_r . K^c_j / sqrt(D),
    O_r = sum_j pi_rj V^c_j, plus the mean pooling K^c_j = (1/w_j) sum_{t in B_j} K_t
    (and V^c_j likewise), so dK_t += dK^c_j / w_j for every token t of block j.

With the block mask inside flat rows (reading R21: the tokens of the blocks
ns[f] of flat block f enter one by one, every other kept block through its
representative with weight w_j, one softmax over both), a flat row's terms are
the union of the two kinds above, so its gradient splits the same way: token
terms feed dK_new, dV_new at those tokens, representative terms feed dK^c,
dV^c.

Rows of context blocks that were not selected receive zero gradient in K and V.
"""

import math

import numpy as np

from .isa_oracle import block_grid, gather_concat, pool_blocks


def _softmax_bwd(P, dO, O, Vmat):
    """dS for rows with probabilities P, output O and upstream dO."""
    dP = dO @ Vmat.T
    delta = (dO * O).sum(axis=1, keepdims=True)
    return P * (dP - delta)


def _mixed_rows_bwd(q, dO, K_new, V_new, Kc_new, Vc_new, w_new, exact_blocks, scale):
    """Backward of one flat block's rows under the block mask: the columns are
    the tokens of the K_new blocks in ``exact_blocks`` (weight 1) followed by
    the representatives of the other kept blocks (weight w_j), one softmax.
    Returns (dq, token positions, dK_tok, dV_tok, rep positions, dKc_rep, dVc_rep)."""
    ends = np.cumsum(w_new).astype(np.int64)
    starts = ends - w_new.astype(np.int64)
    exact = np.zeros(len(w_new), dtype=bool)
    exact[np.asarray(exact_blocks, dtype=np.int64)] = True
    tok = (np.concatenate([np.arange(starts[u], ends[u]) for u in np.nonzero(exact)[0]])
           if exact.any() else np.zeros(0, dtype=np.int64))
    rep = np.nonzero(~exact)[0]
    Kcols = np.concatenate([K_new[tok], Kc_new[rep]])
    Vcols = np.concatenate([V_new[tok], Vc_new[rep]])
    logw = np.concatenate([np.zeros(len(tok)), np.log(w_new[rep])])
    S = (q @ Kcols.T) * scale + logw[None, :]
    S -= S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=1, keepdims=True)
    O = P @ Vcols
    dS = _softmax_bwd(P, dO, O, Vcols)
    dq = (dS @ Kcols) * scale
    dKcols = (dS.T @ q) * scale
    dVcols = P.T @ dO
    n = len(tok)
    return dq, tok, dKcols[:n], dVcols[:n], rep, dKcols[n:], dVcols[n:]


def _head_bwd(Qh, Kh, Vh, dOh, L_src, L_ctx, b, sel, flat, ns=None):
    starts, ends, n_src, n_ctx = block_grid(L_src, L_ctx, b)
    n_q = len(starts)
    N, D = Qh.shape
    scale = 1.0 / math.sqrt(D)
    kept = list(range(n_src)) + [n_src + int(j) for j in sel]
    # token rows of K_new, in K_new order, as indices into the original rows
    new_rows = np.concatenate([np.arange(starts[i], ends[i]) for i in kept]) if kept \
        else np.zeros(0, dtype=np.int64)
    K_new = gather_concat(Kh, starts, ends, n_src, sel)
    V_new = gather_concat(Vh, starts, ends, n_src, sel)
    Kc_new = pool_blocks(Kh, starts[kept], ends[kept])
    Vc_new = pool_blocks(Vh, starts[kept], ends[kept])
    w_new = (ends[kept] - starts[kept]).astype(np.float64)

    is_flat = np.zeros(n_q, dtype=bool)
    is_flat[np.asarray(flat, dtype=np.int64)] = True
    block_of_row = np.repeat(np.arange(n_q), ends - starts)
    flat_rows = np.nonzero(is_flat[block_of_row])[0]
    sharp_rows = np.nonzero(~is_flat[block_of_row])[0]

    dQ = np.zeros_like(Qh)
    dK_new = np.zeros_like(K_new)
    dV_new = np.zeros_like(V_new)
    dKc = np.zeros_like(Kc_new)
    dVc = np.zeros_like(Vc_new)

    # exact path (sharp rows)
    if len(sharp_rows):
        q = Qh[sharp_rows]
        S = (q @ K_new.T) * scale
        S -= S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=1, keepdims=True)
        O = P @ V_new
        dO = dOh[sharp_rows]
        dV_new += P.T @ dO
        dS = _softmax_bwd(P, dO, O, V_new)
        dQ[sharp_rows] = (dS @ K_new) * scale
        dK_new += (dS.T @ q) * scale

    # flat rows under the block mask (R21): one mixed softmax per flat block
    if len(flat_rows) and ns is not None and np.asarray(ns).size > 0:
        for f, i in enumerate(np.asarray(flat, dtype=np.int64)):
            rows = np.arange(starts[i], ends[i])
            dq, tok, dkt, dvt, rep, dkr, dvr = _mixed_rows_bwd(
                Qh[rows], dOh[rows], K_new, V_new, Kc_new, Vc_new, w_new, ns[f], scale)
            dQ[rows] = dq
            dK_new[tok] += dkt
            dV_new[tok] += dvt
            dKc[rep] += dkr
            dVc[rep] += dvr
    # Taylor path (flat rows)
    elif len(flat_rows):
        q = Qh[flat_rows]
        S = (q @ Kc_new.T) * scale
        S -= S.max(axis=1, keepdims=True)
        Pi = np.exp(S) * w_new[None, :]
        Pi /= Pi.sum(axis=1, keepdims=True)
        O = Pi @ Vc_new
        dO = dOh[flat_rows]
        dVc += Pi.T @ dO
        dS = _softmax_bwd(Pi, dO, O, Vc_new)
        dQ[flat_rows] = (dS @ Kc_new) * scale
        dKc += (dS.T @ q) * scale

    # scatter back to the original rows
    dK = np.zeros_like(Kh)
    dV = np.zeros_like(Vh)
    dK[new_rows] += dK_new
    dV[new_rows] += dV_new
    for t, blk in enumerate(kept):
        dK[starts[blk]:ends[blk]] += dKc[t] / w_new[t]
        dV[starts[blk]:ends[blk]] += dVc[t] / w_new[t]
    return dQ, dK, dV


def isa_ref_bwd(Q, K, V, dO, L_src, L_ctx, b, sel, flat, ns=None):
    """Gradients (dQ, dK, dV) of sum(dO * O) with the decisions sel, flat fixed.

    sel [B, H, k] and flat [B, H, n_flat] as returned by ``decisions_ref``;
    ns [B, H, n_flat, n_ns] (optional): the block mask of the flat blocks.
    """
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    B, H = Q.shape[:2]
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for bi in range(B):
        for h in range(H):
            dQ[bi, h], dK[bi, h], dV[bi, h] = _head_bwd(
                Q[bi, h], K[bi, h], V[bi, h], dO[bi, h], L_src, L_ctx, b,
                sel[bi][h], flat[bi][h], None if ns is None else ns[bi][h])
    return dQ, dK, dV


def dense_ref_bwd(Q, K, V, dO):
    """Textbook attention backward per head ([summary] 2 "Standard Attention")."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    B, H, N, D = Q.shape
    scale = 1.0 / math.sqrt(D)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for bi in range(B):
        for h in range(H):
            q, k, v, do = Q[bi, h], K[bi, h], V[bi, h], dO[bi, h]
            S = (q @ k.T) * scale
            S -= S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            O = P @ v
            dV[bi, h] = P.T @ do
            dS = _softmax_bwd(P, do, O, v)
            dQ[bi, h] = (dS @ k) * scale
            dK[bi, h] = (dS.T @ q) * scale
    return dQ, dK, dV
