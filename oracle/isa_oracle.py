"""fp64 CPU oracle of the ISA forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.  It shares nothing with the HIP path.

What ISA computes, in the order the pages give it ([notes] "overall
framework"; [summary] section 3), for one (batch, head) at a time:

  1. cut the [source | context] sequence into blocks of b tokens;
  2. pooling attention: block means Q^c, K^c, V^c and the coarse map
     S_coarse = softmax(Q^c K^c^T / sqrt(D));
  3. Context Pre-Selection: average the source-query x context-key sub-block
     of S_coarse over its queries, keep the TopK alpha_s * ceil(L_ctx / b)
     context blocks, gather + concat them after the source into K_new, V_new;
  4. query sharpness M_i = Var(S_coarse[i, :]); sort, and send the alpha_f
     fraction of flattest query blocks to the approximate path;
  5. sharp query blocks: exact online-softmax attention over K_new, V_new;
  6. flat query blocks: block-wise 0-th order Taylor attention, where each
     key block j of K_new is replaced by its representative K^c_j, V^c_j and
     its exponential is weighted by the block length w_j;
  7. merge: O = O / l per row, LSE = m + ln l.

Readings of open points (each used identically by the HIP path):

  R1  pooling = arithmetic mean of the tokens of a block (Q, K and V).
  R2  the source and the context segment are each cut into b-token blocks
      from their own start; the last block of a segment may be partial
      (weight w_j = its token count).  Query blocks = key blocks.
  R3  S_coarse = row softmax of Q^c K^c^T / sqrt(D) over all N_K blocks of the
      unpruned sequence, unweighted, post-softmax.
  R4  c_j = mean over source query blocks i of S_coarse[i, n_src + j].
  R5  k = ceil(alpha_s * n_ctx), clamped to [0, n_ctx]; a 1e-6 guard keeps a
      product that is an integer up to double rounding on that integer.
  R6  TopK order key (c_j descending, j ascending); the selected indices are
      stored ascending; K_new = [all source tokens ; selected context blocks
      in ascending j], V_new likewise.
  R7  M_i = (1/N_K) sum_j (S_coarse[i, j] - 1/N_K)^2 (population variance of
      the coarse row, whose mean is exactly 1/N_K).
  R8  alpha_f is the fraction of query blocks sent to the flat (Taylor)
      path: the blocks with the smallest M_i.
  R9  n_flat = floor(alpha_f * N_Q) (1e-6 guard as in R5); order key
      (M_i ascending, i ascending); the first n_flat blocks are flat.
  R10 every query block (source and context) is routed.
  R11 both paths see only K_new / V_new (pre-selection comes first).
  R12 exact path: softmax(q K_new^T / sqrt(D)) V_new, max-subtracted.
  R13 Taylor path: per query row q (rows are not pooled),
      s_j = q . K^c_j / sqrt(D) over the n_src + k blocks of K_new,
      O = sum_j w_j e^{s_j - m} V^c_j / sum_j w_j e^{s_j - m}.
  R14 by default no exact blocks inside a flat row (no-sparsity ratio
      alpha_ns = 0); R21 gives the gating for alpha_ns > 0.
  R15 each row comes from one path; LSE = m + ln l (natural log).
  R16 no mask.  R17 max subtraction applied.
  R20 (backward) the decisions are constants; see ``isa_oracle_bwd``.
  R21 block mask inside flat query blocks ([notes] key design 2: a block pair
      with mask 1 takes the exact online-softmax update, mask 0 the
      representative update; [summary] 2 "Pooling Attention": the mask comes
      from the top entries of the coarse map; alpha_ns is the no-sparsity
      ratio).  For flat query block i, rank the N_K' blocks of K_new by
      S_coarse[i, j] (the full coarse row of R3, restricted to the kept
      blocks), order key (S_coarse descending, position in K_new ascending),
      and compute the first n_ns = ceil(alpha_ns * N_K') (1e-6 guard, clamped
      to [0, N_K']) token by token; every other block of K_new enters through
      its representative with weight w_j.  Both kinds of terms share one
      softmax per row: l = sum_t e^{s_t - m} + sum_j w_j e^{s^c_j - m}.
      Sharp query blocks are unchanged.
"""

import math

import numpy as np

_GUARD = 1e-6


# --------------------------------------------------------------------------
# Step 1: block grid.  [summary] 2 "Block Sparse Attention": the sequence is
# partitioned into non-overlapping query and key/value blocks; [notes] key
# design 1 counts ceil(L_ctx / b) context blocks.  Reading R2.
# --------------------------------------------------------------------------
def block_grid(L_src, L_ctx, b):
    """Return (starts, ends, n_src, n_ctx) of the blocks, source blocks first."""
    if b <= 0:
        raise ValueError("block size must be positive")
    n_src = -(-L_src // b)
    n_ctx = -(-L_ctx // b)
    starts, ends = [], []
    for i in range(n_src):
        starts.append(i * b)
        ends.append(min((i + 1) * b, L_src))
    for j in range(n_ctx):
        starts.append(L_src + j * b)
        ends.append(min(L_src + (j + 1) * b, L_src + L_ctx))
    return np.array(starts, dtype=np.int64), np.array(ends, dtype=np.int64), n_src, n_ctx


# --------------------------------------------------------------------------
# Step 2: pooling attention.  [summary] 2 "Pooling Attention": pooled query
# and key/value representations at block level and a coarse attention map;
# [notes] key design 2 calls K^c_j, V^c_j the block representative values.
# Readings R1, R3.
# --------------------------------------------------------------------------
def pool_blocks(X, starts, ends):
    """Block means of the rows of X ([N, D]) -> [n_blocks, D] fp64."""
    X = np.asarray(X, dtype=np.float64)
    return np.stack([X[s:e].mean(axis=0) for s, e in zip(starts, ends)]) if len(starts) \
        else np.zeros((0, X.shape[1]))


def coarse_probs(Qc, Kc):
    """S_coarse = row softmax of Q^c K^c^T / sqrt(D) (max-subtracted)."""
    D = Qc.shape[1]
    S = (Qc @ Kc.T) / math.sqrt(D)
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    return E / E.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Step 3: Context Pre-Selection.  [notes] key design 1; [summary] 3
# "Pre-Selection".  Readings R4, R5, R6.
# --------------------------------------------------------------------------
def context_scores(P, n_src):
    """c_j: the source-query x context-key sub-block averaged over queries."""
    return P[:n_src, n_src:].mean(axis=0)


def select_count(alpha_s, n_ctx):
    """k = ceil(alpha_s * n_ctx) clamped to [0, n_ctx] (R5)."""
    k = math.ceil(alpha_s * n_ctx - _GUARD)
    return int(min(max(k, 0), n_ctx))


def top_k_context(c, k):
    """Indices of the k largest c_j, ties to the smaller j, returned ascending."""
    j = np.arange(len(c))
    order = np.lexsort((j, -np.asarray(c)))  # primary key: -c, then j
    return np.sort(order[:k]).astype(np.int64)


def gather_concat(X, starts, ends, n_src, sel):
    """X_new = [source tokens ; tokens of the selected context blocks]."""
    parts = [X[starts[i]:ends[i]] for i in range(n_src)]
    parts += [X[starts[n_src + j]:ends[n_src + j]] for j in sel]
    return np.concatenate(parts, axis=0) if parts else X[:0]


# --------------------------------------------------------------------------
# Step 4: query sharpness and grouping.  [notes] key design 3; [summary] 3
# "Grouped Computation".  Readings R7, R8, R9, R10.
# --------------------------------------------------------------------------
def sharpness(P):
    """M_i = population variance of the coarse row i."""
    N_K = P.shape[1]
    return ((P - 1.0 / N_K) ** 2).mean(axis=1)


def flat_count(alpha_f, n_q):
    """n_flat = floor(alpha_f * N_Q) clamped to [0, N_Q] (R9)."""
    n = math.floor(alpha_f * n_q + _GUARD)
    return int(min(max(n, 0), n_q))


def route_queries(M, n_flat):
    """(flat, sharp) query-block ids, both ascending; flat = n_flat smallest M."""
    i = np.arange(len(M))
    order = np.lexsort((i, np.asarray(M)))  # primary key: M ascending, then i
    flat = np.sort(order[:n_flat]).astype(np.int64)
    sharp = np.setdiff1d(i, flat).astype(np.int64)
    return flat, sharp


# --------------------------------------------------------------------------
# Steps 5-7: the two attention paths and the merge.  [notes] key design 2
# gives both update rules (the exact branch and the representative-value
# branch scaled by the block length) and the final O / l; [notes] overall
# framework merges the two online softmaxes.  Readings R12-R15, R17.
# --------------------------------------------------------------------------
def exact_attention(Qrows, K_new, V_new):
    """Exact softmax attention of each query row over K_new -> (O, LSE)."""
    D = Qrows.shape[1]
    S = (Qrows @ K_new.T) / math.sqrt(D)
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    l = P.sum(axis=1)
    O = (P @ V_new) / l[:, None]
    return O, m[:, 0] + np.log(l)


def taylor_attention(Qrows, Kc_new, Vc_new, w_new):
    """0-th order Taylor attention: block j enters with weight w_j via K^c_j, V^c_j."""
    D = Qrows.shape[1]
    S = (Qrows @ Kc_new.T) / math.sqrt(D)
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m) * np.asarray(w_new, dtype=np.float64)[None, :]
    l = P.sum(axis=1)
    O = (P @ Vc_new) / l[:, None]
    return O, m[:, 0] + np.log(l)


# --------------------------------------------------------------------------
# Block mask inside flat query blocks.  [notes] key design 2 (per block pair:
# exact update when the mask is 1, representative update otherwise) and
# [notes] key design 3 / [summary] 4 "Hyperparameters in ISA" (alpha_ns, the
# no-sparsity ratio).  Reading R21.
# --------------------------------------------------------------------------
def ns_count(alpha_ns, n_kv):
    """n_ns = ceil(alpha_ns * N_K') clamped to [0, N_K'] (R21)."""
    n = math.ceil(alpha_ns * n_kv - _GUARD)
    return int(min(max(n, 0), n_kv))


def top_ns_blocks(p_row, n_ns):
    """Positions (in K_new) of the n_ns largest coarse probabilities of a
    query block, ties to the smaller position, returned ascending."""
    u = np.arange(len(p_row))
    order = np.lexsort((u, -np.asarray(p_row)))  # primary key: -p, then u
    return np.sort(order[:n_ns]).astype(np.int64)


def mixed_attention(Qrows, K_new, V_new, Kc_new, Vc_new, w_new, exact_blocks):
    """Flat-row attention with a block mask (R21): the tokens of the K_new
    blocks in ``exact_blocks`` (positions) enter one by one, every other
    block through K^c_j, V^c_j with weight w_j; one softmax over both."""
    w = np.asarray(w_new, dtype=np.float64)
    ends = np.cumsum(w).astype(np.int64)
    starts = ends - w.astype(np.int64)
    exact = np.zeros(len(w), dtype=bool)
    exact[np.asarray(exact_blocks, dtype=np.int64)] = True
    tok = (np.concatenate([np.arange(starts[u], ends[u]) for u in np.nonzero(exact)[0]])
           if exact.any() else np.zeros(0, dtype=np.int64))
    rep = np.nonzero(~exact)[0]
    D = Qrows.shape[1]
    S_tok = (Qrows @ K_new[tok].T) / math.sqrt(D)
    S_rep = (Qrows @ Kc_new[rep].T) / math.sqrt(D)
    m = np.concatenate([S_tok, S_rep], axis=1).max(axis=1, keepdims=True)
    E_tok = np.exp(S_tok - m)
    E_rep = np.exp(S_rep - m) * w[rep][None, :]
    l = E_tok.sum(axis=1) + E_rep.sum(axis=1)
    O = (E_tok @ V_new[tok] + E_rep @ Vc_new[rep]) / l[:, None]
    return O, m[:, 0] + np.log(l)


def _rows_of_blocks(blocks, starts, ends):
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(starts[i], ends[i]) for i in blocks])


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _chunks(rows, size=2048):
    for s in range(0, len(rows), size):
        yield rows[s:s + size]


def _head_decisions(Qh, Kh, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns=0.0):
    starts, ends, n_src, n_ctx = block_grid(L_src, L_ctx, b)
    Qc = pool_blocks(Qh, starts, ends)
    Kc = pool_blocks(Kh, starts, ends)
    P = coarse_probs(Qc, Kc)
    c = context_scores(P, n_src)
    sel = top_k_context(c, select_count(alpha_s, n_ctx))
    M = sharpness(P)
    flat, sharp = route_queries(M, flat_count(alpha_f, len(starts)))
    kept = np.concatenate([np.arange(n_src), n_src + sel]).astype(np.int64)
    n_ns = ns_count(alpha_ns, len(kept))
    ns = np.stack([top_ns_blocks(P[i, kept], n_ns) for i in flat]) if len(flat) \
        else np.zeros((0, n_ns), dtype=np.int64)
    return dict(c=c, M=M, sel=sel, flat=flat, sharp=sharp, ns=ns.reshape(len(flat), n_ns))


def _head_paths(Qh, Kh, Vh, L_src, L_ctx, b, sel, flat, rows=None, ns=None):
    """Steps 3 (gather) and 5-7 for one head with fixed decisions.

    ``ns`` [n_flat, n_ns] (optional, R21): per flat block (in the order of
    ``flat``) the K_new positions computed exactly."""
    starts, ends, n_src, n_ctx = block_grid(L_src, L_ctx, b)
    n_q = len(starts)
    K_new = gather_concat(Kh, starts, ends, n_src, sel)
    V_new = gather_concat(Vh, starts, ends, n_src, sel)
    kept = list(range(n_src)) + [n_src + int(j) for j in sel]
    Kc_new = pool_blocks(Kh, starts[kept], ends[kept])
    Vc_new = pool_blocks(Vh, starts[kept], ends[kept])
    w_new = (ends[kept] - starts[kept]).astype(np.float64)

    is_flat = np.zeros(n_q, dtype=bool)
    is_flat[np.asarray(flat, dtype=np.int64)] = True
    block_of_row = np.repeat(np.arange(n_q), ends - starts)
    N, D = Qh.shape
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.zeros((len(rows), Vh.shape[1]))
    lse = np.zeros(len(rows))
    flat_mask = is_flat[block_of_row[rows]]
    for pos in _chunks(np.nonzero(~flat_mask)[0]):
        O[pos], lse[pos] = exact_attention(Qh[rows[pos]], K_new, V_new)
    if ns is None or np.asarray(ns).size == 0:
        for pos in _chunks(np.nonzero(flat_mask)[0]):
            O[pos], lse[pos] = taylor_attention(Qh[rows[pos]], Kc_new, Vc_new, w_new)
    else:
        flat = np.asarray(flat, dtype=np.int64)
        for f, i in enumerate(flat):
            pos = np.nonzero(block_of_row[rows] == i)[0]
            if len(pos):
                O[pos], lse[pos] = mixed_attention(Qh[rows[pos]], K_new, V_new, Kc_new, Vc_new,
                                                   w_new, ns[f])
    return O, lse


def decisions_ref(Q, K, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns=0.0):
    """Steps 1-4 for every (batch, head).

    Returns dict of arrays indexed [B, H, ...]: c (context scores), M
    (sharpness), sel (selected context blocks), flat and sharp (query blocks),
    ns (R21: per flat block the K_new positions computed exactly, [.., n_flat,
    n_ns]).  k, n_flat and n_ns depend only on the shapes, so every head has
    the same sizes.
    """
    Q, K = _f64(Q), _f64(K)
    B, H = Q.shape[:2]
    per_head = [_head_decisions(Q[bi, h], K[bi, h], L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns)
                for bi in range(B) for h in range(H)]
    out = {}
    for key in ("c", "M", "sel", "flat", "sharp", "ns"):
        arr = np.stack([d[key] for d in per_head]) if per_head else np.zeros((0, 0))
        out[key] = arr.reshape((B, H) + arr.shape[1:])
    return out


def isa_ref_fixed(Q, K, V, L_src, L_ctx, b, sel, flat, rows=None, ns=None):
    """Steps 3 (gather) and 5-7 with the decisions supplied.

    sel [B, H, k] and flat [B, H, n_flat] are the selected context blocks and
    the flat query blocks of every head; ns [B, H, n_flat, n_ns] (optional,
    R21) the exact K_new blocks of every flat block.  ``rows`` (optional)
    restricts the output to those token rows of every head; each row is
    computed exactly as in the full evaluation.  Returns (O [B,H,R,D],
    LSE [B,H,R]).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, D = Q.shape
    R = N if rows is None else len(rows)
    O = np.zeros((B, H, R, V.shape[3]))
    LSE = np.zeros((B, H, R))
    for bi in range(B):
        for h in range(H):
            O[bi, h], LSE[bi, h] = _head_paths(Q[bi, h], K[bi, h], V[bi, h], L_src, L_ctx, b,
                                               sel[bi][h], flat[bi][h], rows,
                                               None if ns is None else ns[bi][h])
    return O, LSE


def isa_ref(Q, K, V, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns=0.0):
    """The whole ISA forward: dict(O, LSE, c, M, sel, flat, sharp, ns), [B, H, ...]."""
    dec = decisions_ref(Q, K, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns)
    O, LSE = isa_ref_fixed(Q, K, V, L_src, L_ctx, b, dec["sel"], dec["flat"],
                           ns=dec["ns"] if alpha_ns > 0 else None)
    out = dict(O=O, LSE=LSE)
    out.update(dec)
    return out


def dense_ref(Q, K, V, rows=None):
    """Textbook softmax(Q K^T / sqrt(D)) V per head -> (O, LSE).

    [summary] 2 "Standard Attention".  ``rows`` restricts the query rows.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, D = Q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((B, H, len(rows), V.shape[3]))
    LSE = np.zeros((B, H, len(rows)))
    for bi in range(B):
        for h in range(H):
            for chunk in _chunks(np.arange(len(rows))):
                O[bi, h, chunk], LSE[bi, h, chunk] = exact_attention(
                    Q[bi, h, rows[chunk]], K[bi, h], V[bi, h])
    return O, LSE
