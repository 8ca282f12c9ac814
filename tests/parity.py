"""Parity helpers: compare the HIP path with the fp64 oracle (test infrastructure).

Decisions (TopK selection, routing) must be bit-identical, except for entries
whose oracle key lies within a RELATIVE 1e-5 band of the cut: |x - x_cut| <=
1e-5 |x_cut|, with x_cut the midpoint of the oracle's two values either side of
the cut (an absolute 1e-5 band would be vacuous: c_j is about 1/N_K and M_i
about 1e-10 to 1e-7).  Outputs are compared with the oracle run on the GPU's own
decisions, so an exempted near-tie cannot turn into an output mismatch.
"""

import numpy as np
import torch

import oracle as orc
from synth import to_f64

BAND = 1e-5
# bf16 inputs, fp32 accumulation: the pages' tolerance for this path.
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
# fp32 end to end (a reading: no bar is printed for fp32; fp32 rounding of
# 1/sqrt(D)-scaled logits over a few hundred keys stays far below these).
FP32_MAX_ABS, FP32_MEAN_ABS = 1e-4, 1e-5


def to_gpu(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def from_gpu(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def out_f64(t):
    """GPU output tensor -> float64 numpy."""
    if t.dtype == torch.bfloat16:
        return to_f64(from_gpu(t), "bf16")
    return t.double().cpu().numpy()


def _band_exempt(keys, order, count):
    """Boolean mask of entries inside the relative band around the cut."""
    n = len(keys)
    if count <= 0 or count >= n:
        return np.zeros(n, dtype=bool)
    cut = 0.5 * (keys[order[count - 1]] + keys[order[count]])
    return np.abs(keys - cut) <= BAND * abs(cut)


def check_selection(sel_gpu, c_ref, k):
    """sel_gpu [k] vs the oracle's TopK of c_ref; returns the number of exemptions."""
    c_ref = np.asarray(c_ref)
    j = np.arange(len(c_ref))
    order = np.lexsort((j, -c_ref))
    want = set(order[:k].tolist())
    got = set(np.asarray(sel_gpu).tolist())
    assert len(got) == k and list(np.asarray(sel_gpu)) == sorted(got), "sel not ascending/unique"
    diff = want ^ got
    exempt = _band_exempt(c_ref, order, k)
    bad = [x for x in diff if not exempt[x]]
    assert not bad, f"selection differs outside the band at blocks {sorted(bad)}"
    return len(diff)


def check_routing(flat_gpu, sharp_gpu, M_ref, n_flat):
    M_ref = np.asarray(M_ref)
    i = np.arange(len(M_ref))
    order = np.lexsort((i, M_ref))
    want = set(order[:n_flat].tolist())
    got = set(np.asarray(flat_gpu).tolist())
    sharp = np.asarray(sharp_gpu)
    assert len(got) == n_flat and list(np.asarray(flat_gpu)) == sorted(got)
    assert list(sharp) == sorted(set(range(len(M_ref))) - got), "sharp is not the complement"
    diff = want ^ got
    exempt = _band_exempt(M_ref, order, n_flat)
    bad = [x for x in diff if not exempt[x]]
    assert not bad, f"routing differs outside the band at blocks {sorted(bad)}"
    return len(diff)


def check_ns(ns_gpu, p_kept, n_ns):
    """One flat block's exact K_new positions vs the oracle's top n_ns of its
    coarse probabilities over the kept blocks (R21); returns the exemptions."""
    p_kept = np.asarray(p_kept)
    u = np.arange(len(p_kept))
    order = np.lexsort((u, -p_kept))
    want = set(order[:n_ns].tolist())
    got = set(np.asarray(ns_gpu).tolist())
    assert len(got) == n_ns and list(np.asarray(ns_gpu)) == sorted(got), "ns not ascending/unique"
    diff = want ^ got
    exempt = _band_exempt(p_kept, order, n_ns)
    bad = [x for x in diff if not exempt[x]]
    assert not bad, f"block mask differs outside the band at K_new positions {sorted(bad)}"
    return len(diff)


def check_close(got, ref, max_abs, mean_abs, what=""):
    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    mx, mn = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= max_abs and mn <= mean_abs, \
        f"{what}: max-abs {mx:.3e} (bar {max_abs:.1e}), mean-abs {mn:.3e} (bar {mean_abs:.1e})"
    return mx, mn


def per_head_decisions(q, k, dtype, L_src, L_ctx, b, alpha_s, alpha_f):
    """Oracle decisions head by head from stored inputs (bf16 bits or fp32)."""
    B, H = q.shape[:2]
    out = {key: [] for key in ("c", "M", "sel", "flat", "sharp")}
    for bi in range(B):
        for h in range(H):
            d = orc.decisions_ref(to_f64(q[bi:bi + 1, h:h + 1], dtype),
                                  to_f64(k[bi:bi + 1, h:h + 1], dtype),
                                  L_src, L_ctx, b, alpha_s, alpha_f)
            for key in out:
                out[key].append(d[key][0, 0])
    return {key: np.stack(v).reshape((B, H) + np.shape(v[0])) for key, v in out.items()}


def fixed_ref_rows(q, k, v, dtype, L_src, L_ctx, b, sel, flat, rows, heads=None):
    """Oracle outputs (O, LSE) at token ``rows`` with the given decisions, head by head.

    ``heads``: optional list of (b, h) pairs; default every head.  Returns arrays
    [len(heads), len(rows), D] and [len(heads), len(rows)].
    """
    B, H = q.shape[:2]
    heads = [(bi, h) for bi in range(B) for h in range(H)] if heads is None else heads
    Os, Ls = [], []
    for bi, h in heads:
        sl = (slice(bi, bi + 1), slice(h, h + 1))
        O, L = orc.isa_ref_fixed(to_f64(q[sl], dtype), to_f64(k[sl], dtype), to_f64(v[sl], dtype),
                                 L_src, L_ctx, b, sel[bi:bi + 1, h:h + 1], flat[bi:bi + 1, h:h + 1],
                                 rows=rows)
        Os.append(O[0, 0])
        Ls.append(L[0, 0])
    return np.stack(Os), np.stack(Ls)


def check_in_value_range(o, v):
    """Each output row is a convex combination of value rows: exact rows weight
    rows of V, flat rows the block means of V (rounded once to the storage
    type, so still inside V's range), a masked flat row both.  Every element of
    O therefore lies between the smallest and the largest value of its head in
    that dim.  Holds at any size; checked at every row.  o, v: GPU tensors
    [B, H, N, D]."""
    lo = v.amin(dim=2, keepdim=True).float()
    hi = v.amax(dim=2, keepdim=True).float()
    tol = 1e-6 * torch.maximum(lo.abs(), hi.abs())  # fp32 accumulation
    of = o.float()
    bad = int(((of < lo - tol) | (of > hi + tol)).sum().item())
    assert bad == 0, f"{bad} elements of O outside the value range of their head"
