"""Seeded synthetic [source | context] inputs for ISA.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.  It holds
none of the method's arithmetic: it only draws random tensors with the
structure of an in-context video-editing sequence (source tokens first, then
context tokens) and rounds them to the storage dtype.

The pages measure on real video latents of a 14B editing model at 5K-50K
tokens ([notes] "research background"; [summary] 1 Introduction); those are
not available, and these generators stand in for them.  ([notes]: the
papernotes.org ICML 2026 notes "Lightning Unified Video Editing via In-Context
Sparse Attention"; [summary]: the paperlayer.ai summary "LIVEditor-14B:
Lightning Unified Video Editing via In-Context Sparse Attention" of arXiv
2605.04569v2.)

Recipe (per (batch, head), in this order, from ``numpy.random.default_rng(seed)``):
  Q, K, V ~ N(0, 1) of shape (N, D), drawn as float32;
  variant "icl" (bf16 workloads):
      mu = a N(0, 1)_D vector scaled to unit norm;
      salient = choice(n_ctx, n_sal, replace=False), n_sal = floor(0.1 n_ctx + 0.5);
      g ~ U(0.25, 2.0), one per query block;
      K[:L_src] += mu; K[L_src:] *= 0.5; K[salient context block] += mu;
  variant "tiny" (the fp32 CPU-checkable case):
      salient = choice(n_ctx, n_sal, replace=False), n_sal = max(1, floor(0.25 n_ctx + 0.5));
      g ~ U(0.25, 2.0), one per query block;
      K[L_src:] *= 0.5; K[salient context block] += mean of the source keys;
  then every query block i is multiplied by g_i; finally, when a gradient
  is requested, dO ~ N(0, 1) of shape (N, D).
bf16 tensors are rounded from float32 with round-to-nearest-even and
returned as their uint16 bit patterns.
"""

import numpy as np

# The workloads, by name: a tiny fp32 case, then the bf16 cases at the pages'
# 5K-50K token scale (H = 40 heads of D = 128, blocks of 64 tokens).
CONFIGS = {
    "tiny_fp32_N512": dict(name="tiny_fp32_N512", B=1, H=2, D=64, L_src=256, L_ctx=256, block=64,
            alpha_s=0.5, alpha_f=0.5, dtype="fp32", variant="tiny", seed=1001),
    "isa_bf16_N8192": dict(name="isa_bf16_N8192", B=1, H=40, D=128, L_src=4096, L_ctx=4096, block=64,
            alpha_s=0.25, alpha_f=0.5, dtype="bf16", variant="icl", seed=1002),
    "isa_bf16_N32768": dict(name="isa_bf16_N32768", B=1, H=40, D=128, L_src=16384, L_ctx=16384, block=64,
            alpha_s=0.25, alpha_f=0.5, dtype="bf16", variant="icl", seed=1003),
    "isa_bf16_N51200": dict(name="isa_bf16_N51200", B=1, H=40, D=128, L_src=25600, L_ctx=25600, block=64,
            alpha_s=0.25, alpha_f=0.5, dtype="bf16", variant="icl", seed=1004,
            sweep_alpha_s=(0.125, 0.25, 0.5), sweep_alpha_f=(0.25, 0.5, 0.75)),
    "isa_fwd_bwd_bf16_B2_N16384": dict(name="isa_fwd_bwd_bf16_B2_N16384", B=2, H=40, D=128, L_src=8192, L_ctx=8192,
            block=64, alpha_s=0.25, alpha_f=0.5, dtype="bf16", variant="icl", seed=1005,
            grad=True),
}


def round_to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x, dtype):
    """Storage array ('bf16' bits or 'fp32') -> float64 values (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def generate(B, H, L_src, L_ctx, D, block, seed, variant="icl", dtype="bf16",
             grad=False, heads=None):
    """Draw Q, K, V (and dO if ``grad``) of shape [B, H, N, D].

    Returns dict(q, k, v[, do]) holding uint16 bf16 bits (dtype "bf16") or
    float32 arrays (dtype "fp32").  ``heads`` (optional list of flat b*H+h
    indices) keeps only those heads, drawn from the same stream as the full
    tensor, so a sample equals the corresponding slice of the full draw.
    """
    N = L_src + L_ctx
    n_src = -(-L_src // block)
    n_ctx = -(-L_ctx // block)
    n_q = n_src + n_ctx
    rng = np.random.default_rng(seed)
    keep = list(range(B * H)) if heads is None else list(heads)
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    names = ("q", "k", "v", "do") if grad else ("q", "k", "v")
    out = {nm: np.zeros((len(keep), N, D), dtype=out_dtype) for nm in names}
    slot = {bh: i for i, bh in enumerate(keep)}
    bounds = [(i * block, min((i + 1) * block, L_src)) for i in range(n_src)] + \
             [(L_src + j * block, min(L_src + (j + 1) * block, N)) for j in range(n_ctx)]
    for bh in range(max(keep) + 1 if keep else 0):
        q = rng.standard_normal((N, D), dtype=np.float32)
        k = rng.standard_normal((N, D), dtype=np.float32)
        v = rng.standard_normal((N, D), dtype=np.float32)
        if variant == "icl":
            mu = rng.standard_normal(D).astype(np.float32)
            mu /= np.float32(np.linalg.norm(mu))
            n_sal = int(np.floor(0.1 * n_ctx + 0.5))
            sal = rng.choice(n_ctx, n_sal, replace=False) if n_ctx else []
            g = rng.uniform(0.25, 2.0, size=n_q).astype(np.float32)
            k[:L_src] += mu
            k[L_src:] *= np.float32(0.5)
            for j in sal:
                s, e = bounds[n_src + j]
                k[s:e] += mu
        elif variant == "tiny":
            n_sal = max(1, int(np.floor(0.25 * n_ctx + 0.5))) if n_ctx else 0
            sal = rng.choice(n_ctx, n_sal, replace=False) if n_ctx else []
            g = rng.uniform(0.25, 2.0, size=n_q).astype(np.float32)
            src_mean = k[:L_src].mean(axis=0) if L_src else np.zeros(D, np.float32)
            k[L_src:] *= np.float32(0.5)
            for j in sal:
                s, e = bounds[n_src + j]
                k[s:e] += src_mean
        elif variant == "plain":
            g = np.ones(n_q, dtype=np.float32)
        else:
            raise ValueError(f"unknown variant {variant!r}")
        for i, (s, e) in enumerate(bounds):
            q[s:e] *= g[i]
        tensors = dict(q=q, k=k, v=v)
        if grad:
            tensors["do"] = rng.standard_normal((N, D), dtype=np.float32)
        if bh in slot:
            for nm in names:
                t = tensors[nm]
                out[nm][slot[bh]] = round_to_bf16_bits(t) if dtype == "bf16" else t
    if heads is None:
        return {nm: a.reshape(B, H, N, D) for nm, a in out.items()}
    return {nm: a.reshape(1, len(keep), N, D) for nm, a in out.items()}


def generate_config(name, heads=None, **overrides):
    """Inputs of one of the named workloads (see CONFIGS)."""
    c = dict(CONFIGS[name])
    c.update(overrides)
    return generate(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["block"], c["seed"],
                    variant=c["variant"], dtype=c["dtype"], grad=c.get("grad", False),
                    heads=heads)
