"""fp64 CPU oracle of the decoupled rotary position embedding -- TEST
INFRASTRUCTURE ONLY (same rules as ``isa_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may import it).

[notes] "training strategy": to remove the positional bias that the unequal
lengths of source and context cause, the editor numbers the positions of the
source and of the context each from 0 (a decoupled RoPE).  The pages fix
nothing else about the embedding.  Readings (each used identically by the HIP
path):

  R22 the rotary embedding is the one-dimensional rotation of RoFormer (Su et
      al., "RoFormer: Enhanced Transformer with Rotary Position Embedding",
      2021, eq. 34): dimensions (2i, 2i+1) of a head form a pair that is
      rotated by the angle pos * base^(-2i/D), i = 0 .. D/2 - 1.  The base is
      a parameter (10000 in RoFormer).
  R23 positions: source token t has pos = t, context token t (t >= L_src) has
      pos = t - L_src.
  R24 the embedding is applied to Q and K (not V) before every step of ISA,
      so pooling, the coarse map, pre-selection, routing and both paths all
      see the rotated Q and K.  The rotated values are rounded once, with
      round-to-nearest-even, to the storage type of the inputs (bf16 or fp32),
      as the layer that applies the embedding stores its result.
"""

import math

import numpy as np


def round_to_bf16(x):
    """fp64 -> nearest bf16 value (ties to even), returned as fp64.

    Rounds the fp64 value directly (no detour through fp32, which would round
    twice).  bf16 keeps 8 significant bits: x = m * 2^e with 0.5 <= |m| < 1,
    so the kept value is rint(m * 2^8) * 2^(e - 8), rint rounding ties to even.
    Zero stays zero; the inputs here are far from bf16's overflow and
    subnormal range.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_to_dtype(x, dtype):
    """fp64 -> the values of the storage type ("bf16" or "fp32"), as fp64.
    "fp64" stores unrounded (used by the finite-difference pins)."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def rope_positions(L_src, L_ctx):
    """R23: positions of the N = L_src + L_ctx tokens, each segment from 0."""
    return np.concatenate([np.arange(L_src), np.arange(L_ctx)]).astype(np.float64)


def rope_inv_freq(D, base):
    """R22: base^(-2i/D) for the D/2 pairs."""
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / D)


def rotate_pairs(X, theta):
    """Rotate pair i = (X[..., 2i], X[..., 2i+1]) of every row by theta[row, i].

    X [..., N, D] fp64, theta [N, D/2].  Unrounded (the rotation itself)."""
    X = np.asarray(X, dtype=np.float64)
    c, s = np.cos(theta), np.sin(theta)
    x, y = X[..., 0::2], X[..., 1::2]
    out = np.empty_like(X)
    out[..., 0::2] = x * c - y * s
    out[..., 1::2] = x * s + y * c
    return out


def decoupled_rope(X, L_src, base, dtype):
    """R22-R24 for [..., N, D] (the N axis is [source | context]).

    Returns the rotated X rounded to ``dtype``, as fp64."""
    X = np.asarray(X, dtype=np.float64)
    N, D = X.shape[-2], X.shape[-1]
    if D % 2:
        raise ValueError("the head dimension must be even")
    theta = rope_positions(L_src, N - L_src)[:, None] * rope_inv_freq(D, base)[None, :]
    return round_to_dtype(rotate_pairs(X, theta), dtype)


def isa_ref_rope(Q, K, V, L_src, L_ctx, b, alpha_s, alpha_f, rope_base, dtype, alpha_ns=0.0):
    """The ISA forward with the decoupled RoPE applied to Q and K first (R24).

    Returns isa_ref's dict plus the rotated inputs Qr, Kr."""
    from .isa_oracle import isa_ref

    Qr = decoupled_rope(Q, L_src, rope_base, dtype)
    Kr = decoupled_rope(K, L_src, rope_base, dtype)
    out = isa_ref(Qr, Kr, V, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns)
    out["Qr"], out["Kr"] = Qr, Kr
    return out


def isa_ref_bwd_rope(Q, K, V, dO, L_src, L_ctx, b, sel, flat, rope_base, dtype, ns=None):
    """Gradients (dQ, dK, dV) of sum(dO * O) of the ISA forward with the
    decoupled RoPE (R24) and the decisions sel, flat fixed (R20).

    The embedding turns each pair of Q and K by an angle that depends only on
    the token's position: Q' = R Q with R orthogonal, so the chain rule gives
    dQ = R^T dQ', each pair of dQ' turned back by the same angle, and likewise
    for K; V is not rotated.  dQ', dK', dV are the backward of the rotated
    forward (isa_ref_bwd at the rotated inputs).  The rounding of the rotated
    values to the storage type (R24) is a storage step, not a part of the
    function: the gradient is that of the rotation itself, evaluated at the
    rounded Q', K' the forward used (as a layer stores its output and
    back-propagates through its arithmetic)."""
    from .isa_oracle_bwd import isa_ref_bwd

    Q = np.asarray(Q, dtype=np.float64)
    N, D = Q.shape[-2], Q.shape[-1]
    Qr = decoupled_rope(Q, L_src, rope_base, dtype)
    Kr = decoupled_rope(K, L_src, rope_base, dtype)
    dQr, dKr, dV = isa_ref_bwd(Qr, Kr, V, dO, L_src, L_ctx, b, sel, flat, ns)
    theta = rope_positions(L_src, N - L_src)[:, None] * rope_inv_freq(D, rope_base)[None, :]
    return rotate_pairs(dQr, -theta), rotate_pairs(dKr, -theta), dV


def rope_angle(pos, i, D, base):
    """One angle, from the scalar formula (used by the pins)."""
    return pos * math.pow(base, -2.0 * i / D)
