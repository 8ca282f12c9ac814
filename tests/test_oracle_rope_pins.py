"""Pins of the oracle's decoupled rotary embedding (readings R22-R24), against
what the mathematics and the pages fix.

[notes] "training strategy": source and context positions are each numbered
from 0.  RoFormer (Su et al. 2021, eq. 34) defines the rotation.  The pins:
the rounding to bf16 (ties to even, one rounding from fp64) on hand-picked
values; the positions; the frequencies' closed forms; the rotation against
complex multiplication (an independent formulation); a worked D = 4 example
computed by hand (pair layout and direction); norm preservation; the
relative-position property of the dot product; the decoupling itself
(a context token is rotated like the source token at the same offset).
"""

import math

import numpy as np

import oracle as orc
from synth import bf16_bits_to_f32, round_to_bf16_bits


def test_bf16_rounding_ties_and_single_rounding():
    one = 1.0
    # halfway between 1 and 1 + 2^-7: ties to the even neighbour 1
    assert orc.round_to_bf16(one + 2.0 ** -8) == 1.0
    # halfway between 1 + 2^-7 and 1 + 2^-6: ties to the even neighbour 1 + 2^-6
    assert orc.round_to_bf16(one + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above the tie: rounds up.  Through fp32 first, the 2^-30 would be
    # lost and the tie would round down: the rounding must be a single one.
    assert orc.round_to_bf16(one + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert orc.round_to_bf16(-(one + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)
    assert orc.round_to_bf16(0.0) == 0.0
    assert orc.round_to_bf16(3.0) == 3.0
    assert orc.round_to_bf16(0.1) == 0.10009765625          # 0x3DCD


def test_bf16_rounding_matches_an_fp32_rounding_on_fp32_values():
    # For values that are exact in fp32 there is one rounding either way, so
    # the fp64 rounding must agree with the generator's fp32 -> bf16 rounding.
    x = np.random.default_rng(3).standard_normal(20000).astype(np.float32)
    want = bf16_bits_to_f32(round_to_bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(orc.round_to_bf16(x.astype(np.float64)), want)


def test_storage_rounding_is_the_single_rounding():
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -8])
    np.testing.assert_array_equal(orc.round_to_dtype(x, "bf16"), [1.0 + 2.0 ** -7, 1.0])


def test_fp32_rounding():
    x = np.array([1.0 + 2.0 ** -30, 0.1])
    np.testing.assert_array_equal(orc.round_to_dtype(x, "fp32"),
                                  x.astype(np.float32).astype(np.float64))


def test_positions_restart_at_the_context():
    np.testing.assert_array_equal(orc.rope_positions(3, 2), [0, 1, 2, 0, 1])
    np.testing.assert_array_equal(orc.rope_positions(2, 0), [0, 1])


def test_frequencies_closed_form():
    f = orc.rope_inv_freq(8, 10000.0)
    assert f[0] == 1.0
    assert math.isclose(f[2], 10000.0 ** -0.5, rel_tol=1e-15)   # i = D/4 -> base^(-1/2)
    assert math.isclose(f[1], 0.1, rel_tol=1e-15)               # 10000^(-2/8)


def test_worked_example_d4():
    # D = 4, base 100, one token at position 1 holding (1, 0, 0, 1):
    # pair 0 (dims 0, 1) turns by 1 rad: (1, 0) -> (cos 1, sin 1);
    # pair 1 (dims 2, 3) turns by 100^(-1/2) = 0.1 rad: (0, 1) -> (-sin 0.1, cos 0.1).
    X = np.array([[[0.0, 0.0, 0.0, 0.0], [1.0, 0.0, 0.0, 1.0]]])
    theta = orc.rope_positions(2, 0)[:, None] * orc.rope_inv_freq(4, 100.0)[None, :]
    got = orc.rotate_pairs(X, theta)
    want = [math.cos(1.0), math.sin(1.0), -math.sin(0.1), math.cos(0.1)]
    np.testing.assert_allclose(got[0, 1], want, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(got[0, 0], 0.0)


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((3, 40, 16))
    theta = rng.uniform(-50, 50, (40, 8))
    got = orc.rotate_pairs(X, theta)
    z = (X[..., 0::2] + 1j * X[..., 1::2]) * np.exp(1j * theta)
    np.testing.assert_allclose(got[..., 0::2], z.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[..., 1::2], z.imag, rtol=0, atol=1e-13)
    # each pair keeps its length
    np.testing.assert_allclose(got[..., 0::2] ** 2 + got[..., 1::2] ** 2,
                               X[..., 0::2] ** 2 + X[..., 1::2] ** 2, rtol=1e-13)


def test_dot_product_depends_on_the_position_difference_only():
    rng = np.random.default_rng(11)
    D, base = 64, 10000.0
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    f = orc.rope_inv_freq(D, base)

    def dot(m, n):
        a = orc.rotate_pairs(q[None, :], m * f[None, :])[0]
        b = orc.rotate_pairs(k[None, :], n * f[None, :])[0]
        return a @ b

    for m, n, s in [(5, 2, 7), (100, 300, 1000), (0, 9, 4)]:
        assert math.isclose(dot(m, n), dot(m + s, n + s), rel_tol=1e-10, abs_tol=1e-10)
    assert not math.isclose(dot(5, 2), dot(5, 3), rel_tol=1e-6)


def test_decoupling_context_rotates_like_the_source():
    rng = np.random.default_rng(5)
    L_src, L_ctx, D, base = 9, 6, 8, 500.0
    X = orc.round_to_bf16(rng.standard_normal((2, L_src + L_ctx, D)))
    got = orc.decoupled_rope(X, L_src, base, "bf16")
    # the context alone, as a source-only sequence, gets the same rotation
    ctx_alone = orc.decoupled_rope(X[:, L_src:], L_ctx, base, "bf16")
    np.testing.assert_array_equal(got[:, L_src:], ctx_alone)
    src_alone = orc.decoupled_rope(X[:, :L_src], L_src, base, "bf16")
    np.testing.assert_array_equal(got[:, :L_src], src_alone)
    # position 0 of each segment is the identity (inputs already bf16)
    np.testing.assert_array_equal(got[:, 0], X[:, 0])
    np.testing.assert_array_equal(got[:, L_src], X[:, L_src])
    # and the other positions do turn
    assert np.abs(got[:, 1] - X[:, 1]).max() > 1e-3


def test_isa_with_rope_is_isa_on_the_rotated_inputs():
    from synth import generate, to_f64

    g = generate(1, 2, 256, 192, 64, 64, seed=21, variant="icl", dtype="bf16")
    Q, K, V = (to_f64(g[n], "bf16") for n in ("q", "k", "v"))
    out = orc.isa_ref_rope(Q, K, V, 256, 192, 64, 0.5, 0.5, 10000.0, "bf16")
    Qr = orc.decoupled_rope(Q, 256, 10000.0, "bf16")
    Kr = orc.decoupled_rope(K, 256, 10000.0, "bf16")
    ref = orc.isa_ref(Qr, Kr, V, 256, 192, 64, 0.5, 0.5)
    np.testing.assert_array_equal(out["O"], ref["O"])
    np.testing.assert_array_equal(out["sel"], ref["sel"])
    # the rotated inputs are values of the storage type
    np.testing.assert_array_equal(orc.round_to_bf16(out["Qr"]), out["Qr"])
    # the rotation changes the result (it is not silently skipped)
    plain = orc.isa_ref(Q, K, V, 256, 192, 64, 0.5, 0.5)
    assert np.abs(plain["O"] - out["O"]).max() > 1e-3


def test_rope_backward_finite_differences():
    """The decision-frozen backward with the rotary embedding (R20 with R24)
    against central finite differences of the forward it differentiates: the
    rotated inputs stored unrounded ("fp64"), the decisions fixed from the
    rotated inputs.  A wrong direction of the turn back (R instead of R^T) or
    a missing turn fails at every non-zero angle; position 0 of each segment
    (angle 0) is the only place the two agree."""
    rng = np.random.default_rng(41)
    L_src, L_ctx, b, D, base = 8, 12, 4, 4, 50.0
    N = L_src + L_ctx
    Q, K, V, dO = (rng.standard_normal((1, 1, N, D)) for _ in range(4))
    Qr = orc.decoupled_rope(Q, L_src, base, "fp64")
    Kr = orc.decoupled_rope(K, L_src, base, "fp64")
    d = orc.decisions_ref(Qr, Kr, L_src, L_ctx, b, 0.5, 0.5)
    assert len(d["flat"][0, 0]) > 0 and len(d["sharp"][0, 0]) > 0
    sel, flat = d["sel"], d["flat"]
    dQ, dK, dV = orc.isa_ref_bwd_rope(Q, K, V, dO, L_src, L_ctx, b, sel, flat, base, "fp64")

    def loss():
        O, _ = orc.isa_ref_fixed(orc.decoupled_rope(Q, L_src, base, "fp64"),
                                 orc.decoupled_rope(K, L_src, base, "fp64"), V,
                                 L_src, L_ctx, b, sel, flat)
        return float((O * dO).sum())

    eps = 1e-6
    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + eps
            lp = loss()
            X[idx] = old - eps
            lm = loss()
            X[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        scale = np.abs(num).max()
        np.testing.assert_allclose(G, num, atol=1e-6 * scale, rtol=0)
    # the turn back matters: the unrotated gradient of the rotated forward differs
    dQr, _, _ = orc.isa_ref_bwd(Qr, Kr, V, dO, L_src, L_ctx, b, sel, flat)
    assert np.abs(dQr - dQ).max() > 1e-3 * np.abs(dQ).max()
