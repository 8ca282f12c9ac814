"""GPU parity of the decision-frozen ISA backward against the fp64 oracle.

The forward runs on the GPU first; its decisions (sel, flat, sharp) are given
to both the GPU backward and the oracle's isa_ref_bwd.  Bars (the pages print
none; a reading, derived from bf16 operands with fp32 accumulation): for each of
dQ, dK, dV, relative Frobenius error <= 1e-2 and max-abs error <= 2e-2 of the
largest reference magnitude.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import generate, generate_config, CONFIGS, to_f64
from tests.parity import out_f64, to_gpu

pytestmark = pytest.mark.gpu

REL_FRO, MAX_FRAC = 1e-2, 2e-2


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _fwd_bwd(inp, B, H, L_src, L_ctx, D, alpha_s, alpha_f, alpha_ns=0.0, block=64):
    plan = isa.isa_plan_create(B, H, L_src, L_ctx, D, block, alpha_s, alpha_f, alpha_ns)
    q, k, v, do = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v", "do"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    dq, dk, dv = isa.isa_backward(plan, q, k, v, o, do, lse, aux)
    torch.cuda.synchronize()
    return plan, (dq, dk, dv), {key: t.cpu().numpy() for key, t in aux.items()}


def _check_grads(got, ref, what=""):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = np.asarray(g, dtype=np.float64)
        rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
        mx = np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)
        assert rel <= REL_FRO and mx <= MAX_FRAC, \
            f"{what} {name}: rel-Frobenius {rel:.3e} (bar {REL_FRO}), max-abs/max|ref| {mx:.3e}"
        _say(f"{what} {name}: rel-Frobenius {rel:.2e}, max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("B,H,L_src,L_ctx,D,alpha_s,alpha_f,seed", [
    (1, 2, 512, 512, 128, 0.5, 0.5, 41),
    (1, 3, 640, 448, 128, 0.25, 0.5, 42),   # 17 blocks: odd worklists, 12 pooled rows
    (2, 2, 1024, 768, 64, 0.34, 0.3, 43),   # D = 64, B = 2
    (1, 2, 512, 512, 128, 0.5, 0.0, 44),    # exact path only
    (1, 2, 512, 512, 128, 0.5, 1.0, 45),    # Taylor path only
    (1, 2, 512, 512, 128, 0.0, 0.5, 46),    # no context kept
    (1, 2, 512, 0, 128, 0.5, 0.5, 47),      # no context at all
])
def test_backward_small_full_parity(B, H, L_src, L_ctx, D, alpha_s, alpha_f, seed):
    _say(f"bwd B{B} H{H} L_src{L_src} L_ctx{L_ctx} D{D} as{alpha_s} af{alpha_f} seed{seed}")
    inp = generate(B, H, L_src, L_ctx, D, 64, seed=seed, variant="icl", grad=True)
    plan, grads, aux = _fwd_bwd(inp, B, H, L_src, L_ctx, D, alpha_s, alpha_f)
    ref = orc.isa_ref_bwd(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v", "do")),
                          L_src, L_ctx, 64, aux["sel"], aux["flat"])
    _check_grads([out_f64(g) for g in grads], ref, "full")
    # context rows of blocks that were not kept get exactly zero
    dk = out_f64(grads[1])
    for bi in range(B):
        for h in range(H):
            for j in range(L_ctx // 64):
                if j not in aux["sel"][bi, h]:
                    assert not dk[bi, h, L_src + 64 * j:L_src + 64 * (j + 1)].any()


@pytest.mark.parametrize("B,H,L_src,L_ctx,D,alpha_s,alpha_f,alpha_ns,seed", [
    (1, 2, 1024, 1024, 128, 0.5, 0.5, 0.0625, 61),  # the pages' ratio: 2 of 24 blocks exact
    (1, 3, 640, 448, 128, 0.25, 0.45, 0.25, 62),    # 7 flat blocks: a lone dQ pair member
    (2, 2, 1024, 768, 64, 0.34, 0.3, 0.2, 63),      # D = 64, B = 2, N_K' = 21: a half key group
    (1, 2, 1024, 1024, 128, 0.5, 1.0, 0.125, 64),   # every block flat: no sharp rows
    (1, 2, 512, 512, 128, 0.5, 0.5, 1.0, 65),       # every kept block exact in flat rows
])
def test_backward_block_mask_parity(B, H, L_src, L_ctx, D, alpha_s, alpha_f, alpha_ns, seed):
    """The block mask inside flat rows: the GPU backward against isa_ref_bwd
    with the forward's ns."""
    _say(f"bwd mask B{B} H{H} L_src{L_src} L_ctx{L_ctx} D{D} as{alpha_s} af{alpha_f} "
         f"ans{alpha_ns} seed{seed}")
    inp = generate(B, H, L_src, L_ctx, D, 64, seed=seed, variant="icl", grad=True)
    plan, grads, aux = _fwd_bwd(inp, B, H, L_src, L_ctx, D, alpha_s, alpha_f, alpha_ns)
    assert plan.info["n_ns"] > 0 and plan.info["n_flat"] > 0
    ref = orc.isa_ref_bwd(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v", "do")),
                          L_src, L_ctx, 64, aux["sel"], aux["flat"], aux["ns"])
    _check_grads([out_f64(g) for g in grads], ref, "mask")
    dk = out_f64(grads[1])
    for bi in range(B):
        for h in range(H):
            for j in range(L_ctx // 64):
                if j not in aux["sel"][bi, h]:
                    assert not dk[bi, h, L_src + 64 * j:L_src + 64 * (j + 1)].any()


@pytest.mark.parametrize("B,H,L_src,L_ctx,D,b,alpha_s,alpha_f,alpha_ns,seed", [
    (1, 2, 1000, 1100, 128, 64, 0.5, 0.5, 0.0, 71),    # both segments end in a partial block
    (1, 2, 40, 600, 128, 64, 0.5, 0.5, 0.0, 72),       # the source is one partial block
    (1, 2, 512, 40, 128, 64, 1.0, 0.5, 0.0, 73),       # the context is one partial block, kept
    (2, 2, 700, 900, 64, 64, 0.34, 0.3, 0.0, 74),      # D = 64, B = 2, partial blocks
    (1, 2, 512, 512, 128, 32, 0.5, 0.5, 0.0, 75),      # b = 32: two blocks per tile
    (1, 3, 500, 300, 64, 32, 0.34, 0.45, 0.0, 76),     # b = 32, partial, odd block counts
    (1, 2, 1024, 1024, 128, 128, 0.5, 0.5, 0.0, 77),   # b = 128: two tiles per block
    (2, 2, 700, 900, 64, 128, 0.5, 0.3, 0.0, 78),      # b = 128, partial (one-tile blocks)
    (1, 2, 1000, 1100, 128, 64, 0.5, 0.5, 0.125, 79),  # partial blocks with the block mask
])
def test_backward_general_blocks_parity(B, H, L_src, L_ctx, D, b, alpha_s, alpha_f, alpha_ns,
                                        seed):
    """Partial blocks (either segment not a multiple of b) and b = 32, 128: the
    GPU backward against isa_ref_bwd on the same grid."""
    _say(f"bwd blocks B{B} H{H} L_src{L_src} L_ctx{L_ctx} D{D} b{b} as{alpha_s} af{alpha_f} "
         f"ans{alpha_ns} seed{seed}")
    inp = generate(B, H, L_src, L_ctx, D, b, seed=seed, variant="icl", grad=True)
    plan, grads, aux = _fwd_bwd(inp, B, H, L_src, L_ctx, D, alpha_s, alpha_f, alpha_ns, b)
    ref = orc.isa_ref_bwd(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v", "do")),
                          L_src, L_ctx, b, aux["sel"], aux["flat"], aux.get("ns"))
    _check_grads([out_f64(g) for g in grads], ref, "blocks")
    starts, ends, n_src, n_ctx = orc.block_grid(L_src, L_ctx, b)
    dk = out_f64(grads[1])
    for bi in range(B):
        for h in range(H):
            for j in range(n_ctx):
                if j not in aux["sel"][bi, h]:
                    assert not dk[bi, h, starts[n_src + j]:ends[n_src + j]].any()


def test_backward_block_mask_deterministic():
    _say("bwd mask determinism B1 H2 N2048 ans 0.0625 seed 66")
    inp = generate(1, 2, 1024, 1024, 128, 64, seed=66, variant="icl", grad=True)
    _, g1, _ = _fwd_bwd(inp, 1, 2, 1024, 1024, 128, 0.25, 0.5, 0.0625)
    _, g2, _ = _fwd_bwd(inp, 1, 2, 1024, 1024, 128, 0.25, 0.5, 0.0625)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_all_kept_all_exact_is_dense_backward():
    _say("bwd as1 af0 vs dense backward, seed 48")
    inp = generate(1, 2, 512, 512, 128, 64, seed=48, variant="icl", grad=True)
    _, grads, _ = _fwd_bwd(inp, 1, 2, 512, 512, 128, 1.0, 0.0)
    ref = orc.dense_ref_bwd(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v", "do")))
    _check_grads([out_f64(g) for g in grads], ref, "dense")


def test_backward_deterministic():
    _say("bwd determinism B1 H2 N2048 seed 49")
    inp = generate(1, 2, 1024, 1024, 128, 64, seed=49, variant="icl", grad=True)
    _, g1, _ = _fwd_bwd(inp, 1, 2, 1024, 1024, 128, 0.25, 0.5)
    _, g2, _ = _fwd_bwd(inp, 1, 2, 1024, 1024, 128, 0.25, 0.5)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_workload_b2_n16384():
    c = CONFIGS["isa_fwd_bwd_bf16_B2_N16384"]
    B, H, L_src, L_ctx, D = c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"]
    _say(f"bwd workload {c['name']} seed {c['seed']}")
    inp = generate_config("isa_fwd_bwd_bf16_B2_N16384")
    plan, grads, aux = _fwd_bwd(inp, B, H, L_src, L_ctx, D, c["alpha_s"], c["alpha_f"])
    got = [out_f64(g) for g in grads]
    for g in got:
        assert np.isfinite(g).all()
    # four heads spanning both batch entries
    for bi, h in ((0, 3), (0, 22), (1, 11), (1, 29)):
        sl = (slice(bi, bi + 1), slice(h, h + 1))
        ref = orc.isa_ref_bwd(*(to_f64(inp[x][sl], "bf16") for x in ("q", "k", "v", "do")),
                              L_src, L_ctx, 64, aux["sel"][sl], aux["flat"][sl])
        _check_grads([g[sl] for g in got], ref, f"head ({bi},{h})")
    # every head: sum_t dV_t = sum_r dO_r and sum_t dK_t = 0 (each P or pi row
    # sums to one, each dS row to zero, and the Taylor broadcast gives every
    # token of block j the share dV^c_j / w_j), to the rounding of the bf16
    # operands and outputs, compared with the root sum of squares of the terms
    dk, dv = got[1], got[2]
    do = to_f64(inp["do"], "bf16")
    err_v = np.abs(dv.sum(axis=2) - do.sum(axis=2)) / np.sqrt((dv ** 2).sum(axis=2)
                                                              + (do ** 2).sum(axis=2))
    err_k = np.abs(dk.sum(axis=2)) / np.sqrt((dk ** 2).sum(axis=2))
    assert err_v.max() <= 0.05 and err_k.max() <= 0.05, (err_v.max(), err_k.max())
    _say(f"every head: |sum dV - sum dO| / RSS max {err_v.max():.2e}, "
         f"|sum dK| / RSS max {err_k.max():.2e}")


def test_backward_block_mask_workload_b2_n16384():
    """The backward workload with the block mask at the pages' ratio
    alpha_ns = 0.0625: two heads (one per batch entry) in full against the
    oracle, every head by the gradient-sum identities."""
    c = CONFIGS["isa_fwd_bwd_bf16_B2_N16384"]
    B, H, L_src, L_ctx, D = c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"]
    _say(f"bwd mask workload {c['name']} ans 0.0625 seed {c['seed']}")
    inp = generate_config("isa_fwd_bwd_bf16_B2_N16384")
    plan, grads, aux = _fwd_bwd(inp, B, H, L_src, L_ctx, D, c["alpha_s"], c["alpha_f"], 0.0625)
    assert plan.info["n_ns"] > 0
    got = [out_f64(g) for g in grads]
    for g in got:
        assert np.isfinite(g).all()
    for bi, h in ((0, 17), (1, 6)):
        sl = (slice(bi, bi + 1), slice(h, h + 1))
        ref = orc.isa_ref_bwd(*(to_f64(inp[x][sl], "bf16") for x in ("q", "k", "v", "do")),
                              L_src, L_ctx, 64, aux["sel"][sl], aux["flat"][sl], aux["ns"][sl])
        _check_grads([g[sl] for g in got], ref, f"mask head ({bi},{h})")
    dk, dv = got[1], got[2]
    do = to_f64(inp["do"], "bf16")
    err_v = np.abs(dv.sum(axis=2) - do.sum(axis=2)) / np.sqrt((dv ** 2).sum(axis=2)
                                                              + (do ** 2).sum(axis=2))
    err_k = np.abs(dk.sum(axis=2)) / np.sqrt((dk ** 2).sum(axis=2))
    assert err_v.max() <= 0.05 and err_k.max() <= 0.05, (err_v.max(), err_k.max())
    _say(f"every head: |sum dV - sum dO| / RSS max {err_v.max():.2e}, "
         f"|sum dK| / RSS max {err_k.max():.2e}")
