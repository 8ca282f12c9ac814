"""GPU parity of the decoupled rotary embedding (readings R22-R24) against the
fp64 oracle, through the C ABI.

The library rotates Q and K inside its pooling kernel and runs every later
step on the rotated copies; the oracle rotates in fp64, rounds once to the
storage type and runs its plain ISA.  The decisions must agree bit for bit
(up to the near-tie band), so the rotated inputs must agree too.  Every case
prints its name, shape and seed (flushed) before touching the GPU.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import generate, round_to_bf16_bits, to_f64
from tests.parity import (BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS, FP32_MEAN_ABS, check_close,
                          check_in_value_range, check_ns, check_routing, check_selection, out_f64,
                          to_gpu)

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _rotated(x_store, dtype, L_src, base):
    """Oracle rotation of stored inputs, as fp64 values of the storage type."""
    return orc.decoupled_rope(to_f64(x_store, dtype), L_src, base, dtype)


def _parity(inp, dtype, B, H, L_src, L_ctx, D, a_s, a_f, base, a_ns=0.0, rows=None,
            heads=None):
    plan = isa.isa_plan_create(B, H, L_src, L_ctx, D, 64, a_s, a_f, a_ns,
                               dtype=TORCH_DT[dtype], rope_base=base)
    info = plan.info
    q, k, v = (to_gpu(inp[x], dtype) for x in ("q", "k", "v"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    torch.cuda.synchronize()
    lse = lse.cpu().numpy()
    aux = {key: t.cpu().numpy() for key, t in aux.items()}
    # the inputs are not modified: the rotation goes to the workspace
    np.testing.assert_array_equal(q.cpu().view(torch.int16 if dtype == "bf16" else torch.int32)
                                  .numpy(), inp["q"].view(np.int16 if dtype == "bf16" else np.int32))

    Qr = _rotated(inp["q"], dtype, L_src, base)
    Kr = _rotated(inp["k"], dtype, L_src, base)
    V = to_f64(inp["v"], dtype)
    ex = [0, 0, 0]
    for bi in range(B):
        for h in range(H):
            d = orc.decisions_ref(Qr[bi:bi + 1, h:h + 1], Kr[bi:bi + 1, h:h + 1], L_src, L_ctx,
                                  64, a_s, a_f, a_ns)
            ex[0] += check_selection(aux["sel"][bi, h], d["c"][0, 0], info["k"])
            ex[1] += check_routing(aux["flat"][bi, h], aux["sharp"][bi, h], d["M"][0, 0],
                                   info["n_flat"])
            if a_ns > 0 and info["n_flat"] > 0 and ex[0] == 0 and ex[1] == 0:
                # the mask ranks coarse logits of the kept blocks per flat block
                ex[2] += _check_mask(aux, bi, h, Qr, Kr, L_src, L_ctx, info)
    bars = (BF16_MAX_ABS, BF16_MEAN_ABS) if dtype == "bf16" else (FP32_MAX_ABS, FP32_MEAN_ABS)
    ns = aux.get("ns")
    heads = [(bi, h) for bi in range(B) for h in range(H)] if heads is None else heads
    O_gpu = out_f64(o)
    for bi, h in heads:
        sl = (slice(bi, bi + 1), slice(h, h + 1))
        O_ref, L_ref = orc.isa_ref_fixed(Qr[sl], Kr[sl], V[sl], L_src, L_ctx, 64,
                                         aux["sel"][sl], aux["flat"][sl], rows=rows,
                                         ns=None if ns is None else ns[sl])
        got = O_gpu[bi, h] if rows is None else O_gpu[bi, h, rows]
        got_l = lse[bi, h] if rows is None else lse[bi, h, rows]
        mx, mn = check_close(got, O_ref[0, 0], *bars, what=f"O head ({bi},{h})")
        check_close(got_l, L_ref[0, 0], 5e-3 if dtype == "bf16" else 1e-5,
                    1e-3 if dtype == "bf16" else 1e-6, what=f"LSE head ({bi},{h})")
    assert torch.isfinite(o.float()).all()
    check_in_value_range(o, to_gpu(inp["v"], dtype))
    _say(f"ok max-abs {mx:.2e} mean-abs {mn:.2e} exemptions {ex}")
    return o


def _check_mask(aux, bi, h, Qr, Kr, L_src, L_ctx, info):
    starts, ends, n_src, _ = orc.block_grid(L_src, L_ctx, 64)
    Qc = orc.pool_blocks(Qr[bi, h], starts, ends)
    Kc = orc.pool_blocks(Kr[bi, h], starts, ends)
    P = orc.coarse_probs(Qc, Kc)
    kept = np.concatenate([np.arange(n_src), n_src + aux["sel"][bi, h]]).astype(np.int64)
    n = 0
    for f, i in enumerate(aux["flat"][bi, h]):
        n += check_ns(aux["ns"][bi, h, f], P[i, kept], info["n_ns"])
    return n


@pytest.mark.parametrize("B,H,L_src,L_ctx,D,a_s,a_f,base,seed", [
    (1, 2, 512, 384, 128, 0.5, 0.5, 10000.0, 91),
    (1, 2, 700, 500, 128, 0.5, 0.5, 10000.0, 92),      # partial blocks (tails 60 and 52)
    (2, 2, 256, 256, 64, 0.5, 0.3, 500.0, 93),         # D = 64, B = 2, a small base
    (1, 2, 512, 512, 128, 1.0, 0.0, 10000.0, 94),      # alpha_s = 1, alpha_f = 0: dense over Kr
])
def test_rope_bf16_full_parity(B, H, L_src, L_ctx, D, a_s, a_f, base, seed):
    _say(f"rope bf16 B{B} H{H} L_src{L_src} L_ctx{L_ctx} D{D} as{a_s} af{a_f} base{base} "
         f"seed{seed}")
    inp = generate(B, H, L_src, L_ctx, D, 64, seed=seed, variant="icl")
    _parity(inp, "bf16", B, H, L_src, L_ctx, D, a_s, a_f, base)


def test_rope_fp32_full_parity():
    _say("rope fp32 B1 H2 L_src256 L_ctx200 D64 base 100 seed 95")
    inp = generate(1, 2, 256, 200, 64, 64, seed=95, variant="tiny", dtype="fp32")
    _parity(inp, "fp32", 1, 2, 256, 200, 64, 0.5, 0.5, 100.0)


def test_rope_with_block_mask():
    _say("rope bf16 mask B1 H2 L_src640 L_ctx640 ans0.25 seed 96")
    inp = generate(1, 2, 640, 640, 128, 64, seed=96, variant="icl")
    _parity(inp, "bf16", 1, 2, 640, 640, 128, 0.5, 0.5, 10000.0, a_ns=0.25)


def test_rope_dense_equivalence_against_rotated_inputs():
    # alpha_s = 1, alpha_f = 0: the library's ISA with the embedding equals its
    # own dense kernel run on the oracle's rotated inputs
    L = 512
    _say(f"rope dense equivalence B1 H2 L_src{L} L_ctx{L} seed 97")
    inp = generate(1, 2, L, L, 128, 64, seed=97, variant="icl")
    o = _parity(inp, "bf16", 1, 2, L, L, 128, 1.0, 0.0, 10000.0)
    qr = to_gpu(round_to_bf16_bits(_rotated(inp["q"], "bf16", L, 10000.0).astype(np.float32)),
                "bf16")
    kr = to_gpu(round_to_bf16_bits(_rotated(inp["k"], "bf16", L, 10000.0).astype(np.float32)),
                "bf16")
    od, _ = isa.isa_dense_forward(qr, kr, to_gpu(inp["v"], "bf16"))
    torch.cuda.synchronize()
    assert torch.equal(o, od)


def test_rope_workload_scale():
    # 4 heads at N = 8192: every decision of every head, sampled rows of two heads
    L_src = L_ctx = 4096
    N = L_src + L_ctx
    _say(f"rope workload B1 H4 L_src{L_src} L_ctx{L_ctx} seed 98")
    inp = generate(1, 4, L_src, L_ctx, 128, 64, seed=98, variant="icl")
    rng = np.random.default_rng(98)
    rows = np.unique(np.concatenate([rng.choice(N, 300, replace=False), [0, L_src, N - 1]]))
    _parity(inp, "bf16", 1, 4, L_src, L_ctx, 128, 0.25, 0.5, 10000.0, rows=rows,
            heads=[(0, 1), (0, 3)])


@pytest.mark.parametrize("B,H,L_src,L_ctx,D,alpha_s,alpha_f,base,seed,b,alpha_ns", [
    (1, 2, 512, 512, 128, 0.5, 0.5, 10000.0, 81, 64, 0.0),
    (1, 3, 640, 448, 128, 0.25, 0.5, 100.0, 82, 64, 0.0),   # 17 blocks, a fast-turning base
    (2, 2, 1024, 768, 64, 0.34, 0.3, 10000.0, 83, 64, 0.0),  # D = 64, B = 2
    (1, 2, 1000, 600, 128, 0.5, 0.5, 10000.0, 84, 64, 0.0),  # partial blocks
    (1, 2, 1024, 1024, 128, 0.5, 0.5, 10000.0, 85, 128, 0.0),  # b = 128
    (1, 2, 1024, 1024, 128, 0.5, 0.5, 10000.0, 86, 64, 0.0625),  # with the block mask
])
def test_rope_backward_parity(B, H, L_src, L_ctx, D, alpha_s, alpha_f, base, seed, b, alpha_ns):
    """The decision-frozen backward with the rotary embedding against the
    oracle's isa_ref_bwd_rope (the backward at the rotated inputs, dQ and dK
    turned back).  Bars as the other backward tests: relative Frobenius <= 1e-2
    and max-abs <= 2e-2 of the largest reference magnitude per tensor."""
    _say(f"rope bwd B{B} H{H} L_src{L_src} L_ctx{L_ctx} D{D} as{alpha_s} af{alpha_f} "
         f"base{base} seed{seed}")
    inp = generate(B, H, L_src, L_ctx, D, b, seed=seed, variant="icl", grad=True)
    plan = isa.isa_plan_create(B, H, L_src, L_ctx, D, b, alpha_s, alpha_f, alpha_ns,
                               rope_base=base)
    q, k, v, do = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v", "do"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    dq, dk, dv = isa.isa_backward(plan, q, k, v, o, do, lse, aux)
    torch.cuda.synchronize()
    sel, flat = aux["sel"].cpu().numpy(), aux["flat"].cpu().numpy()
    ns = aux["ns"].cpu().numpy() if "ns" in aux else None
    ref = orc.isa_ref_bwd_rope(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v", "do")),
                               L_src, L_ctx, b, sel, flat, base, "bf16", ns)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        g = out_f64(g)
        rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
        mx = np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)
        _say(f"rope bwd {name}: rel-Frobenius {rel:.2e}, max-abs/max|ref| {mx:.2e}")
        assert rel <= 1e-2 and mx <= 2e-2, f"{name}: rel {rel:.3e} max {mx:.3e}"
