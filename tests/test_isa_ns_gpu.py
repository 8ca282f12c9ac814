"""GPU parity of the block mask inside flat query blocks (alpha_ns > 0,
reading R21: the top ceil(alpha_ns * N_K') K_new blocks of each flat query
block's coarse row are computed token by token, the others through their
representatives) against the fp64 oracle, through the C ABI.

Decisions: sel and routing as in the other parity tests, and every flat
block's exact list against the oracle's ranking of the coarse probabilities
over the GPU's kept blocks (relative 1e-5 band at the cut).  Outputs: the
oracle run with the GPU's own decisions.  Every case prints its name, shape and
seed (flushed) before touching the GPU.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import CONFIGS, generate, generate_config, to_f64
from tests.parity import (BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS, FP32_MEAN_ABS, check_close,
                          check_in_value_range, check_ns, check_routing, check_selection, out_f64,
                          to_gpu)

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(inp, dtype, B, H, L_src, L_ctx, D, a_s, a_f, a_ns):
    plan = isa.isa_plan_create(B, H, L_src, L_ctx, D, 64, a_s, a_f, a_ns, dtype=TORCH_DT[dtype])
    q, k, v = (to_gpu(inp[x], dtype) for x in ("q", "k", "v"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    torch.cuda.synchronize()
    return plan, o, lse.cpu().numpy(), {key: t.cpu().numpy() for key, t in aux.items()}


def _check_all_decisions(inp, dtype, plan, aux, L_src, L_ctx, a_s, a_f):
    info = plan.info
    B, H = aux["sel"].shape[:2]
    starts, ends, n_src, _ = orc.block_grid(L_src, L_ctx, 64)
    ex = [0, 0, 0]
    for bi in range(B):
        for h in range(H):
            sl = (slice(bi, bi + 1), slice(h, h + 1))
            q64, k64 = to_f64(inp["q"][sl], dtype), to_f64(inp["k"][sl], dtype)
            d = orc.decisions_ref(q64, k64, L_src, L_ctx, 64, a_s, a_f)
            ex[0] += check_selection(aux["sel"][bi, h], d["c"][0, 0], info["k"])
            ex[1] += check_routing(aux["flat"][bi, h], aux["sharp"][bi, h], d["M"][0, 0],
                                   info["n_flat"])
            P = orc.coarse_probs(orc.pool_blocks(q64[0, 0], starts, ends),
                                 orc.pool_blocks(k64[0, 0], starts, ends))
            kept = np.concatenate([np.arange(n_src), n_src + aux["sel"][bi, h]])
            for f, i in enumerate(aux["flat"][bi, h]):
                ex[2] += check_ns(aux["ns"][bi, h, f], P[i, kept], info["n_ns"])
    return ex


def _parity(inp, dtype, B, H, L_src, L_ctx, D, a_s, a_f, a_ns, bars):
    plan, o, lse, aux = _run(inp, dtype, B, H, L_src, L_ctx, D, a_s, a_f, a_ns)
    assert plan.info["n_ns"] == orc.ns_count(a_ns, plan.info["n_kv_blocks"])
    ex = _check_all_decisions(inp, dtype, plan, aux, L_src, L_ctx, a_s, a_f)
    O_ref, L_ref = orc.isa_ref_fixed(*(to_f64(inp[x], dtype) for x in ("q", "k", "v")),
                                     L_src, L_ctx, 64, aux["sel"], aux["flat"], ns=aux["ns"])
    mx, mn = check_close(out_f64(o), O_ref, *bars, what="O")
    check_close(lse, L_ref, 5e-3 if dtype == "bf16" else 1e-5, 1e-3 if dtype == "bf16" else 1e-6,
                what="LSE")
    _say(f"ok n_ns {plan.info['n_ns']} max-abs {mx:.2e} mean-abs {mn:.2e} "
         f"exemptions sel/route/mask {ex}")
    return plan, o, aux, O_ref


@pytest.mark.parametrize("B,H,L_src,L_ctx,D,a_s,a_f,a_ns,seed", [
    (1, 3, 640, 448, 128, 0.25, 0.5, 0.0625, 61),  # n_ns = 1: one exact block per flat row
    (2, 2, 1024, 1024, 64, 0.5, 0.25, 0.25, 62),   # D = 64, B = 2
    (1, 2, 2048, 1536, 128, 0.34, 0.7, 0.5, 63),   # half the blocks exact
    (1, 2, 512, 512, 128, 0.5, 1.0, 0.3, 64),      # every query block flat
    (1, 2, 512, 0, 128, 0.5, 0.5, 0.5, 65),        # no context at all
])
def test_mask_bf16_small_full_parity(B, H, L_src, L_ctx, D, a_s, a_f, a_ns, seed):
    _say(f"mask bf16 B{B} H{H} L_src{L_src} L_ctx{L_ctx} D{D} as{a_s} af{a_f} ans{a_ns} seed{seed}")
    inp = generate(B, H, L_src, L_ctx, D, 64, seed=seed, variant="icl")
    _parity(inp, "bf16", B, H, L_src, L_ctx, D, a_s, a_f, a_ns, (BF16_MAX_ABS, BF16_MEAN_ABS))


def test_mask_fp32_tiny():
    c = CONFIGS["tiny_fp32_N512"]
    _say(f"mask fp32 {c['name']} ans 0.34")
    inp = generate_config("tiny_fp32_N512")
    _parity(inp, "fp32", c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["alpha_s"],
            c["alpha_f"], 0.34, (FP32_MAX_ABS, FP32_MEAN_ABS))


def test_mask_every_block_exact_is_the_exact_path():
    # alpha_ns = 1: a flat row attends to every token of K_new, as a sharp row does
    _say("mask bf16 ans 1.0 vs exact path, B1 H2 N1024 seed 66")
    inp = generate(1, 2, 512, 512, 128, 64, seed=66, variant="icl")
    plan, o, aux, _ = _parity(inp, "bf16", 1, 2, 512, 512, 128, 0.5, 0.5, 1.0,
                              (BF16_MAX_ABS, BF16_MEAN_ABS))
    assert (aux["ns"] == np.arange(plan.info["n_kv_blocks"])).all()
    # the same rows through the exact path (alpha_f = 0): close to bf16 resolution
    _, o_exact, _, _ = _run(inp, "bf16", 1, 2, 512, 512, 128, 0.5, 0.0, 0.0)
    rows = np.concatenate([np.arange(64 * i, 64 * i + 64) for i in aux["flat"][0, 0]])
    check_close(out_f64(o)[0, 0, rows], out_f64(o_exact)[0, 0, rows], 8e-3, 5e-4, "vs exact path")


def test_mask_changes_only_flat_rows_and_is_deterministic():
    _say("mask bf16 determinism and sharp rows, B1 H4 N2048 seed 67")
    inp = generate(1, 4, 1024, 1024, 128, 64, seed=67, variant="icl")
    _, o0, l0, a0 = _run(inp, "bf16", 1, 4, 1024, 1024, 128, 0.25, 0.5, 0.0)
    _, o1, l1, a1 = _run(inp, "bf16", 1, 4, 1024, 1024, 128, 0.25, 0.5, 0.125)
    _, o2, l2, a2 = _run(inp, "bf16", 1, 4, 1024, 1024, 128, 0.25, 0.5, 0.125)
    assert torch.equal(o1, o2) and np.array_equal(l1, l2)
    for key in a1:
        np.testing.assert_array_equal(a1[key], a2[key])
    for h in range(4):
        sharp = np.concatenate([np.arange(64 * i, 64 * i + 64) for i in a1["sharp"][0, h]])
        assert torch.equal(o0[0, h, sharp], o1[0, h, sharp])


def test_mask_workload_n32768_pages_default():
    # the pages' default no-sparsity ratio at the 32K workload: every decision
    # of every head, sampled output rows of four heads
    c = CONFIGS["isa_bf16_N32768"]
    a_ns = 0.0625
    B, H, L_src, L_ctx, D = c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"]
    _say(f"mask workload {c['name']} ans {a_ns} seed {c['seed']}")
    inp = generate_config("isa_bf16_N32768")
    plan, o, lse, aux = _run(inp, "bf16", B, H, L_src, L_ctx, D, c["alpha_s"], c["alpha_f"], a_ns)
    assert plan.info["n_ns"] == 20
    ex = _check_all_decisions(inp, "bf16", plan, aux, L_src, L_ctx, c["alpha_s"], c["alpha_f"])
    rng = np.random.default_rng(c["seed"] + 7)
    N = L_src + L_ctx
    rows = np.unique(np.concatenate([np.sort(rng.choice(N, 320, replace=False)), [0, N - 1]]))
    heads = sorted(rng.choice(H, 4, replace=False).tolist())
    O_gpu = out_f64(o)
    for h in heads:
        sl = (slice(0, 1), slice(h, h + 1))
        O_ref, L_ref = orc.isa_ref_fixed(*(to_f64(inp[x][sl], "bf16") for x in ("q", "k", "v")),
                                         L_src, L_ctx, 64, aux["sel"][sl], aux["flat"][sl],
                                         rows=rows, ns=aux["ns"][sl])
        check_close(O_gpu[0, h, rows], O_ref[0, 0], BF16_MAX_ABS, BF16_MEAN_ABS, f"O head {h}")
        check_close(lse[0, h, rows], L_ref[0, 0], 5e-3, 1e-3, f"LSE head {h}")
    assert torch.isfinite(o.float()).all()
    check_in_value_range(o, to_gpu(inp["v"], "bf16"))
    _say(f"ok exemptions sel/route/mask {ex}")
