"""GPU parity of partial blocks against the fp64 oracle, through the C ABI.

The source and the context are each cut into 64-token blocks from their own
start, so with L_src or L_ctx not a multiple of 64 the last block of a segment
is partial ([notes] key design 1 counts ceil(L_ctx / b) context blocks;
reading R2: a partial block weighs its token count).  Every output row is
compared, so a partial query block that wrote past its tail (into the next
segment) would show.  Every case prints its name, shape and seed (flushed)
before touching the GPU.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import generate, to_f64
from tests.parity import (BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS, FP32_MEAN_ABS, check_close,
                          check_in_value_range, check_routing, check_selection, out_f64,
                          per_head_decisions, to_gpu)
from tests.test_isa_ns_gpu import _check_all_decisions

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(inp, dtype, B, H, L_src, L_ctx, D, a_s, a_f, a_ns=0.0):
    plan = isa.isa_plan_create(B, H, L_src, L_ctx, D, 64, a_s, a_f, a_ns, dtype=TORCH_DT[dtype])
    q, k, v = (to_gpu(inp[x], dtype) for x in ("q", "k", "v"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    torch.cuda.synchronize()
    return plan, o, lse.cpu().numpy(), {key: t.cpu().numpy() for key, t in aux.items()}


def _parity(inp, dtype, B, H, L_src, L_ctx, D, a_s, a_f, a_ns=0.0, rows=None, heads=None):
    plan, o, lse, aux = _run(inp, dtype, B, H, L_src, L_ctx, D, a_s, a_f, a_ns)
    info = plan.info
    if a_ns > 0 and info["n_flat"] > 0:
        ex = _check_all_decisions(inp, dtype, plan, aux, L_src, L_ctx, a_s, a_f)
    else:
        ref = per_head_decisions(inp["q"], inp["k"], dtype, L_src, L_ctx, 64, a_s, a_f)
        ex = [0, 0]
        for bi in range(B):
            for h in range(H):
                ex[0] += check_selection(aux["sel"][bi, h], ref["c"][bi, h], info["k"])
                ex[1] += check_routing(aux["flat"][bi, h], aux["sharp"][bi, h], ref["M"][bi, h],
                                       info["n_flat"])
    bars = (BF16_MAX_ABS, BF16_MEAN_ABS) if dtype == "bf16" else (FP32_MAX_ABS, FP32_MEAN_ABS)
    ns = aux.get("ns")
    heads = [(bi, h) for bi in range(B) for h in range(H)] if heads is None else heads
    O_gpu = out_f64(o)
    for bi, h in heads:
        sl = (slice(bi, bi + 1), slice(h, h + 1))
        O_ref, L_ref = orc.isa_ref_fixed(*(to_f64(inp[x][sl], dtype) for x in ("q", "k", "v")),
                                         L_src, L_ctx, 64, aux["sel"][sl], aux["flat"][sl],
                                         rows=rows, ns=None if ns is None else ns[sl])
        got = O_gpu[bi, h] if rows is None else O_gpu[bi, h, rows]
        got_l = lse[bi, h] if rows is None else lse[bi, h, rows]
        mx, mn = check_close(got, O_ref[0, 0], *bars, what=f"O head ({bi},{h})")
        check_close(got_l, L_ref[0, 0], 5e-3 if dtype == "bf16" else 1e-5,
                    1e-3 if dtype == "bf16" else 1e-6, what=f"LSE head ({bi},{h})")
    assert torch.isfinite(o.float()).all()
    check_in_value_range(o, to_gpu(inp["v"], dtype))
    _say(f"ok max-abs {mx:.2e} mean-abs {mn:.2e} exemptions {ex}")
    return plan, o, aux


@pytest.mark.parametrize("B,H,L_src,L_ctx,D,a_s,a_f,seed", [
    (1, 2, 100, 200, 128, 0.5, 0.5, 71),         # tails 36 and 8
    (2, 2, 1000, 1000, 64, 0.34, 0.3, 72),       # tails 40 and 40, D = 64, B = 2
    (1, 3, 300, 130, 128, 1.0, 0.5, 73),         # every context block kept: the tail too
    (1, 2, 64 * 5 + 1, 64 * 3 + 63, 128, 0.5, 0.5, 74),  # tails 1 and 63
    (1, 2, 130, 0, 128, 0.5, 0.5, 75),           # no context, source tail of 2
    (1, 2, 50, 0, 128, 0.5, 1.0, 76),            # a single partial block, flat
    (1, 2, 700, 500, 128, 0.5, 0.0, 77),         # every query exact
    (1, 2, 700, 500, 128, 1.0, 1.0, 78),         # every query flat, every block kept
])
def test_partial_bf16_full_parity(B, H, L_src, L_ctx, D, a_s, a_f, seed):
    _say(f"partial bf16 B{B} H{H} L_src{L_src} L_ctx{L_ctx} D{D} as{a_s} af{a_f} seed{seed}")
    inp = generate(B, H, L_src, L_ctx, D, 64, seed=seed, variant="icl")
    _parity(inp, "bf16", B, H, L_src, L_ctx, D, a_s, a_f)


def test_partial_fp32_full_parity():
    _say("partial fp32 B1 H2 L_src200 L_ctx180 D64 seed 79")
    inp = generate(1, 2, 200, 180, 64, 64, seed=79, variant="tiny", dtype="fp32")
    _parity(inp, "fp32", 1, 2, 200, 180, 64, 0.5, 0.5)


@pytest.mark.parametrize("a_s,a_ns,seed", [(0.5, 0.4, 80), (1.0, 0.3, 81), (1.0, 1.0, 82)])
def test_partial_with_block_mask(a_s, a_ns, seed):
    _say(f"partial bf16 mask L_src500 L_ctx700 as{a_s} ans{a_ns} seed{seed}")
    inp = generate(1, 2, 500, 700, 128, 64, seed=seed, variant="icl")
    _parity(inp, "bf16", 1, 2, 500, 700, 128, a_s, 0.5, a_ns)


def test_partial_fp32_with_block_mask():
    _say("partial fp32 mask L_src200 L_ctx180 D64 ans 0.5 seed 83")
    inp = generate(1, 2, 200, 180, 64, 64, seed=83, variant="tiny", dtype="fp32")
    _parity(inp, "fp32", 1, 2, 200, 180, 64, 1.0, 0.5, 0.5)


def test_partial_workload_scale():
    # 8 heads at the 32K scale with tails of 1 and 60 tokens: every decision of
    # every head; all tail rows and 300 sampled rows of two heads
    L_src, L_ctx = 16001, 16700
    N = L_src + L_ctx
    _say(f"partial workload B1 H8 L_src{L_src} L_ctx{L_ctx} seed 84")
    inp = generate(1, 8, L_src, L_ctx, 128, 64, seed=84, variant="icl")
    rng = np.random.default_rng(84)
    tails = np.concatenate([np.arange(16000 - 64, L_src + 64), np.arange(N - 124, N)])
    rows = np.unique(np.concatenate([rng.choice(N, 300, replace=False), tails]))
    _parity(inp, "bf16", 1, 8, L_src, L_ctx, 128, 0.25, 0.5, rows=rows, heads=[(0, 2), (0, 5)])
