"""GPU parity of block lengths other than 64 (b = 32 and b = 128) against the
fp64 oracle, through the C ABI.

The pages leave b open ([notes] key design 1 counts ceil(L_ctx / b) context
blocks).  The attention kernels read every block list in 32-row slices, so a
64-row tile is two 32-token blocks (b = 32) or half of a 128-token block;
partial blocks leave slices partly or wholly empty, which the kernels mask.
Cases cover aligned and partial segments (tails below and above 32 and 64
tokens, a wholly empty key tile), odd block counts, fp32, the rotary
embedding, and a workload-scale case.  Every case prints its name, shape and
seed (flushed) before touching the GPU.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import generate, to_f64
from tests.parity import (BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS, FP32_MEAN_ABS, check_close,
                          check_in_value_range, check_routing, check_selection, out_f64, to_gpu)

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _parity(inp, dtype, B, H, L_src, L_ctx, D, b, a_s, a_f, rope_base=0.0, rows=None,
            heads=None):
    plan = isa.isa_plan_create(B, H, L_src, L_ctx, D, b, a_s, a_f, dtype=TORCH_DT[dtype],
                               rope_base=rope_base)
    info = plan.info
    q, k, v = (to_gpu(inp[x], dtype) for x in ("q", "k", "v"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    torch.cuda.synchronize()
    lse = lse.cpu().numpy()
    aux = {key: t.cpu().numpy() for key, t in aux.items()}
    Q, K, V = (to_f64(inp[x], dtype) for x in ("q", "k", "v"))
    if rope_base > 0:
        Q = orc.decoupled_rope(Q, L_src, rope_base, dtype)
        K = orc.decoupled_rope(K, L_src, rope_base, dtype)
    ex = [0, 0]
    for bi in range(B):
        for h in range(H):
            d = orc.decisions_ref(Q[bi:bi + 1, h:h + 1], K[bi:bi + 1, h:h + 1], L_src, L_ctx, b,
                                  a_s, a_f)
            ex[0] += check_selection(aux["sel"][bi, h], d["c"][0, 0], info["k"])
            ex[1] += check_routing(aux["flat"][bi, h], aux["sharp"][bi, h], d["M"][0, 0],
                                   info["n_flat"])
    bars = (BF16_MAX_ABS, BF16_MEAN_ABS) if dtype == "bf16" else (FP32_MAX_ABS, FP32_MEAN_ABS)
    heads = [(bi, h) for bi in range(B) for h in range(H)] if heads is None else heads
    O_gpu = out_f64(o)
    for bi, h in heads:
        sl = (slice(bi, bi + 1), slice(h, h + 1))
        O_ref, L_ref = orc.isa_ref_fixed(Q[sl], K[sl], V[sl], L_src, L_ctx, b, aux["sel"][sl],
                                         aux["flat"][sl], rows=rows)
        got = O_gpu[bi, h] if rows is None else O_gpu[bi, h, rows]
        got_l = lse[bi, h] if rows is None else lse[bi, h, rows]
        mx, mn = check_close(got, O_ref[0, 0], *bars, what=f"O head ({bi},{h})")
        check_close(got_l, L_ref[0, 0], 5e-3 if dtype == "bf16" else 1e-5,
                    1e-3 if dtype == "bf16" else 1e-6, what=f"LSE head ({bi},{h})")
    assert torch.isfinite(o.float()).all()
    check_in_value_range(o, to_gpu(inp["v"], dtype))
    _say(f"ok max-abs {mx:.2e} mean-abs {mn:.2e} exemptions {ex}")


@pytest.mark.parametrize("b,L_src,L_ctx,D,a_s,a_f,seed", [
    (32, 512, 384, 128, 0.5, 0.5, 101),          # aligned, 28 blocks
    (32, 500, 300, 128, 0.5, 0.5, 102),          # tails 20 and 12, odd block counts
    (32, 321, 95, 64, 0.34, 0.3, 103),           # tails 1 and 31, D = 64
    (128, 1024, 768, 128, 0.5, 0.5, 104),        # aligned
    (128, 1000, 700, 128, 0.5, 0.5, 105),        # tails 104 and 60: slices of 8 and 28 rows
    (128, 128 * 3 + 5, 128 * 2 + 33, 128, 1.0, 0.5, 106),  # tails 5 and 33; the context tail
                                                           # kept: a wholly empty key tile
    (128, 640, 0, 128, 0.5, 0.5, 107),           # no context
    (128, 700, 500, 64, 0.5, 0.0, 108),          # every query exact, D = 64
    (32, 400, 400, 128, 1.0, 1.0, 109),          # every query flat, every block kept
])
def test_block_length_bf16_full_parity(b, L_src, L_ctx, D, a_s, a_f, seed):
    _say(f"blocks bf16 b{b} B1 H2 L_src{L_src} L_ctx{L_ctx} D{D} as{a_s} af{a_f} seed{seed}")
    inp = generate(1, 2, L_src, L_ctx, D, b, seed=seed, variant="icl")
    _parity(inp, "bf16", 1, 2, L_src, L_ctx, D, b, a_s, a_f)


@pytest.mark.parametrize("b,seed", [(32, 110), (128, 111)])
def test_block_length_fp32_full_parity(b, seed):
    _say(f"blocks fp32 b{b} B1 H2 L_src300 L_ctx260 D64 seed{seed}")
    inp = generate(1, 2, 300, 260, 64, b, seed=seed, variant="tiny", dtype="fp32")
    _parity(inp, "fp32", 1, 2, 300, 260, 64, b, 0.5, 0.5)


@pytest.mark.parametrize("b,seed", [(32, 112), (128, 113)])
def test_block_length_with_rope(b, seed):
    _say(f"blocks bf16 rope b{b} B1 H2 L_src700 L_ctx500 seed{seed}")
    inp = generate(1, 2, 700, 500, 128, b, seed=seed, variant="icl")
    _parity(inp, "bf16", 1, 2, 700, 500, 128, b, 0.5, 0.5, rope_base=10000.0)


@pytest.mark.parametrize("b", [32, 128])
def test_block_length_workload_scale(b):
    # 4 heads at N = 8192 with partial tails: every decision, sampled rows of two heads
    L_src, L_ctx = 4100, 4000
    N = L_src + L_ctx
    _say(f"blocks workload b{b} B1 H4 L_src{L_src} L_ctx{L_ctx} seed 114")
    inp = generate(1, 4, L_src, L_ctx, 128, b, seed=114, variant="icl")
    rng = np.random.default_rng(114)
    rows = np.unique(np.concatenate([rng.choice(N, 300, replace=False),
                                     np.arange(L_src - 70, L_src + 70), np.arange(N - 70, N)]))
    _parity(inp, "bf16", 1, 4, L_src, L_ctx, 128, b, 0.25, 0.5, rows=rows,
            heads=[(0, 0), (0, 3)])
