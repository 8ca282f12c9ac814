"""GPU checks of the exact-path kernel's softmax reference.

The kernel exponentiates each key tile against a running reference (the row
maxima of the first tile) instead of the tile's own maxima, and checks the
row sums of a tile before any product reads its exponentials: a sum above
2^8 raises the reference (O and l are rescaled by a power of two), one above
2^64 marks the workgroup for a second launch that recomputes it from the
exact row maxima over every tile.  These inputs
make a late key block score far above the first tile, so that both rare paths
run, and compare the result with the fp64 oracle:
  scale 10:  the block's scores exceed the first tile's by about 30 log2 units
             (row sums near 2^30: a rebase);
  scale 60:  by well over 128 log2 units (the exponentials overflow: the
             fix-up launch).
The same inputs go through the dense call (identity key table, whole tiles),
through ISA with every block kept and exact on partial blocks (the kernel's
partial-tile variant) and at b = 128 (two tiles per block).
"""

import sys

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import generate, round_to_bf16_bits, to_f64
from tests.parity import BF16_MAX_ABS, BF16_MEAN_ABS, check_close, out_f64, to_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(L_src, L_ctx, b, seed, scale, rows):
    """ICL-structured bf16 inputs with K rows ``rows`` multiplied by ``scale``
    (then rounded to bf16 again)."""
    inp = generate(1, 2, L_src, L_ctx, 128, b, seed=seed, variant="icl")
    k = to_f64(inp["k"], "bf16")
    k[:, :, rows] *= scale
    inp["k"] = round_to_bf16_bits(k.astype(np.float32))
    return inp


def _check(o, lse, inp, what):
    O_ref, L_ref = orc.dense_ref(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v")))
    got = out_f64(o)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - O_ref)
    _say(f"{what}: O max-abs {err.max():.3e} mean-abs {err.mean():.3e}, max |O| {np.abs(O_ref).max():.2f}")
    check_close(got, O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, f"{what} O")
    check_close(lse.cpu().numpy(), L_ref, 5e-3, 1e-3, f"{what} LSE")


@pytest.mark.parametrize("scale", [1.0, 10.0, 60.0])
def test_dense_late_block_scores_far_above_the_first_tile(scale):
    _say(f"exact reference: dense B1 H2 N2048 D128, K block 20 x{scale}, seed 501")
    inp = _inputs(1024, 1024, 64, 501, scale, slice(1280, 1344))
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o, lse = isa.isa_dense_forward(q, k, v)
    torch.cuda.synchronize()
    _check(o, lse, inp, f"dense x{scale}")


@pytest.mark.parametrize("scale", [10.0, 60.0])
def test_isa_partial_tiles_late_block_scores_far_above_the_first_tile(scale):
    # every block kept and exact: ISA equals dense attention; the segments end
    # in partial blocks, so the partial-tile variant runs
    _say(f"exact reference: ISA all exact, L_src 1000 L_ctx 1100, K rows 1500-1563 x{scale}, "
         "seed 502")
    inp = _inputs(1000, 1100, 64, 502, scale, slice(1500, 1564))
    plan = isa.isa_plan_create(1, 2, 1000, 1100, 128, 64, 1.0, 0.0)
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o, lse, _ = isa.isa_forward(plan, q, k, v)
    torch.cuda.synchronize()
    _check(o, lse, inp, f"ISA partial x{scale}")


@pytest.mark.parametrize("scale", [10.0, 60.0])
def test_isa_b128_late_block_scores_far_above_the_first_tile(scale):
    _say(f"exact reference: ISA all exact, b 128, N2048, K rows 1536-1663 x{scale}, seed 503")
    inp = _inputs(1024, 1024, 128, 503, scale, slice(1536, 1664))
    plan = isa.isa_plan_create(1, 2, 1024, 1024, 128, 128, 1.0, 0.0)
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o, lse, _ = isa.isa_forward(plan, q, k, v)
    torch.cuda.synchronize()
    _check(o, lse, inp, f"ISA b128 x{scale}")


def test_first_tile_holds_the_largest_scores():
    # the opposite extreme: the first tile dominates and every later tile's
    # exponentials are tiny against its reference
    _say("exact reference: dense N2048, K block 0 x10, seed 504")
    inp = _inputs(1024, 1024, 64, 504, 10.0, slice(0, 64))
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o, lse = isa.isa_dense_forward(q, k, v)
    torch.cuda.synchronize()
    _check(o, lse, inp, "dense first x10")
