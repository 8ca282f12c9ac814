"""GPU checks of the kernel paths that only the diagnostic switches of
isa_debug_set_flags reach, through the C ABI.

Global-memory table paths of the block-mask (flat) and Taylor kernels:
Both kernels copy their block and row tables into LDS when the tables are
short enough (every shape a parity test can afford) and read them from global
memory otherwise.  isa_debug_set_flags(ISA_DEBUG_GLOBAL_TABLES) forces the
global path: the tables hold the same indices either way, so the outputs and
the LSE must equal those of the default path bit for bit; one case is also
checked against the fp64 oracle.  Partial blocks (segment tails) are included
because the exact tiles of the block mask read their valid-token count from the
block grid on both paths.

The 4-wave kernel on block tables (ISA_DEBUG_4WAVE_EXACT): by default the
exact path and the dense baseline run on the one-wave-per-SIMD kernel (the
ping-pong kernel at b = 32) and the 4-wave kernel reads only pooled rows
through a row table; with the switch it reads whole blocks through the block
table instead.  Those cases are checked against the fp64 oracle, at every
block length and with partial blocks; so is the ping-pong kernel
(ISA_DEBUG_PINGPONG_EXACT) beside the default one.

Every case prints its name, shape and seed (flushed) before touching the GPU.
"""

import sys

import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import generate, to_f64
from tests.parity import check_close, out_f64, to_gpu
from tests.test_isa_ns_gpu import _parity
from tests.test_isa_blocks_gpu import _parity as _block_parity
from tests.parity import BF16_MAX_ABS, BF16_MEAN_ABS

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _forward(inp, L_src, L_ctx, D, a_s, a_f, a_ns):
    plan = isa.isa_plan_create(1, 2, L_src, L_ctx, D, 64, a_s, a_f, a_ns, dtype=torch.bfloat16)
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    torch.cuda.synchronize()
    return o, lse, aux


@pytest.mark.parametrize("L_src,L_ctx,D,a_s,a_f,a_ns,seed", [
    (1000, 700, 128, 0.5, 0.5, 0.25, 301),   # block mask, tails 40 and 60
    (640, 640, 128, 0.5, 0.5, 0.0625, 302),  # block mask, whole blocks
    (700, 500, 64, 0.5, 0.5, 0.0, 303),      # Taylor path, D = 64, tails
    (1024, 1024, 128, 0.25, 0.75, 0.0, 304), # Taylor path, most blocks flat
])
def test_global_tables_equal_lds_tables(L_src, L_ctx, D, a_s, a_f, a_ns, seed):
    _say(f"table paths B1 H2 L_src{L_src} L_ctx{L_ctx} D{D} as{a_s} af{a_f} ans{a_ns} seed{seed}")
    inp = generate(1, 2, L_src, L_ctx, D, 64, seed=seed, variant="icl")
    o1, l1, a1 = _forward(inp, L_src, L_ctx, D, a_s, a_f, a_ns)
    isa.isa_debug_set_flags(isa.ISA_DEBUG_GLOBAL_TABLES)
    try:
        o2, l2, a2 = _forward(inp, L_src, L_ctx, D, a_s, a_f, a_ns)
    finally:
        isa.isa_debug_set_flags(0)
    for key in a1:
        assert torch.equal(a1[key], a2[key]), key
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)
    _say("ok bit-identical")


def test_global_tables_block_mask_oracle_parity():
    L_src, L_ctx = 1000, 700
    _say(f"table paths oracle B1 H2 L_src{L_src} L_ctx{L_ctx} ans0.25 seed 305")
    inp = generate(1, 2, L_src, L_ctx, 128, 64, seed=305, variant="icl")
    isa.isa_debug_set_flags(isa.ISA_DEBUG_GLOBAL_TABLES)
    try:
        _parity(inp, "bf16", 1, 2, L_src, L_ctx, 128, 0.5, 0.5, 0.25,
                (BF16_MAX_ABS, BF16_MEAN_ABS))
    finally:
        isa.isa_debug_set_flags(0)


@pytest.mark.parametrize("b,L_src,L_ctx,D,a_s,a_f,seed", [
    (64, 1024, 1024, 128, 0.25, 0.5, 311),   # aligned
    (64, 1000, 700, 64, 0.5, 0.25, 312),     # tails 40 and 60, D = 64
    (32, 500, 300, 128, 0.5, 0.5, 313),      # tails 20 and 12
    (128, 1000, 700, 128, 0.5, 0.0, 314),    # tails 104 and 60, every query exact
])
def test_4wave_exact_path_matches_oracle(b, L_src, L_ctx, D, a_s, a_f, seed):
    _say(f"4-wave exact B1 H2 L_src{L_src} L_ctx{L_ctx} D{D} b{b} as{a_s} af{a_f} seed{seed}")
    inp = generate(1, 2, L_src, L_ctx, D, b, seed=seed, variant="icl")
    isa.isa_debug_set_flags(isa.ISA_DEBUG_4WAVE_EXACT)
    try:
        _block_parity(inp, "bf16", 1, 2, L_src, L_ctx, D, b, a_s, a_f)
    finally:
        isa.isa_debug_set_flags(0)


@pytest.mark.parametrize("D", [128, 64])
def test_4wave_dense_matches_oracle(D):
    N, seed = 1536, 315 + D
    _say(f"4-wave dense bf16 B1 H2 N{N} D{D} seed{seed}")
    inp = generate(1, 2, N // 2, N // 2, D, 64, seed=seed, variant="plain")
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    od, ld = isa.isa_dense_forward(q, k, v)
    isa.isa_debug_set_flags(isa.ISA_DEBUG_4WAVE_EXACT)
    try:
        o4, l4 = isa.isa_dense_forward(q, k, v)
    finally:
        isa.isa_debug_set_flags(0)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.dense_ref(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v")))
    mx, mn = check_close(out_f64(o4), O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "O (4-wave)")
    check_close(l4.cpu().numpy(), L_ref, 5e-3, 1e-3, "LSE (4-wave)")
    # the default kernel (one wave per SIMD) on the same input, also against the
    # oracle: the two take their exponentials against different references
    # (the running row max, the first tile's row max), so their bits differ
    check_close(out_f64(od), O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "O (default)")
    check_close(ld.cpu().numpy(), L_ref, 5e-3, 1e-3, "LSE (default)")
    _say(f"ok max-abs {mx:.2e} mean-abs {mn:.2e}")


# The one-wave-per-SIMD kernel (the default for block tables at D = 128 with
# 64- and 128-token blocks) and the 8-wave ping-pong kernel
# (ISA_DEBUG_PINGPONG_EXACT) on the same keys in the same tile order, each
# against the oracle.  (The ping-pong kernel takes each tile's exponentials
# against the running row max; the one-wave kernel against the first tile's
# row max, raised only when a tile's row sum exceeds 2^8: their bits differ.)
# The cases cover one to twenty-one key tiles (the three-tile prefetch ring and
# the tiles past the end), odd and even tile counts (the loop body runs two
# tiles per trip), both block lengths, and partial and empty half tiles.
@pytest.mark.parametrize("b,L_src,L_ctx,a_s,a_f,seed", [
    (64, 1024, 1024, 0.25, 0.5, 321),    # aligned, 20 key tiles
    (64, 1088, 960, 0.25, 0.5, 322),     # aligned, 21 key tiles (odd)
    (128, 1024, 1024, 0.5, 0.25, 323),   # 128-token blocks
    (64, 1000, 700, 0.5, 0.5, 324),      # partial tiles (tails 40 and 60)
    (128, 1000, 700, 0.5, 0.0, 325),     # partial and empty half tiles
    (64, 64, 64, 1.0, 0.0, 326),         # two key tiles
    (64, 128, 64, 0.0, 0.0, 327),        # two key tiles, nothing kept
    (64, 64, 0, 0.0, 0.0, 328),          # one key tile
])
def test_w64_and_pingpong_exact_paths_match_oracle(b, L_src, L_ctx, a_s, a_f, seed):
    _say(f"w64 and ping-pong B1 H2 L_src{L_src} L_ctx{L_ctx} D128 b{b} as{a_s} af{a_f} seed{seed}")
    inp = generate(1, 2, L_src, L_ctx, 128, b, seed=seed, variant="icl")
    _block_parity(inp, "bf16", 1, 2, L_src, L_ctx, 128, b, a_s, a_f)
    isa.isa_debug_set_flags(isa.ISA_DEBUG_PINGPONG_EXACT)
    try:
        _block_parity(inp, "bf16", 1, 2, L_src, L_ctx, 128, b, a_s, a_f)
    finally:
        isa.isa_debug_set_flags(0)
    _say("ok both kernels")


@pytest.mark.parametrize("N", [64, 128, 192, 320, 2048])
def test_w64_and_pingpong_dense_match_oracle(N):
    seed = 330 + N // 64
    _say(f"w64 and ping-pong dense bf16 B1 H2 N{N} D128 seed{seed}")
    inp = generate(1, 2, N, 0, 128, 64, seed=seed, variant="plain")
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o1, l1 = isa.isa_dense_forward(q, k, v)
    isa.isa_debug_set_flags(isa.ISA_DEBUG_PINGPONG_EXACT)
    try:
        o2, l2 = isa.isa_dense_forward(q, k, v)
    finally:
        isa.isa_debug_set_flags(0)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.dense_ref(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v")))
    mx, mn = check_close(out_f64(o1), O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "O (w64 dense)")
    check_close(l1.cpu().numpy(), L_ref, 5e-3, 1e-3, "LSE (w64 dense)")
    check_close(out_f64(o2), O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "O (ping-pong dense)")
    check_close(l2.cpu().numpy(), L_ref, 5e-3, 1e-3, "LSE (ping-pong dense)")
    _say(f"ok max-abs {mx:.2e} mean-abs {mn:.2e}")
