"""GPU checks of the global-memory table paths of the block-mask (flat) and
Taylor kernels, through the C ABI.

Both kernels copy their block and row tables into LDS when the tables are
short enough (every shape a parity test can afford) and read them from global
memory otherwise.  isa_debug_set_flags(ISA_DEBUG_GLOBAL_TABLES) forces the
global path: the tables hold the same indices either way, so the outputs and
the LSE must equal those of the default path bit for bit; one case is also
checked against the fp64 oracle.  Partial blocks (segment tails) are included
because the exact tiles of the block mask read their valid-token count from the
block grid on both paths.  Every case prints its name, shape and seed (flushed)
before touching the GPU.
"""

import sys

import pytest
import torch

import sparse_attention_context_block_amd as isa
from synth import generate
from tests.parity import to_gpu
from tests.test_isa_ns_gpu import _parity
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
