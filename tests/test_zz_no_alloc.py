"""The allocation-free forward (isa_forward_noalloc: the library's static
per-device workspace) against isa_forward (a caller-allocated workspace),
through the C ABI.  Both run the same kernels, so the outputs and every
decision must agree bit for bit.  Two calls in a row, the second smaller, show
that nothing of the first call's workspace contents leaks into the second; a
third call after the first checks that no device memory is taken per call."""

import sys

import pytest
import torch

import sparse_attention_context_block_amd as isa
from synth import generate
from tests.parity import to_gpu

pytestmark = pytest.mark.gpu

FIELDS = ("sel", "flat", "sharp", "ctx_score", "sharpness", "ns")


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _case(B, H, L_src, L_ctx, block, alpha_ns, seed):
    plan = isa.isa_plan_create(B, H, L_src, L_ctx, 128, block, 0.25, 0.5, alpha_ns=alpha_ns)
    assert plan.info["workspace_bytes"] <= isa.ISA_STATIC_WORKSPACE_BYTES
    inp = generate(B, H, L_src, L_ctx, 128, block, seed)
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    return plan, q, k, v


def _reference(plan, q, k, v):
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    torch.cuda.synchronize()
    return o, lse, aux


def _noalloc(plan, q, k, v, ref_aux):
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    aux = {f: torch.full_like(t, -1) for f, t in ref_aux.items()}
    isa.isa_forward_noalloc(plan, q, k, v, o, lse, aux)
    torch.cuda.synchronize()
    return o, lse, aux


def _same(got, ref):
    o, lse, aux = got
    ro, rlse, raux = ref
    assert torch.equal(o, ro)
    assert torch.equal(lse, rlse)
    assert set(aux) == set(raux)
    for f in aux:
        assert torch.equal(aux[f], raux[f]), f


# (first call, second smaller call): plain forward; the block mask (its
# coarse logits and per-block lists are workspace); partial blocks
CASES = [
    ((2, 4, 2048, 2048, 64, 0.0, 11), (1, 2, 512, 768, 64, 0.0, 12)),
    ((1, 4, 2048, 2048, 64, 0.0625, 21), (1, 2, 1024, 1024, 64, 0.125, 22)),
    ((1, 3, 1000, 1500, 64, 0.0, 31), (1, 1, 300, 200, 32, 0.0, 32)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_forward_equals_isa_forward_on_two_calls(first, second):
    for i, cfg in enumerate((first, second)):
        _say(f"isa_forward_noalloc call {i + 1}: B,H,L_src,L_ctx,b,alpha_ns,seed={cfg}")
        plan, q, k, v = _case(*cfg)
        ref = _reference(plan, q, k, v)
        _same(_noalloc(plan, q, k, v, ref[2]), ref)


def test_noalloc_forward_takes_no_device_memory_per_call():
    _say("isa_forward_noalloc: free device memory unchanged across calls")
    plan, q, k, v = _case(1, 4, 2048, 2048, 64, 0.0, 41)
    ref = _reference(plan, q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    isa.isa_forward_noalloc(plan, q, k, v, o, lse)  # resolves the array, loads the kernels
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        isa.isa_forward_noalloc(plan, q, k, v, o, lse)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])


def test_noalloc_forward_rejects_a_plan_beyond_the_array():
    _say("isa_forward_noalloc: plan beyond the static workspace")
    plan = isa.isa_plan_create(1, 40, 16384, 16384, 128, rope_base=10000.0)
    assert plan.info["workspace_bytes"] > isa.ISA_STATIC_WORKSPACE_BYTES
    x = torch.empty((1, 40, 32768, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(isa.IsaError, match="ISA_ERR_WORKSPACE"):
        isa.isa_forward_noalloc(plan, x, x, x, x)
