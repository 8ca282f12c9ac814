"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Every case prints its name, shape and seed (flushed) before touching the GPU.
Small cases compare every output element; the full-size workloads compare
every decision of every head and sampled output rows (the oracle computes
each row exactly as in a full evaluation).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import CONFIGS, generate, generate_config, to_f64
from tests.parity import (BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS, FP32_MEAN_ABS, check_close,
                          check_in_value_range,
                          check_routing, check_selection, fixed_ref_rows, from_gpu, out_f64,
                          per_head_decisions, to_gpu)

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run_isa(inp, dtype, B, H, L_src, L_ctx, D, alpha_s, alpha_f, block=64):
    plan = isa.isa_plan_create(B, H, L_src, L_ctx, D, block, alpha_s, alpha_f,
                               dtype=TORCH_DT[dtype])
    q, k, v = (to_gpu(inp[x], dtype) for x in ("q", "k", "v"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    torch.cuda.synchronize()
    aux = {key: t.cpu().numpy() for key, t in aux.items()}
    return plan, o, lse.cpu().numpy(), aux


def _check_decisions(aux, ref, info):
    B, H = aux["sel"].shape[:2]
    ex_sel = ex_route = 0
    for bi in range(B):
        for h in range(H):
            ex_sel += check_selection(aux["sel"][bi, h], ref["c"][bi, h], info["k"])
            ex_route += check_routing(aux["flat"][bi, h], aux["sharp"][bi, h], ref["M"][bi, h],
                                      info["n_flat"])
    # the coarse statistics themselves (fp64 on the GPU)
    if ref["c"].size:
        np.testing.assert_allclose(aux["ctx_score"], ref["c"], rtol=1e-9, atol=0)
    np.testing.assert_allclose(aux["sharpness"], ref["M"], rtol=1e-7, atol=1e-30)
    return ex_sel, ex_route


def _full_parity(inp, dtype, B, H, L_src, L_ctx, D, alpha_s, alpha_f, bars):
    plan, o, lse, aux = _run_isa(inp, dtype, B, H, L_src, L_ctx, D, alpha_s, alpha_f)
    ref = per_head_decisions(inp["q"], inp["k"], dtype, L_src, L_ctx, 64, alpha_s, alpha_f)
    ex = _check_decisions(aux, ref, plan.info)
    O_ref, L_ref = orc.isa_ref_fixed(to_f64(inp["q"], dtype), to_f64(inp["k"], dtype),
                                     to_f64(inp["v"], dtype), L_src, L_ctx, 64,
                                     aux["sel"], aux["flat"])
    mx, mn = check_close(out_f64(o), O_ref, *bars, what="O")
    check_close(lse, L_ref, 5e-3 if dtype == "bf16" else 1e-5, 1e-3 if dtype == "bf16" else 1e-6,
                what="LSE")
    _say(f"ok max-abs {mx:.2e} mean-abs {mn:.2e} exemptions sel/route {ex}")
    return o, aux, O_ref


# --------------------------------------------------------------- dense -----
@pytest.mark.parametrize("D", [128, 64])
def test_dense_bf16_matches_oracle(D):
    _say(f"dense bf16 B1 H2 N640 D{D} seed 7")
    inp = generate(1, 2, 320, 320, D, 64, seed=7, variant="icl")
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o, lse = isa.isa_dense_forward(q, k, v)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.dense_ref(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v")))
    check_close(out_f64(o), O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "dense O")
    # bf16 storage of O dominates the error: it must stay near bf16 resolution
    rel = np.linalg.norm(out_f64(o) - O_ref) / np.linalg.norm(O_ref)
    assert rel < 5e-3, rel
    check_close(lse.cpu().numpy(), L_ref, 5e-3, 1e-3, "dense LSE")


def test_dense_fp32_matches_oracle():
    _say("dense fp32 B1 H2 N512 D64 seed 8")
    inp = generate(1, 2, 256, 256, 64, 64, seed=8, variant="tiny", dtype="fp32")
    q, k, v = (to_gpu(inp[x], "fp32") for x in ("q", "k", "v"))
    o, lse = isa.isa_dense_forward(q, k, v)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.dense_ref(inp["q"], inp["k"], inp["v"])
    check_close(o.cpu().numpy(), O_ref, FP32_MAX_ABS, FP32_MEAN_ABS, "dense fp32 O")
    check_close(lse.cpu().numpy(), L_ref, 1e-5, 1e-6, "dense fp32 LSE")


def test_dense_bf16_long_keys():
    _say("dense bf16 B1 H1 N4096 D128 seed 9")
    inp = generate(1, 1, 2048, 2048, 128, 64, seed=9, variant="icl")
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o, _ = isa.isa_dense_forward(q, k, v)
    torch.cuda.synchronize()
    rows = np.arange(0, 4096, 37)
    O_ref, _ = orc.dense_ref(*(to_f64(inp[x], "bf16") for x in ("q", "k", "v")), rows=rows)
    check_close(out_f64(o)[:, :, rows], O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "dense O")


# --------------------------------------------------------- ISA, small ------
def test_isa_tiny_fp32_config():
    c = CONFIGS["tiny_fp32_N512"]
    _say(f"ISA tiny fp32 {c}")
    inp = generate_config("tiny_fp32_N512")
    _full_parity(inp, "fp32", c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["alpha_s"],
                 c["alpha_f"], (FP32_MAX_ABS, FP32_MEAN_ABS))


@pytest.mark.parametrize("B,H,L_src,L_ctx,D,alpha_s,alpha_f,seed", [
    (1, 3, 640, 448, 128, 0.25, 0.5, 11),   # 17 blocks: odd sharp count, 12-row Taylor tile
    (2, 2, 1024, 1024, 64, 0.5, 0.25, 12),  # D = 64, B = 2
    (1, 2, 2048, 1536, 128, 0.34, 0.7, 13), # uneven ratios
])
def test_isa_bf16_small_full_parity(B, H, L_src, L_ctx, D, alpha_s, alpha_f, seed):
    _say(f"ISA bf16 B{B} H{H} L_src{L_src} L_ctx{L_ctx} D{D} as{alpha_s} af{alpha_f} seed{seed}")
    inp = generate(B, H, L_src, L_ctx, D, 64, seed=seed, variant="icl")
    _full_parity(inp, "bf16", B, H, L_src, L_ctx, D, alpha_s, alpha_f,
                 (BF16_MAX_ABS, BF16_MEAN_ABS))


@pytest.mark.parametrize("alpha_s,alpha_f,L_ctx", [
    (0.0, 0.5, 512),   # no context kept
    (1.0, 0.5, 512),   # every context block kept
    (0.5, 0.0, 512),   # every query exact
    (0.5, 1.0, 512),   # every query on the Taylor path
    (0.5, 0.5, 0),     # no context at all
])
def test_isa_bf16_degenerate_ratios(alpha_s, alpha_f, L_ctx):
    _say(f"ISA bf16 degenerate as{alpha_s} af{alpha_f} L_ctx{L_ctx} seed 14")
    inp = generate(1, 2, 512, L_ctx, 128, 64, seed=14, variant="icl")
    _full_parity(inp, "bf16", 1, 2, 512, L_ctx, 128, alpha_s, alpha_f,
                 (BF16_MAX_ABS, BF16_MEAN_ABS))


def test_isa_all_kept_all_exact_equals_dense_kernel():
    _say("ISA bf16 as1 af0 vs dense kernel, seed 15")
    inp = generate(1, 2, 512, 512, 128, 64, seed=15, variant="icl")
    plan, o, lse, aux = _run_isa(inp, "bf16", 1, 2, 512, 512, 128, 1.0, 0.0)
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    od, lsed = isa.isa_dense_forward(q, k, v)
    torch.cuda.synchronize()
    # same keys in the same order through the same kernel: identical bits
    assert torch.equal(o, od)
    np.testing.assert_array_equal(lse, lsed.cpu().numpy())


def test_isa_deterministic_bitwise():
    _say("ISA bf16 determinism B1 H4 N2048 seed 16")
    inp = generate(1, 4, 1024, 1024, 128, 64, seed=16, variant="icl")
    _, o1, l1, a1 = _run_isa(inp, "bf16", 1, 4, 1024, 1024, 128, 0.25, 0.5)
    _, o2, l2, a2 = _run_isa(inp, "bf16", 1, 4, 1024, 1024, 128, 0.25, 0.5)
    assert torch.equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    for key in a1:
        np.testing.assert_array_equal(a1[key], a2[key])


def test_gather_is_byte_exact():
    _say("gather bf16 B1 H3 L_src640 L_ctx1024 seed 17")
    inp = generate(1, 3, 640, 1024, 128, 64, seed=17, variant="icl")
    plan, _, _, aux = _run_isa(inp, "bf16", 1, 3, 640, 1024, 128, 0.4, 0.5)
    k, v = to_gpu(inp["k"], "bf16"), to_gpu(inp["v"], "bf16")
    k_new, v_new = isa.isa_gather(plan, k, v, torch.from_numpy(aux["sel"]).cuda())
    torch.cuda.synchronize()
    starts, ends, n_src, _ = orc.block_grid(640, 1024, 64)
    for h in range(3):
        for src, got in ((inp["k"], k_new), (inp["v"], v_new)):
            want = orc.gather_concat(src[0, h], starts, ends, n_src, aux["sel"][0, h])
            np.testing.assert_array_equal(from_gpu(got)[0, h], want)


def test_tolerance_rejects_wrong_answers():
    # negative controls: the bars must reject O = 0, O = dense attention, and
    # the output with flat and sharp routing swapped
    _say("negative controls bf16 B1 H2 N8192-like seed 18")
    L = 2048
    inp = generate(1, 2, L, L, 128, 64, seed=18, variant="icl")
    plan, o, _, aux = _run_isa(inp, "bf16", 1, 2, L, L, 128, 0.25, 0.5)
    q64, k64, v64 = (to_f64(inp[x], "bf16") for x in ("q", "k", "v"))
    O_ref, _ = orc.isa_ref_fixed(q64, k64, v64, L, L, 64, aux["sel"], aux["flat"])
    check_close(out_f64(o), O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "ISA O")
    O_dense, _ = orc.dense_ref(q64, k64, v64)
    O_swap, _ = orc.isa_ref_fixed(q64, k64, v64, L, L, 64, aux["sel"], aux["sharp"])
    for name, wrong in (("zero", np.zeros_like(O_ref)), ("dense", O_dense), ("swapped", O_swap)):
        with pytest.raises(AssertionError):
            check_close(wrong, O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, name)


# ------------------------------------------------- full-size workloads -----
def _sample_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(N, size=n, replace=False))
    return np.unique(np.concatenate([rows, [0, N - 1]]))


def _workload_parity(name, alpha_s=None, alpha_f=None, heads_out=4, rows_out=384, inp=None):
    c = dict(CONFIGS[name])
    if alpha_s is not None:
        c["alpha_s"], c["alpha_f"] = alpha_s, alpha_f
    B, H, L_src, L_ctx, D = c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"]
    _say(f"workload {c['name']} B{B} H{H} N{L_src + L_ctx} as{c['alpha_s']} af{c['alpha_f']} "
         f"seed {c['seed']}")
    if inp is None:
        inp = generate_config(name)
    plan, o, lse, aux = _run_isa(inp, "bf16", B, H, L_src, L_ctx, D, c["alpha_s"], c["alpha_f"])
    ref = per_head_decisions(inp["q"], inp["k"], "bf16", L_src, L_ctx, 64, c["alpha_s"],
                             c["alpha_f"])
    ex = _check_decisions(aux, ref, plan.info)
    N = L_src + L_ctx
    rows = _sample_rows(N, rows_out, c["seed"])
    rng = np.random.default_rng(c["seed"] + 1)
    all_heads = [(bi, h) for bi in range(B) for h in range(H)]
    heads = [all_heads[i] for i in sorted(rng.choice(len(all_heads), heads_out, replace=False))]
    O_ref, L_ref = fixed_ref_rows(inp["q"], inp["k"], inp["v"], "bf16", L_src, L_ctx, 64,
                                  aux["sel"], aux["flat"], rows, heads)
    O_gpu = out_f64(o)
    got = np.stack([O_gpu[bi, h, rows] for bi, h in heads])
    got_l = np.stack([lse[bi, h, rows] for bi, h in heads])
    mx, mn = check_close(got, O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "O (sampled rows)")
    check_close(got_l, L_ref, 5e-3, 1e-3, "LSE (sampled rows)")
    # properties that hold at every row: finite, and each row a convex
    # combination of value rows
    assert torch.isfinite(o.float()).all()
    check_in_value_range(o, to_gpu(inp["v"], "bf16"))
    _say(f"ok max-abs {mx:.2e} mean-abs {mn:.2e} exemptions sel/route {ex}")
    return inp


def test_workload_n8192_bf16():
    _workload_parity("isa_bf16_N8192", heads_out=8, rows_out=512)


def test_workload_n32768_bf16_headline():
    _workload_parity("isa_bf16_N32768", heads_out=4, rows_out=384)


_N51200_INPUT = {}


def _n51200_input():
    # one draw of the N=51200 workload serves all nine ratio pairs
    if "inp" not in _N51200_INPUT:
        _N51200_INPUT["inp"] = generate_config("isa_bf16_N51200")
    return _N51200_INPUT["inp"]


# The pages sweep the select ratio and the flat ratio one at a time ([summary] 4
# "Hyperparameters in ISA"; [notes] key findings); this covers the whole grid,
# from the least exact-path work (alpha_s 0.125, alpha_f 0.75) to the most
# (alpha_s 0.5, alpha_f 0.25).
@pytest.mark.parametrize("a_f", CONFIGS["isa_bf16_N51200"]["sweep_alpha_f"])
@pytest.mark.parametrize("a_s", CONFIGS["isa_bf16_N51200"]["sweep_alpha_s"])
def test_workload_n51200_bf16_sweep(a_s, a_f):
    _workload_parity("isa_bf16_N51200", a_s, a_f, heads_out=2, rows_out=256,
                     inp=_n51200_input())


# The sequence-length sweep's shortest and longest inputs (B=1, H=40, D=128,
# L_src = L_ctx = N/2, ratios of the 32K workload; [notes] research background
# and [summary] 1: 5K-50K tokens, about 64K at 544x960), drawn as the bench's
# sweep draws them.
@pytest.mark.parametrize("N", (5120, 65536))
def test_sweep_length_parity(N):
    B, H, D, b, a_s, a_f = 1, 40, 128, 64, 0.25, 0.5
    seed = 2000 + N // 1024
    _say(f"sweep length N{N} B{B} H{H} D{D} as{a_s} af{a_f} seed {seed}")
    inp = generate(B, H, N // 2, N // 2, D, b, seed=seed, variant="icl")
    plan, o, lse, aux = _run_isa(inp, "bf16", B, H, N // 2, N // 2, D, a_s, a_f)
    ref = per_head_decisions(inp["q"], inp["k"], "bf16", N // 2, N // 2, b, a_s, a_f)
    ex = _check_decisions(aux, ref, plan.info)
    rows = _sample_rows(N, 256, seed)
    rng = np.random.default_rng(seed + 1)
    heads = [(0, int(h)) for h in sorted(rng.choice(H, 3, replace=False))]
    O_ref, L_ref = fixed_ref_rows(inp["q"], inp["k"], inp["v"], "bf16", N // 2, N // 2, b,
                                  aux["sel"], aux["flat"], rows, heads)
    O_gpu = out_f64(o)
    got = np.stack([O_gpu[bi, h, rows] for bi, h in heads])
    got_l = np.stack([lse[bi, h, rows] for bi, h in heads])
    mx, mn = check_close(got, O_ref, BF16_MAX_ABS, BF16_MEAN_ABS, "O (sampled rows)")
    check_close(got_l, L_ref, 5e-3, 1e-3, "LSE (sampled rows)")
    assert torch.isfinite(o.float()).all()
    check_in_value_range(o, to_gpu(inp["v"], "bf16"))
    _say(f"ok max-abs {mx:.2e} mean-abs {mn:.2e} exemptions sel/route {ex}")


def test_workload_b2_n16384_forward():
    _workload_parity("isa_fwd_bwd_bf16_B2_N16384", heads_out=4, rows_out=384)
