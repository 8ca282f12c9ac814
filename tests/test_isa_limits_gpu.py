"""GPU parity at the plan's limits, through the C ABI.

A head of 4096 blocks is the longest a plan accepts (N = 262144 tokens at
b = 64).  These cases run B*H = 5*13 = 65 such heads, so the last head of Q,
K, V and O starts 64 * 2^25 = 2^31 elements (4 GiB of bf16) into its tensor:
every per-head offset beyond 32 bits is exercised.  The heads repeat two drawn heads (head i holds
the inputs of drawn head i mod 2), which keeps the host work to two heads.
Every head must then reproduce its drawn head bit for bit (each step is
deterministic and no step mixes heads), and the two drawn heads are checked
against the oracle: every decision, and sampled output rows.  At this length
the Taylor path's row table (2560 entries) and the block mask's tables exceed
their LDS copies, so those kernels read them from global memory.

The backward at the same shape cannot be compared with the oracle (its dK, dV
need every query row), so besides the head-by-head identity it is checked
against properties that hold at any size: finite gradients, exact zeros on the
context rows of unselected blocks, sum_t dV_t = sum_r dO_r (every exact
row's P and every flat row's pi sum to one, and the Taylor broadcast gives each
token of block j the share dV^c_j / w_j, so each query row passes its dO on
whole) and sum_t dK_t = 0 (each row of dS = P (dP - delta) sums to zero).

Every case prints its name, shape and seed (flushed) before touching the GPU.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import generate, to_f64
from tests.parity import (BF16_MAX_ABS, BF16_MEAN_ABS, check_close, check_in_value_range,
                          check_ns, check_routing, check_selection, out_f64, to_gpu)

pytestmark = pytest.mark.gpu

B, H = 5, 13
L = 131072            # L_src = L_ctx: 2048 + 2048 blocks of 64
D = 128
A_S, A_F = 0.25, 0.5
SEED = 71


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def drawn():
    # the first two heads of the [5, 13] draw, as bf16 bits [1, 2, N, D], with dO
    return generate(B, H, L, L, D, 64, seed=SEED, variant="icl", heads=[0, 1], grad=True)


@pytest.fixture(scope="module")
def tiled(drawn):
    _say(f"limits: tiling 2 drawn heads to B{B} H{H} N{2 * L} D{D} on cuda:0")
    idx = torch.arange(B * H, device="cuda") % 2
    out = {}
    for x in ("q", "k", "v", "do"):
        base = to_gpu(drawn[x], "bf16")[0]                # [2, N, D]
        out[x] = base.index_select(0, idx).reshape(B, H, 2 * L, D)
        del base
    torch.cuda.synchronize()
    yield out
    out.clear()
    torch.cuda.empty_cache()


def _drawn_head(arr, h):
    return to_f64(arr[:, h:h + 1], "bf16")                # [1, 1, N, D]


@pytest.mark.parametrize("a_ns", [0.0, 0.0625])
def test_limit_4096_blocks_65_heads(drawn, tiled, a_ns):
    N = 2 * L
    _say(f"limits bf16 B{B} H{H} N{N} D{D} as{A_S} af{A_F} ans{a_ns} seed {SEED} "
         f"(heads repeat 2 drawn heads)")
    plan = isa.isa_plan_create(B, H, L, L, D, 64, A_S, A_F, a_ns)
    info = plan.info
    assert info["n_q_blocks"] == 4096 and info["n_kv_blocks"] == 2560
    o, lse, aux = isa.isa_forward(plan, tiled["q"], tiled["k"], tiled["v"], aux=True)
    torch.cuda.synchronize()
    _say("limits: forward done; comparing every head with its drawn head")

    # every head equals its drawn head, bit for bit (outputs on the GPU)
    of = o.view(B * H, N, D).view(torch.int16)
    lf = lse.view(B * H, N)
    for i in range(2, B * H):
        assert torch.equal(of[i], of[i % 2]), f"O of head {i} differs from head {i % 2}"
        assert torch.equal(lf[i], lf[i % 2]), f"LSE of head {i} differs from head {i % 2}"
    dec = {key: t.cpu().numpy().reshape((B * H,) + t.shape[2:]) for key, t in aux.items()}
    for key, a in dec.items():
        for i in range(2, B * H):
            np.testing.assert_array_equal(a[i], a[i % 2], err_msg=f"{key} of head {i}")
    if a_ns > 0:
        assert "ns" in dec and dec["ns"].shape[1:] == (info["n_flat"], info["n_ns"])

    # the drawn heads against the oracle
    starts, ends, n_src, _ = orc.block_grid(L, L, 64)
    rng = np.random.default_rng(SEED + 1)
    rows = np.unique(np.concatenate([np.sort(rng.choice(N, 256, replace=False)),
                                     [0, L - 1, L, N - 1]]))
    O_gpu, lse_gpu = out_f64(o[0, :2]), lse[0, :2].cpu().numpy()
    ex = [0, 0, 0]
    for h in range(2):
        q64, k64, v64 = (_drawn_head(drawn[x], h) for x in ("q", "k", "v"))
        d = orc.decisions_ref(q64, k64, L, L, 64, A_S, A_F)
        ex[0] += check_selection(dec["sel"][h], d["c"][0, 0], info["k"])
        ex[1] += check_routing(dec["flat"][h], dec["sharp"][h], d["M"][0, 0], info["n_flat"])
        np.testing.assert_allclose(dec["ctx_score"][h], d["c"][0, 0], rtol=1e-9, atol=0)
        np.testing.assert_allclose(dec["sharpness"][h], d["M"][0, 0], rtol=1e-7, atol=1e-30)
        ns = None
        if a_ns > 0:
            P = orc.coarse_probs(orc.pool_blocks(q64[0, 0], starts, ends),
                                 orc.pool_blocks(k64[0, 0], starts, ends))
            kept = np.concatenate([np.arange(n_src), n_src + dec["sel"][h]])
            for f, i in enumerate(dec["flat"][h]):
                ex[2] += check_ns(dec["ns"][h, f], P[i, kept], info["n_ns"])
            ns = dec["ns"][h][None, None]
        O_ref, L_ref = orc.isa_ref_fixed(q64, k64, v64, L, L, 64, dec["sel"][h][None, None],
                                         dec["flat"][h][None, None], rows=rows, ns=ns)
        check_close(O_gpu[h, rows], O_ref[0, 0], BF16_MAX_ABS, BF16_MEAN_ABS, f"O head {h}")
        check_close(lse_gpu[h, rows], L_ref[0, 0], 5e-3, 1e-3, f"LSE head {h}")
    assert torch.isfinite(o).all()
    check_in_value_range(o, tiled["v"])
    _say(f"ok exemptions sel/route/mask {ex}")


def test_limit_longest_sequence_b128():
    # the longest head a plan accepts: 4096 blocks of 128 tokens, N = 524288
    Lb, b, seed = 262144, 128, 73
    N = 2 * Lb
    _say(f"limits bf16 B1 H1 N{N} D{D} b{b} as{A_S} af{A_F} seed {seed}")
    inp = generate(1, 1, Lb, Lb, D, b, seed=seed, variant="icl")
    plan = isa.isa_plan_create(1, 1, Lb, Lb, D, b, A_S, A_F)
    info = plan.info
    assert info["n_q_blocks"] == 4096
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k", "v"))
    o, lse, aux = isa.isa_forward(plan, q, k, v, aux=True)
    torch.cuda.synchronize()
    _say("limits: forward done; checking against the oracle")
    dec = {key: t.cpu().numpy()[0, 0] for key, t in aux.items()}
    q64, k64, v64 = (to_f64(inp[x], "bf16") for x in ("q", "k", "v"))
    d = orc.decisions_ref(q64, k64, Lb, Lb, b, A_S, A_F)
    ex = (check_selection(dec["sel"], d["c"][0, 0], info["k"]),
          check_routing(dec["flat"], dec["sharp"], d["M"][0, 0], info["n_flat"]))
    rng = np.random.default_rng(seed + 1)
    rows = np.unique(np.concatenate([np.sort(rng.choice(N, 256, replace=False)),
                                     [0, Lb - 1, Lb, N - 1]]))
    O_ref, L_ref = orc.isa_ref_fixed(q64, k64, v64, Lb, Lb, b, dec["sel"][None, None],
                                     dec["flat"][None, None], rows=rows)
    check_close(out_f64(o)[0, 0, rows], O_ref[0, 0], BF16_MAX_ABS, BF16_MEAN_ABS, "O")
    check_close(lse.cpu().numpy()[0, 0, rows], L_ref[0, 0], 5e-3, 1e-3, "LSE")
    assert torch.isfinite(o).all()
    check_in_value_range(o, v)
    _say(f"ok exemptions sel/route {ex}")


def test_limit_backward_65_heads(drawn, tiled):
    N = 2 * L
    _say(f"limits backward bf16 B{B} H{H} N{N} D{D} as{A_S} af{A_F} seed {SEED} "
         f"(heads repeat 2 drawn heads)")
    plan = isa.isa_plan_create(B, H, L, L, D, 64, A_S, A_F)
    o, lse, aux = isa.isa_forward(plan, tiled["q"], tiled["k"], tiled["v"], aux=True)
    grads = isa.isa_backward(plan, tiled["q"], tiled["k"], tiled["v"], o, tiled["do"], lse, aux)
    torch.cuda.synchronize()
    del o, lse
    _say("limits: backward done; comparing every head with its drawn head")
    for name, g in zip(("dQ", "dK", "dV"), grads):
        gf = g.view(B * H, N, D).view(torch.int16)
        for i in range(2, B * H):
            assert torch.equal(gf[i], gf[i % 2]), f"{name} of head {i} differs from head {i % 2}"
        assert torch.isfinite(g).all(), name
    sel = aux["sel"].cpu().numpy().reshape(B * H, -1)
    dk, dv = (out_f64(g[0, :2]) for g in grads[1:])
    n_src, n_ctx = L // 64, L // 64
    for h in range(2):
        # unselected context blocks: exact zeros
        dropped = np.setdiff1d(np.arange(n_ctx), sel[h])
        rows = (L + 64 * dropped[:, None] + np.arange(64)[None, :]).ravel()
        assert not dk[h, rows].any() and not dv[h, rows].any(), f"head {h}: unselected rows"
        # every query row passes its dO on whole: sum_t dV_t = sum_r dO_r, to
        # the rounding of the bf16 P, pi and dV (random signs: compared with
        # the root sum of squares of the terms)
        do = _drawn_head(drawn["do"], h)[0, 0]
        lhs, rhs = dv[h].sum(axis=0), do.sum(axis=0)
        scale = np.sqrt((dv[h] ** 2).sum(axis=0) + (do ** 2).sum(axis=0))
        err = np.abs(lhs - rhs) / scale
        assert err.max() <= 0.05, f"head {h}: sum dV vs sum dO, {err.max():.3e} of the RSS"
        err_k = np.abs(dk[h].sum(axis=0)) / np.sqrt((dk[h] ** 2).sum(axis=0))
        assert err_k.max() <= 0.05, f"head {h}: sum dK, {err_k.max():.3e} of the RSS"
        _say(f"head {h}: {len(dropped)} unselected blocks zero; |sum dV - sum dO| / RSS "
             f"max {err.max():.2e}; |sum dK| / RSS max {err_k.max():.2e}")
