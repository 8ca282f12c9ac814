"""C-ABI host tests (CPU only): the library loads, exports every symbol the
header declares, and plan creation validates and sizes problems without any
HIP call.  No compute entry point is called here."""

import ctypes
import os
import re

import pytest

import oracle as orc
import sparse_attention_context_block_amd as isa
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isa.h")
TESTING_HEADER = os.path.join(ROOT, "include", "isa_testing.h")


def _declared_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(isa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(isa.LIB_PATH)
    declared = _declared_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/isa.h but not exported"
    assert sorted(isa.EXPORTS) == declared
    hooks = _declared_functions(TESTING_HEADER)
    for name in hooks:
        assert hasattr(lib, name), f"{name} declared in include/isa_testing.h but not exported"
    assert sorted(isa.TESTING_EXPORTS) == hooks
    # the product header declares no global switch
    assert not set(hooks) & set(declared)


def test_debug_flags_accept_known_bits_only():
    # host-only setter: no HIP call
    isa.isa_debug_set_flags(isa.ISA_DEBUG_GLOBAL_TABLES)
    isa.isa_debug_set_flags(isa.ISA_DEBUG_4WAVE_EXACT)
    isa.isa_debug_set_flags(isa.ISA_DEBUG_GLOBAL_TABLES | isa.ISA_DEBUG_4WAVE_EXACT)
    isa.isa_debug_set_flags(isa.ISA_DEBUG_GLOBAL_TABLES | isa.ISA_DEBUG_PINGPONG_EXACT)
    isa.isa_debug_set_flags(0)
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        isa.isa_debug_set_flags(8)
    with pytest.raises(RuntimeError, match="INVALID_ARG"):  # two exact-path kernels at once
        isa.isa_debug_set_flags(isa.ISA_DEBUG_4WAVE_EXACT | isa.ISA_DEBUG_PINGPONG_EXACT)
    assert isa._lib().isa_debug_set_flags(0x80000000) == 1  # ISA_ERR_INVALID_ARG
    isa.isa_debug_set_flags(0)


def test_status_strings():
    for s in range(5):
        assert isa.isa_status_string(s).startswith("ISA_")
    assert "UNKNOWN" in isa.isa_status_string(99)
    assert isa.isa_last_hip_error() == 0


@pytest.mark.parametrize("name", list(CONFIGS))
def test_plan_info_matches_oracle_counts(name):
    c = CONFIGS[name]
    dt = "bf16" if c["dtype"] == "bf16" else "fp32"
    import torch
    p = isa.isa_plan_create(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["block"],
                            c["alpha_s"], c["alpha_f"],
                            dtype=torch.bfloat16 if dt == "bf16" else torch.float32)
    info = p.info
    starts, ends, n_src, n_ctx = orc.block_grid(c["L_src"], c["L_ctx"], c["block"])
    n_q = len(starts)
    k = orc.select_count(c["alpha_s"], n_ctx)
    n_flat = orc.flat_count(c["alpha_f"], n_q)
    assert (info["n_src_blocks"], info["n_ctx_blocks"], info["n_q_blocks"]) == (n_src, n_ctx, n_q)
    assert info["k"] == k and info["n_kv_blocks"] == n_src + k
    assert info["l_new"] == c["L_src"] + k * c["block"]
    assert info["n_flat"] == n_flat and info["n_sharp"] == n_q - n_flat
    assert info["workspace_bytes"] > 0


def test_plan_counts_at_headline_shape():
    p = isa.isa_plan_create(1, 40, 16384, 16384, 128, 64, 0.25, 0.5)
    assert p.info["k"] == 64 and p.info["n_kv_blocks"] == 320 and p.info["l_new"] == 20480
    assert p.info["n_flat"] == 256 and p.info["n_sharp"] == 256


@pytest.mark.parametrize("alpha_s,alpha_f", [(0.125, 0.25), (0.25, 0.5), (0.5, 0.75),
                                             (0.0, 0.0), (1.0, 1.0), (0.1, 0.3), (0.33, 0.66)])
def test_plan_counts_follow_the_rounding_rule(alpha_s, alpha_f):
    p = isa.isa_plan_create(1, 2, 25600, 25600, 128, 64, alpha_s, alpha_f)
    assert p.info["k"] == orc.select_count(alpha_s, 400)
    assert p.info["n_flat"] == orc.flat_count(alpha_f, 800)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), isa.ISA_ERR_INVALID_ARG),
    (dict(H=-2), isa.ISA_ERR_INVALID_ARG),
    (dict(D=0), isa.ISA_ERR_INVALID_ARG),
    (dict(L_src=0), isa.ISA_ERR_INVALID_ARG),
    (dict(L_ctx=-64), isa.ISA_ERR_INVALID_ARG),
    (dict(block=0), isa.ISA_ERR_INVALID_ARG),
    (dict(alpha_s=1.5), isa.ISA_ERR_INVALID_ARG),
    (dict(alpha_f=-0.1), isa.ISA_ERR_INVALID_ARG),
    (dict(alpha_s=float("nan")), isa.ISA_ERR_INVALID_ARG),
    (dict(block=96), isa.ISA_ERR_UNSUPPORTED),
    (dict(block=16), isa.ISA_ERR_UNSUPPORTED),
    (dict(block=256), isa.ISA_ERR_UNSUPPORTED),
    (dict(block=32, alpha_ns=0.25), isa.ISA_ERR_UNSUPPORTED),   # the block mask needs b = 64
    (dict(block=128, alpha_ns=0.25), isa.ISA_ERR_UNSUPPORTED),
    (dict(D=96), isa.ISA_ERR_UNSUPPORTED),
    (dict(alpha_ns=1.5), isa.ISA_ERR_INVALID_ARG),
    (dict(L_src=64 * 4097, L_ctx=0), isa.ISA_ERR_UNSUPPORTED),
])
def test_plan_validation(kw, status):
    args = dict(B=1, H=2, L_src=256, L_ctx=256, D=128, block=64, alpha_s=0.5, alpha_f=0.5)
    args.update(kw)
    with pytest.raises(isa.IsaError) as e:
        isa.isa_plan_create(**args)
    assert e.value.status == status


@pytest.mark.parametrize("alpha_ns", [0.0, 0.0625, 0.3, 1.0])
def test_block_mask_count_and_workspace(alpha_ns):
    # the count follows the oracle's rounding (R21); the mask adds only its
    # per-block lists [B, H, n_flat, n_ns] to the workspace, and only when it
    # is used: the coarse logits it ranks are recomputed per flat block, never
    # stored as an [N_Q, N_Q] matrix
    base = isa.isa_plan_create(1, 3, 4096, 4096, 128, 64, 0.25, 0.5)
    p = isa.isa_plan_create(1, 3, 4096, 4096, 128, 64, 0.25, 0.5, alpha_ns)
    n_kv = p.info["n_kv_blocks"]
    assert n_kv == 64 + 16
    assert p.info["n_ns"] == orc.ns_count(alpha_ns, n_kv)
    extra = p.info["workspace_bytes"] - base.info["workspace_bytes"]
    if p.info["n_ns"] == 0:
        assert extra == 0
    else:
        need = 3 * p.info["n_flat"] * p.info["n_ns"] * 4
        assert need <= extra <= need + 256


def test_block_mask_workspace_does_not_grow_with_the_square_of_the_blocks():
    # at the longest head (4096 blocks) an [N_Q, N_Q] fp64 matrix alone would
    # be 128 MiB per head; the mask's lists are n_flat * n_ns * 4 bytes
    for L in (16384, 131072):
        base = isa.isa_plan_create(1, 1, L, L, 128, 64, 0.25, 0.5)
        p = isa.isa_plan_create(1, 1, L, L, 128, 64, 0.25, 0.5, 0.0625)
        lists = p.info["n_flat"] * p.info["n_ns"] * 4
        assert p.info["workspace_bytes"] - base.info["workspace_bytes"] <= lists + 256


@pytest.mark.parametrize("L_src,L_ctx", [(100, 200), (50, 0), (64, 1), (1000, 1000), (4097, 63)])
def test_partial_blocks_grid(L_src, L_ctx):
    # each segment is cut from its own start; the counts follow the oracle's grid
    p = isa.isa_plan_create(1, 2, L_src, L_ctx, 128, 64, 0.5, 0.5)
    starts, ends, n_src, n_ctx = orc.block_grid(L_src, L_ctx, 64)
    assert (p.info["n_src_blocks"], p.info["n_ctx_blocks"]) == (n_src, n_ctx)
    assert p.info["n_q_blocks"] == len(starts)
    assert p.info["k"] == orc.select_count(0.5, n_ctx)
    assert p.info["n_flat"] == orc.flat_count(0.5, len(starts))


def test_unaligned_gather_unsupported_backward_checks_its_workspace():
    # isa_gather needs whole blocks (K_new's length would depend on sel); the
    # backward takes partial blocks and b = 32, 128, and refuses too small a
    # workspace before any launch
    lib = isa._lib()
    p = isa.isa_plan_create(1, 2, 100, 200, 128, 64, 0.5, 0.5)
    fake = ctypes.c_void_p(0x1000)
    assert lib.isa_gather(p.handle, fake, fake, fake, fake, fake, None) == isa.ISA_ERR_UNSUPPORTED
    a = isa.isa_aux_t()
    a.sel = a.flat = a.sharp = 0x1000
    for b, (L_src, L_ctx) in ((64, (100, 200)), (32, (100, 200)), (128, (300, 500))):
        p = isa.isa_plan_create(1, 2, L_src, L_ctx, 128, b, 0.5, 0.5)
        need = lib.isa_backward_workspace_bytes(p.handle)
        assert need > 0
        st = lib.isa_backward(p.handle, fake, fake, fake, fake, fake, fake, ctypes.byref(a),
                              fake, fake, fake, fake, need - 1, None)
        assert st == isa.ISA_ERR_WORKSPACE


def test_backward_with_block_mask_needs_ns():
    # the block mask's backward reads the forward's ns; a null pointer is
    # refused before any launch
    lib = isa._lib()
    p = isa.isa_plan_create(1, 2, 256, 256, 128, 64, 0.5, 0.5, 0.25)
    assert p.info["n_ns"] > 0 and p.info["n_flat"] > 0
    fake = ctypes.c_void_p(0x1000)
    a = isa.isa_aux_t()
    a.sel = a.flat = a.sharp = 0x1000
    st = lib.isa_backward(p.handle, fake, fake, fake, fake, fake, fake, ctypes.byref(a),
                          fake, fake, fake, fake, 1 << 40, None)
    assert st == isa.ISA_ERR_INVALID_ARG


def test_backward_block_mask_workspace():
    # the mask adds its exact-block tables (mask rows, the dQ pairs' unions,
    # the key groups' lists) to the backward workspace; too small a workspace
    # is refused before any launch
    lib = isa._lib()
    B, H, L_src, L_ctx = 2, 3, 1024, 3072
    base = isa.isa_plan_create(B, H, L_src, L_ctx, 128, 64, 0.25, 0.5)
    p = isa.isa_plan_create(B, H, L_src, L_ctx, 128, 64, 0.25, 0.5, 0.0625)
    n_flat, n_ns, n_kv = p.info["n_flat"], p.info["n_ns"], p.info["n_kv_blocks"]
    need = lib.isa_backward_workspace_bytes(p.handle)
    extra = need - lib.isa_backward_workspace_bytes(base.handle)
    tables = 4 * B * H * (n_flat * ((n_kv + 31) // 32) + ((n_flat + 1) // 2) * (2 * n_ns + 1)
                          + (n_kv + 1) // 2 + 1 + n_flat * n_ns)
    assert tables <= extra <= tables + 5 * 256
    fake = ctypes.c_void_p(0x1000)
    a = isa.isa_aux_t()
    a.sel = a.flat = a.sharp = a.ns = 0x1000
    st = lib.isa_backward(p.handle, fake, fake, fake, fake, fake, fake, ctypes.byref(a),
                          fake, fake, fake, fake, need - 1, None)
    assert st == isa.ISA_ERR_WORKSPACE


@pytest.mark.parametrize("base", [-1.0, float("nan"), float("inf")])
def test_rope_base_validation(base):
    with pytest.raises(isa.IsaError) as e:
        isa.isa_plan_create(1, 2, 256, 256, 128, 64, 0.5, 0.5, rope_base=base)
    assert e.value.status == isa.ISA_ERR_INVALID_ARG


def test_rope_workspace_holds_the_rotated_q_and_k():
    plain = isa.isa_plan_create(2, 3, 700, 500, 128, 64, 0.5, 0.5)
    rope = isa.isa_plan_create(2, 3, 700, 500, 128, 64, 0.5, 0.5, rope_base=10000.0)
    tokens = 2 * 3 * 1200 * 128 * 2
    assert rope.info["workspace_bytes"] >= plain.info["workspace_bytes"] + 2 * tokens
    assert {k: v for k, v in rope.info.items() if k != "workspace_bytes"} == \
        {k: v for k, v in plain.info.items() if k != "workspace_bytes"}


def test_backward_with_rope_takes_the_rotated_copies_in_its_workspace():
    # the backward re-rotates Q and K into its workspace (two [B, H, N, D]
    # copies) and turns dQ, dK back; the check of the workspace size comes
    # before any launch
    lib = isa._lib()
    base = isa.isa_plan_create(1, 2, 256, 256, 128, 64, 0.5, 0.5)
    p = isa.isa_plan_create(1, 2, 256, 256, 128, 64, 0.5, 0.5, rope_base=10000.0)
    need = lib.isa_backward_workspace_bytes(p.handle)
    extra = need - lib.isa_backward_workspace_bytes(base.handle)
    assert 2 * 2 * 512 * 128 * 2 <= extra <= 2 * 2 * 512 * 128 * 2 + 512
    fake = ctypes.c_void_p(0x1000)
    a = isa.isa_aux_t()
    a.sel = a.flat = a.sharp = 0x1000
    st = lib.isa_backward(p.handle, fake, fake, fake, fake, fake, fake, ctypes.byref(a),
                          fake, fake, fake, fake, need - 16, None)
    assert st == isa.ISA_ERR_WORKSPACE


@pytest.mark.parametrize("block,L_src,L_ctx", [(32, 500, 300), (128, 1000, 700), (32, 512, 384),
                                               (128, 1024, 0)])
def test_other_block_lengths_follow_the_oracle_counts(block, L_src, L_ctx):
    p = isa.isa_plan_create(1, 2, L_src, L_ctx, 128, block, 0.34, 0.5)
    starts, ends, n_src, n_ctx = orc.block_grid(L_src, L_ctx, block)
    assert (p.info["n_src_blocks"], p.info["n_ctx_blocks"]) == (n_src, n_ctx)
    assert p.info["k"] == orc.select_count(0.34, n_ctx)
    assert p.info["n_flat"] == orc.flat_count(0.5, len(starts))
    # the block mask is refused only when some query block is flat
    q = isa.isa_plan_create(1, 2, L_src, L_ctx, 128, block, 0.34, 0.0, 0.5)
    assert q.info["n_flat"] == 0


def test_backward_needs_bf16():
    # the backward kernels take bf16 operands; an fp32 plan is refused before
    # any launch, at every block length
    lib = isa._lib()
    fake = ctypes.c_void_p(0x1000)
    a = isa.isa_aux_t()
    a.sel = a.flat = a.sharp = 0x1000
    for block in (32, 64, 128):
        p = isa.isa_plan_create(1, 2, 512, 512, 128, block, 0.5, 0.5, dtype=isa.ISA_DTYPE_FP32)
        st = lib.isa_backward(p.handle, fake, fake, fake, fake, fake, fake, ctypes.byref(a),
                              fake, fake, fake, fake, 1 << 40, None)
        assert st == isa.ISA_ERR_UNSUPPORTED


def test_null_arguments_rejected_before_any_launch():
    lib = isa._lib()
    assert lib.isa_plan_create(None, None) == isa.ISA_ERR_INVALID_ARG
    assert lib.isa_plan_get_info(None, None) == isa.ISA_ERR_INVALID_ARG
    assert lib.isa_plan_destroy(None) == isa.ISA_OK
    p = isa.isa_plan_create(1, 2, 256, 256, 128)
    # null tensors / workspace: rejected on the host, nothing launched
    assert lib.isa_forward(p.handle, None, None, None, None, None, None, None, 0, None) \
        == isa.ISA_ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)
    assert lib.isa_forward(p.handle, fake, fake, fake, fake, None, None, None, 0, None) \
        == isa.ISA_ERR_WORKSPACE
    assert lib.isa_forward(p.handle, fake, fake, fake, fake, None, None, fake, 16, None) \
        == isa.ISA_ERR_WORKSPACE
    misaligned = ctypes.c_void_p(0x1004)
    assert lib.isa_forward(p.handle, misaligned, fake, fake, fake, None, None, fake, 1 << 40,
                           None) == isa.ISA_ERR_INVALID_ARG
    assert lib.isa_forward(None, fake, fake, fake, fake, None, None, fake, 1 << 40, None) \
        == isa.ISA_ERR_INVALID_ARG
    assert lib.isa_gather(p.handle, None, fake, fake, fake, fake, None) == isa.ISA_ERR_INVALID_ARG
    assert lib.isa_dense_forward(1, 1, 100, 128, 0, fake, fake, fake, fake, None, None) \
        == isa.ISA_ERR_UNSUPPORTED
    assert lib.isa_dense_forward(1, 1, 128, 128, 0, None, fake, fake, fake, None, None) \
        == isa.ISA_ERR_INVALID_ARG
    assert lib.isa_dense_forward(-1, 1, 128, 128, 0, fake, fake, fake, fake, None, None) \
        == isa.ISA_ERR_INVALID_ARG


def test_empty_problem_is_a_no_op():
    lib = isa._lib()
    p = isa.isa_plan_create(0, 4, 256, 256, 128)
    assert p.info["workspace_bytes"] >= 0
    assert lib.isa_forward(p.handle, None, None, None, None, None, None, None, 0, None) == isa.ISA_OK
    assert lib.isa_forward_noalloc(p.handle, None, None, None, None, None, None, None) == isa.ISA_OK
    assert lib.isa_dense_forward(0, 3, 128, 128, 0, None, None, None, None, None, None) == isa.ISA_OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    p = isa.isa_plan_create(1, 1, 64, 64, 64)
    x = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        isa.isa_forward(p, x, x, x)
    with pytest.raises(TypeError):
        isa.isa_dense_forward(x, x, x)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no CPU fallback: without the HIP library every entry point raises
    monkeypatch.setattr(isa, "_L", None)
    monkeypatch.setattr(isa, "LIB_PATH", str(tmp_path / "libisa.so"))
    with pytest.raises(RuntimeError, match="not built"):
        isa.isa_plan_create(1, 1, 64, 64, 64)
    with pytest.raises(RuntimeError, match="not built"):
        isa._lib()


def test_injected_launch_failure_reaches_isa_error():
    # The launch wrapper's failure hook: the first launch reports hipErrorLaunchFailure
    # (719) without being issued, so no HIP call happens and no GPU is needed.  The
    # status must come back as ISA_ERR_HIP, with the HIP code in isa_last_hip_error,
    # and the binding must turn it into IsaError.
    lib = isa._lib()
    p = isa.isa_plan_create(1, 2, 256, 256, 128)
    fake = ctypes.c_void_p(0x1000)
    ws = p.info["workspace_bytes"]
    isa.isa_testing_fail_launch(0, 719)
    st = lib.isa_forward(p.handle, fake, fake, fake, fake, None, None, fake, ws, None)
    assert st == isa.ISA_ERR_HIP
    assert isa.isa_last_hip_error() == 719
    with pytest.raises(isa.IsaError, match=r"ISA_ERR_HIP.*hipError 719") as e:
        isa._check(st, "isa_forward")
    assert e.value.status == isa.ISA_ERR_HIP
    # the hook fires once: the dense entry point (its first launch) fails the same way
    isa.isa_testing_fail_launch(0, 98)
    assert lib.isa_dense_forward(1, 1, 128, 128, 0, fake, fake, fake, fake, None, None) \
        == isa.ISA_ERR_HIP
    assert isa.isa_last_hip_error() == 98
    # invalid arguments to the hook
    with pytest.raises(isa.IsaError, match="INVALID_ARG"):
        isa.isa_testing_fail_launch(-1, 5)
    isa.isa_testing_fail_launch(0, 0)  # disarmed


def test_plan_log(tmp_path):
    # ISA_LOG=1 prints each plan's derived sizes to stderr (in a child process,
    # so the environment is read fresh)
    import subprocess
    import sys
    code = ("import sparse_attention_context_block_amd as isa; "
            "isa.isa_plan_create(1, 40, 16384, 16384, 128, 64, 0.25, 0.5)")
    env = dict(os.environ, ISA_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "[isa] plan" in r.stderr and "k=64" in r.stderr and "L_new=20480" in r.stderr
    env["ISA_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert "[isa] plan" not in r.stderr


def test_backward_binding_validates_decisions():
    # the backward kernels read sel/flat/sharp unchecked, so the binding refuses
    # wrong dtypes or shapes (ValueError) and host tensors (TypeError) before
    # any launch
    import torch
    p = isa.isa_plan_create(1, 2, 256, 256, 128)
    info = p.info
    shapes = {"sel": (1, 2, info["k"]), "flat": (1, 2, info["n_flat"]),
              "sharp": (1, 2, info["n_sharp"])}
    good = {f: torch.zeros(sh, dtype=torch.int32) for f, sh in shapes.items()}
    for f in shapes:
        bad = dict(good, **{f: good[f].to(torch.int64)})  # e.g. oracle output moved over
        with pytest.raises(ValueError, match=f"aux\\['{f}'\\].*int32"):
            isa._decision_aux(p, bad)
        bad = dict(good, **{f: torch.zeros(1, 2, shapes[f][2] + 1, dtype=torch.int32)})
        with pytest.raises(ValueError, match=f"aux\\['{f}'\\]"):
            isa._decision_aux(p, bad)
        missing = {g: t for g, t in good.items() if g != f}
        with pytest.raises(ValueError, match="lacks"):
            isa._decision_aux(p, missing)
    with pytest.raises(TypeError, match="GPU"):  # right dtype and shape, host memory
        isa._decision_aux(p, good)
    x = torch.zeros(1, 2, 512, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        isa.isa_backward(p, x, x, x, x, x, torch.zeros(1, 2, 512), good)


def test_noalloc_forward_limit_checked_on_the_host():
    """isa_forward_noalloc refuses a plan whose workspace exceeds the static
    array before any HIP call (so this runs without a GPU); the bound in the
    binding matches the header's."""
    text = open(HEADER).read()
    assert re.search(r"#define ISA_STATIC_WORKSPACE_BYTES \(\(size_t\)128 << 20\)", text)
    assert isa.ISA_STATIC_WORKSPACE_BYTES == 128 << 20
    lib = isa._lib()
    assert lib.isa_forward_noalloc(None, None, None, None, None, None, None, None) \
        == isa.ISA_ERR_INVALID_ARG
    # the rotated Q and K live in the workspace: 2 x 40 x 32768 x 128 x 2 bytes alone
    big = isa.isa_plan_create(1, 40, 16384, 16384, 128, rope_base=10000.0)
    assert big.info["workspace_bytes"] > isa.ISA_STATIC_WORKSPACE_BYTES
    fake = ctypes.c_void_p(0x1000)
    assert lib.isa_forward_noalloc(big.handle, fake, fake, fake, fake, None, None, None) \
        == isa.ISA_ERR_WORKSPACE
    # the headline shape fits
    head = isa.isa_plan_create(1, 40, 16384, 16384, 128)
    assert head.info["workspace_bytes"] <= isa.ISA_STATIC_WORKSPACE_BYTES
