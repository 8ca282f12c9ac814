"""In-context Sparse Attention (ISA) for AMD Instinct MI355X (gfx950).

Thin Python binding of ``libisa.so`` (declared in ``include/isa.h``).  Every
function here only marshals arguments: torch supplies device memory and the
current HIP stream, and every step of the computation runs in the library's
HIP kernels.  There is no CPU fallback: if the library is not built, or a
tensor is not on the GPU, the call raises.

Names follow the C ABI: ``isa_plan_create``, ``isa_plan_get_info``,
``isa_forward``, ``isa_gather``, ``isa_dense_forward``, ``isa_backward``,
``isa_status_string``, ``isa_last_hip_error``.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libisa.so")

ISA_OK, ISA_ERR_INVALID_ARG, ISA_ERR_UNSUPPORTED, ISA_ERR_WORKSPACE, ISA_ERR_HIP = range(5)
ISA_DTYPE_BF16, ISA_DTYPE_FP32 = 0, 1
ISA_PROFILE_STAGES = 6
ISA_STATIC_WORKSPACE_BYTES = 128 << 20
STAGE_NAMES = ("pool", "coarse_rowstats", "coarse_colsum", "select_route", "attn_exact",
               "attn_taylor")
_DTYPES = {torch.bfloat16: ISA_DTYPE_BF16, torch.float32: ISA_DTYPE_FP32}

# Every symbol include/isa.h declares, and the test hooks of include/isa_testing.h.
EXPORTS = ("isa_plan_create", "isa_plan_get_info", "isa_plan_destroy", "isa_forward",
           "isa_forward_profiled", "isa_forward_noalloc", "isa_gather", "isa_dense_forward", "isa_backward",
           "isa_backward_workspace_bytes", "isa_status_string", "isa_last_hip_error")
TESTING_EXPORTS = ("isa_debug_set_flags", "isa_testing_fail_launch")


class IsaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {isa_status_string(status)}"
                         + (f" (hipError {isa_last_hip_error()})" if status == ISA_ERR_HIP else ""))


class isa_plan_desc_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L_src", ctypes.c_int32),
                ("L_ctx", ctypes.c_int32), ("D", ctypes.c_int32), ("block", ctypes.c_int32),
                ("alpha_s", ctypes.c_double), ("alpha_f", ctypes.c_double),
                ("alpha_ns", ctypes.c_double), ("dtype", ctypes.c_int),
                ("rope_base", ctypes.c_double)]


class isa_plan_info_t(ctypes.Structure):
    _fields_ = [("n_src_blocks", ctypes.c_int64), ("n_ctx_blocks", ctypes.c_int64),
                ("n_q_blocks", ctypes.c_int64), ("k", ctypes.c_int64),
                ("n_kv_blocks", ctypes.c_int64), ("l_new", ctypes.c_int64),
                ("n_flat", ctypes.c_int64), ("n_sharp", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("n_ns", ctypes.c_int64)]


class isa_aux_t(ctypes.Structure):
    _fields_ = [("sel", ctypes.c_void_p), ("flat", ctypes.c_void_p), ("sharp", ctypes.c_void_p),
                ("ctx_score", ctypes.c_void_p), ("sharpness", ctypes.c_void_p),
                ("ns", ctypes.c_void_p)]


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m sparse_attention_context_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.isa_plan_create.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(isa_plan_desc_t)]
        L.isa_plan_get_info.argtypes = [vp, ctypes.POINTER(isa_plan_info_t)]
        L.isa_plan_destroy.argtypes = [vp]
        L.isa_forward.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(isa_aux_t), vp, sz, vp]
        L.isa_forward_profiled.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(isa_aux_t),
                                           vp, sz, vp, ctypes.POINTER(vp)]
        L.isa_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(isa_aux_t), vp]
        L.isa_gather.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.isa_dense_forward.argtypes = [i32, i32, i32, i32, ctypes.c_int, vp, vp, vp, vp, vp, vp]
        L.isa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(isa_aux_t),
                                   vp, vp, vp, vp, sz, vp]
        L.isa_backward_workspace_bytes.argtypes = [vp]
        L.isa_backward_workspace_bytes.restype = sz
        L.isa_status_string.argtypes = [ctypes.c_int]
        L.isa_status_string.restype = ctypes.c_char_p
        L.isa_last_hip_error.argtypes = []
        L.isa_debug_set_flags.argtypes = [ctypes.c_uint32]
        L.isa_testing_fail_launch.argtypes = [i32, i32]
        for name in ("isa_plan_create", "isa_plan_get_info", "isa_plan_destroy", "isa_forward",
                     "isa_forward_profiled", "isa_forward_noalloc", "isa_gather", "isa_dense_forward", "isa_backward",
                     "isa_last_hip_error", "isa_debug_set_flags", "isa_testing_fail_launch"):
            getattr(L, name).restype = ctypes.c_int
        _L = L
    return _L


def isa_status_string(status):
    return _lib().isa_status_string(int(status)).decode()


def isa_last_hip_error():
    return int(_lib().isa_last_hip_error())


# Test hooks (include/isa_testing.h): not needed to run ISA.
ISA_DEBUG_GLOBAL_TABLES = 1
ISA_DEBUG_4WAVE_EXACT = 2
ISA_DEBUG_PINGPONG_EXACT = 4


def isa_debug_set_flags(flags):
    """Kernel-path switches (isa_testing.h); raises on unknown bits."""
    _check(_lib().isa_debug_set_flags(int(flags)), "isa_debug_set_flags")


def isa_testing_fail_launch(skip, hip_error):
    """Arm the launch wrapper to report hip_error after `skip` good launches
    (isa_testing.h); hip_error 0 disarms."""
    _check(_lib().isa_testing_fail_launch(int(skip), int(hip_error)), "isa_testing_fail_launch")


def _check(status, what):
    if status != ISA_OK:
        raise IsaError(status, what)


class Plan:
    """Owns an ``isa_plan_t``; ``info`` holds isa_plan_get_info's fields."""

    def __init__(self, handle, desc):
        self.handle = handle
        self.desc = desc
        self.info = isa_plan_get_info(self)

    def __del__(self):
        if getattr(self, "handle", None) and _L is not None:
            _L.isa_plan_destroy(self.handle)
            self.handle = None


def isa_plan_create(B, H, L_src, L_ctx, D, block=64, alpha_s=0.25, alpha_f=0.5, alpha_ns=0.0,
                    dtype=torch.bfloat16, rope_base=0.0):
    desc = isa_plan_desc_t(B, H, L_src, L_ctx, D, block, alpha_s, alpha_f, alpha_ns,
                           _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
                           rope_base)
    h = ctypes.c_void_p()
    _check(_lib().isa_plan_create(ctypes.byref(h), ctypes.byref(desc)), "isa_plan_create")
    return Plan(h, desc)


def isa_plan_get_info(plan):
    info = isa_plan_info_t()
    _check(_lib().isa_plan_get_info(plan.handle, ctypes.byref(info)), "isa_plan_get_info")
    return {f: getattr(info, f) for f, _ in isa_plan_info_t._fields_}


def _dev(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _torch_dtype(plan):
    return torch.bfloat16 if plan.desc.dtype == ISA_DTYPE_BF16 else torch.float32


def isa_forward(plan, q, k, v, o=None, lse=None, aux=False, workspace=None, stream=None,
                events=None):
    """Run the ISA forward.  Returns (o, lse, aux_dict or None).

    ``aux=True`` also returns the decisions: sel, flat, sharp (int32),
    ctx_score, sharpness (float64), each [B, H, ...], and with a block mask
    (info n_ns > 0) ns [B, H, n_flat, n_ns] (int32).  ``events``: optional
    list of ISA_PROFILE_STAGES + 1 torch.cuda.Event(enable_timing=True),
    recorded before the first stage and after every stage
    (isa_forward_profiled).
    """
    d, info = plan.desc, plan.info
    N = d.L_src + d.L_ctx
    shape = (d.B, d.H, N, d.D)
    dt = _torch_dtype(plan)
    dev = q.device
    ptrs = [_dev(x, dt, shape, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v"))]
    if o is None:
        o = torch.empty(shape, dtype=dt, device=dev)
    if lse is None:
        lse = torch.empty((d.B, d.H, N), dtype=torch.float32, device=dev)
    out_aux = None
    a = isa_aux_t()
    if aux:
        bh = (d.B, d.H)
        out_aux = dict(
            sel=torch.empty(bh + (info["k"],), dtype=torch.int32, device=dev),
            flat=torch.empty(bh + (info["n_flat"],), dtype=torch.int32, device=dev),
            sharp=torch.empty(bh + (info["n_sharp"],), dtype=torch.int32, device=dev),
            ctx_score=torch.empty(bh + (info["n_ctx_blocks"],), dtype=torch.float64, device=dev),
            sharpness=torch.empty(bh + (info["n_q_blocks"],), dtype=torch.float64, device=dev))
        if info["n_ns"] > 0 and info["n_flat"] > 0:
            out_aux["ns"] = torch.empty(bh + (info["n_flat"], info["n_ns"]), dtype=torch.int32,
                                        device=dev)
        for f, t in out_aux.items():
            setattr(a, f, t.data_ptr() if t.numel() else None)
    if workspace is None:
        workspace = torch.empty(max(info["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
    args = (plan.handle, *ptrs, _dev(o, dt, shape, "o"),
            _dev(lse, torch.float32, shape[:3], "lse"), ctypes.byref(a),
            workspace.data_ptr(), workspace.numel(), _stream(stream))
    if events is None:
        _check(_lib().isa_forward(*args), "isa_forward")
    else:
        if len(events) != ISA_PROFILE_STAGES + 1:
            raise ValueError(f"need {ISA_PROFILE_STAGES + 1} events")
        for ev in events:  # torch creates the underlying hipEvent_t on first record
            if not ev.cuda_event:
                ev.record()
        arr = (ctypes.c_void_p * len(events))(*[ev.cuda_event for ev in events])
        _check(_lib().isa_forward_profiled(*args, arr), "isa_forward_profiled")
    return o, lse, out_aux


def isa_forward_noalloc(plan, q, k, v, o, lse=None, aux=None, stream=None):
    """The ISA forward with the library's static per-device workspace
    (isa_forward_noalloc): allocates nothing, so every output is the caller's.
    ``o``: [B, H, N, D]; ``lse``: [B, H, N] float32 or None (not written);
    ``aux``: None or a dict of preallocated decision tensors, any subset of
    the keys isa_forward(aux=True) returns, with the same dtypes and shapes.
    Plans whose workspace_bytes exceed ISA_STATIC_WORKSPACE_BYTES raise
    IsaError (ISA_ERR_WORKSPACE).  Calls that overlap on one device race."""
    d, info = plan.desc, plan.info
    N = d.L_src + d.L_ctx
    shape = (d.B, d.H, N, d.D)
    dt = _torch_dtype(plan)
    ptrs = [_dev(x, dt, shape, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lse_p = None if lse is None else _dev(lse, torch.float32, shape[:3], "lse")
    a = isa_aux_t()
    if aux:
        bh = (d.B, d.H)
        spec = dict(sel=(torch.int32, bh + (info["k"],)),
                    flat=(torch.int32, bh + (info["n_flat"],)),
                    sharp=(torch.int32, bh + (info["n_sharp"],)),
                    ctx_score=(torch.float64, bh + (info["n_ctx_blocks"],)),
                    sharpness=(torch.float64, bh + (info["n_q_blocks"],)),
                    ns=(torch.int32, bh + (info["n_flat"], info["n_ns"])))
        for f, t in aux.items():
            if f not in spec:
                raise ValueError(f"aux: unknown field {f!r}")
            dtype_f, shape_f = spec[f]
            setattr(a, f, _dev(t, dtype_f, shape_f, f"aux[{f!r}]") if t.numel() else None)
    _check(_lib().isa_forward_noalloc(plan.handle, *ptrs, lse_p, ctypes.byref(a),
                                      _stream(stream)), "isa_forward_noalloc")
    return o, lse


def isa_gather(plan, k, v, sel, k_new=None, v_new=None, stream=None):
    """Materialise K_new, V_new [B, H, l_new, D] from sel [B, H, k] (into k_new,
    v_new if given)."""
    d, info = plan.desc, plan.info
    shape = (d.B, d.H, d.L_src + d.L_ctx, d.D)
    dt = _torch_dtype(plan)
    kp, vp = _dev(k, dt, shape, "k"), _dev(v, dt, shape, "v")
    sp = _dev(sel, torch.int32, (d.B, d.H, info["k"]), "sel") if info["k"] else None
    new_shape = (d.B, d.H, info["l_new"], d.D)
    if k_new is None:
        k_new = torch.empty(new_shape, dtype=dt, device=k.device)
    if v_new is None:
        v_new = torch.empty_like(k_new)
    _dev(k_new, dt, new_shape, "k_new")
    _dev(v_new, dt, new_shape, "v_new")
    _check(_lib().isa_gather(plan.handle, kp, vp, sp, k_new.data_ptr(), v_new.data_ptr(),
                             _stream(stream)), "isa_gather")
    return k_new, v_new


def isa_dense_forward(q, k, v, o=None, lse=None, stream=None):
    """The library's dense attention softmax(Q K^T / sqrt(D)) V.  Returns (o, lse)."""
    B, H, N, D = q.shape
    dt = q.dtype
    ptrs = [_dev(x, dt, (B, H, N, D), nm) for x, nm in ((q, "q"), (k, "k"), (v, "v"))]
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(_lib().isa_dense_forward(B, H, N, D, _DTYPES[dt], *ptrs,
                                    _dev(o, dt, (B, H, N, D), "o"),
                                    _dev(lse, torch.float32, (B, H, N), "lse"), _stream(stream)),
           "isa_dense_forward")
    return o, lse


def _decision_aux(plan, aux):
    """isa_aux_t with the forward's decisions sel, flat, sharp (and, with the
    block mask, ns) for the backward.

    The backward kernels read these ids unchecked, so each must be an int32,
    contiguous [B, H, count] tensor of this plan (ValueError otherwise) on the
    GPU (TypeError otherwise)."""
    d, info = plan.desc, plan.info
    a = isa_aux_t()
    shapes = {"sel": (d.B, d.H, info["k"]), "flat": (d.B, d.H, info["n_flat"]),
              "sharp": (d.B, d.H, info["n_sharp"])}
    if info["n_ns"] > 0 and info["n_flat"] > 0:  # the block mask of the flat blocks
        shapes["ns"] = (d.B, d.H, info["n_flat"], info["n_ns"])
    for f, shape in shapes.items():
        if f not in aux:
            raise ValueError(f"aux lacks {f!r}")
        t = aux[f]
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 \
                or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"aux[{f!r}]: expected contiguous int32 {shape}, got "
                             f"{getattr(t, 'dtype', type(t))} {tuple(getattr(t, 'shape', ()))}")
    for f, shape in shapes.items():
        if not aux[f].is_cuda:
            raise TypeError(f"aux[{f!r}] must be a GPU tensor")
        setattr(a, f, aux[f].data_ptr() if shape[-1] else None)
    return a


def isa_backward(plan, q, k, v, o, do, lse, aux, workspace=None, stream=None):
    """Gradients (dq, dk, dv) with the forward's decisions (aux) held fixed."""
    d, info = plan.desc, plan.info
    shape = (d.B, d.H, d.L_src + d.L_ctx, d.D)
    dt = _torch_dtype(plan)
    ptrs = [_dev(x, dt, shape, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"),
                                                 (do, "do"))]
    a = _decision_aux(plan, aux)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nbytes = _lib().isa_backward_workspace_bytes(plan.handle)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = _lib().isa_backward(plan.handle, *ptrs, _dev(lse, torch.float32, shape[:3], "lse"),
                             ctypes.byref(a), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                             workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(st, "isa_backward")
    return dq, dk, dv
