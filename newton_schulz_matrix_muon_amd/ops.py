"""Thin ctypes binding of libmuon_ns.so (include/muon_ns.h).

Argument marshalling only: torch tensors are described to the C ABI by pointer, dtype,
shape and strides, the workspace is a torch allocation, and the stream is torch's
current stream. Every step of the computation runs in the library's HIP kernels. If the
library is missing this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmuon_ns.so")

F32, BF16, F16 = 0, 1, 2
STANDARD, GRAM = 0, 1
STATUS = {0: "MNS_OK", -1: "MNS_ERR_ARG", -2: "MNS_ERR_DTYPE", -3: "MNS_ERR_SHAPE",
          -4: "MNS_ERR_WORKSPACE", -5: "MNS_ERR_HIP", -6: "MNS_ERR_UNSUPPORTED"}

# Defaults of the guide's optimizer listing (lr, momentum, weight decay, steps, eps).
DEFAULT_STEPS = 5
DEFAULT_EPS = 1e-7
STABILIZED_RESTART_MASK = 1 << 2


class MnsTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("stride", ctypes.c_int64)]


class MnsNsParams(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int32), ("coeffs", ctypes.POINTER(ctypes.c_float)),
                ("eps", ctypes.c_float), ("iter_dtype", ctypes.c_int32),
                ("restart_mask", ctypes.c_uint32)]


class MnsStepParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("scale_coeff", ctypes.c_float),
                ("nesterov", ctypes.c_int32), ("variant", ctypes.c_int32)]


class MnsError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({_lib().mns_status_string(code).decode()})"
                         + (f", hipError {_lib().mns_last_hip_error()}" if code == -5 else ""))


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m newton_schulz_matrix_muon_amd.build`")
        # torch carries its own HIP runtime (soname libamdhip64.so.7). Loading it first makes
        # the library bind to that same runtime; loaded the other way round, the library would
        # pull in the system runtime and the process would hold two, and the library's one
        # would not see the device torch's tensors and streams live on.
        _torch()
        _LIB = declare(ctypes.CDLL(LIB_PATH))
    return _LIB


def declare(lib):
    """Set the argument and result types of every C function on a loaded copy of the library
    (needs no GPU and does not import torch); returns the library."""
    P = ctypes.POINTER
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.mns_workspace_bytes.argtypes = [ctypes.c_int, P(MnsTensor), P(MnsNsParams),
                                        ctypes.c_int64, P(sz)]
    for fn in (lib.muon_ns_batched, lib.gram_ns_batched):
        fn.argtypes = [P(MnsTensor), P(MnsTensor), P(MnsNsParams), vp, sz, vp, vp]
    lib.muon_step.argtypes = [P(MnsTensor), P(MnsTensor), P(MnsTensor), P(MnsTensor),
                              P(MnsStepParams), P(MnsNsParams), vp, sz, vp, vp]
    lib.muon_step_noalloc.argtypes = [P(MnsTensor), P(MnsTensor), P(MnsTensor), P(MnsTensor),
                                      P(MnsStepParams), P(MnsNsParams), vp, vp]
    lib.gram_ns_trace.argtypes = [P(MnsTensor), P(MnsTensor), P(MnsNsParams), vp, sz, vp, vp]
    lib.mns_workspace_bytes_grouped.argtypes = [ctypes.c_int, ctypes.c_int, P(MnsTensor),
                                                P(MnsNsParams), P(sz)]
    for fn in (lib.muon_ns_grouped, lib.gram_ns_grouped):
        fn.argtypes = [ctypes.c_int, P(MnsTensor), P(MnsTensor), P(MnsNsParams), vp, sz, vp, vp]
    lib.muon_step_grouped.argtypes = [ctypes.c_int, P(MnsTensor), P(MnsTensor), P(MnsTensor),
                                      P(MnsTensor), P(MnsStepParams), P(MnsNsParams), vp, sz,
                                      vp, vp]
    pp = P(vp)
    lib.adamw_step.argtypes = [ctypes.c_int, pp, pp, pp, pp, P(ctypes.c_int64), ctypes.c_int32,
                               P(MnsAdamwParams), vp]
    lib.adamw_step.restype = ctypes.c_int
    lib.mns_status_string.argtypes = [ctypes.c_int]
    lib.mns_status_string.restype = ctypes.c_char_p
    lib.mns_last_hip_error.argtypes = []
    lib.mns_version.argtypes = []
    lib.mns_timing_enable.argtypes = [ctypes.c_int]
    lib.mns_timing_reset.argtypes = []
    lib.mns_timing_query.argtypes = [ctypes.c_int, P(ctypes.c_double), P(ctypes.c_int64)]
    lib.mns_timing_kinds.argtypes = []
    lib.mns_kernel_kind_name.argtypes = [ctypes.c_int]
    lib.mns_kernel_kind_name.restype = ctypes.c_char_p
    for f in (lib.mns_workspace_bytes, lib.muon_ns_batched, lib.gram_ns_batched, lib.gram_ns_trace,
              lib.mns_workspace_bytes_grouped, lib.muon_ns_grouped, lib.gram_ns_grouped,
              lib.muon_step_grouped,
              lib.muon_step, lib.muon_step_noalloc, lib.mns_last_hip_error, lib.mns_version, lib.mns_timing_enable,
              lib.mns_timing_reset, lib.mns_timing_query, lib.mns_timing_kinds):
        f.restype = ctypes.c_int
    return lib


def lib():
    """The loaded ctypes library (raises ImportError if it has not been built)."""
    return _lib()


def _check(code: int, what: str):
    if code != 0:
        raise MnsError(code, what)


def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def describe(t) -> MnsTensor:
    """mns_tensor for a 2-D (one matrix) or 3-D (batch) tensor with unit column stride."""
    if t.dim() == 2:
        t3 = t.unsqueeze(0)
    elif t.dim() == 3:
        t3 = t
    else:
        raise ValueError("expected a 2-D matrix or a 3-D batch")
    if t3.stride(-1) != 1:
        raise ValueError("rows must be contiguous (stride(-1) == 1)")
    b, r, c = t3.shape
    ld = t3.stride(-2) if r > 1 else c
    stride = t3.stride(0) if b > 1 else r * ld
    return MnsTensor(t3.data_ptr(), dtype_code(t3), b, r, c, ld, stride)


# ------------------------------------------------------------------ argument checks
# The C ABI takes bare device pointers; these checks run before any library call so that a
# host tensor, a mismatched dtype or a short buffer raises here instead of reaching a kernel.
# Dtype, shape and size checks come first and device checks last.

def _batch(t) -> int:
    return t.shape[0] if t.dim() == 3 else 1


def _check_same_shape(what, ref, **named):
    for name, t in named.items():
        if t is not None and tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{what}: {name} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")


def _check_flags(what, flags, total):
    if flags is None:
        return
    torch = _torch()
    if flags.dtype != torch.int32:
        raise TypeError(f"{what}: flags must be int32, got {flags.dtype}")
    if not flags.is_contiguous():
        raise ValueError(f"{what}: flags must be contiguous")
    if flags.numel() < total:
        raise ValueError(f"{what}: flags holds {flags.numel()} entries, the call needs {total}")


def _check_workspace(what, ws):
    if ws is not None and not ws.is_contiguous():
        raise ValueError(f"{what}: workspace must be contiguous")


def _check_device(what, ref, **named):
    """Every named tensor (None skipped) is a device tensor on ref's device."""
    if not ref.is_cuda:
        raise ValueError(f"{what}: tensors must be device tensors (got {ref.device})")
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != ref.device:
            raise ValueError(f"{what}: {name} is on {t.device}, expected {ref.device}")


def _ws_bytes(ws) -> int:
    return ws.numel() * ws.element_size()


def ns_params(steps: int = DEFAULT_STEPS, coeffs: Optional[Sequence] = None,
              eps: float = DEFAULT_EPS, iter_dtype: Optional[int] = None, io_dtype: int = BF16,
              restart_mask: int = STABILIZED_RESTART_MASK):
    keep = None
    cptr = None
    if coeffs is not None:
        flat = []
        for row in coeffs:
            flat.extend(float(v) for v in row)
        if len(flat) != 3 * steps:
            raise ValueError("coeffs must hold one (a, b, c) triple per step")
        keep = (ctypes.c_float * len(flat))(*flat)
        cptr = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
    if iter_dtype is None:
        iter_dtype = F32 if io_dtype == F32 else F16
    p = MnsNsParams(steps, cptr, eps, iter_dtype, restart_mask)
    p._keep = keep  # keep the coefficient array alive with the struct
    return p


def _stream_ptr(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def workspace_bytes(variant: int, G, params: MnsNsParams, max_batch_chunk: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib().mns_workspace_bytes(variant, ctypes.byref(describe(G)), ctypes.byref(params),
                                      max_batch_chunk, ctypes.byref(out)), "mns_workspace_bytes")
    return out.value


def _workspace(variant, G, params, workspace):
    torch = _torch()
    if workspace is None:
        workspace = torch.empty(workspace_bytes(variant, G, params), dtype=torch.uint8,
                                device=G.device)
    return workspace


def _ns(variant, G, out, params, workspace, flags):
    torch = _torch()
    what = "muon_ns_batched" if variant == STANDARD else "gram_ns_batched"
    if out is not None:
        _check_same_shape(what, G, out=out)
        if out.dtype != G.dtype:
            raise TypeError(f"{what}: out must have G's dtype {G.dtype}, got {out.dtype}")
    _check_flags(what, flags, _batch(G))
    _check_workspace(what, workspace)
    _check_device(what, G, out=out, flags=flags, workspace=workspace)
    out = torch.empty_like(G) if out is None else out
    ws = _workspace(variant, G, params, workspace)
    fn = _lib().muon_ns_batched if variant == STANDARD else _lib().gram_ns_batched
    fptr = ctypes.c_void_p(flags.data_ptr()) if flags is not None else None
    _check(fn(ctypes.byref(describe(G)), ctypes.byref(describe(out)), ctypes.byref(params),
              ctypes.c_void_p(ws.data_ptr()), _ws_bytes(ws), fptr, _stream_ptr(G)), what)
    return out


def muon_ns(G, *, steps: int = DEFAULT_STEPS, coeffs=None, eps: float = DEFAULT_EPS,
            iter_dtype: Optional[int] = None, out=None, workspace=None, flags=None):
    """Standard Newton-Schulz of a matrix or batch (C ABI ``muon_ns_batched``)."""
    p = ns_params(steps, coeffs, eps, iter_dtype, dtype_code(G), 0)
    return _ns(STANDARD, G, out, p, workspace, flags)


def gram_ns(G, *, steps: int = DEFAULT_STEPS, coeffs=None, eps: float = DEFAULT_EPS,
            iter_dtype: Optional[int] = None, restart_mask: int = STABILIZED_RESTART_MASK,
            out=None, workspace=None, flags=None):
    """Gram Newton-Schulz (C ABI ``gram_ns_batched``); restart_mask=0 is the naive variant."""
    p = ns_params(steps, coeffs, eps, iter_dtype, dtype_code(G), restart_mask)
    return _ns(GRAM, G, out, p, workspace, flags)


def muon_step(W, G, M, *, lr: float, momentum: float, weight_decay: float,
              scale_coeff: float = 0.2, nesterov: bool = False, variant: int = GRAM,
              steps: int = DEFAULT_STEPS, coeffs=None, eps: float = DEFAULT_EPS,
              iter_dtype: Optional[int] = None, restart_mask: int = STABILIZED_RESTART_MASK,
              U_out=None, workspace=None, flags=None):
    """One fused Muon step (C ABI ``muon_step``); W and M are updated in place."""
    torch = _torch()
    what = "muon_step"
    _check_same_shape(what, G, W=W, M=M, U_out=U_out)
    if M.dtype != torch.float32:
        raise TypeError(f"{what}: the momentum buffer M must be float32, got {M.dtype}")
    _check_flags(what, flags, _batch(G))
    _check_workspace(what, workspace)
    _check_device(what, G, W=W, M=M, U_out=U_out, flags=flags, workspace=workspace)
    p = ns_params(steps, coeffs, eps, iter_dtype, dtype_code(G),
                  restart_mask if variant == GRAM else 0)
    sp = MnsStepParams(lr, momentum, weight_decay, scale_coeff, 1 if nesterov else 0, variant)
    ws = _workspace(variant, G, p, workspace)
    fptr = ctypes.c_void_p(flags.data_ptr()) if flags is not None else None
    u = ctypes.byref(describe(U_out)) if U_out is not None else None
    _check(_lib().muon_step(ctypes.byref(describe(W)), ctypes.byref(describe(G)),
                            ctypes.byref(describe(M)), u, ctypes.byref(sp), ctypes.byref(p),
                            ctypes.c_void_p(ws.data_ptr()), _ws_bytes(ws), fptr, _stream_ptr(G)),
           what)
    return W


# Size of the static device scratch behind muon_step_noalloc (MNS_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 256 << 20


def muon_step_noalloc(W, G, M, *, lr: float, momentum: float, weight_decay: float,
                      scale_coeff: float = 0.2, nesterov: bool = False, variant: int = GRAM,
                      steps: int = DEFAULT_STEPS, coeffs=None, eps: float = DEFAULT_EPS,
                      iter_dtype: Optional[int] = None, restart_mask: int = STABILIZED_RESTART_MASK,
                      U_out=None, flags=None):
    """One fused Muon step without a workspace (C ABI ``muon_step_noalloc``: the library's
    static device scratch); W and M are updated in place."""
    torch = _torch()
    what = "muon_step_noalloc"
    _check_same_shape(what, G, W=W, M=M, U_out=U_out)
    if M.dtype != torch.float32:
        raise TypeError(f"{what}: the momentum buffer M must be float32, got {M.dtype}")
    _check_flags(what, flags, _batch(G))
    _check_device(what, G, W=W, M=M, U_out=U_out, flags=flags)
    p = ns_params(steps, coeffs, eps, iter_dtype, dtype_code(G),
                  restart_mask if variant == GRAM else 0)
    sp = MnsStepParams(lr, momentum, weight_decay, scale_coeff, 1 if nesterov else 0, variant)
    fptr = ctypes.c_void_p(flags.data_ptr()) if flags is not None else None
    u = ctypes.byref(describe(U_out)) if U_out is not None else None
    _check(_lib().muon_step_noalloc(ctypes.byref(describe(W)), ctypes.byref(describe(G)),
                                    ctypes.byref(describe(M)), u, ctypes.byref(sp), ctypes.byref(p),
                                    fptr, _stream_ptr(G)), what)
    return W


# ------------------------------------------------------------------ grouped calls
MAX_GROUPS = 4


def _tensor_array(ts):
    arr = (MnsTensor * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = t if isinstance(t, MnsTensor) else describe(t)
    return arr


def workspace_bytes_grouped(variant: int, Gs, params: MnsNsParams) -> int:
    """Workspace that lets a grouped call process every group side by side."""
    n = ctypes.c_size_t()
    _check(_lib().mns_workspace_bytes_grouped(variant, len(Gs), _tensor_array(Gs), ctypes.byref(params),
                                              ctypes.byref(n)), "mns_workspace_bytes_grouped")
    return n.value


def _check_groups(what, Gs, flags, workspace, **lists):
    """Group lists of equal length (1 .. MAX_GROUPS), flags covering every matrix of every
    group, everything on the first G's device."""
    n = len(Gs)
    if not 1 <= n <= MAX_GROUPS:
        raise ValueError(f"{what}: between 1 and {MAX_GROUPS} groups, got {n}")
    for name, ts in lists.items():
        if ts is not None and len(ts) != n:
            raise ValueError(f"{what}: {name} has {len(ts)} entries for {n} groups")
    _check_flags(what, flags, sum(_batch(G) for G in Gs))
    _check_workspace(what, workspace)
    named = {"flags": flags, "workspace": workspace}
    for i, G in enumerate(Gs):
        named[f"G[{i}]"] = G
        for name, ts in lists.items():
            if ts is not None:
                named[f"{name}[{i}]"] = ts[i]
    _check_device(what, Gs[0], **named)


def _ns_grouped(variant, Gs, outs, params, workspace, flags):
    torch = _torch()
    what = "muon_ns_grouped" if variant == STANDARD else "gram_ns_grouped"
    if outs is not None:
        if len(outs) != len(Gs):
            raise ValueError(f"{what}: outs has {len(outs)} entries for {len(Gs)} groups")
        for i, (G, O) in enumerate(zip(Gs, outs)):
            _check_same_shape(what, G, **{f"outs[{i}]": O})
            if O.dtype != G.dtype:
                raise TypeError(f"{what}: outs[{i}] must have dtype {G.dtype}, got {O.dtype}")
    _check_groups(what, Gs, flags, workspace, outs=outs)
    outs = [torch.empty_like(G) for G in Gs] if outs is None else list(outs)
    if workspace is None:
        workspace = torch.empty(workspace_bytes_grouped(variant, Gs, params), dtype=torch.uint8,
                                device=Gs[0].device)
    fn = _lib().muon_ns_grouped if variant == STANDARD else _lib().gram_ns_grouped
    fptr = ctypes.c_void_p(flags.data_ptr()) if flags is not None else None
    _check(fn(len(Gs), _tensor_array(Gs), _tensor_array(outs), ctypes.byref(params),
              ctypes.c_void_p(workspace.data_ptr()), _ws_bytes(workspace), fptr, _stream_ptr(Gs[0])),
           what)
    return outs


def muon_ns_grouped(Gs, *, steps: int = DEFAULT_STEPS, coeffs=None, eps: float = DEFAULT_EPS,
                    iter_dtype: Optional[int] = None, outs=None, workspace=None, flags=None):
    """Standard Newton-Schulz of several batches of different shapes (C ABI ``muon_ns_grouped``)."""
    p = ns_params(steps, coeffs, eps, iter_dtype, dtype_code(Gs[0]), 0)
    return _ns_grouped(STANDARD, Gs, outs, p, workspace, flags)


def gram_ns_grouped(Gs, *, steps: int = DEFAULT_STEPS, coeffs=None, eps: float = DEFAULT_EPS,
                    iter_dtype: Optional[int] = None, restart_mask: int = STABILIZED_RESTART_MASK,
                    outs=None, workspace=None, flags=None):
    """Gram Newton-Schulz of several batches of different shapes (C ABI ``gram_ns_grouped``)."""
    p = ns_params(steps, coeffs, eps, iter_dtype, dtype_code(Gs[0]), restart_mask)
    return _ns_grouped(GRAM, Gs, outs, p, workspace, flags)


def muon_step_grouped(Ws, Gs, Ms, *, lr: float, momentum: float, weight_decay: float,
                      scale_coeff: float = 0.2, nesterov: bool = False, variant: int = GRAM,
                      steps: int = DEFAULT_STEPS, coeffs=None, eps: float = DEFAULT_EPS,
                      iter_dtype: Optional[int] = None, restart_mask: int = STABILIZED_RESTART_MASK,
                      U_outs=None, workspace=None, flags=None):
    """One fused Muon step over several batches of different shapes (C ABI
    ``muon_step_grouped``); every W and M is updated in place."""
    torch = _torch()
    what = "muon_step_grouped"
    for name, ts in (("Ws", Ws), ("Ms", Ms), ("U_outs", U_outs)):
        if ts is not None and len(ts) != len(Gs):
            raise ValueError(f"{what}: {name} has {len(ts)} entries for {len(Gs)} groups")
    for i, G in enumerate(Gs):
        _check_same_shape(what, G, **{f"Ws[{i}]": Ws[i], f"Ms[{i}]": Ms[i],
                                      f"U_outs[{i}]": U_outs[i] if U_outs is not None else None})
        if Ms[i].dtype != torch.float32:
            raise TypeError(f"{what}: Ms[{i}] must be float32, got {Ms[i].dtype}")
    _check_groups(what, Gs, flags, workspace, Ws=Ws, Ms=Ms, U_outs=U_outs)
    p = ns_params(steps, coeffs, eps, iter_dtype, dtype_code(Gs[0]),
                  restart_mask if variant == GRAM else 0)
    sp = MnsStepParams(lr, momentum, weight_decay, scale_coeff, 1 if nesterov else 0, variant)
    if workspace is None:
        workspace = torch.empty(workspace_bytes_grouped(variant, Gs, p), dtype=torch.uint8,
                                device=Gs[0].device)
    fptr = ctypes.c_void_p(flags.data_ptr()) if flags is not None else None
    u = _tensor_array(U_outs) if U_outs is not None else None
    _check(_lib().muon_step_grouped(len(Gs), _tensor_array(Ws), _tensor_array(Gs), _tensor_array(Ms),
                                    u, ctypes.byref(sp), ctypes.byref(p),
                                    ctypes.c_void_p(workspace.data_ptr()), _ws_bytes(workspace), fptr,
                                    _stream_ptr(Gs[0])), what)
    return Ws


# ------------------------------------------------------------------ AdamW (hybrid optimizer)
class MnsAdamwParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32),
                ("bias_correction", ctypes.c_int32)]


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, lr: float, beta1: float = 0.9,
               beta2: float = 0.95, eps: float = 1e-8, weight_decay: float = 0.1, step: int = 1,
               bias_correction: bool = False):
    """One AdamW step over lists of contiguous tensors (C ABI ``adamw_step``); params and both
    fp32 moments are updated in place."""
    torch = _torch()
    n = len(params)
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == n) or n == 0:
        raise ValueError("params, grads and moments must be non-empty lists of equal length")
    pdt = params[0].dtype
    for i, (p_, g_, m_, v_) in enumerate(zip(params, grads, exp_avgs, exp_avg_sqs)):
        if p_.dtype != pdt:
            raise TypeError(f"adamw_step: params[{i}] is {p_.dtype}; every parameter must be {pdt}")
        if g_.dtype != pdt:
            raise TypeError(f"adamw_step: grads[{i}] is {g_.dtype}, its parameter is {pdt}")
        if m_.dtype != torch.float32 or v_.dtype != torch.float32:
            raise TypeError(f"adamw_step: the moments of tensor {i} must be float32")
        if not (p_.numel() == g_.numel() == m_.numel() == v_.numel()):
            raise ValueError("each parameter, gradient and moment pair must have equal sizes")
    for group in (params, grads, exp_avgs, exp_avg_sqs):
        for t in group:
            if not t.is_contiguous():
                raise ValueError("AdamW tensors must be contiguous")
    named = {}
    for i in range(n):
        named.update({f"params[{i}]": params[i], f"grads[{i}]": grads[i],
                      f"exp_avgs[{i}]": exp_avgs[i], f"exp_avg_sqs[{i}]": exp_avg_sqs[i]})
    _check_device("adamw_step", params[0], **named)
    arr = lambda ts: (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])
    numels = (ctypes.c_int64 * n)(*[t.numel() for t in params])
    ap = MnsAdamwParams(lr, beta1, beta2, eps, weight_decay, step, 1 if bias_correction else 0)
    _check(_lib().adamw_step(n, arr(params), arr(grads), arr(exp_avgs), arr(exp_avg_sqs), numels,
                             dtype_code(params[0]), ctypes.byref(ap), _stream_ptr(params[0])),
           "adamw_step")
    return params


def hybrid_step(matrix_groups, vector_params, *, muon: dict, adamw: dict):
    """The hybrid optimizer step: Muon for the 2-D matrices (``matrix_groups``: list of
    (W, G, M) batches, one grouped call) and AdamW for everything else (``vector_params``:
    list of (param, grad, exp_avg, exp_avg_sq)), enqueued on the current stream."""
    if matrix_groups:
        Ws, Gs, Ms = (list(x) for x in zip(*matrix_groups))
        muon_step_grouped(Ws, Gs, Ms, **muon)
    if vector_params:
        ps, gs, ms, vs = (list(x) for x in zip(*vector_params))
        adamw_step(ps, gs, ms, vs, **adamw)


def gram_trace(G, *, steps: int = DEFAULT_STEPS, coeffs=None, eps: float = DEFAULT_EPS,
               iter_dtype: Optional[int] = None, restart_mask: int = STABILIZED_RESTART_MASK):
    """(O, trace) for the first matrix of G: the Gram iterate after each step 1 .. K-1 as a
    [K-1, n, n] fp32 tensor (C ABI ``gram_ns_trace``)."""
    torch = _torch()
    _check_device("gram_ns_trace", G)
    G1 = G[0] if G.dim() == 3 else G
    p = ns_params(steps, coeffs, eps, iter_dtype, dtype_code(G1), restart_mask)
    n = min(G1.shape)
    out = torch.empty_like(G1)
    trace = torch.empty(steps - 1, n, n, dtype=torch.float32, device=G1.device)
    ws = _workspace(GRAM, G1, p, None)
    _check(_lib().gram_ns_trace(ctypes.byref(describe(G1)), ctypes.byref(describe(out)),
                                 ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), _ws_bytes(ws),
                                 ctypes.c_void_p(trace.data_ptr()), _stream_ptr(G1)),
           "gram_ns_trace")
    return out, trace


# ------------------------------------------------------------------ launch timing

def timing_enable(on: bool = True):
    _check(_lib().mns_timing_enable(1 if on else 0), "mns_timing_enable")


def timing_reset():
    _check(_lib().mns_timing_reset(), "mns_timing_reset")


def timing_query() -> dict:
    """{kind_name: (total_ms, launches)} over the events recorded since the last reset."""
    L = _lib()
    out = {}
    for k in range(L.mns_timing_kinds()):
        ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
        _check(L.mns_timing_query(k, ctypes.byref(ms), ctypes.byref(n)), "mns_timing_query")
        out[L.mns_kernel_kind_name(k).decode()] = (ms.value, n.value)
    return out
