"""Causal kernelized linear attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``liblinattn.so`` (declared in
``include/la.h``).  It only marshals arguments: checks dtypes, shapes and
contiguity, allocates outputs and the workspace with PyTorch, and passes raw
device pointers and the current HIP stream to the library.  Every step of
the computation runs in the library's HIP kernels; there is no fallback, and
a missing library raises an error.

    forward(Q, K, V, phi="elu1", causal=True, chunk=64, ...)  -> O [, S_N, z_N]
    decode_step(S, z, q, k, v, phi="elu1", ...)               -> o (S, z updated)
    feature_map(X, phi="elu1", ...)                           -> Phi (fp32)
"""

from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "la.h")

LA_F32, LA_BF16 = 0, 1
# "favor_precise": FAVOR+ whose prefill output pass projects with omega in
# bf16 hi + lo (for inputs of large norm; la.h, LA_PHI_FAVOR_PRECISE)
PHI = {"elu1": 0, "favor": 1, "identity": 2, "favor_precise": 3}
FAVOR = ("favor", "favor_precise")
LA_FORWARD_KERNELS = 3
LA_BACKWARD_KERNELS = 5
STATUS = {0: "LA_OK", 1: "LA_ERR_NULL", 2: "LA_ERR_SHAPE", 3: "LA_ERR_UNSUPPORTED",
          4: "LA_ERR_ALIGN", 5: "LA_ERR_WORKSPACE", 6: "LA_ERR_HIP", 7: "LA_ERR_SCRATCH"}

_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_SIGS = {
    "la_set_span_tokens": (_i, [_i]),
    "la_get_span_tokens": (_i, []),
    "la_forward_workspace_bytes": (ctypes.c_size_t, [_i] * 10),
    "la_forward_config": (_i, [_i] * 10 + [ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "la_forward": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5 + [ctypes.c_size_t, _vp]),
    "la_forward_timed": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5 + [ctypes.c_size_t, _vp, _vp]),
    "la_forward_noalloc": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5),
    "la_decode_step": (_i, [_vp] * 8 + [_i] * 7 + [_vp, _vp]),
    "la_forward_decay_config": (_i, [_i] * 9 + [ctypes.POINTER(_i)]),
    "la_forward_decay": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5 + [ctypes.c_size_t, _vp]),
    "la_forward_decay_timed": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5 + [ctypes.c_size_t, _vp, _vp]),
    "la_decode_step_decay": (_i, [_vp] * 8 + [_i] * 7 + [_vp, _i, _vp]),
    "la_forward_gated_workspace_bytes": (ctypes.c_size_t, [_i] * 9),
    "la_forward_gated_config": (_i, [_i] * 9 + [ctypes.POINTER(_i)]),
    "la_forward_gated": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5 + [ctypes.c_size_t, _vp]),
    "la_forward_gated_timed": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5 + [ctypes.c_size_t, _vp, _vp]),
    "la_decode_step_gated": (_i, [_vp] * 8 + [_i] * 7 + [_vp, _i, _vp]),
    "la_backward_workspace_bytes": (ctypes.c_size_t, [_i] * 9),
    "la_backward_config": (_i, [_i] * 9 + [ctypes.POINTER(_i)]),
    "la_backward": (_i, [_vp] * 8 + [_i] * 9 + [_vp, ctypes.c_size_t, _vp]),
    "la_backward_timed": (_i, [_vp] * 8 + [_i] * 9 + [_vp, ctypes.c_size_t, _vp, _vp]),
    "la_forward_gla_workspace_bytes": (ctypes.c_size_t, [_i] * 9),
    "la_forward_gla_config": (_i, [_i] * 9 + [ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "la_forward_gla": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5 + [ctypes.c_size_t, _vp]),
    "la_forward_gla_timed": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _i, _i] + [_vp] * 5 + [ctypes.c_size_t, _vp, _vp]),
    "la_decode_step_gla": (_i, [_vp] * 8 + [_i] * 7 + [_vp, _i, _vp]),
    "la_feature_map": (_i, [_vp, _vp, ctypes.c_longlong, _i, _i, _i, _i, _vp, _vp]),
    "la_status_string": (ctypes.c_char_p, [_i]),
    "la_version": (_i, []),
    "la_hip_error_string": (ctypes.c_char_p, []),
    "la_event_create": (_i, [ctypes.POINTER(_vp)]),
    "la_event_destroy": (_i, [_vp]),
    "la_event_elapsed_ms": (_i, [_vp, _vp, ctypes.POINTER(ctypes.c_float)]),
}


class LinAttnError(RuntimeError):
    """A non-zero la_status from the library."""

    def __init__(self, status, where):
        self.status = status
        detail = status_string(status)
        if status == 6:
            detail += ": " + load_library().la_hip_error_string().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")


def load_library(path=None):
    """Load liblinattn.so (built by ``build.py``).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m kernelized_linear_attention_elu_amd.build` "
            "(there is no non-HIP fallback)")
    # PyTorch ships its own HIP runtime and links it by a different file name
    # than the system one this library was linked against.  Loading torch
    # first lets the library bind to the runtime already in the process;
    # the other order would put two HIP/HSA runtimes in one process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions():
    """Names of the functions declared in include/la.h."""
    with open(HEADER_PATH, encoding="utf-8") as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_\w+)\s*\(", text)))


def status_string(status):
    return load_library().la_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise LinAttnError(status, where)


# ------------------------------------------------------------------ torch marshalling

def _torch():
    import torch
    return torch


def _io_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _omega_rows(omega, phi, d):
    """Feature count r: omega's rows for FAVOR+ (omega must be [r, d]), else d."""
    if phi not in FAVOR:
        return d
    if omega is None or omega.dim() != 2 or omega.shape[1] != d:
        raise ValueError(f"FAVOR+ needs omega of shape [r, {d}], got "
                         f"{None if omega is None else tuple(omega.shape)}")
    return omega.shape[0]


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def set_span_tokens(tokens):
    """Process-wide span length of the chunkwise prefill (tokens, a multiple of
    16; 0 restores the library's own choice): la_set_span_tokens."""
    _check(load_library().la_set_span_tokens(int(tokens or 0)), "la_set_span_tokens")


def workspace_bytes(B, H, N, d, dv, io="bf16", phi="elu1", r=0, causal=True, chunk=64, gated=False, gla=False):
    """Workspace bytes of la_forward (la_forward_gated with ``gated``,
    la_forward_gla with ``gla``; the decay call needs no more than
    la_forward's causal size)."""
    io_code = LA_BF16 if io == "bf16" else LA_F32
    if gla:
        return int(load_library().la_forward_gla_workspace_bytes(B, H, N, d, dv, io_code, PHI[phi], r, chunk))
    if gated:
        return int(load_library().la_forward_gated_workspace_bytes(B, H, N, d, dv, io_code, PHI[phi], r, chunk))
    return int(load_library().la_forward_workspace_bytes(B, H, N, d, dv, io_code, PHI[phi], r, int(causal), chunk))


def forward_config(B, H, N, d, dv, io="bf16", phi="elu1", r=0, causal=True, chunk=64, decay=False, gated=False,
                   gla=False):
    """(n_span, single_pass) that la_forward (la_forward_decay with
    ``decay``, la_forward_gated with ``gated``, la_forward_gla with ``gla``)
    uses for this shape."""
    io_code = LA_BF16 if io == "bf16" else LA_F32
    n, sp = ctypes.c_int(), ctypes.c_int()
    if gla:
        _check(load_library().la_forward_gla_config(B, H, N, d, dv, io_code, PHI[phi], r, chunk, ctypes.byref(n),
                                                    ctypes.byref(sp)), "la_forward_gla_config")
        return n.value, False
    if gated:
        _check(load_library().la_forward_gated_config(B, H, N, d, dv, io_code, PHI[phi], r, chunk, ctypes.byref(n)),
               "la_forward_gated_config")
        return n.value, False
    if decay:
        _check(load_library().la_forward_decay_config(B, H, N, d, dv, io_code, PHI[phi], r, chunk, ctypes.byref(n)),
               "la_forward_decay_config")
        return n.value, False
    _check(load_library().la_forward_config(B, H, N, d, dv, io_code, PHI[phi], r, int(causal), chunk,
                                            ctypes.byref(n), ctypes.byref(sp)), "la_forward_config")
    return n.value, bool(sp.value)


def _gamma_arg(gamma, H, dev, causal=True):
    """Per-head decay: a fp32 device tensor of H values (or None)."""
    if gamma is None:
        return None
    torch = _torch()
    if not causal:
        raise ValueError("the decay is defined for the causal form only")
    _require(gamma, "gamma", torch.float32, dev)
    if tuple(gamma.shape) != (H,):
        raise ValueError(f"gamma must have shape ({H},), got {tuple(gamma.shape)}")
    return gamma


def _log_gate_arg(log_gate, shape, dev, causal=True, name="log_gate"):
    """Per-token gates: a fp32 device tensor of natural-log gates (or None)."""
    if log_gate is None:
        return None
    torch = _torch()
    if not causal:
        raise ValueError("the gates are defined for the causal form only")
    _require(log_gate, name, torch.float32, dev)
    if tuple(log_gate.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(log_gate.shape)}")
    return log_gate


def forward(Q, K, V, *, phi="elu1", omega=None, causal=True, chunk=64, S0=None, z0=None,
            return_state=False, out=None, workspace=None, events=None, gamma=None, normalize=True,
            log_gate=None, log_gate_ch=None):
    """Causal (or non-causal) linear attention over Q, K [B,H,N,d], V [B,H,N,dv].

    Returns O [B,H,N,dv] (same dtype as Q); with ``return_state`` also the
    final state S_N [B,H,r,dv] and z_N [B,H,r] (fp32).  ``S0``/``z0`` give an
    initial state.  ``events``: optional list of 2*LA_FORWARD_KERNELS event
    handles from :func:`event_create` recorded around the library's kernels.
    ``gamma``: optional fp32 device tensor [H] of per-head decays in (0, 1]
    (causal only; la_forward_decay), with ``normalize=False`` for the
    unnormalised read-out.  ``log_gate``: optional fp32 device tensor
    [B,H,N] of per-token natural-log gates log a_t (causal only;
    la_forward_gated), likewise with ``normalize``.  ``log_gate_ch``:
    optional fp32 device tensor [B,H,N,r] of per-token, per-key-channel
    natural-log gates (causal only; la_forward_gla).
    """
    torch = _torch()
    lib = load_library()
    if Q.dim() != 4 or K.dim() != 4 or V.dim() != 4:
        raise ValueError("Q, K, V must be [B, H, N, d]")
    B, H, N, d = Q.shape
    dv = V.shape[-1]
    if K.shape != Q.shape or V.shape[:3] != Q.shape[:3]:
        raise ValueError("shape mismatch between Q, K, V")
    dev = Q.device
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _require(t, name, Q.dtype, dev)
    io = _io_code(Q)
    _require(omega, "omega", torch.float32, dev)
    r = _omega_rows(omega, phi, d)
    if (S0 is None) != (z0 is None):
        raise ValueError("give both S0 and z0 or neither")
    _require(S0, "S0", torch.float32, dev)
    _require(z0, "z0", torch.float32, dev)
    if S0 is not None and (tuple(S0.shape) != (B, H, r, dv) or tuple(z0.shape) != (B, H, r)):
        raise ValueError("S0 must be [B,H,r,dv] and z0 [B,H,r]")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=Q.dtype, device=dev)
    _require(out, "out", Q.dtype, dev)
    if tuple(out.shape) != (B, H, N, dv):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, N, dv)}")
    S_out = z_out = None
    if return_state:
        S_out = torch.empty((B, H, r, dv), dtype=torch.float32, device=dev)
        z_out = torch.empty((B, H, r), dtype=torch.float32, device=dev)
    gamma = _gamma_arg(gamma, H, dev, causal)
    log_gate = _log_gate_arg(log_gate, (B, H, N), dev, causal)
    log_gate_ch = _log_gate_arg(log_gate_ch, (B, H, N, r), dev, causal, name="log_gate_ch")
    n_decay = sum(x is not None for x in (gamma, log_gate, log_gate_ch))
    if n_decay > 1:
        raise ValueError("give at most one of gamma, log_gate, log_gate_ch")
    if n_decay == 0 and not normalize:
        raise ValueError("normalize=False is available with a decay (gamma, log_gate or log_gate_ch) only")
    if n_decay and phi in FAVOR:
        raise ValueError("the decay is available for the pointwise feature maps only")
    if log_gate_ch is not None:
        need = int(lib.la_forward_gla_workspace_bytes(B, H, N, d, dv, io, PHI[phi], r, chunk))
    elif log_gate is not None:
        need = int(lib.la_forward_gated_workspace_bytes(B, H, N, d, dv, io, PHI[phi], r, chunk))
    else:
        need = int(lib.la_forward_workspace_bytes(B, H, N, d, dv, io, PHI[phi], r, int(causal), chunk))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    tail = [chunk, _ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(dev)]
    head = [_ptr(Q), _ptr(K), _ptr(V), _ptr(out), B, H, N, d, dv, io, PHI[phi], r]
    if log_gate_ch is not None:
        args = head + [_ptr(log_gate_ch), int(bool(normalize))] + tail
        fn, name = ((lib.la_forward_gla, "la_forward_gla") if events is None
                    else (lib.la_forward_gla_timed, "la_forward_gla_timed"))
    elif log_gate is not None:
        args = head + [_ptr(log_gate), int(bool(normalize))] + tail
        fn, name = ((lib.la_forward_gated, "la_forward_gated") if events is None
                    else (lib.la_forward_gated_timed, "la_forward_gated_timed"))
    elif gamma is None:
        args = head + [_ptr(omega), int(causal)] + tail
        fn, name = (lib.la_forward, "la_forward") if events is None else (lib.la_forward_timed, "la_forward_timed")
    else:
        args = head + [_ptr(gamma), int(bool(normalize))] + tail
        fn, name = ((lib.la_forward_decay, "la_forward_decay") if events is None
                    else (lib.la_forward_decay_timed, "la_forward_decay_timed"))
    if events is None:
        _check(fn(*args), name)
    else:
        arr = (ctypes.c_void_p * (2 * LA_FORWARD_KERNELS))(*events)
        _check(fn(*args, arr), name)
    if return_state:
        return out, S_out, z_out
    return out


def forward_noalloc(Q, K, V, *, phi="elu1", omega=None, causal=True, chunk=64, S0=None, z0=None,
                    return_state=False, out=None):
    """la_forward_noalloc: the same result as :func:`forward`, computed with
    the library's fixed per-GPU scratch instead of a workspace (the entry
    point allocates nothing; this binding allocates ``out`` and the returned
    state through torch unless they are given)."""
    torch = _torch()
    lib = load_library()
    if Q.dim() != 4 or K.dim() != 4 or V.dim() != 4:
        raise ValueError("Q, K, V must be [B, H, N, d]")
    B, H, N, d = Q.shape
    dv = V.shape[-1]
    if K.shape != Q.shape or V.shape[:3] != Q.shape[:3]:
        raise ValueError("shape mismatch between Q, K, V")
    dev = Q.device
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _require(t, name, Q.dtype, dev)
    io = _io_code(Q)
    _require(omega, "omega", torch.float32, dev)
    r = _omega_rows(omega, phi, d)
    if (S0 is None) != (z0 is None):
        raise ValueError("give both S0 and z0 or neither")
    _require(S0, "S0", torch.float32, dev)
    _require(z0, "z0", torch.float32, dev)
    if S0 is not None and (tuple(S0.shape) != (B, H, r, dv) or tuple(z0.shape) != (B, H, r)):
        raise ValueError("S0 must be [B,H,r,dv] and z0 [B,H,r]")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=Q.dtype, device=dev)
    _require(out, "out", Q.dtype, dev)
    if tuple(out.shape) != (B, H, N, dv):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, N, dv)}")
    S_out = z_out = None
    if return_state:
        S_out = torch.empty((B, H, r, dv), dtype=torch.float32, device=dev)
        z_out = torch.empty((B, H, r), dtype=torch.float32, device=dev)
    _check(lib.la_forward_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), B, H, N, d, dv, io, PHI[phi], r,
                                  _ptr(omega), int(causal), chunk, _ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out),
                                  _stream(dev)), "la_forward_noalloc")
    if return_state:
        return out, S_out, z_out
    return out


def backward(Q, K, V, O, dO, *, phi="elu1", chunk=64, out=None, workspace=None, events=None):
    """Gradients (dQ, dK, dV) of sum(dO * O) for the causal normalised output
    O = forward(Q, K, V, phi=phi) (la_backward; bf16, d = d_v in {64, 128}).  ``out``:
    optional (dQ, dK, dV) tensors to fill.  ``events``: optional list of
    2*LA_BACKWARD_KERNELS event handles."""
    torch = _torch()
    lib = load_library()
    if Q.dim() != 4:
        raise ValueError("Q, K, V, O, dO must be [B, H, N, d]")
    B, H, N, d = Q.shape
    dv = V.shape[-1]
    dev = Q.device
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O), ("dO", dO)):
        _require(t, name, Q.dtype, dev)
    if K.shape != Q.shape or V.shape[:3] != Q.shape[:3] or O.shape != V.shape or dO.shape != V.shape:
        raise ValueError("shape mismatch between Q, K, V, O, dO")
    io = _io_code(Q)
    if out is None:
        out = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    dQ, dK, dV = out
    for name, t, ref in (("dQ", dQ, Q), ("dK", dK, K), ("dV", dV, V)):
        _require(t, name, Q.dtype, dev)
        if t.shape != ref.shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")
    need = int(lib.la_backward_workspace_bytes(B, H, N, d, dv, io, PHI[phi], 0, chunk))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    args = [_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), B, H, N, d, dv, io,
            PHI[phi], 0, chunk, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)]
    if events is None:
        _check(lib.la_backward(*args), "la_backward")
    else:
        arr = (ctypes.c_void_p * (2 * LA_BACKWARD_KERNELS))(*events)
        _check(lib.la_backward_timed(*args, arr), "la_backward_timed")
    return dQ, dK, dV


def decode_step(S, z, q, k, v, *, phi="elu1", omega=None, inplace=True, out=None, gamma=None, normalize=True,
                log_gate=None, log_gate_ch=None):
    """One decode step for every (batch, head): S, z updated in place (or new
    tensors when ``inplace=False``).  Returns o, or (o, S_new, z_new).
    ``gamma``: optional fp32 device tensor [H] of per-head decays
    (la_decode_step_decay), with ``normalize=False`` for o = phi(q)^T S'.
    ``log_gate``: optional fp32 device tensor [B,H], this token's natural-log
    gate per sequence and head (la_decode_step_gated).  ``log_gate_ch``:
    optional fp32 device tensor [B,H,r], this token's natural-log gates per
    key channel (la_decode_step_gla)."""
    torch = _torch()
    lib = load_library()
    B, H, d = q.shape
    dv = v.shape[-1]
    r = S.shape[-2]
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, q.dtype, dev)
    _require(S, "S", torch.float32, dev)
    _require(z, "z", torch.float32, dev)
    _require(omega, "omega", torch.float32, dev)
    if _omega_rows(omega, phi, d) != r:
        raise ValueError(f"S has {r} feature rows; phi={phi} gives {_omega_rows(omega, phi, d)}")
    if (tuple(S.shape) != (B, H, r, dv) or tuple(z.shape) != (B, H, r) or tuple(k.shape) != (B, H, d)
            or tuple(v.shape) != (B, H, dv)):
        raise ValueError("decode shapes: S [B,H,r,dv], z [B,H,r], q,k [B,H,d], v [B,H,dv]")
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    _require(out, "out", q.dtype, dev)
    if tuple(out.shape) != (B, H, dv):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, dv)}")
    gamma = _gamma_arg(gamma, H, dev)
    log_gate = _log_gate_arg(log_gate, (B, H), dev)
    log_gate_ch = _log_gate_arg(log_gate_ch, (B, H, r), dev, name="log_gate_ch")
    n_decay = sum(x is not None for x in (gamma, log_gate, log_gate_ch))
    if n_decay > 1:
        raise ValueError("give at most one of gamma, log_gate, log_gate_ch")
    if n_decay == 0 and not normalize:
        raise ValueError("normalize=False is available with a decay (gamma, log_gate or log_gate_ch) only")
    S_new, z_new = (S, z) if inplace else (torch.empty_like(S), torch.empty_like(z))
    if log_gate_ch is not None:
        st = lib.la_decode_step_gla(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S_new),
                                    _ptr(z_new), B, H, d, dv, _io_code(q), PHI[phi], r, _ptr(log_gate_ch),
                                    int(bool(normalize)), _stream(dev))
        _check(st, "la_decode_step_gla")
    elif log_gate is not None:
        st = lib.la_decode_step_gated(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S_new),
                                      _ptr(z_new), B, H, d, dv, _io_code(q), PHI[phi], r, _ptr(log_gate),
                                      int(bool(normalize)), _stream(dev))
        _check(st, "la_decode_step_gated")
    elif gamma is None:
        st = lib.la_decode_step(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S_new),
                                _ptr(z_new), B, H, d, dv, _io_code(q), PHI[phi], r, _ptr(omega), _stream(dev))
        _check(st, "la_decode_step")
    else:
        st = lib.la_decode_step_decay(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S_new),
                                      _ptr(z_new), B, H, d, dv, _io_code(q), PHI[phi], r, _ptr(gamma),
                                      int(bool(normalize)), _stream(dev))
        _check(st, "la_decode_step_decay")
    return out if inplace else (out, S_new, z_new)


def feature_map(X, *, phi="elu1", omega=None, out=None):
    """phi applied to the rows of X [..., d]; returns fp32 [..., r] (written
    into ``out`` when given: contiguous fp32 of that shape on X's device)."""
    torch = _torch()
    lib = load_library()
    d = X.shape[-1]
    rows = X.numel() // d if d else 0
    _require(X, "X", X.dtype, X.device)
    _require(omega, "omega", torch.float32, X.device)
    r = _omega_rows(omega, phi, d)
    shape = tuple(X.shape[:-1]) + (r,)
    if out is None:
        Y = torch.empty(shape, dtype=torch.float32, device=X.device)
    else:
        _require(out, "out", torch.float32, X.device)
        if tuple(out.shape) != shape:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
        Y = out
    st = lib.la_feature_map(_ptr(X), _ptr(Y), rows, d, _io_code(X), PHI[phi], r, _ptr(omega), _stream(X.device))
    _check(st, "la_feature_map")
    return Y


def event_create():
    ev = ctypes.c_void_p()
    _check(load_library().la_event_create(ctypes.byref(ev)), "la_event_create")
    return ev.value


def event_destroy(ev):
    _check(load_library().la_event_destroy(ev), "la_event_destroy")


def event_elapsed_ms(a, b):
    ms = ctypes.c_float()
    _check(load_library().la_event_elapsed_ms(a, b, ctypes.byref(ms)), "la_event_elapsed_ms")
    return ms.value
