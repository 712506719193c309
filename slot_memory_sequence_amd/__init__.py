"""libgsa: Gated Slot Attention / gated linear attention on MI355X (gfx950).

Thin Python binding over the C ABI declared in ``include/gsa.h``.  It only
marshals arguments (device pointers, sizes, the current HIP stream) and
allocates outputs/workspace through PyTorch; every step of the computation
runs in the library's HIP kernels.  There is no CPU fallback: if the built
library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

# Load PyTorch's HIP runtime first: libgsa links libamdhip64.so.7 by soname, so
# the process then holds exactly one HIP runtime and torch's streams, events
# and allocations are valid handles for the library.
import torch as _torch_rt  # noqa: F401

__all__ = ["lib", "gsa_fwd", "gsa_fwd_varlen", "gla_fwd", "gsa_decode_step", "gla_decode_step",
           "GsaError", "LIB_PATH",
           "NONLINEARITIES", "gsa_fwd_varlen_workspace_bytes",
           "gsa_fwd_supported", "gla_fwd_supported", "gsa_decode_supported",
           "gsa_fwd_workspace_bytes", "gla_fwd_workspace_bytes", "status_string",
           "gsa_bwd", "gsa_bwd_varlen", "gsa_autograd", "gsa_fwd_train", "gsa_bwd_train",
           "gsa_train_states_bytes", "gsa_train_supported"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsa.so")
DTYPE_F32, DTYPE_BF16 = 0, 1
# gsa_slot_nonlinearity codes: the softmax read of GSA and the element-wise
# ablations (none, Swish, ReLU, ReLU^2)
NONLINEARITIES = {"softmax": 0, "identity": 1, "swish": 2, "relu": 3, "relu2": 4}
# gsa_gate_input codes of gla_fwd_ex: logits, or per-token log-decays given directly
GATE_INPUTS = {"logit": 0, "log_decay": 1}

if not os.path.exists(LIB_PATH):
    raise ImportError("libgsa.so is not built (run __graft_entry__.build() or "
                      "python slot_memory_sequence_amd/build.py): " + LIB_PATH)

_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
lib = ctypes.CDLL(LIB_PATH)
lib.gsa_abi_version.restype = _I
lib.gsa_status_string.restype = ctypes.c_char_p
lib.gsa_status_string.argtypes = [_I]
lib.gsa_fwd_supported.argtypes = [_I] * 5
lib.gla_fwd_supported.argtypes = [_I] * 4
lib.gsa_decode_supported.argtypes = [_I] * 4
lib.gsa_fwd_workspace_bytes.restype = _S
lib.gsa_fwd_workspace_bytes.argtypes = [_I] * 9
lib.gla_fwd_workspace_bytes.restype = _S
lib.gla_fwd_workspace_bytes.argtypes = [_I] * 8
lib.gsa_fwd.restype = _I
lib.gsa_fwd.argtypes = [_P] * 9 + [_I] * 7 + [_F, _I, _P, _S, _I, _P]
lib.gla_fwd.restype = _I
lib.gla_fwd.argtypes = [_P] * 7 + [_I] * 6 + [_F, _I, _P, _S, _I, _P]
lib.gsa_fwd_events.restype = _I
lib.gsa_fwd_events.argtypes = [_P] * 9 + [_I] * 7 + [_F, _I, _P, _S, _I, _P, _P]
lib.gla_fwd_events.restype = _I
lib.gla_fwd_events.argtypes = [_P] * 7 + [_I] * 6 + [_F, _I, _P, _S, _I, _P, _P]
lib.gsa_decode_step.restype = _I
lib.gsa_decode_step.argtypes = [_P] * 7 + [_I] * 5 + [_F, _I, _P]
lib.gsa_decode_step_events.restype = _I
lib.gsa_decode_step_events.argtypes = [_P] * 7 + [_I] * 5 + [_F, _I, _P, _P]
lib.gsa_fwd_ex.restype = _I
lib.gsa_fwd_ex.argtypes = [_P] * 9 + [_I] * 7 + [_F, _I, _P, _S, _I, _I, _P, _P]
lib.gsa_decode_step_ex.restype = _I
lib.gla_fwd_ex.restype = _I
lib.gla_fwd_ex.argtypes = [_P] * 7 + [_I] * 6 + [_F, _I, _P, _S, _I, _I, _P, _P]
lib.gla_decode_supported.argtypes = [_I] * 3
lib.gla_decode_step.restype = _I
lib.gla_decode_step.argtypes = [_P] * 6 + [_I] * 4 + [_F, _I, _I, _P, _P]
lib.gsa_measure_hbm.restype = _I
lib.gsa_measure_hbm.argtypes = [_P, _P, _S, _I, _P, _P]
lib.gsa_measure_mfma_bf16.restype = _I
lib.gsa_measure_mfma_bf16.argtypes = [_P, _S, _I, ctypes.POINTER(ctypes.c_double), _P, _P]
MEASURE_MFMA_WORKGROUPS = 1024
lib.gsa_fwd_varlen.restype = _I
lib.gsa_fwd_varlen.argtypes = [_P] * 5 + [_I, _I] + [_P] * 5 + [_I] * 4 + [_F, _I, _P, _S, _I, _P, _P]
lib.gsa_fwd_varlen_workspace_bytes.restype = _S
lib.gsa_fwd_varlen_workspace_bytes.argtypes = [_P] + [_I] * 8
lib.gsa_decode_step_ex.argtypes = [_P] * 7 + [_I] * 5 + [_F, _I, _I, _P, _P]
lib.gsa_bwd_supported.argtypes = [_I] * 4
lib.gsa_bwd_workspace_bytes.argtypes = [_I] * 6
lib.gsa_bwd_workspace_bytes.restype = _S
lib.gsa_bwd_workspace_bytes_ex.argtypes = [_I] * 8
lib.gsa_bwd_workspace_bytes_ex.restype = _S
lib.gsa_bwd.argtypes = [_P] * 15 + [_I] * 6 + [_F, _I, _P, _S, _P, _P]
lib.gsa_bwd_ex.argtypes = [_P] * 15 + [_I] * 6 + [_F, _I, _P, _S, _I, _P, _P]
lib.gsa_bwd_varlen_workspace_bytes.argtypes = [_P] + [_I] * 5
lib.gsa_bwd_varlen_workspace_bytes.restype = _S
lib.gsa_bwd_varlen.argtypes = [_P] * 5 + [_P, _I, _I] + [_P] * 10 + [_I] * 3 + [_F, _I, _P, _S, _P, _P]
lib.gsa_train_states_bytes.restype = _S
lib.gsa_train_states_bytes.argtypes = [_I] * 7
lib.gsa_fwd_train_workspace_bytes.restype = _S
lib.gsa_fwd_train_workspace_bytes.argtypes = [_I] * 7
lib.gsa_fwd_train.restype = _I
lib.gsa_fwd_train.argtypes = [_P] * 9 + [_I] * 6 + [_F, _I, _P, _S, _P, _S, _I, _P, _P]
lib.gsa_bwd_train.restype = _I
lib.gsa_bwd_train.argtypes = [_P] * 15 + [_I] * 6 + [_F, _I, _P, _S, _P, _S, _I, _P, _P]
lib.gsa_fwd_noalloc_scratch_bytes.restype = _S
lib.gsa_fwd_noalloc_scratch_bytes.argtypes = []
lib.gsa_fwd_noalloc.restype = _I
lib.gsa_fwd_noalloc.argtypes = [_P] * 9 + [_I] * 7 + [_F, _I, _I, _I, _P, _P]


class GsaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s: status %d (%s)" % (fn, status, status_string(status)))


def status_string(s: int) -> str:
    return lib.gsa_status_string(int(s)).decode()


def gsa_fwd_supported(dk, dv, m, C=64, dtype=DTYPE_BF16) -> bool:
    return bool(lib.gsa_fwd_supported(dk, dv, m, C, dtype))


def gla_fwd_supported(dk, dv, C=64, dtype=DTYPE_BF16) -> bool:
    return bool(lib.gla_fwd_supported(dk, dv, C, dtype))


def gsa_decode_supported(dk, dv, m, dtype=DTYPE_BF16) -> bool:
    return bool(lib.gsa_decode_supported(dk, dv, m, dtype))


def gsa_fwd_workspace_bytes(B, H, T, dk, dv, m, C=64, dtype=DTYPE_BF16, chunks_per_segment=0):
    return int(lib.gsa_fwd_workspace_bytes(B, H, T, dk, dv, m, C, dtype, chunks_per_segment))


def gla_fwd_workspace_bytes(B, H, T, dk, dv, C=64, dtype=DTYPE_BF16, chunks_per_segment=0):
    return int(lib.gla_fwd_workspace_bytes(B, H, T, dk, dv, C, dtype, chunks_per_segment))


def _cu_array(cu_seqlens):
    """Host int32 offsets [n + 1] as a ctypes array (kept alive by the caller)."""
    vals = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    if len(vals) < 1:
        raise ValueError("cu_seqlens needs at least one entry (0)")
    return (ctypes.c_int * len(vals))(*vals), len(vals) - 1


def gsa_fwd_varlen_workspace_bytes(cu_seqlens, H, dk, dv, m, C=64, dtype=DTYPE_BF16,
                                   chunks_per_segment=0):
    arr, n = _cu_array(cu_seqlens)
    return int(lib.gsa_fwd_varlen_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), n, H, dk, dv,
                                                  m, C, dtype, chunks_per_segment))


# ------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _dt(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError("q/k/v/g must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype=None):
    torch = _torch()
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s" % (name, dtype))


def _shape(t, name, shape):
    """Raise ValueError unless t (nullable) has exactly this shape.  Runs on
    the tensors' metadata only, before anything reaches the library: the C ABI
    takes bare pointers, so a tensor of the wrong shape would otherwise be
    indexed past its end by the kernels."""
    if t is None:
        return
    if not hasattr(t, "shape"):
        raise TypeError("%s must be a tensor" % name)
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(int(x) for x in shape),
                                                          tuple(t.shape)))


def _ndim(t, name, n):
    if not hasattr(t, "shape"):
        raise TypeError("%s must be a tensor" % name)
    if len(t.shape) != n:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, n, tuple(t.shape)))


def _wsbytes(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _events(events, n=4):
    """None, or n raw hipEvent_t handles (ints or None) -> void*[n]."""
    if events is None:
        return None
    if len(events) != n:
        raise ValueError("expected %d event handles, got %d" % (n, len(events)))
    arr = (ctypes.c_void_p * n)(*[None if e is None else int(e) for e in events])
    return ctypes.cast(arr, ctypes.c_void_p)


def _nl(nonlinearity):
    if isinstance(nonlinearity, str):
        if nonlinearity not in NONLINEARITIES:
            raise ValueError("unknown slot non-linearity %r (one of %s)"
                             % (nonlinearity, ", ".join(NONLINEARITIES)))
        return NONLINEARITIES[nonlinearity]
    return int(nonlinearity)  # a raw code; the library validates it


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _fwd_prep(q, k, v, g, k0, v0, out, k_final, v_final, final_state):
    """Shape and dtype checks of a GSA forward's tensors; allocates the
    missing outputs.  Returns ((B, H, T, dk, dv, m), out, k_final, v_final)."""
    torch = _torch()
    _ndim(q, "q", 4)
    B, H, T, dk = q.shape
    _ndim(v, "v", 4)
    _ndim(g, "g", 4)
    dv, m = v.shape[-1], g.shape[-1]
    for n, t, sh in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)), ("g", g, (B, H, T, m)),
                     ("k0", k0, (B, H, m, dk)), ("v0", v0, (B, H, m, dv)), ("out", out, (B, H, T, dv)),
                     ("k_final", k_final, (B, H, m, dk)), ("v_final", v_final, (B, H, m, dv))):
        _shape(t, n, sh)
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g), ("out", out)):
        _check(t, n, q.dtype)
    for n, t in (("k0", k0), ("v0", v0), ("k_final", k_final), ("v_final", v_final)):
        _check(t, n, torch.float32)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state:
        if k_final is None:
            k_final = torch.empty((B, H, m, dk), dtype=torch.float32, device=q.device)
        if v_final is None:
            v_final = torch.empty((B, H, m, dv), dtype=torch.float32, device=q.device)
    return (B, H, T, dk, dv, m), out, k_final, v_final


def gsa_fwd(q, k, v, g, k0=None, v0=None, *, tau=8.0, C=64, final_state=False,
            chunks_per_segment=0, out=None, k_final=None, v_final=None, workspace=None,
            stream=None, events=None, nonlinearity="softmax"):
    """Chunkwise GSA forward.  q, k [B,H,T,dk]; v [B,H,T,dv]; g [B,H,T,m] (gate
    logits); optional float32 initial slot states k0 [B,H,m,dk], v0 [B,H,m,dv].
    nonlinearity: the slot read, "softmax" (GSA) or one of the element-wise
    ablations "identity", "swish", "relu", "relu2".
    Returns (o, k_final, v_final) -- the finals are None unless final_state."""
    torch = _torch()
    (B, H, T, dk, dv, m), out, k_final, v_final = _fwd_prep(q, k, v, g, k0, v0, out, k_final, v_final,
                                                             final_state)
    dt = _dt(q)
    nbytes = gsa_fwd_workspace_bytes(B, H, T, dk, dv, m, C, dt, chunks_per_segment)
    if nbytes == (1 << 64) - 1:
        raise ValueError("invalid problem size")
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    st = lib.gsa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(k0), _ptr(v0), _ptr(out),
                        _ptr(k_final), _ptr(v_final), B, H, T, dk, dv, m, C, float(tau), dt,
                        _ptr(workspace), _wsbytes(workspace),
                        int(chunks_per_segment), _nl(nonlinearity), _stream(stream),
                        _events(events))
    if st:
        raise GsaError("gsa_fwd", st)
    return out, k_final, v_final


def gsa_fwd_noalloc(q, k, v, g, k0=None, v0=None, *, out, k_final=None, v_final=None, tau=8.0,
                    C=64, chunks_per_segment=0, stream=None, events=None, nonlinearity="softmax"):
    """gsa_fwd without a workspace: the scratch space comes from the
    library's fixed per-GPU array (gsa_fwd_noalloc_scratch_bytes() bytes), so
    nothing is allocated, here or in the library -- the caller passes every
    output buffer.  Calls that overlap on one GPU race (they share the
    array).  Returns (out, k_final, v_final)."""
    torch = _torch()
    _ndim(q, "q", 4)
    B, H, T, dk = q.shape
    _ndim(v, "v", 4)
    _ndim(g, "g", 4)
    dv, m = v.shape[-1], g.shape[-1]
    if out is None:
        raise TypeError("out is required (nothing is allocated)")
    for n, t, sh in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)), ("g", g, (B, H, T, m)),
                     ("k0", k0, (B, H, m, dk)), ("v0", v0, (B, H, m, dv)), ("out", out, (B, H, T, dv)),
                     ("k_final", k_final, (B, H, m, dk)), ("v_final", v_final, (B, H, m, dv))):
        _shape(t, n, sh)
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g), ("out", out)):
        _check(t, n, q.dtype)
    for n, t in (("k0", k0), ("v0", v0), ("k_final", k_final), ("v_final", v_final)):
        _check(t, n, torch.float32)
    st = lib.gsa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(k0), _ptr(v0), _ptr(out),
                             _ptr(k_final), _ptr(v_final), B, H, T, dk, dv, m, C, float(tau), _dt(q),
                             int(chunks_per_segment), _nl(nonlinearity), _stream(stream),
                             _events(events))
    if st:
        raise GsaError("gsa_fwd_noalloc", st)
    return out, k_final, v_final


def gsa_fwd_varlen(q, k, v, g, cu_seqlens, k0=None, v0=None, *, tau=8.0, C=64,
                   final_state=False, chunks_per_segment=0, out=None, k_final=None,
                   v_final=None, workspace=None, stream=None, events=None):
    """GSA forward over a packed batch of variable-length sequences.  q, k
    [H,total,dk]; v [H,total,dv]; g [H,total,m] (bf16, head-major packed);
    cu_seqlens: host offsets [n+1] (list, numpy or CPU tensor), cu[0] = 0;
    optional float32 initial states k0 [n,H,m,dk], v0 [n,H,m,dv].
    Returns (o [H,total,dv], k_final, v_final) -- finals None unless
    final_state; they are the decode states of gsa_decode_step."""
    torch = _torch()
    _ndim(q, "q", 3)
    H, total, dk = q.shape
    _ndim(v, "v", 3)
    _ndim(g, "g", 3)
    dv, m = v.shape[-1], g.shape[-1]
    arr, n = _cu_array(cu_seqlens)
    if arr[n] != total:
        raise ValueError("cu_seqlens[-1] = %d but the arrays hold %d tokens" % (arr[n], total))
    for nm, t, sh in (("k", k, (H, total, dk)), ("v", v, (H, total, dv)), ("g", g, (H, total, m)),
                      ("k0", k0, (n, H, m, dk)), ("v0", v0, (n, H, m, dv)), ("out", out, (H, total, dv)),
                      ("k_final", k_final, (n, H, m, dk)), ("v_final", v_final, (n, H, m, dv))):
        _shape(t, nm, sh)
    for nm, t in (("q", q), ("k", k), ("v", v), ("g", g), ("out", out)):
        _check(t, nm, q.dtype)
    for nm, t in (("k0", k0), ("v0", v0), ("k_final", k_final), ("v_final", v_final)):
        _check(t, nm, torch.float32)
    dt = _dt(q)
    if out is None:
        out = torch.empty((H, total, dv), dtype=q.dtype, device=q.device)
    if final_state:
        if k_final is None:
            k_final = torch.empty((n, H, m, dk), dtype=torch.float32, device=q.device)
        if v_final is None:
            v_final = torch.empty((n, H, m, dv), dtype=torch.float32, device=q.device)
    nbytes = int(lib.gsa_fwd_varlen_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), n, H, dk,
                                                    dv, m, C, dt, chunks_per_segment))
    if nbytes == (1 << 64) - 1:
        raise ValueError("invalid cu_seqlens or problem size")
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    st = lib.gsa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), ctypes.cast(arr, ctypes.c_void_p),
                            n, H, _ptr(k0), _ptr(v0), _ptr(out), _ptr(k_final), _ptr(v_final),
                            dk, dv, m, C, float(tau), dt, _ptr(workspace),
                            _wsbytes(workspace), int(chunks_per_segment),
                            _stream(stream), _events(events))
    if st:
        raise GsaError("gsa_fwd_varlen", st)
    return out, k_final, v_final


def gla_fwd(q, k, v, g, s0=None, *, tau=16.0, C=64, final_state=False,
            chunks_per_segment=0, out=None, s_final=None, workspace=None, stream=None,
            events=None, gate="logit"):
    """Chunkwise GLA forward.  q, k, g [B,H,T,dk]; v [B,H,T,dv]; optional float32
    initial state s0 [B,H,dk,dv].  gate: "logit" (alpha = sigmoid(g)^(1/tau))
    or "log_decay" (g holds log alpha per token and key dimension; tau unused).
    Returns (o, s_final or None)."""
    torch = _torch()
    _ndim(q, "q", 4)
    B, H, T, dk = q.shape
    _ndim(v, "v", 4)
    dv = v.shape[-1]
    for n, t, sh in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)), ("g", g, (B, H, T, dk)),
                     ("s0", s0, (B, H, dk, dv)), ("out", out, (B, H, T, dv)),
                     ("s_final", s_final, (B, H, dk, dv))):
        _shape(t, n, sh)
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g), ("out", out)):
        _check(t, n, q.dtype)
    for n, t in (("s0", s0), ("s_final", s_final)):
        _check(t, n, torch.float32)
    dt = _dt(q)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state and s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    nbytes = gla_fwd_workspace_bytes(B, H, T, dk, dv, C, dt, chunks_per_segment)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if gate not in GATE_INPUTS:
        raise ValueError("gate must be one of %s" % ", ".join(GATE_INPUTS))
    st = lib.gla_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(out),
                        _ptr(s_final), B, H, T, dk, dv, C, float(tau), dt, _ptr(workspace),
                        _wsbytes(workspace), int(chunks_per_segment),
                        GATE_INPUTS[gate], _stream(stream), _events(events))
    if st:
        raise GsaError("gla_fwd", st)
    return out, s_final


def gsa_decode_step(q, k, v, g, k_state, v_state, *, tau=8.0, out=None, stream=None,
                    events=None, nonlinearity="softmax"):
    """One recurrent GSA step.  q, k [N,H,dk]; v [N,H,dv]; g [N,H,m]; float32
    k_state [N,H,m,dk] and v_state [N,H,m,dv] are advanced in place.  Returns o.
    events: None or two hipEvent_t handles that take the kernel's start and end.
    nonlinearity: as for gsa_fwd."""
    torch = _torch()
    _ndim(q, "q", 3)
    N, H, dk = q.shape
    _ndim(v, "v", 3)
    _ndim(g, "g", 3)
    dv, m = v.shape[-1], g.shape[-1]
    for n, t, sh in (("k", k, (N, H, dk)), ("v", v, (N, H, dv)), ("g", g, (N, H, m)),
                     ("k_state", k_state, (N, H, m, dk)), ("v_state", v_state, (N, H, m, dv)),
                     ("out", out, (N, H, dv))):
        _shape(t, n, sh)
    if k_state is None or v_state is None:
        raise TypeError("k_state and v_state are required")
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g), ("out", out)):
        _check(t, n, q.dtype)
    _check(k_state, "k_state", torch.float32)
    _check(v_state, "v_state", torch.float32)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    st = lib.gsa_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(k_state),
                                _ptr(v_state), _ptr(out), N, H, dk, dv, m, float(tau), _dt(q),
                                _nl(nonlinearity), _stream(stream), _events(events, 2))
    if st:
        raise GsaError("gsa_decode_step", st)
    return out


def gla_decode_step(q, k, v, g, s_state, *, tau=16.0, gate="logit", out=None, stream=None,
                    events=None):
    """One recurrent GLA step.  q, k, g [N,H,dk]; v [N,H,dv]; float32 s_state
    [N,H,dk,dv] advanced in place (e.g. gla_fwd's s_final).  gate as for
    gla_fwd.  Returns o [N,H,dv]."""
    torch = _torch()
    _ndim(q, "q", 3)
    N, H, dk = q.shape
    _ndim(v, "v", 3)
    dv = v.shape[-1]
    for n, t, sh in (("k", k, (N, H, dk)), ("v", v, (N, H, dv)), ("g", g, (N, H, dk)),
                     ("s_state", s_state, (N, H, dk, dv)), ("out", out, (N, H, dv))):
        _shape(t, n, sh)
    if s_state is None:
        raise TypeError("s_state is required")
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g), ("out", out)):
        _check(t, n, q.dtype)
    _check(s_state, "s_state", torch.float32)
    if gate not in GATE_INPUTS:
        raise ValueError("gate must be one of %s" % ", ".join(GATE_INPUTS))
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    st = lib.gla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s_state), _ptr(out), N, H, dk,
                             dv, float(tau), _dt(q), GATE_INPUTS[gate], _stream(stream),
                             _events(events, 2))
    if st:
        raise GsaError("gla_decode_step", st)
    return out


def gsa_bwd_supported(dk, dv, m, dtype=DTYPE_BF16) -> bool:
    return bool(lib.gsa_bwd_supported(dk, dv, m, dtype))


def gsa_bwd_workspace_bytes(B, H, T, dk, dv, m, dtype=None, nonlinearity="softmax") -> int:
    """Workspace bytes of gsa_bwd for this storage type (DTYPE_F32 /
    DTYPE_BF16) and slot read; without a dtype, enough for any call."""
    if dtype is None:
        return int(lib.gsa_bwd_workspace_bytes(B, H, T, dk, dv, m))
    return int(lib.gsa_bwd_workspace_bytes_ex(B, H, T, dk, dv, m, int(dtype), _nl(nonlinearity)))


def _bwd_prep(q, k, v, g, d_o, k0, v0, d_kf, d_vf, out, state_grads):
    """Shape and dtype checks of a GSA backward's tensors; allocates the
    gradients.  Returns ((B, H, T, dk, dv, m), [d_q, d_k, d_v, d_g], [d_k0, d_v0])."""
    torch = _torch()
    _ndim(q, "q", 4)
    B, H, T, dk = q.shape
    _ndim(v, "v", 4)
    _ndim(g, "g", 4)
    dv, m = v.shape[-1], g.shape[-1]
    for n, t, sh in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)), ("g", g, (B, H, T, m)),
                     ("d_o", d_o, (B, H, T, dv)), ("k0", k0, (B, H, m, dk)), ("v0", v0, (B, H, m, dv)),
                     ("d_kf", d_kf, (B, H, m, dk)), ("d_vf", d_vf, (B, H, m, dv))):
        _shape(t, n, sh)
    if d_o is None:
        raise TypeError("d_o is required")
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g), ("d_o", d_o)):
        _check(t, n, q.dtype)
    for n, t in (("k0", k0), ("v0", v0), ("d_kf", d_kf), ("d_vf", d_vf)):
        _check(t, n, torch.float32)
    if out is None:
        outs = [torch.empty_like(x) for x in (q, k, v, g)]
    else:
        outs = list(out)
        for n, t, x in zip(("d_q", "d_k", "d_v", "d_g"), outs, (q, k, v, g)):
            _check(t, n, q.dtype)
            if t.shape != x.shape:
                raise ValueError("%s must have shape %s" % (n, tuple(x.shape)))
    sg = [None, None]
    if state_grads:
        sg = [torch.empty((B, H, m, d), dtype=torch.float32, device=q.device) for d in (dk, dv)]
    return (B, H, T, dk, dv, m), outs, sg


def gsa_bwd(q, k, v, g, d_o, k0=None, v0=None, d_kf=None, d_vf=None, *, tau=8.0,
            state_grads=False, out=None, workspace=None, stream=None, events=None,
            nonlinearity="softmax"):
    """GSA backward (softmax read): the gradients of gsa_fwd(q, k, v, g, k0,
    v0, tau=tau) given d_o [B,H,T,dv] (the gradient of o) and optional float32
    d_kf [B,H,m,dk] / d_vf [B,H,m,dv] (those of the final states).
    Returns (d_q, d_k, d_v, d_g, d_k0, d_v0); d_k0 / d_v0 (float32) are None
    unless state_grads.  out: optional (d_q, d_k, d_v, d_g) to write into.
    nonlinearity: the slot read of the forward being differentiated, as for
    gsa_fwd."""
    torch = _torch()
    (B, H, T, dk, dv, m), outs, sg = _bwd_prep(q, k, v, g, d_o, k0, v0, d_kf, d_vf, out, state_grads)
    nbytes = gsa_bwd_workspace_bytes(B, H, T, dk, dv, m, _dt(q), nonlinearity)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    st = lib.gsa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(d_o), _ptr(k0), _ptr(v0),
                        _ptr(d_kf), _ptr(d_vf), *(_ptr(x) for x in outs), _ptr(sg[0]), _ptr(sg[1]),
                        B, H, T, dk, dv, m, float(tau), _dt(q), _ptr(workspace),
                        _wsbytes(workspace), _nl(nonlinearity),
                        _stream(stream), _events(events))
    if st:
        raise GsaError("gsa_bwd", st)
    return (*outs, sg[0], sg[1])


def gsa_train_states_bytes(B, H, T, dk, dv, m, dtype=DTYPE_BF16) -> int:
    """Bytes of the segment start states gsa_fwd_train keeps for
    gsa_bwd_train (0: nothing to keep, or the pair is not compiled here)."""
    return int(lib.gsa_train_states_bytes(B, H, T, dk, dv, m, dtype))


def gsa_train_supported(q, v, g, nonlinearity="softmax") -> bool:
    """Whether gsa_fwd_train / gsa_bwd_train run for these tensors and read
    (bf16, the matrix-core backward's shapes, not ReLU)."""
    dk, dv, m = q.shape[-1], v.shape[-1], g.shape[-1]
    return (q.dtype == _torch().bfloat16 and _nl(nonlinearity) != NONLINEARITIES["relu"] and
            gsa_fwd_supported(dk, dv, m, 64, DTYPE_BF16) and gsa_bwd_supported(dk, dv, m, DTYPE_BF16))


def gsa_fwd_train(q, k, v, g, k0=None, v0=None, *, tau=8.0, final_state=False, out=None, k_final=None,
                  v_final=None, states=None, workspace=None, stream=None, events=None,
                  nonlinearity="softmax"):
    """gsa_fwd that also keeps the segment start states of the backward's
    split (a uint8 device tensor of gsa_train_states_bytes bytes, allocated
    when `states` is None).  Returns (o, k_final, v_final, states)."""
    torch = _torch()
    (B, H, T, dk, dv, m), out, k_final, v_final = _fwd_prep(q, k, v, g, k0, v0, out, k_final, v_final,
                                                             final_state)
    dt = _dt(q)
    sb = gsa_train_states_bytes(B, H, T, dk, dv, m, dt)
    if sb == (1 << 64) - 1:
        raise ValueError("invalid problem size")
    if states is None:
        states = torch.empty(max(sb, 1), dtype=torch.uint8, device=q.device)
    nbytes = int(lib.gsa_fwd_train_workspace_bytes(B, H, T, dk, dv, m, dt))
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    st = lib.gsa_fwd_train(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(k0), _ptr(v0), _ptr(out),
                           _ptr(k_final), _ptr(v_final), B, H, T, dk, dv, m, float(tau), dt,
                           _ptr(workspace), _wsbytes(workspace), _ptr(states), _wsbytes(states),
                           _nl(nonlinearity), _stream(stream), _events(events))
    if st:
        raise GsaError("gsa_fwd_train", st)
    return out, k_final, v_final, states


def gsa_bwd_train(q, k, v, g, d_o, states, k0=None, v0=None, d_kf=None, d_vf=None, *, tau=8.0,
                  state_grads=False, out=None, workspace=None, stream=None, events=None,
                  nonlinearity="softmax"):
    """gsa_bwd given the states gsa_fwd_train kept for the same inputs (they
    replace the backward's own recomputation of the segment start states).
    Returns (d_q, d_k, d_v, d_g, d_k0, d_v0) as gsa_bwd."""
    torch = _torch()
    (B, H, T, dk, dv, m), outs, sg = _bwd_prep(q, k, v, g, d_o, k0, v0, d_kf, d_vf, out, state_grads)
    nbytes = gsa_bwd_workspace_bytes(B, H, T, dk, dv, m, _dt(q), nonlinearity)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    st = lib.gsa_bwd_train(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(d_o), _ptr(k0), _ptr(v0),
                           _ptr(d_kf), _ptr(d_vf), *(_ptr(x) for x in outs), _ptr(sg[0]), _ptr(sg[1]),
                           B, H, T, dk, dv, m, float(tau), _dt(q), _ptr(workspace), _wsbytes(workspace),
                           _ptr(states), _wsbytes(states), _nl(nonlinearity), _stream(stream),
                           _events(events))
    if st:
        raise GsaError("gsa_bwd_train", st)
    return (*outs, sg[0], sg[1])


def gsa_bwd_varlen_workspace_bytes(cu_seqlens, H, dk, dv, m) -> int:
    arr, n = _cu_array(cu_seqlens)
    return int(lib.gsa_bwd_varlen_workspace_bytes(ctypes.cast(arr, _P), n, H, dk, dv, m))


def gsa_bwd_varlen(q, k, v, g, d_o, cu_seqlens, k0=None, v0=None, d_kf=None, d_vf=None, *,
                   tau=8.0, state_grads=False, workspace=None, stream=None, events=None):
    """GSA backward over a packed batch (layout of gsa_fwd_varlen: q, k, g, d_o
    [H, total, d]; host offsets cu_seqlens; states [n, H, m, d]).  Returns
    (d_q, d_k, d_v, d_g, d_k0, d_v0); the state gradients are None unless
    state_grads."""
    torch = _torch()
    _ndim(q, "q", 3)
    H, total, dk = q.shape
    _ndim(v, "v", 3)
    _ndim(g, "g", 3)
    dv, m = v.shape[-1], g.shape[-1]
    arr, n = _cu_array(cu_seqlens)
    if arr[n] != total:
        raise ValueError("cu_seqlens[-1] = %d but the arrays hold %d tokens" % (arr[n], total))
    for nm, t, sh in (("k", k, (H, total, dk)), ("v", v, (H, total, dv)), ("g", g, (H, total, m)),
                      ("d_o", d_o, (H, total, dv)), ("k0", k0, (n, H, m, dk)), ("v0", v0, (n, H, m, dv)),
                      ("d_kf", d_kf, (n, H, m, dk)), ("d_vf", d_vf, (n, H, m, dv))):
        _shape(t, nm, sh)
    if d_o is None:
        raise TypeError("d_o is required")
    for nm, t in (("q", q), ("k", k), ("v", v), ("g", g), ("d_o", d_o)):
        _check(t, nm, q.dtype)
    for nm, t in (("k0", k0), ("v0", v0), ("d_kf", d_kf), ("d_vf", d_vf)):
        _check(t, nm, torch.float32)
    outs = [torch.empty_like(x) for x in (q, k, v, g)]
    sg = [None, None]
    if state_grads:
        sg = [torch.empty((n, H, m, d), dtype=torch.float32, device=q.device) for d in (dk, dv)]
    nbytes = int(lib.gsa_bwd_varlen_workspace_bytes(ctypes.cast(arr, _P), n, H, dk, dv, m))
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    st = lib.gsa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(d_o), ctypes.cast(arr, _P), n, H,
                            _ptr(k0), _ptr(v0), _ptr(d_kf), _ptr(d_vf), *(_ptr(x) for x in outs),
                            _ptr(sg[0]), _ptr(sg[1]), dk, dv, m, float(tau), _dt(q), _ptr(workspace),
                            _wsbytes(workspace), _stream(stream),
                            _events(events))
    if st:
        raise GsaError("gsa_bwd_varlen", st)
    return (*outs, sg[0], sg[1])


def _autograd_function():
    torch = _torch()

    class GsaFunction(torch.autograd.Function):
        """gsa_fwd (final states returned) with gsa_bwd as its backward (the
        training pair gsa_fwd_train / gsa_bwd_train where it runs)."""

        @staticmethod
        def forward(ctx, q, k, v, g, k0, v0, tau, nonlinearity):
            ctx.set_materialize_grads(False)
            # where the training pair runs, the forward keeps the segment start
            # states and the backward reads them instead of recomputing them
            states = None
            if gsa_train_supported(q, v, g, nonlinearity):
                o, kf, vf, states = gsa_fwd_train(q, k, v, g, k0, v0, tau=tau, final_state=True,
                                                  nonlinearity=nonlinearity)
            else:
                o, kf, vf = gsa_fwd(q, k, v, g, k0, v0, tau=tau, final_state=True,
                                    nonlinearity=nonlinearity)
            ctx.save_for_backward(q, k, v, g, k0, v0)
            ctx.states = states
            ctx.tau, ctx.nonlinearity = tau, nonlinearity
            return o, kf, vf

        @staticmethod
        @torch.autograd.function.once_differentiable
        def backward(ctx, d_o, d_kf, d_vf):
            q, k, v, g, k0, v0 = ctx.saved_tensors
            if d_o is None:
                d_o = torch.zeros_like(v)
            dkf = None if d_kf is None else d_kf.contiguous()
            dvf = None if d_vf is None else d_vf.contiguous()
            if ctx.states is not None:
                grads = gsa_bwd_train(q, k, v, g, d_o.contiguous(), ctx.states, k0, v0, dkf, dvf,
                                      tau=ctx.tau, state_grads=True, nonlinearity=ctx.nonlinearity)
                ctx.states = None
            else:
                grads = gsa_bwd(q, k, v, g, d_o.contiguous(), k0, v0, dkf, dvf, tau=ctx.tau,
                                state_grads=True, nonlinearity=ctx.nonlinearity)
            dk0 = grads[4] if k0 is not None and ctx.needs_input_grad[4] else None
            dv0 = grads[5] if v0 is not None and ctx.needs_input_grad[5] else None
            return grads[0], grads[1], grads[2], grads[3], dk0, dv0, None, None

    return GsaFunction


_GSA_FUNCTION = None


def gsa_autograd(q, k, v, g, k0=None, v0=None, *, tau=8.0, nonlinearity="softmax"):
    """Differentiable GSA: returns (o, k_final, v_final) like gsa_fwd with
    final_state=True, and back-propagates through gsa_bwd (all the kernels of
    this library; the function only routes tensors)."""
    global _GSA_FUNCTION
    if _GSA_FUNCTION is None:
        _GSA_FUNCTION = _autograd_function()
    return _GSA_FUNCTION.apply(q, k, v, g, k0, v0, float(tau), nonlinearity)


# ------------------------------------------------------------ calibration
def measure_hbm(dst, src=None, *, stream=None, events=None):
    """Stream dst's bytes through HBM: copy src -> dst (equal byte sizes, a
    multiple of 16), or with src None add 1.0 to every float of dst in place.
    Returns the bytes moved (2 * nbytes).  events: None or two hipEvent_t
    handles stamped at the kernel's start and end."""
    _check(dst, "dst")
    if src is not None:
        _check(src, "src")
    nb = dst.numel() * dst.element_size()
    if src is not None and src.numel() * src.element_size() != nb:
        raise ValueError("src and dst sizes differ")
    st = lib.gsa_measure_hbm(_ptr(src), _ptr(dst), nb, 0 if src is not None else 1, _stream(stream),
                             _events(events, 2))
    if st:
        raise GsaError("gsa_measure_hbm", st)
    return 2 * nb


def measure_mfma_bf16(iterations, *, sink=None, stream=None, events=None):
    """The bf16 MFMA calibration loop; returns (sink, dense flops).  Every sink
    entry ends at 1024 * iterations + 496."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(MEASURE_MFMA_WORKGROUPS, dtype=torch.float32, device="cuda")
    _check(sink, "sink", torch.float32)
    if sink.numel() < MEASURE_MFMA_WORKGROUPS:
        raise ValueError("sink needs %d floats" % MEASURE_MFMA_WORKGROUPS)
    fl = ctypes.c_double()
    st = lib.gsa_measure_mfma_bf16(_ptr(sink), sink.numel(), int(iterations), ctypes.byref(fl),
                                   _stream(stream), _events(events, 2))
    if st:
        raise GsaError("gsa_measure_mfma_bf16", st)
    return sink, fl.value
