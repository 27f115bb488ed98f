"""MI355X (gfx950) Kimi Delta Attention: chunked prefill, recurrent decode, state pools.

A thin ctypes binding over ``libkda.so`` (C ABI in ``include/kda.h``).  This
module only marshals arguments: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and the current stream.
If the library is missing the calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KDAError",
    "chunk_fwd",
    "chunk_fwd_workspace_size",
    "chunk_fwd_no_alloc",
    "no_alloc_max_workspace",
    "device_status",
    "set_handoff_poll_limit",
    "handoff_poll_limit",
    "balanced_schedule",
    "DEVICE_HANDOFF_TIMEOUT",
    "chunk_bwd",
    "chunk_bwd_workspace_size",
    "recurrent_step",
    "fused_decode_step",
    "spec_verify_step",
    "conv_cache_bytes",
    "state_io",
    "state_bytes",
    "library",
    "LIB_PATH",
    "KDA_F32",
    "KDA_BF16",
    "STATE_ZERO",
    "STATE_COPY",
    "STATE_GATHER",
    "STATE_SCATTER",
    "GATE_LOG_DECAY",
    "GATE_LOWER_BOUND",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
STATE_ZERO, STATE_COPY, STATE_GATHER, STATE_SCATTER = 0, 1, 2, 3
_STATUS = {0: "KDA_SUCCESS", 1: "KDA_ERROR_INVALID_VALUE", 2: "KDA_ERROR_UNSUPPORTED",
           3: "KDA_ERROR_WORKSPACE", 4: "KDA_ERROR_LAUNCH"}


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(status, status)}")
        self.status = status


GATE_LOG_DECAY = 0
GATE_LOWER_BOUND = 1
DEVICE_HANDOFF_TIMEOUT = 0x1  # KDA_DEVICE_HANDOFF_TIMEOUT


class Gate(ctypes.Structure):
    """kda_gate: how g and beta are read (zero = log-decay g, beta as given)."""
    _fields_ = [
        ("mode", ctypes.c_int),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("lower_bound", ctypes.c_float),
        ("beta_logits", ctypes.c_int32),
    ]


class ChunkFwdArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("io_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p),
        ("final_state", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("segments", ctypes.c_int32),
        ("gate", Gate),
    ]


class ChunkBwdArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("io_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p),
        ("dO", ctypes.c_void_p),
        ("dfinal_state", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("dg", ctypes.c_void_p),
        ("dbeta", ctypes.c_void_p),
        ("dinitial_state", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class RecurrentStepArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("io_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("state_indices", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32),
        ("o", ctypes.c_void_p),
        ("gate", Gate),
    ]


class FusedStepArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("io_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("conv_weight", ctypes.c_void_p),
        ("conv_cache", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("state_indices", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32),
        ("l2_eps", ctypes.c_float),
        ("out_norm", ctypes.c_int32),
        ("norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("o", ctypes.c_void_p),
        ("gate", Gate),
    ]


class SpecVerifyArgs(ctypes.Structure):
    _fields_ = [
        ("step", FusedStepArgs),
        ("window", ctypes.c_int32),
        ("replay_q", ctypes.c_void_p),
        ("replay_k", ctypes.c_void_p),
        ("replay_v", ctypes.c_void_p),
        ("replay_g", ctypes.c_void_p),
        ("replay_beta", ctypes.c_void_p),
        ("replay_window", ctypes.c_int32),
        ("num_replay", ctypes.c_void_p),
    ]


CONV_WIDTH = 4

_LIB = None


def library(path: str = LIB_PATH):
    """Open libkda.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"libkda.so not found at {path}; build it with "
                           "`python -m gated_delta_rule_10_amd.build`")
    lib = ctypes.CDLL(path)
    lib.kda_chunk_fwd.argtypes = [ctypes.POINTER(ChunkFwdArgs), ctypes.c_void_p]
    lib.kda_chunk_fwd_no_alloc.argtypes = [ctypes.POINTER(ChunkFwdArgs), ctypes.c_void_p]
    lib.kda_chunk_fwd_no_alloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_no_alloc_max_workspace.argtypes = []
    lib.kda_chunk_fwd_no_alloc_max_workspace.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(ChunkFwdArgs),
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_recurrent_step.argtypes = [ctypes.POINTER(RecurrentStepArgs), ctypes.c_void_p]
    lib.kda_chunk_bwd.argtypes = [ctypes.POINTER(ChunkBwdArgs), ctypes.c_void_p]
    lib.kda_chunk_bwd_workspace_size.argtypes = [ctypes.POINTER(ChunkBwdArgs),
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_chunk_bwd_min_workspace_size.argtypes = [ctypes.POINTER(ChunkBwdArgs),
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_fused_decode_step.argtypes = [ctypes.POINTER(FusedStepArgs), ctypes.c_void_p]
    lib.kda_spec_verify_step.argtypes = [ctypes.POINTER(SpecVerifyArgs), ctypes.c_void_p]
    lib.kda_conv_cache_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
    lib.kda_conv_cache_bytes.restype = ctypes.c_size_t
    lib.kda_state_io.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_void_p]
    for fn in ("kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_recurrent_step",
               "kda_state_io"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.kda_state_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
    lib.kda_state_bytes.restype = ctypes.c_size_t
    lib.kda_device_status.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_uint32)]
    lib.kda_device_status.restype = ctypes.c_int
    lib.kda_set_handoff_poll_limit.argtypes = [ctypes.c_int32]
    lib.kda_set_handoff_poll_limit.restype = ctypes.c_int
    lib.kda_handoff_poll_limit.argtypes = []
    lib.kda_handoff_poll_limit.restype = ctypes.c_int32
    lib.kda_balanced_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.kda_balanced_schedule.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {dt}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t=None) -> ctypes.c_void_p:
    dev = t.device if t is not None else None
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(st: int, what: str):
    if st != 0:
        raise KDAError(st, what)


def _need(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _out_like(out, like, name="out"):
    """A new output shaped like ``like``, or the caller's, checked (the kernels
    see only its pointer)."""
    if out is None:
        return torch.empty_like(like)
    _need(out, name, dtype=like.dtype, ndim=like.dim())
    if out.shape != like.shape:
        raise ValueError(f"{name} must be {list(like.shape)}")
    return out


def _gate(H, A_log, dt_bias, lower_bound, beta_logits):
    """Fill a kda_gate: the lower-bounded gate when A_log is given, else log-decay g."""
    gt = Gate()
    gt.beta_logits = 1 if beta_logits else 0
    if A_log is None:
        if dt_bias is not None:
            raise ValueError("dt_bias needs A_log (the lower-bounded gate)")
        gt.mode = GATE_LOG_DECAY
        return gt
    _need(A_log, "A_log", dtype=torch.float32)
    if A_log.numel() != H:
        raise ValueError(f"A_log must hold {H} values")
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", dtype=torch.float32)
        if dt_bias.numel() != H * 128:
            raise ValueError(f"dt_bias must hold {H} x 128 values")
    gt.mode = GATE_LOWER_BOUND
    gt.A_log = A_log.data_ptr()
    gt.dt_bias = None if dt_bias is None else dt_bias.data_ptr()
    gt.lower_bound = float(lower_bound)
    return gt


def _chunk_args(q, N, cu_seqlens, cu_seqlens_host, scale, segments):
    """Fill the size fields of kda_chunk_fwd_args; returns (args, host_array)."""
    T, H, D = q.shape
    a = ChunkFwdArgs()
    host = None
    a.num_seqs = N
    if cu_seqlens_host is not None:
        host = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
        a.cu_seqlens_host = host
        a.seq_len = 0
    else:
        if T % N:
            raise ValueError("T_total must be a multiple of the number of sequences")
        a.seq_len = T // N
    a.num_heads, a.head_dim, a.chunk_size = H, D, 64
    a.io_dtype = _dtype_code(q.dtype)
    a.scale = float(scale)
    a.segments = int(segments)
    return a, host


def chunk_fwd_workspace_size(q, num_seqs=None, cu_seqlens_host=None, segments=0) -> int:
    """Workspace bytes for a prefill of ``q``'s shape (host only, no GPU work)."""
    lib = library()
    N = len(cu_seqlens_host) - 1 if cu_seqlens_host is not None else (num_seqs or 1)
    a, host = _chunk_args(q, N, None, cu_seqlens_host, 1.0, segments)
    if cu_seqlens_host is not None:
        a.cu_seqlens = 16  # non-null marker: only the host copy is read here
    out = ctypes.c_size_t(0)
    _check(lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(out)),
           "kda_chunk_fwd_workspace_size")
    del host
    return int(out.value)


def _chunk_fwd_setup(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, initial_state,
                     output_final_state, scale, segments, num_seqs, out, final_state, A_log,
                     dt_bias, lower_bound, beta_logits, allocate):
    """Check the tensors and fill kda_chunk_fwd_args (everything but the
    workspace).  With ``allocate`` a missing o / final state is allocated;
    without, the caller must pass them.  Returns (args, host array, o, final)."""
    _need(q, "q", ndim=3)
    for name, t in (("k", k), ("v", v)):
        _need(t, name, dtype=q.dtype, ndim=3)
    _need(g, "g", dtype=torch.float32, ndim=3)
    _need(beta, "beta", dtype=torch.float32, ndim=2)
    T, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or g.shape != q.shape or beta.shape != (T, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = num_seqs or (initial_state.shape[0] if initial_state is not None else 1)
    if initial_state is not None:
        _need(initial_state, "initial_state", dtype=torch.float32, ndim=4)
        if initial_state.shape != (N, H, D, D):
            raise ValueError(f"initial_state must be [{N}, {H}, {D}, {D}]")
    if out is None and not allocate:
        raise ValueError("out is required (this call allocates nothing)")
    o = _out_like(out, q)
    if not output_final_state:
        final_state = None
    elif final_state is None:
        if not allocate:
            raise ValueError("final_state is required with output_final_state "
                             "(this call allocates nothing)")
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=q.device)
    else:  # the caller's: the kernels see only its pointer
        _need(final_state, "final_state", dtype=torch.float32, ndim=4)
        if final_state.shape != (N, H, D, D):
            raise ValueError(f"final_state must be [{N}, {H}, {D}, {D}]")
    if cu_seqlens is not None and cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.tolist()  # one device-to-host copy
    a, host = _chunk_args(q, N, cu_seqlens, cu_seqlens_host, scale, segments)
    a.gate = _gate(H, A_log, dt_bias, lower_bound, beta_logits)
    a.cu_seqlens = None if cu_seqlens is None else cu_seqlens.data_ptr()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.g, a.beta = g.data_ptr(), beta.data_ptr()
    a.initial_state = None if initial_state is None else initial_state.data_ptr()
    a.final_state = None if final_state is None else final_state.data_ptr()
    a.o = o.data_ptr()
    return a, host, o, final_state


def chunk_fwd(q, k, v, g, beta, cu_seqlens=None, cu_seqlens_host=None, initial_state=None,
              output_final_state=True, scale=1.0, segments=0, num_seqs=None, out=None,
              final_state=None, workspace=None, A_log=None, dt_bias=None, lower_bound=-5.0,
              beta_logits=False):
    """Chunkwise KDA prefill forward.

    q, k, v: [T, H, 128] bf16 or fp32 (same dtype); g: [T, H, 128] fp32 log-decay;
    beta: [T, H] fp32; cu_seqlens: int32 [N+1] on the device (packed batch) or None
    for ``num_seqs`` (default 1, or initial_state.shape[0]) sequences of equal
    length; initial_state: [N, H, 128, 128] fp32 or None.
    With ``A_log`` ([H] fp32) g holds raw gate logits and the kernels apply the
    lower-bounded gate lower_bound * sigmoid(exp(A_log) (g + dt_bias)) (dt_bias
    [H, 128] fp32 or None); with ``beta_logits`` beta holds logits (sigmoid
    applied in the kernels).
    Returns (o [T, H, 128], final_state [N, H, 128, 128] fp32 or None).
    """
    lib = library()
    a, host, o, final_state = _chunk_fwd_setup(
        q, k, v, g, beta, cu_seqlens, cu_seqlens_host, initial_state, output_final_state, scale,
        segments, num_seqs, out, final_state, A_log, dt_bias, lower_bound, beta_logits, True)
    ws_bytes = ctypes.c_size_t(0)
    _check(lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(ws_bytes)),
           "kda_chunk_fwd_workspace_size")
    if ws_bytes.value:
        if workspace is not None:
            _need(workspace, "workspace", dtype=torch.uint8, ndim=1)
        if workspace is None or workspace.numel() < ws_bytes.value:
            workspace = torch.empty(ws_bytes.value, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel()
    _check(lib.kda_chunk_fwd(ctypes.byref(a), _stream(q)), "kda_chunk_fwd")
    del host
    return o, final_state


def chunk_fwd_no_alloc(q, k, v, g, beta, out, final_state=None, cu_seqlens=None,
                       cu_seqlens_host=None, initial_state=None, output_final_state=True,
                       scale=1.0, segments=0, num_seqs=None, A_log=None, dt_bias=None,
                       lower_bound=-5.0, beta_logits=False):
    """chunk_fwd for callers that cannot allocate: the same computation (same
    bits) with the workspace taken from the library's per-GPU buffer of
    no_alloc_max_workspace() bytes.  ``out`` (and ``final_state`` unless
    output_final_state is False) must be given; nothing is allocated on the
    device.  Calls that overlap in time on one GPU race on the buffer.  Raises
    KDAError (KDA_ERROR_WORKSPACE) when the call needs a larger workspace."""
    lib = library()
    a, host, o, final_state = _chunk_fwd_setup(
        q, k, v, g, beta, cu_seqlens, cu_seqlens_host, initial_state, output_final_state, scale,
        segments, num_seqs, out, final_state, A_log, dt_bias, lower_bound, beta_logits, False)
    _check(lib.kda_chunk_fwd_no_alloc(ctypes.byref(a), _stream(q)), "kda_chunk_fwd_no_alloc")
    del host
    return o, final_state


def no_alloc_max_workspace() -> int:
    """Bytes of the per-GPU buffer behind chunk_fwd_no_alloc."""
    return int(library().kda_chunk_fwd_no_alloc_max_workspace())


def device_status(clear: bool = True, device=None) -> int:
    """KDA_DEVICE_* bits the kernels have set on the current (or given) GPU since
    the last clear, read after the current stream's queued work has finished."""
    lib = library()
    bits = ctypes.c_uint32(0)
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        _check(lib.kda_device_status(_stream(torch.empty(0, device=dev)), 1 if clear else 0,
                                     ctypes.byref(bits)), "kda_device_status")
    return int(bits.value)


def set_handoff_poll_limit(polls: int) -> None:
    """Polls of a hand-over flag before a balanced-schedule workgroup gives up
    (process-wide; 0 = give up at once, for tests of that path)."""
    _check(library().kda_set_handoff_poll_limit(int(polls)), "kda_set_handoff_poll_limit")


def handoff_poll_limit() -> int:
    return int(library().kda_handoff_poll_limit())


def balanced_schedule(num_seqs: int, seq_len: int, num_heads: int, compute_units: int):
    """The balanced schedule the prefill would use for this fixed-length batch on
    a GPU with `compute_units` units (host only): a list of (chain, first chunk,
    end chunk, role, wait workgroup) per workgroup in dispatch order, or None when
    the prefill runs whole chains."""
    lib = library()
    n = ctypes.c_int64(0)
    _check(lib.kda_balanced_schedule(num_seqs, seq_len, num_heads, compute_units, None, 0,
                                     ctypes.byref(n)), "kda_balanced_schedule")
    if n.value == 0:
        return None
    buf = (ctypes.c_int32 * (5 * n.value))()
    _check(lib.kda_balanced_schedule(num_seqs, seq_len, num_heads, compute_units, buf, n.value,
                                     ctypes.byref(n)), "kda_balanced_schedule")
    return [tuple(buf[5 * i:5 * i + 5]) for i in range(n.value)]


def chunk_bwd_workspace_size(q, num_seqs=None, cu_seqlens_host=None, minimum=False) -> int:
    """Workspace bytes for the backward of a prefill of ``q``'s shape (host only):
    the whole pack in one pass, or with ``minimum`` the smallest workspace the
    backward accepts (the largest single sequence's; smaller workspaces are used
    for groups of sequences in turn)."""
    lib = library()
    T, H, D = q.shape
    a = ChunkBwdArgs()
    host = None
    if cu_seqlens_host is not None:
        host = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
        a.num_seqs = len(cu_seqlens_host) - 1
        a.cu_seqlens_host = host
        a.cu_seqlens = 16  # non-null marker: only the host copy is read here
    else:
        a.num_seqs = num_seqs or 1
        a.seq_len = T // a.num_seqs
    a.num_heads, a.head_dim = H, D
    a.io_dtype = _dtype_code(q.dtype)
    a.scale = 1.0
    out = ctypes.c_size_t(0)
    query = lib.kda_chunk_bwd_min_workspace_size if minimum else lib.kda_chunk_bwd_workspace_size
    _check(query(ctypes.byref(a), ctypes.byref(out)), "kda_chunk_bwd_workspace_size")
    del host
    return int(out.value)


def chunk_bwd(q, k, v, g, beta, dO, cu_seqlens=None, cu_seqlens_host=None, initial_state=None,
              dfinal_state=None, scale=1.0, num_seqs=None, want_dinitial=True, workspace=None,
              grads=None, max_workspace_bytes=None):
    """Backward of chunk_fwd (log-decay g, beta as given): gradients of
    L = <dO, o> + <dfinal_state, S_T>.

    Shapes as in chunk_fwd; dO: [T, H, 128] in q's dtype; dfinal_state:
    [N, H, 128, 128] fp32 or None.  Returns a dict of fp32 dq, dk, dv, dg
    [T, H, 128], dbeta [T, H] and dinitial_state [N, H, 128, 128] (None unless
    want_dinitial).  ``grads`` may pass preallocated outputs with those keys.
    ``workspace`` (uint8) is used as given: at least the minimum size, and below
    the whole pack's the sequences run in groups.  Without one, a workspace for
    the whole pack is allocated, or of ``max_workspace_bytes`` if that is less
    (but not below the minimum).
    """
    lib = library()
    _need(q, "q", ndim=3)
    for name, t in (("k", k), ("v", v), ("dO", dO)):
        _need(t, name, dtype=q.dtype, ndim=3)
    _need(g, "g", dtype=torch.float32, ndim=3)
    _need(beta, "beta", dtype=torch.float32, ndim=2)
    T, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or g.shape != q.shape or dO.shape != q.shape \
            or beta.shape != (T, H):
        raise ValueError("shape mismatch among q, k, v, g, beta, dO")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1)
        N = cu_seqlens.shape[0] - 1
        if cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.tolist()
    else:
        N = num_seqs or (initial_state.shape[0] if initial_state is not None else 1)
    for name, t in (("initial_state", initial_state), ("dfinal_state", dfinal_state)):
        if t is not None:
            _need(t, name, dtype=torch.float32, ndim=4)
            if t.shape != (N, H, D, D):
                raise ValueError(f"{name} must be [{N}, {H}, {D}, {D}]")
    f32 = dict(dtype=torch.float32, device=q.device)
    out = dict(grads) if grads is not None else {}
    for name in ("dq", "dk", "dv", "dg"):
        out.setdefault(name, torch.empty((T, H, D), **f32))
    out.setdefault("dbeta", torch.empty((T, H), **f32))
    if want_dinitial:
        out.setdefault("dinitial_state", torch.empty((N, H, D, D), **f32))
    else:
        out["dinitial_state"] = None
    shapes = {"dq": (T, H, D), "dk": (T, H, D), "dv": (T, H, D), "dg": (T, H, D),
              "dbeta": (T, H), "dinitial_state": (N, H, D, D)}
    for name, shape in shapes.items():  # caller-supplied outputs: the kernels trust them
        t = out[name]
        if t is None:
            continue
        _need(t, name, dtype=torch.float32, ndim=len(shape))
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}")
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1)
    a = ChunkBwdArgs()
    host = None
    a.num_seqs = N
    if cu_seqlens_host is not None:
        host = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
        a.cu_seqlens_host = host
        a.cu_seqlens = cu_seqlens.data_ptr()
    else:
        if T % N:
            raise ValueError("T_total must be a multiple of the number of sequences")
        a.seq_len = T // N
    a.num_heads, a.head_dim = H, D
    a.io_dtype = _dtype_code(q.dtype)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g, a.beta, a.dO = (t.data_ptr() for t in (q, k, v, g, beta, dO))
    a.initial_state = None if initial_state is None else initial_state.data_ptr()
    a.dfinal_state = None if dfinal_state is None else dfinal_state.data_ptr()
    a.dq, a.dk, a.dv, a.dg, a.dbeta = (out[n].data_ptr() for n in ("dq", "dk", "dv", "dg",
                                                                     "dbeta"))
    a.dinitial_state = None if out["dinitial_state"] is None else out["dinitial_state"].data_ptr()
    if workspace is None:
        full, least = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _check(lib.kda_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(full)),
               "kda_chunk_bwd_workspace_size")
        _check(lib.kda_chunk_bwd_min_workspace_size(ctypes.byref(a), ctypes.byref(least)),
               "kda_chunk_bwd_min_workspace_size")
        size = full.value
        if max_workspace_bytes is not None:
            size = max(least.value, min(size, int(max_workspace_bytes)))
        workspace = torch.empty(max(size, 1), dtype=torch.uint8, device=q.device)
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _check(lib.kda_chunk_bwd(ctypes.byref(a), _stream(q)), "kda_chunk_bwd")
    del host
    return out


def recurrent_step(q, k, v, g, beta, state, state_indices=None, scale=1.0, out=None,
                   A_log=None, dt_bias=None, lower_bound=-5.0, beta_logits=False):
    """One decode token per row, applied in place to ``state`` ([slots, H, 128, 128] fp32).

    q, k, v: [B, H, 128]; g: [B, H, 128] fp32; beta: [B, H] fp32;
    state_indices: int32 [B] (slot per row; negative = skip) or None (identity).
    A_log, dt_bias, lower_bound, beta_logits: the gate front end, as in chunk_fwd.
    Returns o [B, H, 128].
    """
    lib = library()
    _need(q, "q", ndim=3)
    for name, t in (("k", k), ("v", v)):
        _need(t, name, dtype=q.dtype, ndim=3)
    _need(g, "g", dtype=torch.float32, ndim=3)
    _need(beta, "beta", dtype=torch.float32, ndim=2)
    _need(state, "state", dtype=torch.float32, ndim=4)
    B, H, D = q.shape
    if state_indices is not None:
        _need(state_indices, "state_indices", dtype=torch.int32, ndim=1)
    o = _out_like(out, q)
    a = RecurrentStepArgs()
    a.batch, a.num_heads, a.head_dim = B, H, D
    a.io_dtype = _dtype_code(q.dtype)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g, a.beta = (t.data_ptr() for t in (q, k, v, g, beta))
    a.state = state.data_ptr()
    a.state_indices = None if state_indices is None else state_indices.data_ptr()
    a.num_slots = state.shape[0]
    a.o = o.data_ptr()
    a.gate = _gate(H, A_log, dt_bias, lower_bound, beta_logits)
    _check(lib.kda_recurrent_step(ctypes.byref(a), _stream(q)), "kda_recurrent_step")
    return o


def _fused_args(q, k, v, g, beta, state, conv_cache, conv_weight, state_indices, scale,
                l2_eps, out_norm, norm_weight, norm_eps, o, A_log, dt_bias, lower_bound,
                beta_logits, token_dims):
    """Check and fill kda_fused_step_args; q, k, v, g are [B, (T,) H, 128]."""
    _need(q, "q", ndim=token_dims + 1)
    for name, t in (("k", k), ("v", v)):
        _need(t, name, dtype=q.dtype, ndim=token_dims + 1)
    _need(g, "g", dtype=torch.float32, ndim=token_dims + 1)
    _need(beta, "beta", dtype=torch.float32, ndim=token_dims)
    _need(state, "state", dtype=torch.float32, ndim=4)
    _need(conv_cache, "conv_cache", dtype=q.dtype, ndim=5)
    _need(conv_weight, "conv_weight", dtype=torch.float32, ndim=4)
    B, H, D = q.shape[0], q.shape[-2], q.shape[-1]
    if k.shape != q.shape or v.shape != q.shape or g.shape != q.shape or \
            beta.shape != q.shape[:-1]:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if conv_cache.shape[1:] != (3, CONV_WIDTH - 1, H, D) or conv_cache.shape[0] != state.shape[0]:
        raise ValueError(f"conv_cache must be [{state.shape[0]}, 3, {CONV_WIDTH - 1}, {H}, {D}]")
    if conv_weight.shape != (3, H, D, CONV_WIDTH):
        raise ValueError(f"conv_weight must be [3, {H}, {D}, {CONV_WIDTH}]")
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", dtype=torch.float32)
        if norm_weight.numel() != D:
            raise ValueError(f"norm_weight must hold {D} values")
    if state_indices is not None:
        _need(state_indices, "state_indices", dtype=torch.int32, ndim=1)
    a = FusedStepArgs()
    a.batch, a.num_heads, a.head_dim = B, H, D
    a.io_dtype = _dtype_code(q.dtype)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g, a.beta = (t.data_ptr() for t in (q, k, v, g, beta))
    a.conv_weight, a.conv_cache = conv_weight.data_ptr(), conv_cache.data_ptr()
    a.state = state.data_ptr()
    a.state_indices = None if state_indices is None else state_indices.data_ptr()
    a.num_slots = state.shape[0]
    a.l2_eps, a.out_norm, a.norm_eps = float(l2_eps), 1 if out_norm else 0, float(norm_eps)
    a.norm_weight = None if norm_weight is None else norm_weight.data_ptr()
    a.o = o.data_ptr()
    a.gate = _gate(H, A_log, dt_bias, lower_bound, beta_logits)
    return a


def fused_decode_step(q, k, v, g, beta, state, conv_cache, conv_weight, state_indices=None,
                      scale=1.0, l2_eps=1e-6, out_norm=True, norm_weight=None, norm_eps=1e-6,
                      out=None, A_log=None, dt_bias=None, lower_bound=-5.0, beta_logits=False):
    """One decode token per row with the front end (short convolution of q, k, v
    continuing from ``conv_cache``, Swish, L2 norm of q and k), the recurrence and
    the output RMSNorm, in one kernel; ``state`` and ``conv_cache`` are updated in
    place.

    q, k, v: [B, H, 128] raw projections (bf16 or fp32); g: [B, H, 128] fp32;
    beta: [B, H] fp32; state: [slots, H, 128, 128] fp32; conv_cache:
    [slots, 3, 3, H, 128] in q's dtype; conv_weight: [3, H, 128, 4] fp32;
    norm_weight: [128] fp32 or None.  The gate arguments are those of chunk_fwd.
    Returns o [B, H, 128].
    """
    lib = library()
    o = _out_like(out, q)
    a = _fused_args(q, k, v, g, beta, state, conv_cache, conv_weight, state_indices, scale,
                    l2_eps, out_norm, norm_weight, norm_eps, o, A_log, dt_bias, lower_bound,
                    beta_logits, token_dims=2)
    _check(lib.kda_fused_decode_step(ctypes.byref(a), _stream(q)), "kda_fused_decode_step")
    return o


def spec_verify_step(q, k, v, g, beta, state, conv_cache, conv_weight, replay=None,
                     num_replay=None, state_indices=None, scale=1.0, l2_eps=1e-6,
                     out_norm=True, norm_weight=None, norm_eps=1e-6, out=None, A_log=None,
                     dt_bias=None, lower_bound=-5.0, beta_logits=False):
    """Speculative-decode verification with replay, one kernel.

    q, k, v, g: [B, T, H, 128] the new window (raw projections, log-decay or gate
    logits); beta: [B, T, H].  ``replay``: dict of the previous window's q, k, v,
    g [B, Tr, H, 128] and beta [B, Tr, H], or None; ``num_replay``: int32 [B] on
    the device (accepted tokens of the replay window, clamped to [0, Tr]) or None
    for all.  The accepted replay tokens advance ``state`` and ``conv_cache`` in
    place; the new window's outputs are returned ([B, T, H, 128]) and its state
    is dropped.  Other arguments as in fused_decode_step.
    """
    lib = library()
    o = _out_like(out, q)
    a = _fused_args(q, k, v, g, beta, state, conv_cache, conv_weight, state_indices, scale,
                    l2_eps, out_norm, norm_weight, norm_eps, o, A_log, dt_bias, lower_bound,
                    beta_logits, token_dims=3)
    va = SpecVerifyArgs()
    va.step = a
    va.window = q.shape[1]
    if replay is not None:
        rq = replay["q"]
        _need(rq, "replay q", dtype=q.dtype, ndim=4)
        if rq.shape[0] != q.shape[0] or rq.shape[2:] != q.shape[2:]:
            raise ValueError("replay window must be [B, Tr, H, 128]")
        for name in ("k", "v"):
            _need(replay[name], f"replay {name}", dtype=q.dtype, ndim=4)
            if replay[name].shape != rq.shape:
                raise ValueError("replay shape mismatch")
        _need(replay["g"], "replay g", dtype=torch.float32, ndim=4)
        _need(replay["beta"], "replay beta", dtype=torch.float32, ndim=3)
        if replay["g"].shape != rq.shape or replay["beta"].shape != rq.shape[:-1]:
            raise ValueError("replay shape mismatch")
        va.replay_q, va.replay_k, va.replay_v = (replay[n].data_ptr() for n in ("q", "k", "v"))
        va.replay_g, va.replay_beta = replay["g"].data_ptr(), replay["beta"].data_ptr()
        va.replay_window = rq.shape[1]
    if num_replay is not None:
        _need(num_replay, "num_replay", dtype=torch.int32, ndim=1)
        va.num_replay = num_replay.data_ptr()
    _check(lib.kda_spec_verify_step(ctypes.byref(va), _stream(q)), "kda_spec_verify_step")
    return o


def conv_cache_bytes(num_heads: int, head_dim: int = 128,
                     dtype: torch.dtype = torch.bfloat16) -> int:
    return int(library().kda_conv_cache_bytes(num_heads, head_dim, _dtype_code(dtype)))


def state_io(op: int, dst, src=None, indices=None, count=None):
    """Zero / copy / gather / scatter states between pools ([slots, H, 128, 128])."""
    lib = library()
    _need(dst, "dst", ndim=4)
    if src is not None:
        _need(src, "src", ndim=4)
    if indices is not None:
        _need(indices, "indices", dtype=torch.int32, ndim=1)
    H, D = dst.shape[1], dst.shape[2]
    if count is None:
        count = indices.shape[0] if indices is not None else (
            src.shape[0] if src is not None and op == STATE_COPY else dst.shape[0])
    st = lib.kda_state_io(int(op), _ptr(src), _dtype_code(src.dtype) if src is not None else 0,
                          src.shape[0] if src is not None else 0, _ptr(dst),
                          _dtype_code(dst.dtype), dst.shape[0], _ptr(indices), int(count), H, D,
                          _stream(dst))
    _check(st, "kda_state_io")
    return dst


def state_bytes(num_heads: int, head_dim: int = 128, dtype: torch.dtype = torch.float32) -> int:
    return int(library().kda_state_bytes(num_heads, head_dim, _dtype_code(dtype)))
