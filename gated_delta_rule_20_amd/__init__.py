"""MI355X-native Kimi Delta Attention (KDA) core.

A thin ctypes binding over ``libkda.so`` (C ABI in ``include/kda.h``).  It
only marshals arguments: every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no
fallback: if the library is missing or the tensors are not on a ROCm device,
the calls raise.

"Kimi K3 Technical Report: Open Frontier Intelligence", §2.1.1 eq. (1) (the
recurrence), eqs. (3)-(4) (chunkwise form), eq. (5) (gate).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "NOALLOC_WORKSPACE_BYTES", "recurrent_step", "recurrent_replay", "chunk_fwd_workspace_size", "load_library",
           "Fusion", "KDAError", "LIB_PATH", "EXPORTED_SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")
EXPORTED_SYMBOLS = ("kda_chunk_fwd_workspace_size", "kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_recurrent_step",
                    "kda_recurrent_replay", "kda_status_string", "kda_last_error_message")

KDA_F32, KDA_BF16 = 0, 1
_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class KDAError(RuntimeError):
    """A kda_* call returned a non-success status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


class LayerFusion(ctypes.Structure):
    _fields_ = [("conv_width", ctypes.c_int32), ("conv_weight", ctypes.c_void_p),
                ("conv_state", ctypes.c_void_p), ("conv_state_out", ctypes.c_void_p),
                ("conv_checkpoints", ctypes.c_void_p), ("qk_norm_eps", ctypes.c_float),
                ("gate", ctypes.c_void_p), ("o_norm_weight", ctypes.c_void_p), ("o_norm_eps", ctypes.c_float)]


class ChunkFwdArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("g_min", ctypes.c_float), ("scale", ctypes.c_float),
                ("cu_seqlens", ctypes.c_void_p), ("N", ctypes.c_int32),
                ("initial_state", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("final_state", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("checkpoints", ctypes.c_void_p),
                ("checkpoint_every", ctypes.c_int32), ("checkpoint_slots", ctypes.c_int32),
                ("fusion", ctypes.POINTER(LayerFusion))]


class StepArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("H", ctypes.c_int32), ("Dk", ctypes.c_int32),
                ("Dv", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("g_min", ctypes.c_float), ("scale", ctypes.c_float),
                ("state", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("fusion", ctypes.POINTER(LayerFusion))]


class ReplayArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("H", ctypes.c_int32), ("Dk", ctypes.c_int32),
                ("Dv", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("T_replay", ctypes.c_int32), ("T_new", ctypes.c_int32), ("n_commit", ctypes.c_int32),
                ("k_r", ctypes.c_void_p), ("v_r", ctypes.c_void_p), ("g_r", ctypes.c_void_p),
                ("beta_r", ctypes.c_void_p), ("n_replay", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("g_min", ctypes.c_float), ("scale", ctypes.c_float),
                ("state", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("q_r", ctypes.c_void_p), ("fusion", ctypes.POINTER(LayerFusion))]


class Fusion:
    """The layer's prologue (eq. (2)) and epilogue (eq. (6)) fused into a call.

    Prologue (on when ``conv_weight`` is given, [H, 2*Dk + Dv, W] fp32, W <= 4):
    q, k, v are the projections before the short convolution and beta holds
    logits; the kernels apply ShortConv, Swish, L2Norm (q, k; eps ``qk_eps``)
    and Sigmoid (beta).  ``conv_state`` [N, H, W-1, 2*Dk + Dv] in the input
    dtype: read by chunk_fwd (None = zeros), updated in place by the decode
    calls.  chunk_fwd also takes ``conv_state_out`` and, with checkpoints,
    ``conv_checkpoints`` [N, slots, H, W-1, 2*Dk + Dv].
    Epilogue (on when ``gate`` is given, logits shaped like the output):
    the output becomes Sigmoid(gate) * RMSNorm(o~) with per-head weights
    ``o_norm_weight`` [H, Dv] fp32 and eps ``o_eps``.
    """

    def __init__(self, conv_weight=None, conv_state=None, conv_state_out=None, conv_checkpoints=None,
                 qk_eps: float = 1e-6, gate=None, o_norm_weight=None, o_eps: float = 1e-6):
        self.conv_weight, self.conv_state = conv_weight, conv_state
        self.conv_state_out, self.conv_checkpoints = conv_state_out, conv_checkpoints
        self.qk_eps, self.gate, self.o_norm_weight, self.o_eps = qk_eps, gate, o_norm_weight, o_eps

    def _args(self, N, H, Dk, Dv, dtype, out_shape, slots=None):
        """Checked ctypes view; shapes are verified here since the ABI takes bare pointers."""
        f = LayerFusion()
        C = 2 * Dk + Dv
        if self.conv_weight is not None:
            w = _dev(self.conv_weight, "conv_weight", torch.float32)
            if w.dim() != 3 or tuple(w.shape[:2]) != (H, C) or not 1 <= w.shape[2] <= 4:
                raise ValueError(f"conv_weight must be [H, 2*Dk + Dv, W] = [{H}, {C}, 1..4], got {tuple(w.shape)}")
            W = w.shape[2]
            for name, t, lead in (("conv_state", self.conv_state, (N, H)),
                                  ("conv_state_out", self.conv_state_out, (N, H)),
                                  ("conv_checkpoints", self.conv_checkpoints, None)):
                if t is None:
                    continue
                _dev(t, name, dtype)
                want = (N, H, W - 1, C) if lead else (N, slots, H, W - 1, C)
                if slots is None and lead is None:
                    raise ValueError("conv_checkpoints needs checkpoints")
                if tuple(t.shape) != want:
                    raise ValueError(f"{name} must be {want}, got {tuple(t.shape)}")
            f.conv_width = W
            f.conv_weight = _ptr(w)
            f.conv_state, f.conv_state_out = _ptr(self.conv_state), _ptr(self.conv_state_out)
            f.conv_checkpoints = _ptr(self.conv_checkpoints)
            f.qk_norm_eps = float(self.qk_eps)
        elif any(t is not None for t in (self.conv_state, self.conv_state_out, self.conv_checkpoints)):
            raise ValueError("convolution buffers given without conv_weight")
        if self.gate is not None:
            _dev(self.gate, "gate", dtype)
            if tuple(self.gate.shape) != tuple(out_shape):
                raise ValueError(f"gate must have the output's shape {tuple(out_shape)}, got {tuple(self.gate.shape)}")
            wo = _dev(self.o_norm_weight, "o_norm_weight", torch.float32)
            if wo is None or tuple(wo.shape) != (H, Dv):
                raise ValueError(f"o_norm_weight must be [H, Dv] = {(H, Dv)}")
            f.gate, f.o_norm_weight, f.o_norm_eps = _ptr(self.gate), _ptr(wo), float(self.o_eps)
        return f

    @property
    def prologue(self) -> bool:
        return self.conv_weight is not None


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} not found: build it with gated_delta_rule_20_amd.build.build()")
    lib = ctypes.CDLL(path)
    lib.kda_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(ChunkFwdArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_fwd.argtypes = [ctypes.POINTER(ChunkFwdArgs), ctypes.c_void_p]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkFwdArgs), ctypes.c_void_p]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_recurrent_step.argtypes = [ctypes.POINTER(StepArgs), ctypes.c_void_p]
    lib.kda_recurrent_step.restype = ctypes.c_int
    lib.kda_recurrent_replay.argtypes = [ctypes.POINTER(ReplayArgs), ctypes.c_void_p]
    lib.kda_recurrent_replay.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error_message.argtypes = []
    lib.kda_last_error_message.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(lib, fn, status):
    if status != 0:
        raise KDAError(fn, status, lib.kda_last_error_message().decode() or
                       lib.kda_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _same_lead(q, k, v, g, beta, A_log, H):
    """q, k, g share one shape; v and beta share its leading axes; A_log is [H]."""
    if k.shape != q.shape or g.shape != q.shape:
        raise ValueError(f"k and g must have q's shape {tuple(q.shape)}, got {tuple(k.shape)}, {tuple(g.shape)}")
    if v.shape[:-1] != q.shape[:-1] or beta.shape != q.shape[:-1]:
        raise ValueError(f"v must be [..., Dv] and beta [...] over q's leading axes {tuple(q.shape[:-1])}, "
                         f"got {tuple(v.shape)}, {tuple(beta.shape)}")
    if A_log is not None and A_log.numel() != H:
        raise ValueError(f"A_log must have H = {H} entries, got {A_log.numel()}")


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _chunk_args(q, k, v, g, beta, A_log, g_min, scale, cu_seqlens, N, h0, o, hT, ws, ws_bytes,
                ckpt=None, ckpt_every=0):
    if cu_seqlens is not None:
        T, H, Dk = q.shape[-3:]
        B = 1
    else:
        B, T, H, Dk = q.shape
    a = ChunkFwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv = B, T, H, Dk, v.shape[-1]
    a.dtype = _DTYPES[q.dtype]
    a.q, a.k, a.v, a.g, a.beta = (_ptr(x) for x in (q, k, v, g, beta))
    a.A_log = _ptr(A_log)
    a.g_min, a.scale = float(g_min), float(scale)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.N = int(N)
    a.initial_state, a.o, a.final_state = _ptr(h0), _ptr(o), _ptr(hT)
    a.workspace, a.workspace_bytes = _ptr(ws), int(ws_bytes)
    a.checkpoints = _ptr(ckpt)
    a.checkpoint_every = int(ckpt_every) if ckpt is not None else 0
    a.checkpoint_slots = int(ckpt.shape[1]) if ckpt is not None else 0
    return a


def chunk_fwd_workspace_size(q, v, *, cu_seqlens=None, N=None, prologue: bool = False) -> int:
    """Workspace bytes kda_chunk_fwd needs for q [B,T,H,Dk] (or [T,H,Dk] with
    cu_seqlens) and v [..., Dv]; ``prologue``: a fusion with the eq. (2)
    prologue on (passed through; the prologue needs no workspace)."""
    lib = load_library()
    n = (cu_seqlens.numel() - 1) if cu_seqlens is not None else 0
    a = _chunk_args(q, q, v, q, q, None, -5.0, 1.0, cu_seqlens, N if N is not None else n,
                    None, None, None, None, 0)
    if prologue:
        f = LayerFusion()
        f.conv_width = 1
        a.fusion = ctypes.pointer(f)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    out = ctypes.c_size_t(0)
    _check(lib, "kda_chunk_fwd_workspace_size", lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(out)))
    return out.value


def chunk_fwd(q, k, v, g, beta, *, A_log=None, g_min: float = -5.0, scale: float = 1.0,
              cu_seqlens=None, initial_state=None, output_final_state: bool = True,
              out=None, final_state=None, workspace=None, stream=None,
              checkpoints=None, checkpoint_every: int = 0, fusion: Fusion | None = None):
    """Chunkwise-parallel KDA forward (``kda_chunk_fwd``).

    q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H] (bf16 or fp32).
    With cu_seqlens ([N+1] int32 on device) the token axis is packed: pass
    [T, H, D] / [T, H] (or with a leading 1).  ``g`` holds log-decays, or
    decay logits z when ``A_log`` ([H] fp32) is given (eq. (5) gate in-kernel).
    initial_state / final_state: [N, H, Dk, Dv] fp32 (final_state may be the
    same tensor as initial_state for in-place resume).
    checkpoints: optional [N, slots, H, Dk, Dv] fp32; slot j receives the state
    after (j + 1) * checkpoint_every * 64 tokens of each sequence when that
    position lies strictly inside it (other slots are left as they are).
    fusion: optional :class:`Fusion` (layer prologue / epilogue in the kernels).
    Returns (o, final_state or None).
    """
    lib = load_library()
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _dev(t, name, q.dtype)
    _dev(A_log, "A_log", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(initial_state, "initial_state", torch.float32)
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        H, Dk = q.shape[-2:]
    else:
        N = q.shape[0]
        H, Dk = q.shape[2], q.shape[3]
    Dv = v.shape[-1]
    _same_lead(q, k, v, g, beta, A_log, H)
    if out is None:
        out = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    _dev(out, "out", q.dtype)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _dev(final_state, "final_state", torch.float32)
    _dev(checkpoints, "checkpoints", torch.float32)
    # The C ABI takes bare pointers: sizes are checked here, before the launch.
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and tuple(t.shape) != (N, H, Dk, Dv):
            raise ValueError(f"{name} must be [N, H, Dk, Dv] = {(N, H, Dk, Dv)}, got {tuple(t.shape)}")
    if out.shape != v.shape:
        raise ValueError(f"out must have v's shape {tuple(v.shape)}, got {tuple(out.shape)}")
    if checkpoints is not None:
        if (checkpoints.dim() != 5 or checkpoints.shape[0] != N or checkpoints.shape[1] < 1
                or tuple(checkpoints.shape[2:]) != (H, Dk, Dv) or checkpoint_every < 1):
            raise ValueError(f"checkpoints must be [N, slots >= 1, H, Dk, Dv] with N, H, Dk, Dv = "
                             f"{(N, H, Dk, Dv)} and checkpoint_every >= 1; got {tuple(checkpoints.shape)}, "
                             f"every={checkpoint_every}")
    if workspace is _NO_WORKSPACE:  # kda_chunk_fwd_noalloc: the library's own fixed array
        fn, workspace, ws_bytes = "kda_chunk_fwd_noalloc", None, 0
    else:
        fn = "kda_chunk_fwd"
        need = chunk_fwd_workspace_size(q, v, cu_seqlens=cu_seqlens, N=N,
                                        prologue=fusion is not None and fusion.prologue)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a = _chunk_args(q, k, v, g, beta, A_log, g_min, scale, cu_seqlens, N, initial_state,
                    out, final_state, workspace, ws_bytes, checkpoints, checkpoint_every)
    if fusion is not None:
        fa = fusion._args(N, H, Dk, Dv, q.dtype, out.shape,
                          slots=None if checkpoints is None else checkpoints.shape[1])
        a.fusion = ctypes.pointer(fa)
    _check(lib, fn, getattr(lib, fn)(ctypes.byref(a), _stream(stream, q.device)))
    return out, final_state


_NO_WORKSPACE = object()
NOALLOC_WORKSPACE_BYTES = 64 << 20  # KDA_NOALLOC_WORKSPACE_BYTES


def chunk_fwd_noalloc(q, k, v, g, beta, *, out, final_state=None, A_log=None, g_min: float = -5.0,
                      scale: float = 1.0, cu_seqlens=None, initial_state=None, stream=None,
                      checkpoints=None, checkpoint_every: int = 0, fusion: Fusion | None = None):
    """``kda_chunk_fwd_noalloc``: :func:`chunk_fwd` with the library's fixed
    device workspace (NOALLOC_WORKSPACE_BYTES per device) instead of one the
    caller provides.  Nothing is allocated: ``out`` is required and
    ``final_state`` is written only when given.  Shapes that need a larger
    workspace raise KDAError (KDA_ERROR_WORKSPACE).  Calls that overlap on one
    device share the array and race."""
    return chunk_fwd(q, k, v, g, beta, A_log=A_log, g_min=g_min, scale=scale, cu_seqlens=cu_seqlens,
                     initial_state=initial_state, output_final_state=False, out=out,
                     final_state=final_state, workspace=_NO_WORKSPACE, stream=stream,
                     checkpoints=checkpoints, checkpoint_every=checkpoint_every, fusion=fusion)


def recurrent_step(q, k, v, g, beta, state, *, A_log=None, g_min: float = -5.0,
                   scale: float = 1.0, out=None, stream=None, fusion: Fusion | None = None):
    """One decode token per sequence, state [N, H, Dk, Dv] fp32 updated in
    place.  q, k, g: [N, H, Dk]; v: [N, H, Dv]; beta: [N, H].  ``fusion``: optional
    :class:`Fusion` (its conv_state is updated in place too).  Returns o."""
    lib = load_library()
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _dev(t, name, q.dtype)
    _dev(state, "state", torch.float32)
    _dev(A_log, "A_log", torch.float32)
    if q.dim() != 3:
        raise ValueError(f"q must be [N, H, Dk], got {tuple(q.shape)}")
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    _same_lead(q, k, v, g, beta, A_log, H)
    if tuple(state.shape) != (N, H, Dk, Dv):
        raise ValueError(f"state must be [N, H, Dk, Dv] = {(N, H, Dk, Dv)}, got {tuple(state.shape)}")
    if out is None:
        out = torch.empty((N, H, Dv), dtype=q.dtype, device=q.device)
    _dev(out, "out", q.dtype)
    if out.shape != v.shape:
        raise ValueError(f"out must have v's shape {tuple(v.shape)}, got {tuple(out.shape)}")
    a = StepArgs()
    a.N, a.H, a.Dk, a.Dv, a.dtype = N, H, Dk, Dv, _DTYPES[q.dtype]
    a.q, a.k, a.v, a.g, a.beta = (_ptr(x) for x in (q, k, v, g, beta))
    a.A_log = _ptr(A_log)
    a.g_min, a.scale = float(g_min), float(scale)
    a.state, a.o = _ptr(state), _ptr(out)
    if fusion is not None:
        fa = fusion._args(N, H, Dk, Dv, q.dtype, out.shape)
        a.fusion = ctypes.pointer(fa)
    _check(lib, "kda_recurrent_step", lib.kda_recurrent_step(ctypes.byref(a), _stream(stream, q.device)))
    return out


def recurrent_replay(q, k, v, g, beta, state, *, replay=None, n_replay=None, n_commit=None,
                     A_log=None, g_min: float = -5.0, scale: float = 1.0, out=None, stream=None,
                     q_r=None, fusion: Fusion | None = None):
    """Speculative-decoding step with replay, state [N, H, Dk, Dv] fp32 in place.

    New window: q, k, g [N, T, H, Dk]; v [N, T, H, Dv]; beta [N, T, H] (T may be 0
    when all are None).  ``replay``: optional cached window (k_r, v_r, g_r, beta_r)
    of shapes [N, Tr, H, ...]; ``n_replay`` ([N] int32 on the device, or None = Tr)
    tokens of it are replayed first, without output.  The state written back is
    the one after the replayed tokens and the first ``n_commit`` new tokens
    (default: all of them).  ``fusion``: optional :class:`Fusion`; with its
    prologue the replayed window's query projections ``q_r`` [N, Tr, H, Dk] are
    needed too.  Returns o [N, T, H, Dv] (None when T = 0)."""
    lib = load_library()
    ref = q if q is not None else replay[0]
    if ref.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {ref.dtype}")
    dt = ref.dtype
    _dev(state, "state", torch.float32)
    _dev(A_log, "A_log", torch.float32)
    N, H, Dk, Dv = state.shape
    T_new = 0
    if q is not None:
        for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
            _dev(t, name, dt)
        if q.dim() != 4 or q.shape[0] != N or q.shape[2:] != (H, Dk):
            raise ValueError(f"q must be [N, T, H, Dk] with N, H, Dk = {(N, H, Dk)}, got {tuple(q.shape)}")
        _same_lead(q, k, v, g, beta, A_log, H)
        if v.shape[-1] != Dv:
            raise ValueError(f"v must end in Dv = {Dv}, got {tuple(v.shape)}")
        T_new = q.shape[1]
        if out is None:
            out = torch.empty(v.shape, dtype=dt, device=q.device)
        _dev(out, "out", dt)
        if out.shape != v.shape:
            raise ValueError(f"out must have v's shape {tuple(v.shape)}, got {tuple(out.shape)}")
    n_commit = T_new if n_commit is None else int(n_commit)
    a = ReplayArgs()
    a.N, a.H, a.Dk, a.Dv, a.dtype = N, H, Dk, Dv, _DTYPES[dt]
    a.T_new, a.n_commit = T_new, n_commit
    a.T_replay = 0
    if replay is not None:
        k_r, v_r, g_r, beta_r = replay
        for name, t in (("k_r", k_r), ("v_r", v_r), ("g_r", g_r), ("beta_r", beta_r)):
            _dev(t, name, dt)
        if k_r.dim() != 4 or k_r.shape[0] != N or k_r.shape[2:] != (H, Dk):
            raise ValueError(f"k_r must be [N, Tr, H, Dk] with N, H, Dk = {(N, H, Dk)}, got {tuple(k_r.shape)}")
        _same_lead(k_r, k_r, v_r, g_r, beta_r, A_log, H)
        if v_r.shape[-1] != Dv:
            raise ValueError(f"v_r must end in Dv = {Dv}, got {tuple(v_r.shape)}")
        a.T_replay = k_r.shape[1]
        a.k_r, a.v_r, a.g_r, a.beta_r = (_ptr(x) for x in (k_r, v_r, g_r, beta_r))
        _dev(n_replay, "n_replay", torch.int32)
        if n_replay is not None and tuple(n_replay.shape) != (N,):
            raise ValueError(f"n_replay must be [N] = [{N}], got {tuple(n_replay.shape)}")
        a.n_replay = _ptr(n_replay)
    if q is not None:
        a.q, a.k, a.v, a.g, a.beta = (_ptr(x) for x in (q, k, v, g, beta))
        a.o = _ptr(out)
    a.A_log = _ptr(A_log)
    a.g_min, a.scale = float(g_min), float(scale)
    a.state = _ptr(state)
    if q_r is not None:
        _dev(q_r, "q_r", dt)
        if replay is None or q_r.shape != replay[0].shape:
            raise ValueError("q_r must have k_r's shape")
        a.q_r = _ptr(q_r)
    if fusion is not None:
        out_shape = out.shape if out is not None else (N, 0, H, Dv)
        fa = fusion._args(N, H, Dk, Dv, dt, out_shape)
        a.fusion = ctypes.pointer(fa)
    _check(lib, "kda_recurrent_replay", lib.kda_recurrent_replay(ctypes.byref(a), _stream(stream, state.device)))
    return out
