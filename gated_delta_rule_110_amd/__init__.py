"""libkda: the KDA chunked forward pass on gfx950, its decode step and its
gradient, and their thin Python binding.

The binding only marshals arguments: it checks dtypes, devices and
contiguity, allocates the output and workspace with torch when the caller
does not pass them, and calls ``kda_fwd`` from ``libkda.so`` through ctypes on
torch's current HIP stream.  Every step of the computation runs in the HIP
kernels; there is no CPU or PyTorch fallback, and a missing library is an
error.

``fwd`` takes its arguments in the order of the forward call described on
"Debajo del capó: CUTLASS en Hopper" (7minutos.es):
q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
final_state, cu_seqlens.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

from ._build import LIB as LIB_PATH
from ._build import build

__all__ = ["fwd", "fwd_noalloc", "noalloc_max_workspace", "decode", "bwd", "bwd_workspace_size",
           "kda_attention", "KdaFunction", "workspace_size", "chain_segments_for",
           "pipelined_for", "KdaArgumentError", "library", "KdaError", "build", "LIB_PATH", "KDA_BF16",
           "KDA_FP32"]

KDA_BF16 = 1
KDA_FP32 = 2
HEAD_DIM = 128

_STATUS_NAMES = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_UNSUPPORTED",
                 4: "KDA_ERR_PARAM", 5: "KDA_ERR_DTYPE", 6: "KDA_ERR_ALIGN",
                 7: "KDA_ERR_WORKSPACE", 8: "KDA_ERR_HIP", 9: "KDA_ERR_SCRATCH"}


class KdaError(RuntimeError):
    """A non-OK status from libkda; ``status`` holds the kda_status_t code."""

    def __init__(self, status: int, message: str):
        super().__init__("%s (%d): %s" % (_STATUS_NAMES.get(status, "?"), status, message))
        self.status = status


class KdaArgumentError(KdaError, ValueError):
    """A status the library returns for its arguments before launching anything
    (every status but KDA_ERR_HIP); also a ValueError."""


KDA_ERR_HIP = 8


def _raise_status(lib, st: int):
    msg = lib.kda_status_string(st).decode()
    raise (KdaError if st == KDA_ERR_HIP else KdaArgumentError)(st, msg)


class KdaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("K", ctypes.c_int64), ("V", ctypes.c_int64), ("num_seqs", ctypes.c_int64),
                ("initial_state_dtype", ctypes.c_int32), ("final_state_dtype", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("phase_events", ctypes.c_void_p), ("chain_segments", ctypes.c_int64),
                ("launch_piece", ctypes.c_int64), ("pipeline", ctypes.c_int64),
                ("forward_workspace", ctypes.c_void_p), ("save_states", ctypes.c_int64)]


_lock = threading.Lock()
_lib = None


def library() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by ``build()``); raises if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libkda.so is not built (%s); run gated_delta_rule_110_amd.build()"
                                   % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            P = ctypes.c_void_p
            lib.kda_fwd.restype = ctypes.c_int
            lib.kda_fwd.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_float,
                                    P, P, P, P, ctypes.POINTER(KdaDesc), P]
            lib.kda_fwd_noalloc.restype = ctypes.c_int
            lib.kda_fwd_noalloc.argtypes = lib.kda_fwd.argtypes
            lib.kda_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
            lib.kda_fwd_noalloc_max_workspace.argtypes = []
            lib.kda_decode.restype = ctypes.c_int
            lib.kda_decode.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_float,
                                       P, P, P, ctypes.POINTER(KdaDesc), P]
            lib.kda_fwd_workspace_size.restype = ctypes.c_size_t
            lib.kda_fwd_workspace_size.argtypes = [ctypes.POINTER(KdaDesc)]
            lib.kda_fwd_pipelined.restype = ctypes.c_int
            lib.kda_fwd_pipelined.argtypes = [ctypes.POINTER(KdaDesc)]
            lib.kda_fwd_chain_segments.restype = ctypes.c_int64
            lib.kda_fwd_chain_segments.argtypes = [ctypes.POINTER(KdaDesc)]
            lib.kda_bwd.restype = ctypes.c_int
            lib.kda_bwd.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_float, P, P, P, P,
                                    P, P, P, P, P, P, P, P, ctypes.POINTER(KdaDesc), P]
            lib.kda_bwd_workspace_size.restype = ctypes.c_size_t
            lib.kda_bwd_workspace_size.argtypes = [ctypes.POINTER(KdaDesc)]
            lib.kda_status_string.restype = ctypes.c_char_p
            lib.kda_status_string.argtypes = [ctypes.c_int]
            _lib = lib
    return _lib


def _desc(B, T, H, N, h0_dtype=0, ht_dtype=0, workspace=None, nbytes=0, chain_segments=0,
          launch_piece=0, pipeline=0, save_states=0) -> KdaDesc:
    return KdaDesc(B, T, H, HEAD_DIM, HEAD_DIM, N, h0_dtype, ht_dtype,
                   ctypes.c_void_p(workspace), nbytes, None, chain_segments, launch_piece, pipeline, None,
                   save_states)


def workspace_size(B: int, T: int, H: int, num_seqs: Optional[int] = None, chain_segments: int = 0,
                   pipeline: int = 0, save_states: bool = False) -> int:
    """Workspace bytes ``fwd`` needs for these shapes (and chain split, and
    the saved states with ``save_states``)."""
    d = _desc(B, T, H, B if num_seqs is None else num_seqs, chain_segments=chain_segments, pipeline=pipeline,
              save_states=int(bool(save_states)))
    return int(library().kda_fwd_workspace_size(ctypes.byref(d)))


def pipelined_for(B: int, T: int, H: int, chain_segments: int = 0, pipeline: int = 0) -> bool:
    """Whether ``fwd`` runs these shapes (without cu_seqlens) on the pipelined forward."""
    d = _desc(B, T, H, B, chain_segments=chain_segments, pipeline=pipeline)
    r = int(library().kda_fwd_pipelined(ctypes.byref(d)))
    if r < 0:
        raise ValueError("invalid shapes")
    return r == 1


def chain_segments_for(B: int, T: int, H: int, chain_segments: int = 0) -> int:
    """Segments ``fwd`` splits each state chain into for these shapes without cu_seqlens."""
    d = _desc(B, T, H, B, chain_segments=chain_segments)
    return int(library().kda_fwd_chain_segments(ctypes.byref(d)))


def _state_dtype(t: Optional[torch.Tensor], name: str) -> int:
    if t is None:
        return 0
    if t.dtype == torch.float32:
        return KDA_FP32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise ValueError("%s must be bf16 or fp32, got %s" % (name, t.dtype))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_fwd_args(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens,
                    chain_segments, launch_piece, allocate_out, pipeline=0):
    """Validate the forward's tensors and build its descriptor (no workspace yet).
    Returns ``(descriptor, device, out)``."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if t.dtype != torch.bfloat16:
            raise ValueError("%s must be bfloat16, got %s" % (name, t.dtype))
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t.dtype != torch.float32:
            raise ValueError("%s must be float32, got %s" % (name, t.dtype))
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or tuple(v.shape[:3]) != (B, T, H) or \
            tuple(beta.shape) != (B, T, H):
        raise ValueError("shape mismatch among q/k/v/g/beta")
    if tuple(A_log.shape) != (H,) or tuple(dt_bias.shape) != (H, K):
        raise ValueError("A_log must be [H] and dt_bias [H,K]")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int64 tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if out is None:
        if not allocate_out:
            raise ValueError("out must be given")
        out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=q.device)
    tensors = [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("out", out),
               ("A_log", A_log), ("dt_bias", dt_bias), ("initial_state", initial_state),
               ("final_state", final_state), ("cu_seqlens", cu_seqlens)]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    for name, t in tensors:
        if t is None:
            continue
        if t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (B, T, H, V):
        raise ValueError("out must be bf16 [B,T,H,V]")
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and tuple(t.shape) != (N, H, K, V):
            raise ValueError("%s must be [N,H,K,V] = %s" % (name, (N, H, K, V)))
    h0d = _state_dtype(initial_state, "initial_state")
    htd = _state_dtype(final_state, "final_state")
    d = _desc(B, T, H, N, h0d, htd, chain_segments=int(chain_segments), launch_piece=int(launch_piece),
              pipeline=int(pipeline))
    d.K, d.V = K, V
    return d, dev, out


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
        scale: float, out: Optional[torch.Tensor], A_log: torch.Tensor, dt_bias: torch.Tensor,
        lower_bound: float, initial_state: Optional[torch.Tensor] = None,
        final_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None,
        phase_events=None, chain_segments: int = 0,
        launch_piece: int = 0, pipeline: int = 0,
        save_states: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """KDA forward on the current HIP stream.  Returns ``(out, final_state)``.

    q, k, g: bf16 [B,T,H,128]; v: bf16 [B,T,H,128]; beta: bf16 logits [B,T,H];
    A_log: fp32 [H]; dt_bias: fp32 [H,128]; lower_bound in [-5, 0];
    initial_state / final_state: bf16 or fp32 [N,H,128,128] or None;
    cu_seqlens: int64 [N+1] on the device (then B == 1) or None;
    out: bf16 [B,T,H,128] or None (allocated); workspace: uint8 device tensor
    of at least ``workspace_size`` bytes or None (allocated); phase_events:
    None or the address of a caller-owned array of 4 hipEvent_t (instrumentation);
    chain_segments: 0 (automatic), 1 (never) or the number of segments each
    sequence's state chain is split into (batches without cu_seqlens);
    launch_piece: kda_desc_t::launch_piece (0: the library's launch size);
    pipeline: kda_desc_t::pipeline (0: the two-kernel forward, 1: the pipelined one where it applies);
    save_states: also store the state entering every chunk in the workspace,
    for ``bwd(..., forward_workspace=workspace, forward_states=True)``
    (``kda_desc_t::save_states``).
    """
    lib = library()
    d, dev, out = _check_fwd_args(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state,
                                  cu_seqlens, chain_segments, launch_piece, allocate_out=True,
                                  pipeline=pipeline)
    d.save_states = int(bool(save_states))
    need = int(lib.kda_fwd_workspace_size(ctypes.byref(d)))
    with torch.cuda.device(dev):
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
            raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
        d.workspace = ctypes.c_void_p(workspace.data_ptr())
        d.workspace_bytes = workspace.numel() * workspace.element_size()
        d.phase_events = phase_events
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                         _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                         _ptr(final_state), _ptr(cu_seqlens), _ptr(out), ctypes.byref(d),
                         ctypes.c_void_p(stream))
    if st != 0:
        _raise_status(lib, st)
    return out, final_state


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                scale: float, out: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor,
                lower_bound: float, initial_state: Optional[torch.Tensor] = None,
                final_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                chain_segments: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``kda_fwd_noalloc``: the forward of ``fwd`` in the library's static
    scratch, allocating nothing (``out`` must be given).  Calls that can
    overlap on one GPU share the scratch and race.  Returns ``(out, final_state)``."""
    lib = library()
    d, dev, out = _check_fwd_args(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state,
                                  cu_seqlens, chain_segments, 0, allocate_out=False)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.kda_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                 _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                                 _ptr(final_state), _ptr(cu_seqlens), _ptr(out), ctypes.byref(d),
                                 ctypes.c_void_p(stream))
    if st != 0:
        _raise_status(lib, st)
    return out, final_state


def noalloc_max_workspace() -> int:
    """Bytes of the static scratch ``fwd_noalloc`` runs in."""
    return int(library().kda_fwd_noalloc_max_workspace())


def bwd_workspace_size(B: int, T: int, H: int, num_seqs: Optional[int] = None, chain_segments: int = 0) -> int:
    """Workspace bytes ``bwd`` needs for these shapes."""
    d = _desc(B, T, H, B if num_seqs is None else num_seqs, chain_segments=chain_segments)
    return int(library().kda_bwd_workspace_size(ctypes.byref(d)))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
        scale: float, A_log: torch.Tensor, dt_bias: torch.Tensor, lower_bound: float,
        d_out: torch.Tensor, d_final_state: Optional[torch.Tensor] = None,
        initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, launch_piece: int = 0, chain_segments: int = 0,
        with_d_initial: bool = True, phase_events=None, outputs: Optional[dict] = None,
        forward_workspace: Optional[torch.Tensor] = None, forward_states: bool = False) -> dict:
    """Gradient of ``fwd`` (``kda_bwd``) on the current HIP stream: for the loss
    gradients ``d_out`` (bf16 [B,T,H,128]) and ``d_final_state`` (bf16 or fp32
    [N,H,128,128], or None for zeros) returns a dict of fp32 tensors dq, dk, dg
    ([B,T,H,128]), dv ([B,T,H,128]), dbeta ([B,T,H]), dA_log ([H]), ddt_bias
    ([H,128]) and d_initial_state ([N,H,128,128], or None without
    ``with_d_initial``).  Inputs as for ``fwd``, chain_segments included (the
    reverse chains split as the forward's do); phase_events: None or the
    address of a caller-owned array of 6 hipEvent_t (instrumentation);
    outputs: None, or a dict of caller-allocated fp32 tensors of those names and
    shapes that the call writes into (what graph capture needs);
    forward_workspace: None, or the ``workspace`` tensor of an earlier ``fwd``
    call on the same inputs, untouched since (its intermediates are read
    instead of recomputed: ``kda_desc_t::forward_workspace``);
    forward_states: that call ran with ``save_states`` and the same
    chain_segments, and its states are read as well (``kda_desc_t::save_states``)."""
    lib = library()
    d, dev, d_out = _check_fwd_args(q, k, v, g, beta, d_out, A_log, dt_bias, initial_state, d_final_state,
                                    cu_seqlens, chain_segments, launch_piece, allocate_out=False)
    B, T, H, K = q.shape
    N = d.num_seqs
    need = int(lib.kda_bwd_workspace_size(ctypes.byref(d)))
    f32 = dict(dtype=torch.float32, device=dev)
    shapes = {"dq": (B, T, H, K), "dk": (B, T, H, K), "dv": (B, T, H, K), "dg": (B, T, H, K), "dbeta": (B, T, H),
              "dA_log": (H,), "ddt_bias": (H, K), "d_initial_state": (N, H, K, K)}
    if outputs is None:
        res = {n: torch.empty(sh, **f32) for n, sh in shapes.items()}
        if not with_d_initial:
            res["d_initial_state"] = None
    else:
        res = dict(outputs)
        for n, sh in shapes.items():
            t = res.get(n)
            if t is None and n == "d_initial_state":
                res[n] = None
                continue
            if t is None or t.dtype != torch.float32 or tuple(t.shape) != sh or t.device != dev or \
                    not t.is_contiguous():
                raise ValueError("outputs[%r] must be a contiguous fp32 %s tensor on %s" % (n, sh, dev))
    with torch.cuda.device(dev):
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
            raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
        d.workspace = ctypes.c_void_p(workspace.data_ptr())
        d.workspace_bytes = workspace.numel() * workspace.element_size()
        d.phase_events = phase_events
        if forward_workspace is not None:
            # the intermediates end where the unsplit two-kernel forward's workspace does;
            # with the states, the forward's whole workspace
            fd = KdaDesc.from_buffer_copy(d)
            if forward_states:
                fd.save_states = 1
            else:
                fd.chain_segments = 1
            fd.pipeline = 0
            if forward_workspace.device != dev or \
                    forward_workspace.numel() * forward_workspace.element_size() < int(lib.kda_fwd_workspace_size(ctypes.byref(fd))):
                raise ValueError("forward_workspace must be the workspace of a fwd call on these shapes")
            d.forward_workspace = ctypes.c_void_p(forward_workspace.data_ptr())
            d.save_states = int(bool(forward_states))
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(A_log),
                         _ptr(dt_bias), float(lower_bound), _ptr(initial_state), _ptr(cu_seqlens), _ptr(d_out),
                         _ptr(d_final_state), _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dg"]),
                         _ptr(res["dbeta"]), _ptr(res["d_initial_state"]), _ptr(res["dA_log"]),
                         _ptr(res["ddt_bias"]), ctypes.byref(d), ctypes.c_void_p(stream))
    if st != 0:
        _raise_status(lib, st)
    return res


class KdaFunction(torch.autograd.Function):
    """``fwd`` with ``bwd`` as its gradient, for autograd.  Inputs as for ``fwd``
    (q, k, v, g, beta bf16; A_log, dt_bias fp32; initial_state bf16, fp32 or
    None); ``final_dtype`` is the dtype of the returned final state, or None for
    no final state.  The gradients come from one ``kda_bwd`` call, in fp32,
    cast to each input's dtype.  With ``keep_intermediates`` the forward also
    stores the state entering every chunk and its workspace (about 136.5 KiB
    per 64-token chunk and head) is held until the backward, which then reads
    the intermediates and the states from it instead of recomputing the
    forward (``kda_desc_t::forward_workspace``, ``kda_desc_t::save_states``)."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, A_log, dt_bias, initial_state, scale, lower_bound, cu_seqlens,
                final_dtype, chain_segments, keep_intermediates=False):
        final = None
        B, T, H, K = q.shape
        N = B if cu_seqlens is None else cu_seqlens.numel() - 1
        if final_dtype is not None:
            final = torch.empty((N, H, K, v.shape[-1]), dtype=final_dtype, device=q.device)
        ws = None
        # only when a backward can follow (otherwise the plain, faster forward)
        if keep_intermediates and any(ctx.needs_input_grad):
            ws = torch.empty(max(workspace_size(B, T, H, N, chain_segments=chain_segments, save_states=True), 1),
                             dtype=torch.uint8, device=q.device)
        out, fin = fwd(q, k, v, g, beta, scale, None, A_log, dt_bias, lower_bound, initial_state, final,
                       cu_seqlens, workspace=ws, chain_segments=chain_segments, save_states=ws is not None)
        ctx.save_for_backward(q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens)
        ctx.fwd_ws = ws
        ctx.scale, ctx.lower_bound, ctx.chain_segments = float(scale), float(lower_bound), int(chain_segments)
        return out, fin

    @staticmethod
    def backward(ctx, d_out, d_fin):
        q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens = ctx.saved_tensors
        if d_out is None:
            d_out = torch.zeros(v.shape, dtype=torch.bfloat16, device=v.device)
        d_out = d_out.to(torch.bfloat16).contiguous()
        if d_fin is not None:
            d_fin = d_fin.contiguous()
        want_h0 = initial_state is not None and ctx.needs_input_grad[7]
        res = bwd(q, k, v, g, beta, ctx.scale, A_log, dt_bias, ctx.lower_bound, d_out, d_final_state=d_fin,
                  initial_state=initial_state, cu_seqlens=cu_seqlens, chain_segments=ctx.chain_segments,
                  with_d_initial=want_h0, forward_workspace=ctx.fwd_ws, forward_states=ctx.fwd_ws is not None)
        ctx.fwd_ws = None
        d_h0 = res["d_initial_state"].to(initial_state.dtype) if want_h0 else None
        return (res["dq"].to(q.dtype), res["dk"].to(k.dtype), res["dv"].to(v.dtype), res["dg"].to(g.dtype),
                res["dbeta"].to(beta.dtype), res["dA_log"], res["ddt_bias"], d_h0,
                None, None, None, None, None, None)


def kda_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                  scale: float, A_log: torch.Tensor, dt_bias: torch.Tensor, lower_bound: float,
                  initial_state: Optional[torch.Tensor] = None, final_state_dtype: Optional[torch.dtype] = None,
                  cu_seqlens: Optional[torch.Tensor] = None,
                  chain_segments: int = 0,
                  keep_intermediates: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The KDA forward as an autograd operation (``KdaFunction``): returns
    ``(out, final_state)``, the final state in ``final_state_dtype`` (bf16 or
    fp32) or None, and backpropagates into q, k, v, g, beta, A_log, dt_bias and
    the initial state through ``kda_bwd``.  keep_intermediates: hold the
    forward's workspace until the backward (more memory, a shorter backward)."""
    return KdaFunction.apply(q, k, v, g, beta, A_log, dt_bias, initial_state, scale, lower_bound, cu_seqlens,
                             final_state_dtype, chain_segments, keep_intermediates)


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
           scale: float, out: Optional[torch.Tensor], A_log: torch.Tensor, dt_bias: torch.Tensor,
           lower_bound: float, initial_state: Optional[torch.Tensor] = None,
           final_state: Optional[torch.Tensor] = None,
           launch_piece: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One recurrent KDA step per sequence on the current HIP stream.

    q, k, g, v: bf16 [N,1,H,128]; beta: bf16 [N,1,H]; states: bf16 or fp32
    [N,H,128,128] or None (final_state may be the same tensor as
    initial_state for an in-place update); out: bf16 [N,1,H,128] or None;
    launch_piece: kda_desc_t::launch_piece (0: the library's launch size).
    Returns ``(out, final_state)``."""
    lib = library()
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if t.dtype != torch.bfloat16:
            raise ValueError("%s must be bfloat16, got %s" % (name, t.dtype))
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t.dtype != torch.float32:
            raise ValueError("%s must be float32, got %s" % (name, t.dtype))
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be [N,1,H,K]")
    N, _, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or tuple(v.shape[:3]) != (N, 1, H) or \
            tuple(beta.shape) != (N, 1, H):
        raise ValueError("shape mismatch among q/k/v/g/beta")
    if tuple(A_log.shape) != (H,) or tuple(dt_bias.shape) != (H, K):
        raise ValueError("A_log must be [H] and dt_bias [H,K]")
    if out is None:
        out = torch.empty((N, 1, H, V), dtype=torch.bfloat16, device=q.device)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("out", out), ("A_log", A_log),
                    ("dt_bias", dt_bias), ("initial_state", initial_state), ("final_state", final_state)):
        if t is None:
            continue
        if t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (N, 1, H, V):
        raise ValueError("out must be bf16 [N,1,H,V]")
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and tuple(t.shape) != (N, H, K, V):
            raise ValueError("%s must be [N,H,K,V] = %s" % (name, (N, H, K, V)))
    d = _desc(N, 1, H, N, _state_dtype(initial_state, "initial_state"), _state_dtype(final_state, "final_state"),
              launch_piece=int(launch_piece))
    d.K, d.V = K, V
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(A_log),
                            _ptr(dt_bias), float(lower_bound), _ptr(initial_state), _ptr(final_state),
                            _ptr(out), ctypes.byref(d), ctypes.c_void_p(stream))
    if st != 0:
        _raise_status(lib, st)
    return out, final_state
