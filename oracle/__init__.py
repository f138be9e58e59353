"""fp64 CPU oracle for the KDA forward pass and its gradient -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and it shares no code with the HIP path.

``fwd`` wraps the plain C token recurrence in ``kda_oracle.c`` (the definition,
written out in fp64); ``fwd_f64`` and ``bwd`` wrap ``kda_oracle_bwd.c``, the same
recurrence on fp64 inputs and its vector-Jacobian product run backwards over
the tokens; ``brute`` is an independent arbitrary-precision route
through explicit transition matrices, used only on tiny inputs to pin the C
code.  The gate reading, the L2-norm epsilon and every other choice the pages
leave open are stated in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_SRC_BWD = os.path.join(_HERE, "kda_oracle_bwd.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None

EPS = 1e-6  # the L2-norm epsilon the oracle adopts (stated in kda_oracle.c)


_CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"]


def build(force: bool = False) -> str:
    """Compile kda_oracle.c and kda_oracle_bwd.c with gcc (-O2, OpenMP, no fast-math)."""
    stamp = max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_BWD))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < stamp:
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc"] + _CFLAGS + [_SRC, _SRC_BWD, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, P, I64,
                                   D, P, P, D, P, P, P, ctypes.c_int]
    for name in ("kda_softplus", "kda_sigmoid"):
        getattr(lib, name).restype = D
        getattr(lib, name).argtypes = [D]
    lib.kda_gate.restype = D
    lib.kda_gate.argtypes = [D, D, D, D]
    # a variant built from kda_oracle.c alone (a planted forward mistake) has no gradient
    if hasattr(lib, "kda_oracle_bwd_f64"):
        lib.kda_oracle_fwd_f64.restype = ctypes.c_int
        lib.kda_oracle_fwd_f64.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, P, I64,
                                           D, P, P, D, P, P, P, ctypes.c_int]
        lib.kda_oracle_bwd_f64.restype = ctypes.c_int
        lib.kda_oracle_bwd_f64.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, P, I64,
                                           D, P, P, D, P, P, P,
                                           P, P, P, P, P, P, P, P, ctypes.c_int]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def compile_variant(src_text: str, out_path: str, bwd_text: str | None = None) -> str:
    """Compile C source text (e.g. kda_oracle.c with a planted mistake) the same
    way as the oracle; used by the tests that check the pins catch mistakes.
    With ``bwd_text`` (kda_oracle_bwd.c, possibly mutated) the gradient is
    compiled in as well."""
    srcs = [out_path + ".c"]
    with open(srcs[0], "w") as f:
        f.write(src_text)
    if bwd_text is not None:
        srcs.append(out_path + ".bwd.c")
        with open(srcs[1], "w") as f:
            f.write(bwd_text)
    subprocess.check_call(["gcc"] + _CFLAGS + srcs + ["-o", out_path, "-lm"])
    return out_path


def source() -> str:
    with open(_SRC) as f:
        return f.read()


def source_bwd() -> str:
    with open(_SRC_BWD) as f:
        return f.read()


class Oracle:
    """The oracle bound to one compiled library (the default one unless a path is given)."""

    def __init__(self, lib_path=None):
        self.lib = _load() if lib_path is None else _bind(ctypes.CDLL(lib_path))

    def fwd(self, *args, **kw):
        return _fwd(self.lib, *args, **kw)

    def fwd_f64(self, *args, **kw):
        return _fwd_f64(self.lib, *args, **kw)

    def bwd(self, *args, **kw):
        return _bwd(self.lib, *args, **kw)

    def gate(self, g, A_log, dt_bias, lower_bound):
        return self.lib.kda_gate(g, A_log, dt_bias, lower_bound)

    def softplus(self, x):
        return self.lib.kda_softplus(x)

    def sigmoid(self, x):
        return self.lib.kda_sigmoid(x)


def _bf16_bits(x) -> np.ndarray:
    """Raw bf16 bit patterns (uint16, C-contiguous) of a torch bf16 tensor or a uint16 array."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("numpy inputs must be uint16 bf16 bit patterns")
        return np.ascontiguousarray(x)
    import torch
    if x.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor, got %s" % x.dtype)
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _f64(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.float64)
    return np.ascontiguousarray(x.detach().cpu().double().numpy())


def _f32(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.float32)
    return np.ascontiguousarray(x.detach().cpu().float().numpy())


def fwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
        initial_state=None, cu_seqlens=None, num_threads: int = 0):
    """Run the oracle (see ``_fwd``)."""
    return _fwd(_load(), q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
                initial_state=initial_state, cu_seqlens=cu_seqlens, num_threads=num_threads)


def _fwd(lib, q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
         initial_state=None, cu_seqlens=None, num_threads: int = 0):
    """Run the oracle.  Returns ``(out, final_state)`` as fp64 numpy arrays of
    shapes [B,T,H,V] and [N,H,K,V].

    q,k,g: bf16 [B,T,H,K]; v: bf16 [B,T,H,V]; beta: bf16 [B,T,H];
    A_log fp32 [H]; dt_bias fp32 [H,K]; lower_bound and scale are floats
    (rounded to fp32 first, as the library receives them);
    initial_state: any float tensor [N,H,K,V] (converted exactly to fp64) or None;
    cu_seqlens: int64 [N+1] or None.
    """
    qb, kb, vb, gb, bb = (_bf16_bits(t) for t in (q, k, v, g, beta))
    B, T, H, K = qb.shape
    V = vb.shape[-1]
    assert kb.shape == qb.shape and gb.shape == qb.shape
    assert vb.shape == (B, T, H, V) and bb.shape == (B, T, H)
    A = _f32(A_log).reshape(H)
    dtb = _f32(dt_bias).reshape(H, K)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens if isinstance(cu_seqlens, np.ndarray)
                                             else cu_seqlens.cpu().numpy(), dtype=np.int64))
        N = cu.shape[0] - 1
    else:
        cu = None
        N = B
    h0 = None if initial_state is None else _f64(initial_state).reshape(N, H, K, V)
    out = np.zeros((B, T, H, V), dtype=np.float64)
    fin = np.zeros((N, H, K, V), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = lib.kda_oracle_fwd(ptr(qb), ptr(kb), ptr(vb), ptr(gb), ptr(bb), B, T, H, K, V,
                            ptr(cu), N, float(np.float32(scale)), ptr(A), ptr(dtb),
                            float(np.float32(lower_bound)), ptr(h0), ptr(fin), ptr(out),
                            int(num_threads))
    if rc != 0:
        raise ValueError("kda_oracle_fwd failed with code %d" % rc)
    return out, fin


def _cu_of(cu_seqlens, B):
    if cu_seqlens is None:
        return None, B
    if hasattr(cu_seqlens, "cpu"):
        cu_seqlens = cu_seqlens.cpu().numpy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    return cu, cu.shape[0] - 1


def _f64_inputs(q, k, v, g, beta, A_log, dt_bias):
    qd, kd, vd, gd, bd = (_f64(t) for t in (q, k, v, g, beta))
    B, T, H, K = qd.shape
    V = vd.shape[-1]
    assert kd.shape == qd.shape and gd.shape == qd.shape
    assert vd.shape == (B, T, H, V) and bd.shape == (B, T, H)
    return qd, kd, vd, gd, bd, _f64(A_log).reshape(H), _f64(dt_bias).reshape(H, K), (B, T, H, K, V)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd_f64(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
            initial_state=None, cu_seqlens=None, num_threads: int = 0):
    """The forward recurrence on fp64 inputs (see ``_fwd_f64``)."""
    return _fwd_f64(_load(), q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
                    initial_state=initial_state, cu_seqlens=cu_seqlens, num_threads=num_threads)


def _fwd_f64(lib, q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
             initial_state=None, cu_seqlens=None, num_threads: int = 0):
    """The forward recurrence with every input in fp64 (no bf16 rounding, scale
    and lower_bound used as given).  Shapes as ``fwd``; returns ``(out, final)``."""
    qd, kd, vd, gd, bd, A, dtb, (B, T, H, K, V) = _f64_inputs(q, k, v, g, beta, A_log, dt_bias)
    cu, N = _cu_of(cu_seqlens, B)
    h0 = None if initial_state is None else _f64(initial_state).reshape(N, H, K, V)
    out = np.zeros((B, T, H, V))
    fin = np.zeros((N, H, K, V))
    rc = lib.kda_oracle_fwd_f64(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(gd), _ptr(bd), B, T, H, K, V, _ptr(cu), N,
                                float(scale), _ptr(A), _ptr(dtb), float(lower_bound), _ptr(h0), _ptr(fin),
                                _ptr(out), int(num_threads))
    if rc != 0:
        raise ValueError("kda_oracle_fwd_f64 failed with code %d" % rc)
    return out, fin


def bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, d_final=None,
        initial_state=None, cu_seqlens=None, num_threads: int = 0):
    """The gradient of the forward pass (see ``_bwd``)."""
    return _bwd(_load(), q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, d_final=d_final,
                initial_state=initial_state, cu_seqlens=cu_seqlens, num_threads=num_threads)


def _bwd(lib, q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, d_final=None,
         initial_state=None, cu_seqlens=None, num_threads: int = 0):
    """Vector-Jacobian product of ``fwd_f64``: given the loss gradients ``d_out``
    [B,T,H,V] and ``d_final`` [N,H,K,V] (or None: zero), returns a dict of fp64
    arrays dq, dk, dg [B,T,H,K], dv [B,T,H,V], dbeta [B,T,H], d_initial
    [N,H,K,V], dA_log [H] and ddt_bias [H,K]."""
    qd, kd, vd, gd, bd, A, dtb, (B, T, H, K, V) = _f64_inputs(q, k, v, g, beta, A_log, dt_bias)
    cu, N = _cu_of(cu_seqlens, B)
    h0 = None if initial_state is None else _f64(initial_state).reshape(N, H, K, V)
    do = _f64(d_out).reshape(B, T, H, V)
    dfin = None if d_final is None else _f64(d_final).reshape(N, H, K, V)
    res = {"dq": np.zeros((B, T, H, K)), "dk": np.zeros((B, T, H, K)), "dv": np.zeros((B, T, H, V)),
           "dg": np.zeros((B, T, H, K)), "dbeta": np.zeros((B, T, H)), "d_initial": np.zeros((N, H, K, V)),
           "dA_log": np.zeros(H), "ddt_bias": np.zeros((H, K))}
    rc = lib.kda_oracle_bwd_f64(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(gd), _ptr(bd), B, T, H, K, V, _ptr(cu), N,
                                float(scale), _ptr(A), _ptr(dtb), float(lower_bound), _ptr(h0), _ptr(do),
                                _ptr(dfin), _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dg"]),
                                _ptr(res["dbeta"]), _ptr(res["d_initial"]), _ptr(res["dA_log"]),
                                _ptr(res["ddt_bias"]), int(num_threads))
    if rc != 0:
        raise ValueError("kda_oracle_bwd_f64 failed with code %d" % rc)
    return res


def gate(g: float, A_log: float, dt_bias: float, lower_bound: float) -> float:
    """The oracle's per-channel log-decay (scalar entry point, for pins)."""
    return _load().kda_gate(g, A_log, dt_bias, lower_bound)


def softplus(x: float) -> float:
    return _load().kda_softplus(x)


def sigmoid(x: float) -> float:
    return _load().kda_sigmoid(x)
