"""The oracle: a plain sequential fp64 CPU loop of the KDA recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and imports nothing from it.

``kda_ref.c`` holds the loop (see its header for the equations and the pages'
passages it follows).  This module only compiles it with gcc and marshals
numpy arrays through ctypes.  ``chunk_form.py`` holds a second, independent
formulation (the chunkwise algebra), used by tests to pin the loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_ref.c")
_LIB = os.path.join(_HERE, "libkdaref.so")
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99", "-D_POSIX_C_SOURCE=200809L",
           "-shared", "-fPIC", "-pthread"]

IO_F32 = 0
IO_BF16 = 1

# input transforms (kda_ref.c): L2-normalise q and k, beta = sigmoid(beta),
# log alpha = -5 sigmoid(exp(A_log[h]) (g + gate_bias[h, i]))
L2NORM = 1
BETA_SIGMOID = 2
GATE = 4

_lib = None


def build(force: bool = False) -> str:
    """Compile kda_ref.c into libkdaref.so with gcc (plain C, no HIP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        f = lib.kdaref_forward_ex
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _io_array(x):
    """Return (contiguous array, dtype code).  bf16 travels as raw uint16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, IO_F32
    if x.dtype == np.uint16:
        return x, IO_BF16
    raise TypeError("q/k/v must be float32 or uint16 (bf16 bit patterns), got %s" % x.dtype)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(q, k, v, g, beta, S0=None, scale=None, cu_seqlens=None, chains=None,
            delta_rule=True, threads=None, flags=0, A_log=None, gate_bias=None):
    """Run the fp64 recurrence.

    Batched layout (``cu_seqlens is None``): q, k, g are [B, T, H, dk]; v is
    [B, T, H, dv]; beta is [B, T, H].  Packed layout: q, k, g are
    [T_total, H, dk], v is [T_total, H, dv], beta is [T_total, H] and
    ``cu_seqlens`` ([N+1] int) gives the sequence boundaries.

    q, k, v: float32 arrays, or uint16 arrays holding bf16 bit patterns (the
    exact values a bf16 kernel receives).  g, beta: float32.  S0: None (zeros)
    or [N, H, dk, dv] (any float dtype; upcast exactly to fp64).

    Gated DeltaNet ("Kimi Unveils Delta Attention and K3 Architecture
    Updates", section 3): g without the dk axis ([B, T, H] or [T_total, H]) is
    one gate per (token, head), the same for every key channel; it is
    broadcast over dk (a copy, no arithmetic) and the recurrence is unchanged.

    ``flags`` (L2NORM | BETA_SIGMOID | GATE) applies kda_ref.c's input
    transforms to the raw q, k, beta and g; ``A_log`` [H] and ``gate_bias``
    ([H, dk], or [H] with a per-head gate, broadcast like g) go with GATE.

    ``chains``: iterable of (n, h) pairs (or flat ids n*H+h) to compute;
    default all.  Returns (outs, S_final) where ``outs[c]`` is the fp64
    [len_c, dv] output of chain c and ``S_final`` is [n_chains, dk, dv] fp64.
    """
    lib = _load()
    q, dt = _io_array(q)
    k, dt2 = _io_array(k)
    v, dt3 = _io_array(v)
    if not (dt == dt2 == dt3):
        raise TypeError("q, k, v must share one dtype")
    g = np.asarray(g, dtype=np.float32)
    if g.ndim == q.ndim - 1:
        g = np.broadcast_to(g[..., None], q.shape)
    a_log = None if A_log is None else np.ascontiguousarray(A_log, dtype=np.float32)
    gbias = None
    if gate_bias is not None:
        gbias = np.asarray(gate_bias, dtype=np.float32)
        if gbias.ndim == 1:
            gbias = np.broadcast_to(gbias[:, None], (gbias.shape[0], q.shape[-1]))
        gbias = np.ascontiguousarray(gbias)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    if cu_seqlens is None:
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        cu = None
        lens = [T] * B
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        T, H, dk = q.shape
        dv = v.shape[-1]
        B = cu.shape[0] - 1
        lens = [int(cu[n + 1] - cu[n]) for n in range(B)]
    if scale is None:
        scale = dk ** -0.5
    if chains is None:
        ids = np.arange(B * H, dtype=np.int32)
    else:
        ids = np.array([c if np.isscalar(c) else c[0] * H + c[1] for c in chains], dtype=np.int32)
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(S0, dtype=np.float64).reshape(B, H, dk, dv)
    total = int(sum(lens[int(c) // H] for c in ids))
    out = np.zeros((max(total, 1), dv), dtype=np.float64)
    S_final = np.zeros((len(ids), dk, dv), dtype=np.float64)
    rc = lib.kdaref_forward_ex(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(g), _ptr(beta), _ptr(s0),
                               _ptr(cu), B, T, H, dk, dv, float(scale), 1 if delta_rule else 0,
                               int(flags), _ptr(a_log), _ptr(gbias), _ptr(ids), len(ids),
                               _ptr(out), _ptr(S_final), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("kdaref_forward rejected its arguments")
    outs = []
    off = 0
    for c in ids:
        L = lens[int(c) // H]
        outs.append(out[off:off + L])
        off += L
    return outs, S_final


def forward_dense(q, k, v, g, beta, S0=None, scale=None, cu_seqlens=None, delta_rule=True,
                  threads=None, flags=0, A_log=None, gate_bias=None):
    """All chains, reassembled into the input layout: returns (out, S_final)
    with out shaped like v (fp64) and S_final [N, H, dk, dv] (fp64)."""
    q_ = np.asarray(q)
    H = q_.shape[-2]
    outs, S_final = forward(q, k, v, g, beta, S0=S0, scale=scale, cu_seqlens=cu_seqlens,
                            delta_rule=delta_rule, threads=threads, flags=flags, A_log=A_log,
                            gate_bias=gate_bias)
    v_ = np.asarray(v)
    dv = v_.shape[-1]
    dk = q_.shape[-1]
    out = np.zeros(v_.shape, dtype=np.float64)
    if cu_seqlens is None:
        B = q_.shape[0]
        for c, o in enumerate(outs):
            out[c // H, :, c % H, :] = o
        return out, S_final.reshape(B, H, dk, dv)
    cu = np.asarray(cu_seqlens)
    N = cu.shape[0] - 1
    for c, o in enumerate(outs):
        n, h = c // H, c % H
        out[cu[n]:cu[n + 1], h, :] = o
    return out, S_final.reshape(N, H, dk, dv)
