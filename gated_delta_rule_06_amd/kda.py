"""Python binding of the KDA C ABI (include/kda.h): argument marshalling only.

Every step of the forward runs in ``libkda.so``'s HIP kernels; this module
checks tensor shapes/dtypes, passes raw device pointers and the current HIP
stream, and turns status codes into exceptions.  PyTorch only provides device
memory and streams.  There is no fallback: if the library is missing, importing
this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_IO_F32 = 0
KDA_IO_BF16 = 1
CHUNK = 64
KDA_PRO_QK_L2NORM = 1
KDA_PRO_BETA_SIGMOID = 2
KDA_PRO_GATE = 4


class _Prologue(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("A_log", ctypes.c_void_p),
                ("gate_bias", ctypes.c_void_p)]


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libkda.so is not built (%s); run `python -m gated_delta_rule_06_amd.build`"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i, sz, f = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.kda_chunk_fwd.restype = i
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.kda_chunk_fwd_varlen.restype = i
    lib.kda_chunk_fwd_varlen.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, i, i, i, i, i, f, i, i,
                                         vp, sz, vp]
    lib.kda_decode_step.restype = i
    lib.kda_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, vp, i, i, i, i, f, i, vp]
    lib.kda_recurrent_fwd.restype = i
    lib.kda_recurrent_fwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, i, i, i, i, i, f, i, vp]
    lib.kda_recurrent_fwd_varlen.restype = i
    lib.kda_recurrent_fwd_varlen.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, i, i, i, i, i, f,
                                             i, vp]
    for name in ("chunk_fwd", "chunk_fwd_varlen", "decode_step", "recurrent_fwd",
                 "recurrent_fwd_varlen"):
        kf, gf = getattr(lib, "kda_" + name), getattr(lib, "kda_gdn_" + name)
        gf.restype = kf.restype
        gf.argtypes = kf.argtypes
    pp = ctypes.POINTER(_Prologue)
    lib.kda_chunk_fwd_fused.restype = i
    lib.kda_chunk_fwd_fused.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, i, i, i, i, i, f, i, i,
                                        i, pp, vp, sz, vp]
    lib.kda_recurrent_fwd_fused.restype = i
    lib.kda_recurrent_fwd_fused.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, i, i, i, i, i, f,
                                            i, i, pp, vp]
    lib.kda_decode_step_fused.restype = i
    lib.kda_decode_step_fused.argtypes = [vp, vp, vp, fp, fp, fp, vp, i, i, i, i, f, i, i, pp, vp]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd_workspace_size.argtypes = [i] * 7
    lib.kda_chunk_fwd_varlen_workspace_size.restype = sz
    lib.kda_chunk_fwd_varlen_workspace_size.argtypes = [i] * 7
    lib.kda_backward_workspace_size.restype = sz
    lib.kda_backward_workspace_size.argtypes = [i] * 6
    lib.kda_backward.restype = i
    lib.kda_backward.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, fp, fp, fp, fp, fp, vp, i, i, i,
                                 i, i, f, i, i, vp, sz, vp]
    lib.kda_backward_noalloc.restype = i
    lib.kda_backward_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, fp, fp, fp, fp, fp,
                                         vp, i, i, i, i, i, f, i, i, vp]
    lib.kda_noalloc_scratch_bytes.restype = sz
    lib.kda_noalloc_scratch_bytes.argtypes = []
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i]
    lib.kda_version.restype = i
    lib.kda_version.argtypes = []
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.kda_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _io_code(dtype):
    if dtype == torch.bfloat16:
        return KDA_IO_BF16
    if dtype == torch.float32:
        return KDA_IO_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % dtype)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _gate(log_alpha, rows_shape, dk):
    """(expected log_alpha shape, entry-point prefix): KDA takes one gate per key
    channel ([..., H, d_k]); Gated DeltaNet one per (token, head) ([..., H])."""
    if log_alpha is not None and log_alpha.dim() == len(rows_shape):
        return tuple(rows_shape), "kda_gdn_"
    return tuple(rows_shape) + (dk,), "kda_"


def _prologue(H, dk, per_head, device, qk_l2norm, beta_sigmoid, A_log, gate_bias):
    """The input transforms as a kda_prologue, or None when none is asked for.
    A_log ([H]) switches the gate transform on; gate_bias is [H, d_k] ([H]
    with per-head gates) or None."""
    flags = (KDA_PRO_QK_L2NORM if qk_l2norm else 0) | (KDA_PRO_BETA_SIGMOID if beta_sigmoid else 0)
    if gate_bias is not None and A_log is None:
        raise ValueError("gate_bias needs A_log (the gate transform)")
    if A_log is not None:
        flags |= KDA_PRO_GATE
        _check(A_log, "A_log", (H,), torch.float32, device)
        _check(gate_bias, "gate_bias", (H,) if per_head else (H, dk), torch.float32, device)
    if not flags:
        return None
    return _Prologue(flags, None if A_log is None else A_log.data_ptr(),
                     None if gate_bias is None else gate_bias.data_ptr())


# The chunk-parallel schedule runs plain KDA calls of at most this many (sequence,
# head) chains; other calls of so few chains use no workspace at all (the
# balanced schedule needs more chains than resident workgroups).
_PAR_MAX_CHAINS = 64


def _workspace(nbytes, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


_TRANSFORMS_DOC = """
    Optional input transforms, applied inside the kernels: qk_l2norm
    normalises q and k per (token, head); beta_sigmoid takes beta as logits;
    A_log ([H] fp32) makes log_alpha the raw gate projection g, with log alpha
    = -5 sigmoid(exp(A_log[h]) (g + gate_bias)), gate_bias [H, d_k] ([H] for
    per-head gates) or None."""


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, scale=None, chunk=CHUNK, out=None,
              S_final=None, output_final_state=True, qk_l2norm=False, beta_sigmoid=False,
              A_log=None, gate_bias=None, workspace=None, balanced=True):
    """Chunkwise prefill.  q, k: [B, T, H, d_k]; v: [B, T, H, d_v]; beta:
    [B, T, H]; log_alpha: [B, T, H, d_k] (KDA) or [B, T, H] (Gated DeltaNet, one
    gate per token and head); S0: [B, H, d_k, d_v] fp32 or None.  workspace:
    a uint8 device tensor of at least chunk_fwd_workspace_size() bytes, or None
    (allocated).  balanced=False with no workspace passes none (one workgroup
    per chain; shapes that take the chunk-parallel schedule then fail, since
    it needs one).  Returns (o, S_final)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if scale is None:
        scale = dk ** -0.5
    gshape, pre = _gate(log_alpha, (B, T, H), dk)
    for name, t, shp, dt in (("q", q, (B, T, H, dk), q.dtype), ("k", k, (B, T, H, dk), q.dtype),
                             ("v", v, (B, T, H, dv), q.dtype),
                             ("log_alpha", log_alpha, gshape, torch.float32),
                             ("beta", beta, (B, T, H), torch.float32),
                             ("S0", S0, (B, H, dk, dv), torch.float32)):
        _check(t, name, shp, dt, dev)
    io = _io_code(q.dtype)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (B, T, H, dv), q.dtype, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    pro = _prologue(H, dk, pre == "kda_gdn_", dev, qk_l2norm, beta_sigmoid, A_log, gate_bias)
    # the chunk-parallel schedule (plain KDA calls of few long chains) needs a
    # workspace; for other shapes it enables the balanced schedule
    ws, wsb = None, 0
    if workspace is not None:
        ws, wsb = workspace, workspace.numel()
    elif balanced and (B * H > _PAR_MAX_CHAINS or (pro is None and pre == "kda_")):
        ws, wsb = _workspace(lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io), dev)
    if pro is None:
        fn = pre + "chunk_fwd"
        st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                              _ptr(out), _ptr(S_final), B, T, H, dk, dv, float(scale), int(chunk),
                              io, _ptr(ws), wsb, _stream(dev))
    else:
        fn = "kda_chunk_fwd_fused"
        st = lib.kda_chunk_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                     _ptr(S0), _ptr(out), _ptr(S_final), None, B, T, H, dk, dv,
                                     float(scale), int(chunk), io, int(pre == "kda_gdn_"),
                                     ctypes.byref(pro), _ptr(ws), wsb, _stream(dev))
    if st != 0:
        raise KdaError(st, fn)
    return out, S_final


def chunk_fwd_workspace_size(B, T, H, dk, dv, io="bf16", chunk=CHUNK):
    """Bytes of workspace kda_chunk_fwd takes for these sizes: the
    chunk-parallel schedule's factors where it runs, else the balanced
    schedule's (0 for unsupported sizes)."""
    return int(lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk,
                                                KDA_IO_BF16 if io == "bf16" else KDA_IO_F32))


def chunk_fwd_varlen(q, k, v, log_alpha, beta, cu_seqlens, S0=None, scale=None, chunk=CHUNK,
                     out=None, S_final=None, output_final_state=True, qk_l2norm=False,
                     beta_sigmoid=False, A_log=None, gate_bias=None, balanced=True,
                     workspace=None):
    """Packed variable-length prefill.  q, k: [T_total, H, d_k]; v: [T_total,
    H, d_v]; beta: [T_total, H]; log_alpha: [T_total, H, d_k] (KDA) or
    [T_total, H] (Gated DeltaNet); cu_seqlens: int32 [N+1] on the device; S0:
    [N, H, d_k, d_v] fp32 or None.  balanced: give the library a workspace,
    so that calls with more chains than resident workgroups split sequences
    evenly over the workgroups (same bits); False keeps one workgroup per
    chain.  workspace: a uint8 device tensor of at least
    kda_chunk_fwd_varlen_workspace_size() bytes to use for that, or None
    (allocated).  Returns (o, S_final)."""
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    gshape, pre = _gate(log_alpha, (Tt, H), dk)
    for name, t, shp, dt in (("q", q, (Tt, H, dk), q.dtype), ("k", k, (Tt, H, dk), q.dtype),
                             ("v", v, (Tt, H, dv), q.dtype),
                             ("log_alpha", log_alpha, gshape, torch.float32),
                             ("beta", beta, (Tt, H), torch.float32),
                             ("cu_seqlens", cu_seqlens, (N + 1,), torch.int32),
                             ("S0", S0, (N, H, dk, dv), torch.float32)):
        _check(t, name, shp, dt, dev)
    io = _io_code(q.dtype)
    if out is None:
        out = torch.empty((Tt, H, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (Tt, H, dv), q.dtype, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", (N, H, dk, dv), torch.float32, dev)
    pro = _prologue(H, dk, pre == "kda_gdn_", dev, qk_l2norm, beta_sigmoid, A_log, gate_bias)
    ws, wsb = None, 0
    if balanced and workspace is not None:
        ws, wsb = workspace, workspace.numel()
    elif balanced and (N * H > _PAR_MAX_CHAINS or (pro is None and pre == "kda_")):
        ws, wsb = _workspace(lib.kda_chunk_fwd_varlen_workspace_size(N, Tt, H, dk, dv, chunk, io),
                             dev)
    if pro is None:
        fn = pre + "chunk_fwd_varlen"
        st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                              _ptr(out), _ptr(S_final), _ptr(cu_seqlens), N, Tt, H, dk, dv,
                              float(scale), int(chunk), io, _ptr(ws), wsb, _stream(dev))
    else:
        fn = "kda_chunk_fwd_fused"
        st = lib.kda_chunk_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                     _ptr(S0), _ptr(out), _ptr(S_final), _ptr(cu_seqlens), N, Tt,
                                     H, dk, dv, float(scale), int(chunk), io,
                                     int(pre == "kda_gdn_"), ctypes.byref(pro), _ptr(ws), wsb,
                                     _stream(dev))
    if st != 0:
        raise KdaError(st, fn)
    return out, S_final


def decode_step(q, k, v, log_alpha, beta, S_inout, scale=None, out=None, qk_l2norm=False,
                beta_sigmoid=False, A_log=None, gate_bias=None):
    """One fused recurrent step.  q, k: [N, H, d_k]; v: [N, H, d_v]; beta:
    [N, H]; log_alpha: [N, H, d_k] (KDA) or [N, H] (Gated DeltaNet); S_inout:
    [N, H, d_k, d_v] fp32, updated in place.  Returns o."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if scale is None:
        scale = dk ** -0.5
    gshape, pre = _gate(log_alpha, (N, H), dk)
    for name, t, shp, dt in (("q", q, (N, H, dk), q.dtype), ("k", k, (N, H, dk), q.dtype),
                             ("v", v, (N, H, dv), q.dtype),
                             ("log_alpha", log_alpha, gshape, torch.float32),
                             ("beta", beta, (N, H), torch.float32),
                             ("S_inout", S_inout, (N, H, dk, dv), torch.float32)):
        _check(t, name, shp, dt, dev)
    io = _io_code(q.dtype)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (N, H, dv), q.dtype, dev)
    pro = _prologue(H, dk, pre == "kda_gdn_", dev, qk_l2norm, beta_sigmoid, A_log, gate_bias)
    if pro is None:
        fn = pre + "decode_step"
        st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                              _ptr(S_inout), _ptr(out), N, H, dk, dv, float(scale), io,
                              _stream(dev))
    else:
        fn = "kda_decode_step_fused"
        st = lib.kda_decode_step_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                       _ptr(S_inout), _ptr(out), N, H, dk, dv, float(scale), io,
                                       int(pre == "kda_gdn_"), ctypes.byref(pro), _stream(dev))
    if st != 0:
        raise KdaError(st, fn)
    return out


def recurrent_fwd(q, k, v, log_alpha, beta, S0=None, scale=None, out=None, S_final=None,
                  output_final_state=True, qk_l2norm=False, beta_sigmoid=False, A_log=None,
                  gate_bias=None):
    """Token-by-token recurrence for short sequences (multi-token decode,
    speculative verification).  Shapes as chunk_fwd (KDA or Gated DeltaNet
    gates).  Pass S_final=S0 to update a state in place.  Returns (o, S_final)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if scale is None:
        scale = dk ** -0.5
    gshape, pre = _gate(log_alpha, (B, T, H), dk)
    for name, t, shp, dt in (("q", q, (B, T, H, dk), q.dtype), ("k", k, (B, T, H, dk), q.dtype),
                             ("v", v, (B, T, H, dv), q.dtype),
                             ("log_alpha", log_alpha, gshape, torch.float32),
                             ("beta", beta, (B, T, H), torch.float32),
                             ("S0", S0, (B, H, dk, dv), torch.float32)):
        _check(t, name, shp, dt, dev)
    io = _io_code(q.dtype)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (B, T, H, dv), q.dtype, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    pro = _prologue(H, dk, pre == "kda_gdn_", dev, qk_l2norm, beta_sigmoid, A_log, gate_bias)
    if pro is None:
        fn = pre + "recurrent_fwd"
        st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                              _ptr(out), _ptr(S_final), B, T, H, dk, dv, float(scale), io,
                              _stream(dev))
    else:
        fn = "kda_recurrent_fwd_fused"
        st = lib.kda_recurrent_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                         _ptr(S0), _ptr(out), _ptr(S_final), None, B, T, H, dk,
                                         dv, float(scale), io, int(pre == "kda_gdn_"),
                                         ctypes.byref(pro), _stream(dev))
    if st != 0:
        raise KdaError(st, fn)
    return out, S_final


def recurrent_fwd_varlen(q, k, v, log_alpha, beta, cu_seqlens, S0=None, scale=None, out=None,
                         S_final=None, output_final_state=True, qk_l2norm=False,
                         beta_sigmoid=False, A_log=None, gate_bias=None):
    """Token-by-token recurrence over packed sequences (varlen decode).
    Shapes as chunk_fwd_varlen (KDA or Gated DeltaNet gates); S_final=S0
    updates the states in place.  Returns (o, S_final)."""
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    gshape, pre = _gate(log_alpha, (Tt, H), dk)
    for name, t, shp, dt in (("q", q, (Tt, H, dk), q.dtype), ("k", k, (Tt, H, dk), q.dtype),
                             ("v", v, (Tt, H, dv), q.dtype),
                             ("log_alpha", log_alpha, gshape, torch.float32),
                             ("beta", beta, (Tt, H), torch.float32),
                             ("cu_seqlens", cu_seqlens, (N + 1,), torch.int32),
                             ("S0", S0, (N, H, dk, dv), torch.float32)):
        _check(t, name, shp, dt, dev)
    io = _io_code(q.dtype)
    if out is None:
        out = torch.empty((Tt, H, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (Tt, H, dv), q.dtype, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", (N, H, dk, dv), torch.float32, dev)
    pro = _prologue(H, dk, pre == "kda_gdn_", dev, qk_l2norm, beta_sigmoid, A_log, gate_bias)
    if pro is None:
        fn = pre + "recurrent_fwd_varlen"
        st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                              _ptr(out), _ptr(S_final), _ptr(cu_seqlens), N, Tt, H, dk, dv,
                              float(scale), io, _stream(dev))
    else:
        fn = "kda_recurrent_fwd_fused"
        st = lib.kda_recurrent_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                         _ptr(S0), _ptr(out), _ptr(S_final), _ptr(cu_seqlens), N,
                                         Tt, H, dk, dv, float(scale), io, int(pre == "kda_gdn_"),
                                         ctypes.byref(pro), _stream(dev))
    if st != 0:
        raise KdaError(st, fn)
    return out, S_final


def backward_workspace_size(N, T, H, dk, dv, packed=False):
    """Bytes of workspace kda_backward needs (T = T_total when packed)."""
    return int(lib.kda_backward_workspace_size(N, T, H, dk, dv, int(bool(packed))))


def backward(q, k, v, log_alpha, beta, d_out, S0=None, dS_final=None, cu_seqlens=None,
             scale=None, want_dS0=True, workspace=None):
    """Gradients of the forward for dL/dout = ``d_out`` (shaped like out, q's
    dtype) and dL/dS_final = ``dS_final`` ([N, H, dk, dv] fp32, or None = 0).
    The inputs are the forward's: batched [B, T, H, .] or, with ``cu_seqlens``,
    packed [T_total, H, .]; KDA or Gated DeltaNet gates.  ``workspace``: a
    uint8 tensor of at least backward_workspace_size() bytes, or None (one is
    allocated).  Returns a dict of fp32 tensors dq, dk, dv, dlog_alpha (shaped
    like log_alpha), dbeta and dS0 (None unless ``want_dS0``)."""
    packed = cu_seqlens is not None
    lead = tuple(q.shape[:-2])
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    dev = q.device
    if packed:
        (Tt,) = lead
        N, T = cu_seqlens.shape[0] - 1, Tt
    else:
        N, T = lead
    if scale is None:
        scale = dk ** -0.5
    gshape, pre = _gate(log_alpha, lead + (H,), dk)
    for name, t, shp, dt in (("q", q, lead + (H, dk), q.dtype), ("k", k, lead + (H, dk), q.dtype),
                             ("v", v, lead + (H, dv), q.dtype),
                             ("log_alpha", log_alpha, gshape, torch.float32),
                             ("beta", beta, lead + (H,), torch.float32),
                             ("d_out", d_out, lead + (H, dv), q.dtype),
                             ("cu_seqlens", cu_seqlens, (N + 1,), torch.int32),
                             ("S0", S0, (N, H, dk, dv), torch.float32),
                             ("dS_final", dS_final, (N, H, dk, dv), torch.float32)):
        _check(t, name, shp, dt, dev)
    io = _io_code(q.dtype)
    f32 = dict(dtype=torch.float32, device=dev)
    res = {"dq": torch.empty(lead + (H, dk), **f32), "dk": torch.empty(lead + (H, dk), **f32),
           "dv": torch.empty(lead + (H, dv), **f32), "dlog_alpha": torch.empty(gshape, **f32),
           "dbeta": torch.empty(lead + (H,), **f32),
           "dS0": torch.empty((N, H, dk, dv), **f32) if want_dS0 else None}
    need = backward_workspace_size(N, T, H, dk, dv, packed)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    st = lib.kda_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                          _ptr(d_out), _ptr(dS_final), _ptr(res["dq"]), _ptr(res["dk"]),
                          _ptr(res["dv"]), _ptr(res["dlog_alpha"]), _ptr(res["dbeta"]),
                          _ptr(res["dS0"]), _ptr(cu_seqlens), N, T, H, dk, dv, float(scale), io,
                          int(pre == "kda_gdn_"), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != 0:
        raise KdaError(st, "kda_backward")
    return res


def backward_noalloc(q, k, v, log_alpha, beta, d_out, out, S0=None, dS_final=None,
                     cu_seqlens=None, scale=None):
    """kda_backward_noalloc: the backward with the library's static scratch as
    its workspace, for callers that cannot allocate.  ``out`` is a dict of
    caller-allocated fp32 output tensors shaped as backward() returns them
    (dq, dk, dv, dlog_alpha, dbeta; dS0 optional); neither this function nor
    the library allocates anything.  Problems needing more than
    noalloc_scratch_bytes() of workspace raise KdaError (KDA_ERR_SCRATCH)."""
    packed = cu_seqlens is not None
    lead = tuple(q.shape[:-2])
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    dev = q.device
    if packed:
        (Tt,) = lead
        N, T = cu_seqlens.shape[0] - 1, Tt
    else:
        N, T = lead
    if scale is None:
        scale = dk ** -0.5
    gshape, pre = _gate(log_alpha, lead + (H,), dk)
    for name, t, shp, dt in (("q", q, lead + (H, dk), q.dtype), ("k", k, lead + (H, dk), q.dtype),
                             ("v", v, lead + (H, dv), q.dtype),
                             ("log_alpha", log_alpha, gshape, torch.float32),
                             ("beta", beta, lead + (H,), torch.float32),
                             ("d_out", d_out, lead + (H, dv), q.dtype),
                             ("cu_seqlens", cu_seqlens, (N + 1,), torch.int32),
                             ("S0", S0, (N, H, dk, dv), torch.float32),
                             ("dS_final", dS_final, (N, H, dk, dv), torch.float32),
                             ("dq", out["dq"], lead + (H, dk), torch.float32),
                             ("dk", out["dk"], lead + (H, dk), torch.float32),
                             ("dv", out["dv"], lead + (H, dv), torch.float32),
                             ("dlog_alpha", out["dlog_alpha"], gshape, torch.float32),
                             ("dbeta", out["dbeta"], lead + (H,), torch.float32),
                             ("dS0", out.get("dS0"), (N, H, dk, dv), torch.float32)):
        _check(t, name, shp, dt, dev)
    st = lib.kda_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                  _ptr(S0), _ptr(d_out), _ptr(dS_final), _ptr(out["dq"]),
                                  _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
                                  _ptr(out["dbeta"]), _ptr(out.get("dS0")), _ptr(cu_seqlens), N, T,
                                  H, dk, dv, float(scale), _io_code(q.dtype),
                                  int(pre == "kda_gdn_"), _stream(dev))
    if st != 0:
        raise KdaError(st, "kda_backward_noalloc")
    return out


def noalloc_scratch_bytes():
    """Size of the static scratch array behind backward_noalloc (bytes)."""
    return int(lib.kda_noalloc_scratch_bytes())


for _f in (chunk_fwd, chunk_fwd_varlen, decode_step, recurrent_fwd, recurrent_fwd_varlen):
    _f.__doc__ = (_f.__doc__ or "") + _TRANSFORMS_DOC
