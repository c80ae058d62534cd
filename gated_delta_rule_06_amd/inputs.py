"""Seeded synthetic inputs for the KDA forward (prefill, varlen, decode).

This module draws random numbers and lays them out; it contains none of the
method's arithmetic.  Both the HIP path and the fp64 oracle are fed from it.

Recipe (the pages fix only shapes and distributions; the rest is chosen here):

* q, k ~ N(0, 1) per element, then L2-normalised per (token, head) vector in
  fp32 (keys and queries are normalised before the op, "Linear Attention,
  From Scratch to Kimi 3", section 7);
* v ~ N(0, 1);
* log_alpha = -exp(N(-3, 1)) per (token, head, key channel), natural log;
* beta = sigmoid(N(0, 1)) per (token, head);
* S0 ~ N(0, 0.02^2) when an initial state is requested;
* varlen: lengths ~ U{lo..hi} inclusive from ``numpy.random.default_rng(seed)``,
  packed along the token axis with cu_seqlens; in each head a seeded choice of
  ``long_channels`` key channels draws log_alpha = -exp(N(-8, 0.5)) instead
  (a decay horizon of a few thousand tokens).
* strong_gate_channels: in every head a seeded choice of n key channels
  redraws log_alpha ~ U[lo, hi] (default [-5, -2]) per token: fast-forgetting
  channels down to the gate transform's floor of -5 per token, up to e^-320
  over a 64-token chunk.
* gate="gdn" (Gated DeltaNet) draws one log_alpha per (token, head), shape
  [..., H], from the same -exp(N(-3, 1)); gate="kda" one per key channel.
* Draw order: q, k, v, g, beta, S0 (lengths first for varlen).  Random numbers
  come from one ``torch.Generator`` on the target device, so a seed gives the
  same tensors on every run of one device type.
* bf16 tensors are cast from the fp32 values with round-to-nearest-even, after
  normalisation.  The oracle reads the cast values.
* backward cotangents (grad_inputs): dL/dout ~ N(0, 1) in v's dtype, dL/dS_final
  ~ N(0, 0.1^2) fp32, drawn after the inputs from a generator of their own.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = ["prefill_inputs", "varlen_lengths", "varlen_inputs", "decode_inputs",
           "raw_layer_inputs", "strong_gate_channels", "grad_inputs", "to_host",
           "bf16_bits_from_f32", "CONFIGS"]

_IO = {"bf16": torch.bfloat16, "f32": torch.float32}

# The workloads the path is measured and checked on.
CONFIGS = {
    "single_head_f32": dict(B=1, T=256, H=1, dk=64, dv=64, io="f32", S0=False, chunk=64),
    "prefill_h16_s0": dict(B=1, T=4096, H=16, dk=128, dv=128, io="bf16", S0=True, chunk=64),
    "prefill_b8_h32_t8192": dict(B=8, T=8192, H=32, dk=128, dv=128, io="bf16", S0=False, chunk=64),
    "decode_n256_h32": dict(N=256, H=32, dk=128, dv=128, io="bf16", steps=128),
    "varlen_16seq_h32": dict(n_seq=16, lo=1024, hi=65536, H=32, dk=128, dv=128, io="bf16",
                             long_channels=8, chunk=64),
    # multi-token decode: 256 sequences of U{1..8} new tokens on resident states
    "recurrent_n256_h32": dict(n_seq=256, lo=1, hi=8, H=32, dk=128, dv=128, io="bf16", S0=True),
}


def _gen(device, seed):
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _unit_normal(shape, gen, device):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def _log_alpha(shape, gen, device, long_mask=None):
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    mu = torch.full_like(z, -3.0)
    sd = torch.ones_like(z)
    if long_mask is not None:
        # long_mask: [H, dk] bool, broadcast over tokens
        mu = torch.where(long_mask, torch.full_like(z, -8.0), mu)
        sd = torch.where(long_mask, torch.full_like(z, 0.5), sd)
    return -torch.exp(mu + sd * z)


def _draw(rows_shape, H, dk, dv, io, gen, device, with_S0, n_seq, s0_std, long_mask=None,
          gate="kda"):
    dt = _IO[io]
    q = _unit_normal((*rows_shape, H, dk), gen, device).to(dt)
    k = _unit_normal((*rows_shape, H, dk), gen, device).to(dt)
    v = torch.randn((*rows_shape, H, dv), generator=gen, device=device, dtype=torch.float32).to(dt)
    if gate == "gdn":
        g = _log_alpha((*rows_shape, H), gen, device)
    else:
        g = _log_alpha((*rows_shape, H, dk), gen, device, long_mask)
    beta = torch.sigmoid(torch.randn((*rows_shape, H), generator=gen, device=device,
                                     dtype=torch.float32))
    S0 = None
    if with_S0:
        S0 = s0_std * torch.randn((n_seq, H, dk, dv), generator=gen, device=device,
                                  dtype=torch.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)


def prefill_inputs(B, T, H, dk, dv, io="bf16", seed=0, with_S0=False, s0_std=0.02,
                   device="cpu", gate="kda"):
    """Batched prefill inputs in the [B, T, H, d] layout."""
    gen = _gen(device, seed)
    d = _draw((B, T), H, dk, dv, io, gen, device, with_S0, B, s0_std, gate=gate)
    d.update(B=B, T=T, H=H, dk=dk, dv=dv, io=io, cu_seqlens=None)
    return d


def varlen_lengths(n_seq, lo, hi, seed=0):
    """Sequence lengths ~ U{lo..hi} (inclusive) from numpy's default_rng(seed)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=n_seq, endpoint=True).astype(np.int64)


def varlen_inputs(lengths, H, dk, dv, io="bf16", seed=0, with_S0=False, s0_std=0.02,
                  long_channels=0, device="cpu", gate="kda"):
    """Packed inputs [T_total, H, d] plus int32 cu_seqlens [N+1] (on ``device``)."""
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T_total = int(cu[-1])
    gen = _gen(device, seed)
    long_mask = None
    if long_channels:
        long_mask = torch.zeros((H, dk), dtype=torch.bool, device=device)
        for h in range(H):
            idx = torch.randperm(dk, generator=gen, device=device)[:long_channels]
            long_mask[h, idx] = True
    d = _draw((T_total,), H, dk, dv, io, gen, device, with_S0, len(lengths), s0_std, long_mask,
              gate=gate)
    d.update(N=len(lengths), T_total=T_total, H=H, dk=dk, dv=dv, io=io,
             cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device),
             lengths=lengths, long_mask=long_mask)
    return d


def decode_inputs(N, H, dk, dv, steps, io="bf16", seed=0, s0_std=0.02, device="cpu",
                  gate="kda"):
    """State S [N, H, dk, dv] fp32 ~ N(0, s0_std^2) and ``steps`` fresh tokens.

    Returns dict with S (fp32), and per-step stacked q, k [steps, N, H, dk],
    v [steps, N, H, dv], g [steps, N, H, dk], beta [steps, N, H].
    """
    gen = _gen(device, seed)
    S = s0_std * torch.randn((N, H, dk, dv), generator=gen, device=device, dtype=torch.float32)
    d = _draw((steps, N), H, dk, dv, io, gen, device, False, N, s0_std, gate=gate)
    d.update(S=S, N=N, H=H, dk=dk, dv=dv, io=io, steps=steps)
    return d


def raw_layer_inputs(d, H, dk, seed=0, gate="kda", strong_decay=False, device="cpu",
                     gate_mu=-4.0):
    """Turn an input dict into raw layer inputs for the in-kernel transforms:
    q and k scaled per (token, head) by exp(N(0, 0.5)) (no longer unit),
    beta replaced by logits ~ N(0, 1), log_alpha replaced by a raw gate
    projection ~ N(gate_mu, 1) (N(3, 1) with strong_decay), plus A_log [H] ~
    N(0, 0.3^2) and a gate bias ~ N(0, 0.5^2) of shape [H, dk] ([H] for
    per-head gates).  The I/O dtype of q and k is kept."""
    gen = _gen(device, seed + 7919)
    qk_shape = d["q"].shape
    for name in ("q", "k"):
        c = torch.exp(0.5 * torch.randn(qk_shape[:-1] + (1,), generator=gen, device=device))
        d[name] = (d[name].float() * c).to(d[name].dtype)
    d["beta"] = torch.randn(d["beta"].shape, generator=gen, device=device)
    mu = 3.0 if strong_decay else gate_mu
    d["g"] = mu + torch.randn(d["g"].shape, generator=gen, device=device)
    d["A_log"] = 0.3 * torch.randn((H,), generator=gen, device=device)
    bshape = (H,) if gate == "gdn" else (H, dk)
    d["gate_bias"] = 0.5 * torch.randn(bshape, generator=gen, device=device)
    return d


def strong_gate_channels(d, n_channels, lo=-5.0, hi=-2.0, seed=0):
    """Per-channel KDA inputs (batched or packed): in every head a seeded
    choice of ``n_channels`` key channels redraws log_alpha ~ U[lo, hi] per
    token, from a generator of its own.  Modifies d["g"] in place and records
    the choice as d["strong_idx"] ([H, n_channels] int64)."""
    g = d["g"]
    dev = g.device
    gen = _gen(dev, seed + 15485863)
    H, dk = g.shape[-2], g.shape[-1]
    rows = g.shape[:-2]
    chosen = []
    for h in range(H):
        idx = torch.randperm(dk, generator=gen, device=dev)[:n_channels]
        u = torch.rand(rows + (n_channels,), generator=gen, device=dev, dtype=torch.float32)
        g[..., h, idx] = lo + (hi - lo) * u
        chosen.append(idx)
    d["strong_idx"] = torch.stack(chosen) if chosen else None
    return d


def grad_inputs(d, seed=0, with_dS_final=True, device="cpu"):
    """Cotangents for the backward of the forward on ``d``: d_out ~ N(0, 1)
    shaped like v (v's dtype) and dS_final ~ N(0, 0.1^2) [N, H, dk, dv] fp32
    (or None).  Adds them to ``d`` as "d_out" and "dS_final"."""
    gen = _gen(device, seed + 104729)
    n_seq = d["B"] if d.get("cu_seqlens") is None else d["N"]
    d["d_out"] = torch.randn(d["v"].shape, generator=gen, device=device,
                             dtype=torch.float32).to(d["v"].dtype)
    d["dS_final"] = None
    if with_dS_final:
        d["dS_final"] = 0.1 * torch.randn((n_seq, d["H"], d["dk"], d["dv"]), generator=gen,
                                          device=device, dtype=torch.float32)
    return d


def bf16_bits_from_f32(x):
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def to_host(t):
    """A device/CPU tensor as the numpy array the oracle reads: bf16 -> uint16
    bit patterns (exact values), fp32 -> float32, ints unchanged."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
