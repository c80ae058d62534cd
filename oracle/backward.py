"""The oracle's backward: reverse-mode derivatives of the KDA recurrence, fp64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP library and imports nothing from it.

The pages give no backward.  Chunkwise KDA is described as the training form
("Kimi Unveils Delta Attention and K3 Architecture Updates", section 6;
"Linear Attention, From Scratch to Kimi 3", section 9), so its gradients are
those of the forward recurrence, written out here by the chain rule, one
step at a time and in the reverse order of the forward's steps.  Forward step
t, per (sequence, head), state S in the key-by-value orientation (d_k x d_v),
as in kda_ref.c:

    a      = exp(g_t)                 decay of the key rows
    Sbar   = Diag(a) S_{t-1}
    p      = Sbar^T k_t
    e      = beta_t (v_t - p)
    S_t    = Sbar + k_t e^T
    o_t    = scale * S_t^T q_t

Given dL/do_t for every t and dL/dS_T (or zero), with dS = dL/dS_t:

    dS    += scale * q_t do_t^T          (o_t reads S_t)
    dq_t   = scale * S_t do_t
    de     = dS^T k_t                    (S_t = Sbar + k_t e^T)
    dk_t   = dS e
    dv_t   = beta_t de                   (e = beta (v - p))
    dbeta_t = de . (v_t - p)
    dp     = -beta_t de
    dk_t  += Sbar dp                     (p = Sbar^T k_t)
    dSbar  = dS + k_t dp^T
    dg_t   = rowsum(Sbar * dSbar)        (Sbar = Diag(exp g) S_{t-1})
    dS     = Diag(a) dSbar               -> dL/dS_{t-1}

and dL/dS0 is the dS left after the first token.  Gated DeltaNet gates (one
per token and head) take the sum of dg_t over the key channels.

Parity of this module is pinned in tests/test_oracle_pins.py against central
finite differences of kda_ref.c's forward loop (a separate implementation).
"""
from __future__ import annotations

import numpy as np


def _as_f64(x):
    """bf16 bit patterns (uint16) or float arrays -> exact fp64 values."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _chain_backward(q, k, v, g, beta, do, S0, dSf, scale):
    """One chain: q, k, g [L, dk]; v, do [L, dv]; beta [L]; S0, dSf [dk, dv]."""
    L, dk = q.shape
    dv = v.shape[1]
    # forward, keeping what the backward reads
    S = S0.copy()
    Sbar_t, S_t, p_t, e_t = [], [], [], []
    for t in range(L):
        a = np.exp(g[t])
        Sbar = a[:, None] * S
        p = Sbar.T @ k[t]
        e = beta[t] * (v[t] - p)
        S = Sbar + np.outer(k[t], e)
        Sbar_t.append(Sbar); S_t.append(S); p_t.append(p); e_t.append(e)
    dq = np.zeros((L, dk)); dk_ = np.zeros((L, dk)); dv_ = np.zeros((L, dv))
    dg = np.zeros((L, dk)); db = np.zeros(L)
    dS = dSf.copy()
    for t in range(L - 1, -1, -1):
        a = np.exp(g[t])
        dS = dS + scale * np.outer(q[t], do[t])
        dq[t] = scale * (S_t[t] @ do[t])
        de = dS.T @ k[t]
        dk_[t] = dS @ e_t[t]
        dv_[t] = beta[t] * de
        db[t] = de @ (v[t] - p_t[t])
        dp = -beta[t] * de
        dk_[t] += Sbar_t[t] @ dp
        dSbar = dS + np.outer(k[t], dp)
        dg[t] = np.sum(Sbar_t[t] * dSbar, axis=1)
        dS = a[:, None] * dSbar
    return dq, dk_, dv_, dg, db, dS


def backward(q, k, v, g, beta, do, S0=None, dS_final=None, scale=None, cu_seqlens=None):
    """Gradients of L(o, S_final) for the given dL/do (``do``, shaped like v)
    and dL/dS_final (``dS_final`` [N, H, dk, dv] or None = 0).

    Layouts as ``oracle.forward``: batched q, k, g [B, T, H, dk], v [B, T, H, dv],
    beta [B, T, H]; packed [T_total, H, .] with ``cu_seqlens``.  g without the
    dk axis is one gate per (token, head) (Gated DeltaNet); its gradient then has
    that shape too.  q, k, v, do: float32 or uint16 bf16 bit patterns.

    Returns a dict of fp64 arrays: dq, dk (like q), dv (like v), dg (like g),
    dbeta (like beta), dS0 [N, H, dk, dv].
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    scalar_gate = g.ndim == q.ndim - 1
    gk = np.broadcast_to(g[..., None], q.shape) if scalar_gate else g
    dk_dim, dv_dim = q.shape[-1], v.shape[-1]
    if scale is None:
        scale = dk_dim ** -0.5
    if cu_seqlens is None:
        B, T, H = q.shape[:3]
        bounds = [(n, None) for n in range(B)]
        N = B
    else:
        cu = np.asarray(cu_seqlens)
        N = cu.shape[0] - 1
        H = q.shape[1]
        bounds = [(n, (int(cu[n]), int(cu[n + 1]))) for n in range(N)]
    S0 = (np.zeros((N, H, dk_dim, dv_dim)) if S0 is None
          else np.asarray(S0, dtype=np.float64).reshape(N, H, dk_dim, dv_dim))
    dSf = (np.zeros((N, H, dk_dim, dv_dim)) if dS_final is None
           else np.asarray(dS_final, dtype=np.float64).reshape(N, H, dk_dim, dv_dim))
    res = {"dq": np.zeros(q.shape), "dk": np.zeros(k.shape), "dv": np.zeros(v.shape),
           "dg": np.zeros(gk.shape), "dbeta": np.zeros(beta.shape),
           "dS0": np.zeros((N, H, dk_dim, dv_dim))}
    for n, rng in bounds:
        for h in range(H):
            if rng is None:
                sel = (n, slice(None), h)
            else:
                sel = (slice(rng[0], rng[1]), h)
            out = _chain_backward(q[sel], k[sel], v[sel], gk[sel], beta[sel], do[sel],
                                  S0[n, h], dSf[n, h], scale)
            for name, val in zip(("dq", "dk", "dv", "dg", "dbeta"), out[:5]):
                res[name][sel] = val
            res["dS0"][n, h] = out[5]
    if scalar_gate:
        res["dg"] = res["dg"].sum(axis=-1)
    return res
