"""Chunkwise KDA in fp64 numpy: a second, independent formulation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It is not the HIP
algorithm and shares nothing with it; tests use it to pin the sequential loop
in ``kda_ref.c`` (both must agree to rounding, for any chunk size) and as a
stage-by-stage reference.

It follows "Kimi Unveils Delta Attention and K3 Architecture Updates",
section 6 (Chunkwise KDA), rewritten in the key-by-value orientation used by
the loop (S is d_k x d_v, decay multiplies key rows; the page's own prose uses
the transpose, where decay multiplies columns from the right):

* 6.1  chunk-local decays.  D_{0:i} = diag(exp(G_i)) and
       D_{j+1:i} = diag(exp(G_i - G_j)) with G the inclusive prefix sum of g
       inside the chunk (section 6.6: differences of prefix sums).
* 6.2  provisional errors ebar_i = beta_i (v_i - S_c^T D_{0:i} k_i).
* 6.3  rho_ij = beta_i <k_j, D_{j+1:i} k_i> for j < i, R strictly lower,
       E = (I + R)^{-1} Ebar  (rows are tokens; the page stacks columns).
* 6.4  S_{c+1} = D_{0:C-1} S_c + K_end^T E, K_end row j = D_{j+1:C-1} k_j.
* 6.5  chi_ij = s <k_j, D_{j+1:i} q_i> for j <= i,
       O = s (D_{0:i} q_i)_i S_c + A_qk E.

The triangular system is solved with ``numpy.linalg.solve`` (a library
primitive).  A last partial chunk is simply a shorter chunk.
"""
from __future__ import annotations

import numpy as np


def chunk_stages(q, k, v, g, beta, S, scale):
    """All section-6 quantities for ONE chunk of one chain.

    q, k, g: [C, dk]; v: [C, dv]; beta: [C]; S: [dk, dv] incoming state.
    Returns a dict with G, R, Akk=(I+R)^-1, Aqk, Ebar, E, K_end, O, S_next
    (all fp64).
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64); S = np.asarray(S, np.float64)
    C = q.shape[0]
    G = np.cumsum(g, axis=0)                       # 6.6: chunk-local cumulative log decay
    # 6.2 provisional errors from the incoming state only
    Ebar = beta[:, None] * (v - (np.exp(G) * k) @ S)
    # 6.3 causal key-key coefficients and A_kk
    R = np.zeros((C, C))
    Aqk = np.zeros((C, C))
    for i in range(C):
        for j in range(i + 1):
            dec = np.exp(G[i] - G[j])              # D_{j+1:i}
            if j < i:
                R[i, j] = beta[i] * np.dot(k[j], dec * k[i])
            Aqk[i, j] = scale * np.dot(k[j], dec * q[i])   # 6.5, diagonal included
    E = np.linalg.solve(np.eye(C) + R, Ebar)
    Akk = np.linalg.solve(np.eye(C) + R, np.eye(C))
    # 6.4 fast-forward the state
    K_end = np.exp(G[-1][None, :] - G) * k
    S_next = np.exp(G[-1])[:, None] * S + K_end.T @ E
    # 6.5 outputs
    O = scale * (np.exp(G) * q) @ S + Aqk @ E
    return dict(G=G, R=R, Akk=Akk, Aqk=Aqk, Ebar=Ebar, E=E, K_end=K_end, O=O, S_next=S_next)


def chain_forward(q, k, v, g, beta, S0, scale, chunk):
    """One chain [T, d] processed chunk by chunk.  Returns (O [T, dv], S_T)."""
    T = q.shape[0]
    S = np.zeros((q.shape[1], v.shape[1])) if S0 is None else np.asarray(S0, np.float64)
    outs = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        st = chunk_stages(q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1], S, scale)
        outs.append(st["O"])
        S = st["S_next"]
    O = np.concatenate(outs, axis=0) if outs else np.zeros((0, v.shape[1]))
    return O, S


def forward(q, k, v, g, beta, S0=None, scale=None, chunk=64):
    """Batched [B, T, H, d] fp64 chunkwise forward.  Returns (out, S_final)."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    out = np.zeros((B, T, H, dv))
    S_final = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            s0 = None if S0 is None else np.asarray(S0, np.float64)[b, h]
            O, S = chain_forward(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h], beta[b, :, h],
                                 s0, scale, chunk)
            out[b, :, h] = O
            S_final[b, h] = S
    return out, S_final
