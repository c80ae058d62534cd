"""Helpers shared by the GPU parity tests: run the oracle on host copies of
exactly the tensors the HIP path received and compare element by element.

The comparison (``assert_close``) bounds three rel-L2 figures by the same
tolerance, separately for the outputs o and the final states S_T:

* the whole sample (all compared chains flattened together);
* every chain on its own (the per-chain maximum);
* every 64-token block of every chain's outputs on its own (the per-block
  maximum), so that an error confined to a few rows of a long chain cannot
  hide under the rest of the chain.
"""
import numpy as np
import torch

import oracle
from gated_delta_rule_06_amd.inputs import to_host

# rel-L2 bounds: fp32 I/O and bf16 I/O with fp32 state
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
BLOCK_ROWS = 64


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return num / den if den > 0 else num


def tol_for(io):
    return TOL_BF16 if io == "bf16" else TOL_F32


def _pro_args_many(d, heads, flags):
    """Oracle keyword arguments for the input transforms of the given heads
    (one oracle head per compared chain)."""
    if not flags:
        return {}
    ox = {"flags": flags}
    if flags & oracle.GATE:
        idx = torch.tensor(heads, dtype=torch.long, device=d["A_log"].device)
        ox["A_log"] = to_host(d["A_log"].index_select(0, idx).contiguous())
        ox["gate_bias"] = to_host(d["gate_bias"].index_select(0, idx).contiguous())
    return ox


def oracle_batched(d, chains=None, scale=None, flags=0, threads=None):
    """fp64 oracle on the chains (b, h) of a batched input dict.  Returns
    (list of [T, dv] outputs, [n, dk, dv] final states) in chain order.
    The chains are gathered into one batch (one oracle head per chain) so that
    the oracle runs them in parallel threads.  ``flags``: the oracle's input
    transforms (A_log and gate_bias from d)."""
    B, H = d["B"], d["H"]
    if chains is None:
        chains = [(b, h) for b in range(B) for h in range(H)]
    chains = list(chains)
    if not chains:
        return [], np.zeros((0,))
    pick = lambda t: torch.stack([t[b, :, h] for (b, h) in chains], dim=1).unsqueeze(0).contiguous()
    s0 = None
    if d["S0"] is not None:
        s0 = to_host(torch.stack([d["S0"][b, h] for (b, h) in chains]).unsqueeze(0).contiguous())
    o, S = oracle.forward(to_host(pick(d["q"])), to_host(pick(d["k"])), to_host(pick(d["v"])),
                          to_host(pick(d["g"])), to_host(pick(d["beta"])), S0=s0, scale=scale,
                          threads=threads, **_pro_args_many(d, [h for (_, h) in chains], flags))
    return list(o), S


def oracle_varlen(d, chains=None, scale=None, flags=0, threads=None):
    """fp64 oracle on chains (n, h) of a packed input dict.  Chains of one
    head go to the oracle together (packed, in parallel threads)."""
    H = d["H"]
    cu = to_host(d["cu_seqlens"]).astype(np.int64)
    if chains is None:
        chains = [(n, h) for n in range(d["N"]) for h in range(H)]
    chains = list(chains)
    outs, states = [None] * len(chains), [None] * len(chains)
    for h in sorted(set(h for (_, h) in chains)):
        idx = [i for i, (_, hh) in enumerate(chains) if hh == h]
        seqs = [chains[i][0] for i in idx]
        lens = [int(cu[n + 1] - cu[n]) for n in seqs]
        cu1 = np.zeros(len(seqs) + 1, np.int32)
        cu1[1:] = np.cumsum(lens)

        def pack(t):
            parts = [t[int(cu[n]):int(cu[n + 1]), h:h + 1] for n in seqs]
            return to_host(torch.cat(parts, dim=0).contiguous())

        s0 = None
        if d["S0"] is not None:
            s0 = to_host(torch.stack([d["S0"][n, h:h + 1] for n in seqs]).contiguous())
        o, S = oracle.forward(pack(d["q"]), pack(d["k"]), pack(d["v"]), pack(d["g"]),
                              pack(d["beta"]), S0=s0, scale=scale, cu_seqlens=cu1,
                              threads=threads, **_pro_args_many(d, [h], flags))
        for j, i in enumerate(idx):
            outs[i] = o[j]
            states[i] = S[j]
    return outs, np.stack(states)


def gpu_chains_batched(out, S_final, chains):
    o = [out[b, :, h].float().cpu().numpy() for (b, h) in chains]
    s = np.stack([S_final[b, h].cpu().numpy() for (b, h) in chains])
    return o, s


def gpu_chains_varlen(out, S_final, cu, chains):
    cu = cu.cpu().numpy().astype(np.int64)
    o = [out[cu[n]:cu[n + 1], h].float().cpu().numpy() for (n, h) in chains]
    s = np.stack([S_final[n, h].cpu().numpy() for (n, h) in chains])
    return o, s


def concat(xs, dv):
    xs = [np.asarray(x, np.float64).reshape(-1, dv) for x in xs]
    return np.concatenate(xs, axis=0) if xs else np.zeros((0, dv))


def chain_errors(o_gpu, s_gpu, o_ref, s_ref):
    """Per-chain rel-L2 of the outputs (None for empty chains) and states,
    and the per-64-token-block maximum of the outputs."""
    eo, es, eb = [], [], 0.0
    for c in range(len(o_ref)):
        og = np.asarray(o_gpu[c], np.float64)
        orf = np.asarray(o_ref[c], np.float64)
        if orf.size:
            eo.append(rel_l2(og, orf))
            for r0 in range(0, orf.shape[0], BLOCK_ROWS):
                eb = max(eb, rel_l2(og[r0:r0 + BLOCK_ROWS], orf[r0:r0 + BLOCK_ROWS]))
        es.append(rel_l2(np.asarray(s_gpu)[c], np.asarray(s_ref)[c]))
    return eo, es, eb


def assert_close(o_gpu, s_gpu, o_ref, s_ref, tol, what=""):
    dv = s_ref.shape[-1]
    eo = rel_l2(concat(o_gpu, dv), concat(o_ref, dv))
    es = rel_l2(s_gpu, s_ref)
    co, cs, cb = chain_errors(o_gpu, s_gpu, o_ref, s_ref)
    mo = max(co) if co else 0.0
    ms = max(cs) if cs else 0.0
    print("%s rel-L2 o=%.3e S=%.3e; per-chain max o=%.3e S=%.3e; per-64-row max o=%.3e "
          "(%d chains, tol %.1e)" % (what, eo, es, mo, ms, cb, len(cs), tol), flush=True)
    assert np.isfinite(eo) and eo <= tol, "%s: output rel-L2 %.3e > %.1e" % (what, eo, tol)
    assert np.isfinite(es) and es <= tol, "%s: state rel-L2 %.3e > %.1e" % (what, es, tol)
    assert np.isfinite(mo) and mo <= tol, "%s: per-chain output rel-L2 %.3e > %.1e" % (what, mo, tol)
    assert np.isfinite(ms) and ms <= tol, "%s: per-chain state rel-L2 %.3e > %.1e" % (what, ms, tol)
    assert np.isfinite(cb) and cb <= tol, "%s: per-block output rel-L2 %.3e > %.1e" % (what, cb, tol)
    return eo, es
