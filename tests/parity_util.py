"""Helpers shared by the GPU parity tests: run the oracle on host copies of
exactly the tensors the HIP path received and compare element by element."""
import numpy as np
import torch

import oracle
from gated_delta_rule_06_amd.inputs import to_host

# rel-L2 bounds: fp32 I/O and bf16 I/O with fp32 state
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return num / den if den > 0 else num


def tol_for(io):
    return TOL_BF16 if io == "bf16" else TOL_F32


def _pro_args(d, h, flags):
    """Oracle keyword arguments for the input transforms of head h."""
    if not flags:
        return {}
    ox = {"flags": flags}
    if flags & oracle.GATE:
        ox["A_log"] = to_host(d["A_log"][h:h + 1].contiguous())
        ox["gate_bias"] = to_host(d["gate_bias"][h:h + 1].contiguous())
    return ox


def oracle_batched(d, chains=None, scale=None, flags=0):
    """fp64 oracle on the chains (b, h) of a batched input dict.  Returns
    (list of [T, dv] outputs, [n, dk, dv] final states) in chain order.
    ``flags``: the oracle's input transforms (A_log and gate_bias from d)."""
    B, H = d["B"], d["H"]
    if chains is None:
        chains = [(b, h) for b in range(B) for h in range(H)]
    outs, states = [], []
    for (b, h) in chains:
        sl = lambda t: None if t is None else to_host(t[b:b + 1, :, h:h + 1].contiguous())
        s0 = None if d["S0"] is None else to_host(d["S0"][b:b + 1, h:h + 1].contiguous())
        o, S = oracle.forward(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]),
                              to_host(d["beta"][b:b + 1, :, h:h + 1].contiguous()), S0=s0,
                              scale=scale, **_pro_args(d, h, flags))
        outs.append(o[0])
        states.append(S[0])
    return outs, np.stack(states) if states else np.zeros((0,))


def oracle_varlen(d, chains=None, scale=None, flags=0):
    """fp64 oracle on chains (n, h) of a packed input dict."""
    H = d["H"]
    cu = to_host(d["cu_seqlens"]).astype(np.int64)
    if chains is None:
        chains = [(n, h) for n in range(d["N"]) for h in range(H)]
    outs, states = [], []
    for (n, h) in chains:
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda t: to_host(t[a:b, h:h + 1].contiguous())
        s0 = None if d["S0"] is None else to_host(d["S0"][n:n + 1, h:h + 1].contiguous())
        cu1 = np.array([0, b - a], np.int32)
        o, S = oracle.forward(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]),
                              S0=s0, scale=scale, cu_seqlens=cu1, **_pro_args(d, h, flags))
        outs.append(o[0])
        states.append(S[0])
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


def assert_close(o_gpu, s_gpu, o_ref, s_ref, tol, what=""):
    dv = s_ref.shape[-1]
    eo = rel_l2(concat(o_gpu, dv), concat(o_ref, dv))
    es = rel_l2(s_gpu, s_ref)
    print("%s rel-L2 o=%.3e S=%.3e (tol %.1e)" % (what, eo, es, tol), flush=True)
    assert np.isfinite(eo) and eo <= tol, "%s: output rel-L2 %.3e > %.1e" % (what, eo, tol)
    assert np.isfinite(es) and es <= tol, "%s: state rel-L2 %.3e > %.1e" % (what, es, tol)
    return eo, es
