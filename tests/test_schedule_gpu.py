"""Schedule invariance and determinism on the GPU, through the C ABI.

"Kimi Unveils Delta Attention and K3 Architecture Updates", section 6: the
chunkwise form must give exactly the states and outputs of the token-by-token
recurrence, however the tokens are grouped.  The state is the method's whole
memory ("Linear Attention, From Scratch to Kimi 3", section 9: prefill hands a
state to decode), so:

* a prefill split in two, the second half started from the first half's
  S_final, matches one oracle run over the whole sequence; split at a chunk
  boundary it is bit-identical to the unsplit prefill (the state is carried in
  fp32 either way);
* a prefill of T1 tokens followed by T2 decode steps matches one oracle run
  over T1 + T2 tokens;
* packed (varlen) calls give, bit for bit, what separate batched calls give
  for each sequence;
* every call is deterministic: a rerun on the same inputs is bit-identical
  (no atomics, no order-dependent reductions).
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_06_amd import inputs
from parity_util import assert_close, gpu_chains_batched, oracle_batched, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def kda():
    from gated_delta_rule_06_amd import kda as k
    return k


def note(msg):
    print(msg, flush=True)


def _slice_t(d, a, b):
    """Tokens [a, b) of a batched input dict (contiguous copies)."""
    e = dict(d)
    for n in ("q", "k", "v", "g", "beta"):
        e[n] = d[n][:, a:b].contiguous()
    e["T"] = b - a
    return e


# ------------------------------------------------------------------ determinism

def test_reruns_are_bit_identical():
    note("determinism: chunk, packed chunk, decode, recurrent, backward")
    K = kda()
    d = inputs.prefill_inputs(2, 300, 3, 128, 128, io="bf16", seed=11, with_S0=True, device=DEV)
    runs = [K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"]) for _ in range(2)]
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(runs[0], runs[1])), "chunk_fwd"

    dv_ = inputs.varlen_inputs([70, 0, 129, 5], 2, 128, 128, io="bf16", seed=12, with_S0=True,
                               long_channels=8, device=DEV)
    runs = [K.chunk_fwd_varlen(dv_["q"], dv_["k"], dv_["v"], dv_["g"], dv_["beta"],
                               dv_["cu_seqlens"], S0=dv_["S0"]) for _ in range(2)]
    runs_r = [K.recurrent_fwd_varlen(dv_["q"], dv_["k"], dv_["v"], dv_["g"], dv_["beta"],
                                     dv_["cu_seqlens"], S0=dv_["S0"]) for _ in range(2)]
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(runs[0], runs[1])), "chunk_fwd_varlen"
    assert all(torch.equal(a, b) for a, b in zip(runs_r[0], runs_r[1])), "recurrent_fwd_varlen"

    dd = inputs.decode_inputs(8, 4, 128, 128, 3, io="bf16", seed=13, device=DEV)
    outs = []
    for _ in range(2):
        S = dd["S"].clone()
        o = [K.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["g"][t], dd["beta"][t], S)
             for t in range(3)]
        outs.append((torch.stack(o), S))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), "decode"

    # the chunk-parallel schedule (few long chains)
    dp = inputs.prefill_inputs(1, 1100, 4, 128, 128, io="bf16", seed=15, with_S0=True, device=DEV)
    assert K.chunk_fwd_workspace_size(1, 1100, 4, 128, 128) > 0
    runs = [K.chunk_fwd(dp["q"], dp["k"], dp["v"], dp["g"], dp["beta"], S0=dp["S0"])
            for _ in range(2)]
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(runs[0], runs[1])), "chunk-parallel"

    inputs.grad_inputs(d, seed=14, device=DEV)
    g1 = K.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_out"], S0=d["S0"],
                    dS_final=d["dS_final"])
    g2 = K.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_out"], S0=d["S0"],
                    dS_final=d["dS_final"])
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), "backward " + n


# ------------------------------------------------------------------ split prefill

@pytest.mark.parametrize("T1,T2,io,dk", [(200, 190, "bf16", 128), (77, 60, "f32", 64)])
def test_split_prefill_matches_one_oracle_run(T1, T2, io, dk):
    """chunk_fwd over [0, T1), then over [T1, T1 + T2) from its S_final,
    against one oracle run over all T1 + T2 tokens (split inside a chunk)."""
    note("split prefill T1=%d T2=%d io=%s" % (T1, T2, io))
    K = kda()
    d = inputs.prefill_inputs(2, T1 + T2, 2, dk, dk, io=io, seed=T1, with_S0=True, device=DEV)
    a, b = _slice_t(d, 0, T1), _slice_t(d, T1, T1 + T2)
    o1, S1 = K.chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], S0=d["S0"])
    o2, S2 = K.chunk_fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], S0=S1)
    torch.cuda.synchronize()
    chains = [(x, h) for x in range(2) for h in range(2)]
    ro, rs = oracle_batched(d, chains)
    go, gs = gpu_chains_batched(torch.cat([o1, o2], dim=1), S2, chains)
    assert_close(go, gs, ro, rs, tol_for(io), "split prefill")


def test_split_at_chunk_boundary_is_bit_identical():
    """Split at token 128 (a chunk boundary): the second call starts from the
    exact fp32 state the unsplit call holds there, so every bit agrees."""
    note("split prefill at a chunk boundary")
    K = kda()
    d = inputs.prefill_inputs(2, 300, 3, 128, 128, io="bf16", seed=5, with_S0=True, device=DEV)
    ow, Sw = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    a, b = _slice_t(d, 0, 128), _slice_t(d, 128, 300)
    o1, S1 = K.chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], S0=d["S0"])
    o2, S2 = K.chunk_fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], S0=S1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=1), ow)
    assert torch.equal(S2, Sw)


# ------------------------------------------------------------------ prefill -> decode

@pytest.mark.parametrize("T1,T2,io,dk", [(150, 12, "bf16", 128), (64, 9, "f32", 64)])
def test_prefill_then_decode_matches_one_oracle_run(T1, T2, io, dk):
    """chunk_fwd over T1 tokens, then T2 kda_decode_step calls on its S_final,
    against one oracle run over the T1 + T2 tokens."""
    note("prefill %d then decode %d io=%s" % (T1, T2, io))
    K = kda()
    B, H = 3, 2
    d = inputs.prefill_inputs(B, T1 + T2, H, dk, dk, io=io, seed=T1 + T2, with_S0=True, device=DEV)
    a = _slice_t(d, 0, T1)
    o1, S = K.chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], S0=d["S0"])
    outs = [o1]
    for t in range(T1, T1 + T2):
        o = K.decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                          d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                          d["beta"][:, t].contiguous(), S)
        outs.append(o[:, None])
    torch.cuda.synchronize()
    chains = [(x, h) for x in range(B) for h in range(H)]
    ro, rs = oracle_batched(d, chains)
    go, gs = gpu_chains_batched(torch.cat(outs, dim=1), S, chains)
    assert_close(go, gs, ro, rs, tol_for(io), "prefill+decode")


# ------------------------------------------------------------------ packed vs separate

@pytest.mark.parametrize("gate", ["kda", "gdn"])
def test_packed_equals_separate_batched_calls(gate):
    """Each packed sequence gives, bit for bit, what a batched call on that
    sequence alone gives: prefill, multi-token recurrence and backward."""
    note("packed vs separate gate=%s" % gate)
    K = kda()
    lens = [130, 1, 64, 0, 77]
    d = inputs.varlen_inputs(lens, 2, 128, 128, io="bf16", seed=21, with_S0=True,
                             long_channels=0 if gate == "gdn" else 8, device=DEV, gate=gate)
    inputs.grad_inputs(d, seed=21, device=DEV)
    cu = d["cu_seqlens"].cpu().numpy()
    op, Sp = K.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                S0=d["S0"])
    orp, Srp = K.recurrent_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                      S0=d["S0"])
    gp = K.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_out"], S0=d["S0"],
                    dS_final=d["dS_final"], cu_seqlens=d["cu_seqlens"])
    for n, L in enumerate(lens):
        a, b = int(cu[n]), int(cu[n + 1])
        one = lambda t: t[a:b].unsqueeze(0).contiguous()
        s0 = d["S0"][n:n + 1].contiguous()
        o1, S1 = K.chunk_fwd(one(d["q"]), one(d["k"]), one(d["v"]), one(d["g"]), one(d["beta"]),
                             S0=s0)
        or1, Sr1 = K.recurrent_fwd(one(d["q"]), one(d["k"]), one(d["v"]), one(d["g"]),
                                   one(d["beta"]), S0=s0)
        g1 = K.backward(one(d["q"]), one(d["k"]), one(d["v"]), one(d["g"]), one(d["beta"]),
                        one(d["d_out"]), S0=s0, dS_final=d["dS_final"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o1[0], op[a:b]) and torch.equal(S1[0], Sp[n]), ("chunk", n)
        assert torch.equal(or1[0], orp[a:b]) and torch.equal(Sr1[0], Srp[n]), ("recurrent", n)
        for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
            assert torch.equal(g1[name][0], gp[name][a:b]), ("backward", name, n)
        assert torch.equal(g1["dS0"][0], gp["dS0"][n]), ("backward dS0", n)
