"""GPU parity of the in-kernel input transforms (kda_*_fused with a
kda_prologue: q/k L2 norm, beta sigmoid, the -5 sigmoid gate) against the
fp64 oracle applying the same transforms to the same raw inputs.  Bars as for
the plain calls: rel-L2 <= 1e-4 (fp32 I/O), <= 2e-2 (bf16 I/O)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_06_amd import inputs
from gated_delta_rule_06_amd.inputs import to_host
from parity_util import (assert_close, gpu_chains_batched, gpu_chains_varlen, oracle_batched,
                         oracle_varlen, rel_l2, tol_for)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ALL = oracle.L2NORM | oracle.BETA_SIGMOID | oracle.GATE


def kda():
    from gated_delta_rule_06_amd import kda as k
    return k


def note(msg):
    print(msg, flush=True)


def kw(d, flags):
    """Binding keyword arguments for the transforms in ``flags``."""
    out = {"qk_l2norm": bool(flags & oracle.L2NORM),
           "beta_sigmoid": bool(flags & oracle.BETA_SIGMOID)}
    if flags & oracle.GATE:
        out["A_log"] = d["A_log"]
        out["gate_bias"] = d["gate_bias"]
    return out


CHUNK_CASES = [
    # (B, T, H, dk, dv, io, gate, flags, strong_decay)
    (2, 150, 2, 128, 128, "bf16", "kda", ALL, False),
    (1, 130, 2, 64, 64, "f32", "kda", ALL, False),
    (2, 90, 3, 128, 64, "bf16", "gdn", ALL, False),
    (1, 100, 2, 128, 128, "bf16", "kda", oracle.L2NORM, False),
    (1, 70, 2, 64, 128, "bf16", "kda", oracle.BETA_SIGMOID, False),
    (1, 80, 2, 64, 64, "f32", "gdn", oracle.GATE, False),
    (1, 96, 2, 128, 128, "bf16", "kda", ALL, True),     # log alpha near -5 in every channel
    (1, 65, 1, 64, 64, "f32", "gdn", ALL, True),
]


@pytest.mark.parametrize("B,T,H,dk,dv,io,gate,flags,strong", CHUNK_CASES)
def test_fused_chunk_fwd_matches_oracle(B, T, H, dk, dv, io, gate, flags, strong):
    note("fused chunk B=%d T=%d H=%d dk=%d dv=%d io=%s gate=%s flags=%d strong=%s"
         % (B, T, H, dk, dv, io, gate, flags, strong))
    d = inputs.prefill_inputs(B, T, H, dk, dv, io=io, seed=3 * T + B, with_S0=True, device=DEV,
                              gate=gate)
    d = inputs.raw_layer_inputs(d, H, dk, seed=T, gate=gate, strong_decay=strong, device=DEV)
    o, S = kda().chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"], **kw(d, flags))
    torch.cuda.synchronize()
    chains = [(b, h) for b in range(B) for h in range(H)]
    ro, rs = oracle_batched(d, chains, flags=flags)
    go, gs = gpu_chains_batched(o, S, chains)
    assert_close(go, gs, ro, rs, tol_for(io), "fused chunk")


def test_fused_guard_path_matches_oracle():
    """The token-by-token guard path with the q/k norm and beta transforms:
    raw log alpha (no gate transform) at -20 in 8 channels over tokens
    40 .. 110, so the chunks holding them decay below 2^-120 within a
    16-token block; the other chunks take the MFMA path."""
    note("fused guard path")
    flags = oracle.L2NORM | oracle.BETA_SIGMOID
    d = inputs.prefill_inputs(2, 150, 2, 128, 128, io="bf16", seed=17, with_S0=True, device=DEV)
    g = d["g"].clone()
    d = inputs.raw_layer_inputs(d, 2, 128, seed=17, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9)
    idx = torch.randperm(128, generator=gen, device=DEV)[:8]
    sl = g[:, 40:110]
    sl[..., idx] = -20.0
    d["g"] = g
    o, S = kda().chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"], **kw(d, flags))
    torch.cuda.synchronize()
    chains = [(b, h) for b in range(2) for h in range(2)]
    ro, rs = oracle_batched(d, chains, flags=flags)
    go, gs = gpu_chains_batched(o, S, chains)
    assert_close(go, gs, ro, rs, tol_for("bf16"), "fused guard path")


@pytest.mark.parametrize("lens,gate", [([70, 0, 1, 129], "kda"), ([33, 64, 0], "gdn")])
def test_fused_chunk_varlen_matches_oracle(lens, gate):
    note("fused chunk varlen lens=%s gate=%s" % (lens, gate))
    H, dk, dv = 2, 128, 128
    d = inputs.varlen_inputs(lens, H, dk, dv, io="bf16", seed=len(lens), with_S0=True,
                             device=DEV, gate=gate)
    d = inputs.raw_layer_inputs(d, H, dk, seed=1, gate=gate, device=DEV)
    o, S = kda().chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                  S0=d["S0"], **kw(d, ALL))
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(d["N"]) for h in range(H)]
    ro, rs = oracle_varlen(d, chains, flags=ALL)
    go, gs = gpu_chains_varlen(o, S, d["cu_seqlens"], chains)
    assert_close(go, gs, ro, rs, tol_for("bf16"), "fused varlen")


@pytest.mark.parametrize("B,T,H,dk,dv,io,gate", [(2, 7, 3, 128, 128, "bf16", "kda"),
                                                 (2, 40, 2, 64, 64, "f32", "kda"),
                                                 (3, 5, 2, 128, 64, "bf16", "gdn")])
def test_fused_recurrent_matches_oracle(B, T, H, dk, dv, io, gate):
    note("fused recurrent B=%d T=%d H=%d dk=%d dv=%d io=%s gate=%s" % (B, T, H, dk, dv, io, gate))
    d = inputs.prefill_inputs(B, T, H, dk, dv, io=io, seed=T, with_S0=True, device=DEV, gate=gate)
    d = inputs.raw_layer_inputs(d, H, dk, seed=2, gate=gate, device=DEV)
    o, S = kda().recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"],
                               **kw(d, ALL))
    torch.cuda.synchronize()
    chains = [(b, h) for b in range(B) for h in range(H)]
    ro, rs = oracle_batched(d, chains, flags=ALL)
    go, gs = gpu_chains_batched(o, S, chains)
    assert_close(go, gs, ro, rs, tol_for(io), "fused recurrent")


def test_fused_recurrent_varlen_in_place_matches_oracle():
    note("fused recurrent varlen")
    H, dk, dv = 2, 128, 128
    d = inputs.varlen_inputs([3, 0, 8, 1], H, dk, dv, io="bf16", seed=4, with_S0=True,
                             device=DEV)
    d = inputs.raw_layer_inputs(d, H, dk, seed=3, device=DEV)
    S = d["S0"].clone()
    o, _ = kda().recurrent_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                      d["cu_seqlens"], S0=S, S_final=S, **kw(d, ALL))
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(4) for h in range(H)]
    ro, rs = oracle_varlen(d, chains, flags=ALL)
    go, gs = gpu_chains_varlen(o, S, d["cu_seqlens"], chains)
    assert_close(go, gs, ro, rs, tol_for("bf16"), "fused recurrent varlen")


@pytest.mark.parametrize("N,H,dk,dv,io,gate", [(4, 3, 128, 128, "bf16", "kda"),
                                               (3, 2, 64, 64, "f32", "gdn")])
def test_fused_decode_steps_match_oracle(N, H, dk, dv, io, gate):
    steps = 6
    note("fused decode N=%d H=%d dk=%d dv=%d io=%s gate=%s" % (N, H, dk, dv, io, gate))
    d = inputs.decode_inputs(N, H, dk, dv, steps, io=io, seed=9, device=DEV, gate=gate)
    d = inputs.raw_layer_inputs(d, H, dk, seed=4, gate=gate, device=DEV)
    S = d["S"].clone()
    outs = [kda().decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], S,
                              **kw(d, ALL)) for t in range(steps)]
    torch.cuda.synchronize()
    tm = lambda x: to_host(x.transpose(0, 1).contiguous())
    outs_ref, S_ref = [], []
    ro, rs = oracle.forward_dense(tm(d["q"]), tm(d["k"]), tm(d["v"]), tm(d["g"]), tm(d["beta"]),
                                  S0=to_host(d["S"]), flags=ALL, A_log=to_host(d["A_log"]),
                                  gate_bias=to_host(d["gate_bias"]))
    go = torch.stack(outs, 1).float().cpu().numpy()
    tol = tol_for(io) if io == "bf16" else 1e-5
    eo, es = rel_l2(go, ro), rel_l2(S.cpu().numpy(), rs)
    note("fused decode rel-L2 o=%.3e S=%.3e" % (eo, es))
    assert eo <= tol and es <= tol


def test_fused_without_transforms_equals_plain_call():
    """kda_chunk_fwd_fused with no prologue is the plain call, bit for bit."""
    import ctypes
    k = kda()
    d = inputs.prefill_inputs(1, 100, 2, 128, 128, io="bf16", seed=1, with_S0=True, device=DEV)
    o1, S1 = k.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(S1)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = k.lib.kda_chunk_fwd_fused(P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]),
                                   P(d["S0"]), P(o2), P(S2), None, 1, 100, 2, 128, 128,
                                   128 ** -0.5, 64, 1, 0, None, None, 0,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
