"""GPU parity of the Gated DeltaNet calls (kda_gdn_*: one gate per token and
head) against the fp64 oracle, through the C ABI.  The oracle takes the same
per-(token, head) gates (it broadcasts them over the key channels).  Bars:
rel-L2 <= 1e-4 for fp32 I/O, <= 2e-2 for bf16 I/O with fp32 state."""
import numpy as np
import pytest
import torch

from gated_delta_rule_06_amd import inputs
from parity_util import (assert_close, gpu_chains_batched, gpu_chains_varlen, oracle_batched,
                         oracle_varlen, rel_l2, tol_for)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def kda():
    from gated_delta_rule_06_amd import kda as k
    return k


def note(msg):
    print(msg, flush=True)


CHUNK_CASES = [
    # (B, T, H, dk, dv, io, with_S0)
    (1, 256, 1, 64, 64, "f32", False),
    (2, 77, 2, 64, 64, "f32", True),
    (2, 300, 3, 128, 128, "bf16", True),
    (1, 63, 2, 128, 64, "bf16", False),
    (3, 130, 2, 64, 128, "bf16", True),
    (1, 1, 2, 128, 128, "bf16", True),
]


@pytest.mark.parametrize("B,T,H,dk,dv,io,with_S0", CHUNK_CASES)
def test_gdn_chunk_fwd_matches_oracle(B, T, H, dk, dv, io, with_S0):
    note("gdn chunk_fwd B=%d T=%d H=%d dk=%d dv=%d io=%s S0=%s" % (B, T, H, dk, dv, io, with_S0))
    d = inputs.prefill_inputs(B, T, H, dk, dv, io=io, seed=17 * B + T, with_S0=with_S0,
                              device=DEV, gate="gdn")
    assert d["g"].shape == (B, T, H)
    o, S = kda().chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    torch.cuda.synchronize()
    chains = [(b, h) for b in range(B) for h in range(H)]
    ro, rs = oracle_batched(d, chains)
    go, gs = gpu_chains_batched(o, S, chains)
    assert_close(go, gs, ro, rs, tol_for(io), "gdn chunk")


@pytest.mark.parametrize("gate,io", [("-3", "bf16"), ("-30", "f32"), ("uniform", "f32"),
                                     ("strong_then_weak", "f32")])
def test_gdn_chunk_strong_decay_matches_oracle(gate, io):
    """Decays far beyond one chunk's range: log alpha = -3 or -30 for every token
    (a chunk decays by e^-192 or e^-1920), or uniform in [-8, 0], or -100 for the
    first 32 tokens of each chunk and -0.01 for the rest (the later tokens' decay
    ratios must not inherit the rounding of the large early sums).  The
    scalar-gate chunk step scales its products by per-token ratios
    Gamma_i / Gamma_j <= 1, so it needs no guard; the results must still match."""
    note("gdn chunk strong decay gate=%s io=%s" % (gate, io))
    dim = 128 if io == "bf16" else 64      # fp32 I/O runs d_k = d_v = 64
    d = inputs.prefill_inputs(1, 150, 2, dim, dim, io=io, seed=3, with_S0=True, device=DEV,
                              gate="gdn")
    if gate == "uniform":
        gen = torch.Generator().manual_seed(11)
        d["g"] = (-8.0 * torch.rand(d["g"].shape, generator=gen)).to(DEV)
    elif gate == "strong_then_weak":
        g = torch.full_like(d["g"], -0.01)
        g[:, (torch.arange(g.shape[1], device=g.device) % 64) < 32] = -100.0
        d["g"] = g.contiguous()
    else:
        d["g"] = torch.full_like(d["g"], float(gate))
    o, S = kda().chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    torch.cuda.synchronize()
    chains = [(0, 0), (0, 1)]
    ro, rs = oracle_batched(d, chains)
    go, gs = gpu_chains_batched(o, S, chains)
    assert_close(go, gs, ro, rs, tol_for(io), "gdn strong decay")


@pytest.mark.parametrize("lens,H,dk,dv,io,with_S0", [
    ([70, 0, 1, 129, 64], 2, 128, 128, "bf16", True),
    ([5, 0, 0, 9], 3, 64, 64, "f32", False),
])
def test_gdn_chunk_varlen_matches_oracle(lens, H, dk, dv, io, with_S0):
    note("gdn varlen lens=%s H=%d dk=%d dv=%d io=%s" % (lens, H, dk, dv, io))
    d = inputs.varlen_inputs(lens, H, dk, dv, io=io, seed=len(lens), with_S0=with_S0,
                             device=DEV, gate="gdn")
    o, S = kda().chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                  S0=d["S0"])
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(d["N"]) for h in range(H)]
    ro, rs = oracle_varlen(d, chains)
    go, gs = gpu_chains_varlen(o, S, d["cu_seqlens"], chains)
    assert_close(go, gs, ro, rs, tol_for(io), "gdn varlen")


@pytest.mark.parametrize("N,H,dk,dv,io", [(4, 3, 128, 128, "bf16"), (3, 2, 64, 64, "f32")])
def test_gdn_decode_steps_match_oracle(N, H, dk, dv, io):
    steps = 9
    note("gdn decode N=%d H=%d dk=%d dv=%d io=%s" % (N, H, dk, dv, io))
    d = inputs.decode_inputs(N, H, dk, dv, steps, io=io, seed=8, device=DEV, gate="gdn")
    assert d["g"].shape == (steps, N, H)
    S = d["S"].clone()
    outs = [kda().decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], S)
            for t in range(steps)]
    torch.cuda.synchronize()
    import oracle
    from gated_delta_rule_06_amd.inputs import to_host
    tm = lambda x: to_host(x.transpose(0, 1).contiguous())
    ro, rs = oracle.forward_dense(tm(d["q"]), tm(d["k"]), tm(d["v"]), tm(d["g"]), tm(d["beta"]),
                                  S0=to_host(d["S"]))
    go = torch.stack(outs, 1).float().cpu().numpy()
    tol = tol_for(io) if io == "bf16" else 1e-5
    eo, es = rel_l2(go, ro), rel_l2(S.cpu().numpy(), rs)
    note("gdn decode rel-L2 o=%.3e S=%.3e" % (eo, es))
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("B,T,H,dk,dv,io", [(2, 9, 3, 128, 128, "bf16"), (2, 40, 2, 64, 128, "f32")])
def test_gdn_recurrent_fwd_matches_oracle(B, T, H, dk, dv, io):
    note("gdn recurrent B=%d T=%d H=%d dk=%d dv=%d io=%s" % (B, T, H, dk, dv, io))
    d = inputs.prefill_inputs(B, T, H, dk, dv, io=io, seed=5 + T, with_S0=True, device=DEV,
                              gate="gdn")
    o, S = kda().recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    torch.cuda.synchronize()
    chains = [(b, h) for b in range(B) for h in range(H)]
    ro, rs = oracle_batched(d, chains)
    go, gs = gpu_chains_batched(o, S, chains)
    assert_close(go, gs, ro, rs, tol_for(io), "gdn recurrent")


def test_gdn_recurrent_varlen_in_place_matches_oracle():
    note("gdn recurrent varlen")
    d = inputs.varlen_inputs([3, 0, 8, 1], 2, 128, 128, io="bf16", seed=2, with_S0=True,
                             device=DEV, gate="gdn")
    S = d["S0"].clone()
    o, _ = kda().recurrent_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                      d["cu_seqlens"], S0=S, S_final=S)
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(4) for h in range(2)]
    ro, rs = oracle_varlen(d, chains)
    go, gs = gpu_chains_varlen(o, S, d["cu_seqlens"], chains)
    assert_close(go, gs, ro, rs, tol_for("bf16"), "gdn recurrent varlen")


def test_gdn_headline_prefill_sampled_chains():
    """B=8, H=32, T=8192, d=128 bf16 with per-(token, head) gates, in the
    benchmark's launch; the oracle checks sampled chains."""
    note("gdn prefill_b8_h32_t8192 full")
    d = inputs.prefill_inputs(8, 8192, 32, 128, 128, io="bf16", seed=0, device=DEV, gate="gdn")
    o, S = kda().chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    assert torch.isfinite(S).all()
    chains = [(0, 0), (3, 17), (7, 31)]
    ro, rs = oracle_batched(d, chains)
    go, gs = gpu_chains_batched(o, S, chains)
    assert_close(go, gs, ro, rs, tol_for("bf16"), "gdn headline")
