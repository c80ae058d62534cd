"""GPU parity of the token-by-token recurrent calls (kda_recurrent_fwd and
kda_recurrent_fwd_varlen) against the fp64 oracle, through the C ABI.  Bars
as for the other calls: rel-L2 <= 1e-4 for fp32 I/O, <= 2e-2 for bf16 I/O
with fp32 state, on the outputs and the final states."""
import numpy as np
import pytest
import torch

from gated_delta_rule_06_amd import inputs
from parity_util import (assert_close, gpu_chains_batched, gpu_chains_varlen, oracle_batched,
                         oracle_varlen, tol_for)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def kda():
    from gated_delta_rule_06_amd import kda as k
    return k


def note(msg):
    print(msg, flush=True)


DENSE_CASES = [
    # (B, T, H, dk, dv, io, with_S0)
    (2, 7, 3, 128, 128, "bf16", True),
    (3, 1, 2, 64, 64, "f32", True),       # one token: the decode step
    (1, 33, 2, 64, 128, "f32", False),
    (2, 17, 2, 128, 64, "bf16", True),
    (2, 5, 2, 128, 128, "f32", True),
    (1, 300, 1, 128, 128, "f32", True),   # long: error growth over many steps
    (2, 2, 5, 64, 64, "bf16", False),
]


@pytest.mark.parametrize("B,T,H,dk,dv,io,with_S0", DENSE_CASES)
def test_recurrent_fwd_matches_oracle(B, T, H, dk, dv, io, with_S0):
    note("recurrent_fwd B=%d T=%d H=%d dk=%d dv=%d io=%s S0=%s" % (B, T, H, dk, dv, io, with_S0))
    d = inputs.prefill_inputs(B, T, H, dk, dv, io=io, seed=31 * B + T, with_S0=with_S0,
                              device=DEV)
    o, S = kda().recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    torch.cuda.synchronize()
    chains = [(b, h) for b in range(B) for h in range(H)]
    ro, rs = oracle_batched(d, chains)
    go, gs = gpu_chains_batched(o, S, chains)
    assert_close(go, gs, ro, rs, tol_for(io), "recurrent")


def test_recurrent_in_place_equals_out_of_place():
    """S_final == S0 (the serving call) gives bit-identical results."""
    note("recurrent in place")
    d = inputs.prefill_inputs(3, 6, 4, 128, 128, io="bf16", seed=5, with_S0=True, device=DEV)
    o1, S1 = kda().recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    S = d["S0"].clone()
    o2, S2 = kda().recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S, S_final=S)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S)


def test_recurrent_zero_tokens_copies_the_state():
    note("recurrent T=0")
    d = inputs.prefill_inputs(2, 0, 3, 64, 64, io="f32", seed=1, with_S0=True, device=DEV)
    Sf = torch.full_like(d["S0"], float("nan"))
    o, S = kda().recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"], S_final=Sf)
    o2, S2 = kda().recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=None)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S, d["S0"])
    assert torch.count_nonzero(S2) == 0


def test_recurrent_matches_decode_steps():
    """T tokens in one call against T chained decode steps: both follow the
    same recurrence (their reductions are ordered differently)."""
    note("recurrent vs decode")
    N, H, dk, dv, T = 4, 3, 128, 128, 6
    d = inputs.decode_inputs(N, H, dk, dv, T, io="bf16", seed=11, device=DEV)
    S = d["S"].clone()
    outs = [kda().decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], S)
            for t in range(T)]
    tm = lambda x: x.transpose(0, 1).contiguous()       # [T, N, ...] -> [N, T, ...]
    o, Sr = kda().recurrent_fwd(tm(d["q"]), tm(d["k"]), tm(d["v"]), tm(d["g"]), tm(d["beta"]),
                                S0=d["S"])
    torch.cuda.synchronize()
    od = torch.stack(outs, 1).float()
    assert (o.float() - od).norm() / od.norm() < 1e-2
    assert (Sr - S).norm() / S.norm() < 1e-4


VARLEN_CASES = [
    # (lens, H, dk, dv, io, with_S0)
    ([3, 0, 1, 8, 5], 2, 128, 128, "bf16", True),
    ([1, 1, 1, 1, 1, 1, 1], 3, 64, 64, "f32", True),
    ([0], 2, 128, 64, "bf16", True),
    ([40, 2, 0, 17], 2, 64, 128, "f32", False),
    ([9, 0, 0, 4], 3, 128, 128, "f32", True),
]


@pytest.mark.parametrize("lens,H,dk,dv,io,with_S0", VARLEN_CASES)
def test_recurrent_varlen_matches_oracle(lens, H, dk, dv, io, with_S0):
    note("recurrent_varlen lens=%s H=%d dk=%d dv=%d io=%s" % (lens, H, dk, dv, io))
    d = inputs.varlen_inputs(lens, H, dk, dv, io=io, seed=7 + len(lens), with_S0=with_S0,
                             device=DEV)
    o, S = kda().recurrent_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                      d["cu_seqlens"], S0=d["S0"])
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(d["N"]) for h in range(H)]
    ro, rs = oracle_varlen(d, chains)
    go, gs = gpu_chains_varlen(o, S, d["cu_seqlens"], chains)
    if sum(lens) == 0:
        np.testing.assert_array_equal(gs, rs)   # state copied through untouched
    else:
        assert_close(go, gs, ro, rs, tol_for(io), "recurrent varlen")


def test_recurrent_varlen_full_size_sampled():
    """256 sequences of U{1..8} tokens on resident states (32 heads, 512 MiB
    of fp32 state), updated in place as in the benchmark; the oracle checks
    sampled (sequence, head) chains, the empty and longest among them."""
    cfg = inputs.CONFIGS["recurrent_n256_h32"]
    lens = inputs.varlen_lengths(cfg["n_seq"], cfg["lo"], cfg["hi"], seed=0)
    note("recurrent_n256_h32 total=%d" % int(lens.sum()))
    d = inputs.varlen_inputs(lens, cfg["H"], cfg["dk"], cfg["dv"], io=cfg["io"], seed=0,
                             with_S0=True, device=DEV)
    S = d["S0"].clone()
    o, _ = kda().recurrent_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                      d["cu_seqlens"], S0=S, S_final=S)
    torch.cuda.synchronize()
    assert torch.isfinite(S).all()
    chains = [(0, 0), (int(np.argmax(lens)), 7), (int(np.argmin(lens)), 31), (255, 16)]
    ro, rs = oracle_varlen(d, chains)
    go, gs = gpu_chains_varlen(o, S, d["cu_seqlens"], chains)
    assert_close(go, gs, ro, rs, tol_for("bf16"), "recurrent full")
