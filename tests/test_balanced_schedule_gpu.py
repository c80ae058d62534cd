"""GPU: the balanced schedule of prefill calls, packed and batched.  With a
workspace and more (sequence, head) chains than resident workgroups (up to
four times as many; every case here stays in that range), the library cuts the
concatenated sequences into equal slices (McNaughton's wrap-around rule) and
hands the fp32 state of a split sequence from one workgroup to the next.
Chunks stay aligned to their sequence, so the results must equal those of the
one-workgroup-per-chain kernel bit for bit; split chains are also checked
against the fp64 oracle.

White-box: after a call the workspace holds the plan the kernels used (u32
ticket count at byte 0 = workgroups launched; i64 slice length at byte 8 and
total chunk count at byte 16), which shows that the balanced kernels ran."""
import numpy as np
import pytest
import torch

from gated_delta_rule_06_amd import inputs
from parity_util import assert_close, gpu_chains_varlen, oracle_varlen, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
C = 64


def kda():
    from gated_delta_rule_06_amd import kda as k
    return k


def note(msg):
    print(msg, flush=True)


def units(lens):
    return [max(1, -(-int(L) // C)) for L in lens]


def plan_of(ws, H):
    """(workgroups, machines, slice length, total chunks) read back from the workspace."""
    w = ws[:24].cpu().numpy()
    tickets = int(w[0:4].view(np.uint32)[0])
    T, total = (int(x) for x in w[8:24].view(np.int64))
    return tickets, tickets // H, T, total


def split_sequences(lens, T):
    """Sequences that cross a slice boundary (split over two workgroups)."""
    pre = np.concatenate([[0], np.cumsum(units(lens))])
    return [n for n in range(len(lens)) if (pre[n] // T) != ((pre[n + 1] - 1) // T)]


def both(d, ws, **kw):
    K = kda()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"])
    a = K.chunk_fwd_varlen(*args, S0=d["S0"], workspace=ws, **kw)
    b = K.chunk_fwd_varlen(*args, S0=d["S0"], balanced=False, **kw)
    torch.cuda.synchronize()
    return a, b


def workspace_for(d):
    n = kda().lib.kda_chunk_fwd_varlen_workspace_size(
        d["N"], d["T_total"], d["H"], d["dk"], d["dv"], 64, 1 if d["io"] == "bf16" else 0)
    assert n > 0
    return torch.zeros(n, dtype=torch.uint8, device=DEV)


def check_plan(ws, lens, H):
    tickets, M, T, total = plan_of(ws, H)
    u = units(lens)
    assert total == sum(u), "the plan kernel did not run"
    assert tickets == M * H and M >= 2, "the balanced kernel did not run"
    assert T == max(-(-total // M), max(u))
    return M, T


CASES = [
    # (name, n_seq, lo, hi, H, dk, dv, io, gate, with_S0, seed)
    ("skewed bf16", 40, 0, 3000, 8, 128, 128, "bf16", "kda", True, 1),
    ("many short with empties", 60, 0, 140, 16, 128, 128, "bf16", "kda", False, 2),
    ("gated deltanet", 48, 1, 2000, 8, 128, 128, "bf16", "gdn", True, 3),
    ("fp32 64x64", 120, 0, 300, 4, 64, 64, "f32", "kda", True, 4),
    ("bf16 128x64", 70, 0, 1500, 8, 128, 64, "bf16", "kda", True, 5),
    ("one head", 700, 0, 300, 1, 128, 128, "bf16", "kda", True, 6),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_balanced_equals_per_chain_kernel(case):
    name, n_seq, lo, hi, H, dk, dv, io, gate, with_S0, seed = case
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=n_seq)
    lens[0] = max(lens[0], 1)
    note("balanced %s: %d sequences, %d tokens, H=%d" % (name, n_seq, int(lens.sum()), H))
    d = inputs.varlen_inputs(lens, H, dk, dv, io=io, seed=seed, with_S0=with_S0,
                             long_channels=0 if gate == "gdn" else min(8, dk // 4), device=DEV,
                             gate=gate)
    ws = workspace_for(d)
    (oa, Sa), (ob, Sb) = both(d, ws)
    M, T = check_plan(ws, lens, H)
    note("  %d machines, slices of %d chunks, %d sequences split"
         % (M, T, len(split_sequences(lens, T))))
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)


def test_balanced_split_chains_match_oracle():
    """The split sequences of a skewed mix at two heads each, against the
    oracle (plus two unsplit ones)."""
    rng = np.random.default_rng(11)
    lens = rng.integers(200, 2500, size=36)
    H = 8
    d = inputs.varlen_inputs(lens, H, 128, 128, io="bf16", seed=11, with_S0=True,
                             long_channels=8, device=DEV)
    ws = workspace_for(d)
    o, S = kda().chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                  S0=d["S0"], workspace=ws)
    torch.cuda.synchronize()
    M, T = check_plan(ws, lens, H)
    split = split_sequences(lens, T)
    assert split, "no sequence was split"
    whole = [n for n in range(len(lens)) if n not in split][:2]
    note("oracle on split sequences %s and whole ones %s" % (split, whole))
    chains = [(n, h) for n in split + whole for h in (n % H, (n + 3) % H)]
    ro, rs = oracle_varlen(d, chains)
    go, gs = gpu_chains_varlen(o, S, d["cu_seqlens"], chains)
    assert_close(go, gs, ro, rs, tol_for("bf16"), "balanced split chains")


def test_balanced_fast_forgetting_and_guard_path():
    """Block-start references and the token-by-token guard path inside split
    pieces: 8 of 128 channels at log alpha ~ U[-5, -2], and log alpha = -20
    over a stretch of tokens in one channel of every head."""
    rng = np.random.default_rng(12)
    lens = rng.integers(100, 3000, size=40)
    H = 8
    d = inputs.varlen_inputs(lens, H, 128, 128, io="bf16", seed=12, with_S0=True, device=DEV)
    inputs.strong_gate_channels(d, 8, -5.0, -2.0, seed=12)
    d["g"][1000:1100, :, 5] = -20.0
    ws = workspace_for(d)
    (oa, Sa), (ob, Sb) = both(d, ws)
    check_plan(ws, lens, H)
    assert torch.isfinite(oa.float()).all() and torch.isfinite(Sa).all()
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)


def test_balanced_without_states_and_with_transforms():
    """No S0 and no final state (the hand-over still goes through the
    workspace), and the in-kernel input transforms."""
    rng = np.random.default_rng(13)
    lens = rng.integers(0, 2000, size=44)
    H = 8
    d = inputs.varlen_inputs(lens, H, 128, 128, io="bf16", seed=13, with_S0=False, device=DEV)
    ws = workspace_for(d)
    (oa, _), (ob, _) = both(d, ws, output_final_state=False)
    check_plan(ws, lens, H)
    assert torch.equal(oa, ob)
    r = inputs.raw_layer_inputs(d, H, 128, seed=13, device=DEV)
    kw = dict(qk_l2norm=True, beta_sigmoid=True, A_log=r["A_log"], gate_bias=r["gate_bias"])
    ws.zero_()
    (oa, Sa), (ob, Sb) = both(r, ws, **kw)
    check_plan(ws, lens, H)
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)


def test_balanced_calls_in_a_row():
    """Two calls on one workspace, the second with fewer sequences: the plan
    kernel resets the hand-over flags each call."""
    H = 8
    K = kda()
    for n_seq, seed in ((60, 14), (36, 15)):
        rng = np.random.default_rng(seed)
        lens = rng.integers(0, 2500, size=n_seq)
        d = inputs.varlen_inputs(lens, H, 128, 128, io="bf16", seed=seed, with_S0=True,
                                 device=DEV)
        if n_seq == 60:
            ws = workspace_for(d)
        (oa, Sa), (ob, Sb) = both(d, ws)
        check_plan(ws, lens, H)
        assert torch.equal(oa, ob) and torch.equal(Sa, Sb), n_seq


# ------------------------------------------------------------------ batched layout

BATCHED = [
    # (name, B, T, H, dk, dv, io, gate, with_S0)
    ("kda 10 x 300 tokens", 10, 300, 32, 128, 128, "bf16", "kda", True),
    ("gated deltanet 5 x 200", 5, 200, 64, 128, 128, "bf16", "gdn", False),
    ("one token each", 300, 1, 1, 128, 128, "bf16", "kda", True),
    ("fp32 64x64", 90, 130, 4, 64, 64, "f32", "kda", True),
]


def batched_both(d, ws, **kw):
    K = kda()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    a = K.chunk_fwd(*args, S0=d["S0"], workspace=ws, **kw)
    b = K.chunk_fwd(*args, S0=d["S0"], balanced=False, **kw)
    torch.cuda.synchronize()
    return a, b


def batched_workspace(B, T, H, dk, dv, io):
    n = kda().chunk_fwd_workspace_size(B, T, H, dk, dv, io=io)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("case", BATCHED, ids=[c[0] for c in BATCHED])
def test_balanced_batched_equals_per_chain_kernel(case):
    name, B, T, H, dk, dv, io, gate, with_S0 = case
    note("balanced batched %s: B=%d T=%d H=%d" % (name, B, T, H))
    d = inputs.prefill_inputs(B, T, H, dk, dv, io=io, seed=B + T, with_S0=with_S0, device=DEV,
                              gate=gate)
    ws = batched_workspace(B, T, H, dk, dv, io)
    (oa, Sa), (ob, Sb) = batched_both(d, ws)
    M, Ts = check_plan(ws, [T] * B, H)
    note("  %d machines, slices of %d chunks, %d sequences split"
         % (M, Ts, len(split_sequences([T] * B, Ts))))
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)


def test_balanced_batched_transforms_and_oracle():
    """The input transforms through the balanced batched schedule, and the split
    sequences against the oracle."""
    from parity_util import gpu_chains_batched, oracle_batched
    B, T, H = 10, 200, 32
    d = inputs.prefill_inputs(B, T, H, 128, 128, io="bf16", seed=77, with_S0=True, device=DEV)
    ws = batched_workspace(B, T, H, 128, 128, "bf16")
    (oa, Sa), (ob, Sb) = batched_both(d, ws)
    M, Ts = check_plan(ws, [T] * B, H)
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)
    split = split_sequences([T] * B, Ts)
    assert split, "no sequence was split"
    chains = [(b, h) for b in split for h in (b % H, (b + 7) % H)]
    ro, rs = oracle_batched(d, chains)
    go, gs = gpu_chains_batched(oa, Sa, chains)
    assert_close(go, gs, ro, rs, tol_for("bf16"), "balanced batched split chains")
    r = inputs.raw_layer_inputs(d, H, 128, seed=77, device=DEV)
    kw = dict(qk_l2norm=True, beta_sigmoid=True, A_log=r["A_log"], gate_bias=r["gate_bias"])
    (oa, Sa), (ob, Sb) = batched_both(r, ws, **kw)
    check_plan(ws, [T] * B, H)
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)


def test_balanced_without_hand_over(monkeypatch):
    """With no polls allowed (KDA_SPLIT_SPIN_POLLS=0) every workgroup that
    would wait for a handed-over state recomputes the sequence from its start
    instead: the bounded wait's other branch, same bits."""
    monkeypatch.setenv("KDA_SPLIT_SPIN_POLLS", "0")
    rng = np.random.default_rng(16)
    lens = rng.integers(0, 3000, size=40)
    H = 8
    d = inputs.varlen_inputs(lens, H, 128, 128, io="bf16", seed=16, with_S0=True, device=DEV)
    ws = workspace_for(d)
    (oa, Sa), (ob, Sb) = both(d, ws)
    M, T = check_plan(ws, lens, H)
    assert split_sequences(lens, T), "no sequence was split"
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)
    B, Tb = 10, 300
    db = inputs.prefill_inputs(B, Tb, 32, 128, 128, io="bf16", seed=16, with_S0=True, device=DEV)
    wb = batched_workspace(B, Tb, 32, 128, 128, "bf16")
    (oa, Sa), (ob, Sb) = batched_both(db, wb)
    check_plan(wb, [Tb] * B, 32)
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)


def test_balanced_random_mixes():
    """Twelve seeded length mixes and head counts (1 to 32 heads; empty, short,
    ragged and long sequences; with and without S0), each with 1 to 4 chains
    per resident workgroup: every output and final state equal to one
    workgroup per chain's."""
    rng = np.random.default_rng(2024)
    done = 0
    while done < 12:
        H = int(rng.choice([1, 2, 4, 8, 16, 32]))
        kind = done % 4
        n_lo, n_hi = -(-260 // H), 1024 // H
        n_seq = int(rng.integers(n_lo, n_hi + 1))
        if kind == 0:
            lens = rng.integers(0, 400, size=n_seq)
        elif kind == 1:
            lens = rng.integers(1, 65, size=n_seq)
        elif kind == 2:
            lens = np.where(rng.random(n_seq) < 0.1, rng.integers(2000, 6000, size=n_seq),
                            rng.integers(0, 200, size=n_seq))
        else:
            lens = rng.integers(500, 1500, size=n_seq)
        if int(lens.sum()) * H > 4_000_000:
            continue
        with_S0 = bool(rng.integers(0, 2))
        note("random mix %d: H=%d, %d sequences, %d tokens, S0=%s"
             % (done, H, n_seq, int(lens.sum()), with_S0))
        d = inputs.varlen_inputs(lens, H, 128, 128, io="bf16", seed=100 + done, with_S0=with_S0,
                                 device=DEV)
        ws = workspace_for(d)
        (oa, Sa), (ob, Sb) = both(d, ws)
        check_plan(ws, lens, H)
        assert torch.equal(oa, ob) and torch.equal(Sa, Sb), done
        done += 1
