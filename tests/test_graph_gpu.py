"""The calls under HIP graph capture: each call enqueues kernels only (no
memset, no allocation in the library), so a captured sequence of calls
replays to exactly the eager result.  Every replay is checked against the
eager run from the same starting state, with eager work and synchronisation
between the replays."""
import pytest
import torch

from gated_delta_rule_06_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def kda():
    from gated_delta_rule_06_amd import kda as k
    return k


def test_decode_steps_replay_like_eager():
    K = kda()
    steps = 4
    d = inputs.decode_inputs(16, 4, 128, 128, steps, io="bf16", seed=41, device=DEV)
    S0 = d["S"].clone()
    S = d["S"]
    out = torch.empty((16, 4, 128), dtype=torch.bfloat16, device=DEV)

    def run():
        for t in range(steps):
            K.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], S, out=out)

    run()   # warm-up, eager
    torch.cuda.synchronize()
    S.copy_(S0)
    run()
    torch.cuda.synchronize()
    S_ref, o_ref = S.clone(), out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    other = inputs.decode_inputs(8, 2, 64, 64, 1, io="f32", seed=42, device=DEV)
    for rep in range(3):
        S.copy_(S0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(S, S_ref) and torch.equal(out, o_ref), rep
        # eager work between the replays
        K.decode_step(other["q"][0], other["k"][0], other["v"][0], other["g"][0],
                      other["beta"][0], other["S"])
        torch.cuda.synchronize()


@pytest.mark.parametrize("B,T,H", [(1, 1000, 4), (2, 300, 3)])
def test_prefill_replays_like_eager(B, T, H):
    """Both prefill schedules: the chunk-parallel one (few long chains, with
    its workspace) and the one-workgroup-per-chain kernel."""
    K = kda()
    d = inputs.prefill_inputs(B, T, H, 128, 128, io="bf16", seed=B * T, with_S0=True, device=DEV)
    out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device=DEV)
    Sf = torch.empty((B, H, 128, 128), dtype=torch.float32, device=DEV)
    n = K.chunk_fwd_workspace_size(B, T, H, 128, 128)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)

    def run():
        K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"], out=out, S_final=Sf,
                    workspace=ws if n else None)

    run()
    torch.cuda.synchronize()
    o_ref, S_ref = out.clone(), Sf.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        out.zero_()
        Sf.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(Sf, S_ref), rep
        run()   # eager work between the replays
        torch.cuda.synchronize()


def test_balanced_packed_prefill_replays_like_eager():
    """The balanced schedule of a packed call (a plan kernel that clears the
    hand-over flags, then the split kernel) under capture, replayed with eager
    calls on the same workspace in between."""
    import numpy as np
    K = kda()
    H = 8
    lens = np.random.default_rng(43).integers(0, 2000, size=40)
    d = inputs.varlen_inputs(lens, H, 128, 128, io="bf16", seed=43, with_S0=True, device=DEV)
    out = torch.empty_like(d["v"])
    Sf = torch.empty((40, H, 128, 128), dtype=torch.float32, device=DEV)
    n = K.lib.kda_chunk_fwd_varlen_workspace_size(40, int(lens.sum()), H, 128, 128, 64, 1)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)

    def run():
        K.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                           S0=d["S0"], out=out, S_final=Sf, workspace=ws)

    run()
    torch.cuda.synchronize()
    o_ref, S_ref = out.clone(), Sf.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        out.zero_()
        Sf.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(Sf, S_ref), rep
        run()   # eager work between the replays
        torch.cuda.synchronize()
