"""kda_backward_noalloc (the backward with the library's static scratch as
its workspace, for callers that cannot allocate) against kda_backward (the
same kernels with a caller workspace), through the C ABI: two calls in a row,
the second smaller, each bit-identical to the allocating call and within the
backward's bar (rel-L2 <= 1e-4) of it; a problem beyond the scratch size is
rejected before any work."""
import numpy as np
import pytest
import torch

from gated_delta_rule_06_amd import inputs
from parity_util import rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


def kda():
    from gated_delta_rule_06_amd import kda as k
    return k


def _outs(d, gate):
    lead = tuple(d["q"].shape[:-2])
    H, dk, dv = d["H"], d["dk"], d["dv"]
    n = d["B"] if d.get("cu_seqlens") is None else d["N"]
    f = dict(dtype=torch.float32, device=DEV)
    g = lead + (H,) if gate == "gdn" else lead + (H, dk)
    # filled with NaN so that any element the call fails to write shows up
    return {"dq": torch.full(lead + (H, dk), float("nan"), **f),
            "dk": torch.full(lead + (H, dk), float("nan"), **f),
            "dv": torch.full(lead + (H, dv), float("nan"), **f),
            "dlog_alpha": torch.full(g, float("nan"), **f),
            "dbeta": torch.full(lead + (H,), float("nan"), **f),
            "dS0": torch.full((n, H, dk, dv), float("nan"), **f)}


def _case(d, gate, what):
    K = kda()
    ref = K.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_out"], S0=d["S0"],
                     dS_final=d["dS_final"], cu_seqlens=d.get("cu_seqlens"))
    got = K.backward_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_out"],
                             _outs(d, gate), S0=d["S0"], dS_final=d["dS_final"],
                             cu_seqlens=d.get("cu_seqlens"))
    torch.cuda.synchronize()
    for n in NAMES:
        a, b = got[n].cpu().numpy(), ref[n].cpu().numpy()
        assert np.isfinite(a).all(), (what, n)
        e = rel_l2(a, b)
        print("%s %s rel-L2 vs kda_backward %.1e" % (what, n, e), flush=True)
        assert e <= 1e-4, (what, n, e)
        assert np.array_equal(a, b), (what, n)


def test_noalloc_backward_matches_allocating_call_twice():
    """Two calls in a row on the same scratch, the second with a smaller input
    (the scratch keeps the first call's contents)."""
    K = kda()
    big = inputs.prefill_inputs(2, 700, 4, 128, 128, io="bf16", seed=71, with_S0=True, device=DEV)
    inputs.grad_inputs(big, seed=71, device=DEV)
    need = K.backward_workspace_size(2, 700, 4, 128, 128)
    assert need <= K.noalloc_scratch_bytes()
    _case(big, "kda", "no-alloc first call (B2 T700 H4 d128 bf16)")
    small = inputs.varlen_inputs([9, 0, 33], 2, 64, 64, io="f32", seed=72, with_S0=True,
                                 device=DEV, gate="gdn")
    inputs.grad_inputs(small, seed=72, device=DEV)
    _case(small, "gdn", "no-alloc second call (packed 9/0/33 H2 d64 fp32 gdn)")


def test_noalloc_backward_rejects_problems_beyond_the_scratch():
    K = kda()
    T = 4096
    assert K.backward_workspace_size(1, T, 8, 128, 128) > K.noalloc_scratch_bytes()
    d = inputs.prefill_inputs(1, T, 8, 128, 128, io="bf16", seed=73, device=DEV)
    inputs.grad_inputs(d, seed=73, device=DEV)
    out = _outs(d, "kda")
    with pytest.raises(K.KdaError) as err:
        K.backward_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_out"], out)
    assert err.value.status == -8
    torch.cuda.synchronize()
    assert torch.isnan(out["dq"]).all()   # nothing was enqueued
