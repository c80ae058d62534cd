"""Pins of the oracle's backward (oracle/backward.py) against central finite
differences of the oracle's forward loop (oracle/kda_ref.c, a separate
implementation), plus one closed form.

The loss is L = sum(W_o * o) + sum(W_S * S_final) for fixed random weights, so
dL/do = W_o and dL/dS_final = W_S.  Every input element (q, k, v, g, beta, S0)
is perturbed by +-h in its own storage precision; the actual step (after fp32
rounding) divides the fp64 difference of L.  A dropped term in any of the chain
rule's lines (the read-after-write dS, either half of dk, dbeta, the decay in
dS or in dg) moves some gradient by O(1) and fails.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as obwd


def _inputs(rng, lens, H, dk, dv, scalar_gate, packed):
    T = sum(lens) if packed else lens[0]
    lead = (T,) if packed else (len(lens), T)
    q = rng.standard_normal(lead + (H, dk)).astype(np.float32) * 0.6
    k = rng.standard_normal(lead + (H, dk)).astype(np.float32) * 0.6
    v = rng.standard_normal(lead + (H, dv)).astype(np.float32)
    gshape = lead + ((H,) if scalar_gate else (H, dk))
    g = (-np.exp(rng.standard_normal(gshape) - 1.5)).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal(lead + (H,))))).astype(np.float32)
    S0 = rng.standard_normal((len(lens), H, dk, dv)) * 0.5
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32) if packed else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, cu=cu)


def _loss(d, Wo, WS, scale):
    o, Sf = oracle.forward_dense(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"],
                                 scale=scale, cu_seqlens=d["cu"], threads=1)
    return float(np.sum(Wo * o) + np.sum(WS * Sf))


def _fd(d, name, idx, Wo, WS, scale):
    x = d[name]
    keep = x[idx]
    h = 1e-3 if x.dtype == np.float32 else 1e-5
    xp = x.dtype.type(keep + h)
    xm = x.dtype.type(keep - h)
    x[idx] = xp
    lp = _loss(d, Wo, WS, scale)
    x[idx] = xm
    lm = _loss(d, Wo, WS, scale)
    x[idx] = keep
    return (lp - lm) / (float(xp) - float(xm))


@pytest.mark.parametrize("lens,packed,scalar_gate", [
    ([4, 4], False, False),
    ([3, 0, 4], True, False),
    ([5], False, True),
])
def test_backward_matches_finite_differences(lens, packed, scalar_gate):
    rng = np.random.default_rng(7 + len(lens))
    H, dk, dv, scale = 2, 4, 3, 0.7
    d = _inputs(rng, lens, H, dk, dv, scalar_gate, packed)
    Wo = rng.standard_normal(d["v"].shape)
    WS = rng.standard_normal(d["S0"].shape)
    grads = obwd.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], Wo, S0=d["S0"],
                          dS_final=WS, scale=scale, cu_seqlens=d["cu"])
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    worst = 0.0
    for name, gname in names.items():
        an = grads[gname]
        assert an.shape == d[name].shape, (gname, an.shape, d[name].shape)
        for idx in np.ndindex(*d[name].shape):
            fd = _fd(d, name, idx, Wo, WS, scale)
            err = abs(fd - an[idx]) / (1.0 + abs(an[idx]))
            worst = max(worst, err)
            assert err < 1e-5, (gname, idx, fd, an[idx])
    print("worst scaled FD error %.2e" % worst)


def test_backward_without_writes_is_a_fixed_state_readout():
    """beta = 0 and g = 0: S_t = S0 for every t and o_t = scale S0^T q_t, so
    dq_t = scale S0 do_t, dS0 = dS_final + scale sum_t q_t do_t^T, dk = dv = 0,
    dbeta_t = (S0^T k_t) . ... = de . (v_t - S0^T k_t) with de = dS_t^T k_t, and
    dg_t = rowsum(S0 * dS_t) where dS_t collects the later readouts."""
    rng = np.random.default_rng(3)
    T, dk, dv, s = 5, 3, 2, 0.5
    q = rng.standard_normal((1, T, 1, dk)).astype(np.float32)
    k = rng.standard_normal((1, T, 1, dk)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, dv)).astype(np.float32)
    g = np.zeros((1, T, 1, dk), np.float32)
    beta = np.zeros((1, T, 1), np.float32)
    S0 = rng.standard_normal((1, 1, dk, dv))
    do = rng.standard_normal((1, T, 1, dv))
    dSf = rng.standard_normal((1, 1, dk, dv))
    r = obwd.backward(q, k, v, g, beta, do, S0=S0, dS_final=dSf, scale=s)
    S = S0[0, 0]
    qs, ks, vs, dos = q[0, :, 0].astype(np.float64), k[0, :, 0].astype(np.float64), \
        v[0, :, 0].astype(np.float64), do[0, :, 0]
    np.testing.assert_allclose(r["dq"][0, :, 0], s * dos @ S.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dS0"][0, 0], dSf[0, 0] + s * qs.T @ dos, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-12)
    np.testing.assert_allclose(r["dv"], 0.0, atol=1e-12)
    for t in range(T):
        dSt = dSf[0, 0] + s * sum(np.outer(qs[u], dos[u]) for u in range(t, T))
        np.testing.assert_allclose(r["dg"][0, t, 0], np.sum(S * dSt, axis=1), rtol=1e-12,
                                   atol=1e-12)
        de = dSt.T @ ks[t]
        np.testing.assert_allclose(r["dbeta"][0, t, 0], de @ (vs[t] - S.T @ ks[t]), rtol=1e-12,
                                   atol=1e-12)
