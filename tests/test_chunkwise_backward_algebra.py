"""The chunkwise backward's algebra, written out in fp64 numpy and checked
against the oracle's backward (oracle/backward.py, pinned by finite
differences of the forward loop).

This is the decomposition the bf16 MFMA backward computes ("Kimi Unveils Delta
Attention and K3 Architecture Updates", section 6: chunk-local decay, the WY
factors W and U from the unit-lower-triangular inverse, the state update and
the outputs per chunk), taken in reverse mode chunk by chunk: 32-token chunks,
every per-token factor referenced to the chunk's middle token (r = b_15), the
state decay split as Diag(e^r) before the chunk's products and Diag(e^{b_L-r})
after them, and dlog alpha formed as suffix sums of per-token terms plus the
K_end terms as a sum over earlier tokens plus the incoming state's decay.  A
mistake in any of those steps (a wrong reference, a missing term of dS, dk or
dbeta, a wrong sign in the pair terms of dlog alpha) moves some gradient far
beyond the fp64 rounding these tests allow.  Runs on the CPU only."""
import numpy as np
import pytest

from oracle import backward as obwd

C = 32


def chunkwise_backward(q, k, v, g, beta, do, S0, dSf, scale):
    """One chain, key-by-value state: q, k, g [T, dk], v, do [T, dv], beta [T]."""
    T, D = q.shape
    nc = (T + C - 1) // C
    pad = nc * C - T

    def padded(x):
        return np.concatenate([x, np.zeros((pad,) + x.shape[1:])]) if pad else x

    q, k, v, g, do, beta = map(padded, (q, k, v, g, do, beta))

    def chunk(m):
        sl = slice(m * C, (m + 1) * C)
        b = np.cumsum(g[sl], axis=0)
        r, bl = b[15], b[C - 1]
        P = np.exp(b - r)
        QG, KG, KI = scale * q[sl] * P, k[sl] * P, k[sl] / P
        A = np.tril(KG @ KI.T, -1)
        Aqk = np.tril(QG @ KI.T)
        Tm = np.linalg.inv(np.eye(C) + beta[sl, None] * A)
        W = Tm @ (beta[sl, None] * KG)
        U = Tm @ (beta[sl, None] * v[sl])
        return sl, r, bl, P, QG, KG, KI, A, Aqk, Tm, W, U

    S = S0.copy()
    states = []
    for m in range(nc):
        states.append(S.copy())
        sl, r, bl, P, QG, KG, KI, A, Aqk, Tm, W, U = chunk(m)
        Sm = np.exp(r)[:, None] * S
        E = U - W @ Sm
        S = np.exp(bl - r)[:, None] * (Sm + KI.T @ E)
    dq, dk, dv, dg = (np.zeros_like(x) for x in (q, k, v, g))
    dbeta = np.zeros(len(beta))
    dS = dSf.copy()
    for m in reversed(range(nc)):
        sl, r, bl, P, QG, KG, KI, A, Aqk, Tm, W, U = chunk(m)
        Sm = np.exp(r)[:, None] * states[m]
        E = U - W @ Sm
        dSm = np.exp(bl - r)[:, None] * dS
        dO = do[sl]
        dE = KI @ dSm + Aqk.T @ dO
        dAqk = np.tril(dO @ E.T)
        dW = -dE @ Sm.T
        dYv, dYk = Tm.T @ dE, Tm.T @ dW
        dL = np.tril(-(dYv @ U.T + dYk @ W.T), -1)
        dA = beta[sl, None] * dL
        dv[sl] = beta[sl, None] * dYv
        dbeta[sl] = (dL * A).sum(1) + (dYv * v[sl]).sum(1) + (dYk * KG).sum(1)
        dQG = dO @ Sm.T + dAqk @ KI
        dKG = beta[sl, None] * dYk + dA @ KI
        dKI = dA.T @ KG + dAqk.T @ QG
        dKIe = E @ dSm.T
        dq[sl] = scale * P * dQG
        dk[sl] = P * dKG + (dKI + dKIe) / P
        db = QG * dQG + KG * dKG - KI * dKI
        ke = KI * dKIe
        suffix = np.cumsum(db[::-1], axis=0)[::-1]
        before = np.concatenate([np.zeros((1, D)), np.cumsum(ke, axis=0)[:-1]])
        dg[sl] = suffix + before + (dSm * Sm).sum(1)
        dS = np.exp(r)[:, None] * (dSm + QG.T @ dO - W.T @ dE)
    return dict(dq=dq[:T], dk=dk[:T], dv=dv[:T], dg=dg[:T], dbeta=dbeta[:T], dS0=dS)


def _case(T, D, gate, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, D))
    k = rng.standard_normal((T, D))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, D))
    if gate == "mild":
        g = -rng.uniform(0.01, 0.5, (T, D))
    else:   # near the edge of the chunkwise factors' range: each half chunk decays by ~e^-70
        g = -4.4 + 0.3 * (rng.uniform(0, 1, (T, D)) - 0.5)
    beta = rng.uniform(0, 1, T)
    do = rng.standard_normal((T, D))
    S0 = rng.standard_normal((D, D)) * 0.1
    dSf = rng.standard_normal((D, D))
    return q, k, v, g, beta, do, S0, dSf, D ** -0.5


@pytest.mark.parametrize("T,gate", [(1, "mild"), (20, "mild"), (32, "mild"), (77, "mild"),
                                    (130, "mild"), (45, "strong"), (96, "strong")])
def test_chunkwise_backward_algebra_matches_oracle(T, gate):
    q, k, v, g, beta, do, S0, dSf, s = _case(T, 16, gate, seed=T)
    got = chunkwise_backward(q, k, v, g, beta, do, S0, dSf, s)
    one = lambda x: x[None, :, None]
    ref = obwd.backward(one(q), one(k), one(v), one(g), one(beta), one(do), S0=S0[None, None],
                        dS_final=dSf[None, None], scale=s)
    for name, oname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"),
                        ("dbeta", "dbeta"), ("dS0", "dS0")):
        x = got[name]
        y = np.asarray(ref[oname], dtype=np.float64).reshape(x.shape)
        err = np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)
        assert err < 1e-12, (T, gate, name, err)
