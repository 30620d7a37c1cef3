"""Fit of the rational tanh used by the tanh form of the gate's logistic
function (kda_chunk_mfma.hip, the sigmoid="tanh" option).

tanh(y) ~ y P(y^2) / Q(y^2) on 0 < y <= 9 with P and Q of degree 4 in y^2 and
P(0) = Q(0) = 1 (tanh is odd and tanh(y) / y -> 1).  The coefficients come
from least squares on the linearised relative error t Q - y P = 0, with the
weights of the worst points raised over 40 rounds (a cheap approach to the
minimax fit).  Prints the coefficients as fp32 values and the maximum error of
the fp32 evaluation in the kernel's order (clamp to +-9, Horner, y P / Q).

Usage: python -m gated_delta_rule_36_amd.fit_tanh
"""
import numpy as np

CLAMP = 9.0
DEG = 5  # coefficients of P and of Q (degree 4 in y^2)


def fit():
    y = np.linspace(1e-4, CLAMP, 20001)
    t = np.tanh(y)
    u = y * y
    w = np.ones_like(y)
    for _ in range(40):
        a = np.concatenate([-(y[:, None] * u[:, None] ** np.arange(DEG)),
                            t[:, None] * u[:, None] ** np.arange(1, DEG)], axis=1)
        sol, *_ = np.linalg.lstsq(a * (w / t)[:, None], -t * (w / t), rcond=None)
        p, q = sol[:DEG], np.concatenate([[1.0], sol[DEG:]])
        rel = np.abs(y * np.polyval(p[::-1], u) / np.polyval(q[::-1], u) - t) / t
        w = w * (1 + 2 * rel / rel.max())
    return p.astype(np.float32), q.astype(np.float32)


def tanh32(y, p, q):
    """fp32 evaluation in the kernel's order."""
    y = np.clip(np.asarray(y, np.float32), -CLAMP, CLAMP).astype(np.float32)
    u = (y * y).astype(np.float32)
    pn = np.full_like(u, p[-1])
    qd = np.full_like(u, q[-1])
    for k in range(DEG - 2, -1, -1):
        pn = (pn * u + p[k]).astype(np.float32)
        qd = (qd * u + q[k]).astype(np.float32)
    return (y * pn).astype(np.float32) * (np.float32(1) / qd).astype(np.float32)


if __name__ == "__main__":
    p, q = fit()
    print("P:", [float(v) for v in p])
    print("Q:", [float(v) for v in q])
    ys = np.linspace(-20, 20, 400001)
    print("max |tanh32 - tanh| on [-20, 20]:", float(np.abs(tanh32(ys, p, q) - np.tanh(ys)).max()))
