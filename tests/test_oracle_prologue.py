"""Pins of the oracle's input prologue (L2-normalised q and k, beta =
sigmoid(b), g = -c softplus(x), the preparation the workloads apply before the
recurrence) against facts that do not come from the oracle's own formulas:

- outputs: unit rows pointing along the input, a zero row stays zero; beta and
  g against scipy's expit and numpy's logaddexp (softplus(x) = log(e^0 + e^x)),
  sigmoid(0) = 1/2 and softplus(0) = log 2 exactly;
- gradients: central differences of a random linear functional of every
  output, and the normalisation's gradient is orthogonal to its input row
  (scaling a row does not change its direction).
"""
import numpy as np
import pytest
from scipy.special import expit


def rand(rng, shape_tok=(2, 5, 3), Dk=6):
    q = rng.standard_normal(shape_tok + (Dk,)) * rng.uniform(0.2, 3.0, shape_tok + (1,))
    k = rng.standard_normal(shape_tok + (Dk,)) * rng.uniform(0.2, 3.0, shape_tok + (1,))
    b = rng.standard_normal(shape_tok) * 3
    x = rng.standard_normal(shape_tok) * 4
    return q, k, b, x


def test_prologue_outputs(oracle_lib):
    rng = np.random.default_rng(71)
    q, k, b, x = rand(rng)
    q[0, 1, 2] = 0.0
    qn, kn, beta, g = oracle_lib.prologue(q, k, b, x, gate_scale=0.1)
    nq = np.linalg.norm(qn, axis=-1)
    assert np.all(qn[0, 1, 2] == 0.0)
    nq[0, 1, 2] = 1.0
    assert np.abs(nq - 1).max() < 1e-14 and np.abs(np.linalg.norm(kn, axis=-1) - 1).max() < 1e-14
    cos = np.sum(kn * k, -1) / np.linalg.norm(k, axis=-1)
    assert np.abs(cos - 1).max() < 1e-14
    assert np.abs(beta - expit(b)).max() < 1e-15
    assert np.abs(g - (-0.1) * np.logaddexp(0.0, x)).max() < 1e-15
    _, _, b0, g0 = oracle_lib.prologue(q[:1, :1, :1], k[:1, :1, :1], np.zeros((1, 1, 1)), np.zeros((1, 1, 1)), 1.0)
    assert b0[0, 0, 0] == 0.5 and g0[0, 0, 0] == -np.log(2.0)
    _, _, _, gn = oracle_lib.prologue(q, k, b, None)
    assert gn is None


@pytest.mark.parametrize("c", [0.1, 1.0])
def test_prologue_gradients(oracle_lib, c):
    rng = np.random.default_rng(72)
    q, k, b, x = rand(rng, (1, 3, 2), 4)
    wq, wk = rng.standard_normal(q.shape), rng.standard_normal(k.shape)
    wb, wg = rng.standard_normal(b.shape), rng.standard_normal(x.shape)

    def f(q_, k_, b_, x_):
        a, bb, cc, dd = oracle_lib.prologue(q_, k_, b_, x_, c)
        return float(np.sum(a * wq) + np.sum(bb * wk) + np.sum(cc * wb) + np.sum(dd * wg))
    dq, dk, db, dx = oracle_lib.prologue_bwd(q, k, b, x, c, wq, wk, wb, wg)
    h = 1e-6
    args = [q, k, b, x]
    for i, grad in enumerate((dq, dk, db, dx)):
        fd = np.zeros_like(args[i])
        it = np.nditer(args[i], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[i][idx] += h
            am[i][idx] -= h
            fd[idx] = (f(*ap) - f(*am)) / (2 * h)
        assert np.abs(grad - fd).max() < 1e-8 * max(1.0, np.abs(fd).max()), i
    # scale invariance of the normalisation: the gradient is orthogonal to the row
    assert np.abs(np.sum(dq * q, -1)).max() < 1e-12
    # a zero row has a zero gradient
    q[0, 0, 0] = 0.0
    dq0, _, _, _ = oracle_lib.prologue_bwd(q, k, b, x, c, wq, wk, wb, wg)
    assert np.all(dq0[0, 0, 0] == 0.0)
