"""The identity behind the inference forward's W_up fold (large batches),
checked in float64 on random weights whose LayerNorm input sits far from
zero mean: with Wc = W_up minus its column means over the d outputs,
  var(u) = a^T (Wc^T Wc) a / d  and
  W_a LayerNorm(u) = rstd * (W_a diag(gamma) Wc) a + W_a beta,
u = W_up a, LayerNorm over the d features with biased variance (the
LayerNorm of the layer formula, y = W_mix [LayerNorm(W_up a) ; x])."""
import numpy as np


def test_w_up_fold_identity():
    rng = np.random.default_rng(7)
    d, de, n, eps = 96, 32, 6, 1e-5
    # a common column shift puts u's mean tens of times above its spread
    W_up = (rng.standard_normal((d, de)) / np.sqrt(de)
            + 8.0 * rng.standard_normal(de))
    W_a = rng.standard_normal((d, d)) / np.sqrt(d)
    gamma = 1.0 + 0.1 * rng.standard_normal(d)
    beta = 0.1 * rng.standard_normal(d)
    a = rng.standard_normal((n, de))

    u = a @ W_up.T
    mu = u.mean(axis=1, keepdims=True)
    var = ((u - mu) ** 2).mean(axis=1)
    assert np.median(np.abs(mu[:, 0]) / np.sqrt(var)) > 10
    h = gamma * (u - mu) / np.sqrt(var[:, None] + eps) + beta
    y_ref = h @ W_a.T

    Wc = W_up - W_up.mean(axis=0, keepdims=True)
    G = Wc.T @ Wc                     # d_e x d_e
    Mc = (W_a * gamma) @ Wc           # d x d_e
    var_f = np.einsum("ik,kl,il->i", a, G, a) / d
    y_f = (a @ Mc.T) / np.sqrt(var_f[:, None] + eps) + W_a @ beta
    np.testing.assert_allclose(var_f, var, rtol=1e-10)
    np.testing.assert_allclose(y_f, y_ref, rtol=1e-9, atol=1e-11)
