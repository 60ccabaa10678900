"""Pins of the gradient oracle (oracle/scan_grad.py) against the C oracle's forward.

The gradient oracle restates the scan in torch and lets autograd differentiate it.  Two
things pin it to something other than itself:
  * its forward must equal the C oracle's (titans_oracle.c, written separately, plain C)
    to rounding, for every depth, a ragged last chunk and each attentional bias;
  * its cotangents must match central finite differences of the C oracle's forward:
    for output cotangents (dy, dtheta_T, ds_T) the scalar f = <dy, y> + <dtheta_T, theta_T>
    + <ds_T, s_T>; for a random direction u of one input x, <df/dx, u> must equal
    (f(x + h u) - f(x - h u)) / 2h.  One check per input isolates a wrong cotangent of
    any one of them (a dropped second-derivative term shows in k, v and theta0, a wrong
    coefficient derivative in the gates).
"""
import numpy as np
import pytest

import oracle
from oracle import scan_grad


def _case(widths, B=1, H=2, T=13, seed=0, scale_s0=0.1):
    rng = np.random.default_rng(seed)
    d = widths[0]
    P = oracle.param_count(widths)

    def unit(shape):
        x = rng.standard_normal(shape)
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    th0 = np.concatenate([rng.standard_normal((B, H, widths[l] * widths[l - 1]))
                          / np.sqrt(widths[l - 1]) for l in range(1, len(widths))], axis=-1)
    inp = {
        "q": unit((B, T, H, d)), "k": unit((B, T, H, d)), "v": rng.standard_normal((B, T, H, d)),
        "alpha": sig(rng.normal(-2.0, 1.0, (B, T, H))),
        "eta": 0.5 * sig(rng.normal(0.0, 1.0, (B, T, H))),
        "beta": sig(rng.normal(1.0, 1.0, (B, T, H))),
        "theta0": th0, "s0": scale_s0 * rng.standard_normal((B, H, P)),
    }
    cot = (rng.standard_normal((B, T, H, d)), rng.standard_normal((B, H, P)),
           rng.standard_normal((B, H, P)))
    return inp, cot


def _f(inp, chunk, widths, cot, bias):
    y, th, s = oracle.scan(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"], inp["beta"],
                           inp["theta0"], inp["s0"], chunk, widths, bias=bias)
    return float(np.sum(y * cot[0]) + np.sum(th * cot[1]) + np.sum(s * cot[2]))


CASES = [
    ((4, 4), 4, None),             # linear memory
    ((4, 6, 4), 5, None),          # one hidden layer, ragged last chunk (T = 13)
    ((3, 5, 4, 3), 4, None),       # two hidden layers
    ((4, 6, 4), 13, None),         # one chunk
    ((4, 6, 4), 1, None),          # fully sequential
    ((4, 6, 4), 5, ("huber", 0.3)),
    ((4, 6, 4), 5, ("lp", 3.0)),
]


@pytest.mark.parametrize("widths,chunk,bias", CASES)
def test_forward_equals_c_oracle(widths, chunk, bias):
    import torch

    inp, _ = _case(widths)
    ref = oracle.scan(*(inp[n] for n in scan_grad.NAMES), chunk, widths, bias=bias)
    with torch.no_grad():
        out = scan_grad.scan(*(torch.tensor(inp[n]) for n in scan_grad.NAMES), chunk, widths,
                             bias)
    for a, b in zip(out, ref):
        np.testing.assert_allclose(a.numpy(), b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("widths,chunk,bias", CASES)
def test_cotangents_match_finite_differences(widths, chunk, bias):
    inp, cot = _case(widths, seed=1)
    grads = scan_grad.scan_vjp(inp, chunk, widths, *cot, bias=bias)
    rng = np.random.default_rng(7)
    h = 1e-5
    for name in scan_grad.NAMES:
        u = rng.standard_normal(inp[name].shape)
        plus = dict(inp, **{name: inp[name] + h * u})
        minus = dict(inp, **{name: inp[name] - h * u})
        fd = (_f(plus, chunk, widths, cot, bias) - _f(minus, chunk, widths, cot, bias)) / (2 * h)
        an = float(np.sum(grads[name] * u))
        assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (name, an, fd)


def test_cotangents_vanish_without_outputs_and_zero_length():
    """With zero output cotangents every input cotangent is zero; with T = 0 the state
    cotangents pass straight through (theta_T = theta0, s_T = s0)."""
    widths = (4, 6, 4)
    inp, cot = _case(widths, T=5)
    zero = tuple(np.zeros_like(c) for c in cot)
    g = scan_grad.scan_vjp(inp, 3, widths, *zero)
    for name in scan_grad.NAMES:
        assert not np.any(g[name])
    inp0, cot0 = _case(widths, T=0)
    g0 = scan_grad.scan_vjp(inp0, 3, widths, *cot0)
    np.testing.assert_array_equal(g0["theta0"], cot0[1])
    np.testing.assert_array_equal(g0["s0"], cot0[2])


def test_single_token_closed_form():
    """T = 1, linear memory (y = W q read before the write): the state cotangents have a
    closed form.  theta_1 = (1 - alpha) W - eta s_1, s_1 = beta s_0 + (1 - beta) g with
    g = 2 (W k - v) k^T, so with dy = 0 and ds_T = 0:
      d s_0     = -eta beta dtheta,
      d v       = 2 eta (1 - beta) dtheta k,
      d alpha   = -<dtheta, W>,   d eta = -<dtheta, s_1>,   d beta = eta <dtheta, g - s_0>."""
    widths = (3, 3)
    inp, cot = _case(widths, B=1, H=1, T=1, seed=3)
    dth = cot[1]
    g = scan_grad.scan_vjp(inp, 1, widths, np.zeros_like(cot[0]), dth, np.zeros_like(cot[2]))
    W = inp["theta0"][0, 0].reshape(3, 3)
    s0 = inp["s0"][0, 0].reshape(3, 3)
    k, v = inp["k"][0, 0, 0], inp["v"][0, 0, 0]
    al, et, be = inp["alpha"][0, 0, 0], inp["eta"][0, 0, 0], inp["beta"][0, 0, 0]
    D = dth[0, 0].reshape(3, 3)
    grad = 2.0 * np.outer(W @ k - v, k)
    s1 = be * s0 + (1 - be) * grad
    np.testing.assert_allclose(g["s0"][0, 0], (-et * be * D).reshape(-1), rtol=1e-12)
    np.testing.assert_allclose(g["v"][0, 0, 0], 2 * et * (1 - be) * D @ k, rtol=1e-12)
    np.testing.assert_allclose(g["alpha"][0, 0, 0], -np.sum(D * W), rtol=1e-12)
    np.testing.assert_allclose(g["eta"][0, 0, 0], -np.sum(D * s1), rtol=1e-12)
    np.testing.assert_allclose(g["beta"][0, 0, 0], et * np.sum(D * (grad - s0)), rtol=1e-12)
