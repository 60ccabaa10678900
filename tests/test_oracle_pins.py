"""Pins for the fp64 oracle, each against something other than the oracle itself.

The Titans pages print no worked numeric example, so the oracle is pinned by
what the mathematics fixes: central finite differences and a library autograd
for the gradient, a library MLP for the forward, the closed-form delta rule
(the explainer relates the update to DeltaNet's), exact recall with
orthonormal keys, the eta = 0 and alpha = 1 special cases, a scalar closed form
with momentum and decay, the other letters used by the summary page, and the
streaming / permutation / broadcast invariants.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import chunk_form



@pytest.fixture(autouse=True, scope="module")
def _float64_default():
    """float64 as torch's default dtype for this module's tests only (restored after, so
    it does not leak into tests collected later)."""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)


def _rand_theta(widths, rng, scale=1.0):
    parts = []
    for l in range(1, len(widths)):
        parts.append(rng.standard_normal(widths[l] * widths[l - 1]) * scale / np.sqrt(widths[l - 1]))
    return np.concatenate(parts)


def _seq_inputs(rng, T, d, H=1, B=1):
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, H, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, d))
    alpha = 1 / (1 + np.exp(-(rng.standard_normal((B, T, H)) - 3)))
    eta = 0.3 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    beta = 1 / (1 + np.exp(-(rng.standard_normal((B, T, H)) + 1)))
    return q, k, v, alpha, eta, beta


def _torch_mlp(widths, theta):
    """torch.nn MLP (bias-free Linear, SiLU between layers) holding theta."""
    layers = []
    off = 0
    for l in range(1, len(widths)):
        lin = torch.nn.Linear(widths[l - 1], widths[l], bias=False)
        n = widths[l] * widths[l - 1]
        with torch.no_grad():
            lin.weight.copy_(torch.from_numpy(theta[off:off + n].reshape(widths[l], widths[l - 1])))
        off += n
        layers.append(lin)
        if l < len(widths) - 1:
            layers.append(torch.nn.SiLU())
    return torch.nn.Sequential(*layers)


def _torch_grad(widths, theta, k, v):
    net = _torch_mlp(widths, theta)
    out = net(torch.from_numpy(np.asarray(k, float)))
    loss = ((out - torch.from_numpy(np.asarray(v, float))) ** 2).sum()
    loss.backward()
    return float(loss.detach()), np.concatenate([m.weight.grad.numpy().reshape(-1)
                                        for m in net if isinstance(m, torch.nn.Linear)])


WIDTHS = [(4, 4), (4, 8, 4), (3, 5, 6, 2, 3), (5, 7, 3)]


# ---------------------------------------------------------------- gradient pins

@pytest.mark.parametrize("widths", WIDTHS)
def test_grad_matches_central_differences(widths):
    rng = np.random.default_rng(1)
    theta = _rand_theta(widths, rng)
    k = rng.standard_normal(widths[0])
    v = rng.standard_normal(widths[-1])
    loss, g = oracle.mlp_grad(widths, theta, k, v)
    h = 1e-6
    fd = np.empty_like(theta)
    for i in range(theta.size):
        tp, tm = theta.copy(), theta.copy()
        tp[i] += h
        tm[i] -= h
        fd[i] = (oracle.mlp_loss(widths, tp, k, v) - oracle.mlp_loss(widths, tm, k, v)) / (2 * h)
    assert np.linalg.norm(g - fd) <= 1e-7 * np.linalg.norm(fd)
    assert loss == pytest.approx(oracle.mlp_loss(widths, theta, k, v), rel=1e-15)


@pytest.mark.parametrize("widths", WIDTHS)
def test_forward_and_grad_match_torch_library(widths):
    rng = np.random.default_rng(2)
    theta = _rand_theta(widths, rng, scale=2.0)
    for _ in range(3):
        x = rng.standard_normal(widths[0])
        v = rng.standard_normal(widths[-1])
        ref = _torch_mlp(widths, theta)(torch.from_numpy(x)).detach().numpy()
        np.testing.assert_allclose(oracle.mlp_forward(widths, theta, x), ref, rtol=1e-13, atol=1e-13)
        l_ref, g_ref = _torch_grad(widths, theta, x, v)
        l, g = oracle.mlp_grad(widths, theta, x, v)
        assert l == pytest.approx(l_ref, rel=1e-13)
        np.testing.assert_allclose(g, g_ref, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------- delta rule (L = 1)

@pytest.mark.parametrize("C", [1, 4, 10, 64])
def test_linear_memory_no_momentum_no_decay_is_delta_rule(C):
    """L=1, alpha=beta=0: W <- W - 2 eta (W_c k - v) k^T with W_c the chunk-start matrix."""
    rng = np.random.default_rng(3)
    d, T = 6, 23
    q, k, v, _, eta, _ = _seq_inputs(rng, T, d)
    zeros = np.zeros((1, T, 1))
    W0 = rng.standard_normal((d, d)) / np.sqrt(d)
    y, thT, sT = oracle.scan(q, k, v, zeros, eta, zeros, W0.reshape(1, -1), np.zeros((1, d * d)),
                             C, (d, d))
    W = W0.copy()
    y_ref = np.zeros((T, d))
    for c0 in range(0, T, C):
        Wc = W.copy()
        for t in range(c0, min(T, c0 + C)):
            y_ref[t] = W @ q[0, t, 0]
            W = W - 2 * eta[0, t, 0] * np.outer(Wc @ k[0, t, 0] - v[0, t, 0], k[0, t, 0])
    np.testing.assert_allclose(y[0, :, 0], y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(thT[0, 0].reshape(d, d), W, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_exact_recall_and_read_before_write():
    """eta=1/2, alpha=beta=0, L=1, C=1: W_{t+1} = W_t (I - k k^T) + v k^T, so every
    written key recalls its value exactly, the orthogonal complement is untouched,
    and reading a key at its own token still returns the old memory."""
    rng = np.random.default_rng(4)
    d, T = 8, 5
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = basis[:, :T].T                        # T orthonormal keys
    vals = rng.standard_normal((T, d))
    W0 = rng.standard_normal((d, d))
    q = keys.copy()                              # read each key at its own token
    k = keys.copy()
    half = np.full((1, T, 1), 0.5)
    zeros = np.zeros((1, T, 1))
    y, thT, _ = oracle.scan(q[None, :, None], k[None, :, None], vals[None, :, None], zeros, half,
                            zeros, W0.reshape(1, -1), np.zeros((1, d * d)), 1, (d, d))
    WT = thT[0, 0].reshape(d, d)
    np.testing.assert_allclose(WT @ keys.T, vals.T, atol=1e-13)
    for x in basis[:, T:].T:
        np.testing.assert_allclose(WT @ x, W0 @ x, atol=1e-13)
    # token t reads with the weights before its own write: W_0 k_t (earlier keys are orthogonal)
    np.testing.assert_allclose(y[0, :, 0], (W0 @ keys.T).T, atol=1e-13)


# ------------------------------------------------------------ special cases

@pytest.mark.parametrize("C", [1, 5, 32])
def test_eta_zero_is_pure_decay(C):
    rng = np.random.default_rng(5)
    widths = (4, 8, 4)
    T = 17
    q, k, v, alpha, _, beta = _seq_inputs(rng, T, 4)
    theta0 = _rand_theta(widths, rng)
    zeros = np.zeros((1, T, 1))
    y, thT, _ = oracle.scan(q, k, v, alpha, zeros, beta, theta0[None], np.zeros((1, theta0.size)),
                            C, widths)
    decay = np.concatenate([[1.0], np.cumprod(1 - alpha[0, :, 0])])
    np.testing.assert_allclose(thT[0, 0], decay[T] * theta0, rtol=1e-14)
    for t in range(T):
        net = _torch_mlp(widths, decay[t] * theta0)
        ref = net(torch.from_numpy(q[0, t, 0])).detach().numpy()
        np.testing.assert_allclose(y[0, t, 0], ref, rtol=1e-12, atol=1e-14)


def test_alpha_one_beta_zero_keeps_one_token():
    """alpha=1, beta=0, C=1: theta_T = -eta_{T-1} grad l(theta_{T-1}; k_{T-1}, v_{T-1})."""
    rng = np.random.default_rng(6)
    widths = (4, 8, 4)
    T = 9
    q, k, v, _, eta, _ = _seq_inputs(rng, T, 4)
    ones, zeros = np.ones((1, T, 1)), np.zeros((1, T, 1))
    theta0 = _rand_theta(widths, rng)
    s0 = np.zeros((1, theta0.size))
    _, th_prev, _ = oracle.scan(q[:, :T - 1], k[:, :T - 1], v[:, :T - 1], ones[:, :T - 1],
                                eta[:, :T - 1], zeros[:, :T - 1], theta0[None], s0, 1, widths)
    _, thT, sT = oracle.scan(q, k, v, ones, eta, zeros, theta0[None], s0, 1, widths)
    _, g = _torch_grad(widths, th_prev[0, 0], k[0, T - 1, 0], v[0, T - 1, 0])
    np.testing.assert_allclose(sT[0, 0], g, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(thT[0, 0], -eta[0, T - 1, 0] * g, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("s0_val", [0.0, 0.7])
def test_scalar_memory_momentum_and_decay_closed_form(s0_val):
    """d=1, L=1, k=1, v=0, q=1, one chunk: every frozen gradient is 2 w0, so
       s_t = beta^{t+1} s0 + 2 w0 (1 - beta^{t+1}) and, with r = 1 - alpha,
       theta_t = r^t w0 - 2 eta w0 (1 - r^t)/(1 - r) - eta (s0 - 2 w0) beta (r^t - beta^t)/(r - beta)."""
    T, w0, al, et, be = 40, 0.9, 0.03, 0.2, 0.8
    ones = np.ones((1, T, 1, 1))
    y, thT, sT = oracle.scan(ones, ones, 0 * ones, np.full((1, T, 1), al), np.full((1, T, 1), et),
                             np.full((1, T, 1), be), np.array([[w0]]), np.array([[s0_val]]), T,
                             (1, 1))
    r = 1 - al

    def theta_at(t):
        return (r ** t * w0 - 2 * et * w0 * (1 - r ** t) / (1 - r)
                - et * (s0_val - 2 * w0) * be * (r ** t - be ** t) / (r - be))

    expect_y = np.array([theta_at(t) for t in range(T)])
    np.testing.assert_allclose(y[0, :, 0, 0], expect_y, rtol=1e-13)
    assert thT[0, 0, 0] == pytest.approx(theta_at(T), rel=1e-13)
    assert sT[0, 0, 0] == pytest.approx(be ** T * s0_val + 2 * w0 * (1 - be ** T), rel=1e-13)


# ------------------------------------------------ the summary page's letters

@pytest.mark.parametrize("C", [1, 4])
def test_summary_page_letters_give_the_same_memory(C):
    """The summary page writes M_t = (1-alpha_t) M_{t-1} + S_t, S_t = eta'_t S_{t-1} - theta'_t grad.
    With S_t = -eta_t s_t and M_t = theta_{t+1}, eta'_t = beta_t eta_t / eta_{t-1} (eta_{-1} = 1,
    S_{-1} = -s0) and theta'_t = eta_t (1 - beta_t) this is the same recurrence."""
    rng = np.random.default_rng(7)
    widths = (3, 6, 3)
    T = 14
    q, k, v, alpha, eta, beta = _seq_inputs(rng, T, 3)
    theta0 = _rand_theta(widths, rng)
    s0 = 0.1 * rng.standard_normal(theta0.size)
    y, thT, sT = oracle.scan(q, k, v, alpha, eta, beta, theta0[None], s0[None], C, widths)
    M = theta0.copy()
    S = -s0.copy()
    eta_prev = 1.0
    y_ref = np.zeros((T, 3))
    for c0 in range(0, T, C):
        Mc = M.copy()
        for t in range(c0, min(T, c0 + C)):
            y_ref[t] = _torch_mlp(widths, M)(torch.from_numpy(q[0, t, 0])).detach().numpy()
            _, g = _torch_grad(widths, Mc, k[0, t, 0], v[0, t, 0])
            e, b, a = eta[0, t, 0], beta[0, t, 0], alpha[0, t, 0]
            S = (b * e / eta_prev) * S - e * (1 - b) * g
            M = (1 - a) * M + S
            eta_prev = e
    np.testing.assert_allclose(y[0, :, 0], y_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(thT[0, 0], M, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(sT[0, 0], -S / eta_prev, rtol=1e-11, atol=1e-13)


def test_chunk_one_is_the_unchunked_recurrence():
    """C=1: the chunk-start weights are the current weights, i.e. plain test-time GD."""
    rng = np.random.default_rng(8)
    widths = (4, 8, 4)
    T = 12
    q, k, v, alpha, eta, beta = _seq_inputs(rng, T, 4)
    theta0 = _rand_theta(widths, rng)
    s0 = 0.05 * rng.standard_normal(theta0.size)
    y, thT, sT = oracle.scan(q, k, v, alpha, eta, beta, theta0[None], s0[None], 1, widths)
    th, s = theta0.copy(), s0.copy()
    for t in range(T):
        ref = _torch_mlp(widths, th)(torch.from_numpy(q[0, t, 0])).detach().numpy()
        np.testing.assert_allclose(y[0, t, 0], ref, rtol=1e-12, atol=1e-14)
        _, g = _torch_grad(widths, th, k[0, t, 0], v[0, t, 0])
        s = beta[0, t, 0] * s + (1 - beta[0, t, 0]) * g
        th = (1 - alpha[0, t, 0]) * th - eta[0, t, 0] * s
    np.testing.assert_allclose(thT[0, 0], th, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sT[0, 0], s, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------- invariants

def test_streaming_split_is_exact_when_aligned_to_chunks():
    rng = np.random.default_rng(9)
    widths = (4, 8, 4)
    T, C, T1 = 30, 5, 15
    q, k, v, alpha, eta, beta = _seq_inputs(rng, T, 4, H=2, B=2)
    theta0 = np.stack([_rand_theta(widths, rng) for _ in range(2)])
    s0 = np.zeros_like(theta0)
    y, thT, sT = oracle.scan(q, k, v, alpha, eta, beta, theta0, s0, C, widths)
    sl = slice(0, T1)
    y1, th1, s1 = oracle.scan(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], eta[:, sl], beta[:, sl],
                              theta0, s0, C, widths)
    sl = slice(T1, T)
    y2, th2, s2 = oracle.scan(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], eta[:, sl], beta[:, sl],
                              th1, s1, C, widths)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(th2, thT) and np.array_equal(s2, sT)
    # a split that is not on a chunk boundary changes where gradients freeze
    sl = slice(0, 13)
    _, th1, s1 = oracle.scan(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], eta[:, sl], beta[:, sl],
                             theta0, s0, C, widths)
    sl = slice(13, T)
    _, th2, _ = oracle.scan(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], eta[:, sl], beta[:, sl],
                            th1, s1, C, widths)
    assert not np.allclose(th2, thT, rtol=1e-9, atol=0)


def test_heads_and_batch_are_independent_and_theta0_broadcasts():
    rng = np.random.default_rng(10)
    widths = (4, 8, 4)
    B, T, H, C = 2, 11, 3, 4
    q, k, v, alpha, eta, beta = _seq_inputs(rng, T, 4, H=H, B=B)
    theta0 = np.stack([_rand_theta(widths, rng) for _ in range(H)])
    s0 = 0.01 * rng.standard_normal(theta0.shape)
    y, thT, sT = oracle.scan(q, k, v, alpha, eta, beta, theta0, s0, C, widths)
    yb, thb, sb = oracle.scan(q, k, v, alpha, eta, beta, np.stack([theta0] * B), np.stack([s0] * B),
                              C, widths)
    assert np.array_equal(y, yb) and np.array_equal(thT, thb) and np.array_equal(sT, sb)
    perm = [2, 0, 1]
    yp, thp, sp = oracle.scan(q[:, :, perm], k[:, :, perm], v[:, :, perm], alpha[:, :, perm],
                              eta[:, :, perm], beta[:, :, perm], theta0[perm], s0[perm], C, widths)
    assert np.array_equal(yp, y[:, :, perm]) and np.array_equal(thp, thT[:, perm])
    # each (b, h) alone gives the same result as inside the batch
    y1, th1, _ = oracle.scan(q[1:, :, 2:], k[1:, :, 2:], v[1:, :, 2:], alpha[1:, :, 2:],
                             eta[1:, :, 2:], beta[1:, :, 2:], theta0[2:], s0[2:], C, widths)
    assert np.array_equal(y1[0, :, 0], y[1, :, 2]) and np.array_equal(th1[0, 0], thT[1, 2])


def test_empty_sequence_returns_initial_state():
    widths = (4, 8, 4)
    rng = np.random.default_rng(11)
    theta0 = _rand_theta(widths, rng)[None]
    s0 = rng.standard_normal(theta0.shape)
    e = np.zeros((1, 0, 1, 4))
    g = np.zeros((1, 0, 1))
    y, thT, sT = oracle.scan(e, e, e, g, g, g, theta0, s0, 8, widths)
    assert y.shape == (1, 0, 1, 4)
    assert np.array_equal(thT[0], theta0) and np.array_equal(sT[0], s0)


# -------------------------------------- the GPU's matrix form == the oracle

@pytest.mark.parametrize("widths", [(4, 4), (4, 8, 4), (4, 6, 5, 4)])
@pytest.mark.parametrize("C", [1, 2, 3, 16, 64])
def test_chunk_matrix_form_equals_sequential_oracle(widths, C):
    rng = np.random.default_rng(12)
    T, H, B = 37, 2, 1
    d = widths[0]
    q, k, v, alpha, eta, beta = _seq_inputs(rng, T, d, H=H, B=B)
    theta0 = np.stack([_rand_theta(widths, rng) for _ in range(H)])
    s0 = 0.05 * rng.standard_normal(theta0.shape)
    y, thT, sT = oracle.scan(q, k, v, alpha, eta, beta, theta0, s0, C, widths)
    y2, th2, s2 = chunk_form.chunk_scan(q, k, v, alpha, eta, beta, theta0, s0, C, widths)
    scale = np.abs(y).max()
    assert np.abs(y - y2).max() <= 1e-12 * scale
    assert np.abs(thT - th2).max() <= 1e-12 * np.abs(thT).max()
    assert np.abs(sT - s2).max() <= 1e-12 * np.abs(sT).max()


def test_retrieve_is_the_read_with_fixed_weights():
    rng = np.random.default_rng(13)
    widths = (4, 8, 4)
    q = rng.standard_normal((2, 5, 3, 4))
    theta = np.stack([_rand_theta(widths, rng) for _ in range(3)])
    y = oracle.retrieve(q, theta, widths)
    for b in range(2):
        for t in range(5):
            for h in range(3):
                ref = _torch_mlp(widths, theta[h])(torch.from_numpy(q[b, t, h])).detach().numpy()
                np.testing.assert_allclose(y[b, t, h], ref, rtol=1e-13, atol=1e-14)
    # eta = 0 scan reads exactly the decayed initial weights (alpha = 0: the initial weights)
    zeros = np.zeros((2, 5, 3))
    ys, _, _ = oracle.scan(q, q, q, zeros, zeros, zeros, theta, np.zeros_like(theta), 2, widths)
    assert np.array_equal(ys, y)


# ------------------------------------------------------- attentional biases
#
# The pages name two alternative attentional biases (the MIRAS variants: YAAD with a
# Huber loss, MONETA with generalized norms) without formulas.  The oracle reads them as
# per-component losses of the residual r = M(k) - v, summed: Huber with threshold delta,
# r^2 inside |r| <= delta and 2 delta |r| - delta^2 outside; l_p, |r|^p.  These pins fix
# each definition by values computed by hand, by its own finite differences, by its
# reduction to the squared loss and by closed-form updates of a linear memory.

def _identity_residual(r):
    """A linear memory W = I with k = r and v = 0: the residual is r itself."""
    d = len(r)
    return (d, d), np.eye(d).reshape(-1), np.asarray(r, dtype=np.float64), np.zeros(d)


def test_bias_loss_values_by_hand():
    widths, theta, k, v = _identity_residual([0.5, -3.0, 1.0, -0.2])
    assert oracle.mlp_loss(widths, theta, k, v) == pytest.approx(0.25 + 9 + 1 + 0.04, rel=1e-15)
    # delta = 1: 0.25 + (2*3 - 1) + 1 + 0.04
    assert oracle.mlp_loss(widths, theta, k, v, ("huber", 1.0)) == pytest.approx(6.29, rel=1e-14)
    # delta = 0.4: (0.8*0.5 - 0.16) + (0.8*3 - 0.16) + (0.8 - 0.16) + 0.04
    assert oracle.mlp_loss(widths, theta, k, v, ("huber", 0.4)) == pytest.approx(
        0.24 + 2.24 + 0.64 + 0.04, rel=1e-14)
    assert oracle.mlp_loss(widths, theta, k, v, ("lp", 3.0)) == pytest.approx(
        0.125 + 27 + 1 + 0.008, rel=1e-14)
    assert oracle.mlp_loss(widths, theta, k, v, ("lp", 1.0)) == pytest.approx(4.7, rel=1e-14)
    # the gradient of a linear memory is loss'(r) k^T; with W = I, k = r its diagonal is
    # loss'(r_i) r_i: Huber delta = 1 clips the slope of -3 at -2
    _, g = oracle.mlp_grad(widths, theta, k, v, ("huber", 1.0))
    np.testing.assert_allclose(np.diag(g.reshape(4, 4)), [1.0 * 0.5, -2.0 * -3.0, 2.0, 0.08],
                               rtol=1e-15)
    _, g = oracle.mlp_grad(widths, theta, k, v, ("lp", 3.0))
    np.testing.assert_allclose(np.diag(g.reshape(4, 4)),
                               [3 * 0.25 * 0.5, -3 * 9 * -3.0, 3.0, -3 * 0.04 * -0.2], rtol=1e-14)


BIASES = [("huber", 0.3), ("huber", 2.0), ("lp", 1.5), ("lp", 3.0)]


@pytest.mark.parametrize("bias", BIASES)
@pytest.mark.parametrize("widths", [(4, 8, 4), (5, 7, 3)])
def test_bias_grad_matches_central_differences(widths, bias):
    rng = np.random.default_rng(11)
    theta = _rand_theta(widths, rng)
    k = rng.standard_normal(widths[0])
    v = rng.standard_normal(widths[-1])
    r = oracle.mlp_forward(widths, theta, k) - v
    if bias[0] == "huber":  # some components on each side of the threshold, none at it
        assert (np.abs(r) < bias[1]).any() or bias[1] < 0.5
        assert np.abs(np.abs(r) - bias[1]).min() > 1e-3
    loss, g = oracle.mlp_grad(widths, theta, k, v, bias)
    h = 1e-6
    fd = np.empty_like(theta)
    for i in range(theta.size):
        tp, tm = theta.copy(), theta.copy()
        tp[i] += h
        tm[i] -= h
        fd[i] = (oracle.mlp_loss(widths, tp, k, v, bias) - oracle.mlp_loss(widths, tm, k, v, bias)) / (2 * h)
    assert np.linalg.norm(g - fd) <= 1e-7 * np.linalg.norm(fd)
    assert loss == pytest.approx(oracle.mlp_loss(widths, theta, k, v, bias), rel=1e-15)


def test_bias_reduces_to_the_squared_loss():
    rng = np.random.default_rng(12)
    widths, T, C = (4, 8, 4), 30, 7
    q, k, v, alpha, eta, beta = _seq_inputs(rng, T, 4, H=2, B=2)
    th0 = np.stack([_rand_theta(widths, rng) for _ in range(2)])
    s0 = 0.1 * rng.standard_normal(th0.shape)
    ref = oracle.scan(q, k, v, alpha, eta, beta, th0, s0, C, widths)
    for bias in (("huber", 1e30), ("lp", 2.0)):
        out = oracle.scan(q, k, v, alpha, eta, beta, th0, s0, C, widths, bias=bias)
        for a, b in zip(out, ref):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    out = oracle.scan(q, k, v, alpha, eta, beta, th0, s0, C, widths, bias=("huber", 0.05))
    assert np.abs(out[1] - ref[1]).max() > 1e-3  # a small threshold does change the memory


@pytest.mark.parametrize("bias", [("huber", 0.2), ("lp", 1.0), ("lp", 3.0)])
@pytest.mark.parametrize("C", [1, 4])
def test_linear_memory_biased_delta_rule(bias, C):
    """L=1, alpha=beta=0: W <- W - eta loss'(W_c k - v) k^T, loss' written out here:
    2 clip(r, -delta, delta) for Huber, sign(r) for l_1, 3 |r| r for l_3."""
    rng = np.random.default_rng(13)
    d, T = 5, 21
    q, k, v, _, eta, _ = _seq_inputs(rng, T, d)
    zeros = np.zeros((1, T, 1))
    W0 = rng.standard_normal((d, d)) / np.sqrt(d)
    y, thT, _ = oracle.scan(q, k, v, zeros, eta, zeros, W0.reshape(1, -1), np.zeros((1, d * d)),
                            C, (d, d), bias=bias)
    if bias[0] == "huber":
        dl = lambda r: 2 * np.clip(r, -bias[1], bias[1])  # noqa: E731
    elif bias[1] == 1.0:
        dl = np.sign
    else:
        dl = lambda r: 3 * np.abs(r) * r  # noqa: E731
    W = W0.copy()
    y_ref = np.zeros((T, d))
    for c0 in range(0, T, C):
        Wc = W.copy()
        for t in range(c0, min(T, c0 + C)):
            y_ref[t] = W @ q[0, t, 0]
            W = W - eta[0, t, 0] * np.outer(dl(Wc @ k[0, t, 0] - v[0, t, 0]), k[0, t, 0])
    np.testing.assert_allclose(y[0, :, 0], y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(thT[0, 0].reshape(d, d), W, rtol=1e-12, atol=1e-12)


def test_bias_arguments_are_checked():
    rng = np.random.default_rng(14)
    q, k, v, alpha, eta, beta = _seq_inputs(rng, 3, 4)
    th0 = _rand_theta((4, 4), rng)[None]
    for bias in (("huber", 0.0), ("huber", -1.0), ("lp", 0.5)):
        with pytest.raises(ValueError):
            oracle.scan(q, k, v, alpha, eta, beta, th0, np.zeros_like(th0), 2, (4, 4), bias=bias)


# ------------------------------------------------------------ surprise norm
#
# The optional per-token output || g_t ||: the norm of the gradient each token writes
# with (at the chunk-start weights, under the chosen attentional bias).

@pytest.mark.parametrize("bias", [None, ("huber", 0.3)])
@pytest.mark.parametrize("C", [1, 3])
def test_surprise_is_the_norm_of_the_token_gradient(C, bias):
    """Recomputed here from the (finite-difference pinned) single-token gradient at the
    chunk-start weights, which the scan's own theta_T sequence supplies."""
    rng = np.random.default_rng(21)
    widths, T = (4, 6, 4), 7
    q, k, v, alpha, eta, beta = _seq_inputs(rng, T, 4)
    th0 = _rand_theta(widths, rng)[None]
    s0 = np.zeros_like(th0)
    y, thT, sT, sur = oracle.scan(q, k, v, alpha, eta, beta, th0, s0, C, widths, bias=bias,
                                  surprise=True)
    for t in range(T):
        c0 = t - t % C  # the chunk's start weights: the state after the first c0 tokens
        if c0 == 0:
            thc = th0[0]
        else:
            thc = oracle.scan(q[:, :c0], k[:, :c0], v[:, :c0], alpha[:, :c0], eta[:, :c0],
                              beta[:, :c0], th0, s0, C, widths, bias=bias)[1][0, 0]
        _, g = oracle.mlp_grad(widths, thc, k[0, t, 0], v[0, t, 0], bias)
        assert sur[0, t, 0] == pytest.approx(np.linalg.norm(g), rel=1e-12)
    ref = oracle.scan(q, k, v, alpha, eta, beta, th0, s0, C, widths, bias=bias)
    for a, b in zip((y, thT, sT), ref):
        np.testing.assert_array_equal(a, b)


def test_surprise_of_a_linear_memory_closed_form():
    """L = 1: g_t = 2 (W_c k - v) k^T, so || g_t || = 2 || W_c k - v || || k ||."""
    rng = np.random.default_rng(22)
    d, T, C = 5, 9, 4
    q, k, v, _, eta, _ = _seq_inputs(rng, T, d)
    zeros = np.zeros((1, T, 1))
    W0 = rng.standard_normal((d, d)) / np.sqrt(d)
    *_, sur = oracle.scan(q, k, v, zeros, eta, zeros, W0.reshape(1, -1), np.zeros((1, d * d)),
                          C, (d, d), surprise=True)
    W = W0.copy()
    for c0 in range(0, T, C):
        Wc = W.copy()
        for t in range(c0, min(T, c0 + C)):
            r = Wc @ k[0, t, 0] - v[0, t, 0]
            assert sur[0, t, 0] == pytest.approx(2 * np.linalg.norm(r) * np.linalg.norm(k[0, t, 0]),
                                                 rel=1e-12)
            W = W - 2 * eta[0, t, 0] * np.outer(r, k[0, t, 0])


def test_state_conditioning_is_a_property_of_the_method():
    """The GPU tests' state bars are a multiple of how far theta_T moves when k and v carry
    one bf16 rounding (each element times 1 + 2^-9 u, u ~ U(-1, 1)).  That sensitivity must
    be the recurrence's, not an artefact of one implementation: the sequential oracle and the
    independent NumPy chunk-form restatement give the same figure on the same perturbation,
    and it is far above float64 rounding (a bf16-operand kernel cannot do better than a
    multiple of it)."""
    import synthetic

    wl = synthetic.sustained("h16_d64_b8_t16k").with_(batch=1, heads=1, seq_len=1024)
    inp = synthetic.make_inputs(wl, 0)
    q, k, v = (inp.qkv_f32(n).astype(np.float64) for n in ("q", "k", "v"))
    g = [getattr(inp, n).astype(np.float64) for n in ("alpha", "eta", "beta")]
    rng = np.random.default_rng(7)
    pk = k * (1.0 + 2.0 ** -9 * rng.uniform(-1, 1, k.shape))
    pv = v * (1.0 + 2.0 ** -9 * rng.uniform(-1, 1, v.shape))
    th0, s0 = inp.theta0.astype(np.float64), inp.s0.astype(np.float64)

    def kappa(fn):
        _, t, _ = fn(q, k, v, *g, th0, s0, wl.chunk, wl.widths)
        _, tp, _ = fn(q, pk, pv, *g, th0, s0, wl.chunk, wl.widths)
        return np.linalg.norm(tp - t) / np.linalg.norm(t)

    k_oracle = kappa(oracle.scan)
    k_chunk = kappa(chunk_form.chunk_scan)
    assert 1e-3 < k_oracle < 2e-2
    assert abs(k_oracle - k_chunk) <= 1e-3 * k_oracle
