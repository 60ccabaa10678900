"""Reverse-mode derivatives of the chunked Titans memory scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import this module.  The scan is written out again token by token in
float64 torch CPU ops -- the same steps, in the same order, as ``titans_oracle.c``:

  read      y_t = M_{theta_t}(q_t)                (weights before token t's write)
  surprise  g_t = grad_theta || M_theta(k_t) - v_t ||^2 at the chunk-start weights,
            by explicit backpropagation (factor 2, no 1/2)
  momentum  s_{t+1} = beta_t s_t + (1 - beta_t) g_t
  write     theta_{t+1} = (1 - alpha_t) theta_t - eta_t s_{t+1}

(Titans paper explainer, 0h-n0.github.io, sections on the memory module, the momentum and
the forget gate; lowest.today Titans summary, "Funzione Obiettivo" and "Addestramento
Parallelizzato").  torch.autograd differentiates that program: for output cotangents
(dy, d theta_T, d s_T) it returns the cotangents of every input.  The second derivatives
the chunk-frozen gradients bring in (d g_t / d theta_c, d g_t / d k_t, d g_t / d v_t) come
from autograd tracing the explicit backpropagation, not from a hand derivation.
"""
from __future__ import annotations

import torch


def _silu(z):
    return z * torch.sigmoid(z)


def _silu_prime(z):
    s = torch.sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def _weights(theta, widths):
    Ws, off = [], 0
    for l in range(1, len(widths)):
        n = widths[l] * widths[l - 1]
        Ws.append(theta[off:off + n].reshape(widths[l], widths[l - 1]))
        off += n
    return Ws


def _mlp(Ws, x):
    h = x
    for i, W in enumerate(Ws):
        z = W @ h
        h = _silu(z) if i < len(Ws) - 1 else z
    return h


def _loss_prime(r, bias):
    """Derivative of the per-component loss at residual r."""
    if bias is None or bias[0] == "l2":
        return 2.0 * r
    if bias[0] == "huber":
        return 2.0 * torch.clamp(r, -bias[1], bias[1])
    if bias[0] == "lp":
        return bias[1] * torch.sign(r) * torch.abs(r) ** (bias[1] - 1.0)
    raise ValueError(bias)


def _grad(Ws, k, v, bias=None):
    """grad_theta of the loss of M(k) against v as one flat vector (explicit
    backpropagation)."""
    hs, zs = [k], []
    for i, W in enumerate(Ws):
        z = W @ hs[-1]
        zs.append(z)
        hs.append(_silu(z) if i < len(Ws) - 1 else z)
    delta = _loss_prime(hs[-1] - v, bias)
    gs = [None] * len(Ws)
    for i in range(len(Ws) - 1, -1, -1):
        gs[i] = torch.outer(delta, hs[i])
        if i > 0:
            delta = (Ws[i].T @ delta) * _silu_prime(zs[i - 1])
    return torch.cat([g.reshape(-1) for g in gs])


def scan(q, k, v, alpha, eta, beta, theta0, s0, chunk, widths, bias=None):
    """The scan in torch (differentiable).  q, k, v: [B, T, H, d]; gates [B, T, H];
    theta0, s0: [B, H, P].  Returns y [B, T, H, d], theta_T, s_T [B, H, P]."""
    B, T, H, _ = q.shape
    ys, ths, ss = [], [], []
    for b in range(B):
        yb, thb, sb = [], [], []
        for h in range(H):
            th, s = theta0[b, h], s0[b, h]
            yrow = []
            for c0 in range(0, T, chunk):
                Wc = _weights(th, widths)  # frozen for this chunk's gradients
                for t in range(c0, min(T, c0 + chunk)):
                    yrow.append(_mlp(_weights(th, widths), q[b, t, h]))
                    g = _grad(Wc, k[b, t, h], v[b, t, h], bias)
                    s = beta[b, t, h] * s + (1.0 - beta[b, t, h]) * g
                    th = (1.0 - alpha[b, t, h]) * th - eta[b, t, h] * s
            yb.append(torch.stack(yrow) if yrow else q.new_zeros((0, widths[-1])))
            thb.append(th)
            sb.append(s)
        ys.append(torch.stack(yb, dim=1))
        ths.append(torch.stack(thb))
        ss.append(torch.stack(sb))
    return torch.stack(ys), torch.stack(ths), torch.stack(ss)


NAMES = ("q", "k", "v", "alpha", "eta", "beta", "theta0", "s0")


def scan_vjp(inputs, chunk, widths, dy, dtheta, ds, bias=None):
    """Cotangents of every input for output cotangents (dy, dtheta, ds).

    inputs: dict of numpy arrays named as NAMES (theta0, s0 per (b, h): [B, H, P]).
    Returns a dict of float64 numpy arrays of the same shapes."""
    xs = {n: torch.tensor(inputs[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    y, th, s = scan(*(xs[n] for n in NAMES), chunk, widths, bias)
    obj = (y * torch.as_tensor(dy, dtype=torch.float64)).sum() + \
        (th * torch.as_tensor(dtheta, dtype=torch.float64)).sum() + \
        (s * torch.as_tensor(ds, dtype=torch.float64)).sum()
    grads = torch.autograd.grad(obj, [xs[n] for n in NAMES], allow_unused=True)
    return {n: (torch.zeros_like(xs[n]) if g is None else g).detach().numpy()
            for n, g in zip(NAMES, grads)}
