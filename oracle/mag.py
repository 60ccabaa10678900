"""Titans MAG block (memory as gate) in fp64 NumPy -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline may import this
module.  One block: a projection front-end, the neural memory as the long-term branch,
sliding-window attention as the short-term branch, and the memory output as a sigmoid gate
on the attention output (explainer, the three architecture variants, MAG:
o_t = sigmoid(y_mem_t) * y_attn_t; lowest.today summary, "Varianti dell'Architettura
Titans", Memory as Gate).  The pages fix the combination; the rest takes the plainest
reading:

  q = normalize(x Wq), k = normalize(x Wk), v = x Wv      per head (d columns each), q and
                                                          k unit L2 norm per (token, head)
  g = x Wg + bg;  alpha = sigmoid(g_a), eta = eta_scale * sigmoid(g_e), beta = sigmoid(g_b)
  y_mem  = the chunked memory scan of (q, k, v, alpha, eta, beta) from (theta0, s0)
  y_attn = causal sliding-window attention over the last `window` tokens (the token
           itself included), softmax(q k^T / sqrt(d)) per head
  o = sigmoid(y_mem) * y_attn,  out = o Wo

x is [B, T, D] with D = H d; Wq, Wk, Wv, Wo are [D, D] (x @ W), Wg is [D, 3H] and bg [3H]
(columns: alpha gates of heads 0..H-1, then eta, then beta).
"""
from __future__ import annotations

import numpy as np

import oracle


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def round_bf16(a):
    """Round to the nearest bfloat16 (ties to even), through float32, by torch's CPU
    conversion; returned as float64."""
    import torch

    t = torch.from_numpy(np.asarray(a, np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def front_end(x, Wq, Wk, Wv, Wg, bg, H, eta_scale, store=None):
    """q, k, v [B, T, H, d] and alpha, eta, beta [B, T, H] from x.

    store="bf16" rounds q, k, v to bfloat16 after the normalization: the block's interface
    keeps them in that format, so the memory and the attention both read the rounded
    values (a long scan is sensitive enough to that rounding that its final state can
    only be compared at the same storage precision)."""
    B, T, _ = x.shape
    d = np.shape(Wq)[1] // H  # the projections may cover a subset of the heads
    x = np.asarray(x, np.float64)

    def heads(w):
        return (x @ np.asarray(w, np.float64)).reshape(B, T, H, d)

    q, k, v = heads(Wq), heads(Wk), heads(Wv)
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    g = x @ np.asarray(Wg, np.float64) + np.asarray(bg, np.float64)
    alpha = _sigmoid(g[..., :H])
    eta = eta_scale * _sigmoid(g[..., H:2 * H])
    beta = _sigmoid(g[..., 2 * H:])
    if store == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif store is not None:
        raise ValueError(f"store={store!r}")
    return q, k, v, alpha, eta, beta


def sliding_window_attention(q, k, v, window):
    """Causal attention of every token over itself and the window - 1 tokens before it,
    per (b, h): softmax over the scaled dot products, then the weighted sum of values."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, T, H, d = q.shape
    out = np.zeros_like(q)
    scale = 1.0 / np.sqrt(d)
    for t in range(T):
        j0 = max(0, t - window + 1)
        s = np.einsum("bhd,bjhd->bhj", q[:, t], k[:, j0:t + 1]) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[:, t] = np.einsum("bhj,bjhd->bhd", p, v[:, j0:t + 1])
    return out


def mag_forward(x, Wq, Wk, Wv, Wg, bg, Wo, widths, chunk, window, eta_scale, theta0, s0):
    """The block's output [B, T, D] and its intermediates (dict, all float64)."""
    x = np.asarray(x, np.float64)
    B, T, D = x.shape
    d = widths[0]
    H = D // d
    q, k, v, alpha, eta, beta = front_end(x, Wq, Wk, Wv, Wg, bg, H, eta_scale)
    y_mem, th, s = oracle.scan(q, k, v, alpha, eta, beta, theta0, s0, chunk, widths)
    y_attn = sliding_window_attention(q, k, v, window)
    o = _sigmoid(y_mem) * y_attn
    out = o.reshape(B, T, D) @ np.asarray(Wo, np.float64)
    return out, {"q": q, "k": k, "v": v, "alpha": alpha, "eta": eta, "beta": beta,
                 "y_mem": y_mem, "y_attn": y_attn, "o": o, "theta_T": th, "s_T": s}
