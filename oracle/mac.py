"""Titans MAC block (memory as context) in fp64 NumPy -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline may import this
module.  The sequence is processed in segments; each segment reads the long-term memory and
the reads join the attention's context as a prefix of keys and values (lowest.today
summary, "Varianti dell'Architettura Titans", Memory as Context; explainer, the three
architecture variants, MAC: the memory output is prepended to the keys and values).  The
rest takes the plainest reading, with the MAG block's front end:

  q, k, v, alpha, eta, beta = the MAG front end of x (oracle/mag.py)
  segments of S tokens from the call start (the last may be shorter); for segment i:
    theta_i = the memory state after every token before the segment (the scan, run segment
              by segment, so its chunks start at each segment start)
    h_t     = M_{theta_i}(q_t) for every token t of the segment (read with fixed weights)
    y_t     = softmax attention of q_t over the keys [h_u for every u in the segment] then
              [k_u for u <= t in the segment], values [h_u ...] then [v_u ...], scores
              q.key / sqrt(d)
    the memory then writes the segment's k, v with its gates (the scan)
  out = y Wo
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import mag


def prefix_attention(q, k, v, h):
    """One segment, per (b, head): query t attends to every prefix entry h_u (as key and as
    value) and to the segment's own (k_u, v_u) for u <= t."""
    q, k, v, h = (np.asarray(a, np.float64) for a in (q, k, v, h))
    B, L, H, d = q.shape
    out = np.zeros_like(q)
    scale = 1.0 / np.sqrt(d)
    for t in range(L):
        keys = np.concatenate([h, k[:, :t + 1]], axis=1)
        vals = np.concatenate([h, v[:, :t + 1]], axis=1)
        s = np.einsum("bhd,bjhd->bhj", q[:, t], keys) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[:, t] = np.einsum("bhj,bjhd->bhd", p, vals)
    return out


def mac_forward(x, Wq, Wk, Wv, Wg, bg, Wo, widths, chunk, segment, eta_scale, theta0, s0,
                store=None):
    """The block's output [B, T, D] and its intermediates (dict, all float64)."""
    x = np.asarray(x, np.float64)
    B, T, D = x.shape
    d = widths[0]
    H = D // d
    q, k, v, alpha, eta, beta = mag.front_end(x, Wq, Wk, Wv, Wg, bg, H, eta_scale, store=store)
    th = np.broadcast_to(np.asarray(theta0, np.float64), (B,) + np.shape(theta0)[-2:]).copy()
    s = np.broadcast_to(np.asarray(s0, np.float64), th.shape).copy()
    h_all = np.zeros_like(q)
    y = np.zeros_like(q)
    for t0 in range(0, T, segment):
        sl = slice(t0, min(T, t0 + segment))
        h_all[:, sl] = oracle.retrieve(q[:, sl], th, widths)
        y[:, sl] = prefix_attention(q[:, sl], k[:, sl], v[:, sl], h_all[:, sl])
        _, th, s = oracle.scan(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], eta[:, sl],
                               beta[:, sl], th, s, chunk, widths)
    out = y.reshape(B, T, D) @ np.asarray(Wo, np.float64)
    return out, {"q": q, "k": k, "v": v, "alpha": alpha, "eta": eta, "beta": beta,
                 "h": h_all, "y_attn": y, "theta_T": th, "s_T": s}
