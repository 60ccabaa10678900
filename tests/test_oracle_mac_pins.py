"""Pins of the MAC block oracle (oracle/mac.py) against things other than itself.

  * prefix attention equals torch's scaled-dot-product attention (a library routine) over
    the concatenated keys [h ; k] with an explicit mask (every prefix entry visible, own
    keys causal);
  * a zero memory reads zero, so the prefix adds L keys of score 0 and value 0:
    y_t = sum_{u<=t} e^{s_u} v_u / (L + sum_{u<=t} e^{s_u}) in closed form;
  * with one segment the prefix is the memory read at theta0, M_theta0(q) (the C oracle's
    retrieve), and the final state is the C oracle's scan over all T; over several
    segments (a multiple of the chunk) the final state is still the one full scan's
    (streaming equivalence).
"""
import numpy as np

import oracle
from oracle import mac, mag


def _weights(D, H, rng):
    def w(shape):
        return rng.standard_normal(shape) / np.sqrt(D)

    return (w((D, D)), w((D, D)), w((D, D)), w((D, 3 * H)),
            np.concatenate([np.full(H, -4.0), np.zeros(H), np.full(H, 2.0)]), w((D, D)))


def test_prefix_attention_equals_library_masked_attention():
    import torch

    rng = np.random.default_rng(0)
    B, L, H, d = 2, 13, 3, 8
    q, k, v, h = (rng.standard_normal((B, L, H, d)) for _ in range(4))
    ours = mac.prefix_attention(q, k, v, h)
    keys = np.concatenate([h, k], axis=1)
    vals = np.concatenate([h, v], axis=1)
    mask = np.zeros((L, 2 * L), dtype=bool)
    for t in range(L):
        mask[t, :L] = True
        mask[t, L:L + t + 1] = True
    tq, tk, tv = (torch.tensor(a).permute(0, 2, 1, 3) for a in (q, keys, vals))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv,
                                                           attn_mask=torch.tensor(mask))
    np.testing.assert_allclose(ours, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)


def test_zero_memory_closed_form():
    rng = np.random.default_rng(1)
    B, L, H, d = 1, 9, 2, 4
    q, k, v = (rng.standard_normal((B, L, H, d)) for _ in range(3))
    ours = mac.prefix_attention(q, k, v, np.zeros((B, L, H, d)))
    for t in range(L):
        e = np.exp(np.einsum("bhd,bjhd->bhj", q[:, t], k[:, :t + 1]) / np.sqrt(d))
        ref = np.einsum("bhj,bjhd->bhd", e, v[:, :t + 1]) / (L + e.sum(-1))[..., None]
        np.testing.assert_allclose(ours[:, t], ref, rtol=1e-13)


def test_one_segment_and_streaming_state():
    rng = np.random.default_rng(2)
    H, d = 2, 8
    D = H * d
    widths = (d, 16, d)
    P = oracle.param_count(widths)
    Wq, Wk, Wv, Wg, bg, Wo = _weights(D, H, rng)
    x = rng.standard_normal((2, 24, D))
    th0 = rng.standard_normal((H, P)) * 0.3
    s0 = np.zeros((H, P))
    out, mid = mac.mac_forward(x, Wq, Wk, Wv, Wg, bg, Wo, widths, 4, 24, 0.1, th0, s0)
    np.testing.assert_array_equal(mid["h"], oracle.retrieve(mid["q"], th0, widths))
    _, th_ref, s_ref = oracle.scan(mid["q"], mid["k"], mid["v"], mid["alpha"], mid["eta"],
                                   mid["beta"], th0, s0, 4, widths)
    np.testing.assert_allclose(mid["theta_T"], th_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out, mid["y_attn"].reshape(2, 24, D) @ Wo, rtol=1e-13)
    _, mid3 = mac.mac_forward(x, Wq, Wk, Wv, Wg, bg, Wo, widths, 4, 8, 0.1, th0, s0)
    np.testing.assert_allclose(mid3["theta_T"], th_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(mid3["s_T"], s_ref, rtol=1e-12, atol=1e-14)
    # later segments read the memory as it stands at their start
    _, th8, _ = oracle.scan(mid["q"][:, :8], mid["k"][:, :8], mid["v"][:, :8],
                            mid["alpha"][:, :8], mid["eta"][:, :8], mid["beta"][:, :8], th0, s0,
                            4, widths)
    np.testing.assert_allclose(mid3["h"][:, 8:16], oracle.retrieve(mid["q"][:, 8:16], th8, widths),
                               rtol=1e-12, atol=1e-14)
    assert not np.allclose(mid3["h"][:, 8:16], mid["h"][:, 8:16])
