"""Pins of the MAG block oracle (oracle/mag.py) against things other than itself.

  * attention: with a window as long as the sequence it equals torch's causal
    scaled-dot-product attention (a library routine); a window of one returns v exactly; a
    window of w equals full causal attention on every token < w, and each token's output is
    a convex combination of the values in its window only (changing a value outside the
    window leaves it unchanged);
  * gate: with a memory that reads zero (theta0 = 0, eta = 0) the block output is
    (y_attn / 2) Wo exactly;
  * front end: rows of x that are unit vectors pick rows of the projection matrices (q, k
    normalized), and the gates are the sigmoids of the matching Wg row plus bg;
  * memory branch: the C oracle's scan of the front end's q, k, v, gates;
  * bf16 storage: round_bf16 agrees with an integer round-to-nearest-even on the float32
    bit pattern (the generator's, an independent implementation) and with exhaustive
    neighbours: no bfloat16 value lies strictly closer.
"""
import numpy as np
import pytest

import oracle
from oracle import mag


def _weights(D, H, rng, scale=1.0):
    def w(shape, fan):
        return rng.standard_normal(shape) / np.sqrt(fan) * scale

    return (w((D, D), D), w((D, D), D), w((D, D), D), w((D, 3 * H), D),
            np.concatenate([np.full(H, -4.0), np.zeros(H), np.full(H, 2.0)]), w((D, D), D))


def test_full_window_equals_library_causal_attention():
    import torch

    rng = np.random.default_rng(0)
    B, T, H, d = 2, 23, 3, 8
    q, k, v = (rng.standard_normal((B, T, H, d)) for _ in range(3))
    ours = mag.sliding_window_attention(q, k, v, window=T)
    tq, tk, tv = (torch.tensor(a).permute(0, 2, 1, 3) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(ours, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)


def test_window_one_and_window_locality():
    rng = np.random.default_rng(1)
    B, T, H, d = 1, 30, 2, 4
    q, k, v = (rng.standard_normal((B, T, H, d)) for _ in range(3))
    np.testing.assert_allclose(mag.sliding_window_attention(q, k, v, 1), v, rtol=1e-15)
    w = 7
    out = mag.sliding_window_attention(q, k, v, w)
    full = mag.sliding_window_attention(q, k, v, T)
    np.testing.assert_allclose(out[:, :w], full[:, :w], rtol=1e-13)
    assert not np.allclose(out[:, w:], full[:, w:])
    v2 = v.copy()
    v2[:, 3] += 100.0  # outside the window of every token t >= 3 + w
    out2 = mag.sliding_window_attention(q, k, v2, w)
    np.testing.assert_array_equal(out2[:, 3 + w:], out[:, 3 + w:])
    assert not np.allclose(out2[:, 3:3 + w], out[:, 3:3 + w])
    # a convex combination: every output lies inside the value range of its window
    t = 20
    lo = v[:, t - w + 1:t + 1].min(axis=1)
    hi = v[:, t - w + 1:t + 1].max(axis=1)
    assert np.all(out[:, t] >= lo - 1e-12) and np.all(out[:, t] <= hi + 1e-12)


def test_zero_memory_halves_the_attention_output():
    rng = np.random.default_rng(2)
    B, T, H, d = 2, 20, 2, 8
    D = H * d
    widths = (d, 16, d)
    x = rng.standard_normal((B, T, D))
    Wq, Wk, Wv, Wg, bg, Wo = _weights(D, H, rng)
    P = oracle.param_count(widths)
    zero = np.zeros((H, P))
    out, mid = mag.mag_forward(x, Wq, Wk, Wv, Wg, bg, Wo, widths, 4, 5, 0.0, zero, zero)
    np.testing.assert_array_equal(mid["y_mem"], 0.0)
    np.testing.assert_allclose(out, (0.5 * mid["y_attn"]).reshape(B, T, D) @ Wo, rtol=1e-14)


def test_front_end_on_unit_rows_and_memory_branch():
    rng = np.random.default_rng(3)
    H, d = 2, 4
    D = H * d
    Wq, Wk, Wv, Wg, bg, Wo = _weights(D, H, rng)
    x = np.eye(D)[None]  # token t is the unit vector e_t
    q, k, v, al, et, be = mag.front_end(x, Wq, Wk, Wv, Wg, bg, H, 0.1)
    for t in range(D):
        for h in range(H):
            row = Wq[t, h * d:(h + 1) * d]
            np.testing.assert_allclose(q[0, t, h], row / np.linalg.norm(row), rtol=1e-14)
            np.testing.assert_allclose(v[0, t, h], Wv[t, h * d:(h + 1) * d], rtol=1e-15)
            np.testing.assert_allclose(al[0, t, h], 1 / (1 + np.exp(-(Wg[t, h] + bg[h]))),
                                       rtol=1e-14)
            np.testing.assert_allclose(et[0, t, h], 0.1 / (1 + np.exp(-(Wg[t, H + h] + bg[H + h]))),
                                       rtol=1e-14)
    widths = (d, 8, d)
    P = oracle.param_count(widths)
    th0 = rng.standard_normal((H, P)) * 0.3
    x = rng.standard_normal((1, 12, D))
    _, mid = mag.mag_forward(x, Wq, Wk, Wv, Wg, bg, Wo, widths, 4, 3, 0.1, th0, np.zeros((H, P)))
    y, _, _ = oracle.scan(mid["q"], mid["k"], mid["v"], mid["alpha"], mid["eta"], mid["beta"],
                          th0, np.zeros((H, P)), 4, widths)
    np.testing.assert_array_equal(mid["y_mem"], y)
    np.testing.assert_allclose(mid["o"], 1 / (1 + np.exp(-y)) * mid["y_attn"], rtol=1e-15)


def test_round_bf16_is_nearest_even():
    import synthetic as S

    rng = np.random.default_rng(4)
    a = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000),
                        [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)]])
    a32 = a.astype(np.float32)
    got = mag.round_bf16(a32)
    ref = S.bf16_bits_to_f32(S.f32_to_bf16_bits(a32)).astype(np.float64)
    np.testing.assert_array_equal(got, ref)
    # ties go to the even mantissa: 1 + 2^-8 -> 1, 1 + 3 * 2^-8 -> 1 + 2^-6
    assert got[-3] == 1.0 and got[-2] == 1.0 + 2.0 ** -6 and got[-1] == -1.0
    # nearest: the two bf16 neighbours (one ulp, 2^-7 relative, up and down) are no closer
    for x, y in zip(a32[:200], got[:200]):
        ulp = 2.0 ** (np.floor(np.log2(abs(y))) - 7) if y != 0 else 0.0
        for n in (y - ulp, y + ulp):
            assert abs(n - x) >= abs(y - x)
    x = np.random.default_rng(5).standard_normal((1, 4, 8))
    W = np.eye(8)
    q, k, v, *_ = mag.front_end(x, W, W, W, np.zeros((8, 3)), np.zeros(3), 1, 0.1, store="bf16")
    np.testing.assert_array_equal(v, mag.round_bf16(x.reshape(1, 4, 1, 8)))
    np.testing.assert_array_equal(q, mag.round_bf16(q))
