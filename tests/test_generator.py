"""The seeded synthetic inputs: reproducible, prefix-consistent, of the stated recipe."""
import numpy as np
import pytest

import synthetic as S


def test_reproducible_and_seed_dependent():
    wl = S.WORKLOADS["h8_d64_b4_t4k"].with_(seq_len=300, batch=2)
    a, b = S.make_inputs(wl, 0), S.make_inputs(wl, 0)
    c = S.make_inputs(wl, 1)
    for n in ("q", "k", "v", "alpha", "eta", "beta", "theta0"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
        assert not np.array_equal(getattr(a, n), getattr(c, n))


def test_prefix_of_a_longer_draw():
    wl = S.WORKLOADS["long_h16_d64_b1_t2m"]
    short = S.make_inputs(wl, 3, seq_len=5000)
    longer = S.make_inputs(wl, 3, seq_len=9000)
    for n in ("q", "k", "v", "alpha", "eta", "beta"):
        assert np.array_equal(getattr(longer, n)[:, :5000], getattr(short, n))
    assert np.array_equal(short.theta0, longer.theta0)


def test_recipe_statistics():
    wl = S.WORKLOADS["h8_d64_b4_t4k"]
    x = S.make_inputs(wl, 0, batch=2, seq_len=4096)
    qf = x.qkv_f32("q").astype(np.float64)
    norms = np.linalg.norm(qf, axis=-1)
    assert np.abs(norms - 1).max() < 8e-3          # L2-normalised, then bf16-rounded
    vf = x.qkv_f32("v").astype(np.float64)
    assert abs(vf.mean()) < 0.01 and abs(vf.std() - 1) < 0.01
    assert 0.025 < x.alpha.mean() < 0.032          # E[sigmoid(N(-4,1))] ~ 0.028
    assert 0.048 < x.eta.mean() < 0.052            # 0.1 * E[sigmoid(N(0,1))] = 0.05
    assert 0.83 < x.beta.mean() < 0.86             # E[sigmoid(N(2,1))] ~ 0.845
    assert x.alpha.min() > 0 and x.beta.max() < 1
    w1 = x.theta0[:, :256 * 64].astype(np.float64)
    w2 = x.theta0[:, 256 * 64:].astype(np.float64)
    assert abs(w1.var() - 1 / 64) < 0.01 / 64 * 10
    assert abs(w2.var() - 1 / 256) < 0.01 / 256 * 10
    assert np.all(x.s0 == 0)
    deep = S.make_inputs("deep_h8_d128_b2_t32k", 0, batch=1, seq_len=4096)
    assert 0.009 < deep.alpha.mean() < 0.013 and 0.023 < deep.eta.mean() < 0.027


def test_bf16_rounding_is_nearest_even():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -2.00781250, 3.0e-39]   # ties and a subnormal
    bits = S.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(S.bf16_bits_to_f32(bits), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_table():
    w = S.WORKLOADS
    assert w["h16_d64_b8_t16k"].params == 32768 and w["h16_d64_b8_t16k"].chunk == 64
    assert w["deep_h8_d128_b2_t32k"].n_layers == 4 and w["deep_h8_d128_b2_t32k"].params == 655360
    assert w["long_h16_d64_b1_t2m"].seq_len == 1 << 21 and w["long_h16_d64_b1_t2m"].chunk == 256
    assert w["tiny_f32_h1_t512"].io == "f32" and w["tiny_f32_h1_t512"].chunk == 16


def test_mag_inputs_prefix_consistent_and_distributed_as_the_recipe():
    import synthetic as S

    wl = S.WORKLOADS[S.HEADLINE].with_(heads=4)
    a = S.make_mag_inputs(wl, 64, seed=2, seq_len=300, batch=2)
    b = S.make_mag_inputs(wl, 64, seed=2, seq_len=100, batch=2)
    assert np.array_equal(a.x[:, :100], b.x)
    for n in ("w_in", "w_out", "b_gate", "theta0"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    D = wl.heads * wl.d
    assert a.x.shape == (2, 300, D) and a.w_in.shape == (3 * D + 3 * wl.heads, D)
    assert a.w_out.shape == (D, D) and a.b_gate.shape == (3 * wl.heads,)
    # every projected feature of x is ~ N(0, 1); the gate biases are (mu_alpha, 0, mu_beta)
    Wq, Wk, Wv, Wg, bg, Wo = a.oracle_weights()
    x = S.bf16_bits_to_f32(a.x).astype(np.float64).reshape(-1, D)
    for W in (Wq, Wv, Wg):
        f = x @ W
        assert abs(f.mean()) < 0.05 and abs(f.std() - 1.0) < 0.05
    np.testing.assert_array_equal(bg, np.repeat([wl.alpha_mu, 0.0, wl.beta_mu], wl.heads))
    c = S.make_mag_inputs(wl, 64, seed=3, seq_len=100, batch=2)
    assert not np.array_equal(c.x, b.x) and not np.array_equal(c.w_in, b.w_in)
