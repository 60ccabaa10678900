"""GPU parity of the MAG block (titans_mag_forward) against the fp64 oracle (oracle/mag.py).

Both sides take the same seeded inputs (synthetic.make_mag_inputs): x and the weights are
bf16 values, which the oracle reads exactly.  The HIP path rounds q, k, v, the memory read
y_mem, the attention probabilities and the gated output o to bf16 where it stores them
(8 significant bits, relative rounding error <= 2^-9 each); the oracle keeps fp64 through.
The bars scale with each token row's RMS (a row of out is D sums over o_i W_i, so an
element's rounding error follows the size of its terms, not its own size, which can cancel
to ~0):

  * out: every term o_i W_i carries the roundings of o (2^-9) and, linearly, of q, k, v, the
    probabilities and y_mem (2^-9 each), so ~3 * 2^-9 relative; summed with random signs
    over D terms an element's error is ~3 * 2^-9 RMS_row(out) = 0.6% with tails of ~4 sigma
    over B T D elements, plus 2^-9 |out| from the final bf16 store.  Bars: per element
    |out - ref| <= 3e-2 RMS_row(ref); per row RMS(out - ref) <= 1e-2 RMS_row(ref).  (A CPU
    model of exactly these roundings reaches 1.5e-2 and 4.4e-3 on the cases below, as the
    kernels do.)
  * theta_T, s_T: the memory scan's own bf16 bars (relative Frobenius error): 1e-1 on the
    short cases; at full size 5x the method's own sensitivity, measured by running the fp64
    scan again with k and v perturbed by one bf16 rounding (at least 2e-2), as the scan's
    full-length tests do -- the scan kernels round about seven operands of that size per
    chunk, which add in quadrature to about 3x that sensitivity.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from oracle import mag as omag

pytestmark = pytest.mark.gpu

BAR_OUT_MAX = 3e-2    # per element, of the token row's RMS
BAR_OUT_RMS = 1e-2    # per token row: RMS of the error, of the row's RMS
BAR_STATE = 1e-1


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run(mi, theta0=None, eta_scale=None):
    import sequence_models_amd as sm

    wl = mi.workload
    B, H = wl.batch, wl.heads
    th0 = mi.theta0 if theta0 is None else theta0
    th0 = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(th0, (B,) + th0.shape))).cuda()
    s0 = torch.zeros_like(th0)
    print(f"mag_forward B={B} T={wl.seq_len} H={H} widths={wl.widths} C={wl.chunk} "
          f"W={mi.window}", flush=True)
    out, th, s = sm.mag_forward(_bf16(mi.x), _bf16(mi.w_in), torch.from_numpy(mi.b_gate).cuda(),
                                _bf16(mi.w_out), th0, s0, wl.chunk, mi.window, wl.widths,
                                wl.eta_scale if eta_scale is None else eta_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), th.cpu().numpy(), s.cpu().numpy()


def _oracle(mi, b0=0, b1=None, T=None, theta0=None, eta_scale=None):
    wl = mi.workload
    x = S.bf16_bits_to_f32(mi.x[b0:b1, :T]).astype(np.float64)
    th0 = (mi.theta0 if theta0 is None else theta0).astype(np.float64)
    return omag.mag_forward(x, *mi.oracle_weights(), wl.widths, wl.chunk, mi.window,
                            wl.eta_scale if eta_scale is None else eta_scale, th0,
                            np.zeros_like(th0))


def _check_out(got, ref, bar_max=None, bar_rms=None):
    rr = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    err = np.abs(got - ref)
    emax = np.max(err / rr)
    erms = np.max(np.sqrt(np.mean(err ** 2, axis=-1, keepdims=True)) / rr)
    print(f"out: max err / row rms = {emax:.3e}, row rms err / row rms = {erms:.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert emax <= (BAR_OUT_MAX if bar_max is None else bar_max)
    assert erms <= (BAR_OUT_RMS if bar_rms is None else bar_rms)


def _check_state(got, ref, name, bar=BAR_STATE):
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"{name}: relative error {rel:.3e} (bar {bar:.2e})", flush=True)
    assert rel <= bar


SENSITIVITY_FACTOR = 5.0


CASES = [
    # (widths, heads, batch, T, chunk, window): ragged T (several 64-token query blocks and
    # 128-row GEMM tiles plus a tail), windows below, at and beyond T, window 1
    ((64, 256, 64), 2, 2, 200, 64, 48),
    ((64, 256, 64), 3, 1, 131, 16, 131),
    ((64, 128, 64), 2, 1, 77, 8, 1),
    ((32, 64, 32), 3, 2, 130, 16, 500),
    ((32, 32, 32, 32), 4, 1, 96, 32, 17),
    ((128, 128, 128), 1, 2, 70, 8, 33),
    ((64, 256, 64), 2, 1, 1, 64, 16),      # one token
    ((64, 128, 64), 2, 1, 129, 8, 64),     # a window of exactly one key block
]


@pytest.mark.parametrize("widths,H,B,T,C,W", CASES)
def test_mag_matches_oracle(widths, H, B, T, C, W):
    wl = S.WORKLOADS["h16_d64_b8_t16k"].with_(widths=tuple(widths), heads=H, chunk=C)
    mi = S.make_mag_inputs(wl, W, seed=11, seq_len=T, batch=B)
    out, th, s = _run(mi)
    ref, mid = _oracle(mi)
    _check_out(out, ref)
    _check_state(th, mid["theta_T"], "theta_T")
    _check_state(s, mid["s_T"], "s_T")


def test_mag_no_tokens_and_empty_batch():
    import sequence_models_amd as sm

    wl = S.WORKLOADS["h16_d64_b8_t16k"].with_(heads=2)
    mi = S.make_mag_inputs(wl, 16, seed=3, seq_len=0, batch=2)
    out, th, s = _run(mi)
    assert out.shape == (2, 0, 128)
    np.testing.assert_array_equal(th, np.broadcast_to(mi.theta0, th.shape))
    np.testing.assert_array_equal(s, 0.0)
    mi0 = S.make_mag_inputs(wl, 16, seed=3, seq_len=5, batch=0)
    out0, th0, _ = _run(mi0)
    assert out0.shape == (0, 5, 128) and th0.shape == (0, 2, wl.params)
    assert sm.mag_workspace_size(torch.empty(0, 5, 128, dtype=torch.bfloat16), 64, 16,
                                 wl.widths) == 0


def test_mag_rejects_bad_arguments():
    import sequence_models_amd as sm

    wl = S.WORKLOADS["h16_d64_b8_t16k"].with_(heads=2)
    mi = S.make_mag_inputs(wl, 16, seed=3, seq_len=8, batch=1)
    x = _bf16(mi.x)
    th = torch.zeros(1, 2, wl.params, dtype=torch.float32, device="cuda")
    args = (x, _bf16(mi.w_in), torch.from_numpy(mi.b_gate).cuda(), _bf16(mi.w_out), th, th.clone())
    with pytest.raises(sm.TitansError, match="window"):
        sm.mag_forward(*args, 64, 0, wl.widths, 0.1)
    with pytest.raises(sm.TitansError, match="eta_scale"):
        sm.mag_forward(*args, 64, 4, wl.widths, float("nan"))
    with pytest.raises(sm.TitansError, match="overlap"):
        sm.mag_forward(*args, 64, 4, wl.widths, 0.1, theta_T=args[4])


# ---- full size: B = 8, T = 16K, 16 heads of d = 64, 64-256-64 memory, C = 64, W = 4096


@pytest.fixture(scope="module")
def headline():
    # alpha gates centred at sigmoid(-7) instead of sigmoid(-4), so that the memory is still
    # O(1) after 16K tokens (with the default gates it decays below fp32's range)
    wl = S.WORKLOADS["h16_d64_b8_t16k"].with_(alpha_mu=-7.0)
    return S.make_mag_inputs(wl, 4096, seed=0)


def test_mag_full_size_zero_memory_sampled_rows(headline):
    """theta0 = 0 and eta = 0 keep the memory at zero, so y_mem = 0 and the block output is
    (y_attn / 2) W_out exactly; the oracle computes the attention of sampled tokens from
    their windows alone (the window start, the first window-edge tokens, the end)."""
    mi = headline
    wl = mi.workload
    zero = np.zeros_like(mi.theta0)
    out, th, _ = _run(mi, theta0=zero, eta_scale=0.0)
    np.testing.assert_array_equal(th, 0.0)
    Wq, Wk, Wv, Wg, bg, Wo = mi.oracle_weights()
    W = mi.window
    got, ref = [], []
    for b, t in [(0, 0), (0, 63), (3, 4095), (3, 4096), (5, 4160), (6, 9001), (7, 16383)]:
        t0 = max(0, t - W + 1)
        x = S.bf16_bits_to_f32(mi.x[b:b + 1, t0:t + 1]).astype(np.float64)
        q, k, v, *_ = omag.front_end(x, Wq, Wk, Wv, Wg, bg, wl.heads, 0.0)
        # the last token's window is the whole slice: one softmax row per head
        s = np.einsum("hd,jhd->hj", q[0, -1], k[0]) / np.sqrt(wl.d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ya = np.einsum("hj,jhd->hd", p, v[0])
        ref.append((0.5 * ya.reshape(-1)) @ Wo)
        got.append(out[b, t])
    _check_out(np.array(got), np.array(ref))


def test_mag_full_size_prefix_and_final_state(headline):
    """The real memory: the first 128 tokens of two batch rows against the oracle block on
    that prefix, and theta_T / s_T of two memories against the oracle scan over all T of
    the front end's q, k, v at the block's bf16 storage precision."""
    mi = headline
    wl = mi.workload
    out, th, s = _run(mi)
    for b in (0, wl.batch - 1):
        ref, _ = _oracle(mi, b, b + 1, 128)
        _check_out(out[b:b + 1, :128], ref)
    Wq, Wk, Wv, Wg, bg, Wo = mi.oracle_weights()
    for b, h in ((1, 5), (6, 15)):
        x = S.bf16_bits_to_f32(mi.x[b:b + 1]).astype(np.float64)
        d = wl.d
        cols = slice(h * d, (h + 1) * d)
        gcols = [h, wl.heads + h, 2 * wl.heads + h]
        # q, k, v as the block stores them (bf16): over 16K tokens the scan amplifies that
        # rounding alone to a few percent of theta_T
        q, k, v, al, et, be = omag.front_end(x, Wq[:, cols], Wk[:, cols], Wv[:, cols],
                                             Wg[:, gcols], bg[gcols], 1, wl.eta_scale,
                                             store="bf16")
        # and once more on k, v perturbed by one bf16 rounding: the method's own sensitivity
        rng = np.random.default_rng(4321 + h)
        pk, pv = (a * (1.0 + 2.0 ** -9 * rng.uniform(-1.0, 1.0, a.shape)) for a in (k, v))

        def two(a, b_):
            return np.concatenate([a, b_], axis=2)

        th0 = mi.theta0[h:h + 1].astype(np.float64)
        _, th_ref, s_ref = oracle.scan(two(q, q), two(k, pk), two(v, pv), two(al, al),
                                       two(et, et), two(be, be), np.concatenate([th0, th0]),
                                       np.zeros((2, wl.params)), wl.chunk, wl.widths)

        def rel(a, r):
            return np.linalg.norm(a - r) / np.linalg.norm(r)

        kappa = max(rel(th_ref[0, 1], th_ref[0, 0]), rel(s_ref[0, 1], s_ref[0, 0]))
        bar = max(2e-2, SENSITIVITY_FACTOR * kappa)
        print(f"({b},{h}) oracle sensitivity to one bf16 rounding of k, v: {kappa:.2e}", flush=True)
        _check_state(th[b, h], th_ref[0, 0], f"theta_T[{b},{h}]", bar)
        _check_state(s[b, h], s_ref[0, 0], f"s_T[{b},{h}]", bar)
