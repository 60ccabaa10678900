"""GPU parity of the MAC block (titans_mac_forward) against the fp64 oracle (oracle/mac.py).

Same inputs and bars as the MAG block (tests/test_gpu_mag.py): the output per token row
relative to the row's RMS (3e-2 per element, 1e-2 per row RMS), the memory state with the
scan's bf16 bar (1e-1); the memory reads h are stored in bf16 like y_mem there.

Rows of a later segment read the memory as the scan left it after thousands of tokens: that
state carries the scan's own bf16 error (bar 1e-1, a few percent measured), and the
segment's reads (a prefix as long as the segment) take about half of each query's attention
weight, so those rows get the state's bar scaled by that weight: 1e-1 per element and 5e-2
per row RMS.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from oracle import mac as omac
from oracle import mag as omag
from tests.test_gpu_mag import _bf16, _check_out, _check_state

pytestmark = pytest.mark.gpu

BAR_LATE_MAX = 1e-1   # rows of a later segment, per element (of the row's RMS)
BAR_LATE_RMS = 5e-2   # rows of a later segment, per row RMS


def _run(mi, segment):
    import sequence_models_amd as sm

    wl = mi.workload
    B = wl.batch
    th0 = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(mi.theta0, (B,) + mi.theta0.shape))).cuda()
    print(f"mac_forward B={B} T={wl.seq_len} H={wl.heads} widths={wl.widths} C={wl.chunk} "
          f"S={segment}", flush=True)
    out, th, s = sm.mac_forward(_bf16(mi.x), _bf16(mi.w_in), torch.from_numpy(mi.b_gate).cuda(),
                                _bf16(mi.w_out), th0, torch.zeros_like(th0), wl.chunk, segment,
                                wl.widths, wl.eta_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), th.cpu().numpy(), s.cpu().numpy()


CASES = [
    # (widths, heads, batch, T, chunk, segment): several segments with a shorter last one,
    # one segment, one-token segments, D not a multiple of 64, d = 128
    ((64, 256, 64), 2, 2, 200, 64, 128),
    ((64, 256, 64), 3, 1, 131, 16, 48),
    ((64, 128, 64), 2, 1, 77, 8, 1000),
    ((64, 128, 64), 2, 1, 12, 1, 1),
    ((32, 64, 32), 3, 2, 130, 16, 64),
    ((128, 128, 128), 1, 2, 70, 8, 32),
    ((64, 256, 64), 2, 1, 1, 64, 64),      # one token
    ((64, 128, 64), 2, 1, 129, 8, 64),     # segments of one key block, a one-token last one
]


@pytest.mark.parametrize("widths,H,B,T,C,Sg", CASES)
def test_mac_matches_oracle(widths, H, B, T, C, Sg):
    wl = S.WORKLOADS["h16_d64_b8_t16k"].with_(widths=tuple(widths), heads=H, chunk=C)
    mi = S.make_mag_inputs(wl, 0, seed=13, seq_len=T, batch=B)
    out, th, s = _run(mi, Sg)
    x = S.bf16_bits_to_f32(mi.x).astype(np.float64)
    ref, mid = omac.mac_forward(x, *mi.oracle_weights(), wl.widths, C, Sg, wl.eta_scale,
                                mi.theta0.astype(np.float64), np.zeros(mi.theta0.shape))
    _check_out(out, ref)
    _check_state(th, mid["theta_T"], "theta_T")
    _check_state(s, mid["s_T"], "s_T")


def test_mac_no_tokens_and_empty_batch():
    wl = S.WORKLOADS["h16_d64_b8_t16k"].with_(heads=2)
    mi = S.make_mag_inputs(wl, 0, seed=3, seq_len=0, batch=2)
    out, th, s = _run(mi, 64)
    assert out.shape == (2, 0, 128)
    np.testing.assert_array_equal(th, np.broadcast_to(mi.theta0, th.shape))
    np.testing.assert_array_equal(s, 0.0)
    out0, th0, _ = _run(S.make_mag_inputs(wl, 0, seed=3, seq_len=5, batch=0), 64)
    assert out0.shape == (0, 5, 128) and th0.shape == (0, 2, wl.params)


# ---- full size: B = 8, T = 16K, 16 heads of d = 64, 64-256-64 memory, C = 64, S = 4096


def test_mac_full_size_sampled_rows_and_state():
    """Sampled rows of the first two segments (the second reads the memory after 4096
    tokens, computed by the oracle scan from the front end's q, k, v at bf16 storage) and
    theta_T / s_T of two memories over all 16K tokens.  Gates centred at sigmoid(-7) keep
    the memory O(1) to the end."""
    Sg = 4096
    wl = S.WORKLOADS["h16_d64_b8_t16k"].with_(alpha_mu=-7.0)
    mi = S.make_mag_inputs(wl, 0, seed=0)
    out, th, s = _run(mi, Sg)
    Wq, Wk, Wv, Wg, bg, Wo = mi.oracle_weights()
    H, d = wl.heads, wl.d
    P = wl.params
    for b, ts in ((2, (0, 77, 4095)), (5, (4096, 4200, 8191))):
        seg0 = ts[0] // Sg * Sg
        x = S.bf16_bits_to_f32(mi.x[b:b + 1, :seg0 + Sg]).astype(np.float64)
        q, k, v, al, et, be = omag.front_end(x, Wq, Wk, Wv, Wg, bg, H, wl.eta_scale, store="bf16")
        th_seg = np.broadcast_to(mi.theta0.astype(np.float64), (1, H, P))
        if seg0:
            _, th_seg, _ = oracle.scan(q[:, :seg0], k[:, :seg0], v[:, :seg0], al[:, :seg0],
                                       et[:, :seg0], be[:, :seg0], th_seg, np.zeros((1, H, P)),
                                       wl.chunk, wl.widths)
        sl = slice(seg0, seg0 + Sg)
        h = omag.round_bf16(oracle.retrieve(q[:, sl], th_seg, wl.widths))
        got, ref = [], []
        for t in ts:
            tl = t - seg0
            keys = np.concatenate([h[0], k[0, sl][:tl + 1]], axis=0)
            vals = np.concatenate([h[0], v[0, sl][:tl + 1]], axis=0)
            sc = np.einsum("hd,jhd->hj", q[0, t], keys) / np.sqrt(d)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            ref.append(np.einsum("hj,jhd->hd", p, vals).reshape(-1) @ Wo)
            got.append(out[b, t])
        if seg0:
            _check_out(np.array(got), np.array(ref), BAR_LATE_MAX, BAR_LATE_RMS)
        else:
            _check_out(np.array(got), np.array(ref))
    for b, h in ((1, 5), (6, 15)):
        x = S.bf16_bits_to_f32(mi.x[b:b + 1]).astype(np.float64)
        cols = slice(h * d, (h + 1) * d)
        gcols = [h, H + h, 2 * H + h]
        q, k, v, al, et, be = omag.front_end(x, Wq[:, cols], Wk[:, cols], Wv[:, cols],
                                             Wg[:, gcols], bg[gcols], 1, wl.eta_scale,
                                             store="bf16")
        _, th_ref, s_ref = oracle.scan(q, k, v, al, et, be, mi.theta0[h:h + 1].astype(np.float64),
                                       np.zeros((1, P)), wl.chunk, wl.widths)
        _check_state(th[b, h], th_ref.reshape(-1), f"theta_T[{b},{h}]")
        _check_state(s[b, h], s_ref.reshape(-1), f"s_T[{b},{h}]")


def test_mac_full_size_zero_memory_late_segments():
    """theta0 = 0 keeps the memory at zero (a bias-free MLP reads 0 and its gradient at 0
    vanishes), so every segment's reads are zero and a query of segment i at offset u sees
    L zero entries plus its own keys: y = sum_{u' <= u} e^{s} v / (L + sum e^{s}).  Rows of
    the last three segments are checked with the storage-only bars."""
    Sg = 4096
    wl = S.WORKLOADS["h16_d64_b8_t16k"]
    mi = S.make_mag_inputs(wl, 0, seed=4)
    zero = np.zeros_like(mi.theta0)
    import sequence_models_amd as sm

    B = wl.batch
    th0 = torch.zeros((B,) + zero.shape, dtype=torch.float32, device="cuda")
    print("mac_forward zero memory, full size", flush=True)
    out, th, _ = sm.mac_forward(_bf16(mi.x), _bf16(mi.w_in), torch.from_numpy(mi.b_gate).cuda(),
                                _bf16(mi.w_out), th0, torch.zeros_like(th0), wl.chunk, Sg,
                                wl.widths, wl.eta_scale)
    torch.cuda.synchronize()
    assert torch.count_nonzero(th).item() == 0
    out = out.float().cpu().numpy()
    Wq, Wk, Wv, Wg, bg, Wo = mi.oracle_weights()
    H, d = wl.heads, wl.d
    got, ref = [], []
    for b, t in ((0, 4096), (1, 6000), (3, 8191), (4, 8192), (6, 12345), (7, 16383)):
        seg0 = t // Sg * Sg
        x = S.bf16_bits_to_f32(mi.x[b:b + 1, seg0:t + 1]).astype(np.float64)
        q, k, v, *_ = omag.front_end(x, Wq, Wk, Wv, Wg, bg, H, 0.0)
        e = np.exp(np.einsum("hd,jhd->hj", q[0, -1], k[0]) / np.sqrt(d))
        y = np.einsum("hj,jhd->hd", e, v[0]) / (Sg + e.sum(axis=1))[:, None]
        ref.append(y.reshape(-1) @ Wo)
        got.append(out[b, t])
    _check_out(np.array(got), np.array(ref))
