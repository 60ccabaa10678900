"""The MAG / MAC oracle pins reject plausible mistakes.

Each case plants one mistake in the block oracles (oracle/mag.py, oracle/mac.py), on the
CPU, and checks that at least one pin of tests/test_oracle_mag_pins.py or
tests/test_oracle_mac_pins.py then fails.
"""
import numpy as np
import pytest

import oracle
from oracle import mac, mag
from tests import test_oracle_mac_pins as mac_pins
from tests import test_oracle_mag_pins as mag_pins


def _window_off_by_one(q, k, v, window):
    """The window one token too long (keys t - window .. t)."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    out = np.zeros_like(q)
    d = q.shape[-1]
    for t in range(q.shape[1]):
        j0 = max(0, t - window)
        s = np.einsum("bhd,bjhd->bhj", q[:, t], k[:, j0:t + 1]) / np.sqrt(d)
        p = np.exp(s - s.max(-1, keepdims=True))
        out[:, t] = np.einsum("bhj,bjhd->bhd", p / p.sum(-1, keepdims=True), v[:, j0:t + 1])
    return out


def _no_scale(q, k, v, window):
    """Scores without the 1 / sqrt(d)."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    out = np.zeros_like(q)
    for t in range(q.shape[1]):
        j0 = max(0, t - window + 1)
        s = np.einsum("bhd,bjhd->bhj", q[:, t], k[:, j0:t + 1])
        p = np.exp(s - s.max(-1, keepdims=True))
        out[:, t] = np.einsum("bhj,bjhd->bhd", p / p.sum(-1, keepdims=True), v[:, j0:t + 1])
    return out


def _causal_prefix(q, k, v, h):
    """Memory reads masked causally (h_u only for u <= t)."""
    q, k, v, h = (np.asarray(a, np.float64) for a in (q, k, v, h))
    out = np.zeros_like(q)
    d = q.shape[-1]
    for t in range(q.shape[1]):
        keys = np.concatenate([h[:, :t + 1], k[:, :t + 1]], axis=1)
        vals = np.concatenate([h[:, :t + 1], v[:, :t + 1]], axis=1)
        s = np.einsum("bhd,bjhd->bhj", q[:, t], keys) / np.sqrt(d)
        p = np.exp(s - s.max(-1, keepdims=True))
        out[:, t] = np.einsum("bhj,bjhd->bhd", p / p.sum(-1, keepdims=True), vals)
    return out


def _mac_reads_after_write(x, Wq, Wk, Wv, Wg, bg, Wo, widths, chunk, segment, eta_scale,
                           theta0, s0, store=None):
    """MAC with each segment reading the memory after its own writes."""
    x = np.asarray(x, np.float64)
    B, T, D = x.shape
    H = D // widths[0]
    q, k, v, al, et, be = mag.front_end(x, Wq, Wk, Wv, Wg, bg, H, eta_scale, store=store)
    th = np.broadcast_to(np.asarray(theta0, np.float64), (B,) + np.shape(theta0)[-2:]).copy()
    s = np.broadcast_to(np.asarray(s0, np.float64), th.shape).copy()
    h_all, y = np.zeros_like(q), np.zeros_like(q)
    for t0 in range(0, T, segment):
        sl = slice(t0, min(T, t0 + segment))
        _, th, s = oracle.scan(q[:, sl], k[:, sl], v[:, sl], al[:, sl], et[:, sl], be[:, sl], th,
                               s, chunk, widths)
        h_all[:, sl] = oracle.retrieve(q[:, sl], th, widths)
        y[:, sl] = mac.prefix_attention(q[:, sl], k[:, sl], v[:, sl], h_all[:, sl])
    return y.reshape(B, T, D) @ Wo, {"q": q, "k": k, "v": v, "alpha": al, "eta": et,
                                     "beta": be, "h": h_all, "y_attn": y, "theta_T": th, "s_T": s}


def _pins_fail(pins):
    """True if at least one of the pin functions raises an AssertionError."""
    for pin in pins:
        try:
            pin()
        except AssertionError:
            return True
    return False


MAG_PINS = [mag_pins.test_full_window_equals_library_causal_attention,
            mag_pins.test_window_one_and_window_locality,
            mag_pins.test_zero_memory_halves_the_attention_output,
            mag_pins.test_front_end_on_unit_rows_and_memory_branch]
MAC_PINS = [mac_pins.test_prefix_attention_equals_library_masked_attention,
            mac_pins.test_zero_memory_closed_form,
            mac_pins.test_one_segment_and_streaming_state]


def test_unplanted_pins_pass():
    assert not _pins_fail(MAG_PINS) and not _pins_fail(MAC_PINS)


@pytest.mark.parametrize("name", ["window_off_by_one", "no_score_scale", "gate_not_sigmoid",
                                  "q_not_normalized"])
def test_mag_pins_reject_planted_mistake(name, monkeypatch):
    if name == "window_off_by_one":
        monkeypatch.setattr(mag, "sliding_window_attention", _window_off_by_one)
    elif name == "no_score_scale":
        monkeypatch.setattr(mag, "sliding_window_attention", _no_scale)
    elif name == "gate_not_sigmoid":
        monkeypatch.setattr(mag, "_sigmoid", np.tanh)
    else:
        front = mag.front_end

        def unnormalized(x, Wq, Wk, Wv, Wg, bg, H, eta_scale, store=None):
            q, k, v, al, et, be = front(x, Wq, Wk, Wv, Wg, bg, H, eta_scale, store)
            B, T, _ = np.shape(x)
            return ((np.asarray(x, np.float64) @ Wq).reshape(B, T, H, -1), k, v, al, et, be)

        monkeypatch.setattr(mag, "front_end", unnormalized)
    assert _pins_fail(MAG_PINS), name


@pytest.mark.parametrize("name", ["causal_reads", "reads_after_write"])
def test_mac_pins_reject_planted_mistake(name, monkeypatch):
    if name == "causal_reads":
        monkeypatch.setattr(mac, "prefix_attention", _causal_prefix)
    else:
        monkeypatch.setattr(mac, "mac_forward", _mac_reads_after_write)
    assert _pins_fail(MAC_PINS), name
