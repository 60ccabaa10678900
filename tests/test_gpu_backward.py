"""Parity of the reverse pass (titans_mem_scan_backward, through the C ABI) against the
gradient oracle (oracle/scan_grad.py: the scan in fp64 torch, differentiated by autograd).

Every cotangent is compared as a relative Frobenius error per (b, h) slice, maximum over
slices.  Bars: 1e-5 on every cotangent computed and stored in fp32 (all of them for fp32
I/O; the gate and state cotangents for bf16 I/O) -- the reverse pass is fp32 throughout
(inputs, bf16 or not, are exact in fp32; products on the fp32 matrix cores), and its
longest chains, the state cotangents carried over every chunk and the gate cotangents
summed over a chunk's coefficient matrices, stay within a few tens of fp32 ulps (measured
1e-7 to 2e-6, the full-size suffix included).  dq, dk, dv in bf16: 4e-3, the bf16 unit
roundoff 2^-8 (an elementwise round-to-nearest moves a vector by at most that relative
Frobenius distance) plus the fp32 part (measured 1.6e-3 to 1.9e-3).

The full-size case uses two properties that hold at any length (the scan is causal and the
chunks start at token 0): with dy zero after the first T0 tokens (T0 a multiple of C) and
zero state cotangents, every cotangent is that of the T0-token prefix problem (and zero
past T0); and with all cotangents present, the cotangents of the last T1 tokens are those of
the suffix problem started from the state at T - T1, which the C oracle's forward gives.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import sequence_models_amd as tm  # noqa: E402
import synthetic  # noqa: E402
from oracle import scan_grad  # noqa: E402
from tests.helpers import rel_err_slices, to_device, to_f64  # noqa: E402

NAMES = scan_grad.NAMES
AXES = {"q": (1, 3), "k": (1, 3), "v": (1, 3), "alpha": (1,), "eta": (1,), "beta": (1,),
        "theta0": (2,), "s0": (2,)}
BAR = {"f32": 1e-5, "bf16": 1e-5}
BAR_IO_BF16 = 4e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _small(widths=(16, 32, 16), B=2, T=37, H=3, C=8, io="f32", seed=5):
    wl = synthetic.Workload("bwd", B, H, T, tuple(widths), C, io)
    return wl, synthetic.make_inputs(wl, seed), synthetic.make_cotangents(wl, seed)


def _oracle_inputs(inp, theta0=None, s0=None):
    wl = inp.workload
    B = wl.batch
    th0 = inp.theta0 if theta0 is None else theta0
    sg0 = inp.s0 if s0 is None else s0
    if th0.ndim == 2:
        th0 = np.broadcast_to(th0, (B,) + th0.shape)
        sg0 = np.broadcast_to(sg0, (B,) + sg0.shape)
    return {"q": inp.qkv_f32("q"), "k": inp.qkv_f32("k"), "v": inp.qkv_f32("v"),
            "alpha": inp.alpha, "eta": inp.eta, "beta": inp.beta,
            "theta0": np.ascontiguousarray(th0, np.float64),
            "s0": np.ascontiguousarray(sg0, np.float64)}


def _dy_dev(cot, io):
    a = np.ascontiguousarray(cot.dy)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def run_bwd(wl, dev, cot, dstate=True, bias=None, **kw):
    dth = torch.from_numpy(cot.dtheta_T).cuda() if dstate else None
    ds = torch.from_numpy(cot.ds_T).cuda() if dstate else None
    return tm.scan_backward(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                            dev["theta0"], dev["s0"], _dy_dev(cot, wl.io), wl.chunk, wl.widths,
                            dtheta_T=dth, ds_T=ds, bias=bias, **kw)


def compare(wl, got, ref, label, bars=None, names=NAMES):
    worst = {}
    for n in names:
        g = to_f64(got[n])
        e = rel_err_slices(g, ref[n], AXES[n])
        worst[n] = e
    log(f"  {label}: " + " ".join(f"{n} {e:.1e}" for n, e in worst.items()))
    for n, e in worst.items():
        bar = (bars or {}).get(n)
        if bar is None:
            bar = BAR_IO_BF16 if (wl.io == "bf16" and n in ("q", "k", "v")) else BAR[wl.io]
        assert e <= bar, (label, n, e, bar)


@pytest.mark.parametrize("C", [1, 5, 8, 37])
@pytest.mark.parametrize("widths", [(16, 16), (16, 32, 16), (8, 24, 12, 8), (8, 5, 7, 8)])
def test_backward_matches_oracle_fp32(widths, C):
    """P = 131 for (8, 5, 7, 8): the state vectors end in a partial 16-byte group."""
    wl, inp, cot = _small(widths=widths, C=C)
    rng = np.random.default_rng(3)
    inp.s0 = (0.05 * rng.standard_normal(inp.theta0.shape)).astype(np.float32)
    log(f"case backward fp32 {widths} C={C}")
    dev = to_device(inp)
    P = wl.params
    if P % 4:  # state rows must start 16 bytes apart: padded [.., P] views
        pad = lambda a: torch.nn.functional.pad(torch.from_numpy(a).cuda(), (0, 4 - P % 4))[..., :P]
        dev["theta0"], dev["s0"] = pad(inp.theta0), pad(inp.s0)
        dth, dsT = pad(cot.dtheta_T), pad(cot.ds_T)
        got = tm.scan_backward(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"],
                               dev["beta"], dev["theta0"], dev["s0"], _dy_dev(cot, wl.io), C,
                               widths, dtheta_T=dth, ds_T=dsT)
        assert got["theta0"].stride(1) % 4 == 0
    else:
        got = run_bwd(wl, dev, cot)
    torch.cuda.synchronize()
    ref = scan_grad.scan_vjp(_oracle_inputs(inp), C, widths, cot.dy_f32(), cot.dtheta_T,
                             cot.ds_T)
    compare(wl, got, ref, f"{widths} C={C}")


@pytest.mark.parametrize("widths,C,T,B,H", [((16, 32, 16), 8, 45, 2, 2),
                                            ((64, 256, 64), 64, 130, 1, 2),
                                            ((128, 256, 128), 32, 70, 1, 1)])
def test_backward_matches_oracle_bf16(widths, C, T, B, H):
    wl, inp, cot = _small(widths=widths, B=B, T=T, H=H, C=C, io="bf16", seed=T)
    log(f"case backward bf16 {widths} C={C} T={T}")
    got = run_bwd(wl, to_device(inp), cot)
    torch.cuda.synchronize()
    ref = scan_grad.scan_vjp(_oracle_inputs(inp), C, widths, cot.dy_f32(), cot.dtheta_T,
                             cot.ds_T)
    compare(wl, got, ref, f"bf16 {widths} C={C} T={T}")


@pytest.mark.parametrize("widths,C,T", [((16, 32, 16), 128, 300), ((16, 24, 16), 256, 600),
                                        ((16, 40, 24, 32, 16), 16, 70), ((8, 16, 8), 4, 4 * 70)])
def test_backward_long_chunks_deep_memories_and_many_segments(widths, C, T):
    """C = 128 / 256 (partial last chunk), a four-layer memory, and 70 chunks of 4 tokens:
    three segments of the sequential part, so its state products cross launches."""
    wl, inp, cot = _small(widths=widths, B=1, T=T, H=2, C=C, seed=C + T)
    log(f"case backward {widths} C={C} T={T}")
    got = run_bwd(wl, to_device(inp), cot)
    torch.cuda.synchronize()
    ref = scan_grad.scan_vjp(_oracle_inputs(inp), C, widths, cot.dy_f32(), cot.dtheta_T,
                             cot.ds_T)
    compare(wl, got, ref, f"{widths} C={C} T={T}")


@pytest.mark.parametrize("bias", [("huber", 0.5), ("lp", 3.0), ("lp", 2.0)])
def test_backward_attentional_bias(bias):
    wl, inp, cot = _small(widths=(16, 32, 16), C=8, T=40, seed=11)
    log(f"case backward bias {bias}")
    got = run_bwd(wl, to_device(inp), cot, bias=bias)
    torch.cuda.synchronize()
    ref = scan_grad.scan_vjp(_oracle_inputs(inp), wl.chunk, wl.widths, cot.dy_f32(),
                             cot.dtheta_T, cot.ds_T, bias=bias)
    compare(wl, got, ref, f"bias {bias}")
    with pytest.raises(tm.TitansError, match="UNSUPPORTED"):
        run_bwd(wl, to_device(inp), cot, bias=("lp", 1.5))


def test_backward_without_state_cotangents_in_place_and_per_batch_state():
    wl, inp, cot = _small(widths=(16, 32, 16), B=2, T=33, H=3, C=8, seed=2)
    dev = to_device(inp)
    log("case backward: NULL state cotangents, in place, [B,H,P] state")
    got = run_bwd(wl, dev, cot, dstate=False)
    torch.cuda.synchronize()
    zero = np.zeros_like(cot.dtheta_T)
    ref = scan_grad.scan_vjp(_oracle_inputs(inp), wl.chunk, wl.widths, cot.dy_f32(), zero, zero)
    compare(wl, got, ref, "no state cotangents")
    # in place: the state cotangents come in and go out through the same buffers
    rng = np.random.default_rng(4)
    th0 = (0.3 * rng.standard_normal((2, 3, wl.params))).astype(np.float32)
    s0 = (0.05 * rng.standard_normal((2, 3, wl.params))).astype(np.float32)
    dev["theta0"] = torch.from_numpy(th0).cuda()
    dev["s0"] = torch.from_numpy(s0).cuda()
    dth = torch.from_numpy(cot.dtheta_T).cuda()
    ds = torch.from_numpy(cot.ds_T).cuda()
    got = tm.scan_backward(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                           dev["theta0"], dev["s0"], _dy_dev(cot, wl.io), wl.chunk, wl.widths,
                           dtheta_T=dth, ds_T=ds, out={"theta0": dth, "s0": ds})
    torch.cuda.synchronize()
    assert got["theta0"].data_ptr() == dth.data_ptr() and got["s0"].data_ptr() == ds.data_ptr()
    ref = scan_grad.scan_vjp(_oracle_inputs(inp, th0, s0), wl.chunk, wl.widths, cot.dy_f32(),
                             cot.dtheta_T, cot.ds_T)
    compare(wl, got, ref, "in place, per-batch state")


def test_backward_strided_inputs():
    wl, inp, cot = _small(widths=(16, 32, 16), B=2, T=29, H=2, C=8, seed=8)
    dev = to_device(inp)
    log("case backward strided q/k/v and gates")
    packed = torch.stack([dev["q"], dev["k"], dev["v"]], dim=3)  # [B,T,H,3,d]
    g = torch.stack([dev["alpha"], dev["eta"], dev["beta"]], dim=-1)
    sd = {"q": packed[:, :, :, 0], "k": packed[:, :, :, 1], "v": packed[:, :, :, 2],
          "alpha": g[..., 0], "eta": g[..., 1], "beta": g[..., 2],
          "theta0": dev["theta0"], "s0": dev["s0"]}
    got = run_bwd(wl, sd, cot)
    torch.cuda.synchronize()
    assert got["q"].stride() == sd["q"].stride() and got["alpha"].stride() == sd["alpha"].stride()
    ref = scan_grad.scan_vjp(_oracle_inputs(inp), wl.chunk, wl.widths, cot.dy_f32(),
                             cot.dtheta_T, cot.ds_T)
    compare(wl, got, ref, "strided")


def test_backward_empty_sequence_passes_state_cotangents_through():
    wl, inp, cot = _small(T=0)
    dev = to_device(inp)
    log("case backward T=0")
    got = run_bwd(wl, dev, cot)
    torch.cuda.synchronize()
    assert torch.equal(got["theta0"].cpu(), torch.from_numpy(cot.dtheta_T))
    assert torch.equal(got["s0"].cpu(), torch.from_numpy(cot.ds_T))
    got = run_bwd(wl, dev, cot, dstate=False)
    torch.cuda.synchronize()
    assert not got["theta0"].any() and not got["s0"].any()


def test_backward_headline_shape_full_size_prefix_and_suffix():
    """The 16-head, d = 64, 64-256-64, C = 64, T = 16384, batch 8 shape at full size (the
    launch the bench times), checked through the prefix and suffix properties on sampled
    memories; the suffix references must be far from zero for the check to mean anything."""
    # the sustained gate mix (alpha = sigmoid(N(-7, 1))): with the workload's own gates the
    # memory decays to ~0 long before T = 16384 and the suffix cotangents would be ~0 too
    wl = synthetic.WORKLOADS["h16_d64_b8_t16k"].with_(alpha_mu=-7.0, name="h16_d64_b8_t16k_sustained")
    inp = synthetic.make_inputs(wl, 0)
    cot = synthetic.make_cotangents(wl, 0)
    dev = to_device(inp)
    T, C = wl.seq_len, wl.chunk
    T0, T1 = 256, 128
    pairs = [(0, 0), (5, 11)]
    # prefix: dy zero past T0, no state cotangents
    dy = _dy_dev(cot, wl.io).clone()
    dy[:, T0:] = 0
    log("case backward headline full size: prefix")
    got = tm.scan_backward(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                           dev["theta0"], dev["s0"], dy, C, wl.widths)
    torch.cuda.synchronize()
    # one memory of this draw, (b, h) = (0, 4), diverges under the sustained gates in the
    # fp64 oracle as well (its state overflows within the first thousand tokens); the
    # exact-zero property is checked on every memory whose forward stays finite
    _, thT, _ = tm.scan(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                        dev["theta0"], dev["s0"], C, wl.widths)
    torch.cuda.synchronize()
    finite = torch.isfinite(thT).all(dim=-1)  # [B, H]
    assert all(bool(finite[b, h]) for b, h in pairs)
    assert int(finite.sum()) >= finite.numel() - 2
    for n in NAMES[:6]:
        past = got[n][:, T0:]
        assert not past.transpose(1, 2)[finite].any(), n
    zero = np.zeros((1, len(pairs), wl.params))
    ref = scan_grad.scan_vjp(_gather(inp, pairs, 0, T0), C, wl.widths,
                             _gather_dy(cot, pairs, 0, T0), zero, zero)
    compare(wl, _pick(got, pairs, 0, T0), ref, "prefix T0=256")
    # suffix: all cotangents; the last T1 tokens from the state at T - T1
    log("case backward headline full size: suffix")
    got = run_bwd(wl, dev, cot)
    torch.cuda.synchronize()
    start = T - T1
    assert start % C == 0
    suf = _gather(inp, pairs, start, T)
    suf["theta0"], suf["s0"] = _oracle_state(inp, pairs, start)
    dth = np.stack([cot.dtheta_T[b, h] for b, h in pairs])[None]
    dsT = np.stack([cot.ds_T[b, h] for b, h in pairs])[None]
    ref = scan_grad.scan_vjp(suf, C, wl.widths, _gather_dy(cot, pairs, start, T), dth, dsT)
    for n in NAMES[:6]:
        assert np.sqrt(np.mean(ref[n] ** 2)) > 1e-3, (n, "suffix reference has decayed")
    compare(wl, _pick(got, pairs, start, T), ref, f"suffix T1={T1}", names=NAMES[:6])


def _pick(got, pairs, t0, t1):
    """The sampled memories of full-size outputs, laid out as the oracle's [1, T, npairs, ...]."""
    sub = {n: torch.stack([got[n][b, t0:t1, h] for b, h in pairs], dim=1)[None]
           for n in NAMES[:6]}
    for n in ("theta0", "s0"):
        sub[n] = torch.stack([got[n][b, h] for b, h in pairs])[None]
    return sub


def _gather(inp, pairs, t0, t1):
    def g(a):
        return np.stack([a[b, t0:t1, h] for b, h in pairs], axis=1)[None].astype(np.float64)

    out = {n: g(inp.qkv_f32(n)) for n in ("q", "k", "v")}
    for n in ("alpha", "eta", "beta"):
        out[n] = g(getattr(inp, n))
    out["theta0"] = np.stack([inp.theta0[h] for _, h in pairs])[None].astype(np.float64)
    out["s0"] = np.stack([inp.s0[h] for _, h in pairs])[None].astype(np.float64)
    return out


def _gather_dy(cot, pairs, t0, t1):
    dy = cot.dy_f32()
    return np.stack([dy[b, t0:t1, h] for b, h in pairs], axis=1)[None].astype(np.float64)


def _oracle_state(inp, pairs, T):
    g = _gather(inp, pairs, 0, T)
    _, th, s = oracle.scan(g["q"], g["k"], g["v"], g["alpha"], g["eta"], g["beta"],
                           g["theta0"], g["s0"], inp.workload.chunk, inp.workload.widths)
    return th, s
