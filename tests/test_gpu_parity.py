"""Parity of the HIP scan / retrieve (through the C ABI) against the fp64 oracle.

Bars: fp32 I/O -- relative error <= 1e-4 on y and theta_T; bf16 q/k/v with
fp32 state -- <= 2e-2 on y and <= 1e-1 on theta_T and s_T (relative Frobenius
error per (b, h), maximum over (b, h)).  The bf16 state bar is derived from the
arithmetic of the fused kernel: every per-chunk increment of theta and s is a
sum of products of bf16-rounded operands (unit roundoff 2^-9, cancellation over
64-wide sums), and a CPU emulation of exactly those rounding points gives
1-6e-2 on the state at these sequence lengths while y stays near 5e-3.  Full-size workloads run at their full shape on
the GPU, in the launch configuration the bench times; the oracle then checks
sampled sequences (whole or a prefix: the scan is causal, so a prefix of y
depends only on the prefix of the inputs).
"""
import os
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
from tests.helpers import state_rel_err, to_device, to_f64, y_rel_err  # noqa: E402

Y_BAR = {"f32": 1e-4, "bf16": 2e-2}
TH_BAR = {"f32": 1e-4, "bf16": 1e-1}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(dev, wl, **kw):
    return tm.scan(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                   dev["theta0"], dev["s0"], wl.chunk, wl.widths, **kw)


def oracle_seq(inp, pairs, T=None, theta0=None, s0=None, bias=None):
    """Oracle on the (b, h) pairs (prefix T), all pairs in one OpenMP-parallel call.
    Returns a list of (y [T,d], theta_T [P], s_T [P])."""
    wl = inp.workload
    T = wl.seq_len if T is None else T
    bs = [b for b, _ in pairs]
    hs = [h for _, h in pairs]

    def gather(a):
        return np.stack([a[b, :T, h] for b, h in pairs], axis=1)[None]  # [1,T,n,...]

    qkv = [gather(inp.qkv_f32(n)) for n in ("q", "k", "v")]
    gates = [gather(getattr(inp, n)) for n in ("alpha", "eta", "beta")]
    th0 = (inp.theta0 if theta0 is None else theta0)[hs]
    sg0 = (inp.s0 if s0 is None else s0)[hs]
    y, th, s = oracle.scan(*qkv, *gates, th0, sg0, wl.chunk, wl.widths, bias=bias)
    del bs
    return [(y[0, :, i], th[0, i], s[0, i]) for i in range(len(pairs))]


def check_pairs(wl, y, thT, sT, pairs, refs, T=None, check_state=True):
    yg = to_f64(y)
    tg = to_f64(thT)
    sg = to_f64(sT)
    for (b, h), (yr, tr, sr) in zip(pairs, refs):
        Tn = yr.shape[0]
        ey = y_rel_err(yg[b:b + 1, :Tn, h:h + 1], yr[None, :, None])
        msg = f"{wl.name} (b={b},h={h}) T={Tn}: y rel err {ey:.2e}"
        if check_state:
            et = state_rel_err(tg[b:b + 1, h:h + 1], tr[None, None])
            es = state_rel_err(sg[b:b + 1, h:h + 1], sr[None, None])
            msg += f", theta_T {et:.2e}, s_T {es:.2e}"
        log(msg)
        assert ey <= Y_BAR[wl.io], msg
        if check_state:
            assert et <= TH_BAR[wl.io], msg
            assert es <= TH_BAR[wl.io], msg


# ---------------------------------------------------------------- workloads
#
# With the specified gates (alpha ~ 0.028 per token) and i.i.d. random q/k/v the
# memory decays to its zero fixed point within a few thousand tokens, so at full
# length theta_T and late y are ~0 in both the oracle and the GPU.  Each full shape is
# therefore also run with a "sustained" gate mix (alpha_t = sigmoid(N(mu, 1)) with mu = -7,
# or -8 for the deep memory) where the memory stays O(1) to the end of the sequence.  With
# C = 256 the frozen-gradient steps of a chunk add up: eta = 0.1 sigmoid(.) then diverges in
# the oracle itself, so that shape uses mu = -10 and eta = 0.02 sigmoid(.).

SUSTAINED = {"h8_d64_b4_t4k": (-7.0, 0.1), "h16_d64_b8_t16k": (-7.0, 0.1),
             "deep_h8_d128_b2_t32k": (-8.0, 0.05), "long_h16_d64_b1_t2m": (-10.0, 0.02)}


def _workload(name, sustained):
    wl = synthetic.WORKLOADS[name]
    if not sustained:
        return wl
    mu, es = SUSTAINED[name]
    return wl.with_(alpha_mu=mu, eta_scale=es, name=wl.name + "_sustained")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_fp32_full(seed):
    wl = synthetic.WORKLOADS["tiny_f32_h1_t512"]
    inp = synthetic.make_inputs(wl, seed)
    log(f"case tiny_f32 seed={seed}")
    dev = to_device(inp)
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    yr, tr, sr = oracle.scan(inp.q, inp.k, inp.v, inp.alpha, inp.eta, inp.beta, inp.theta0, inp.s0,
                             wl.chunk, wl.widths)
    ey, et, es = y_rel_err(to_f64(y), yr), state_rel_err(to_f64(thT), tr), state_rel_err(to_f64(sT), sr)
    log(f"tiny_f32 seed={seed}: y {ey:.2e} theta_T {et:.2e} s_T {es:.2e}")
    assert ey <= 1e-4 and et <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("sustained", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_h8_t4k_sampled(seed, sustained):
    wl = _workload("h8_d64_b4_t4k", sustained)
    inp = synthetic.make_inputs(wl, seed)
    log(f"case {wl.name} seed={seed}")
    y, thT, sT = run_gpu(to_device(inp), wl)
    torch.cuda.synchronize()
    pairs = [(0, 0), (3, 7), (1, 4)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs))


@pytest.mark.parametrize("sustained", [False, True])
def test_headline_sampled(sustained):
    wl = _workload(synthetic.HEADLINE, sustained)
    inp = synthetic.make_inputs(wl, 0)
    log(f"case {wl.name} seed=0")
    y, thT, sT = run_gpu(to_device(inp), wl)
    torch.cuda.synchronize()
    full = [(0, 0), (7, 15)]
    check_pairs(wl, y, thT, sT, full, oracle_seq(inp, full))
    prefix = [(3, 5), (5, 11), (6, 2)]
    check_pairs(wl, y, thT, sT, prefix, oracle_seq(inp, prefix, T=1024), check_state=False)
    # the state after 512 tokens, while it is still O(1) for the specified gates
    pre = synthetic.make_inputs(wl, 0, seq_len=512)
    yp, tp, sp = run_gpu(to_device(pre), pre.workload)
    torch.cuda.synchronize()
    pairs = [(2, 3), (4, 12)]
    check_pairs(pre.workload, yp, tp, sp, pairs, oracle_seq(pre, pairs))


@pytest.mark.parametrize("sustained", [False, True])
def test_deep_memory_prefix_and_state(sustained):
    wl = _workload("deep_h8_d128_b2_t32k", sustained)
    inp = synthetic.make_inputs(wl, 0)
    log(f"case {wl.name} full size seed=0")
    dev = to_device(inp)
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 7)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs, T=512), check_state=False)
    # theta after a 768-token prefix (6 chunks), on the GPU alone vs the oracle
    pre = synthetic.make_inputs(wl, 0, seq_len=768)
    yp, tp, sp = run_gpu(to_device(pre), pre.workload)
    torch.cuda.synchronize()
    pairs = [(0, 3), (1, 6)]
    check_pairs(pre.workload, yp, tp, sp, pairs, oracle_seq(pre, pairs))


@pytest.mark.parametrize("sustained", [False, True])
def test_long_context_prefix_64k(sustained):
    wl = _workload("long_h16_d64_b1_t2m", sustained)
    inp = synthetic.make_inputs(wl, 0, seq_len=65536)
    log(f"case {wl.name} 64K prefix seed=0")
    y, thT, sT = run_gpu(to_device(inp), inp.workload)
    torch.cuda.synchronize()
    pairs = [(0, 0), (0, 9)]
    check_pairs(inp.workload, y, thT, sT, pairs, oracle_seq(inp, pairs))


# -------------------------------------------------------------- edge cases

def _small(widths=(16, 32, 16), B=2, T=37, H=3, C=8, io="f32", seed=5):
    wl = synthetic.Workload("edge", B, H, T, tuple(widths), C, io)
    return wl, synthetic.make_inputs(wl, seed)


GENERIC_MODES = ["single", "phased"]


@pytest.mark.parametrize("mode", GENERIC_MODES)
@pytest.mark.parametrize("C", [1, 2, 5, 8, 37, 64])
@pytest.mark.parametrize("widths", [(16, 16), (16, 32, 16), (8, 24, 12, 8), (16, 40, 24, 32, 16)])
def test_chunk_sizes_and_depths_fp32(C, widths, mode, monkeypatch):
    """The generic family with fp32 I/O: one workgroup per memory, and the chain of
    GPU-wide launches (forced here; it normally serves layers of 128 units or more)."""
    monkeypatch.setenv("TITANS_MEM_GENERIC_MODE", mode)
    wl, inp = _small(widths=widths, C=C)
    log(f"case edge {mode} C={C} widths={widths}")
    assert tm.scan_path(torch.empty(1, 1, 1, widths[0], dtype=torch.float32).cuda(), C, widths) == (
        "generic_fp32" if mode == "single" else "phased_fp32")
    rng = np.random.default_rng(3)
    s0 = (0.05 * rng.standard_normal(inp.theta0.shape)).astype(np.float32)
    inp.s0 = s0
    y, thT, sT = run_gpu(to_device(inp), wl)
    torch.cuda.synchronize()
    yr, tr, sr = oracle.scan(inp.q, inp.k, inp.v, inp.alpha, inp.eta, inp.beta, inp.theta0, s0,
                             C, widths)
    ey, et, es = y_rel_err(to_f64(y), yr), state_rel_err(to_f64(thT), tr), state_rel_err(to_f64(sT), sr)
    log(f"  y {ey:.2e} theta_T {et:.2e} s_T {es:.2e}")
    assert ey <= 1e-4 and et <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("mode", GENERIC_MODES)
@pytest.mark.parametrize("C", [1, 5, 37, 64, 128])
@pytest.mark.parametrize("widths", [(16, 16), (16, 32, 16), (8, 24, 12, 8), (16, 40, 24, 32, 16)])
def test_chunk_sizes_and_depths_bf16_generic(C, widths, mode, monkeypatch):
    """Shapes outside the fused kernels with bf16 I/O: the generic family on bf16 MFMA."""
    monkeypatch.setenv("TITANS_MEM_GENERIC_MODE", mode)
    wl, inp = _small(widths=widths, B=2, T=150, H=3, C=C, io="bf16", seed=C)
    dev = to_device(inp)
    log(f"case bf16 generic {mode} {widths} C={C}")
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == (
        "generic_mfma" if mode == "single" else "phased_mfma")
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 2)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("widths,C,T", [((32, 160, 96, 32), 100, 230), ((128, 128), 70, 150),
                                        ((64, 200, 64), 64, 129),
                                        ((128, 512, 512, 512, 128), 128, 300),
                                        ((128, 512, 128), 256, 600),
                                        ((64, 384, 136, 64), 193, 420)])
def test_phased_wide_memories(widths, C, T, io):
    """Layers of 128+ units run as the chain of GPU-wide launches by default: ragged
    64-wide tiles in every dimension, L = 1, 2, 3, 4, partial last chunks."""
    wl, inp = _small(widths=widths, B=2, T=T, H=2, C=C, io=io, seed=T)
    rng = np.random.default_rng(7)
    inp.s0 = (0.05 * rng.standard_normal(inp.theta0.shape)).astype(np.float32)
    dev = to_device(inp)
    log(f"case phased {io} {widths} C={C} T={T}")
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == (
        "phased_mfma" if io == "bf16" else "phased_fp32")
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    pairs = [(0, 1), (1, 0)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs))


def test_bf16_small_ragged():
    wl, inp = _small(widths=(64, 256, 64), B=1, T=200, H=2, C=64, io="bf16")
    log("case bf16 ragged T=200 C=64")
    y, thT, sT = run_gpu(to_device(inp), wl)
    torch.cuda.synchronize()
    pairs = [(0, 0), (0, 1)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs))


def test_empty_and_degenerate():
    wl, inp = _small(T=0)
    dev = to_device(inp)
    log("case T=0")
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    assert y.shape[1] == 0
    assert torch.equal(thT[0], dev["theta0"]) and torch.equal(thT[1], dev["theta0"])
    assert torch.equal(sT[1], dev["s0"])
    wl, inp = _small(B=0)
    dev = to_device(inp)
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    assert thT.shape[0] == 0


def test_streaming_chain_and_inplace_and_determinism():
    wl, inp = _small(T=40, C=8)
    dev = to_device(inp)
    log("case streaming / in-place / determinism")
    y, thT, sT = run_gpu(dev, wl)
    y2, thT2, sT2 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(thT, thT2) and torch.equal(sT, sT2)
    # two calls, the second continuing in place from the first's state
    B, H = wl.batch, wl.heads
    th = dev["theta0"].expand(B, -1, -1).contiguous()
    s = dev["s0"].expand(B, -1, -1).contiguous()
    half = {n: dev[n][:, :24] for n in ("q", "k", "v", "alpha", "eta", "beta")}
    rest = {n: dev[n][:, 24:] for n in ("q", "k", "v", "alpha", "eta", "beta")}
    ya, _, _ = tm.scan(half["q"], half["k"], half["v"], half["alpha"], half["eta"], half["beta"],
                       th, s, wl.chunk, wl.widths, theta_T=th, s_T=s)
    yb, _, _ = tm.scan(rest["q"], rest["k"], rest["v"], rest["alpha"], rest["eta"], rest["beta"],
                       th, s, wl.chunk, wl.widths, theta_T=th, s_T=s)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([ya, yb], dim=1), y)
    assert torch.equal(th, thT) and torch.equal(s, sT)


def test_strided_inputs_and_per_batch_state():
    wl, inp = _small(B=2, T=33, H=3, C=8)
    dev = to_device(inp)
    log("case strided q/k/v and [B,H,P] state")
    B, T, H, d = dev["q"].shape
    packed = torch.stack([dev["q"], dev["k"], dev["v"]], dim=3)  # [B,T,H,3,d]
    q, k, v = packed[:, :, :, 0], packed[:, :, :, 1], packed[:, :, :, 2]
    g = torch.stack([dev["alpha"], dev["eta"], dev["beta"]], dim=-1)  # [B,T,H,3]
    rng = np.random.default_rng(9)
    th0 = torch.from_numpy(rng.standard_normal((B, H, wl.params)).astype(np.float32) * 0.2).cuda()
    s0 = torch.from_numpy(rng.standard_normal((B, H, wl.params)).astype(np.float32) * 0.01).cuda()
    y, thT, sT = tm.scan(q, k, v, g[..., 0], g[..., 1], g[..., 2], th0, s0, wl.chunk, wl.widths)
    torch.cuda.synchronize()
    yr, tr, sr = oracle.scan(inp.q, inp.k, inp.v, inp.alpha, inp.eta, inp.beta, to_f64(th0),
                             to_f64(s0), wl.chunk, wl.widths)
    assert y_rel_err(to_f64(y), yr) <= 1e-4
    assert state_rel_err(to_f64(thT), tr) <= 1e-4
    assert state_rel_err(to_f64(sT), sr) <= 1e-4


def test_invalid_arguments_raise():
    wl, inp = _small()
    dev = to_device(inp)
    with pytest.raises(tm.TitansError, match="INVALID_ARGUMENT"):
        tm.scan(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"], dev["theta0"],
                dev["s0"], 0, wl.widths)
    with pytest.raises(tm.TitansError, match="UNSUPPORTED"):
        tm.scan(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"], dev["theta0"],
                dev["s0"], 512, wl.widths)
    with pytest.raises(tm.TitansError, match="INVALID_ARGUMENT"):  # y overlapping q
        tm.scan(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"], dev["theta0"],
                dev["s0"], 8, wl.widths, y=dev["q"])


# ----------------------------------------------------------------- retrieve

@pytest.mark.parametrize("io,widths", [("f32", (16, 32, 16)), ("f32", (8, 24, 12, 8)),
                                       ("bf16", (16, 32, 16)), ("bf16", (8, 24, 12, 8)),
                                       ("bf16", (64, 256, 64))])
def test_retrieve_matches_oracle(io, widths):
    wl, inp = _small(widths=widths, B=2, T=45, H=3, io=io)
    dev = to_device(inp)
    log(f"case retrieve {io} {widths}")
    rng = np.random.default_rng(4)
    theta = (rng.standard_normal((2, 3, wl.params)) / 4).astype(np.float32)
    y = tm.retrieve(dev["q"], torch.from_numpy(theta).cuda(), widths)
    torch.cuda.synchronize()
    yr = oracle.retrieve(inp.qkv_f32("q"), theta, widths)
    assert y_rel_err(to_f64(y), yr) <= Y_BAR[io]


@pytest.mark.parametrize("T", [1, 63, 1023, 1025, 2100])
def test_retrieve_mfma_matches_generic_and_oracle(T, monkeypatch):
    """The fused bf16 MFMA retrieve (64-256-64) against the generic kernel and the oracle,
    with per-batch weights, strided q and y and a ragged token count."""
    wl, inp = _small(widths=(64, 256, 64), B=2, T=T, H=3, io="bf16", seed=T)
    dev = to_device(inp)
    log(f"case retrieve mfma T={T}")
    B, H = 2, 3
    rng = np.random.default_rng(T)
    theta = torch.from_numpy((rng.standard_normal((B, H, wl.params)) / 8).astype(np.float32)).cuda()
    packed = torch.stack([dev["q"], dev["k"]], dim=3)  # [B,T,H,2,d]: q rows strided by 2d
    q = packed[:, :, :, 0]
    assert tm.retrieve_path(q, wl.widths) == "fused_mfma"
    y = torch.empty(B, T, H, 2 * wl.d, dtype=torch.bfloat16, device="cuda")[..., : wl.d]
    y = tm.retrieve(q, theta, wl.widths, y=y)
    monkeypatch.setenv("TITANS_MEM_FORCE_GENERIC", "1")
    assert tm.retrieve_path(q, wl.widths) == "generic_mfma"
    y2 = tm.retrieve(q, theta, wl.widths)
    torch.cuda.synchronize()
    sel = slice(0, T, max(1, T // 200))
    yr = oracle.retrieve(inp.qkv_f32("q")[:, sel], to_f64(theta), wl.widths)
    e1 = y_rel_err(to_f64(y[:, sel]), yr)
    e2 = y_rel_err(to_f64(y), to_f64(y2))
    log(f"  mfma vs oracle {e1:.2e}, mfma vs generic {e2:.2e}")
    assert e1 <= 2e-2 and e2 <= 2e-2


@pytest.mark.parametrize("T", [1, 31, 33, 700])
@pytest.mark.parametrize("widths", [(128, 512, 512, 512, 128), (32, 160, 96, 32), (64, 384, 64),
                                    (16, 32, 16)])
def test_retrieve_wide_matches_oracle(widths, T):
    """bf16 memories other than 64-256-64 with widths multiples of 16: weights streamed
    through LDS; per-batch weights, strided q and y, ragged token counts."""
    wl, inp = _small(widths=widths, B=2, T=T, H=3, io="bf16", seed=T + len(widths))
    dev = to_device(inp)
    log(f"case retrieve wide {widths} T={T}")
    B, H = 2, 3
    rng = np.random.default_rng(T)
    scale = [1.0 / np.sqrt(w) for w in widths[:-1]]
    theta = np.concatenate([(rng.standard_normal((B, H, widths[l + 1] * widths[l])) * scale[l])
                            for l in range(len(widths) - 1)], axis=2).astype(np.float32)
    theta_t = torch.from_numpy(theta).cuda()
    packed = torch.stack([dev["q"], dev["k"]], dim=3)
    q = packed[:, :, :, 0]
    assert tm.retrieve_path(q, wl.widths) == "wide_mfma"
    y = torch.empty(B, T, H, 2 * wl.d, dtype=torch.bfloat16, device="cuda")[..., : wl.d]
    y = tm.retrieve(q, theta_t, wl.widths, y=y)
    torch.cuda.synchronize()
    yr = oracle.retrieve(inp.qkv_f32("q"), theta, wl.widths)
    err = y_rel_err(to_f64(y), yr)
    log(f"  wide vs oracle {err:.2e}")
    assert err <= 2e-2


def test_retrieve_headline_shape_sampled():
    wl = synthetic.WORKLOADS[synthetic.HEADLINE]
    inp = synthetic.make_inputs(wl, 0)
    dev = to_device(inp)
    log("case retrieve headline shape")
    y = tm.retrieve(dev["q"], dev["theta0"], wl.widths)
    torch.cuda.synchronize()
    yr = oracle.retrieve(inp.qkv_f32("q")[:, ::64], inp.theta0, wl.widths)
    assert y_rel_err(to_f64(y[:, ::64]), yr) <= 2e-2


# ----------------------------------------------------------- fused kernels
#
# The 64-256-64, C=64, bf16 shape runs on the pair kernel (two workgroups per memory)
# while the pairs fit the GPU, else on the single-workgroup kernel; both are tested.

FUSED = ["pair", "single"]


def _use(kernel, monkeypatch):
    monkeypatch.setenv("TITANS_MEM_FUSED_SINGLE", "1" if kernel == "single" else "0")
    return "fused_pair" if kernel == "pair" else "fused_mfma"


@pytest.mark.parametrize("kernel", FUSED)
def test_fused_matches_oracle_and_generic(kernel, monkeypatch):
    wl, inp = _small(widths=(64, 256, 64), B=2, T=300, H=3, C=64, io="bf16", seed=11)
    dev = to_device(inp)
    log(f"case fused[{kernel}] vs oracle and generic, 64-256-64 T=300")
    expected = _use(kernel, monkeypatch)
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == expected
    y1, t1, s1 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 2), (0, 1)]
    check_pairs(wl, y1, t1, s1, pairs, oracle_seq(inp, pairs))
    monkeypatch.setenv("TITANS_MEM_FORCE_GENERIC", "1")
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == "phased_mfma"
    y2, t2, s2 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    ey = y_rel_err(to_f64(y1), to_f64(y2))
    et = state_rel_err(to_f64(t1), to_f64(t2))
    log(f"  fused[{kernel}] vs generic: y {ey:.2e} theta_T {et:.2e}")
    assert ey <= 2e-2 and et <= 1e-1


@pytest.mark.parametrize("T", [1, 37, 64, 65, 130])
@pytest.mark.parametrize("kernel", FUSED)
def test_fused_short_and_ragged(kernel, T, monkeypatch):
    wl, inp = _small(widths=(64, 256, 64), B=1, T=T, H=2, C=64, io="bf16", seed=T)
    dev = to_device(inp)
    log(f"case fused[{kernel}] T={T}")
    expected = _use(kernel, monkeypatch)
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == expected
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    pairs = [(0, 0), (0, 1)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs))


@pytest.mark.parametrize("kernel", FUSED)
def test_fused_streaming_inplace_determinism(kernel, monkeypatch):
    wl, inp = _small(widths=(64, 256, 64), B=2, T=200, H=3, C=64, io="bf16", seed=3)
    dev = to_device(inp)
    log(f"case fused[{kernel}] streaming / in-place / determinism")
    _use(kernel, monkeypatch)
    y, thT, sT = run_gpu(dev, wl)
    y2, thT2, sT2 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(thT, thT2) and torch.equal(sT, sT2)
    B = wl.batch
    th = dev["theta0"].expand(B, -1, -1).contiguous()
    s = dev["s0"].expand(B, -1, -1).contiguous()
    cut = 128  # a multiple of the chunk: the two calls chain exactly
    half = {n: dev[n][:, :cut] for n in ("q", "k", "v", "alpha", "eta", "beta")}
    rest = {n: dev[n][:, cut:] for n in ("q", "k", "v", "alpha", "eta", "beta")}
    ya, _, _ = tm.scan(half["q"], half["k"], half["v"], half["alpha"], half["eta"], half["beta"],
                       th, s, wl.chunk, wl.widths, theta_T=th, s_T=s)
    yb, _, _ = tm.scan(rest["q"], rest["k"], rest["v"], rest["alpha"], rest["eta"], rest["beta"],
                       th, s, wl.chunk, wl.widths, theta_T=th, s_T=s)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([ya, yb], dim=1), y)
    assert torch.equal(th, thT) and torch.equal(s, sT)


@pytest.mark.parametrize("kernel", FUSED)
def test_fused_strided_inputs_nonzero_momentum(kernel, monkeypatch):
    wl, inp = _small(widths=(64, 256, 64), B=2, T=150, H=2, C=64, io="bf16", seed=21)
    dev = to_device(inp)
    log(f"case fused[{kernel}] strided q/k/v, per-batch theta0 and nonzero s0")
    _use(kernel, monkeypatch)
    packed = torch.stack([dev["q"], dev["k"], dev["v"]], dim=3)  # [B,T,H,3,d]
    q, k, v = packed[:, :, :, 0], packed[:, :, :, 1], packed[:, :, :, 2]
    g = torch.stack([dev["alpha"], dev["eta"], dev["beta"]], dim=-1)
    B, H = wl.batch, wl.heads
    rng = np.random.default_rng(17)
    th0 = torch.from_numpy((rng.standard_normal((B, H, wl.params)) * 0.1).astype(np.float32)).cuda()
    s0 = torch.from_numpy((rng.standard_normal((B, H, wl.params)) * 0.01).astype(np.float32)).cuda()
    y = torch.empty(B, wl.seq_len, H, 2 * wl.d, dtype=torch.bfloat16, device="cuda")[..., : wl.d]
    y, thT, sT = tm.scan(q, k, v, g[..., 0], g[..., 1], g[..., 2], th0, s0, wl.chunk, wl.widths, y=y)
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 1)]
    refs = []
    for b, h in pairs:
        yr, tr, sr = oracle.scan(inp.qkv_f32("q")[b:b + 1, :, h:h + 1], inp.qkv_f32("k")[b:b + 1, :, h:h + 1],
                                 inp.qkv_f32("v")[b:b + 1, :, h:h + 1], inp.alpha[b:b + 1, :, h:h + 1],
                                 inp.eta[b:b + 1, :, h:h + 1], inp.beta[b:b + 1, :, h:h + 1],
                                 to_f64(th0[b, h:h + 1]), to_f64(s0[b, h:h + 1]), wl.chunk, wl.widths)
        refs.append((yr[0, :, 0], tr[0, 0], sr[0, 0]))
    check_pairs(wl, y, thT, sT, pairs, refs)


@pytest.mark.parametrize("C,T", [(128, 300), (192, 385), (256, 600), (256, 100)])
def test_pair_long_chunks_match_oracle(C, T, monkeypatch):
    """Chunks of 128..256 tokens on the pair path: 64-token sub-chunks whose gradients are
    all taken at the chunk-start weights."""
    wl, inp = _small(widths=(64, 256, 64), B=2, T=T, H=3, C=C, io="bf16", seed=C + T)
    dev = to_device(inp)
    log(f"case pair path C={C} T={T}")
    expected = _use("pair", monkeypatch)
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == expected
    y, thT, sT = run_gpu(dev, wl)
    y2, thT2, sT2 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(thT, thT2)
    pairs = [(0, 0), (1, 2)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs))
    monkeypatch.setenv("TITANS_MEM_FORCE_GENERIC", "1")
    yg, tg, _ = run_gpu(dev, wl)
    torch.cuda.synchronize()
    ey, et = y_rel_err(to_f64(y), to_f64(yg)), state_rel_err(to_f64(thT), to_f64(tg))
    log(f"  pair vs generic: y {ey:.2e} theta_T {et:.2e}")
    assert ey <= 2e-2 and et <= 1e-1


def test_scan_and_retrieve_on_a_side_stream():
    """The library enqueues on the caller's stream: a side stream gives the same bits."""
    wl, inp = _small(widths=(64, 256, 64), B=2, T=200, H=3, C=64, io="bf16", seed=51)
    dev = to_device(inp)
    log("case side stream")
    y0, t0, s0 = run_gpu(dev, wl)
    r0 = tm.retrieve(dev["q"], t0, wl.widths)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y1, t1, s1 = run_gpu(dev, wl)
        r1 = tm.retrieve(dev["q"], t1, wl.widths)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(t0, t1) and torch.equal(s0, s1)
    assert torch.equal(r0, r1)


def test_pair_wait_bound_ends_the_kernel(monkeypatch):
    """Failure handling of the pair exchange, forced from the host: one side of every pair
    never posts (test hook) and the waits give up after a few polls. The kernel must end,
    the side that timed out must return NaN for its half of theta_T, and the next normal
    call must be exact again."""
    wl, inp = _small(widths=(64, 256, 64), B=1, T=200, H=2, C=64, io="bf16", seed=41)
    dev = to_device(inp)
    log("case pair wait bound (forced timeout)")
    _use("pair", monkeypatch)
    y0, t0, s0 = run_gpu(dev, wl)
    monkeypatch.setenv("TITANS_MEM_TEST_PAIR_TIMEOUT", "1")
    y1, t1, s1 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    P1 = 256 * 64  # W1 rows h = 0..127 belong to side 0
    assert torch.isnan(t1[:, :, : P1 // 2]).all() and torch.isnan(s1[:, :, : P1 // 2]).all()
    monkeypatch.delenv("TITANS_MEM_TEST_PAIR_TIMEOUT")
    y2, t2, s2 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    assert torch.equal(y2, y0) and torch.equal(t2, t0) and torch.equal(s2, s0)


def test_pair_kernel_matches_single_kernel(monkeypatch):
    """The two fused kernels round at the same points and differ only in summation order."""
    wl = _workload("h8_d64_b4_t4k", True)
    inp = synthetic.make_inputs(wl, 5)
    dev = to_device(inp)
    log("case pair vs single fused kernel, h8 T=4096 sustained")
    _use("pair", monkeypatch)
    y1, t1, s1 = run_gpu(dev, wl)
    _use("single", monkeypatch)
    y2, t2, s2 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    ey = y_rel_err(to_f64(y1), to_f64(y2))
    et = state_rel_err(to_f64(t1), to_f64(t2))
    es = state_rel_err(to_f64(s1), to_f64(s2))
    log(f"  pair vs single: y {ey:.2e} theta_T {et:.2e} s_T {es:.2e}")
    assert ey <= 2e-2 and et <= 1e-1 and es <= 1e-1


def test_fused_path_switch_at_the_compute_unit_limit(monkeypatch):
    """More memories than pairs of compute units: the fused shape runs one workgroup per
    memory (and still matches the oracle)."""
    monkeypatch.delenv("TITANS_MEM_FUSED_SINGLE", raising=False)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H = 8
    B = cus // (2 * H) + 1  # 2 * ceil(B*H / 8) * 8 > cus
    wl, inp = _small(widths=(64, 256, 64), B=B, T=130, H=H, C=64, io="bf16", seed=31)
    dev = to_device(inp)
    log(f"case fused path switch: B*H = {B * H} memories on {cus} compute units")
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == "fused_mfma"
    small = _small(widths=(64, 256, 64), B=B - 1, T=130, H=H, C=64, io="bf16", seed=31)[1]
    assert tm.scan_path(to_device(small)["q"], wl.chunk, wl.widths) == "fused_pair"
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    pairs = [(0, 0), (B - 1, H - 1)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs))


@pytest.mark.parametrize("sustained", [False, True])
def test_headline_sampled_single_kernel(sustained, monkeypatch):
    """The single-workgroup kernel at the full headline shape (the pair kernel runs it by default)."""
    _use("single", monkeypatch)
    test_headline_sampled(sustained)


# ------------------------------------------------------ attentional biases
#
# The Huber and l_p attentional biases replace the output-layer error 2 (O - V) by the
# derivative of the per-component loss in every scan kernel.  Each path against the
# oracle with the same bias (l_1 only with fp32 I/O: its gradient jumps at r = 0, where
# bf16 rounding of the residual flips signs).

BIAS_PATHS = {
    # name: (widths, C, io, env, expected path)
    "generic_f32": ((16, 32, 16), 8, "f32", {"TITANS_MEM_GENERIC_MODE": "single"}, "generic_fp32"),
    "generic_bf16": ((16, 32, 16), 5, "bf16", {"TITANS_MEM_GENERIC_MODE": "single"}, "generic_mfma"),
    "phased_f32": ((32, 160, 32), 40, "f32", {}, "phased_fp32"),
    "phased_bf16": ((32, 160, 32), 40, "bf16", {}, "phased_mfma"),
    "pair": ((64, 256, 64), 64, "bf16", {}, "fused_pair"),
    "pair_c128": ((64, 256, 64), 128, "bf16", {}, "fused_pair"),
    "single": ((64, 256, 64), 64, "bf16", {"TITANS_MEM_FUSED_SINGLE": "1"}, "fused_mfma"),
}


@pytest.mark.parametrize("bias", [("huber", 0.5), ("lp", 1.5), ("lp", 3.0), ("lp", 1.0)])
@pytest.mark.parametrize("path", sorted(BIAS_PATHS))
def test_attentional_bias_matches_oracle(path, bias, monkeypatch):
    widths, C, io, env, expected = BIAS_PATHS[path]
    if bias == ("lp", 1.0) and io == "bf16":
        pytest.skip("l_1 flips the sign of near-zero residuals under bf16 rounding")
    for k_, v_ in env.items():
        monkeypatch.setenv(k_, v_)
    wl, inp = _small(widths=widths, B=2, T=200, H=2, C=C, io=io, seed=C + 7)
    dev = to_device(inp)
    log(f"case bias {bias} on {path}")
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == expected
    y, thT, sT = run_gpu(dev, wl, bias=bias)
    torch.cuda.synchronize()
    pairs = [(0, 1), (1, 0)]
    refs = oracle_seq(inp, pairs, bias=bias)
    check_pairs(wl, y, thT, sT, pairs, refs)
    # the bias changes the memory (else the test would not see a kernel that ignores it)
    y0, t0, _ = run_gpu(dev, wl)
    torch.cuda.synchronize()
    assert state_rel_err(to_f64(t0[:1, 1:2]), refs[0][1][None, None]) > 0.3


# ------------------------------------------------------------ surprise norm

SURPRISE_CASES = {
    # name: (widths, C, io, env, expected path of the surprise call)
    "generic_f32": ((16, 32, 16), 8, "f32", {"TITANS_MEM_GENERIC_MODE": "single"}, "generic_fp32"),
    "generic_bf16": ((8, 24, 12, 8), 5, "bf16", {"TITANS_MEM_GENERIC_MODE": "single"}, "generic_mfma"),
    "phased_f32": ((32, 160, 32), 40, "f32", {}, "phased_fp32"),
    "phased_bf16": ((128, 512, 128), 128, "bf16", {}, "phased_mfma"),
    "fused_shape": ((64, 256, 64), 64, "bf16", {}, "fused_pair"),
    "fused_shape_c128": ((64, 256, 64), 128, "bf16", {}, "fused_pair"),
    "fused_shape_phased": ((64, 256, 64), 64, "bf16", {"TITANS_MEM_FORCE_GENERIC": "1"},
                           "phased_mfma"),
}


@pytest.mark.parametrize("bias", [None, ("huber", 0.5)])
@pytest.mark.parametrize("case", sorted(SURPRISE_CASES))
def test_surprise_matches_oracle(case, bias, monkeypatch):
    """Each token's gradient norm from titans_mem_scan_surprise against the oracle's (same
    relative-error bars as y), with y and the state as in the plain scan."""
    widths, C, io, env, expected = SURPRISE_CASES[case]
    for k_, v_ in env.items():
        monkeypatch.setenv(k_, v_)
    wl, inp = _small(widths=widths, B=2, T=150, H=2, C=C, io=io, seed=C + 3)
    dev = to_device(inp)
    log(f"case surprise {case} bias={bias}")
    assert tm.surprise_path(dev["q"], wl.chunk, wl.widths) == expected
    y, thT, sT, sur = run_gpu(dev, wl, bias=bias, surprise=True)
    torch.cuda.synchronize()
    pairs = [(0, 1), (1, 0)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs, bias=bias))
    q, k, v = [inp.qkv_f32(n) for n in ("q", "k", "v")]
    *_, sr = oracle.scan(q, k, v, inp.alpha, inp.eta, inp.beta, inp.theta0, inp.s0, C, widths,
                         bias=bias, surprise=True)
    sg = to_f64(sur)
    err = max(np.linalg.norm(sg[b, :, h] - sr[b, :, h]) / np.linalg.norm(sr[b, :, h])
              for b in range(2) for h in range(2))
    log(f"  surprise rel err {err:.2e}")
    assert err <= Y_BAR[io]


# ------------------------------------------------- linear memory, sequence-parallel

@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("d,C,nch", [(16, 4, 40), (64, 16, 37), (128, 64, 24), (64, 256, 17)])
def test_linear_memory_parallel_scan(d, C, nch, io, monkeypatch):
    """L = 1: chunk carries composed per group of chunks in parallel, chained over the
    groups, every group's chunks run from its start state; against the oracle and the
    sequential generic kernel, ragged last chunk, in-place streaming of the state."""
    T = C * nch - 3
    wl, inp = _small(widths=(d, d), B=2, T=T, H=2, C=C, io=io, seed=d + C)
    rng = np.random.default_rng(d)
    inp.s0 = (0.05 * rng.standard_normal(inp.theta0.shape)).astype(np.float32)
    dev = to_device(inp)
    log(f"case linear d={d} C={C} T={T} {io}")
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == ("linear_mfma" if io == "bf16" else "linear_fp32")
    y, thT, sT = run_gpu(dev, wl)
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 1), (0, 1)]
    check_pairs(wl, y, thT, sT, pairs, oracle_seq(inp, pairs))
    # the sequential generic kernel on the same inputs
    monkeypatch.setenv("TITANS_MEM_LINEAR", "0")
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths).startswith(("generic", "phased"))
    y2, t2, s2 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    monkeypatch.delenv("TITANS_MEM_LINEAR")
    bar = Y_BAR[io]
    assert y_rel_err(to_f64(y), to_f64(y2)) <= bar
    assert state_rel_err(to_f64(thT), to_f64(t2)) <= TH_BAR[io]
    # in place: theta_T / s_T are theta0 / s0 themselves (per batch row)
    th = dev["theta0"].expand(2, *dev["theta0"].shape).contiguous()
    s0 = dev["s0"].expand(2, *dev["s0"].shape).contiguous()
    tm.scan(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"], th, s0,
            wl.chunk, wl.widths, theta_T=th, s_T=s0)
    torch.cuda.synchronize()
    assert state_rel_err(to_f64(th), to_f64(thT)) <= 1e-6
    assert state_rel_err(to_f64(s0), to_f64(sT)) <= 1e-6
