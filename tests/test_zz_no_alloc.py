"""titans_mem_scan_noalloc (the scan for callers that cannot allocate: its scratch is the
library's static device array) through the C ABI, against titans_mem_scan on the same
inputs: bitwise equal results (the allocation-free call runs the same kernels over segments
of the sequence that chain exactly), on calls in a row with different sizes, the second
smaller than the first; the small case also against the oracle."""
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


def _both(dev, wl, inplace=False):
    """(titans_mem_scan, titans_mem_scan_noalloc) results on the same inputs."""
    B, T, H, d = dev["q"].shape
    P = wl.params
    ref = tm.scan(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                  dev["theta0"], dev["s0"], wl.chunk, wl.widths)
    y = torch.full_like(dev["q"], float("nan"))
    if inplace:
        th = dev["theta0"].expand(B, -1, -1).contiguous()
        s = dev["s0"].expand(B, -1, -1).contiguous()
        out = tm.scan_noalloc(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                              th, s, wl.chunk, wl.widths, y=y, theta_T=th, s_T=s)
    else:
        th = torch.full((B, H, P), float("nan"), dtype=torch.float32, device="cuda")
        s = torch.full_like(th, float("nan"))
        out = tm.scan_noalloc(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                              dev["theta0"], dev["s0"], wl.chunk, wl.widths, y=y, theta_T=th, s_T=s)
    torch.cuda.synchronize()
    return ref, out


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def _equal(ref, out):
    """Bitwise equality (NaN payloads included: under the sustained gates one memory of the
    headline draw diverges, as the fp64 recurrence does)."""
    return all(torch.equal(_bits(a), _bits(b)) for a, b in zip(ref, out))


def test_noalloc_matches_scan_full_size_then_smaller():
    # 1. the headline shape (B*H = 128, T = 16384): several segments of the static array
    wl = synthetic.sustained(synthetic.HEADLINE)
    inp = synthetic.make_inputs(wl, 0)
    dev = to_device(inp)
    print("case noalloc headline shape", flush=True)
    assert tm.scan_path(dev["q"], wl.chunk, wl.widths) == "fused_pair"
    ref, out = _both(dev, wl)
    assert _equal(ref, out)
    del dev, ref, out
    # 2. right after, a smaller ragged problem (the array keeps the last call's contents)
    wl = synthetic.Workload("noalloc_small", 1, 2, 200, (64, 256, 64), 64, "bf16")
    inp = synthetic.make_inputs(wl, 3)
    dev = to_device(inp)
    print("case noalloc small ragged", flush=True)
    ref, out = _both(dev, wl)
    assert _equal(ref, out)
    yr, tr, sr = oracle.scan(inp.qkv_f32("q"), inp.qkv_f32("k"), inp.qkv_f32("v"), inp.alpha,
                             inp.eta, inp.beta, inp.theta0, inp.s0, wl.chunk, wl.widths)
    assert y_rel_err(to_f64(out[0]), yr) <= 2e-2
    assert state_rel_err(to_f64(out[1]), tr) <= 2e-2 and state_rel_err(to_f64(out[2]), sr) <= 2e-2


def test_noalloc_long_chunks_and_in_place():
    wl = synthetic.Workload("noalloc_c128", 2, 3, 300, (64, 256, 64), 128, "bf16")
    inp = synthetic.make_inputs(wl, 5)
    dev = to_device(inp)
    print("case noalloc C=128, in place", flush=True)
    ref, out = _both(dev, wl)
    assert _equal(ref, out)
    ref2, out2 = _both(dev, wl, inplace=True)
    assert _equal(ref2, out2)


def test_noalloc_rejects_other_shapes():
    wl = synthetic.Workload("noalloc_other", 1, 2, 40, (16, 32, 16), 8, "bf16")
    dev = to_device(synthetic.make_inputs(wl, 1))
    y = torch.empty_like(dev["q"])
    th = torch.empty((1, 2, wl.params), dtype=torch.float32, device="cuda")
    s = torch.empty_like(th)
    with pytest.raises(tm.TitansError, match="UNSUPPORTED.*pair path"):
        tm.scan_noalloc(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["eta"], dev["beta"],
                        dev["theta0"], dev["s0"], wl.chunk, wl.widths, y=y, theta_T=th, s_T=s)
