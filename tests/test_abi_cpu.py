"""The C-ABI library loads, exports every function include/titans_mem.h declares, and
rejects invalid calls on the host, before any HIP work.

No call here does device work: every scan/retrieve call is built to fail host
validation (the status is checked to be a validation error, never TITANS_ERR_HIP).
Calls that pass fake pointers are skipped when a GPU is visible.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "titans_mem.h")

tm = pytest.importorskip("sequence_models_amd")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(titans_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"titans_mem_scan", "titans_mem_retrieve", "titans_mem_scan_workspace_size",
            "titans_abi_version", "titans_status_string", "titans_last_error",
            "titans_mem_param_count"} <= set(names)
    lib = ctypes.CDLL(tm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in titans_mem.h but not exported"


def test_version_status_strings_and_param_count():
    assert tm.lib.titans_abi_version() == 6
    assert tm.lib.titans_status_string(0) == b"TITANS_OK"
    assert tm.lib.titans_status_string(3) == b"TITANS_ERR_WORKSPACE"
    assert tm.param_count((64, 256, 64)) == 32768
    assert tm.param_count((128, 512, 512, 512, 128)) == 655360
    assert tm.param_count((16, 64, 16)) == 2048
    assert tm.lib.titans_mem_param_count(ctypes.byref(tm.mlp_desc((4,)))) == -1
    assert tm.lib.titans_mem_param_count(ctypes.byref(tm.mlp_desc((4, 8, 5)))) == -1


def _desc(B=2, T=64, H=4, d=64, C=64, io=1):
    desc = tm.ScanDesc()
    desc.batch, desc.seq_len, desc.heads, desc.chunk, desc.io_dtype = B, T, H, C, io
    desc.qkv_stride[:] = (T * H * d, H * d, d)
    desc.y_stride[:] = (T * H * d, H * d, d)
    desc.gate_stride[:] = (T * H, H, 1)
    return desc


def test_workspace_size_query(monkeypatch):
    mlp = tm.mlp_desc((64, 256, 64))
    # the fused shape (64-256-64, C=64, bf16) runs on groups of workgroups that exchange
    # partial sums through the workspace, after a pass that writes every chunk's gate
    # coefficients (9472 bytes per chunk): quads (a 226 KiB area per memory, memories padded
    # to 8) while four workgroups per memory fit the 256 compute units (B*H <= 64), pairs (a
    # 97 KiB area per memory) up to B*H = 128
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc()), ctypes.byref(mlp)) == b"fused_quad"
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(_desc()),
                                                 ctypes.byref(mlp)) == 8 * 231424 + 8 * 1 * 9472
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(_desc(B=3, T=130, H=3)),
                                                 ctypes.byref(mlp)) == 16 * 231424 + 9 * 3 * 9472
    for B, H, path, area in ((4, 16, b"fused_quad", 231424), (5, 13, b"fused_pair", 99328),
                             (8, 16, b"fused_pair", 99328)):
        d = _desc(B=B, H=H)
        assert tm.lib.titans_mem_scan_path(ctypes.byref(d), ctypes.byref(mlp)) == path
        npad = (B * H + 7) // 8 * 8
        assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(d), ctypes.byref(mlp)) == \
            npad * area + B * H * 9472
    monkeypatch.setenv("TITANS_MEM_PAIR_SIDES", "2")  # keeps pairs (testing switch)
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc()), ctypes.byref(mlp)) == b"fused_pair"
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(_desc()),
                                                 ctypes.byref(mlp)) == 8 * 99328 + 8 * 1 * 9472
    monkeypatch.delenv("TITANS_MEM_PAIR_SIDES")
    # chunks that are multiples of 64 run on the pair path too (64-token sub-chunks whose
    # gradients share the chunk-start weights); other lengths on the generic kernel
    for C, path in ((128, b"fused_quad"), (256, b"fused_quad"), (96, b"phased_mfma"),
                    (32, b"phased_mfma")):
        assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(C=C)), ctypes.byref(mlp)) == path
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(B=64, H=16, C=256)),
                                       ctypes.byref(mlp)) == b"phased_mfma"
    # more memories than pairs of compute units: one workgroup per memory, no workspace
    big = _desc(B=64, H=16)
    assert tm.lib.titans_mem_scan_path(ctypes.byref(big), ctypes.byref(mlp)) == b"fused_mfma"
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(big), ctypes.byref(mlp)) == 0
    monkeypatch.setenv("TITANS_MEM_FUSED_SINGLE", "1")
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc()), ctypes.byref(mlp)) == b"fused_mfma"
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(_desc()), ctypes.byref(mlp)) == 0
    monkeypatch.delenv("TITANS_MEM_FUSED_SINGLE")
    size = tm.lib.titans_mem_scan_workspace_size(ctypes.byref(_desc(C=32)), ctypes.byref(mlp))
    assert 0 < size < 1 << 30 and size % 4 == 0
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(C=32)), ctypes.byref(mlp)) == b"phased_mfma"
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(io=0)), ctypes.byref(mlp)) == b"phased_fp32"
    # the generic family: layers of 128+ units run as a chain of GPU-wide launches, narrower
    # memories on one workgroup each; TITANS_MEM_GENERIC_MODE forces either
    narrow = tm.mlp_desc((64, 96, 64))
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(C=32)), ctypes.byref(narrow)) == b"generic_mfma"
    deep = tm.mlp_desc((128, 512, 512, 512, 128))
    ddesc = _desc(B=2, T=32768, H=8, d=128, C=128)
    assert tm.lib.titans_mem_scan_path(ctypes.byref(ddesc), ctypes.byref(deep)) == b"phased_mfma"
    # per memory: two parity buffers of coefficients (3C+3) and Cm ((C+1) C);
    # Hk and SiLU' of the hidden layers, Delta of every layer, two read buffers (C x 512)
    # and Cm o Hq Hk^T (C x C), each rounded up to 64 floats
    r64 = lambda x: (x + 63) // 64 * 64
    per = (2 * (r64(3 * 128 + 3) + r64(129 * 128)) + 2 * 3 * 128 * 512
           + (3 * 128 * 512 + 128 * 128) + 2 * 128 * 512 + 128 * 128)
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(ddesc), ctypes.byref(deep)) == 16 * per * 4
    monkeypatch.setenv("TITANS_MEM_GENERIC_MODE", "single")
    assert tm.lib.titans_mem_scan_path(ctypes.byref(ddesc), ctypes.byref(deep)) == b"generic_mfma"
    monkeypatch.setenv("TITANS_MEM_GENERIC_MODE", "phased")
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(C=32)), ctypes.byref(narrow)) == b"phased_mfma"
    monkeypatch.delenv("TITANS_MEM_GENERIC_MODE")
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(C=0)), ctypes.byref(mlp)) is None
    assert tm.lib.titans_mem_retrieve_path(ctypes.byref(_desc()), ctypes.byref(mlp)) == b"fused_mfma"
    assert tm.lib.titans_mem_retrieve_path(ctypes.byref(_desc(io=0)), ctypes.byref(mlp)) == b"generic_fp32"
    assert tm.lib.titans_mem_retrieve_path(ctypes.byref(_desc()), ctypes.byref(tm.mlp_desc((64, 128, 64)))) == b"wide_mfma"
    assert tm.lib.titans_mem_retrieve_path(ctypes.byref(_desc(d=16)),
                                           ctypes.byref(tm.mlp_desc((16, 24, 16)))) == b"generic_mfma"
    assert tm.lib.titans_mem_retrieve_path(ctypes.byref(_desc(io=0)),
                                           ctypes.byref(tm.mlp_desc((64, 128, 64)))) == b"generic_fp32"
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(_desc(T=0)), ctypes.byref(mlp)) == 0
    bad = ctypes.c_size_t(-1).value
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(_desc(C=0)), ctypes.byref(mlp)) == bad
    assert tm.lib.titans_mem_scan_workspace_size(None, ctypes.byref(mlp)) == bad
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(_desc(C=300)),
                                                 ctypes.byref(mlp)) == bad


def _scan(desc, mlp, ptrs=None, ws=None, ws_bytes=0):
    p = ptrs or {}
    args = [p.get(n) for n in ("q", "k", "v", "alpha", "eta", "beta", "theta0", "s0", "y",
                               "theta_T", "s_T")]
    st = tm.lib.titans_mem_scan(ctypes.byref(desc) if desc is not None else None,
                                ctypes.byref(mlp) if mlp is not None else None,
                                *args, ws, ws_bytes, None)
    assert st != HIP, "validation let the call through to HIP"
    return st, tm.lib.titans_last_error().decode()


def test_validation_of_descriptors():
    mlp = tm.mlp_desc((64, 256, 64))
    assert _scan(None, mlp)[0] == INVALID
    assert _scan(_desc(), None)[0] == INVALID
    assert _scan(_desc(C=0), mlp)[0] == INVALID
    assert _scan(_desc(B=-1), mlp)[0] == INVALID
    assert _scan(_desc(io=7), mlp)[0] == INVALID
    assert _scan(_desc(), tm.mlp_desc((64, 256, 32)))[0] == INVALID
    assert _scan(_desc(), tm.mlp_desc((64, 1, 1, 1, 1, 64)))[0] == INVALID   # 5 layers
    assert _scan(_desc(C=512), mlp)[0] == UNSUPPORTED
    assert _scan(_desc(d=256), tm.mlp_desc((256, 256, 256)))[0] == UNSUPPORTED
    assert _scan(_desc(), tm.mlp_desc((64, 1024, 64)))[0] == UNSUPPORTED
    st, msg = _scan(_desc(), mlp)   # all pointers NULL
    assert st == INVALID and "non-NULL" in msg
    # attentional bias: kind and parameter are checked before anything else runs
    for bias, prm, text in ((3, 1.0, "titans_bias"), (-1, 1.0, "titans_bias"), (1, 0.0, "Huber"),
                            (1, -2.0, "Huber"), (1, float("nan"), "Huber"), (2, 0.5, "l_p"),
                            (2, float("inf"), "l_p"), (2, float("nan"), "l_p")):
        d = _desc()
        d.bias, d.bias_param = bias, prm
        st, msg = _scan(d, mlp)
        assert st == INVALID and text in msg, (bias, prm, msg)
    for bias, prm in ((0, -5.0), (1, float("inf")), (1, 1e-6), (2, 1.0), (2, 7.5)):
        d = _desc()
        d.bias, d.bias_param = bias, prm
        st, msg = _scan(d, mlp)   # valid bias: the NULL pointers are what fails
        assert st == INVALID and "non-NULL" in msg, (bias, prm, msg)
    # the descriptor's layout matches the header (bias fields after the strides)
    assert ctypes.sizeof(tm.ScanDesc) == 3 * 8 + 2 * 4 + 13 * 8 + 4 + 4


no_fake_pointers_on_gpu = pytest.mark.skipif(
    __import__("torch").cuda.is_available(), reason="fake device pointers are never passed on a GPU box")


def _fake_ptrs(B=2, T=64, H=4, d=64, P=32768, esz=2, base=1 << 40):
    sizes = {"q": B * T * H * d * esz, "k": B * T * H * d * esz, "v": B * T * H * d * esz,
             "y": B * T * H * d * esz, "alpha": B * T * H * 4, "eta": B * T * H * 4,
             "beta": B * T * H * 4, "theta0": H * P * 4, "s0": H * P * 4, "theta_T": B * H * P * 4,
             "s_T": B * H * P * 4}
    out, cur = {}, base
    for n, s in sizes.items():
        out[n] = cur
        cur += (s + 4095) // 4096 * 4096
    return out, cur


@no_fake_pointers_on_gpu
def test_validation_of_overlap_alignment_and_workspace():
    mlp = tm.mlp_desc((64, 256, 64))
    B, T, H, d, P = 2, 64, 4, 64, 32768
    desc = _desc(B, T, H, d, C=32)  # C=32 runs the generic kernel, which needs a workspace
    desc.state_stride[:] = (H * P, P)
    desc.state0_stride[:] = (0, P)
    ptrs, end = _fake_ptrs()
    need = tm.lib.titans_mem_scan_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    # y aliasing q
    bad = dict(ptrs, y=ptrs["q"])
    assert _scan(desc, mlp, bad, end, need)[0] == INVALID
    # theta_T overlapping s0 without being theta0
    bad = dict(ptrs, theta_T=ptrs["s0"])
    assert _scan(desc, mlp, bad, end, need)[0] == INVALID
    # misaligned q
    bad = dict(ptrs, q=ptrs["q"] + 2)
    assert _scan(desc, mlp, bad, end, need)[0] == INVALID
    # workspace too small / missing / overlapping / misaligned
    assert _scan(desc, mlp, ptrs, end, need - 1)[0] == WORKSPACE
    assert _scan(desc, mlp, ptrs, None, 0)[0] == WORKSPACE
    assert _scan(desc, mlp, ptrs, ptrs["v"], need)[0] == INVALID
    assert _scan(desc, mlp, ptrs, end + 16, need)[0] == INVALID
    # y strides that alias distinct tokens
    d2 = _desc(B, T, H, d)
    d2.state_stride[:] = (H * P, P)
    d2.state0_stride[:] = (0, P)
    d2.y_stride[:] = (T * H * d, 0, d)
    assert _scan(d2, mlp, ptrs, end, need)[0] == INVALID
    # theta_T with batch stride 0 writes one memory from several batch rows
    d3 = _desc(B, T, H, d)
    d3.state_stride[:] = (0, P)
    d3.state0_stride[:] = (0, P)
    assert _scan(d3, mlp, ptrs, end, need)[0] == INVALID


@no_fake_pointers_on_gpu
def test_pair_path_workspace_validation():
    """The fused pair path needs its exchange area and coefficient records."""
    mlp = tm.mlp_desc((64, 256, 64))
    B, T, H, P = 2, 64, 4, 32768
    desc = _desc(B, T, H)
    desc.state_stride[:] = (H * P, P)
    desc.state0_stride[:] = (0, P)
    assert tm.lib.titans_mem_scan_path(ctypes.byref(desc), ctypes.byref(mlp)) == b"fused_quad"
    ptrs, end = _fake_ptrs()
    need = tm.lib.titans_mem_scan_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    assert need > 0
    assert _scan(desc, mlp, ptrs, end, need - 1)[0] == WORKSPACE
    assert _scan(desc, mlp, ptrs, None, 0)[0] == WORKSPACE
    assert _scan(desc, mlp, ptrs, end + 128, need)[0] == INVALID  # not 256-byte aligned
    assert _scan(desc, mlp, ptrs, ptrs["y"], need)[0] == INVALID  # overlaps y


@no_fake_pointers_on_gpu
def test_retrieve_validation():
    mlp = tm.mlp_desc((64, 256, 64))
    desc = _desc()
    desc.state_stride[:] = (0, 32768)
    ptrs, _ = _fake_ptrs()
    st = tm.lib.titans_mem_retrieve(ctypes.byref(desc), ctypes.byref(mlp), ptrs["q"],
                                    ptrs["theta0"], ptrs["q"], None)
    assert st == INVALID
    st = tm.lib.titans_mem_retrieve(ctypes.byref(desc), ctypes.byref(mlp), None, None, None, None)
    assert st == INVALID
    st = tm.lib.titans_mem_retrieve(ctypes.byref(desc), ctypes.byref(tm.mlp_desc((64, 999, 64))),
                                    ptrs["q"], ptrs["theta0"], ptrs["y"], None)
    assert st == UNSUPPORTED


def _scan_surprise(desc, mlp, ptrs, surprise, ws=None, ws_bytes=0):
    args = [ptrs.get(n) for n in ("q", "k", "v", "alpha", "eta", "beta", "theta0", "s0", "y",
                                  "theta_T", "s_T")]
    st = tm.lib.titans_mem_scan_surprise(ctypes.byref(desc), ctypes.byref(mlp), *args, surprise,
                                         ws, ws_bytes, None)
    assert st != HIP, "validation let the call through to HIP"
    return st, tm.lib.titans_last_error().decode()


def test_surprise_workspace_follows_the_path(monkeypatch):
    """The fused shape's surprise call runs on pairs (where the plain scan of this small
    shape takes quads) with 65 floats of partial sums per token-head after the pairs'
    workspace; forced onto the generic family it takes the phased path's workspace, as the
    plain scan does there."""
    mlp = tm.mlp_desc((64, 256, 64))
    desc = _desc()
    B, T, H = desc.batch, desc.seq_len, desc.heads
    assert tm.lib.titans_mem_scan_path(ctypes.byref(desc), ctypes.byref(mlp)) == b"fused_quad"
    sur = tm.lib.titans_mem_scan_surprise_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    assert tm.lib.titans_mem_scan_surprise_path(ctypes.byref(desc), ctypes.byref(mlp)) == b"fused_pair"
    monkeypatch.setenv("TITANS_MEM_PAIR_SIDES", "2")
    pair = tm.lib.titans_mem_scan_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    monkeypatch.delenv("TITANS_MEM_PAIR_SIDES")
    assert sur == pair + B * H * T * 65 * 4
    monkeypatch.setenv("TITANS_MEM_FORCE_GENERIC", "1")
    assert tm.lib.titans_mem_scan_path(ctypes.byref(desc), ctypes.byref(mlp)) == b"phased_mfma"
    assert tm.lib.titans_mem_scan_surprise_path(ctypes.byref(desc), ctypes.byref(mlp)) == b"phased_mfma"
    assert tm.lib.titans_mem_scan_surprise_workspace_size(ctypes.byref(desc), ctypes.byref(mlp)) == \
        tm.lib.titans_mem_scan_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    monkeypatch.delenv("TITANS_MEM_FORCE_GENERIC")
    monkeypatch.setenv("TITANS_MEM_FUSED_SINGLE", "1")   # the single-workgroup kernel has no norms
    assert tm.lib.titans_mem_scan_surprise_path(ctypes.byref(desc), ctypes.byref(mlp)) == b"phased_mfma"
    monkeypatch.delenv("TITANS_MEM_FUSED_SINGLE")
    assert tm.lib.titans_mem_scan_surprise_path(ctypes.byref(_desc(io=0)),
                                                ctypes.byref(tm.mlp_desc((64, 96, 64)))) == b"generic_fp32"
    bad = ctypes.c_size_t(-1).value
    assert tm.lib.titans_mem_scan_surprise_workspace_size(ctypes.byref(_desc(C=0)),
                                                          ctypes.byref(mlp)) == bad


@no_fake_pointers_on_gpu
def test_surprise_validation():
    mlp = tm.mlp_desc((64, 256, 64))
    B, T, H, d, P = 2, 64, 4, 64, 32768
    desc = _desc(B, T, H, d)
    desc.state_stride[:] = (H * P, P)
    desc.state0_stride[:] = (0, P)
    ptrs, end = _fake_ptrs()
    sur = end
    ws = end + 4096 * 4
    need = tm.lib.titans_mem_scan_surprise_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    st, msg = _scan_surprise(desc, mlp, ptrs, None, ws, need)
    assert st == INVALID and "surprise" in msg
    assert _scan_surprise(desc, mlp, ptrs, sur + 2, ws, need)[0] == INVALID      # misaligned
    assert _scan_surprise(desc, mlp, ptrs, ptrs["alpha"], ws, need)[0] == INVALID  # an input
    assert _scan_surprise(desc, mlp, ptrs, ptrs["y"], ws, need)[0] == INVALID    # an output
    assert _scan_surprise(desc, mlp, ptrs, ws, ws, need)[0] == INVALID          # the workspace
    assert _scan_surprise(desc, mlp, ptrs, sur, ws, need - 1)[0] == WORKSPACE


def test_linear_memory_path_selection(monkeypatch):
    """L = 1 with the squared-error bias and enough chunks: the sequence-parallel path;
    its workspace holds, per (memory, group), the generic kernel's area, the group's
    composed map and its start state."""
    lin = tm.mlp_desc((64, 64))
    long_ = _desc(B=1, T=4096, H=2, C=16)
    assert tm.lib.titans_mem_scan_path(ctypes.byref(long_), ctypes.byref(lin)) == b"linear_mfma"
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(B=1, T=4096, H=2, C=16, io=0)),
                                       ctypes.byref(lin)) == b"linear_fp32"
    # 4 chunks: no groups of 8 -> the ordinary generic kernel
    assert tm.lib.titans_mem_scan_path(ctypes.byref(_desc(B=1, T=64, H=2, C=16)),
                                       ctypes.byref(lin)) == b"generic_mfma"
    # another bias, the surprise call, a deeper memory: not linear
    d = _desc(B=1, T=4096, H=2, C=16)
    d.bias, d.bias_param = 1, 0.5
    assert tm.lib.titans_mem_scan_path(ctypes.byref(d), ctypes.byref(lin)) == b"generic_mfma"
    assert tm.lib.titans_mem_scan_surprise_path(ctypes.byref(long_), ctypes.byref(lin)) == b"generic_mfma"
    assert tm.lib.titans_mem_scan_path(ctypes.byref(long_), ctypes.byref(tm.mlp_desc((64, 64, 64)))) \
        == b"generic_mfma"
    # 256 chunks, 2 memories: 512 / 2 = 256 groups, capped at 256 / 8 = 32 groups of 8 chunks
    r64 = lambda x: (x + 63) // 64 * 64
    C, dd, P = 16, 64, 64 * 64
    gen = r64(3 * C + 3) + r64((C + 1) * C) + r64(C * dd) + r64(C * dd) + 2 * r64(C * dd) + r64(C * C)
    summ = 16 * r64(dd * dd) + 2 * r64(C * dd) + 2 * r64(C)
    assert tm.lib.titans_mem_scan_workspace_size(ctypes.byref(long_), ctypes.byref(lin)) == \
        2 * 32 * (gen + summ + 2 * P) * 4
    monkeypatch.setenv("TITANS_MEM_LINEAR", "0")
    assert tm.lib.titans_mem_scan_path(ctypes.byref(long_), ctypes.byref(lin)) == b"generic_mfma"


def test_backward_workspace_formula():
    """Per memory: one (theta, s) checkpoint per chunk (each half padded to 16 bytes), then
    for segments of up to 32 chunks three record buffers and one working area per chunk, and
    one working area for the sequential part -- every region rounded up to 64 floats."""
    r64 = lambda x: (x + 63) // 64 * 64
    widths = (16, 32, 16)
    B, T, H, C = 2, 300, 3, 64
    n = widths
    L = len(n) - 1
    P = 16 * 32 * 2
    PH = (P + 3) // 4 * 4
    maxw = max(n)
    hid = sum(r64(C * n[l]) for l in range(1, L))          # layers 1..L-1
    out = sum(r64(C * n[l]) for l in range(1, L + 1))      # layers 1..L
    low = sum(r64(C * n[l]) for l in range(L))             # layers 0..L-1
    rec = (5 * r64(C + 1) + 4 * r64((C + 1) * C) + 64 + low + 2 * hid + out
           + r64(C * n[L]) + 2 * r64(C * n[0]) + 2 * r64(PH))
    chunk = low + hid + out + 3 * L * r64(C * C) + out + hid + out + r64(C * maxw)
    seq = out + hid + out + r64(C * maxw) + 64
    nch = (T + C - 1) // C
    seg = min(nch, 32)
    d = _desc(B, T, H, 16, C, io=0)
    got = tm.lib.titans_mem_scan_backward_workspace_size(ctypes.byref(d),
                                                         ctypes.byref(tm.mlp_desc(widths)))
    assert got == B * H * (nch * 2 * PH + seg * (3 * rec + chunk) + seq) * 4
    long_ = _desc(1, 64 * 200, 2, 16, C, io=0)  # 200 chunks: segments of 32
    got = tm.lib.titans_mem_scan_backward_workspace_size(ctypes.byref(long_),
                                                         ctypes.byref(tm.mlp_desc(widths)))
    assert got == 2 * (200 * 2 * PH + 32 * (3 * rec + chunk) + seq) * 4
    assert tm.lib.titans_mem_scan_backward_workspace_size(
        ctypes.byref(_desc(T=0)), ctypes.byref(tm.mlp_desc(widths))) == 0
    bad = ctypes.c_size_t(-1).value
    assert tm.lib.titans_mem_scan_backward_workspace_size(
        ctypes.byref(_desc(C=0)), ctypes.byref(tm.mlp_desc(widths))) == bad
    lp = _desc()
    lp.bias, lp.bias_param = 2, 1.5   # l_p below p = 2 has no second derivative at 0
    assert tm.lib.titans_mem_scan_backward_workspace_size(
        ctypes.byref(lp), ctypes.byref(tm.mlp_desc((64, 256, 64)))) == bad


_BWD_IN = ("q", "k", "v", "alpha", "eta", "beta", "theta0", "s0", "dy", "dtheta_T", "ds_T")
_BWD_OUT = ("dq", "dk", "dv", "dalpha", "deta", "dbeta", "dtheta0", "ds0")


def _bwd(desc, mlp, ptrs, ws=None, ws_bytes=0):
    args = [ptrs.get(n) for n in _BWD_IN + _BWD_OUT]
    st = tm.lib.titans_mem_scan_backward(ctypes.byref(desc), ctypes.byref(mlp), *args, ws,
                                         ws_bytes, None)
    assert st != HIP, "validation let the call through to HIP"
    return st, tm.lib.titans_last_error().decode()


def _fake_bwd_ptrs(B, T, H, d, P, esz=2, base=1 << 40):
    io = B * T * H * d * esz
    gate = B * T * H * 4
    state = B * H * P * 4
    sizes = {"q": io, "k": io, "v": io, "alpha": gate, "eta": gate, "beta": gate,
             "theta0": state, "s0": state, "dy": io, "dtheta_T": state, "ds_T": state,
             "dq": io, "dk": io, "dv": io, "dalpha": gate, "deta": gate, "dbeta": gate,
             "dtheta0": state, "ds0": state}
    out, cur = {}, base
    for n, s in sizes.items():
        out[n] = cur
        cur += (s + 4095) // 4096 * 4096
    return out, cur


def test_backward_rejects_unsupported_bias_and_null_pointers():
    mlp = tm.mlp_desc((64, 256, 64))
    d = _desc()
    d.bias, d.bias_param = 2, 1.0
    st, msg = _bwd(d, mlp, {})
    assert st == UNSUPPORTED and "l_p" in msg
    for bias, prm in ((0, 0.0), (1, 0.5), (2, 2.0), (2, 3.5)):
        d = _desc()
        d.bias, d.bias_param = bias, prm
        st, msg = _bwd(d, mlp, {})
        assert st == INVALID and "non-NULL" in msg, (bias, prm, msg)


@no_fake_pointers_on_gpu
def test_backward_validation_of_overlap_and_workspace():
    mlp = tm.mlp_desc((64, 256, 64))
    B, T, H, d, P = 2, 64, 4, 64, 32768
    desc = _desc(B, T, H, d)
    desc.state_stride[:] = (H * P, P)
    desc.state0_stride[:] = (H * P, P)
    ptrs, end = _fake_bwd_ptrs(B, T, H, d, P)
    need = tm.lib.titans_mem_scan_backward_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    assert need > 0
    for out in _BWD_OUT:   # every output against an input and against another output
        for other in ("q", "dy", "alpha", "theta0", "dq", "dalpha"):
            if other == out:
                continue
            st, msg = _bwd(desc, mlp, dict(ptrs, **{out: ptrs[other]}), end, need)
            assert st == INVALID, (out, other, msg)
    # the in-place pairs are allowed up to the workspace check
    st, msg = _bwd(desc, mlp, dict(ptrs, dtheta0=ptrs["dtheta_T"], ds0=ptrs["ds_T"]), None, 0)
    assert st == WORKSPACE, msg
    # dtheta_T may not feed the other state output
    st, msg = _bwd(desc, mlp, dict(ptrs, ds0=ptrs["dtheta_T"]), end, need)
    assert st == INVALID
    assert _bwd(desc, mlp, dict(ptrs, dq=ptrs["dq"] + 2), end, need)[0] == INVALID
    assert _bwd(desc, mlp, dict(ptrs, dalpha=ptrs["dalpha"] + 1), end, need)[0] == INVALID
    assert _bwd(desc, mlp, ptrs, end, need - 1)[0] == WORKSPACE
    assert _bwd(desc, mlp, ptrs, end + 64, need)[0] == INVALID
    assert _bwd(desc, mlp, ptrs, ptrs["dv"], need)[0] == INVALID
    shared = _desc(B, T, H, d)
    shared.state_stride[:] = (0, P)   # one dtheta0 written by several batch rows
    shared.state0_stride[:] = (0, P)
    assert _bwd(shared, mlp, ptrs, end, need)[0] == INVALID


# ---------------------------------------------------------------- MAG block

def _mag_desc(B=2, T=100, H=2, C=16, W=32, eta=0.1):
    return tm.MagDesc(B, T, H, C, W, eta, 0)


def _a256(x):
    return (x + 255) // 256 * 256


def test_mag_workspace_formula():
    widths = (64, 256, 64)
    mlp = tm.mlp_desc(widths)
    for B, T, H, C in [(2, 100, 2, 16), (8, 16384, 16, 64), (1, 1, 3, 1)]:
        d = widths[0]
        D, M = H * d, B * T
        ldp = (3 * D + 3 * H + 3) // 4 * 4
        own = _a256(_a256(M * ldp * 4) + 5 * _a256(M * D * 2) + 3 * _a256(M * H * 4))
        sd = _desc(B, T, H, d)
        sd.chunk = C
        P = tm.param_count(widths)
        sd.qkv_stride[:] = (T * D, D, d)
        sd.y_stride[:] = (T * D, D, d)
        sd.gate_stride[:] = (T * H, H, 1)
        sd.state_stride[:] = (H * P, P)
        sd.state0_stride[:] = (H * P, P)
        scan_ws = tm.lib.titans_mem_scan_workspace_size(ctypes.byref(sd), ctypes.byref(mlp))
        got = tm.lib.titans_mag_workspace_size(ctypes.byref(_mag_desc(B, T, H, C)), ctypes.byref(mlp))
        assert got == own + scan_ws, (B, T, H, C)
    assert tm.lib.titans_mag_workspace_size(ctypes.byref(_mag_desc(0, 5, 2)), ctypes.byref(mlp)) == 0


def test_mag_descriptor_validation():
    big = ctypes.c_size_t(-1).value
    ok = tm.mlp_desc((64, 256, 64))
    size = lambda desc, mlp=ok: tm.lib.titans_mag_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    assert size(_mag_desc()) != big
    for bad in (_mag_desc(W=0), _mag_desc(C=0), _mag_desc(H=0), _mag_desc(B=-1),
                _mag_desc(eta=float("nan")), _mag_desc(eta=-1.0), _mag_desc(eta=float("inf")),
                tm.MagDesc(2, 100, 2, 16, 32, 0.1, 7)):
        assert size(bad) == big
    assert size(_mag_desc(), tm.mlp_desc((64, 256, 32))) == big   # output width != d
    assert size(_mag_desc(), tm.mlp_desc((16, 32, 16))) == big     # d not 32 / 64 / 128
    assert size(_mag_desc(H=1025)) == big                         # H d > 65536


_MAG_ORDER = ("x", "w_in", "b_gate", "w_out", "theta0", "s0", "out", "theta_T", "s_T")


def _fake_mag_ptrs(B, T, H, d, P):
    D = H * d
    sizes = {"x": B * T * D * 2, "w_in": (3 * D + 3 * H) * D * 2, "b_gate": 3 * H * 4,
             "w_out": D * D * 2, "theta0": B * H * P * 4, "s0": B * H * P * 4,
             "out": B * T * D * 2, "theta_T": B * H * P * 4, "s_T": B * H * P * 4}
    base, ptrs = 1 << 40, {}
    for n in _MAG_ORDER:
        ptrs[n] = base
        base = _a256(base + sizes[n] + 256)
    return ptrs, base


def _mag(desc, mlp, ptrs, ws, ws_bytes):
    args = [ctypes.c_void_p(ptrs[n]) for n in _MAG_ORDER]
    st = tm.lib.titans_mag_forward(ctypes.byref(desc), ctypes.byref(mlp), *args,
                                   ctypes.c_void_p(ws), ws_bytes, None)
    return st, tm.lib.titans_last_error().decode()


@no_fake_pointers_on_gpu
def test_mag_validation_of_pointers_overlap_and_workspace():
    widths = (64, 256, 64)
    mlp = tm.mlp_desc(widths)
    B, T, H, d = 2, 100, 2, 64
    P = tm.param_count(widths)
    desc = _mag_desc(B, T, H)
    ptrs, end = _fake_mag_ptrs(B, T, H, d, P)
    need = tm.lib.titans_mag_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    for n in _MAG_ORDER:
        st, msg = _mag(desc, mlp, dict(ptrs, **{n: 0}), end, need)
        assert st == INVALID and "NULL" in msg, (n, msg)
    for n, off in (("x", 8), ("w_in", 2), ("w_out", 8), ("out", 2), ("b_gate", 2), ("theta0", 4),
                   ("theta_T", 8)):
        st, msg = _mag(desc, mlp, dict(ptrs, **{n: ptrs[n] + off}), end, need)
        assert st == INVALID and "aligned" in msg, (n, msg)
    for o in ("out", "theta_T", "s_T"):
        for i in ("x", "w_in", "b_gate", "w_out", "theta0", "s0", "out", "theta_T", "s_T"):
            if i == o:
                continue
            st, msg = _mag(desc, mlp, dict(ptrs, **{o: ptrs[i]}), end, need)
            assert st == INVALID and "overlap" in msg, (o, i, msg)
    assert _mag(desc, mlp, ptrs, end, need - 1)[0] == WORKSPACE
    assert _mag(desc, mlp, ptrs, 0, need)[0] == WORKSPACE
    assert _mag(desc, mlp, ptrs, end + 64, need)[0] == INVALID
    st, msg = _mag(desc, mlp, ptrs, ptrs["x"], need)
    assert st == INVALID and "overlap" in msg


# ---------------------------------------------------------------- MAC block

def test_mac_workspace_formula_and_validation():
    widths = (64, 256, 64)
    mlp = tm.mlp_desc(widths)
    P = tm.param_count(widths)
    big = ctypes.c_size_t(-1).value
    for B, T, H, C, Sg in [(2, 100, 2, 16, 48), (8, 16384, 16, 64, 4096), (1, 7, 3, 1, 1000)]:
        d = widths[0]
        D, M = H * d, B * T
        ldp = (3 * D + 3 * H + 3) // 4 * 4
        mag_own = _a256(_a256(M * ldp * 4) + 5 * _a256(M * D * 2) + 3 * _a256(M * H * 4))
        scan_ws = 0
        for L in (min(Sg, T), T % Sg):
            if L == 0:
                continue
            sd = _desc(B, L, H, d)
            sd.chunk = C
            sd.qkv_stride[:] = (T * D, D, d)
            sd.y_stride[:] = (T * D, D, d)
            sd.gate_stride[:] = (T * H, H, 1)
            sd.state_stride[:] = (H * P, P)
            sd.state0_stride[:] = (H * P, P)
            scan_ws = max(scan_ws, tm.lib.titans_mem_scan_workspace_size(ctypes.byref(sd),
                                                                         ctypes.byref(mlp)))
        got = tm.lib.titans_mac_workspace_size(ctypes.byref(tm.MacDesc(B, T, H, C, Sg, 0.1, 0)),
                                               ctypes.byref(mlp))
        assert got == mag_own + _a256(M * D * 2) + scan_ws, (B, T, H, C, Sg)
    size = lambda desc: tm.lib.titans_mac_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
    assert size(tm.MacDesc(0, 5, 2, 16, 8, 0.1, 0)) == 0
    for bad in (tm.MacDesc(2, 100, 2, 16, 0, 0.1, 0), tm.MacDesc(2, 100, 2, 0, 8, 0.1, 0),
                tm.MacDesc(2, 100, 0, 16, 8, 0.1, 0), tm.MacDesc(2, 100, 2, 16, 8, -1.0, 0),
                tm.MacDesc(2, 100, 2, 16, 8, 0.1, 1)):
        assert size(bad) == big


@no_fake_pointers_on_gpu
def test_mac_validation_of_pointers_and_workspace():
    widths = (64, 256, 64)
    mlp = tm.mlp_desc(widths)
    B, T, H, d = 2, 100, 2, 64
    desc = tm.MacDesc(B, T, H, 16, 48, 0.1, 0)
    ptrs, end = _fake_mag_ptrs(B, T, H, d, tm.param_count(widths))
    need = tm.lib.titans_mac_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))

    def call(p, ws, n):
        args = [ctypes.c_void_p(p[k]) for k in _MAG_ORDER]
        st = tm.lib.titans_mac_forward(ctypes.byref(desc), ctypes.byref(mlp), *args,
                                       ctypes.c_void_p(ws), n, None)
        return st, tm.lib.titans_last_error().decode()

    for n in _MAG_ORDER:
        st, msg = call(dict(ptrs, **{n: 0}), end, need)
        assert st == INVALID and "NULL" in msg, (n, msg)
    for o in ("out", "theta_T", "s_T"):
        st, msg = call(dict(ptrs, **{o: ptrs["x"]}), end, need)
        assert st == INVALID and "overlap" in msg
    assert call(ptrs, end, need - 1)[0] == WORKSPACE
    assert call(ptrs, end + 64, need)[0] == INVALID
