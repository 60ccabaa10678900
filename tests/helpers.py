"""Shared test helpers: device transfer of synthetic inputs and error measures."""
import numpy as np

import synthetic


def to_device(inp: synthetic.Inputs, device="cuda:0"):
    """Synthetic inputs as torch tensors on the device (bf16 from the stored bits, exactly)."""
    import torch

    out = {}
    for name in ("q", "k", "v"):
        a = np.ascontiguousarray(getattr(inp, name))
        if a.dtype == np.uint16:
            out[name] = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            out[name] = torch.from_numpy(a).to(device)
    for name in ("alpha", "eta", "beta", "theta0", "s0"):
        out[name] = torch.from_numpy(np.ascontiguousarray(getattr(inp, name))).to(device)
    return out


def to_f64(t) -> np.ndarray:
    """torch tensor (any float dtype, any device) -> float64 numpy."""
    import torch

    return t.detach().to(torch.float64).cpu().numpy()


F32_MIN_NORMAL = 2.0 ** -126

# A reference state below this norm has decayed out of float32's range in practice (the
# memory's zero fixed point): its relative error carries no information, so the state
# checks skip it (and say so) instead of passing against a floor.
DECAYED_STATE = 1e-20


def rel_err_slices(x, ref, axes):
    """max over slices of ||x - ref||_F / max(||ref||_F, floor); `axes` are reduced.

    floor = (smallest normal float32) * sqrt(elements per slice): once the reference has
    decayed below float32's normal range a float32 result cannot carry relative precision,
    so the error is measured against that floor instead (an absolute bar of ~1e-38).
    """
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    count = np.prod([ref.shape[a] for a in axes])
    floor = F32_MIN_NORMAL * np.sqrt(max(count, 1))
    return float(np.max(num / np.maximum(den, floor)))


def y_rel_err(y, y_ref):
    """y: [B,T,H,d]; per-(b,h) Frobenius relative error, max over (b,h)."""
    return rel_err_slices(y, y_ref, axes=(1, 3))


def state_rel_err(th, th_ref):
    """theta: [B,H,P]; per-(b,h) relative error, max over (b,h)."""
    return rel_err_slices(th, th_ref, axes=(2,))


def token_errors(y, y_ref, chunk, floor=2.0 ** -96):
    """Per-token error of one sequence, y and y_ref [T, d].

    e_t = ||y_t - ref_t|| / s_t, with s_t the RMS of the reference rows' norms over the
    chunk that holds token t (a local scale: an element of y_t is a sum over the hidden
    units, so its rounding error follows the size of the chunk's reads, not the size of
    y_t itself, which can cancel).  Chunks whose scale is below `floor` (a memory decayed
    to its zero fixed point, out of float32's relative precision) are left out.
    Returns (max e_t, 99th percentile, index of the worst token, tokens left out)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(y_ref, np.float64)
    T = ref.shape[0]
    err = np.sqrt(np.sum((y - ref) ** 2, axis=-1))
    nrm2 = np.sum(ref ** 2, axis=-1)
    nch = (T + chunk - 1) // chunk
    padded = np.concatenate([nrm2, np.full(nch * chunk - T, np.nan)]).reshape(nch, chunk)
    s = np.repeat(np.sqrt(np.nanmean(padded, axis=1)), chunk)[:T]
    keep = s > floor
    if not keep.any():
        return 0.0, 0.0, -1, T
    e = np.where(keep, err / np.where(keep, s, 1.0), 0.0)
    return float(e.max()), float(np.percentile(e[keep], 99)), int(e.argmax()), int(T - keep.sum())
