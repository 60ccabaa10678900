"""Seeded synthetic inputs for the Titans memory scan (shared by both sides).

This module only draws numbers: it holds none of the scan's arithmetic.  The
GPU tests, the bench and the oracle-side tests all take their inputs from
here, so the HIP path and the oracle see exactly the same values.

Recipe (the memory workloads on the Titans pages carry no data of their own;
these shapes stand in for the 4K training length, the 16K needle-in-a-haystack
length and the ">2M token" context claim):

* q, k, v ~ N(0, 1) per element, drawn in C order over [B, T, H, d]; q and k
  are then L2-normalised per (b, t, h) over d in float64.
* alpha_t = sigmoid(N(mu_alpha, 1)), eta_t = eta_scale * sigmoid(N(0, 1)),
  beta_t = sigmoid(N(2, 1)), one draw per (b, t, h), computed in float64.
* theta0: layer by layer, W_l ~ N(0, 1 / n_{l-1}) per head (shared by every
  batch row); s0 = 0.
* Storage: gates and theta0 are rounded to float32.  q/k/v are float32 for the
  fp32 workload; for bf16 workloads they are rounded float64 -> float32 (RNE)
  -> bfloat16 (RNE) and kept as raw uint16 bit patterns.

Every (tensor, batch row, block of 4096 tokens) has its own PCG64 stream keyed
by ``SeedSequence(seed, spawn_key=(tensor, b, block))``, so a prefix of T is the
same whatever the total length, and blocks can be drawn in parallel.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK_TOKENS = 4096

# tensor ids for the stream keys
_Q, _K, _V, _ALPHA, _ETA, _BETA, _THETA, _DY, _DTHETA, _DS, _X, _WIN, _WOUT = range(13)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    widths: tuple        # n_0 .. n_L (n_0 = n_L = d)
    chunk: int
    io: str              # "f32" or "bf16"
    alpha_mu: float = -4.0
    eta_scale: float = 0.1
    beta_mu: float = 2.0

    @property
    def d(self) -> int:
        return self.widths[0]

    @property
    def n_layers(self) -> int:
        return len(self.widths) - 1

    @property
    def params(self) -> int:
        w = self.widths
        return int(sum(w[i] * w[i - 1] for i in range(1, len(w))))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny fp32 reference: 1 head, batch 1, T=512, C=16, MLP 16->64->16
    "tiny_f32_h1_t512": Workload("tiny_f32_h1_t512", 1, 1, 512, (16, 64, 16), 16, "f32"),
    # 8 heads x d64, batch 4, T=4096, C=64, MLP 64->256->64
    "h8_d64_b4_t4k": Workload("h8_d64_b4_t4k", 4, 8, 4096, (64, 256, 64), 64, "bf16"),
    # 16 heads x d64, batch 8, T=16384, C=64, MLP 64->256->64 (the headline workload)
    "h16_d64_b8_t16k": Workload("h16_d64_b8_t16k", 8, 16, 16384, (64, 256, 64), 64, "bf16"),
    # deeper memory: 8 heads x d128, batch 2, T=32768, C=128, MLP 128->512->512->512->128
    "deep_h8_d128_b2_t32k": Workload("deep_h8_d128_b2_t32k", 2, 8, 32768,
                                     (128, 512, 512, 512, 128), 128, "bf16",
                                     alpha_mu=-5.0, eta_scale=0.05),
    # long-context streaming: 16 heads x d64, batch 1, T=2^21, C=256
    "long_h16_d64_b1_t2m": Workload("long_h16_d64_b1_t2m", 1, 16, 2097152, (64, 256, 64), 256,
                                    "bf16"),
    # derived (not one of the pages' configurations): the long-context shape with a linear
    # memory 64->64 (the delta-rule case) at T=2^18, for the sequence-parallel linear path
    "linear_h16_d64_b1_t256k": Workload("linear_h16_d64_b1_t256k", 1, 16, 262144, (64, 64), 256,
                                        "bf16"),
}

HEADLINE = "h16_d64_b8_t16k"

# Gate mixes that keep every memory O(1) to the end of its sequence.  With the specified
# gates and i.i.d. q/k/v the memory decays to its zero fixed point within a few thousand
# tokens, so each full shape is also run with alpha_t = sigmoid(N(mu, 1)) for a lower mu
# (and, with C = 256, a smaller eta scale: there eta = 0.1 sigmoid(.) diverges in the fp64
# recurrence itself).  (alpha_mu, eta_scale) per workload.
SUSTAINED = {"h8_d64_b4_t4k": (-7.0, 0.1), "h16_d64_b8_t16k": (-7.0, 0.1),
             "deep_h8_d128_b2_t32k": (-8.0, 0.05), "long_h16_d64_b1_t2m": (-10.0, 0.02)}


def sustained(wl: "Workload | str") -> "Workload":
    """The workload with its sustained gate mix (name suffixed "_sustained")."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    mu, es = SUSTAINED[wl.name]
    return wl.with_(alpha_mu=mu, eta_scale=es, name=wl.name + "_sustained")


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: np.ndarray        # [B,T,H,d]: float32, or uint16 bf16 bits
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray    # [B,T,H] float32
    eta: np.ndarray
    beta: np.ndarray
    theta0: np.ndarray   # [H,P] float32
    s0: np.ndarray       # [H,P] float32

    def qkv_f32(self, name: str) -> np.ndarray:
        """q/k/v as float32 values (exact for bf16 storage)."""
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def _rng(seed: int, *key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_vectors(seed, tensor, wl, B, T, normalise, out):
    """Fill out[b, t0:t1] block by block with N(0,1) rows of length d."""
    H, d = wl.heads, wl.d

    def one(bi_blk):
        b, blk = bi_blk
        t0 = blk * BLOCK_TOKENS
        t1 = min(T, t0 + BLOCK_TOKENS)
        x = _rng(seed, tensor, b, blk).standard_normal((BLOCK_TOKENS, H, d))[: t1 - t0]
        if normalise:
            x = x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        x32 = x.astype(np.float32)
        out[b, t0:t1] = f32_to_bf16_bits(x32) if wl.io == "bf16" else x32

    jobs = [(b, blk) for b in range(B) for blk in range((T + BLOCK_TOKENS - 1) // BLOCK_TOKENS)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, jobs))


def _draw_gate(seed, tensor, wl, B, T, transform):
    H = wl.heads
    out = np.empty((B, T, H), dtype=np.float32)
    for b in range(B):
        for blk in range((T + BLOCK_TOKENS - 1) // BLOCK_TOKENS):
            t0 = blk * BLOCK_TOKENS
            t1 = min(T, t0 + BLOCK_TOKENS)
            z = _rng(seed, tensor, b, blk).standard_normal((BLOCK_TOKENS, H))[: t1 - t0]
            out[b, t0:t1] = transform(z).astype(np.float32)
    return out


def make_theta0(wl: Workload, seed: int) -> np.ndarray:
    H, w = wl.heads, wl.widths
    th = np.empty((H, wl.params), dtype=np.float32)
    for h in range(H):
        off = 0
        for l in range(1, len(w)):
            n = w[l] * w[l - 1]
            th[h, off:off + n] = (_rng(seed, _THETA, h, l).standard_normal(n)
                                  / np.sqrt(w[l - 1])).astype(np.float32)
            off += n
    return th


def make_gates(wl: Workload, seed: int, T: int, B: int):
    """alpha, eta, beta [B, T, H] float32 (the same streams as make_inputs draws)."""
    alpha = _draw_gate(seed, _ALPHA, wl, B, T, lambda z: _sigmoid(z + wl.alpha_mu))
    eta = _draw_gate(seed, _ETA, wl, B, T, lambda z: wl.eta_scale * _sigmoid(z))
    beta = _draw_gate(seed, _BETA, wl, B, T, lambda z: _sigmoid(z + wl.beta_mu))
    return alpha, eta, beta


def make_inputs(wl: Workload | str, seed: int = 0, seq_len: int | None = None,
                batch: int | None = None) -> Inputs:
    """Draw the workload's inputs.  seq_len / batch override T / B (prefix-consistent)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B = wl.batch if batch is None else batch
    T = wl.seq_len if seq_len is None else seq_len
    H, d = wl.heads, wl.d
    qdt = np.uint16 if wl.io == "bf16" else np.float32
    q = np.empty((B, T, H, d), dtype=qdt)
    k = np.empty((B, T, H, d), dtype=qdt)
    v = np.empty((B, T, H, d), dtype=qdt)
    _draw_vectors(seed, _Q, wl, B, T, True, q)
    _draw_vectors(seed, _K, wl, B, T, True, k)
    _draw_vectors(seed, _V, wl, B, T, False, v)
    alpha, eta, beta = make_gates(wl, seed, T, B)
    theta0 = make_theta0(wl, seed)
    s0 = np.zeros_like(theta0)
    return Inputs(wl.with_(batch=B, seq_len=T), q, k, v, alpha, eta, beta, theta0, s0)


@dataclasses.dataclass
class Cotangents:
    """Output cotangents for the reverse pass: dy like y, dtheta_T and ds_T [B,H,P]."""
    dy: np.ndarray       # [B,T,H,d]: float32, or uint16 bf16 bits
    dtheta_T: np.ndarray  # [B,H,P] float32
    ds_T: np.ndarray

    def dy_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.dy) if self.dy.dtype == np.uint16 else self.dy


def make_cotangents(wl: Workload | str, seed: int = 0, seq_len: int | None = None,
                    batch: int | None = None, state_scale: float = 0.1) -> Cotangents:
    """Seeded output cotangents (the pages give none; a downstream loss's gradient stands in):
    dy ~ N(0, 1) per element, stored like q (bf16 bits for bf16 workloads, prefix-consistent
    in T like the inputs); dtheta_T, ds_T ~ state_scale * N(0, 1), float32."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B = wl.batch if batch is None else batch
    T = wl.seq_len if seq_len is None else seq_len
    H, d = wl.heads, wl.d
    dy = np.empty((B, T, H, d), dtype=np.uint16 if wl.io == "bf16" else np.float32)
    _draw_vectors(seed, _DY, wl, B, T, False, dy)
    P = wl.params
    dth = np.empty((B, H, P), dtype=np.float32)
    ds = np.empty((B, H, P), dtype=np.float32)
    for b in range(B):
        dth[b] = (state_scale * _rng(seed, _DTHETA, b).standard_normal((H, P))).astype(np.float32)
        ds[b] = (state_scale * _rng(seed, _DS, b).standard_normal((H, P))).astype(np.float32)
    return Cotangents(dy, dth, ds)


@dataclasses.dataclass
class MagInputs:
    """Inputs of one MAG block: x, the projection weights (out x in features, bf16 bits),
    the gate biases and the initial memory.  The weights are drawn so the projected q, k,
    v and gates follow the memory-scan recipe above: with x ~ N(0, 1) and weights
    ~ N(0, 1 / D), every projected feature is ~ N(0, 1); the gate biases are
    (alpha_mu, 0, beta_mu) per head."""
    workload: Workload   # batch, heads, seq_len, widths, chunk, eta_scale, alpha_mu, beta_mu
    window: int
    x: np.ndarray        # [B,T,D] uint16 bf16 bits
    w_in: np.ndarray     # [3D + 3H, D] uint16 bits: q, k, v rows, then alpha, eta, beta rows
    b_gate: np.ndarray   # [3H] float32
    w_out: np.ndarray    # [D, D] uint16 bits
    theta0: np.ndarray   # [H,P] float32 (the same for every batch row)
    s0: np.ndarray       # [H,P] float32

    def oracle_weights(self):
        """(Wq, Wk, Wv, Wg, bg, Wo) as float64 in the x @ W convention."""
        D = self.x.shape[2]
        w = bf16_bits_to_f32(self.w_in).astype(np.float64)
        wo = bf16_bits_to_f32(self.w_out).astype(np.float64)
        return (w[:D].T, w[D:2 * D].T, w[2 * D:3 * D].T, w[3 * D:].T,
                self.b_gate.astype(np.float64), wo.T)


def make_mag_inputs(wl: Workload | str, window: int, seed: int = 0, seq_len: int | None = None,
                    batch: int | None = None) -> MagInputs:
    """x ~ N(0, 1) per element over [B, T, D] (prefix-consistent in T), W_in and W_out rows
    ~ N(0, 1 / D), all rounded to bf16; theta0 as make_theta0, s0 = 0."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B = wl.batch if batch is None else batch
    T = wl.seq_len if seq_len is None else seq_len
    wl = wl.with_(batch=B, seq_len=T, io="bf16")
    H, d = wl.heads, wl.d
    D = H * d
    x = np.empty((B, T, H, d), dtype=np.uint16)
    _draw_vectors(seed, _X, wl, B, T, False, x)
    w_in = _rng(seed, _WIN).standard_normal((3 * D + 3 * H, D)) / np.sqrt(D)
    w_out = _rng(seed, _WOUT).standard_normal((D, D)) / np.sqrt(D)
    b_gate = np.concatenate([np.full(H, wl.alpha_mu), np.zeros(H), np.full(H, wl.beta_mu)])
    theta0 = make_theta0(wl, seed)
    return MagInputs(wl, int(window), x.reshape(B, T, D),
                     f32_to_bf16_bits(w_in.astype(np.float32)), b_gate.astype(np.float32),
                     f32_to_bf16_bits(w_out.astype(np.float32)), theta0, np.zeros_like(theta0))
