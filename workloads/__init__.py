"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws inputs (token streams, document offsets, hidden states
and head weights).  It holds none of the method's arithmetic and is shared by
the tests, the smoke check and the benchmark; both the HIP library and the
fp64 oracle consume what it returns.

No dataset or trained weight is available, so every workload is synthetic:
  * tokens are uniform over a stated id range;
  * document lengths are lognormal with the stated arithmetic mean and
    sigma 1, rounded and clipped to [16, 4096] (chunks are capped at 4,096
    tokens and those below 16 are discarded: LLaDA-8B-MDLM-LoRA card, Training table,
    "Data" row);
  * hidden states are N(0,1), row-wise RMS-normalised for the bf16 shapes;
  * the head W is N(0, 0.02^2), shape [V, H], row-major;
  * bf16 values are produced once by round-to-nearest-even from float32.

Each named workload draws from numpy.random.default_rng(1000 + k) with k its
index below, so every run and every machine sees the same inputs.
"""

import math
from dataclasses import dataclass, field

import numpy as np

NOISE_ABSORB = 0
NOISE_UNIFORM = 1
ALIGNED = 0
SHIFTED = 1


@dataclass
class Workload:
    name: str
    index: int            # 1..5 for the named workloads, seeds the generator
    dtype: str            # "f32" or "bf16"
    H: int
    V: int
    noise: int
    align: int
    mask_id: int
    rand_vocab: int
    eps: float
    softcap: float
    seed: int             # Philox seed of the corruption
    lengths: list = field(default_factory=list)
    token_lo: int = 0
    token_hi: int = 0     # exclusive
    token_skip: int = -1  # an id never drawn (the mask id of workload 4)
    rms_normalise: bool = True

    @property
    def n_tokens(self):
        return int(sum(self.lengths))

    @property
    def n_docs(self):
        return len(self.lengths)


def lognormal_lengths(rng, mean, total=None, count=None, lo=16, hi=4096):
    """Document lengths: lognormal with arithmetic mean ``mean`` and sigma 1
    (so mu = ln(mean) - 1/2), rounded and clipped to [lo, hi].  With ``count``
    draws that many; with ``total`` draws until the sum reaches ``total`` and
    trims the last document so the sum is exactly ``total``."""
    mu = math.log(mean) - 0.5
    if count is not None:
        x = rng.lognormal(mu, 1.0, size=count)
        return [int(v) for v in np.clip(np.rint(x), lo, hi)]
    out = []
    s = 0
    while s < total:
        v = int(np.clip(np.rint(rng.lognormal(mu, 1.0)), lo, hi))
        v = min(v, total - s)
        out.append(v)
        s += v
    return out


def lognormal_stream_offsets(seed, mean, total, lo=16, hi=4096):
    """Document offsets (cu_seqlens, int64) of a ``total``-token stream whose
    lengths are lognormal with arithmetic mean ``mean`` and sigma 1, rounded
    and clipped to [lo, hi], the last one trimmed so the lengths sum to
    ``total``.  Vectorised, for bandwidth-sized streams."""
    rng = np.random.default_rng(seed)
    mu = math.log(mean) - 0.5
    chunks, s = [], 0
    while s < total:
        x = np.clip(np.rint(rng.lognormal(mu, 1.0, size=max(1024, 2 * total // mean))), lo, hi)
        x = x.astype(np.int64)
        chunks.append(x)
        s += int(x.sum())
    lengths = np.concatenate(chunks)
    c = np.cumsum(lengths)
    k = int(np.searchsorted(c, total))
    lengths = lengths[:k + 1].copy()
    lengths[-1] -= int(c[k] - total)
    return np.concatenate([[0], np.cumsum(lengths)])


def make_workload(k):
    """The five named workloads, by index 1..5."""
    rng = np.random.default_rng(1000 + k)
    if k == 1:
        return Workload("tiny-absorb-f32", 1, "f32", H=128, V=1024,
                        noise=NOISE_ABSORB, align=ALIGNED, mask_id=1023,
                        rand_vocab=1024, eps=1e-3, softcap=0.0, seed=0,
                        lengths=[64, 64], token_lo=0, token_hi=1023,
                        rms_normalise=False)
    if k == 2:
        V = 126464
        return Workload("llada8b-1x4096", 2, "bf16", H=4096, V=V,
                        noise=NOISE_ABSORB, align=ALIGNED, mask_id=V - 128,
                        rand_vocab=V, eps=1e-3, softcap=0.0, seed=0,
                        lengths=[4096], token_lo=0, token_hi=V - 128)
    if k == 3:
        V = 126464
        return Workload("llada8b-varlen-12docs", 3, "bf16", H=4096, V=V,
                        noise=NOISE_ABSORB, align=ALIGNED, mask_id=V - 128,
                        rand_vocab=V, eps=1e-3, softcap=0.0, seed=0,
                        lengths=lognormal_lengths(rng, 296, count=12),
                        token_lo=0, token_hi=V - 128)
    if k == 4:
        V = 131072
        return Workload("nemotron3b-packed-16384", 4, "bf16", H=3072, V=V,
                        noise=NOISE_ABSORB, align=ALIGNED, mask_id=100,
                        rand_vocab=V, eps=1e-3, softcap=0.0, seed=0,
                        lengths=lognormal_lengths(rng, 512, total=16384),
                        token_lo=0, token_hi=V, token_skip=100)
    if k == 5:
        V = 262144
        return Workload("diffusiongemma-canvas-8x1024", 5, "bf16", H=2816, V=V,
                        noise=NOISE_UNIFORM, align=ALIGNED, mask_id=-1,
                        rand_vocab=V, eps=1e-3, softcap=30.0, seed=0,
                        lengths=[1024] * 8, token_lo=0, token_hi=V)
    raise ValueError(f"unknown workload {k}")


def draw_tokens(rng, n, lo, hi, skip=-1):
    """Uniform ids in [lo, hi), never ``skip`` (drawn from [lo, hi-1) and
    shifted past it)."""
    if skip >= lo and skip < hi:
        x = rng.integers(lo, hi - 1, size=n, dtype=np.int64)
        x[x >= skip] += 1
    else:
        x = rng.integers(lo, hi, size=n, dtype=np.int64)
    return x.astype(np.int32)


def cu_from_lengths(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def _round_bf16(x32, block=1 << 24):
    """float32 -> nearest bf16 (ties to even; inputs are finite), returned as
    float32 values and as the raw uint16 bit patterns.  Works in blocks to
    bound temporary memory."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    flat = x32.reshape(-1)
    bits = np.empty(flat.shape, dtype=np.uint16)
    vals = np.empty(flat.shape, dtype=np.float32)
    for s in range(0, flat.size, block):
        u = flat[s:s + block].view(np.uint32)
        rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        b = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
        bits[s:s + block] = b
        vals[s:s + block] = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return vals.reshape(x32.shape), bits.reshape(x32.shape)


@dataclass
class Inputs:
    wl: Workload
    x0: np.ndarray          # int32[N]
    cu_seqlens: np.ndarray  # int32[B+1]
    hidden: np.ndarray      # float32[N,H] (values exactly representable in dtype)
    W: np.ndarray           # float32[V,H]
    hidden_bits: np.ndarray = None  # uint16 bf16 patterns, bf16 workloads only
    W_bits: np.ndarray = None


def generate(wl, with_hidden=True, with_head=True):
    """Draw the inputs of a workload.  Same workload -> same arrays."""
    rng = np.random.default_rng(1000 + wl.index)
    # replay the length draws of make_workload so the stream continues past them
    if wl.index == 3:
        lognormal_lengths(rng, 296, count=12)
    elif wl.index == 4:
        lognormal_lengths(rng, 512, total=16384)
    n = wl.n_tokens
    x0 = draw_tokens(rng, n, wl.token_lo, wl.token_hi, wl.token_skip)
    cu = cu_from_lengths(wl.lengths)
    hidden = W = hb = wb = None
    # hidden states and head weights come from their own streams, so drawing
    # one without the other leaves the values unchanged
    if with_hidden:
        rng_h = np.random.default_rng((1000 + wl.index, 1))
        h = rng_h.standard_normal((n, wl.H), dtype=np.float32)
        if wl.rms_normalise:
            h = h / np.sqrt(np.mean(h.astype(np.float64) ** 2, axis=1,
                                    keepdims=True)).astype(np.float32)
        if wl.dtype == "bf16":
            hidden, hb = _round_bf16(h)
        else:
            hidden = h
    if with_head:
        rng_w = np.random.default_rng((1000 + wl.index, 2))
        w = rng_w.standard_normal((wl.V, wl.H), dtype=np.float32)
        w *= np.float32(0.02)
        if wl.dtype == "bf16":
            W, wb = _round_bf16(w)
        else:
            W = w
    return Inputs(wl, x0, cu, hidden, W, hb, wb)


def small_case(seed, n_docs, max_len, H, V, dtype="bf16", noise=NOISE_ABSORB,
               align=ALIGNED, softcap=0.0, eps=1e-3, empty_docs=False,
               philox_seed=None, hidden_scale=1.0, w_scale=0.02, lengths=None):
    """A small random case for parity tests: random document lengths in
    [1, max_len] (some zero when ``empty_docs``), or the given ``lengths``,
    uniform tokens over [0, V-1), mask id V-1, hidden N(0, hidden_scale^2),
    head N(0, w_scale^2)."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(1, max_len + 1, size=n_docs)
        if empty_docs:
            lengths[rng.random(n_docs) < 0.25] = 0
    else:
        lengths = np.asarray(lengths, dtype=np.int64)
    wl = Workload(f"small-{seed}", 0, dtype, H=H, V=V, noise=noise, align=align,
                  mask_id=V - 1, rand_vocab=V, eps=eps, softcap=softcap,
                  seed=seed if philox_seed is None else philox_seed,
                  lengths=[int(v) for v in lengths], token_lo=0, token_hi=V - 1,
                  rms_normalise=False)
    n = wl.n_tokens
    x0 = draw_tokens(rng, n, 0, V - 1)
    cu = cu_from_lengths(wl.lengths)
    h = rng.standard_normal((n, H), dtype=np.float32) * np.float32(hidden_scale)
    w = rng.standard_normal((V, H), dtype=np.float32) * np.float32(w_scale)
    if dtype == "bf16":
        hidden, hb = _round_bf16(h)
        W, wb = _round_bf16(w)
        return Inputs(wl, x0, cu, hidden, W, hb, wb)
    return Inputs(wl, x0, cu, h, w)
