"""Seeded synthetic inputs shared, as data only, by the tests, the bench and
the oracle checks.  This module holds none of the attention arithmetic: it
draws standard-normal samples, rounds them to bfloat16 (round to nearest,
ties to even) when asked, and lays them out in the documented shapes.

Recipe
------
Every (tensor, batch index) slice has its own stream,
``numpy.random.default_rng([seed, tensor_id, b])``, drawn with
``standard_normal(shape, float32)``; tensor ids are q=0, k=1, v=2 (prefill and
MQA/GQA decode) and q_abs=0, latent=1 (MLA).  Varying decode lengths come
first, from ``default_rng([seed, 99]).integers(lo, hi, endpoint=True)``.
Per-slice streams let a check regenerate one sequence of a multi-gigabyte
cache without drawing the rest.  Cache rows at or beyond ``seq_lens[b]`` are
NaN, so any out-of-range read poisons the result.

bfloat16 tensors are kept as ``uint16`` bit patterns (what the device reads),
float16 tensors as numpy ``float16`` (numpy's float32 -> float16 conversion
rounds to nearest even); ``Tensor.f32()`` gives their exact float32 values
(what the oracle reads).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))


def _parallel(fn, items):
    """Run fn over items on a thread pool (numpy releases the GIL in the
    generator and in the rounding); results are independent of the order."""
    items = list(items)
    if len(items) <= 1 or _THREADS == 1:
        for it in items:
            fn(it)
        return
    with ThreadPoolExecutor(max_workers=_THREADS) as ex:
        list(ex.map(fn, items))

__all__ = [
    "bf16_bits",
    "bf16_to_f32",
    "round_bf16",
    "Tensor",
    "prefill_inputs",
    "decode_inputs",
    "mla_inputs",
    "draw_topk",
    "rope_tables",
    "mla_step_inputs",
    "draw_lengths",
    "Workload",
    "WORKLOADS",
]

_BF16_NAN = np.uint16(0x7FC0)


def bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.
    NaN maps to a quiet NaN pattern."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = _BF16_NAN
    return r


def bf16_to_f32(bits):
    """uint16 bfloat16 bit patterns -> exact float32 values."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x):
    return bf16_to_f32(bf16_bits(x))


@dataclass
class Tensor:
    """One input: float32 values (``dtype == "f32"``) or bf16 bit patterns."""
    data: np.ndarray              # float32, uint16 (bf16 bits) or float16
    dtype: str = "f32"

    @property
    def shape(self):
        return self.data.shape

    def f32(self, index=...):
        """Exact float32 values of ``data[index]``."""
        part = self.data[index]
        # (float16 -> float32 is exact)
        return bf16_to_f32(part) if self.dtype == "bf16" else np.asarray(part, dtype=np.float32)


def _draw(seed, tid, b, shape):
    return np.random.default_rng([seed, tid, b]).standard_normal(shape, dtype=np.float32)


def _store(shape, dtype):
    if dtype == "bf16":
        return np.empty(shape, dtype=np.uint16)
    if dtype == "f16":
        return np.empty(shape, dtype=np.float16)
    if dtype == "f32":
        return np.empty(shape, dtype=np.float32)
    raise ValueError(dtype)


def _put(dst, idx, vals, dtype):
    dst[idx] = bf16_bits(vals) if dtype == "bf16" else vals      # float16 stores round to nearest even


def _nan(dtype):
    return _BF16_NAN if dtype == "bf16" else (np.float16(np.nan) if dtype == "f16" else np.float32(np.nan))


def prefill_slice(seed, tid, b, H, T, D):
    """float32 draw of one batch slice ``[H, T, D]`` of q (tid 0), k (1), v (2)."""
    return _draw(seed, tid, b, (H, T, D))


def prefill_inputs(B, Hq, Hkv, T, D, dtype="bf16", seed=0, d_v=None, T_kv=None):
    """q [B,Hq,T,D], k [B,Hkv,T_kv,D], v [B,Hkv,T_kv,d_v], iid N(0,1)
    (T_kv defaults to T, d_v to D)."""
    d_v = D if d_v is None else d_v
    T_kv = T if T_kv is None else T_kv
    out = []
    for tid, (H, TT, dd) in enumerate(((Hq, T, D), (Hkv, T_kv, D), (Hkv, T_kv, d_v))):
        t = _store((B, H, TT, dd), dtype)
        _parallel(lambda b: _put(t, b, _draw(seed, tid, b, (H, TT, dd)), dtype), range(B))
        out.append(Tensor(t, dtype))
    return tuple(out)


def draw_lengths(B, lengths, L_max, seed):
    """seq_lens int32 [B]: None -> all L_max; int -> all equal; (lo, hi) ->
    uniform integers in [lo, hi]; a sequence -> taken as given."""
    if lengths is None:
        return np.full(B, L_max, dtype=np.int32)
    if isinstance(lengths, tuple):
        lo, hi = lengths
        return np.random.default_rng([seed, 99]).integers(lo, hi, endpoint=True, size=B).astype(np.int32)
    if np.ndim(lengths) == 1:
        return np.asarray(lengths, dtype=np.int32).copy()
    return np.full(B, int(lengths), dtype=np.int32)


def _cache(seed, tid, B, H, L_max, D, seq_lens, dtype, nan_pad, squeeze_head=False):
    shape = (B, L_max, D) if squeeze_head else (B, H, L_max, D)
    t = _store(shape, dtype)

    def one(b):
        L = int(seq_lens[b])
        if squeeze_head:
            _put(t, (b, slice(0, L)), _draw(seed, tid, b, (L, D)), dtype)
            if L < L_max:
                t[b, L:] = _nan(dtype) if nan_pad else 0
        else:
            _put(t, (b, slice(None), slice(0, L)), _draw(seed, tid, b, (H, L, D)), dtype)
            if L < L_max:
                t[b, :, L:] = _nan(dtype) if nan_pad else 0

    _parallel(one, range(B))
    return Tensor(t, dtype)


def decode_inputs(B, Hq, Hkv, L_max, D, dtype="bf16", seed=0, lengths=None,
                  nan_pad=True, d_v=None):
    """q [B,Hq,D]; k cache [B,Hkv,L_max,D]; v cache [B,Hkv,L_max,d_v];
    seq_lens int32 [B].  Rows >= seq_lens[b] are NaN when ``nan_pad``."""
    d_v = D if d_v is None else d_v
    seq_lens = draw_lengths(B, lengths, L_max, seed)
    q = _store((B, Hq, D), dtype)
    _parallel(lambda b: _put(q, b, _draw(seed, 0, b, (Hq, D)), dtype), range(B))
    k = _cache(seed, 1, B, Hkv, L_max, D, seq_lens, dtype, nan_pad)
    v = _cache(seed, 2, B, Hkv, L_max, d_v, seq_lens, dtype, nan_pad)
    return Tensor(q, dtype), k, v, seq_lens


def decode_slice(seed, b, Hq, Hkv, L, D, d_v=None):
    """float32 draws of sequence b only: (q [Hq,D], k [Hkv,L,D], v [Hkv,L,d_v])."""
    d_v = D if d_v is None else d_v
    return (_draw(seed, 0, b, (Hq, D)), _draw(seed, 1, b, (Hkv, L, D)),
            _draw(seed, 2, b, (Hkv, L, d_v)))


def mla_inputs(B, H, L_max, d_kv=576, dtype="bf16", seed=0, lengths=None,
               nan_pad=True):
    """q_abs [B,H,d_kv]; latent cache [B,L_max,d_kv]; seq_lens int32 [B]."""
    seq_lens = draw_lengths(B, lengths, L_max, seed)
    q = _store((B, H, d_kv), dtype)
    _parallel(lambda b: _put(q, b, _draw(seed, 0, b, (H, d_kv)), dtype), range(B))
    kv = _cache(seed, 1, B, 1, L_max, d_kv, seq_lens, dtype, nan_pad, squeeze_head=True)
    return Tensor(q, dtype), kv, seq_lens


def draw_topk(B, seq_lens, topk, seed):
    """Selected positions int32 [B, topk]: for sequence b, min(topk, L_b)
    distinct positions drawn uniformly from [0, L_b) with
    ``default_rng([seed, 98, b]).choice(L_b, n, replace=False)``, sorted
    ascending, then -1 padding."""
    idx = np.full((B, topk), -1, dtype=np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        n = min(topk, L)
        sel = np.random.default_rng([seed, 98, b]).choice(L, size=n, replace=False)
        idx[b, :n] = np.sort(sel).astype(np.int32)
    return idx


def rope_tables(positions, dim=64, base=10000.0):
    """Rotary factors (cos, sin) float32 [n, dim] for integer positions, in
    the usual table layout: inv_freq_i = base^(-2i/dim) for i < dim/2,
    angle = position * inv_freq, and both halves of a row repeat the dim/2
    angles.  (Kernel inputs, like a model's position embeddings.)"""
    pos = np.asarray(positions, dtype=np.float64)[:, None]
    inv = base ** (-np.arange(0, dim, 2, dtype=np.float64) / dim)
    ang = np.concatenate([pos * inv, pos * inv], axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def mla_step_inputs(B, H, dtype="bf16", seed=0, d_c=512, d_nope=128, d_r=64, d_v=128):
    """One MLA decode step's inputs: q_nope [B,H,d_nope], q_rope [B,H,d_r],
    the new token's c_kv [B,d_c] and k_pe [B,d_r] (before RoPE), and
    per-head weights w_uk [H,d_c,d_nope], w_uv [H,d_c,d_v] drawn N(0,1) and
    scaled by 1/sqrt(fan-in) (tensor ids 10..15)."""
    def one(tid, shape, scale=1.0):
        t = _store(shape, dtype)
        _put(t, ..., np.random.default_rng([seed, tid]).standard_normal(shape, dtype=np.float32) * np.float32(scale),
             dtype)
        return Tensor(t, dtype)
    return (one(10, (B, H, d_nope)), one(11, (B, H, d_r)), one(12, (B, d_c)), one(13, (B, d_r)),
            one(14, (H, d_c, d_nope), 1 / np.sqrt(d_nope)), one(15, (H, d_c, d_v), 1 / np.sqrt(d_c)))


def mla_slice(seed, b, H, L, d_kv=576):
    """float32 draws of sequence b only: (q_abs [H,d_kv], latent [L,d_kv])."""
    return _draw(seed, 0, b, (H, d_kv)), _draw(seed, 1, b, (L, d_kv))


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                      # "prefill" | "decode" | "mla"
    dtype: str
    shape: dict = field(default_factory=dict)


# The measured and parity-checked shapes (all iid N(0,1), seed 0).
WORKLOADS = {
    w.name: w for w in (
        Workload("mqa_prefill_f32_b1_t128", "prefill", "f32",
                 dict(B=1, Hq=16, Hkv=1, T=128, D=512)),
        Workload("mqa_prefill_bf16_b2_t4096", "prefill", "bf16",
                 dict(B=2, Hq=16, Hkv=1, T=4096, D=512)),
        Workload("mqa_decode_bf16_b64_l8192", "decode", "bf16",
                 dict(B=64, Hq=16, Hkv=1, L=8192, D=512, lengths=None)),
        Workload("gqa_prefill_bf16_b1_t8192", "prefill", "bf16",
                 dict(B=1, Hq=64, Hkv=8, T=8192, D=128)),
        Workload("gqa_decode_bf16_b128_l1024to16384", "decode", "bf16",
                 dict(B=128, Hq=64, Hkv=8, L=16384, D=128, lengths=(1024, 16384))),
        Workload("mla_decode_bf16_b32_l32768", "mla", "bf16",
                 dict(B=32, H=128, L=32768, D=576)),
        # the steps around the absorbed MLA decode (absorption + RoPE, cache
        # append, W_UV up-projection), batch 32, 128 heads
        Workload("mla_step_proj_bf16_b32_h128", "mla_step", "bf16",
                 dict(B=32, H=128, L=32768)),
        # the MQA prefill in fp16 (the zdabc.icu benchmark's GPU dtype)
        Workload("mqa_prefill_f16_b2_t4096", "prefill", "f16",
                 dict(B=2, Hq=16, Hkv=1, T=4096, D=512)),
        # sparse (top-k) MLA decode: 2048 selected rows of a 32768-row cache
        Workload("mla_sparse_decode_bf16_b32_l32768_k2048", "mla_sparse", "bf16",
                 dict(B=32, H=128, L=32768, D=576, topk=2048)),
        # expanded (MHA-mode) MLA prefill: 128 heads, q/k 128 + 64 wide, v 128
        Workload("mla_prefill_bf16_b1_h128_t8192", "prefill", "bf16",
                 dict(B=1, Hq=128, Hkv=128, T=8192, D=192, DV=128)),
        # chunked MQA prefill: 1024 new tokens after 7168 cached ones
        Workload("mqa_chunk_prefill_bf16_b2_q1024_kv8192", "prefill", "bf16",
                 dict(B=2, Hq=16, Hkv=1, T=1024, T_kv=8192, D=512)),
    )
}
