"""Plain fp64 numpy definitions of the attention variants on the hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
HIP library or its Python binding.

Conventions
-----------
* Prefill tensors are ``[B, H, T, d]`` with the last axis contiguous; this is
  the shape convention of the zdabc.icu MQA article (section
  "head_dim = 512 为什么值得注意": Q is [batch, query_heads, sequence, head_dim],
  K and V have one head) and of lzwjava "GQA和MLA详解" §1.
* Decode: ``q`` is ``[B, Hq, d]`` (one new token per sequence) and the caches
  are ``[B, Hkv, L_max, d]`` with ``seq_lens[b]`` valid rows; the query attends
  to every valid cached row (lzwjava §1: at decode q is (B,H,1,d) against a
  cached K of (B,H,T,d)).
* GQA head mapping: query head ``h`` reads KV head ``h // (Hq // Hkv)``; the
  broadcast is materialised with ``np.repeat`` along the head axis, which is
  ``repeat_interleave(group, dim=1)`` (lzwjava §2; walkerchi §三 ``repeat_kv``).
* Inputs are upcast exactly to float64 before any arithmetic.  All outputs are
  float64.
* ``lse`` is the natural-log log-sum-exp of the scaled, masked scores of a
  row: ``lse = max_j s_j + log(sum_j exp(s_j - max_j s_j))``.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "repeat_kv_heads",
    "prefill_ref",
    "prefill_rows_ref",
    "decode_ref",
    "partial_ref",
    "lse_merge",
    "mla_absorbed_ref",
    "mla_sparse_ref",
    "rope_ref",
    "absorb_query",
    "output_project",
    "mla_explicit_ref",
    "kv_values_per_token",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def repeat_kv_heads(x, n_rep):
    """Materialise the GQA/MQA broadcast: ``[B, Hkv, ...] -> [B, Hkv*n_rep, ...]``.

    Each KV head is repeated ``n_rep`` times in place, so query head ``h`` sees
    KV head ``h // n_rep`` (lzwjava "GQA和MLA详解" §2, repeat_interleave on the
    head axis; walkerchi "Full 路线" §三, ``repeat_kv`` expand + reshape).
    """
    x = _f64(x)
    return np.repeat(x, n_rep, axis=1)


def _attend(q_rows, keys, values, scale, visible):
    """softmax(scale * q k^T, masked) @ v for a block of query rows.

    Follows makesence "带你了解Attention" §1.2: score(s,t) = q_s . k_t,
    weights = softmax(score / sqrt(d_k)) (here ``scale`` is the 1/sqrt(d_k)
    factor, passed explicitly), output_s = sum_t weight(s,t) v_t.  The mask
    sets hidden scores to -inf before the softmax (lzwjava §1: softmax of the
    scaled scores plus a causal mask).

    q_rows [R, dk], keys [S, dk], values [S, dv], visible bool [R, S].
    Returns (out [R, dv], lse [R]).  Every row must see at least one key.
    """
    s = scale * (q_rows @ keys.T)                     # [R, S]
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)              # finite: >= 1 visible key
    e = np.exp(s - m)                                 # exp(-inf) = 0 for hidden keys
    l = np.sum(e, axis=1, keepdims=True)
    p = e / l
    out = p @ values
    lse = (m + np.log(l))[:, 0]
    return out, lse


def prefill_ref(q, k, v, scale, causal):
    """Full-sequence attention for MHA / GQA / MQA (prefill).

    q [B, Hq, T, dk]; k [B, Hkv, S, dk]; v [B, Hkv, S, dv]; Hq % Hkv == 0.
    dk and dv may differ (the expanded MLA prefill of makesence §4.4 runs as
    MHA with a 192-wide query/key and a 128-wide value, walkerchi §四 4.2).
    causal: the T queries are the last T tokens of the S-token sequence, so
    query i sits at position S - T + i and key j is visible to it iff
    j <= S - T + i.  For T == S this is the square lower-triangular mask of
    lzwjava §1 (and of SDPA's ``is_causal=True`` in the zdabc.icu benchmark
    section); T < S is a block of new tokens after S - T earlier ones
    (chunked prefill, or several decode tokens at once -- the pages only
    show the square case, so this bottom-right alignment is a reading);
    T > S is rejected, since a query row would see no key.
    Returns (out [B, Hq, T, dv], lse [B, Hq, T]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, T, _ = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and T > S:
        raise ValueError("causal prefill needs T <= S (every query must see a key)")
    n_rep = Hq // Hkv
    k_rep = repeat_kv_heads(k, n_rep)
    v_rep = repeat_kv_heads(v, n_rep)
    if causal:
        visible = np.tril(np.ones((T, S), dtype=bool), k=S - T)
    else:
        visible = np.ones((T, S), dtype=bool)
    out = np.empty((B, Hq, T, v.shape[-1]))
    lse = np.empty((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            out[b, h], lse[b, h] = _attend(q[b, h], k_rep[b, h], v_rep[b, h], scale, visible)
    return out, lse


def prefill_rows_ref(q, k, v, rows, scale, causal):
    """The same definition as :func:`prefill_ref`, evaluated only for the
    listed query rows ``rows = [(b, h, i), ...]`` (used to check full-size
    outputs on a sample).  Returns (out [n, dv], lse [n])."""
    Hq, Hkv = q.shape[1], k.shape[1]
    T, S = q.shape[2], k.shape[2]
    if causal and T > S:
        raise ValueError("causal prefill needs T <= S (every query must see a key)")
    n_rep = Hq // Hkv
    out = np.empty((len(rows), v.shape[-1]))
    lse = np.empty(len(rows))
    for r, (b, h, i) in enumerate(rows):
        g = h // n_rep
        last = S - T + i + 1 if causal else S
        kk = _f64(k[b, g, :last])
        vv = _f64(v[b, g, :last])
        qq = _f64(q[b, h, i])[None, :]
        o, s = _attend(qq, kk, vv, scale, np.ones((1, last), dtype=bool))
        out[r], lse[r] = o[0], s[0]
    return out, lse


def decode_ref(q, k_cache, v_cache, seq_lens, scale):
    """One-token decode against a KV cache (lzwjava §1 decode phase).

    q [B, Hq, dk]; k_cache [B, Hkv, L_max, dk]; v_cache [B, Hkv, L_max, dv];
    seq_lens [B] with 1 <= L_b <= L_max.  The new token attends to all L_b
    cached rows (the cache already holds the current token, as in the HF
    ``past_key_value.update`` call quoted in walkerchi §三); rows >= L_b are
    never read.  Returns (out [B, Hq, dv], lse [B, Hq]).
    """
    B, Hq, _ = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    n_rep = Hq // Hkv
    out = np.empty((B, Hq, v_cache.shape[-1]))
    lse = np.empty((B, Hq))
    for b in range(B):
        L = int(seq_lens[b])
        if not 1 <= L <= k_cache.shape[2]:
            raise ValueError("seq_lens out of range")
        kb = repeat_kv_heads(k_cache[b:b + 1, :, :L], n_rep)[0]   # [Hq, L, dk]
        vb = repeat_kv_heads(v_cache[b:b + 1, :, :L], n_rep)[0]
        for h in range(Hq):
            o, s = _attend(_f64(q[b, h])[None, :], kb[h], vb[h], scale,
                           np.ones((1, L), dtype=bool))
            out[b, h], lse[b, h] = o[0], s[0]
    return out, lse


def partial_ref(q_row, keys, values, scale):
    """Un-normalised attention state of one query row over a block of keys.

    Returns (m, l, o) with m = max_j s_j, l = sum_j exp(s_j - m),
    o = sum_j exp(s_j - m) v_j, where s_j = scale * q.k_j.  This is the state
    that a split-KV decode keeps per chunk; an empty block gives
    (-inf, 0, 0).  The combination rule is :func:`lse_merge`.
    """
    q_row, keys, values = _f64(q_row), _f64(keys), _f64(values)
    if keys.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(values.shape[-1])
    s = scale * (keys @ q_row)
    m = np.max(s)
    e = np.exp(s - m)
    return m, float(np.sum(e)), e @ values


def lse_merge(parts):
    """Combine per-chunk states (m_c, l_c, o_c) into the full-row result.

    With M = max_c m_c: L = sum_c l_c exp(m_c - M), O = sum_c o_c exp(m_c - M) / L.
    This is exact algebra (softmax over a union of key sets); chunks with
    m_c = -inf contribute nothing.  Returns (out [dv], lse).
    """
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    M = np.max(ms)
    L = 0.0
    O = np.zeros_like(_f64(parts[0][2]))
    for m, l, o in parts:
        if m == -np.inf:
            continue
        w = np.exp(m - M)
        L += l * w
        O = O + _f64(o) * w
    return O / L, M + np.log(L)


def mla_absorbed_ref(q_abs, kv_cache, seq_lens, scale, d_v=512):
    """MLA decode computed directly on the cached latent (absorbed form).

    Each cached row is ``[c_kv (d_c) ‖ k_pe (d_R)]`` (walkerchi §四 4.2: the
    ``kv_a_proj_with_mqa`` output is split as kv_lora_rank + qk_rope_head_dim
    = 512 + 64; makesence §4.5: 576 values per token per layer).  The query of
    head h is ``q_abs = [W_UK[h] q_nope ‖ q_rope]`` (lzwjava §3 matrix
    absorption; makesence §4.3).  The whole row is the key; its first ``d_v``
    entries (the latent c_kv) are the value, and the caller applies W_UV to
    the result.  scale is the original head's 1/sqrt(d_nope + d_R).

    q_abs [B, H, d_c + d_R]; kv_cache [B, L_max, d_c + d_R]; seq_lens [B].
    Returns (o_latent [B, H, d_v], lse [B, H]).
    """
    B, H, _ = q_abs.shape
    out = np.empty((B, H, d_v))
    lse = np.empty((B, H))
    for b in range(B):
        L = int(seq_lens[b])
        if not 1 <= L <= kv_cache.shape[1]:
            raise ValueError("seq_lens out of range")
        rows = _f64(kv_cache[b, :L])                     # [L, 576]
        o, s = _attend(_f64(q_abs[b]), rows, rows[:, :d_v], scale,
                       np.ones((H, L), dtype=bool))
        out[b], lse[b] = o, s
    return out, lse


def mla_sparse_ref(q_abs, kv_cache, indices, scale, d_v=512):
    """Absorbed MLA decode over a selected subset of the cached rows.

    DeepSeek sparse attention keeps the MLA cache and lets each query attend
    only to k selected tokens (makesence §5.1: an indexer picks the top-k
    positions, k = 2048 in V3.2).  Here the selection is an input: sequence b
    attends to the rows ``kv_cache[b, indices[b, j]]``; entries outside
    [0, L_max) (e.g. -1 padding for sequences with fewer than k tokens) are
    skipped, and a row listed twice counts twice (the attended set is the
    list as given).  Each attended row is used as in :func:`mla_absorbed_ref`
    (whole row = key, first ``d_v`` values = value).  A sequence with no
    valid entry gets out = 0 and lse = -inf.

    q_abs [B, H, d_c + d_R]; kv_cache [B, L_max, d_c + d_R]; indices int [B, k].
    Returns (o_latent [B, H, d_v], lse [B, H]).
    """
    B, H, _ = q_abs.shape
    L_max = kv_cache.shape[1]
    out = np.zeros((B, H, d_v))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        sel = [int(i) for i in indices[b] if 0 <= int(i) < L_max]
        if not sel:
            continue
        rows = _f64(kv_cache[b, sel])                    # [n, 576], gathered in list order
        o, s = _attend(_f64(q_abs[b]), rows, rows[:, :d_v], scale,
                       np.ones((H, len(sel)), dtype=bool))
        out[b], lse[b] = o, s
    return out, lse


def rope_ref(x, cos, sin):
    """Rotary position embedding of the decoupled RoPE part, in the form the
    pages call (walkerchi §四 4.2: ``apply_rotary_pos_emb(q_rope, k_pe, cos,
    sin)`` with ``cos, sin = position_embeddings``): with the last axis split
    into halves x = [x1 | x2], rotate_half(x) = [-x2 | x1] and
    RoPE(x) = x * cos + rotate_half(x) * sin.  cos and sin hold the rotary
    factors of each row's position, broadcast over the leading axes.
    """
    x, cos, sin = _f64(x), _f64(cos), _f64(sin)
    h = x.shape[-1] // 2
    rot = np.concatenate([-x[..., h:], x[..., :h]], axis=-1)
    return x * cos + rot * sin


def absorb_query(q_nope, q_rope, w_uk):
    """Fold the key up-projection into the query (lzwjava §3; makesence §4.3).

    With k_nope = c_kv @ W_UK[h] (W_UK[h] is [d_c, d_nope]),
    q_nope . k_nope = (W_UK[h] @ q_nope) . c_kv, so the absorbed query of
    head h is ``[W_UK[h] @ q_nope ‖ q_rope]``.
    q_nope [B, H, d_nope]; q_rope [B, H, d_R]; w_uk [H, d_c, d_nope].
    Returns q_abs [B, H, d_c + d_R].
    """
    q_nope, q_rope, w_uk = _f64(q_nope), _f64(q_rope), _f64(w_uk)
    B, H, _ = q_nope.shape
    lat = np.empty((B, H, w_uk.shape[1]))
    for h in range(H):
        lat[:, h] = q_nope[:, h] @ w_uk[h].T
    return np.concatenate([lat, q_rope], axis=-1)


def output_project(o_lat, w_uv):
    """Map the absorbed decode's latent output back to value space (lzwjava
    §3; walkerchi §四 4.3): with V_h = c_kv @ W_UV[h], softmax . V_h =
    (softmax . c_kv) @ W_UV[h], so head h's output is o_lat[:, h] @ W_UV[h].
    o_lat [B, H, d_c]; w_uv [H, d_c, d_v].  Returns [B, H, d_v].
    """
    o_lat, w_uv = _f64(o_lat), _f64(w_uv)
    B, H, _ = o_lat.shape
    out = np.empty((B, H, w_uv.shape[2]))
    for h in range(H):
        out[:, h] = o_lat[:, h] @ w_uv[h]
    return out


def mla_explicit_ref(q_nope, q_rope, c_kv, k_pe, w_uk, w_uv, seq_lens, scale):
    """MLA decode with K and V rebuilt from the latent (no absorption).

    Per head h: K_h = [c_kv @ W_UK[h] ‖ k_pe] (the RoPE key is shared by all
    heads, walkerchi §四 4.2 ``k_pe.expand`` over heads), V_h = c_kv @ W_UV[h]
    (naphjohn "算子讲解手记（一）" §2: K = c_kv W_UK, V = c_kv W_UV), then
    standard attention of q_h = [q_nope ‖ q_rope] over the L_b rows.
    q_nope [B,H,d_nope]; q_rope [B,H,d_R]; c_kv [B,L_max,d_c]; k_pe [B,L_max,d_R];
    w_uk, w_uv [H, d_c, d_nope / d_v].  Returns (out [B, H, d_v], lse [B, H]).
    """
    q_nope, q_rope, c_kv, k_pe = _f64(q_nope), _f64(q_rope), _f64(c_kv), _f64(k_pe)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    B, H, _ = q_nope.shape
    out = np.empty((B, H, w_uv.shape[2]))
    lse = np.empty((B, H))
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(H):
            k_h = np.concatenate([c_kv[b, :L] @ w_uk[h], k_pe[b, :L]], axis=-1)
            v_h = c_kv[b, :L] @ w_uv[h]
            q_h = np.concatenate([q_nope[b, h], q_rope[b, h]])[None, :]
            o, s = _attend(q_h, k_h, v_h, scale, np.ones((1, L), dtype=bool))
            out[b, h], lse[b, h] = o[0], s[0]
    return out, lse


def kv_values_per_token(kind, *, n_heads=None, n_kv_heads=None, head_dim=None,
                        d_c=None, d_rope=None):
    """Cached values per token per layer (closed forms on the pages).

    * MHA: 2 * n_heads * head_dim (naphjohn §1; walkerchi §二 table).
    * GQA: 2 * n_kv_heads * head_dim (lzwjava §2); MQA is n_kv_heads = 1.
    * MLA: d_c + d_rope (lzwjava §3; walkerchi §二 table; makesence §4.5).
    """
    if kind == "mha":
        return 2 * n_heads * head_dim
    if kind in ("gqa", "mqa"):
        return 2 * (1 if kind == "mqa" else n_kv_heads) * head_dim
    if kind == "mla":
        return d_c + d_rope
    raise ValueError(kind)
