"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test ties one part of the oracle to something other than itself: a
pure-Python brute force, a closed form, an invariant the pages state, a
special case that reduces to textbook arithmetic, or a value the pages print.
CPU only.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from synthetic import (prefill_inputs, decode_inputs, mla_inputs, draw_topk, rope_tables, round_bf16, bf16_bits,
                       bf16_to_f32)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# O1: brute force.  A scalar triple loop with math.exp, written from the
# definition (makesence §1.2; lzwjava §1 causal mask; lzwjava §2 head sharing
# with query head h on KV head h // group).  No numpy arithmetic.
# ---------------------------------------------------------------------------

def _brute_row(qv, keys, vals, scale):
    scores = [scale * sum(a * b for a, b in zip(qv, kr)) for kr in keys]
    mx = max(scores)
    w = [math.exp(s - mx) for s in scores]
    tot = sum(w)
    out = [sum(w[j] * vals[j][c] for j in range(len(keys))) / tot for c in range(len(vals[0]))]
    return out, mx + math.log(tot)


def _brute_prefill(q, k, v, scale, causal):
    B, Hq, T, _ = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    out = np.zeros((B, Hq, T, v.shape[-1]))
    lse = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for i in range(T):
                last = i + 1 if causal else k.shape[2]
                keys = [list(map(float, k[b, g, j])) for j in range(last)]
                vals = [list(map(float, v[b, g, j])) for j in range(last)]
                o, s = _brute_row(list(map(float, q[b, h, i])), keys, vals, scale)
                out[b, h, i], lse[b, h, i] = o, s
    return out, lse


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (4, 2), (6, 3), (3, 3)])
@pytest.mark.parametrize("causal", [True, False])
def test_o1_prefill_brute_force(Hq, Hkv, causal):
    rng = np.random.default_rng(11)
    B, T, D, DV = 2, 5, 3, 4
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, DV))
    scale = 1.0 / math.sqrt(D)
    o_ref, l_ref = oracle.prefill_ref(q, k, v, scale, causal)
    o_bf, l_bf = _brute_prefill(q, k, v, scale, causal)
    assert np.max(np.abs(o_ref - o_bf)) <= 1e-12
    assert np.max(np.abs(l_ref - l_bf)) <= 1e-12


def test_o1_prefill_rows_match_full():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 4, 7, 5))
    k = rng.standard_normal((2, 2, 7, 5))
    v = rng.standard_normal((2, 2, 7, 5))
    full, lse = oracle.prefill_ref(q, k, v, 0.3, True)
    rows = [(0, 0, 0), (1, 3, 6), (0, 2, 4), (1, 1, 3)]
    o, l = oracle.prefill_rows_ref(q, k, v, rows, 0.3, True)
    for r, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(o[r] - full[b, h, i])) <= 1e-13
        assert abs(l[r] - lse[b, h, i]) <= 1e-13


def _brute_prefill_positions(q, k, v, scale, q_pos):
    """Brute force with explicit token positions: query row i is the token at
    position q_pos[i] and sees the keys at positions 0..q_pos[i]; q_pos None
    means every key.  Pure Python arithmetic, as in _brute_row."""
    B, Hq, T, _ = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    out = np.zeros((B, Hq, T, v.shape[-1]))
    lse = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for i in range(T):
                seen = [j for j in range(S) if q_pos is None or j <= q_pos[i]]
                keys = [list(map(float, k[b, g, j])) for j in seen]
                vals = [list(map(float, v[b, g, j])) for j in seen]
                o, s_ = _brute_row(list(map(float, q[b, h, i])), keys, vals, scale)
                out[b, h, i], lse[b, h, i] = o, s_
    return out, lse


@pytest.mark.parametrize("T,S", [(3, 7), (1, 6), (5, 5), (4, 9)])
@pytest.mark.parametrize("causal", [True, False])
def test_o1_chunk_prefill_brute_force(T, S, causal):
    """T new tokens after S - T earlier ones: the queries are the LAST T
    tokens of the sequence (token ids taken from the tail of range(S)); the
    query/key width differs from the value width."""
    rng = np.random.default_rng(15)
    B, Hq, Hkv, D, DV = 2, 4, 2, 3, 5
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, DV))
    q_pos = list(range(S))[S - T:] if causal else None
    o_ref, l_ref = oracle.prefill_ref(q, k, v, 0.45, causal)
    o_bf, l_bf = _brute_prefill_positions(q, k, v, 0.45, q_pos)
    assert np.max(np.abs(o_ref - o_bf)) <= 1e-12
    assert np.max(np.abs(l_ref - l_bf)) <= 1e-12
    rows = [(0, 0, 0), (1, 3, T - 1), (0, 2, T // 2)]
    o_r, l_r = oracle.prefill_rows_ref(q, k, v, rows, 0.45, causal)
    for r, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(o_r[r] - o_bf[b, h, i])) <= 1e-12
        assert abs(l_r[r] - l_bf[b, h, i]) <= 1e-12


def test_chunk_rows_equal_square_rows():
    """A chunk of the last T queries against all S keys equals the last T
    rows of the square causal prefill over the S tokens (the chunk is the
    tail of the same sequence).  Pins the direction of the alignment: a
    top-left mask would give the chunk's first row one key instead of
    S - T + 1."""
    q, k, v = (t.f32().astype(np.float64) for t in prefill_inputs(2, 4, 2, 11, 6, "f32", seed=16))
    full, lfull = oracle.prefill_ref(q, k, v, 0.3, True)
    for T in (1, 4, 11):
        part, lpart = oracle.prefill_ref(q[:, :, 11 - T:], k, v, 0.3, True)
        assert np.max(np.abs(part - full[:, :, 11 - T:])) <= 1e-13
        assert np.max(np.abs(lpart - lfull[:, :, 11 - T:])) <= 1e-13


def test_single_token_chunk_is_decode():
    """T = 1 causal is one decode step over the S cached tokens."""
    q, k, v = (t.f32().astype(np.float64) for t in prefill_inputs(3, 4, 1, 1, 5, "f32", seed=17, d_v=7, T_kv=9))
    o, l = oracle.prefill_ref(q, k, v, 0.5, True)
    od, ld = oracle.decode_ref(q[:, :, 0], k, v, np.array([9, 9, 9]), 0.5)
    assert np.max(np.abs(o[:, :, 0] - od)) <= 1e-13
    assert np.max(np.abs(l[:, :, 0] - ld)) <= 1e-13


def test_causal_chunk_longer_than_keys_rejected():
    q, k, v = (t.f32() for t in prefill_inputs(1, 2, 1, 6, 4, "f32", seed=18, T_kv=5))
    with pytest.raises(ValueError):
        oracle.prefill_ref(q, k, v, 0.5, True)
    with pytest.raises(ValueError):
        oracle.prefill_rows_ref(q, k, v, [(0, 0, 0)], 0.5, True)
    oracle.prefill_ref(q, k, v, 0.5, False)    # no mask: any T, S


def test_mla_expanded_prefill_equals_absorbed():
    """Expanded MLA prefill (makesence §4.4: MHA with per-head keys
    K_h = [c_kv W_UK[h] | k_pe] of width d_nope + d_R and values
    V_h = c_kv W_UV[h] of width d_v) gives at causal row t the absorbed
    decode of token t over the first t + 1 latent rows followed by W_UV[h]
    (lzwjava §3), itself pinned to the explicit form above."""
    rng = np.random.default_rng(35)
    B, H, T, dc, dn, dr, dv = 2, 4, 9, 16, 8, 4, 6
    q_nope = rng.standard_normal((B, H, T, dn))
    q_rope = rng.standard_normal((B, H, T, dr))
    c_kv = rng.standard_normal((B, T, dc))
    k_pe = rng.standard_normal((B, T, dr))
    w_uk = rng.standard_normal((H, dc, dn)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dc, dv)) / math.sqrt(dc)
    scale = 1.0 / math.sqrt(dn + dr)
    K = np.stack([np.concatenate([c_kv @ w_uk[h], k_pe], -1) for h in range(H)], axis=1)
    V = np.stack([c_kv @ w_uv[h] for h in range(H)], axis=1)
    Q = np.concatenate([q_nope, q_rope], -1)
    out, lse = oracle.prefill_ref(Q, K, V, scale, True)
    assert out.shape == (B, H, T, dv)
    latent = np.concatenate([c_kv, k_pe], -1)
    for t in range(T):
        q_abs = oracle.absorb_query(q_nope[:, :, t], q_rope[:, :, t], w_uk)
        o_lat, l_abs = oracle.mla_absorbed_ref(q_abs, latent, np.full(B, t + 1), scale, d_v=dc)
        o_t = np.stack([o_lat[:, h] @ w_uv[h] for h in range(H)], axis=1)
        assert np.max(np.abs(o_t - out[:, :, t])) <= 1e-10
        assert np.max(np.abs(l_abs - lse[:, :, t])) <= 1e-10


def test_o1_decode_brute_force():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, L, D = 3, 4, 2, 6, 3
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Hkv, L, D))
    vc = rng.standard_normal((B, Hkv, L, D))
    lens = np.array([6, 1, 4])
    out, lse = oracle.decode_ref(q, kc, vc, lens, 0.7)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = [list(kc[b, g, j]) for j in range(lens[b])]
            vals = [list(vc[b, g, j]) for j in range(lens[b])]
            o, s = _brute_row(list(q[b, h]), keys, vals, 0.7)
            assert np.max(np.abs(out[b, h] - np.array(o))) <= 1e-12
            assert abs(lse[b, h] - s) <= 1e-12


def test_o1_mla_absorbed_brute_force():
    rng = np.random.default_rng(14)
    B, H, L, DK, DV = 2, 3, 5, 6, 4
    q = rng.standard_normal((B, H, DK))
    kv = rng.standard_normal((B, L, DK))
    lens = np.array([5, 2])
    out, lse = oracle.mla_absorbed_ref(q, kv, lens, 0.4, d_v=DV)
    for b in range(B):
        for h in range(H):
            keys = [list(kv[b, j]) for j in range(lens[b])]
            vals = [list(kv[b, j, :DV]) for j in range(lens[b])]   # value = leading latent
            o, s = _brute_row(list(q[b, h]), keys, vals, 0.4)
            assert np.max(np.abs(out[b, h] - np.array(o))) <= 1e-12
            assert abs(lse[b, h] - s) <= 1e-12


# ---------------------------------------------------------------------------
# O2: softmax rows.  With V = identity (one value dimension per key), the
# output row IS the probability row: it must be >= 0, sum to 1, and be exactly
# 0 on masked keys.
# ---------------------------------------------------------------------------

def test_o2_probability_rows():
    rng = np.random.default_rng(21)
    T = 8
    q = rng.standard_normal((1, 2, T, 4)) * 3
    k = rng.standard_normal((1, 1, T, 4)) * 3
    v = np.eye(T)[None, None]                 # v_j = e_j
    p, _ = oracle.prefill_ref(q, k, v, 0.5, True)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(-1) - 1)) <= 1e-12
    for i in range(T):
        assert np.all(p[..., i, i + 1:] == 0.0)       # future keys exactly zero
        assert np.all(p[..., i, : i + 1] > 0)
    # all-ones values give exactly one (weights sum to one)
    o1, _ = oracle.prefill_ref(q, k, np.ones((1, 1, T, 3)), 0.5, False)
    assert np.max(np.abs(o1 - 1)) <= 1e-12


# ---------------------------------------------------------------------------
# O3 / O4: head sharing.  MQA equals MHA on KV copied to every head
# (zdabc.icu benchmark: native MQA against repeated K/V); GQA with G = H is
# MHA and G = 1 is MQA (makesence §3.2); head h uses KV head h // (H/G).
# The repeated tensors are built here by explicit loops, not by the oracle.
# ---------------------------------------------------------------------------

def _hand_repeat(x, Hq, mapping):
    B, _, S, D = x.shape
    out = np.empty((B, Hq, S, D))
    for h in range(Hq):
        out[:, h] = x[:, mapping(h)]
    return out


def test_o3_mqa_equals_mha_on_repeated_kv():
    q, k, v = (t.f32().astype(np.float64) for t in prefill_inputs(1, 8, 1, 9, 16, "f32", seed=3))
    o_mqa, l_mqa = oracle.prefill_ref(q, k, v, 0.25, True)
    k_rep = _hand_repeat(k, 8, lambda h: 0)
    v_rep = _hand_repeat(v, 8, lambda h: 0)
    o_mha, l_mha = oracle.prefill_ref(q, k_rep, v_rep, 0.25, True)
    assert np.array_equal(o_mqa, o_mha) and np.array_equal(l_mqa, l_mha)


def test_o4_gqa_head_mapping():
    Hq, Hkv = 6, 3
    q, k, v = (t.f32().astype(np.float64) for t in prefill_inputs(2, Hq, Hkv, 7, 8, "f32", seed=4))
    o_gqa, _ = oracle.prefill_ref(q, k, v, 0.3, True)
    o_div, _ = oracle.prefill_ref(q, _hand_repeat(k, Hq, lambda h: h // 2),
                                  _hand_repeat(v, Hq, lambda h: h // 2), 0.3, True)
    o_mod, _ = oracle.prefill_ref(q, _hand_repeat(k, Hq, lambda h: h % Hkv),
                                  _hand_repeat(v, Hq, lambda h: h % Hkv), 0.3, True)
    assert np.array_equal(o_gqa, o_div)
    assert np.max(np.abs(o_gqa - o_mod)) > 1e-3       # the tile mapping is a different result
    # G = H is MHA: every head on its own KV head
    o_mha, _ = oracle.prefill_ref(q, _hand_repeat(k, Hq, lambda h: h // 2),
                                  _hand_repeat(v, Hq, lambda h: h // 2), 0.3, True)
    assert np.array_equal(o_mha, o_div)
    # G = 1 is MQA
    k1, v1 = k[:, :1], v[:, :1]
    o_g1, _ = oracle.prefill_ref(q, k1, v1, 0.3, True)
    o_m1, _ = oracle.prefill_ref(q, _hand_repeat(k1, Hq, lambda h: 0), _hand_repeat(v1, Hq, lambda h: 0), 0.3, True)
    assert np.array_equal(o_g1, o_m1)


def test_o4_decode_head_mapping():
    q, kc, vc, lens = decode_inputs(2, 8, 2, 6, 4, "f32", seed=5, lengths=(2, 6))
    q, kc, vc = q.f32().astype(np.float64), kc.f32().astype(np.float64), vc.f32().astype(np.float64)
    out, _ = oracle.decode_ref(q, kc, vc, lens, 0.5)
    for b in range(2):
        L = lens[b]
        for h in range(8):
            g = h // 4
            s = 0.5 * kc[b, g, :L] @ q[b, h]
            w = np.exp(s - s.max())
            ref = (w / w.sum()) @ vc[b, g, :L]
            assert np.max(np.abs(out[b, h] - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# O5: causal mask direction.  Changing keys/values at positions > i must
# leave rows 0..i bitwise unchanged, and row T-1 must change.
# ---------------------------------------------------------------------------

def test_o5_causal_invariance():
    q, k, v = (t.f32().astype(np.float64) for t in prefill_inputs(1, 4, 2, 10, 8, "f32", seed=6))
    base, lbase = oracle.prefill_ref(q, k, v, 0.35, True)
    for i in (0, 3, 8):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1:] += 5.0
        v2[:, :, i + 1:] -= 7.0
        o2, l2 = oracle.prefill_ref(q, k2, v2, 0.35, True)
        assert np.array_equal(o2[:, :, : i + 1], base[:, :, : i + 1])
        assert np.array_equal(l2[:, :, : i + 1], lbase[:, :, : i + 1])
        assert np.max(np.abs(o2[:, :, -1] - base[:, :, -1])) > 1e-3


def test_decode_is_last_causal_row():
    """Decode over L rows equals the last row of causal prefill over those L
    tokens when the decode query is the last prefill query (lzwjava §1:
    decode is one query row against the cached keys)."""
    q, k, v = (t.f32().astype(np.float64) for t in prefill_inputs(2, 4, 1, 9, 8, "f32", seed=7))
    full, lfull = oracle.prefill_ref(q, k, v, 0.2, True)
    out, lse = oracle.decode_ref(q[:, :, -1], k, v, np.array([9, 9]), 0.2)
    assert np.max(np.abs(out - full[:, :, -1])) <= 1e-13
    assert np.max(np.abs(lse - lfull[:, :, -1])) <= 1e-13
    # and over a shorter cache: the row of the token at position L-1
    out5, _ = oracle.decode_ref(q[:, :, 4], k, v, np.array([5, 5]), 0.2)
    assert np.max(np.abs(out5 - full[:, :, 4])) <= 1e-13


# ---------------------------------------------------------------------------
# O6: closed forms.
# ---------------------------------------------------------------------------

def test_o6_first_row_is_v0():
    q, k, v = (t.f32().astype(np.float64) for t in prefill_inputs(1, 3, 1, 4, 5, "f32", seed=8))
    o, lse = oracle.prefill_ref(q, k, v, 0.44, True)
    assert np.array_equal(o[0, :, 0], np.repeat(v[0, :, 0], 3, axis=0))
    assert np.max(np.abs(lse[0, :, 0] - 0.44 * (q[0, :, 0] @ k[0, 0, 0]))) <= 1e-14


def test_o6_zero_query_gives_prefix_mean():
    _, k, v = (t.f32().astype(np.float64) for t in prefill_inputs(1, 2, 1, 6, 4, "f32", seed=9))
    q = np.zeros((1, 2, 6, 4))
    o, lse = oracle.prefill_ref(q, k, v, 0.5, True)
    for i in range(6):
        mean = v[0, 0, : i + 1].sum(0) / (i + 1)
        assert np.max(np.abs(o[0, :, i] - mean)) <= 1e-14
        assert abs(lse[0, 0, i] - math.log(i + 1)) <= 1e-14
    # constant keys give the same uniform weights
    kc = np.ones_like(k)
    o2, _ = oracle.prefill_ref(np.ones((1, 2, 6, 4)), kc, v, 0.5, True)
    assert np.max(np.abs(o2 - o)) <= 1e-13


def test_o6_log_weight_worked_example():
    """Scores chosen as ln(w_j) make the softmax weights exactly w_j / sum(w):
    with q = [1, 0], k_j = [ln(w_j) / scale, 0] and the 2-d values below the
    output is the w-weighted mean of the values (rational arithmetic)."""
    w = [1.0, 2.0, 3.0, 4.0]
    scale = 1.0 / math.sqrt(2.0)
    k = np.array([[math.log(x) / scale, 0.0] for x in w])[None, None]
    v = np.array([[1.0, 10.0], [-2.0, 0.0], [0.5, 4.0], [3.0, -1.0]])[None, None]
    q = np.array([1.0, 0.0])[None, None, None]
    q_all = np.repeat(q, 4, axis=2)
    o, lse = oracle.prefill_ref(q_all, k, v, scale, True)
    for i in range(4):
        ws = w[: i + 1]
        expect = sum(ws[j] * v[0, 0, j] for j in range(i + 1)) / sum(ws)
        assert np.max(np.abs(o[0, 0, i] - expect)) <= 1e-14
        assert abs(lse[0, 0, i] - math.log(sum(ws))) <= 1e-14
    # the scale is applied once: scale 2x makes the weights w_j^2 / sum(w^2)
    o2, _ = oracle.prefill_ref(q_all, k, v, 2 * scale, True)
    ws = [x * x for x in w]
    expect = sum(ws[j] * v[0, 0, j] for j in range(4)) / sum(ws)
    assert np.max(np.abs(o2[0, 0, 3] - expect)) <= 1e-13


def test_o6_dominant_score_and_permutation():
    rng = np.random.default_rng(10)
    L, D = 7, 4
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 1.0
    kc = rng.standard_normal((1, 1, L, D)) * 0.01
    kc[0, 0, 3, 0] = 50.0
    vc = rng.standard_normal((1, 1, L, 3))
    out, _ = oracle.decode_ref(q, kc, vc, np.array([L]), 1.0)
    assert np.max(np.abs(out[0, 0] - vc[0, 0, 3])) <= 1e-19 + 20 * math.exp(-49)
    perm = rng.permutation(L)
    q2 = rng.standard_normal((1, 2, D))
    a, la = oracle.decode_ref(q2, kc, vc, np.array([L]), 0.6)
    b, lb = oracle.decode_ref(q2, kc[:, :, perm], vc[:, :, perm], np.array([L]), 0.6)
    assert np.max(np.abs(a - b)) <= 1e-14 and np.max(np.abs(la - lb)) <= 1e-14


def test_decode_ignores_rows_past_seq_len():
    q, kc, vc, lens = decode_inputs(3, 4, 1, 12, 8, "f32", seed=15, lengths=(1, 12))
    out, lse = oracle.decode_ref(q.f32(), kc.f32(), vc.f32(), lens, 0.3)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))   # NaN padding never read
    for b in range(3):
        L = lens[b]
        o1, _ = oracle.decode_ref(q.f32()[b:b + 1], kc.f32()[b:b + 1, :, :L],
                                  vc.f32()[b:b + 1, :, :L], np.array([L]), 0.3)
        assert np.array_equal(o1[0], out[b])


# ---------------------------------------------------------------------------
# O7: absorbed MLA equals explicit reconstruction (lzwjava §3 matrix
# absorption; makesence §4.3; walkerchi §四 4.5 states the two agree).
# The explicit form is itself checked against the generic (pinned) MHA oracle
# on per-head K/V built here.
# ---------------------------------------------------------------------------

def _mla_case(seed, B=2, H=4, L=9, dc=16, dn=8, dr=4, dv=8):
    rng = np.random.default_rng(seed)
    q_nope = rng.standard_normal((B, H, dn))
    q_rope = rng.standard_normal((B, H, dr))
    c_kv = rng.standard_normal((B, L, dc))
    k_pe = rng.standard_normal((B, L, dr))
    w_uk = rng.standard_normal((H, dc, dn)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dc, dv)) / math.sqrt(dc)
    lens = np.array([L, L - 3] if B == 2 else [L] * B)
    return q_nope, q_rope, c_kv, k_pe, w_uk, w_uv, lens


def test_o7_absorbed_equals_explicit():
    q_nope, q_rope, c_kv, k_pe, w_uk, w_uv, lens = _mla_case(31)
    dn, dr = q_nope.shape[-1], q_rope.shape[-1]
    scale = 1.0 / math.sqrt(dn + dr)
    explicit, l_exp = oracle.mla_explicit_ref(q_nope, q_rope, c_kv, k_pe, w_uk, w_uv, lens, scale)
    q_abs = oracle.absorb_query(q_nope, q_rope, w_uk)
    latent = np.concatenate([c_kv, k_pe], axis=-1)
    o_lat, l_abs = oracle.mla_absorbed_ref(q_abs, latent, lens, scale, d_v=c_kv.shape[-1])
    out = oracle.output_project(o_lat, w_uv)
    assert np.max(np.abs(out - explicit)) <= 1e-10
    assert np.max(np.abs(l_abs - l_exp)) <= 1e-10


def test_o7_output_project_brute_force():
    """Pure-Python sums: out[b, h, v] = sum_c o_lat[b, h, c] W_UV[h][c, v]."""
    rng = np.random.default_rng(34)
    o_lat, w_uv = rng.standard_normal((2, 3, 5)), rng.standard_normal((3, 5, 4))
    out = oracle.output_project(o_lat, w_uv)
    for b in range(2):
        for h in range(3):
            for v in range(4):
                assert abs(out[b, h, v] - sum(o_lat[b, h, c] * w_uv[h, c, v] for c in range(5))) <= 1e-12


def test_o7_absorbed_query_closed_form():
    q_nope, q_rope, c_kv, k_pe, w_uk, _, _ = _mla_case(32)
    q_abs = oracle.absorb_query(q_nope, q_rope, w_uk)
    # dot with any latent row equals the explicit per-head key dot product
    for b in range(2):
        for h in range(4):
            for j in range(3):
                k_h = np.concatenate([c_kv[b, j] @ w_uk[h], k_pe[b, j]])
                q_h = np.concatenate([q_nope[b, h], q_rope[b, h]])
                lat = np.concatenate([c_kv[b, j], k_pe[b, j]])
                assert abs(q_abs[b, h] @ lat - q_h @ k_h) <= 1e-12


def test_o7_explicit_is_mha():
    q_nope, q_rope, c_kv, k_pe, w_uk, w_uv, lens = _mla_case(33, B=1)
    H, L = q_nope.shape[1], c_kv.shape[1]
    scale = 0.3
    ex, _ = oracle.mla_explicit_ref(q_nope, q_rope, c_kv, k_pe, w_uk, w_uv, lens, scale)
    K = np.stack([np.concatenate([c_kv[0] @ w_uk[h], k_pe[0]], -1) for h in range(H)])[None]
    V = np.stack([c_kv[0] @ w_uv[h] for h in range(H)])[None]
    Q = np.concatenate([q_nope, q_rope], -1)
    mha, _ = oracle.decode_ref(Q, K, V, np.array([L]), scale)
    assert np.max(np.abs(mha - ex)) <= 1e-12


def test_mla_ignores_padding_and_uses_leading_latent_as_value():
    q, kv, lens = mla_inputs(2, 4, 10, d_kv=12, dtype="f32", seed=34, lengths=(3, 9))
    out, _ = oracle.mla_absorbed_ref(q.f32(), kv.f32(), lens, 0.5, d_v=8)
    assert np.all(np.isfinite(out))
    # value = first d_v latent columns: changing the trailing (RoPE) columns
    # only through the scores -> with zero query on those columns nothing moves
    qz = q.f32().astype(np.float64).copy(); qz[..., 8:] = 0
    kv2 = kv.f32().astype(np.float64).copy(); kv2[..., 8:] += 3.0
    a, _ = oracle.mla_absorbed_ref(qz, kv.f32(), lens, 0.5, d_v=8)
    b, _ = oracle.mla_absorbed_ref(qz, kv2, lens, 0.5, d_v=8)
    assert np.max(np.abs(a - b)) <= 1e-14


# ---------------------------------------------------------------------------
# RoPE of the decoupled part and the whole MLA decode step around the
# absorbed attention.
# ---------------------------------------------------------------------------

def test_rope_special_angles():
    x = np.arange(1.0, 9.0)                         # halves [1..4 | 5..8]
    one, zero = np.ones(8), np.zeros(8)
    assert np.array_equal(oracle.rope_ref(x, one, zero), x)                       # angle 0: identity
    assert np.array_equal(oracle.rope_ref(x, zero, one), [-5, -6, -7, -8, 1, 2, 3, 4])   # quarter turn
    assert np.array_equal(oracle.rope_ref(x, -one, zero), -x)                     # half turn


def test_rope_is_a_rotation_by_position_difference():
    """<RoPE(q, m), RoPE(k, n)> = <RoPE(q, m - n), k> for the standard tables
    (angle addition: the score depends only on the relative position), and
    every (i, i + 32) pair keeps its norm."""
    rng = np.random.default_rng(40)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in ((7, 3), (100, 0), (5, 9), (4096, 4000)):
        c, s_ = rope_tables([m, n, m - n])
        c, s_ = c.astype(np.float64), s_.astype(np.float64)
        lhs = oracle.rope_ref(q, c[0], s_[0]) @ oracle.rope_ref(k, c[1], s_[1])
        rhs = oracle.rope_ref(q, c[2], s_[2]) @ k
        assert abs(lhs - rhs) <= 1e-5 * (1 + abs(rhs))     # float32 tables
        r = oracle.rope_ref(q, c[0], s_[0])
        assert np.allclose(r[:32] ** 2 + r[32:] ** 2, q[:32] ** 2 + q[32:] ** 2, atol=1e-5)


def test_mla_step_absorbed_equals_explicit_with_rope():
    """The decode step built from its pieces -- absorb the query, rotate the
    RoPE parts, append the new token's row [c_kv | RoPE(k_pe)] to the cache,
    absorbed attention, W_UV -- equals explicit attention on rebuilt
    per-head keys [c_kv W_UK[h] | RoPE(k_pe)] and values c_kv W_UV[h]."""
    rng = np.random.default_rng(41)
    B, H, L, dc, dn, dr, dv = 2, 3, 7, 16, 8, 8, 6
    q_nope, q_rope = rng.standard_normal((B, H, dn)), rng.standard_normal((B, H, dr))
    c_kv, k_pe_raw = rng.standard_normal((B, L, dc)), rng.standard_normal((B, L, dr))
    w_uk = rng.standard_normal((H, dc, dn)) / 4
    w_uv = rng.standard_normal((H, dc, dv)) / 4
    lens = np.array([L, 4])
    pos_tab = rope_tables(np.arange(L), dim=dr)
    cos, sin = (t.astype(np.float64) for t in pos_tab)
    k_pe = oracle.rope_ref(k_pe_raw, cos[None], sin[None])      # cached keys carry their own position
    qc = np.stack([cos[lens[b] - 1] for b in range(B)])[:, None]  # the query is the last token
    qs = np.stack([sin[lens[b] - 1] for b in range(B)])[:, None]
    q_rot = oracle.rope_ref(q_rope, qc, qs)
    scale = 1 / math.sqrt(dn + dr)
    ex, lex = oracle.mla_explicit_ref(q_nope, q_rot, c_kv, k_pe, w_uk, w_uv, lens, scale)
    q_abs = oracle.absorb_query(q_nope, q_rot, w_uk)
    lat, lab = oracle.mla_absorbed_ref(q_abs, np.concatenate([c_kv, k_pe], -1), lens, scale, d_v=dc)
    out = oracle.output_project(lat, w_uv)
    assert np.max(np.abs(out - ex)) <= 1e-10 and np.max(np.abs(lab - lex)) <= 1e-10


# ---------------------------------------------------------------------------
# Sparse (top-k) MLA decode: attention over the listed cache rows only
# (makesence §5.1).
# ---------------------------------------------------------------------------

def test_sparse_mla_brute_force_duplicates_and_skips():
    """Pure-Python loop over the listed rows: -1 and out-of-range entries are
    skipped, a row listed twice enters the softmax twice."""
    rng = np.random.default_rng(36)
    B, H, L, DK, DV = 2, 3, 9, 6, 4
    q = rng.standard_normal((B, H, DK))
    kv = rng.standard_normal((B, L, DK))
    idx = np.array([[4, 0, 4, 8, -1, 11], [2, -1, -1, 7, 3, 30]])
    out, lse = oracle.mla_sparse_ref(q, kv, idx, 0.4, d_v=DV)
    listed = [[4, 0, 4, 8], [2, 7, 3]]
    for b in range(B):
        for h in range(H):
            keys = [list(kv[b, j]) for j in listed[b]]
            vals = [list(kv[b, j, :DV]) for j in listed[b]]
            o, s_ = _brute_row(list(q[b, h]), keys, vals, 0.4)
            assert np.max(np.abs(out[b, h] - np.array(o))) <= 1e-12
            assert abs(lse[b, h] - s_) <= 1e-12


def test_sparse_mla_all_rows_equals_dense():
    """Listing every valid row (then -1 padding) is the dense absorbed decode."""
    q, kv, lens = mla_inputs(2, 4, 10, d_kv=12, dtype="f32", seed=37, lengths=(3, 9))
    idx = np.full((2, 10), -1)
    for b in range(2):
        idx[b, :lens[b]] = np.arange(lens[b])
    sp, lsp = oracle.mla_sparse_ref(q.f32(), kv.f32(), idx, 0.5, d_v=8)
    de, lde = oracle.mla_absorbed_ref(q.f32(), kv.f32(), lens, 0.5, d_v=8)
    assert np.max(np.abs(sp - de)) <= 1e-13
    assert np.max(np.abs(lsp - lde)) <= 1e-13


def test_sparse_mla_order_invariant_and_empty():
    q, kv, lens = mla_inputs(3, 4, 20, d_kv=12, dtype="f32", seed=38)
    idx = draw_topk(3, lens, 7, seed=38)
    base, lb = oracle.mla_sparse_ref(q.f32(), kv.f32(), idx, 0.5, d_v=8)
    perm = idx[:, ::-1].copy()
    p_, lp = oracle.mla_sparse_ref(q.f32(), kv.f32(), perm, 0.5, d_v=8)
    assert np.max(np.abs(p_ - base)) <= 1e-13 and np.max(np.abs(lp - lb)) <= 1e-13
    idx2 = idx.copy()
    idx2[1] = -1                                  # sequence 1 selects nothing
    e, le = oracle.mla_sparse_ref(q.f32(), kv.f32(), idx2, 0.5, d_v=8)
    assert np.all(e[1] == 0) and np.all(le[1] == -np.inf)
    assert np.array_equal(e[[0, 2]], base[[0, 2]])


def test_draw_topk_selects_distinct_positions():
    lens = np.array([50, 5, 8])
    idx = draw_topk(3, lens, 8, seed=3)
    for b in range(3):
        sel = idx[b][idx[b] >= 0]
        assert len(sel) == min(8, lens[b])
        assert len(set(sel.tolist())) == len(sel) and np.all(np.diff(sel) > 0)
        assert sel.min() >= 0 and sel.max() < lens[b]
        assert np.all(idx[b][len(sel):] == -1)


# ---------------------------------------------------------------------------
# O8: split/merge identity for split-KV decode.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cuts", [[0, 17], [0, 5, 17], [0, 1, 2, 16, 17], [0, 8, 8, 17], [0, 6, 12, 17, 17]])
def test_o8_lse_merge_identity(cuts):
    rng = np.random.default_rng(41)
    L, D = 17, 6
    q = rng.standard_normal(D) * 2
    keys = rng.standard_normal((L, D)) * 2
    vals = rng.standard_normal((L, 5))
    whole, lse = oracle.decode_ref(q[None, None], keys[None, None], vals[None, None], np.array([L]), 0.5)
    parts = [oracle.partial_ref(q, keys[a:b], vals[a:b], 0.5) for a, b in zip(cuts[:-1], cuts[1:])]
    o, l = oracle.lse_merge(parts)
    assert np.max(np.abs(o - whole[0, 0])) <= 1e-12
    assert abs(l - lse[0, 0]) <= 1e-12


def test_o8_partial_closed_form():
    m, l, o = oracle.partial_ref(np.array([1.0, 0.0]), np.array([[math.log(2.0), 0], [0.0, 0]]),
                                 np.array([[1.0], [4.0]]), 1.0)
    assert m == math.log(2.0) and abs(l - 1.5) <= 1e-15 and abs(o[0] - 3.0) <= 1e-15
    assert oracle.partial_ref(np.ones(2), np.zeros((0, 2)), np.zeros((0, 3)), 1.0)[1] == 0.0


# ---------------------------------------------------------------------------
# O9: KV-cache size closed forms against the values printed on the pages.
# ---------------------------------------------------------------------------

def test_o9_kv_sizes_match_pages():
    with open(os.path.join(GOLDEN, "kv_cache_sizes.json")) as f:
        entries = json.load(f)["entries"]
    seen = 0
    for e in entries:
        if e["kind"] == "mla":
            vals = oracle.kv_values_per_token("mla", d_c=e["d_c"], d_rope=e["d_rope"])
            if "values_per_token" in e:
                assert vals == e["values_per_token"]; seen += 1
            if "bytes_per_token" in e:
                assert vals * e["bytes_per_value"] == e["bytes_per_token"]; seen += 1
                gb = vals * e["bytes_per_value"] * 1e6 / 1e9
                assert abs(gb - e["gb_per_layer_at_1M_ctx"]) / e["gb_per_layer_at_1M_ctx"] < 0.01
            if "mha_values_per_token" in e:
                mha = oracle.kv_values_per_token("mha", n_heads=e["mha_n_heads"], head_dim=e["mha_head_dim"])
                assert mha == e["mha_values_per_token"]
                assert round(mha / vals) == e["approx_ratio"]; seen += 1
        elif e["kind"] == "mha":
            vals = oracle.kv_values_per_token("mha", n_heads=e["n_heads"], head_dim=e["head_dim"])
            if "bytes_per_token" in e:
                assert vals * e["bytes_per_value"] == e["bytes_per_token"]; seen += 1
                assert abs(vals * 2 * 1e6 / 1e9 - e["gb_per_layer_at_1M_ctx"]) / e["gb_per_layer_at_1M_ctx"] < 0.01
            if "values_per_token" in e:
                assert vals == e["values_per_token"]; seen += 1
                assert abs(vals * 1e6 - e["values_at_1M_ctx_approx"]) / e["values_at_1M_ctx_approx"] < 0.001
                assert abs(e["mla_d_c"] * 1e6 - e["mla_values_at_1M_ctx_approx"]) / e["mla_values_at_1M_ctx_approx"] < 0.01
                assert vals // e["mla_d_c"] == e["approx_ratio"]
        elif e["kind"] == "gqa":
            vals = oracle.kv_values_per_token("gqa", n_kv_heads=e["n_kv_heads"], head_dim=e["head_dim"])
            assert vals * e["bytes_per_value"] == e["bytes_per_token"]; seen += 1
            assert 65536 // (vals * 2) == e["ratio_vs_mha"]
        elif e["kind"] == "mqa":
            mqa = oracle.kv_values_per_token("mqa", head_dim=512)
            mha = oracle.kv_values_per_token("mha", n_heads=e["n_heads"], head_dim=512)
            assert mha // mqa == e["approx_ratio_vs_mha"]; seen += 1
    assert seen >= 7


# ---------------------------------------------------------------------------
# Input generator sanity (data only): bf16 rounding is round-to-nearest-even.
# ---------------------------------------------------------------------------

def test_bf16_rounding_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-39], dtype=np.float32)
    r = round_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                     # tie -> even (mantissa 0)
    assert r[2] == 1.0 + 4 * 2 ** -8       # tie -> even (up)
    assert r[3] == 1.0
    assert r[4] == -2.5
    bits = bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_to_f32(bits))[0]


def test_synthetic_slices_are_reproducible():
    q, k, v = prefill_inputs(2, 4, 1, 6, 8, "bf16", seed=0)
    q2, k2, v2 = prefill_inputs(2, 4, 1, 6, 8, "bf16", seed=0)
    assert np.array_equal(q.data, q2.data) and np.array_equal(v.data, v2.data)
    q3, _, _ = prefill_inputs(2, 4, 1, 6, 8, "bf16", seed=1)
    assert not np.array_equal(q.data, q3.data)
