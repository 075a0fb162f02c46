"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Inputs come from the seeded synthetic generator; the oracle reads the same
bf16-rounded values the device gets, upcast exactly.  Bars: max |err| <=
2e-2 for bf16 inputs, <= 1e-5 for fp32 (both on outputs and on the
natural-log LSE).  Small cases are compared element by element; the
full-size workloads (in the launch configuration the bench times) are
compared element by element in test_parity_full_gpu.py.
"""

import math
import sys

import numpy as np
import pytest

import oracle
from synthetic import (decode_inputs, decode_slice, mla_inputs, mla_slice, mla_step_inputs, prefill_inputs,
                       rope_tables, round_bf16, draw_lengths, draw_topk)

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5
# fp16 (10-bit mantissa; the bf16 bar's error budget scaled by the 8x finer
# rounding of inputs, P and output, with margin)
F16_TOL = 5e-3


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


@pytest.fixture(scope="module")
def mqa():
    import attention_mqa_gqa_amd as m
    return m


def dev(torch, t):
    """synthetic.Tensor -> device tensor with identical bits."""
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.data)).to("cuda")


def host(x):
    return x.float().cpu().numpy().astype(np.float64)


def _maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def test_prefill_f32_mqa_t128_full(torch, mqa):
    """fp32 MQA prefill B=1, Hq=16, Hkv=1, T=128, D=512, causal: every element."""
    _say("prefill f32 B1 Hq16 Hkv1 T128 D512")
    q, k, v = prefill_inputs(1, 16, 1, 128, 512, "f32", seed=0)
    lse = torch.empty((1, 16, 128), dtype=torch.float32, device="cuda")
    out = mqa.mqa_prefill(dev(torch, q), dev(torch, k), dev(torch, v), causal=True, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 1 / math.sqrt(512), True)
    assert _maxerr(host(out), ref) <= F32_TOL
    assert _maxerr(host(lse), ref_lse) <= F32_TOL


@pytest.mark.parametrize("B,Hq,Hkv,T,D,causal", [
    (1, 24, 1, 33, 128, True),     # a 16-row block holds part of a token's 24 heads
    (2, 48, 2, 21, 64, False),     # two KV heads of 24
    (1, 200, 1, 9, 64, True),      # 200 heads over one KV head: 12.5 blocks per token
    (1, 5, 1, 70, 256, True),      # blocks straddle tokens (16 = 3 x 5 + 1)
])
def test_prefill_f32_group_layouts(torch, mqa, B, Hq, Hkv, T, D, causal):
    """fp32 prefill rows are dealt in blocks of 16 (token x head-in-group):
    groups larger than a block and groups that do not divide it."""
    _say(f"prefill f32 B{B} Hq{Hq} Hkv{Hkv} T{T} D{D} causal={causal}")
    q, k, v = prefill_inputs(B, Hq, Hkv, T, D, "f32", seed=50 + Hq)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    out = mqa.mqa_prefill(dev(torch, q), dev(torch, k), dev(torch, v), causal=causal, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 1 / math.sqrt(D), causal)
    assert _maxerr(host(out), ref) <= F32_TOL
    assert _maxerr(host(lse), ref_lse) <= F32_TOL


PREFILL_SMALL = [
    # B, Hq, Hkv, T, D, causal, out dtype
    (2, 16, 1, 200, 512, True, "bf16"),
    (1, 16, 1, 200, 512, False, "f32"),
    (1, 16, 2, 129, 128, True, "f32"),
    (1, 8, 8, 77, 128, True, "bf16"),
    (1, 64, 8, 150, 128, True, "bf16"),
    (2, 4, 1, 1, 512, True, "bf16"),
    (1, 32, 1, 40, 128, True, "bf16"),
    (1, 128, 1, 20, 512, True, "f32"),
    (1, 12, 4, 65, 128, False, "bf16"),
    (1, 12, 1, 99, 512, True, "bf16"),        # group of 12 (not a power of two): 10 tokens per block
    (2, 6, 1, 70, 128, True, "f32"),          # group of 6
    # d = 128 groups above 128 heads (up to the 256 rows of a workgroup):
    # one token of all 256 heads per workgroup; 200 heads (1 token, 56 idle rows)
    (1, 256, 1, 37, 128, True, "bf16"),
    (1, 200, 1, 45, 128, True, "f32"),
    (2, 512, 2, 19, 128, False, "bf16"),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,D,causal,odt", PREFILL_SMALL)
def test_prefill_bf16_small(torch, mqa, B, Hq, Hkv, T, D, causal, odt):
    _say(f"prefill bf16 B{B} Hq{Hq} Hkv{Hkv} T{T} D{D} causal={causal} out={odt}")
    q, k, v = prefill_inputs(B, Hq, Hkv, T, D, "bf16", seed=1)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    out = mqa.mqa_prefill(dev(torch, q), dev(torch, k), dev(torch, v), causal=causal, lse=lse,
                          out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 1 / math.sqrt(D), causal)
    assert np.all(np.isfinite(host(out)))
    assert _maxerr(host(out), ref) <= BF16_TOL
    assert _maxerr(host(lse), ref_lse) <= BF16_TOL


def test_prefill_f32_ragged_and_gqa(torch, mqa):
    _say("prefill f32 B2 Hq6 Hkv3 T37 D128 causal + full")
    q, k, v = prefill_inputs(2, 6, 3, 37, 128, "f32", seed=2)
    for causal in (True, False):
        out = mqa.mqa_prefill(dev(torch, q), dev(torch, k), dev(torch, v), causal=causal, scale=0.3)
        torch.cuda.synchronize()
        ref, _ = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 0.3, causal)
        assert _maxerr(host(out), ref) <= F32_TOL


@pytest.mark.parametrize("D", [64, 192, 256, 320, 384, 448])
def test_prefill_f32_every_width(torch, mqa, D):
    """fp32 prefill at every width the fp32 kernel is built for (64 .. 512 in
    steps of 64; 128 and 512 are covered above), causal and full, GQA."""
    _say(f"prefill f32 B2 Hq6 Hkv2 T45 D{D}")
    q, k, v = prefill_inputs(2, 6, 2, 45, D, "f32", seed=30 + D)
    for causal in (True, False):
        lse = torch.empty((2, 6, 45), dtype=torch.float32, device="cuda")
        out = mqa.mqa_prefill(dev(torch, q), dev(torch, k), dev(torch, v), causal=causal, lse=lse)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 1 / math.sqrt(D), causal)
        assert _maxerr(host(out), ref) <= F32_TOL
        assert _maxerr(host(lse), ref_lse) <= F32_TOL


# ---------------------------------------------------------------------------
# general prefill: T_q != T_kv (bottom-right causal) and d_v != d_qk
# ---------------------------------------------------------------------------

PREFILL_EX_SMALL = [
    # B, Hq, Hkv, T_q, T_kv, d_qk, d_v, causal, out dtype
    (1, 4, 4, 300, 300, 192, 128, True, "bf16"),      # expanded MLA prefill, 2 token blocks, ragged tail
    (2, 3, 3, 77, 77, 192, 128, True, "f32"),
    (1, 8, 8, 130, 530, 192, 128, True, "bf16"),      # a chunk of 130 new tokens after 400
    (1, 2, 2, 100, 100, 192, 128, False, "bf16"),
    (2, 16, 1, 100, 777, 512, 512, True, "bf16"),     # MQA chunked prefill
    (1, 16, 1, 1, 300, 512, 512, True, "f32"),        # one new token
    (1, 64, 8, 200, 1000, 128, 128, True, "bf16"),    # GQA chunk
    (1, 16, 2, 33, 500, 128, 128, False, "bf16"),     # no mask, T_q < T_kv
    (1, 16, 1, 64, 40, 512, 512, False, "bf16"),      # no mask, T_q > T_kv
    # the largest group size (one token of 128 heads per workgroup)
    (1, 128, 1, 37, 37, 512, 512, True, "bf16"),
    (1, 128, 1, 20, 45, 192, 128, True, "bf16"),
    # multi-token decode (a few new tokens against a long cache, bottom-right
    # causal); the cache lengths end inside a key tile
    (2, 16, 1, 4, 2999, 512, 512, True, "bf16"),
    (3, 64, 8, 7, 1001, 128, 128, True, "bf16"),
    (1, 8, 8, 5, 333, 192, 128, True, "f32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tkv,DK,DV,causal,odt", PREFILL_EX_SMALL)
def test_prefill_ex_bf16_small(torch, mqa, B, Hq, Hkv, Tq, Tkv, DK, DV, causal, odt):
    _say(f"prefill_ex bf16 B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tkv{Tkv} DK{DK} DV{DV} causal={causal} out={odt}")
    q, k, v = prefill_inputs(B, Hq, Hkv, Tq, DK, "bf16", seed=3, d_v=DV, T_kv=Tkv)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    out = mqa.mqa_prefill_ex(dev(torch, q), dev(torch, k), dev(torch, v), causal=causal, lse=lse,
                             out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert out.shape == (B, Hq, Tq, DV)
    ref, ref_lse = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 1 / math.sqrt(DK), causal)
    assert np.all(np.isfinite(host(out)))
    assert _maxerr(host(out), ref) <= BF16_TOL
    assert _maxerr(host(lse), ref_lse) <= BF16_TOL


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_ex_f32(torch, mqa, causal):
    """fp32 end to end: expanded-MLA widths and a chunk (T_q < T_kv)."""
    for B, Hq, Hkv, Tq, Tkv, DK, DV in ((2, 4, 2, 37, 90, 192, 128), (1, 6, 3, 20, 61, 128, 128),
                                        (1, 16, 1, 5, 5, 192, 128)):
        _say(f"prefill_ex f32 B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tkv{Tkv} DK{DK} DV{DV} causal={causal}")
        q, k, v = prefill_inputs(B, Hq, Hkv, Tq, DK, "f32", seed=4, d_v=DV, T_kv=Tkv)
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
        out = mqa.mqa_prefill_ex(dev(torch, q), dev(torch, k), dev(torch, v), causal=causal, scale=0.11,
                                 lse=lse)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 0.11, causal)
        assert _maxerr(host(out), ref) <= F32_TOL
        assert _maxerr(host(lse), ref_lse) <= F32_TOL


F16_CASES = [
    # B, Hq, Hkv, T_q, T_kv, d_qk, d_v, causal, out dtype
    (2, 16, 1, 200, 200, 512, 512, True, "f16"),
    (1, 16, 1, 130, 333, 512, 512, True, "f32"),
    (1, 64, 8, 150, 150, 128, 128, True, "f16"),
    (1, 8, 8, 100, 300, 192, 128, True, "f16"),
    (1, 12, 4, 65, 65, 128, 128, False, "f32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tkv,DK,DV,causal,odt", F16_CASES)
def test_prefill_f16(torch, mqa, B, Hq, Hkv, Tq, Tkv, DK, DV, causal, odt):
    """fp16 inputs (the zdabc.icu benchmark's GPU dtype), fp16 or fp32 out."""
    _say(f"prefill f16 B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tkv{Tkv} DK{DK} DV{DV} causal={causal} out={odt}")
    q, k, v = prefill_inputs(B, Hq, Hkv, Tq, DK, "f16", seed=7, d_v=DV, T_kv=Tkv)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.float16
    fn = mqa.mqa_prefill if (Tq == Tkv and DK == DV) else mqa.mqa_prefill_ex
    out = fn(dev(torch, q), dev(torch, k), dev(torch, v), causal=causal, lse=lse, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert out.dtype == out_dtype
    ref, ref_lse = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 1 / math.sqrt(DK), causal)
    err = _maxerr(host(out), ref)
    _say(f"  max |err| {err:.2e}")
    assert err <= F16_TOL
    assert _maxerr(host(lse), ref_lse) <= F16_TOL


def test_prefill_ex_square_matches_prefill(torch, mqa):
    """mqa_prefill_ex with T_q = T_kv and d_v = d_qk is the square entry point,
    bit for bit."""
    _say("prefill_ex square vs prefill B1 Hq16 Hkv1 T150 D512")
    q, k, v = prefill_inputs(1, 16, 1, 150, 512, "bf16", seed=5)
    dq, dk, dv = dev(torch, q), dev(torch, k), dev(torch, v)
    a = mqa.mqa_prefill(dq, dk, dv, causal=True)
    b = mqa.mqa_prefill_ex(dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_calls_follow_the_given_stream(torch, mqa):
    """The library enqueues on the stream it is given: work queued on a side
    stream behind a long kernel still reads the inputs as they are when it
    runs, and the result is the same as on the default stream."""
    _say("prefill + decode on a side stream")
    q, k, v = prefill_inputs(1, 16, 1, 300, 512, "bf16", seed=12)
    dq, dk, dv = dev(torch, q), dev(torch, k), dev(torch, v)
    ref = mqa.mqa_prefill(dq, dk, dv, causal=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = mqa.mqa_prefill(dq, dk, dv, causal=True, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    qd, kc, vc, sl = decode_inputs(3, 16, 1, 500, 512, "bf16", seed=12, lengths=[500, 7, 260])
    dsl = torch.from_numpy(sl).cuda()
    a = mqa.mqa_decode(dev(torch, qd), dev(torch, kc), dev(torch, vc), dsl)
    with torch.cuda.stream(side):
        b = mqa.mqa_decode(dev(torch, qd), dev(torch, kc), dev(torch, vc), dsl, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_binding_rejects_mixed_dtypes(torch, mqa):
    """The C ABI takes one element type per call, so the binding refuses
    16-bit tensors of different types before anything is launched."""
    _say("binding: mixed dtypes rejected")
    bf, hf = torch.bfloat16, torch.float16
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")
    sl = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        mqa.mqa_prefill(z((1, 16, 64, 512), bf), z((1, 1, 64, 512), hf), z((1, 1, 64, 512), bf))
    with pytest.raises(TypeError):
        mqa.mqa_decode(z((2, 16, 128), bf), z((2, 1, 64, 128), bf), z((2, 1, 64, 128), hf), sl)
    with pytest.raises(TypeError):
        mqa.mla_decode_absorbed(z((2, 16, 576), hf), z((2, 64, 576), bf), sl)
    with pytest.raises(TypeError):
        mqa.mla_decode_sparse(z((2, 16, 576), bf), z((2, 64, 576), hf), z((2, 8), torch.int32))
    with pytest.raises(TypeError):
        mqa.mla_output_project(z((2, 16, 512), bf), z((16, 512, 128), hf))


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

DECODE_SMALL = [
    # B, Hq, Hkv, L_max, D, lengths, out dtype
    (5, 16, 1, 3000, 512, [1, 17, 2048, 2049, 3000], "bf16"),
    (4, 64, 8, 5000, 128, [1, 1023, 1024, 5000], "f32"),
    (3, 8, 8, 700, 128, [700, 3, 64], "bf16"),
    (2, 12, 3, 300, 512, [299, 300], "f32"),
    (3, 16, 16, 100, 128, [1, 2, 100], "bf16"),
    (2, 12, 1, 900, 512, [900, 333], "bf16"),  # group of 12 (padded to 16 MFMA columns)
    # more workgroups than the device holds at once: sequences taken longest
    # first (B <= 256), and in index order above that
    (160, 16, 8, 600, 128, (1, 600), "bf16"),
    (300, 8, 8, 64, 128, (1, 64), "f32"),
    # d = 128 with 12 and 16 query heads per KV head (12 of the 16 MFMA
    # columns used; all 16)
    (3, 24, 2, 1500, 128, [1500, 17, 1024], "bf16"),
    (2, 16, 1, 2100, 128, [2100, 999], "f32"),
    (2, 32, 2, 700, 128, [1, 700], "bf16"),
]


@pytest.mark.parametrize("B,Hq,Hkv,L,D,lengths,odt", DECODE_SMALL)
def test_decode_small(torch, mqa, B, Hq, Hkv, L, D, lengths, odt):
    _say(f"decode B{B} Hq{Hq} Hkv{Hkv} L{L} D{D} lens={lengths} out={odt}")
    q, kc, vc, sl = decode_inputs(B, Hq, Hkv, L, D, "bf16", seed=3, lengths=lengths)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    out = mqa.mqa_decode(dev(torch, q), dev(torch, kc), dev(torch, vc), torch.from_numpy(sl).cuda(),
                         lse=lse, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_ref(q.f32(), kc.f32(), vc.f32(), sl, 1 / math.sqrt(D))
    assert np.all(np.isfinite(host(out)))
    assert _maxerr(host(out), ref) <= BF16_TOL
    assert _maxerr(host(lse), ref_lse) <= BF16_TOL


def test_decode_zero_length_and_repeatability(torch, mqa):
    _say("decode zero-length rows, repeatability")
    q, kc, vc, sl = decode_inputs(3, 16, 1, 4500, 512, "bf16", seed=4, lengths=[4500, 1, 2500])
    dsl = torch.tensor([4500, 0, 2500], dtype=torch.int32, device="cuda")
    args = (dev(torch, q), dev(torch, kc), dev(torch, vc), dsl)
    lse = torch.empty((3, 16), dtype=torch.float32, device="cuda")
    out = mqa.mqa_decode(*args, lse=lse)
    out2 = mqa.mqa_decode(*args)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert float(out[1].float().abs().max()) == 0.0
    assert bool(torch.isinf(lse[1]).all()) and float(lse[1].max()) < 0
    ref, _ = oracle.decode_ref(q.f32()[[0, 2]], kc.f32()[[0, 2]], vc.f32()[[0, 2]], np.array([4500, 2500]),
                               1 / math.sqrt(512))
    assert _maxerr(host(out[[0, 2]]), ref) <= BF16_TOL


# ---------------------------------------------------------------------------
# MLA absorbed decode
# ---------------------------------------------------------------------------

MLA_SMALL = [
    # B, H, L_max, lengths, out dtype
    (3, 128, 2000, [1, 999, 2000], "bf16"),
    (2, 16, 300, [300, 33], "f32"),
    (2, 64, 1100, [1100, 1025], "bf16"),
    (2, 48, 500, [500, 77], "bf16"),     # heads not a multiple of 32: a wave's group is partly empty
    (1, 112, 300, [300], "f32"),
]


@pytest.mark.parametrize("B,H,L,lengths,odt", MLA_SMALL)
def test_mla_small(torch, mqa, B, H, L, lengths, odt):
    _say(f"mla B{B} H{H} L{L} lens={lengths} out={odt}")
    q, kv, sl = mla_inputs(B, H, L, 576, "bf16", seed=6, lengths=lengths)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    out = mqa.mla_decode_absorbed(dev(torch, q), dev(torch, kv), torch.from_numpy(sl).cuda(), lse=lse,
                                  out_dtype=out_dtype)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(192)
    ref, ref_lse = oracle.mla_absorbed_ref(q.f32(), kv.f32(), sl, scale)
    assert np.all(np.isfinite(host(out)))
    assert _maxerr(host(out), ref) <= BF16_TOL
    assert _maxerr(host(lse), ref_lse) <= BF16_TOL


@pytest.mark.parametrize("odt", ["bf16", "f32"])
def test_mla_merge_many_splits_ignores_unwritten_partials(torch, mqa, odt):
    """12 splits per sequence (more than the merge keeps in registers), a
    short second sequence whose later splits write no partial, 48 heads (the
    second 32-head group half empty), and a workspace filled with NaN first:
    only the partials this call wrote may reach the output."""
    _say(f"mla merge: 12 splits, lengths [6000, 700], H48, NaN workspace, out={odt}")
    B, H, L = 2, 48, 6000
    q, kv, sl = mla_inputs(B, H, L, 576, "bf16", seed=13, lengths=[6000, 700])
    ws = torch.full((mqa.mla_decode_workspace_size(B, H, L),), 0xFF, dtype=torch.uint8, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    out = mqa.mla_decode_absorbed(dev(torch, q), dev(torch, kv), torch.from_numpy(sl).cuda(), lse=lse,
                                  out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.mla_absorbed_ref(q.f32(), kv.f32(), sl, 1 / math.sqrt(192))
    assert np.all(np.isfinite(host(out)))
    assert _maxerr(host(out), ref) <= BF16_TOL
    assert _maxerr(host(lse), ref_lse) <= BF16_TOL


MLA_F16 = [
    # B, H, L_max, lengths, topk (0: dense), out dtype
    (3, 128, 1500, [1500, 31, 777], 0, "f16"),
    (2, 64, 600, [600, 65], 0, "f32"),
    (2, 128, 3000, [3000, 200], 512, "f16"),   # sparse: 512 listed rows (200 for the short sequence)
    (2, 32, 700, [700, 40], 0, "f16"),          # one block of 32 heads
    (2, 48, 2000, [2000, 90], 256, "f32"),      # sparse, two head blocks, the second half empty
    (1, 16, 300, [300], 64, "f16"),             # sparse, one block with 16 heads
]


@pytest.mark.parametrize("B,H,L,lengths,topk,odt", MLA_F16)
def test_mla_f16(torch, mqa, B, H, L, lengths, topk, odt):
    """fp16 queries and latent cache (dense and sparse), fp16 or fp32 out."""
    _say(f"mla f16 B{B} H{H} L{L} lens={lengths} topk={topk} out={odt}")
    q, kv, sl = mla_inputs(B, H, L, 576, "f16", seed=8, lengths=lengths)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.float16
    scale = 1 / math.sqrt(192)
    if topk:
        idx = draw_topk(B, sl, topk, seed=8)
        out = mqa.mla_decode_sparse(dev(torch, q), dev(torch, kv), torch.from_numpy(idx).cuda(), lse=lse,
                                    out_dtype=out_dtype)
        ref, ref_lse = oracle.mla_sparse_ref(q.f32(), kv.f32(), idx, scale)
    else:
        out = mqa.mla_decode_absorbed(dev(torch, q), dev(torch, kv), torch.from_numpy(sl).cuda(), lse=lse,
                                      out_dtype=out_dtype)
        ref, ref_lse = oracle.mla_absorbed_ref(q.f32(), kv.f32(), sl, scale)
    torch.cuda.synchronize()
    assert out.dtype == out_dtype
    assert np.all(np.isfinite(host(out)))
    err = _maxerr(host(out), ref)
    _say(f"  max |err| {err:.2e}")
    assert err <= F16_TOL
    assert _maxerr(host(lse), ref_lse) <= F16_TOL


@pytest.mark.parametrize("B,Hq,Hkv,L,D,lengths,odt", [(4, 16, 1, 3000, 512, (1, 3000), "f16"),
                                                      (8, 64, 8, 2500, 128, (1000, 2500), "f32")])
def test_decode_f16(torch, mqa, B, Hq, Hkv, L, D, lengths, odt):
    _say(f"decode f16 B{B} Hq{Hq} Hkv{Hkv} L{L} D{D} lens={lengths} out={odt}")
    q, k, v, sl = decode_inputs(B, Hq, Hkv, L, D, "f16", seed=8, lengths=lengths)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.float16
    out = mqa.mqa_decode(dev(torch, q), dev(torch, k), dev(torch, v), torch.from_numpy(sl).cuda(), lse=lse,
                         out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert out.dtype == out_dtype
    ref, ref_lse = oracle.decode_ref(q.f32(), k.f32(), v.f32(), sl, 1 / math.sqrt(D))
    err = _maxerr(host(out), ref)
    _say(f"  max |err| {err:.2e}")
    assert err <= F16_TOL
    assert _maxerr(host(lse), ref_lse) <= F16_TOL


# ---------------------------------------------------------------------------
# the steps around absorbed MLA decode: absorption + RoPE, cache append,
# output up-projection, and one whole decode step
# ---------------------------------------------------------------------------

def _cs(torch, positions):
    c, s_ = rope_tables(positions)
    return (torch.from_numpy(c).cuda(), torch.from_numpy(s_).cuda(), c.astype(np.float64), s_.astype(np.float64))


def test_mla_absorb_query(torch, mqa):
    _say("mla absorb query B37 H128")
    B, H = 37, 128
    qn, qr, _, _, wuk, _ = mla_step_inputs(B, H, seed=20)
    pos = np.random.default_rng(20).integers(0, 40000, size=B)
    dc, ds, c, s_ = _cs(torch, pos)
    q_abs = mqa.mla_absorb_query(dev(torch, qn), dev(torch, qr), dev(torch, wuk), dc, ds)
    torch.cuda.synchronize()
    ref = oracle.absorb_query(qn.f32(), oracle.rope_ref(qr.f32(), c[:, None], s_[:, None]), wuk.f32())
    assert _maxerr(host(q_abs), ref) <= BF16_TOL


def test_mla_cache_append(torch, mqa):
    _say("mla cache append B5 L64")
    B, L = 5, 64
    _, _, ckv, kpe, _, _ = mla_step_inputs(B, 16, seed=21)
    pos = np.array([0, 63, 17, 64, -1], dtype=np.int32)          # the last two are outside the cache: skipped
    dc, ds, c, s_ = _cs(torch, np.clip(pos, 0, None))
    cache = torch.zeros((B, L, 576), dtype=torch.bfloat16, device="cuda")
    mqa.mla_cache_append(cache, dev(torch, ckv), dev(torch, kpe), dc, ds, torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    got = host(cache)
    rot = oracle.rope_ref(kpe.f32(), c, s_)
    for b in range(B):
        if 0 <= pos[b] < L:
            row = got[b, pos[b]]
            assert np.array_equal(row[:512], ckv.f32()[b])                      # copied bits
            assert np.max(np.abs(row[512:] - rot[b])) <= 2 ** -8 * max(1.0, np.max(np.abs(rot[b])))
            got[b, pos[b]] = 0
    assert not got.any()                                                        # nothing else written


@pytest.mark.parametrize("B,odt", [(40, "bf16"), (16, "f32"), (3, "bf16")])
def test_mla_output_project(torch, mqa, B, odt):
    _say(f"mla output projection B{B} H128 out={odt}")
    H = 128
    _, _, _, _, _, wuv = mla_step_inputs(1, H, seed=22)
    o_lat, _, _ = mla_inputs(B, H, 1, 512, "bf16", seed=22)                   # any bf16 [B, H, 512]
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    out = mqa.mla_output_project(dev(torch, o_lat), dev(torch, wuv), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.output_project(o_lat.f32(), wuv.f32())
    assert _maxerr(host(out), ref) <= (F32_TOL * 100 if odt == "f32" else BF16_TOL)


def test_mla_step_f16(torch, mqa):
    """The three step kernels on fp16 tensors: absorption + RoPE, cache
    append (latent bits copied, RoPE part rounded to fp16), W_UV with fp16
    and fp32 output."""
    _say("mla step fp16: absorb B9 H128, append B3 L16, W_UV B20")
    B, H = 9, 128
    qn, qr, ckv, kpe, wuk, wuv = mla_step_inputs(B, H, "f16", seed=25)
    pos = np.random.default_rng(25).integers(0, 40000, size=B)
    dc, ds, c, s_ = _cs(torch, pos)
    q_abs = mqa.mla_absorb_query(dev(torch, qn), dev(torch, qr), dev(torch, wuk), dc, ds)
    torch.cuda.synchronize()
    assert q_abs.dtype == torch.float16
    ref = oracle.absorb_query(qn.f32(), oracle.rope_ref(qr.f32(), c[:, None], s_[:, None]), wuk.f32())
    assert _maxerr(host(q_abs), ref) <= F16_TOL

    L = 16
    p3 = np.array([0, 15, 7], dtype=np.int32)
    dc3, ds3, c3, s3 = _cs(torch, p3)
    cache = torch.zeros((3, L, 576), dtype=torch.float16, device="cuda")
    mqa.mla_cache_append(cache, dev(torch, ckv)[:3].contiguous(), dev(torch, kpe)[:3].contiguous(), dc3, ds3,
                         torch.from_numpy(p3).cuda())
    torch.cuda.synchronize()
    got = host(cache)
    rot = oracle.rope_ref(kpe.f32()[:3], c3, s3)
    for b in range(3):
        row = got[b, p3[b]]
        assert np.array_equal(row[:512], ckv.f32()[b])
        assert np.max(np.abs(row[512:] - rot[b])) <= 2 ** -10 * max(1.0, np.max(np.abs(rot[b])))

    o_lat, _, _ = mla_inputs(20, H, 1, 512, "f16", seed=25)
    for out_dtype in (torch.float16, torch.float32):
        out = mqa.mla_output_project(dev(torch, o_lat), dev(torch, wuv), out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert out.dtype == out_dtype
        assert _maxerr(host(out), oracle.output_project(o_lat.f32(), wuv.f32())) <= F16_TOL


def test_mla_decode_step_end_to_end(torch, mqa):
    """Cache built token by token with mla_cache_append, then one step:
    mla_absorb_query -> mla_decode_absorbed -> mla_output_project, against
    explicit attention on rebuilt per-head keys [c_kv W_UK | RoPE(k_pe)] and
    values c_kv W_UV (bf16 intermediates: q_abs, cache, o_lat)."""
    _say("mla decode step end to end B4 H128 L48")
    B, H, L = 4, 128, 48
    qn, qr, _, _, wuk, wuv = mla_step_inputs(B, H, seed=23)
    lens = np.array([48, 1, 30, 17], dtype=np.int32)
    rng = np.random.default_rng(23)
    from synthetic import Tensor, bf16_bits
    ckv_all = Tensor(bf16_bits(rng.standard_normal((B, L, 512), dtype=np.float32)), "bf16")
    kpe_all = Tensor(bf16_bits(rng.standard_normal((B, L, 64), dtype=np.float32)), "bf16")
    cache = torch.zeros((B, L, 576), dtype=torch.bfloat16, device="cuda")
    dck, dkp = dev(torch, ckv_all), dev(torch, kpe_all)
    for t in range(L):
        pos = np.where(t < lens, t, -1).astype(np.int32)
        dc, ds, _, _ = _cs(torch, np.full(B, t))
        mqa.mla_cache_append(cache, dck[:, t].contiguous(), dkp[:, t].contiguous(), dc, ds,
                             torch.from_numpy(pos).cuda())
    dc, ds, c, s_ = _cs(torch, lens - 1)
    q_abs = mqa.mla_absorb_query(dev(torch, qn), dev(torch, qr), dev(torch, wuk), dc, ds)
    o_lat = mqa.mla_decode_absorbed(q_abs, cache, torch.from_numpy(lens).cuda())
    out = mqa.mla_output_project(o_lat, dev(torch, wuv), out_dtype=torch.float32)
    torch.cuda.synchronize()
    tc, ts = (t.astype(np.float64) for t in rope_tables(np.arange(L)))
    k_rot = oracle.rope_ref(kpe_all.f32(), tc[None], ts[None])
    q_rot = oracle.rope_ref(qr.f32(), c[:, None], s_[:, None])
    ref, _ = oracle.mla_explicit_ref(qn.f32(), q_rot, ckv_all.f32(), k_rot, wuk.f32(), wuv.f32(), lens,
                                     1 / math.sqrt(192))
    assert _maxerr(host(out), ref) <= BF16_TOL


def test_mla_step_graph_replay(torch, mqa):
    """A whole absorbed decode step (absorb + RoPE and cache append on two
    branches, absorbed attention with its merge, W_UV) captured once in a HIP
    graph through the C ABI and replayed: every replay, with the program's
    own eager work and synchronisations in between, equals the eager step
    bit for bit."""
    _say("mla decode step as a HIP graph B6 H128 L96")
    B, H, L = 6, 128, 96
    qn, qr, ckv, kpe, wuk, wuv = (dev(torch, t) for t in mla_step_inputs(B, H, seed=24))
    lens = np.array([96, 1, 50, 95, 17, 64], dtype=np.int32)
    pos = torch.from_numpy(lens - 1).cuda()
    dsl = torch.from_numpy(lens).cuda()
    dc, ds, _, _ = _cs(torch, lens - 1)
    rng = np.random.default_rng(24)
    from synthetic import Tensor, bf16_bits
    cache0 = dev(torch, Tensor(bf16_bits(rng.standard_normal((B, L, 576), dtype=np.float32)), "bf16"))
    q_abs = torch.empty((B, H, 576), dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mqa.mla_decode_workspace_size(B, H, L), dtype=torch.uint8, device="cuda")
    cache = cache0.clone()

    branch = torch.cuda.Stream()

    def step():
        # absorption and cache append as two branches, joined before the
        # attention
        main = torch.cuda.current_stream()
        branch.wait_stream(main)
        mqa.mla_absorb_query(qn, qr, wuk, dc, ds, out=q_abs)
        with torch.cuda.stream(branch):
            mqa.mla_cache_append(cache, ckv, kpe, dc, ds, pos, stream=branch)
        main.wait_stream(branch)
        mqa.mla_decode_absorbed(q_abs, cache, dsl, out=o_lat, workspace=ws)
        mqa.mla_output_project(o_lat, wuv, out=out)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q_abs, cache, o_lat, out)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (q_abs, o_lat, out):
            t.zero_()                            # eager work between replays
        cache.copy_(cache0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((q_abs, cache, o_lat, out), ref):
            assert torch.equal(got, want), f"replay {rep}"


def test_prefill_and_decode_graph_replay(torch, mqa):
    """MQA prefill (16-bit with its packing pass, and fp32), GQA prefill and
    MQA/GQA decode captured once in a HIP graph through the C ABI and
    replayed three times, with eager work between the replays: every replay
    equals the eager calls bit for bit (the library records no memset and
    allocates nothing, so its calls can be captured)."""
    _say("prefill + decode as a HIP graph")
    q, k, v = (dev(torch, t) for t in prefill_inputs(1, 16, 1, 300, 512, "bf16", seed=61))
    qg, kg, vg = (dev(torch, t) for t in prefill_inputs(1, 16, 2, 200, 128, "bf16", seed=62))
    qf, kf, vf = (dev(torch, t) for t in prefill_inputs(1, 4, 1, 70, 256, "f32", seed=63))
    dq, dk, dv, sl = decode_inputs(3, 16, 1, 2100, 512, "bf16", seed=64, lengths=[2100, 5, 1000])
    dq, dk, dv = dev(torch, dq), dev(torch, dk), dev(torch, dv)
    dsl = torch.from_numpy(sl).cuda()
    gq, gk, gv, gsl = decode_inputs(2, 32, 4, 1500, 128, "bf16", seed=65, lengths=[1500, 77])
    gq, gk, gv = dev(torch, gq), dev(torch, gk), dev(torch, gv)
    gsl = torch.from_numpy(gsl).cuda()
    outs = [torch.empty((1, 16, 300, 512), dtype=torch.bfloat16, device="cuda"),
            torch.empty((1, 16, 200, 128), dtype=torch.bfloat16, device="cuda"),
            torch.empty((1, 4, 70, 256), dtype=torch.float32, device="cuda"),
            torch.empty((3, 16, 512), dtype=torch.bfloat16, device="cuda"),
            torch.empty((2, 32, 128), dtype=torch.bfloat16, device="cuda")]
    lses = [torch.empty((1, 16, 300), dtype=torch.float32, device="cuda"),
            torch.empty((3, 16), dtype=torch.float32, device="cuda")]
    ws = [torch.empty(mqa.mqa_prefill_workspace_size(1, 16, 1, 300, 512, mqa.DTYPE_BF16), dtype=torch.uint8, device="cuda"),
          torch.empty(mqa.mqa_prefill_workspace_size(1, 16, 2, 200, 128, mqa.DTYPE_BF16), dtype=torch.uint8, device="cuda"),
          torch.empty(mqa.mqa_decode_workspace_size(3, 16, 1, 2100, 512), dtype=torch.uint8, device="cuda"),
          torch.empty(mqa.mqa_decode_workspace_size(2, 32, 4, 1500, 128), dtype=torch.uint8, device="cuda")]

    def step():
        mqa.mqa_prefill(q, k, v, causal=True, out=outs[0], lse=lses[0], workspace=ws[0])
        mqa.mqa_prefill(qg, kg, vg, causal=True, out=outs[1], workspace=ws[1])
        mqa.mqa_prefill(qf, kf, vf, causal=False, out=outs[2])
        mqa.mqa_decode(dq, dk, dv, dsl, out=outs[3], lse=lses[1], workspace=ws[2])
        mqa.mqa_decode(gq, gk, gv, gsl, out=outs[4], workspace=ws[3])

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs + lses]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs + lses + ws:
            t.zero_()                            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs + lses, ref):
            assert torch.equal(got, want), f"replay {rep}"


# ---------------------------------------------------------------------------
# sparse (top-k) MLA decode
# ---------------------------------------------------------------------------

def _sparse_check(torch, mqa, q, kv, idx, odt="bf16"):
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    out = mqa.mla_decode_sparse(dev(torch, q), dev(torch, kv), torch.from_numpy(idx).cuda(), lse=lse,
                                out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.mla_sparse_ref(q.f32(), kv.f32(), idx, 1 / math.sqrt(192))
    got, got_lse = host(out), host(lse)
    assert np.all(np.isfinite(got))
    assert _maxerr(got, ref) <= BF16_TOL
    empty = np.isinf(ref_lse)
    assert np.array_equal(np.isinf(got_lse), empty)
    if (~empty).any():
        assert _maxerr(got_lse[~empty], ref_lse[~empty]) <= BF16_TOL
    return out


SPARSE_SMALL = [
    # B, H, L_max, lengths, topk, out dtype
    (3, 128, 5000, [5000, 3100, 500], 700, "bf16"),     # 500 < topk: -1 padding
    (2, 64, 3000, None, 1000, "f32"),
    (2, 16, 100, [100, 1], 1, "bf16"),
    (1, 32, 40000, None, 2048, "bf16"),
    (2, 80, 900, [900, 400], 333, "bf16"),   # 80 heads, a list length that ends inside a tile
]


@pytest.mark.parametrize("B,H,L,lengths,topk,odt", SPARSE_SMALL)
def test_mla_sparse_small(torch, mqa, B, H, L, lengths, topk, odt):
    _say(f"mla sparse B{B} H{H} L{L} lens={lengths} topk={topk} out={odt}")
    q, kv, sl = mla_inputs(B, H, L, 576, "bf16", seed=10, lengths=lengths)
    idx = draw_topk(B, sl, topk, seed=10)
    _sparse_check(torch, mqa, q, kv, idx, odt)


def test_mla_sparse_unsorted_duplicates_and_skips(torch, mqa):
    """Unsorted lists, a repeated row, entries outside [0, L_max) (never
    read), and a sequence that selects nothing (out 0, lse -inf)."""
    _say("mla sparse irregular lists B3 H128 L900 topk 300")
    B, H, L, k = 3, 128, 900, 300
    q, kv, sl = mla_inputs(B, H, L, 576, "bf16", seed=11, lengths=[900, 900, 450])
    rng = np.random.default_rng(11)
    idx = np.full((B, k), -1, dtype=np.int32)
    idx[0] = rng.permutation(900)[:k]                       # unsorted, distinct
    idx[0, 17] = idx[0, 3]                                  # a repeated row
    idx[0, 250:260] = [-1, 900, 5000, -7, 2 ** 30, -1, 899, 0, -2 ** 31, 12]
    idx[1] = -1                                             # nothing selected
    idx[2, :200] = rng.permutation(450)[:200]               # NaN rows >= 450 never listed
    _sparse_check(torch, mqa, q, kv, idx)


def test_mla_sparse_all_rows_equals_dense(torch, mqa):
    """Listing rows 0..L_b-1 gives the dense absorbed decode (same kernel
    arithmetic, different chunking)."""
    _say("mla sparse vs dense B2 H128 L1500")
    q, kv, sl = mla_inputs(2, 128, 1500, 576, "bf16", seed=12, lengths=[1500, 777])
    idx = np.full((2, 1500), -1, dtype=np.int32)
    for b in range(2):
        idx[b, :sl[b]] = np.arange(sl[b])
    sp = _sparse_check(torch, mqa, q, kv, idx)
    de = mqa.mla_decode_absorbed(dev(torch, q), dev(torch, kv), torch.from_numpy(sl).cuda())
    torch.cuda.synchronize()
    assert _maxerr(host(sp), host(de)) <= BF16_TOL


# ---------------------------------------------------------------------------
# Running-maximum stress: key magnitudes grow along the sequence, so the
# row maxima keep rising by far more than the kernels' lazy-rescale slack
# (2^8) from tile to tile and every rescale path is taken many times.
# ---------------------------------------------------------------------------

def _grow_keys(t, axis, rate, cols=slice(None)):
    """bf16 Tensor with slice j along `axis` (last-axis columns `cols` only)
    multiplied by (1 + rate * j)."""
    from synthetic import Tensor, bf16_bits
    x = t.f32().copy()
    shape = [1] * x.ndim
    shape[axis] = x.shape[axis]
    x[..., cols] *= (1.0 + rate * np.arange(x.shape[axis], dtype=np.float32)).reshape(shape)
    return Tensor(bf16_bits(x), "bf16")


@pytest.mark.parametrize("B,Hq,Hkv,T,D", [(1, 16, 1, 300, 512), (1, 64, 8, 300, 128)])
def test_prefill_growing_scores(torch, mqa, B, Hq, Hkv, T, D):
    _say(f"prefill growing scores B{B} Hq{Hq} Hkv{Hkv} T{T} D{D}")
    q, k, v = prefill_inputs(B, Hq, Hkv, T, D, "bf16", seed=7)
    k = _grow_keys(k, 2, 0.1)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    out = mqa.mqa_prefill(dev(torch, q), dev(torch, k), dev(torch, v), causal=True, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill_ref(q.f32(), k.f32(), v.f32(), 1 / math.sqrt(D), True)
    assert np.all(np.isfinite(host(out)))
    assert _maxerr(host(out), ref) <= BF16_TOL
    assert _maxerr(host(lse), ref_lse) <= BF16_TOL


@pytest.mark.parametrize("B,Hq,Hkv,L,D,lengths", [(2, 16, 1, 2500, 512, [2500, 700]),
                                                   (2, 64, 8, 2500, 128, [2500, 1300])])
def test_decode_growing_scores(torch, mqa, B, Hq, Hkv, L, D, lengths):
    _say(f"decode growing scores B{B} Hq{Hq} Hkv{Hkv} L{L} D{D}")
    q, kc, vc, sl = decode_inputs(B, Hq, Hkv, L, D, "bf16", seed=8, lengths=lengths)
    kc = _grow_keys(kc, 2, 0.02)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out = mqa.mqa_decode(dev(torch, q), dev(torch, kc), dev(torch, vc), torch.from_numpy(sl).cuda(), lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_ref(q.f32(), kc.f32(), vc.f32(), sl, 1 / math.sqrt(D))
    assert np.all(np.isfinite(host(out)))
    assert _maxerr(host(out), ref) <= BF16_TOL
    assert _maxerr(host(lse), ref_lse) <= BF16_TOL


def test_mla_growing_scores(torch, mqa):
    _say("mla growing scores B2 H128 L1500")
    q, kv, sl = mla_inputs(2, 128, 1500, 576, "bf16", seed=9, lengths=[1500, 640])
    # the latent is also the value: grow only the RoPE part (key-only columns)
    kv = _grow_keys(kv, 1, 0.05, cols=slice(512, 576))
    lse = torch.empty((2, 128), dtype=torch.float32, device="cuda")
    out = mqa.mla_decode_absorbed(dev(torch, q), dev(torch, kv), torch.from_numpy(sl).cuda(), lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.mla_absorbed_ref(q.f32(), kv.f32(), sl, 1 / math.sqrt(192))
    assert np.all(np.isfinite(host(out)))
    assert _maxerr(host(out), ref) <= BF16_TOL
    assert _maxerr(host(lse), ref_lse) <= BF16_TOL
