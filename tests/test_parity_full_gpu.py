"""GPU parity at the full benchmark sizes: EVERY output element and every
log-sum-exp of each workload the bench times, in the launch configuration
the bench uses, against the fp64 oracle.

The oracle is evaluated one (batch, head) slice at a time on a pool of host
threads (each slice is an ordinary call of the oracle function on a
one-head tensor, so its arithmetic is exactly the definition's); each
worker compares its slice with the device result and keeps only the
largest error, so the full fp64 reference is never held in memory at once.

Bars: max |err| <= 2e-2 (bf16 inputs), <= 5e-3 (fp16), on outputs and LSE.
Each workload is also run twice and required to be bitwise repeatable.
"""

import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from synthetic import decode_inputs, draw_topk, mla_inputs, prefill_inputs

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F16_TOL = 5e-3


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _workers():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 4)
    # each prefill slice holds a few T x T fp64 arrays (0.5 GB at T = 8192)
    return max(1, min(8, n))


def _pool_max(fn, items):
    """max over fn(item) on a thread pool, BLAS kept to one thread per worker."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            errs = list(ex.map(fn, items))
    return max(errs)


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
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.data)).to("cuda")


def _host32(x):
    return x.float().cpu().numpy()


def _err(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


# ---------------------------------------------------------------------------
# prefill: every (b, h) slice of the output and LSE
# ---------------------------------------------------------------------------

def _check_prefill_full(q, k, v, out, lse, scale, causal, tol):
    B, Hq = q.shape[0], q.shape[1]
    Hkv = k.shape[1]
    G = Hq // Hkv
    got, got_lse = _host32(out), _host32(lse)
    assert np.all(np.isfinite(got))

    def one(bh):
        b, h = bh
        g = h // G
        ref, ref_lse = oracle.prefill_ref(q.f32((slice(b, b + 1), slice(h, h + 1))),
                                          k.f32((slice(b, b + 1), slice(g, g + 1))),
                                          v.f32((slice(b, b + 1), slice(g, g + 1))), scale, causal)
        return max(_err(got[b, h], ref[0, 0]), _err(got_lse[b, h], ref_lse[0, 0]))

    err = _pool_max(one, [(b, h) for b in range(B) for h in range(Hq)])
    _say(f"  max |err| over every element and lse: {err:.3e}")
    assert err <= tol


PREFILL_FULL = [
    # name, B, Hq, Hkv, T_q, T_kv, d_qk, d_v, dtype
    ("mqa_prefill_bf16_b2_t4096", 2, 16, 1, 4096, 4096, 512, 512, "bf16"),
    ("mqa_prefill_f16_b2_t4096", 2, 16, 1, 4096, 4096, 512, 512, "f16"),
    ("gqa_prefill_bf16_b1_t8192", 1, 64, 8, 8192, 8192, 128, 128, "bf16"),
    ("mla_prefill_bf16_b1_h128_t8192", 1, 128, 128, 8192, 8192, 192, 128, "bf16"),
    ("mqa_chunk_prefill_bf16_b2_q1024_kv8192", 2, 16, 1, 1024, 8192, 512, 512, "bf16"),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,Tq,Tkv,DK,DV,dt", PREFILL_FULL)
def test_prefill_full_size_every_element(torch, mqa, name, B, Hq, Hkv, Tq, Tkv, DK, DV, dt):
    """Causal prefill at the bench's full size (the same entry point, shapes,
    seed and output type as the bench), every output element and LSE."""
    _say(f"{name}: B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tkv{Tkv} d{DK}/{DV} {dt}")
    q, k, v = prefill_inputs(B, Hq, Hkv, Tq, DK, dt, seed=0, d_v=DV, T_kv=Tkv)
    dq, dk, dv = dev(torch, q), dev(torch, k), dev(torch, v)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    fn = mqa.mqa_prefill if (Tq == Tkv and DK == DV) else mqa.mqa_prefill_ex
    out = fn(dq, dk, dv, causal=True, lse=lse)
    out2 = fn(dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    _check_prefill_full(q, k, v, out, lse, 1 / math.sqrt(DK), True, F16_TOL if dt == "f16" else BF16_TOL)


# ---------------------------------------------------------------------------
# decode: every sequence
# ---------------------------------------------------------------------------

def _check_decode_full(q, kc, vc, sl, out, lse, scale):
    got, got_lse = _host32(out), _host32(lse)
    assert np.all(np.isfinite(got))

    def one(b):
        L = int(sl[b])
        ref, ref_lse = oracle.decode_ref(q.f32(slice(b, b + 1)), kc.f32((slice(b, b + 1), slice(None), slice(0, L))),
                                         vc.f32((slice(b, b + 1), slice(None), slice(0, L))), np.array([L]), scale)
        return max(_err(got[b], ref[0]), _err(got_lse[b], ref_lse[0]))

    err = _pool_max(one, range(q.shape[0]))
    _say(f"  max |err| over every sequence: {err:.3e}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("name,B,Hq,Hkv,L,D,lengths", [
    ("mqa_decode_bf16_b64_l8192", 64, 16, 1, 8192, 512, None),
    ("gqa_decode_bf16_b128_l1024to16384", 128, 64, 8, 16384, 128, (1024, 16384)),
])
def test_decode_full_size_every_sequence(torch, mqa, name, B, Hq, Hkv, L, D, lengths):
    _say(f"{name}: B{B} Hq{Hq} Hkv{Hkv} L{L} D{D} lengths={lengths}")
    q, kc, vc, sl = decode_inputs(B, Hq, Hkv, L, D, "bf16", seed=0, lengths=lengths)
    dq, dk, dv = dev(torch, q), dev(torch, kc), dev(torch, vc)
    dsl = torch.from_numpy(sl).cuda()
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out = mqa.mqa_decode(dq, dk, dv, dsl, lse=lse)
    out2 = mqa.mqa_decode(dq, dk, dv, dsl)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    del dk, dv
    _check_decode_full(q, kc, vc, sl, out, lse, 1 / math.sqrt(D))


# ---------------------------------------------------------------------------
# MLA absorbed decode (dense and top-k sparse): every sequence
# ---------------------------------------------------------------------------

def test_mla_full_size_every_sequence(torch, mqa):
    """mla_decode_bf16_b32_l32768: batch 32, H=128, context 32768, 1/sqrt(192)."""
    B, H, L = 32, 128, 32768
    _say(f"mla_decode_bf16_b32_l32768: B{B} H{H} L{L}")
    q, kv, sl = mla_inputs(B, H, L, 576, "bf16", seed=0)
    dq, dkv, dsl = dev(torch, q), dev(torch, kv), torch.from_numpy(sl).cuda()
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out = mqa.mla_decode_absorbed(dq, dkv, dsl, lse=lse)
    out2 = mqa.mla_decode_absorbed(dq, dkv, dsl)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    del dkv
    got, got_lse = _host32(out), _host32(lse)
    assert np.all(np.isfinite(got))
    scale = 1 / math.sqrt(192)

    def one(b):
        ref, ref_lse = oracle.mla_absorbed_ref(q.f32(slice(b, b + 1)), kv.f32(slice(b, b + 1)), sl[b:b + 1], scale)
        return max(_err(got[b], ref[0]), _err(got_lse[b], ref_lse[0]))

    err = _pool_max(one, range(B))
    _say(f"  max |err| over every sequence: {err:.3e}")
    assert err <= BF16_TOL


def test_mla_sparse_full_size_every_sequence(torch, mqa):
    """mla_sparse_decode_bf16_b32_l32768_k2048: 2048 listed rows per sequence."""
    B, H, L, k = 32, 128, 32768, 2048
    _say(f"mla_sparse_decode_bf16_b32_l32768_k2048: B{B} H{H} L{L} topk {k}")
    q, kv, sl = mla_inputs(B, H, L, 576, "bf16", seed=0)
    idx = draw_topk(B, sl, k, seed=0)
    dq, dkv, didx = dev(torch, q), dev(torch, kv), torch.from_numpy(idx).cuda()
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out = mqa.mla_decode_sparse(dq, dkv, didx, lse=lse)
    out2 = mqa.mla_decode_sparse(dq, dkv, didx)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    del dkv
    got, got_lse = _host32(out), _host32(lse)
    assert np.all(np.isfinite(got))
    scale = 1 / math.sqrt(192)

    def one(b):
        ref, ref_lse = oracle.mla_sparse_ref(q.f32(slice(b, b + 1)), kv.f32(slice(b, b + 1)), idx[b:b + 1], scale)
        return max(_err(got[b], ref[0]), _err(got_lse[b], ref_lse[0]))

    err = _pool_max(one, range(B))
    _say(f"  max |err| over every sequence: {err:.3e}")
    assert err <= BF16_TOL


# ---------------------------------------------------------------------------
# split-plan invariance: the same sequences under two different split plans
# ---------------------------------------------------------------------------

def test_decode_split_plan_invariance(torch, mqa):
    """The split-KV plan depends on the cache capacity max_len and the batch:
    the same sequences stored in caches of 8192 and of 32768 rows are cut
    into chunks of different lengths (MQA d=512, batch 80: 2048 vs 2560
    rows; GQA d=128, 5 x 8 KV heads: 1024 vs 1280), so workgroup counts,
    per-wave row ranges and merge orders all differ.  Both results must
    match the oracle and each other within the bar; each is bitwise
    repeatable."""
    _say("decode split-plan invariance: max_len 8192 vs 32768, MQA d=512 and GQA d=128")
    for B, Hq, Hkv, D, lens in ((80, 16, 1, 512, (1, 8192)),
                                (5, 64, 8, 128, [8192, 1024, 3, 5555, 8000])):
        assert mqa.mqa_decode_workspace_size(B, Hq, Hkv, 8192, D) != mqa.mqa_decode_workspace_size(B, Hq, Hkv, 32768, D)
        q, kc, vc, sl = decode_inputs(B, Hq, Hkv, 8192, D, "bf16", seed=21, lengths=lens)
        dq, dk, dv = dev(torch, q), dev(torch, kc), dev(torch, vc)
        dsl = torch.from_numpy(sl).cuda()
        big_k = torch.full((B, Hkv, 32768, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        big_v = big_k.clone()
        big_k[:, :, :8192] = dk
        big_v[:, :, :8192] = dv
        a = mqa.mqa_decode(dq, dk, dv, dsl)
        b = mqa.mqa_decode(dq, big_k, big_v, dsl)
        b2 = mqa.mqa_decode(dq, big_k, big_v, dsl)
        torch.cuda.synchronize()
        assert torch.equal(b, b2)
        ref, _ = oracle.decode_ref(q.f32(), kc.f32(), vc.f32(), sl, 1 / math.sqrt(D))
        assert _err(_host32(a), ref) <= BF16_TOL
        assert _err(_host32(b), ref) <= BF16_TOL
        assert _err(_host32(a), _host32(b)) <= BF16_TOL
        del big_k, big_v


def test_mla_split_plan_invariance(torch, mqa):
    """Absorbed MLA decode of the same 32 sequences in latent caches of 4096
    and 32768 rows: the plan cuts each sequence into chunks of 512 rows in
    the first and into one chunk of 4096 in the second (up to 8 workgroups
    and a merge of their partials vs one workgroup per sequence)."""
    _say("mla split-plan invariance: max_len 4096 vs 32768")
    B, H = 32, 128
    q, kv, sl = mla_inputs(B, H, 4096, 576, "bf16", seed=22, lengths=(1, 4096))
    dq, dkv, dsl = dev(torch, q), dev(torch, kv), torch.from_numpy(sl).cuda()
    big = torch.full((B, 32768, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    big[:, :4096] = dkv
    a = mqa.mla_decode_absorbed(dq, dkv, dsl)
    b = mqa.mla_decode_absorbed(dq, big, dsl)
    b2 = mqa.mla_decode_absorbed(dq, big, dsl)
    torch.cuda.synchronize()
    assert torch.equal(b, b2)
    ref, _ = oracle.mla_absorbed_ref(q.f32(), kv.f32(), sl, 1 / math.sqrt(192))
    assert _err(_host32(a), ref) <= BF16_TOL
    assert _err(_host32(b), ref) <= BF16_TOL
    assert _err(_host32(a), _host32(b)) <= BF16_TOL
