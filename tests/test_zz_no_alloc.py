"""mqa_decode_noalloc (the decode entry point that allocates nothing: its
split partials live in the library's fixed per-device scratch) against
mqa_decode with a caller workspace: the same kernels and plan, so the
results must be identical bit for bit, and both within the bf16 bar of the
fp64 oracle.  Two calls in a row on the shared scratch, the second one
smaller (a different plan and fewer partials than the first left behind),
then a call that needs more than the scratch holds: rejected with
MQA_ERR_WORKSPACE and nothing written.  Driven through the C ABI (ctypes)."""

import ctypes
import math
import sys

import numpy as np
import pytest

import oracle
from synthetic import decode_inputs

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


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


def _dev(torch, t):
    return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).to("cuda").view(torch.bfloat16)


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _noalloc(torch, mqa, q, k, v, sl, out, lse, D):
    B, Hq = q.shape[0], q.shape[1]
    Hkv, L = k.shape[1], k.shape[2]
    stream = torch.cuda.current_stream().cuda_stream
    return mqa.lib.mqa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), sl.data_ptr(), out.data_ptr(),
                                      lse.data_ptr() if lse is not None else None, B, Hq, Hkv, L, D,
                                      1.0 / math.sqrt(D), mqa.DTYPE_BF16, mqa.DTYPE_BF16, ctypes.c_void_p(stream))


@pytest.mark.parametrize("B,Hq,Hkv,L,D,lengths", [
    (64, 16, 1, 8192, 512, None),                      # MQA decode, batch 64, cache 8192 (8.4 MB of partials)
    (5, 64, 8, 3000, 128, [3000, 1, 1024, 2999, 77]),  # then a smaller GQA call on the same scratch
])
def test_noalloc_matches_decode(torch, mqa, B, Hq, Hkv, L, D, lengths):
    _say(f"mqa_decode_noalloc B{B} Hq{Hq} Hkv{Hkv} L{L} D{D}")
    assert mqa.mqa_decode_workspace_size(B, Hq, Hkv, L, D) <= mqa.NOALLOC_SCRATCH_BYTES
    q, kc, vc, sl = decode_inputs(B, Hq, Hkv, L, D, "bf16", seed=31, lengths=lengths)
    dq, dk, dv, dsl = _dev(torch, q), _dev(torch, kc), _dev(torch, vc), torch.from_numpy(sl).cuda()
    ref_out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    ref_lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    mqa.mqa_decode(dq, dk, dv, dsl, out=ref_out, lse=ref_lse)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    assert _noalloc(torch, mqa, dq, dk, dv, dsl, out, lse, D) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(lse, ref_lse)
    # and through the Python binding of the same name
    out2 = torch.empty_like(out)
    mqa.mqa_decode_noalloc(dq, dk, dv, dsl, out=out2)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref_out)
    if B <= 8:
        ref, rl = oracle.decode_ref(q.f32(), kc.f32(), vc.f32(), sl, 1 / math.sqrt(D))
        assert float(np.max(np.abs(out.float().cpu().numpy() - ref))) <= BF16_TOL
        assert float(np.max(np.abs(lse.cpu().numpy() - rl))) <= BF16_TOL


def test_noalloc_rejects_calls_beyond_the_scratch(torch, mqa):
    """MQA decode at batch 2048 x 16 heads, d 512, cache 4096 needs 64.25 MiB
    of partials: more than the 64 MiB scratch, so the call is refused before
    anything is enqueued and the output keeps its contents."""
    _say("mqa_decode_noalloc oversized call")
    B, Hq, Hkv, L, D = 2048, 16, 1, 4096, 512
    assert mqa.mqa_decode_workspace_size(B, Hq, Hkv, L, D) > mqa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")   # never read: the call is refused
    sl = torch.ones((B,), dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = mqa.lib.mqa_decode_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), sl.data_ptr(), out.data_ptr(), None,
                                    B, Hq, Hkv, L, D, 0.044, mqa.DTYPE_BF16, mqa.DTYPE_BF16, ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    assert st == -3
    assert bool((out.float() == 7.0).all())
