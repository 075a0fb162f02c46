"""The Python binding refuses caller-supplied tensors that do not match the
call before anything is launched (the C ABI takes bare pointers and cannot
check sizes): outputs of the wrong shape, LSE buffers of the wrong type,
shape or device, index tensors of the wrong shape, workspaces on the host.
Every case raises ValueError or TypeError; nothing reaches a kernel."""

import pytest

pytestmark = pytest.mark.gpu


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


def _z(torch, shape, dt=None, device="cuda"):
    return torch.zeros(shape, dtype=dt or torch.bfloat16, device=device)


def test_prefill_rejects_bad_out_and_lse(torch, mqa):
    q, k, v = _z(torch, (1, 16, 64, 512)), _z(torch, (1, 1, 64, 512)), _z(torch, (1, 1, 64, 512))
    f32 = torch.float32
    bad = [
        dict(out=_z(torch, (1, 16, 63, 512))),                      # short output
        dict(out=_z(torch, (1, 8, 64, 512))),
        dict(lse=_z(torch, (1, 16, 64))),                           # bf16 lse
        dict(lse=_z(torch, (1, 16, 32), f32)),                      # short lse
        dict(lse=_z(torch, (1, 16, 64), f32, device="cpu")),        # host lse
        dict(workspace=torch.zeros(1 << 22, dtype=torch.uint8)),    # host workspace
    ]
    for kw in bad:
        with pytest.raises((ValueError, TypeError)):
            mqa.mqa_prefill(q, k, v, **kw)
    with pytest.raises((ValueError, TypeError)):
        mqa.mqa_prefill_ex(q, k, v, out=_z(torch, (1, 16, 64, 128)))
    with pytest.raises((ValueError, TypeError)):
        mqa.mqa_prefill_ex(q, k, v, lse=_z(torch, (1, 16, 65), f32))


def test_decode_rejects_bad_buffers(torch, mqa):
    q, kc, vc = _z(torch, (2, 16, 128)), _z(torch, (2, 1, 64, 128)), _z(torch, (2, 1, 64, 128))
    sl = torch.full((2,), 64, dtype=torch.int32, device="cuda")
    f32 = torch.float32
    bad = [
        dict(seq_lens=torch.full((1,), 64, dtype=torch.int32, device="cuda")),   # short seq_lens
        dict(seq_lens=torch.full((2,), 64, dtype=torch.int64, device="cuda")),
        dict(seq_lens=torch.full((2,), 64, dtype=torch.int32)),                  # host seq_lens
        dict(out=_z(torch, (2, 16, 64))),
        dict(lse=_z(torch, (2, 16))),
        dict(lse=_z(torch, (2, 8), f32)),
        dict(workspace=torch.zeros(1 << 20, dtype=torch.uint8)),
    ]
    for kw in bad:
        args = dict(seq_lens=sl)
        args.update(kw)
        s = args.pop("seq_lens")
        with pytest.raises((ValueError, TypeError)):
            mqa.mqa_decode(q, kc, vc, s, **args)


def test_mla_rejects_bad_buffers(torch, mqa):
    q, kv = _z(torch, (2, 16, 576)), _z(torch, (2, 64, 576))
    sl = torch.full((2,), 64, dtype=torch.int32, device="cuda")
    idx = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    f32 = torch.float32
    for kw in (dict(out=_z(torch, (2, 16, 256))), dict(lse=_z(torch, (2, 16))), dict(lse=_z(torch, (1, 16), f32)),
               dict(workspace=torch.zeros(1 << 20, dtype=torch.uint8))):
        with pytest.raises((ValueError, TypeError)):
            mqa.mla_decode_absorbed(q, kv, sl, **kw)
        with pytest.raises((ValueError, TypeError)):
            mqa.mla_decode_sparse(q, kv, idx, **kw)
    with pytest.raises((ValueError, TypeError)):
        mqa.mla_decode_absorbed(q, kv, sl[:1])
    with pytest.raises((ValueError, TypeError)):
        mqa.mla_decode_sparse(q, kv, torch.zeros((1, 8), dtype=torch.int32, device="cuda"))
    with pytest.raises((ValueError, TypeError)):
        mqa.mla_decode_sparse(q, kv, torch.zeros((2, 8), dtype=torch.int32))


def test_mla_step_rejects_bad_buffers(torch, mqa):
    B, H = 2, 16
    f32 = torch.float32
    qn, qr, wuk = _z(torch, (B, H, 128)), _z(torch, (B, H, 64)), _z(torch, (H, 512, 128))
    cs, sn = _z(torch, (B, 64), f32), _z(torch, (B, 64), f32)
    with pytest.raises((ValueError, TypeError)):
        mqa.mla_absorb_query(qn, qr, wuk, cs, sn, out=_z(torch, (B, H, 512)))
    with pytest.raises((ValueError, TypeError)):
        mqa.mla_absorb_query(qn, qr, wuk, cs.cpu(), sn)
    cache = _z(torch, (B, 64, 576))
    with pytest.raises((ValueError, TypeError)):
        mqa.mla_cache_append(cache, _z(torch, (B, 512)), _z(torch, (B, 64)), cs, sn,
                             torch.zeros((B,), dtype=torch.int32))
    with pytest.raises((ValueError, TypeError)):
        mqa.mla_cache_append(cache, _z(torch, (B, 512)), _z(torch, (B, 64)), cs, sn,
                             torch.zeros((B + 1,), dtype=torch.int32, device="cuda"))
    with pytest.raises((ValueError, TypeError)):
        mqa.mla_output_project(_z(torch, (B, H, 512)), _z(torch, (H, 512, 128)), out=_z(torch, (B, H, 64)))
