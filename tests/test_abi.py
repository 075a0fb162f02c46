"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments on the host (before any HIP
call) with the documented status codes."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa_attn.h")

mqa = pytest.importorskip("attention_mqa_gqa_amd")
lib = mqa.lib

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
F32, BF16, F16 = 0, 1, 2
P = ctypes.c_void_p(4096)          # a 16-byte aligned stand-in: never dereferenced on these paths
MIS = ctypes.c_void_p(4096 + 8)    # misaligned


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_functions_are_exported():
    names = _declared_functions()
    assert len(names) == 17, names
    assert sorted(names) == sorted(mqa.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert lib.mqa_attn_abi_version() == 3
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, 7):
        assert lib.mqa_status_string(s)
    assert lib.mqa_last_hip_error_name() == b"hipSuccess"


def _prefill(q=P, k=P, v=P, out=P, lse=None, B=1, Hq=16, Hkv=1, T=128, D=512, scale=0.05, causal=1,
             din=BF16, dout=BF16, ws=P, wsb=1 << 40):
    return lib.mqa_prefill(q, k, v, out, lse, B, Hq, Hkv, T, D, scale, causal, din, dout, ws, wsb, None)


def test_prefill_rejections():
    assert _prefill(Hkv=3) == INVALID                    # Hq % Hkv
    assert _prefill(B=-1) == INVALID
    assert _prefill(T=-5) == INVALID
    assert _prefill(Hq=0) == INVALID
    assert _prefill(scale=float("inf")) == INVALID
    assert _prefill(scale=float("nan")) == INVALID
    assert _prefill(scale=0.0) == INVALID                # softmax scale must be > 0
    assert _prefill(scale=-0.05) == INVALID
    assert _prefill(din=7) == INVALID
    assert _prefill(q=None) == INVALID
    assert _prefill(out=MIS) == INVALID
    assert _prefill(lse=ctypes.c_void_p(4098)) == INVALID
    assert _prefill(D=256) == UNSUPPORTED                # bf16: D in {128, 512}
    assert _prefill(D=512, Hq=256, Hkv=1) == UNSUPPORTED  # group larger than a workgroup's rows
    assert _prefill(din=F32, dout=BF16) == UNSUPPORTED
    assert _prefill(din=BF16, dout=F16) == UNSUPPORTED     # 16-bit out = the input type
    assert _prefill(din=F16, dout=BF16) == UNSUPPORTED
    assert _prefill(din=3) == INVALID
    assert _prefill(din=F32, dout=F32, D=100) == UNSUPPORTED
    assert _prefill(ws=None, wsb=0) == WORKSPACE
    need = lib.mqa_prefill_workspace_size(1, 16, 1, 128, 512, BF16)
    assert _prefill(wsb=need - 1) == WORKSPACE
    assert _prefill(ws=MIS, wsb=need) == INVALID


def test_prefill_empty_calls_are_ok():
    assert _prefill(B=0, q=None, k=None, v=None, out=None) == OK
    assert _prefill(T=0, q=None, k=None, v=None, out=None) == OK


def test_f16_is_accepted_where_supported():
    # validation passes up to the workspace check (no HIP call is made)
    assert _prefill(din=F16, dout=F16, ws=None, wsb=0) == WORKSPACE
    assert _prefill(din=F16, dout=F32, ws=None, wsb=0) == WORKSPACE
    assert _decode(dt=F16, dout=F16, ws=None) == WORKSPACE
    assert lib.mqa_prefill_workspace_size(2, 16, 1, 4096, 512, F16) == lib.mqa_prefill_workspace_size(
        2, 16, 1, 4096, 512, BF16)


def test_prefill_workspace_size():
    # bf16: a transposed V as whole 32-key tiles, and at d = 512 the K tile
    # too (each 1 KB K row carrying 16 bytes of padding); narrower K rows are
    # copied from K itself
    assert lib.mqa_prefill_workspace_size(2, 16, 1, 4096, 512, BF16) == 2 * 1 * 4096 * (1040 + 1024)
    assert lib.mqa_prefill_workspace_size(1, 8, 2, 33, 128, BF16) == 1 * 2 * 64 * 128 * 2
    assert lib.mqa_prefill_workspace_size(1, 16, 1, 128, 512, F32) == 0


def _prefill_ex(q=P, k=P, v=P, out=P, lse=None, B=1, Hq=128, Hkv=128, Tq=64, Tkv=256, DK=192, DV=128,
                scale=0.072, causal=1, din=BF16, dout=BF16, ws=P, wsb=1 << 40):
    return lib.mqa_prefill_ex(q, k, v, out, lse, B, Hq, Hkv, Tq, Tkv, DK, DV, scale, causal, din, dout, ws, wsb,
                              None)


def test_prefill_ex_rejections():
    assert _prefill_ex(Tq=300, Tkv=256) == INVALID         # causal: a query would see no key
    assert _prefill_ex(Tq=64, Tkv=0) == INVALID            # causal and non-causal: no keys
    assert _prefill_ex(Tq=64, Tkv=0, causal=0) == INVALID
    assert _prefill_ex(Tq=-1) == INVALID
    assert _prefill_ex(DV=0) == INVALID
    assert _prefill_ex(Hkv=3) == INVALID
    assert _prefill_ex(scale=0.0) == INVALID
    assert _prefill_ex(DK=192, DV=192) == UNSUPPORTED       # bf16 width pairs: 128/128, 512/512, 192/128
    assert _prefill_ex(DK=128, DV=192) == UNSUPPORTED
    assert _prefill_ex(DK=512, DV=128) == UNSUPPORTED
    assert _prefill_ex(din=F32, dout=F32, DK=256, DV=128) == UNSUPPORTED
    assert _prefill_ex(Hq=512, Hkv=1) == UNSUPPORTED        # group larger than a workgroup's rows
    # fp32: T_q x G rows in blocks of 16 must fit the grid (2^35 rows)
    big = 2 ** 31 - 1
    assert _prefill_ex(din=F32, dout=F32, Hq=64, Hkv=1, Tq=big, Tkv=big, causal=0, ws=None, wsb=0) == UNSUPPORTED
    assert _prefill_ex(ws=None, wsb=0) == WORKSPACE
    need = lib.mqa_prefill_ex_workspace_size(1, 128, 128, 64, 256, 192, 128, BF16)
    assert _prefill_ex(wsb=need - 1) == WORKSPACE


def test_prefill_ex_empty_and_noncausal_shapes():
    assert _prefill_ex(Tq=0, q=None, k=None, v=None, out=None) == OK
    assert _prefill_ex(B=0, q=None, k=None, v=None, out=None) == OK
    assert _prefill_ex(Tq=0, Tkv=0, q=None, k=None, v=None, out=None) == OK


def test_prefill_ex_workspace_size():
    # transposed V tile (d_v) per 32 keys of T_kv (plus the padded K tile at 512)
    assert lib.mqa_prefill_ex_workspace_size(1, 128, 128, 100, 8192, 192, 128, BF16) == 128 * 8192 * 128 * 2
    assert lib.mqa_prefill_ex_workspace_size(2, 16, 1, 7, 33, 512, 512, BF16) == 2 * 1 * 64 * (1040 + 1024)
    assert lib.mqa_prefill_ex_workspace_size(1, 128, 128, 100, 8192, 192, 128, F32) == 0
    # the square entry point is the general one with T_q = T_kv, d_v = d_qk
    for args in ((2, 16, 1, 4096, 512), (1, 8, 2, 33, 128)):
        B, Hq, Hkv, T, D = args
        assert lib.mqa_prefill_workspace_size(B, Hq, Hkv, T, D, BF16) == \
            lib.mqa_prefill_ex_workspace_size(B, Hq, Hkv, T, T, D, D, BF16)


def _decode(q=P, k=P, v=P, sl=P, out=P, lse=None, B=64, Hq=16, Hkv=1, L=8192, D=512, scale=0.05,
            dt=BF16, dout=BF16, ws=P, wsb=1 << 40):
    return lib.mqa_decode(q, k, v, sl, out, lse, B, Hq, Hkv, L, D, scale, dt, dout, ws, wsb, None)


def test_decode_rejections():
    assert _decode(Hkv=3) == INVALID
    assert _decode(sl=None) == INVALID
    assert _decode(sl=ctypes.c_void_p(4098)) == INVALID
    assert _decode(L=0) == INVALID
    assert _decode(scale=0.0) == INVALID
    assert _decode(dt=F32, dout=F32) == UNSUPPORTED
    assert _decode(dt=F16, dout=BF16) == UNSUPPORTED
    assert _decode(D=256) == UNSUPPORTED
    assert _decode(Hq=64, Hkv=2) == UNSUPPORTED          # group of 32 > 16 MFMA columns
    assert _decode(ws=None) == WORKSPACE
    need = lib.mqa_decode_workspace_size(64, 16, 1, 8192, 512)
    assert need > 0
    assert _decode(wsb=need - 4) == WORKSPACE
    assert _decode(B=0, q=None) == OK


def _mla(q=P, kv=P, sl=P, out=P, lse=None, B=32, H=128, L=32768, scale=0.072, dt=BF16, dout=BF16,
         ws=P, wsb=1 << 40):
    return lib.mla_decode_absorbed(q, kv, sl, out, lse, B, H, L, scale, dt, dout, ws, wsb, None)


def test_mla_rejections():
    assert _mla(H=0) == INVALID
    assert _mla(kv=MIS) == INVALID
    assert _mla(scale=-1.0) == INVALID
    assert _mla(H=24) == UNSUPPORTED
    assert _mla(H=256) == UNSUPPORTED
    assert _mla(dt=F32) == UNSUPPORTED
    assert _mla(dt=F16, dout=F16, ws=None) == WORKSPACE   # fp16 accepted (validation only)
    assert _mla(dt=F16, dout=F32, ws=None) == WORKSPACE
    assert _mla(dt=BF16, dout=F16) == UNSUPPORTED          # 16-bit out = the input type
    assert _mla(dt=F16, dout=BF16) == UNSUPPORTED
    assert _mla(ws=None) == WORKSPACE
    need = lib.mla_decode_workspace_size(32, 128, 32768)
    assert _mla(wsb=need - 1) == WORKSPACE
    assert _mla(B=0, q=None) == OK


def _sparse(q=P, kv=P, idx=P, out=P, lse=None, B=32, H=128, L=32768, k=2048, scale=0.072, dt=BF16, dout=BF16,
            ws=P, wsb=1 << 40):
    return lib.mla_decode_sparse(q, kv, idx, out, lse, B, H, L, k, scale, dt, dout, ws, wsb, None)


def test_mla_sparse_rejections():
    assert _sparse(k=0) == INVALID
    assert _sparse(L=0) == INVALID
    assert _sparse(idx=None) == INVALID
    assert _sparse(idx=ctypes.c_void_p(4098)) == INVALID
    assert _sparse(scale=float("nan")) == INVALID
    assert _sparse(H=24) == UNSUPPORTED
    assert _sparse(dt=F32) == UNSUPPORTED
    assert _sparse(dt=F16, dout=F16, ws=None) == WORKSPACE
    assert _sparse(dt=BF16, dout=F16) == UNSUPPORTED
    assert _sparse(ws=None) == WORKSPACE
    need = lib.mla_decode_sparse_workspace_size(32, 128, 2048)
    assert need > 0 and need % (32 * 128 * (512 + 2) * 4) == 0
    assert _sparse(wsb=need - 1) == WORKSPACE
    assert _sparse(B=0, q=None) == OK


def test_mla_step_rejections():
    ab = lambda **k: lib.mla_absorb_query(k.get("qn", P), k.get("qr", P), k.get("w", P), k.get("c", P),
                                          k.get("s", P), k.get("o", P), k.get("B", 4), k.get("H", 128),
                                          k.get("dt", BF16), None)
    assert ab(H=0) == INVALID
    assert ab(w=None) == INVALID
    assert ab(c=ctypes.c_void_p(4098)) == INVALID
    assert ab(o=MIS) == INVALID
    assert ab(dt=F32) == UNSUPPORTED                       # 16-bit only (bf16, fp16)
    assert ab(B=0, qn=None) == OK
    ap = lambda **k: lib.mla_cache_append(k.get("c", P), k.get("k", P), P, P, k.get("pos", P), k.get("kv", P),
                                          k.get("B", 4), k.get("L", 100), k.get("dt", BF16), None)
    assert ap(L=0) == INVALID
    assert ap(pos=None) == INVALID
    assert ap(kv=MIS) == INVALID
    assert ap(dt=F32) == UNSUPPORTED
    assert ap(B=0, c=None) == OK
    op = lambda **k: lib.mla_output_project(k.get("o", P), k.get("w", P), k.get("out", P), k.get("B", 4),
                                            k.get("H", 128), k.get("dt", BF16), k.get("dout", BF16), None)
    assert op(H=-1) == INVALID
    assert op(out=None) == INVALID
    assert op(dt=BF16, dout=F16) == UNSUPPORTED
    assert op(dt=F16, dout=BF16) == UNSUPPORTED
    assert op(dt=F32, dout=F32) == UNSUPPORTED
    assert op(B=0, o=None) == OK


def test_decode_workspace_grows_with_splits():
    a = lib.mqa_decode_workspace_size(64, 16, 1, 8192, 512)
    b = lib.mqa_decode_workspace_size(64, 16, 1, 32768, 512)
    assert b >= a > 0
    # partials: (D + 2) floats per (sequence, head, split)
    assert a % (64 * 16 * (512 + 2) * 4) == 0


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="forces a launch failure: only on a host without a GPU")
def test_launch_failure_is_reported_as_hip_error():
    """Valid arguments on a host with no GPU: validation passes, the kernel
    launch fails in the HIP runtime, and the call returns MQA_ERR_HIP with
    the runtime's error name (the library never aborts).  A later call that
    fails validation returns its own status and leaves the HIP error name as
    it was."""
    need = lib.mqa_prefill_workspace_size(1, 16, 1, 128, 512, BF16)
    assert _prefill(wsb=need) == -4
    assert lib.mqa_last_hip_error_name() not in (b"hipSuccess", b"")
    dws = lib.mqa_decode_workspace_size(2, 16, 1, 64, 512)
    assert lib.mqa_decode(P, P, P, P, P, None, 2, 16, 1, 64, 512, 0.05, BF16, BF16, P, dws, None) == -4
    assert lib.mqa_decode_noalloc(P, P, P, P, P, None, 2, 16, 1, 64, 512, 0.05, BF16, BF16, None) == -4
    mws = lib.mla_decode_workspace_size(2, 16, 64)
    assert lib.mla_decode_absorbed(P, P, P, P, None, 2, 16, 64, 0.07, BF16, BF16, P, mws, None) == -4
    name = lib.mqa_last_hip_error_name()
    assert _prefill(Hkv=3) == INVALID
    assert lib.mqa_last_hip_error_name() == name


PEAKS_HEADER = os.path.join(ROOT, "include", "mqa_peaks.h")


def test_peaks_header_functions_are_exported():
    """libmqa_peaks.so (the attainable-peak probes) exports what its header
    declares, and rejects bad arguments before any launch."""
    from attention_mqa_gqa_amd import peaks
    text = re.sub(r"/\*.*?\*/", "", open(PEAKS_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, flags=re.M)))
    assert names == sorted(peaks.EXPORTED_SYMBOLS)
    pl = peaks.load()
    for n in names:
        assert hasattr(pl, n), n
    assert pl.mqa_peak_mfma_bf16(3, 10, P, P, None) == -1
    assert pl.mqa_peak_mfma_bf16(1, 0, P, P, None) == -1
    assert pl.mqa_peak_hbm_read(MIS, 1 << 20, P, None) == -1
    assert pl.mqa_peak_hbm_copy(P, MIS, 1 << 20, None) == -1
    assert pl.mqa_peak_lds_read(17, 10, P, None) == -1


def test_decode_noalloc_rejections():
    """The allocation-free decode validates like mqa_decode, and refuses a
    call whose partials exceed its fixed scratch before touching the device."""
    f = lib.mqa_decode_noalloc
    assert f(P, P, P, P, P, None, 2, 16, 3, 64, 512, 0.05, BF16, BF16, None) == INVALID
    assert f(P, P, P, None, P, None, 2, 16, 1, 64, 512, 0.05, BF16, BF16, None) == INVALID
    assert f(P, P, P, P, MIS, None, 2, 16, 1, 64, 512, 0.05, BF16, BF16, None) == INVALID
    assert f(P, P, P, P, P, None, 2, 64, 1, 64, 128, 0.05, BF16, BF16, None) == UNSUPPORTED
    assert f(None, None, None, None, None, None, 0, 16, 1, 64, 512, 0.05, BF16, BF16, None) == OK
    assert lib.mqa_decode_workspace_size(2048, 16, 1, 4096, 512) > mqa.NOALLOC_SCRATCH_BYTES
    assert f(P, P, P, P, P, None, 2048, 16, 1, 4096, 512, 0.05, BF16, BF16, None) == WORKSPACE
    assert lib.mqa_decode_workspace_size(64, 16, 1, 65536, 512) <= mqa.NOALLOC_SCRATCH_BYTES
