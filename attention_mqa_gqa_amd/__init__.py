"""Python binding of libmqa_attn.so (MQA / GQA / MLA-absorbed attention on
MI355X).  Argument marshalling only: every step of the computation runs in
the library's HIP kernels.  PyTorch provides device memory and the stream.

The entry points carry the C ABI's names (see ``include/mqa_attn.h``):

* :func:`mqa_prefill`          -- causal or full attention over a sequence;
* :func:`mqa_prefill_ex`       -- the same with T_q != T_kv (bottom-right
  causal) and d_v != d_qk (expanded MLA prefill);
* :func:`mqa_decode`           -- one query token per sequence vs a KV cache;
* :func:`mqa_decode_noalloc`   -- the same without workspace or allocation
  (fixed per-device scratch), for callers that cannot allocate;
* :func:`mla_decode_absorbed`  -- absorbed MLA decode over a latent cache;
* :func:`mla_decode_sparse`    -- the same over selected (top-k) cache rows;
* :func:`mla_absorb_query`, :func:`mla_cache_append`,
  :func:`mla_output_project`   -- the steps either side of the absorbed
  decode (query absorption + RoPE, cache append + RoPE, W_UV).

The library must be built (``python attention_mqa_gqa_amd/build.py``); if it
is missing or cannot be loaded, importing the bindings raises.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LIB_PATH",
    "MqaError",
    "lib",
    "mqa_prefill",
    "mqa_prefill_workspace_size",
    "mqa_prefill_ex",
    "mqa_prefill_ex_workspace_size",
    "mqa_decode",
    "mqa_decode_noalloc",
    "mqa_decode_workspace_size",
    "NOALLOC_SCRATCH_BYTES",
    "mla_decode_absorbed",
    "mla_decode_workspace_size",
    "mla_decode_sparse",
    "mla_decode_sparse_workspace_size",
    "mla_absorb_query",
    "mla_cache_append",
    "mla_output_project",
    "DTYPE_F32",
    "DTYPE_BF16",
    "DTYPE_F16",
    "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmqa_attn.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2

# MQA_DECODE_NOALLOC_SCRATCH_BYTES: the fixed device scratch of mqa_decode_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED_SYMBOLS = (
    "mqa_attn_abi_version",
    "mqa_status_string",
    "mqa_last_hip_error_name",
    "mqa_prefill_workspace_size",
    "mqa_prefill",
    "mqa_prefill_ex_workspace_size",
    "mqa_prefill_ex",
    "mqa_decode_workspace_size",
    "mqa_decode",
    "mqa_decode_noalloc",
    "mla_decode_workspace_size",
    "mla_decode_absorbed",
    "mla_decode_sparse_workspace_size",
    "mla_decode_sparse",
    "mla_absorb_query",
    "mla_cache_append",
    "mla_output_project",
)


class MqaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        detail = ""
        if status == -4:
            detail = f", {lib.mqa_last_hip_error_name().decode()}"
        super().__init__(f"{what}: status {status} ({_status_string(status)}{detail})")


def _load():
    # torch ships its own HIP runtime (soname libamdhip64.so.7).  Load it first
    # so the library binds to that same runtime: with two runtimes in one
    # process ours would not see the device, and torch's stream handles would
    # not belong to the runtime we launch on.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python attention_mqa_gqa_amd/build.py`")
    l = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    l.mqa_attn_abi_version.restype = i
    l.mqa_attn_abi_version.argtypes = []
    l.mqa_status_string.restype = ctypes.c_char_p
    l.mqa_status_string.argtypes = [i]
    l.mqa_last_hip_error_name.restype = ctypes.c_char_p
    l.mqa_last_hip_error_name.argtypes = []
    l.mqa_prefill_workspace_size.restype = sz
    l.mqa_prefill_workspace_size.argtypes = [i, i, i, i, i, i]
    l.mqa_prefill.restype = i
    l.mqa_prefill.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    l.mqa_prefill_ex_workspace_size.restype = sz
    l.mqa_prefill_ex_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    l.mqa_prefill_ex.restype = i
    l.mqa_prefill_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    l.mqa_decode_workspace_size.restype = sz
    l.mqa_decode_workspace_size.argtypes = [i, i, i, i, i]
    l.mqa_decode.restype = i
    l.mqa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    l.mqa_decode_noalloc.restype = i
    l.mqa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    l.mla_decode_workspace_size.restype = sz
    l.mla_decode_workspace_size.argtypes = [i, i, i]
    l.mla_decode_absorbed.restype = i
    l.mla_decode_absorbed.argtypes = [vp, vp, vp, vp, vp, i, i, i, f, i, i, vp, sz, vp]
    l.mla_decode_sparse_workspace_size.restype = sz
    l.mla_decode_sparse_workspace_size.argtypes = [i, i, i]
    l.mla_decode_sparse.restype = i
    l.mla_decode_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp]
    l.mla_absorb_query.restype = i
    l.mla_absorb_query.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, vp]
    l.mla_cache_append.restype = i
    l.mla_cache_append.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, vp]
    l.mla_output_project.restype = i
    l.mla_output_project.argtypes = [vp, vp, vp, i, i, i, i, vp]
    return l


lib = _load()


def _current_raw_stream_public(index):
    import torch
    return torch.cuda.current_stream(index).cuda_stream


def _pick_raw_stream_getter():
    # torch's raw current-stream query (no Stream object per call) when this
    # torch build has it, else the public route
    import torch
    return getattr(torch._C, "_cuda_getCurrentRawStream", None) or _current_raw_stream_public


_current_raw_stream = _pick_raw_stream_getter()


def _status_string(status):
    return lib.mqa_status_string(int(status)).decode()


def _check(status, what):
    if status != 0:
        raise MqaError(status, what)


def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32:
        return DTYPE_F32
    if dt == torch.bfloat16:
        return DTYPE_BF16
    if dt == torch.float16:
        return DTYPE_F16
    raise TypeError(f"unsupported dtype {dt}; use torch.float32, torch.bfloat16 or torch.float16")


def _ptr(t):
    # a plain int: the argtypes declare c_void_p, so ctypes converts it
    return None if t is None else t.data_ptr()


def _stream_ptr(stream, device):
    if stream is not None:
        return stream.cuda_stream
    # the current stream's handle without building a torch Stream object
    # (that costs about 2 us of host time per call)
    return _current_raw_stream(device.index)


def _same_dtype(what, *tensors):
    if any(t.dtype != tensors[0].dtype for t in tensors[1:]):
        raise TypeError(f"{what} must share a dtype")


def _require(t, name, ndim):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _require_on(t, name, device):
    # the library reads every pointer of one call on one device
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")


def _check_out(out, shape, device):
    """Caller-supplied output: contiguous, on the inputs' device, exactly `shape`."""
    _require(out, "out", len(shape))
    _require_on(out, "out", device)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must be {tuple(shape)}, got {tuple(out.shape)}")


def _check_lse(lse, shape, device):
    """Optional log-sum-exp output: float32, contiguous, on the device, exactly `shape`."""
    if lse is None:
        return
    torch = _torch()
    _require(lse, "lse", len(shape))
    _require_on(lse, "lse", device)
    if lse.dtype != torch.float32:
        raise TypeError(f"lse must be float32, got {lse.dtype}")
    if tuple(lse.shape) != tuple(shape):
        raise ValueError(f"lse must be {tuple(shape)}, got {tuple(lse.shape)}")


def _check_index(t, name, shape, device):
    torch = _torch()
    _require(t, name, len(shape))
    _require_on(t, name, device)
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def mqa_prefill_workspace_size(B, Hq, Hkv, T, head_dim, in_dtype):
    return int(lib.mqa_prefill_workspace_size(B, Hq, Hkv, T, head_dim, in_dtype))


def mqa_prefill_ex_workspace_size(B, Hq, Hkv, T_q, T_kv, d_qk, d_v, in_dtype):
    return int(lib.mqa_prefill_ex_workspace_size(B, Hq, Hkv, T_q, T_kv, d_qk, d_v, in_dtype))


def mqa_decode_workspace_size(B, Hq, Hkv, max_len, head_dim):
    return int(lib.mqa_decode_workspace_size(B, Hq, Hkv, max_len, head_dim))


def mla_decode_workspace_size(B, H, max_len):
    return int(lib.mla_decode_workspace_size(B, H, max_len))


def mla_decode_sparse_workspace_size(B, H, topk):
    return int(lib.mla_decode_sparse_workspace_size(B, H, topk))


def _workspace(nbytes, device, workspace):
    """A caller-supplied workspace must be a contiguous tensor on `device`;
    its size is checked by the library (MQA_ERR_WORKSPACE if too small)."""
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    else:
        if not workspace.is_cuda or workspace.device != device:
            raise ValueError(f"workspace must be on {device}, got {workspace.device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
    return workspace, workspace.numel() * workspace.element_size()


def mqa_prefill(q, k, v, causal=True, scale=None, out=None, out_dtype=None, lse=None,
                workspace=None, stream=None):
    """q [B,Hq,T,D], k/v [B,Hkv,T,D] -> out [B,Hq,T,D] (and lse [B,Hq,T] if given)."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, nm, 4)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, T, D] matching q")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share a dtype")
    for t, nm in ((k, "k"), (v, "v")):
        _require_on(t, nm, q.device)
    in_code = _dtype_code(q.dtype)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Hq, T, D), dtype=out_dtype, device=q.device)
    _check_out(out, (B, Hq, T, D), q.device)
    _check_lse(lse, (B, Hq, T), q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = mqa_prefill_workspace_size(B, Hq, Hkv, T, D, in_code)
    ws, wsb = _workspace(nbytes, q.device, workspace)
    st = lib.mqa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, T, D, scale,
                         1 if causal else 0, in_code, _dtype_code(out.dtype), _ptr(ws), wsb,
                         _stream_ptr(stream, q.device))
    _check(st, "mqa_prefill")
    return out


def mqa_prefill_ex(q, k, v, causal=True, scale=None, out=None, out_dtype=None, lse=None,
                   workspace=None, stream=None):
    """q [B,Hq,T_q,d_qk], k [B,Hkv,T_kv,d_qk], v [B,Hkv,T_kv,d_v] ->
    out [B,Hq,T_q,d_v] (and lse [B,Hq,T_q] if given).  causal: the queries
    are the last T_q of the T_kv tokens.  Default scale 1/sqrt(d_qk)."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, nm, 4)
    B, Hq, T_q, DK = q.shape
    Hkv, T_kv = k.shape[1], k.shape[2]
    DV = v.shape[3]
    if k.shape != (B, Hkv, T_kv, DK) or v.shape != (B, Hkv, T_kv, DV):
        raise ValueError("k must be [B, Hkv, T_kv, d_qk] and v [B, Hkv, T_kv, d_v]")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share a dtype")
    for t, nm in ((k, "k"), (v, "v")):
        _require_on(t, nm, q.device)
    in_code = _dtype_code(q.dtype)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Hq, T_q, DV), dtype=out_dtype, device=q.device)
    _check_out(out, (B, Hq, T_q, DV), q.device)
    _check_lse(lse, (B, Hq, T_q), q.device)
    scale = 1.0 / math.sqrt(DK) if scale is None else float(scale)
    nbytes = mqa_prefill_ex_workspace_size(B, Hq, Hkv, T_q, T_kv, DK, DV, in_code)
    ws, wsb = _workspace(nbytes, q.device, workspace)
    st = lib.mqa_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, T_q, T_kv, DK, DV,
                            scale, 1 if causal else 0, in_code, _dtype_code(out.dtype), _ptr(ws), wsb,
                            _stream_ptr(stream, q.device))
    _check(st, "mqa_prefill_ex")
    return out


def mqa_decode(q, k_cache, v_cache, seq_lens, scale=None, out=None, out_dtype=None, lse=None,
               workspace=None, stream=None):
    """q [B,Hq,D], caches [B,Hkv,L_max,D], seq_lens int32 [B] -> out [B,Hq,D]."""
    torch = _torch()
    _require(q, "q", 3)
    _require(k_cache, "k_cache", 4)
    _require(v_cache, "v_cache", 4)
    _same_dtype("q, k_cache, v_cache", q, k_cache, v_cache)
    B, Hq, D = q.shape
    Hkv, L_max = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, Hkv, L_max, D) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, L_max, D] matching q")
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _require_on(t, nm, q.device)
    _check_index(seq_lens, "seq_lens", (B,), q.device)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _check_out(out, (B, Hq, D), q.device)
    _check_lse(lse, (B, Hq), q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = mqa_decode_workspace_size(B, Hq, Hkv, L_max, D)
    ws, wsb = _workspace(nbytes, q.device, workspace)
    st = lib.mqa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out), _ptr(lse),
                        B, Hq, Hkv, L_max, D, scale, _dtype_code(q.dtype), _dtype_code(out.dtype),
                        _ptr(ws), wsb, _stream_ptr(stream, q.device))
    _check(st, "mqa_decode")
    return out


def mqa_decode_noalloc(q, k_cache, v_cache, seq_lens, out, scale=None, lse=None, stream=None):
    """mqa_decode without a workspace and without allocating: the caller
    passes `out` (and optionally `lse`); the split partials go to the
    library's fixed per-device scratch (NOALLOC_SCRATCH_BYTES).  Raises
    MqaError (status -3) when the call needs more scratch than that.  Calls
    that may run concurrently on one device share the scratch and race."""
    torch = _torch()
    _require(q, "q", 3)
    _require(k_cache, "k_cache", 4)
    _require(v_cache, "v_cache", 4)
    _same_dtype("q, k_cache, v_cache", q, k_cache, v_cache)
    B, Hq, D = q.shape
    Hkv, L_max = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, Hkv, L_max, D) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, L_max, D] matching q")
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _require_on(t, nm, q.device)
    _check_index(seq_lens, "seq_lens", (B,), q.device)
    _check_out(out, (B, Hq, D), q.device)
    _check_lse(lse, (B, Hq), q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.mqa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out), _ptr(lse),
                                B, Hq, Hkv, L_max, D, scale, _dtype_code(q.dtype), _dtype_code(out.dtype),
                                _stream_ptr(stream, q.device))
    _check(st, "mqa_decode_noalloc")
    return out


def mla_decode_absorbed(q_abs, kv_cache, seq_lens, scale=None, out=None, out_dtype=None, lse=None,
                        workspace=None, stream=None):
    """q_abs [B,H,576], kv_cache [B,L_max,576], seq_lens int32 [B] -> out [B,H,512]."""
    torch = _torch()
    _require(q_abs, "q_abs", 3)
    _require(kv_cache, "kv_cache", 3)
    _same_dtype("q_abs, kv_cache", q_abs, kv_cache)
    B, H, DK = q_abs.shape
    if DK != 576 or kv_cache.shape[0] != B or kv_cache.shape[2] != 576:
        raise ValueError("q_abs must be [B,H,576] and kv_cache [B,L_max,576]")
    L_max = kv_cache.shape[1]
    _require_on(kv_cache, "kv_cache", q_abs.device)
    _check_index(seq_lens, "seq_lens", (B,), q_abs.device)
    out_dtype = q_abs.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, 512), dtype=out_dtype, device=q_abs.device)
    _check_out(out, (B, H, 512), q_abs.device)
    _check_lse(lse, (B, H), q_abs.device)
    scale = 1.0 / math.sqrt(192.0) if scale is None else float(scale)
    nbytes = mla_decode_workspace_size(B, H, L_max)
    ws, wsb = _workspace(nbytes, q_abs.device, workspace)
    st = lib.mla_decode_absorbed(_ptr(q_abs), _ptr(kv_cache), _ptr(seq_lens), _ptr(out), _ptr(lse),
                                 B, H, L_max, scale, _dtype_code(q_abs.dtype), _dtype_code(out.dtype),
                                 _ptr(ws), wsb, _stream_ptr(stream, q_abs.device))
    _check(st, "mla_decode_absorbed")
    return out


def mla_decode_sparse(q_abs, kv_cache, indices, scale=None, out=None, out_dtype=None, lse=None,
                      workspace=None, stream=None):
    """q_abs [B,H,576], kv_cache [B,L_max,576], indices int32 [B,topk] (rows to
    attend; entries outside [0, L_max) skipped) -> out [B,H,512]."""
    torch = _torch()
    _require(q_abs, "q_abs", 3)
    _require(kv_cache, "kv_cache", 3)
    _same_dtype("q_abs, kv_cache", q_abs, kv_cache)
    B, H, DK = q_abs.shape
    if DK != 576 or kv_cache.shape[0] != B or kv_cache.shape[2] != 576 or indices.dim() != 2:
        raise ValueError("q_abs must be [B,H,576], kv_cache [B,L_max,576] and indices [B,topk]")
    L_max, topk = kv_cache.shape[1], indices.shape[1]
    _require_on(kv_cache, "kv_cache", q_abs.device)
    _check_index(indices, "indices", (B, topk), q_abs.device)
    out_dtype = q_abs.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, 512), dtype=out_dtype, device=q_abs.device)
    _check_out(out, (B, H, 512), q_abs.device)
    _check_lse(lse, (B, H), q_abs.device)
    scale = 1.0 / math.sqrt(192.0) if scale is None else float(scale)
    nbytes = mla_decode_sparse_workspace_size(B, H, topk)
    ws, wsb = _workspace(nbytes, q_abs.device, workspace)
    st = lib.mla_decode_sparse(_ptr(q_abs), _ptr(kv_cache), _ptr(indices), _ptr(out), _ptr(lse),
                               B, H, L_max, topk, scale, _dtype_code(q_abs.dtype), _dtype_code(out.dtype),
                               _ptr(ws), wsb, _stream_ptr(stream, q_abs.device))
    _check(st, "mla_decode_sparse")
    return out


def _rope_tables(cos, sin, B, torch, device):
    for t, nm in ((cos, "cos"), (sin, "sin")):
        _require(t, nm, 2)
        _require_on(t, nm, device)
        if t.dtype != torch.float32 or t.shape != (B, 64):
            raise ValueError(f"{nm} must be float32 [B, 64]")


def mla_absorb_query(q_nope, q_rope, w_uk, cos, sin, out=None, stream=None):
    """q_nope [B,H,128], q_rope [B,H,64], w_uk [H,512,128], cos/sin fp32 [B,64]
    -> q_abs [B,H,576] = [W_UK[h] q_nope | RoPE(q_rope)]."""
    torch = _torch()
    _require(q_nope, "q_nope", 3)
    _require(q_rope, "q_rope", 3)
    _require(w_uk, "w_uk", 3)
    B, H, _ = q_nope.shape
    if q_nope.shape[2] != 128 or q_rope.shape != (B, H, 64) or w_uk.shape != (H, 512, 128):
        raise ValueError("q_nope [B,H,128], q_rope [B,H,64], w_uk [H,512,128]")
    for t, nm in ((q_rope, "q_rope"), (w_uk, "w_uk")):
        _require_on(t, nm, q_nope.device)
    _rope_tables(cos, sin, B, torch, q_nope.device)
    if out is None:
        out = torch.empty((B, H, 576), dtype=q_nope.dtype, device=q_nope.device)
    _check_out(out, (B, H, 576), q_nope.device)
    _same_dtype("q_nope, q_rope, w_uk, out", q_nope, q_rope, w_uk, out)
    st = lib.mla_absorb_query(_ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(cos), _ptr(sin), _ptr(out), B, H,
                              _dtype_code(q_nope.dtype), _stream_ptr(stream, q_nope.device))
    _check(st, "mla_absorb_query")
    return out


def mla_cache_append(kv_cache, c_kv, k_pe, cos, sin, positions, stream=None):
    """kv_cache [B,L_max,576]: row positions[b] of sequence b <- [c_kv[b] | RoPE(k_pe[b])];
    c_kv [B,512], k_pe [B,64], cos/sin fp32 [B,64], positions int32 [B]."""
    torch = _torch()
    _require(kv_cache, "kv_cache", 3)
    _require(c_kv, "c_kv", 2)
    _require(k_pe, "k_pe", 2)
    B, L_max, _ = kv_cache.shape
    if kv_cache.shape[2] != 576 or c_kv.shape != (B, 512) or k_pe.shape != (B, 64):
        raise ValueError("kv_cache [B,L_max,576], c_kv [B,512], k_pe [B,64], positions [B]")
    _same_dtype("kv_cache, c_kv, k_pe", kv_cache, c_kv, k_pe)
    for t, nm in ((c_kv, "c_kv"), (k_pe, "k_pe")):
        _require_on(t, nm, kv_cache.device)
    _check_index(positions, "positions", (B,), kv_cache.device)
    _rope_tables(cos, sin, B, torch, kv_cache.device)
    st = lib.mla_cache_append(_ptr(c_kv), _ptr(k_pe), _ptr(cos), _ptr(sin), _ptr(positions), _ptr(kv_cache), B,
                              L_max, _dtype_code(kv_cache.dtype), _stream_ptr(stream, kv_cache.device))
    _check(st, "mla_cache_append")
    return kv_cache


def mla_output_project(o_lat, w_uv, out=None, out_dtype=None, stream=None):
    """o_lat [B,H,512], w_uv [H,512,128] -> out [B,H,128] = o_lat[b,h] W_UV[h]."""
    torch = _torch()
    _require(o_lat, "o_lat", 3)
    _require(w_uv, "w_uv", 3)
    B, H, _ = o_lat.shape
    if o_lat.shape[2] != 512 or w_uv.shape != (H, 512, 128):
        raise ValueError("o_lat [B,H,512], w_uv [H,512,128]")
    _same_dtype("o_lat, w_uv", o_lat, w_uv)
    out_dtype = o_lat.dtype if out_dtype is None else out_dtype
    _require_on(w_uv, "w_uv", o_lat.device)
    if out is None:
        out = torch.empty((B, H, 128), dtype=out_dtype, device=o_lat.device)
    _check_out(out, (B, H, 128), o_lat.device)
    st = lib.mla_output_project(_ptr(o_lat), _ptr(w_uv), _ptr(out), B, H, _dtype_code(o_lat.dtype),
                                _dtype_code(out.dtype), _stream_ptr(stream, o_lat.device))
    _check(st, "mla_output_project")
    return out
