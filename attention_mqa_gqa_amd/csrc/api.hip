// C ABI of libmqa_attn.so (declared in include/mqa_attn.h).
// Every argument is validated here, on the host, before any HIP call; the
// launchers in the kernel files receive only requests they support.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/mqa_attn.h"
#include "kernels.hpp"
#include "layout.hpp"

namespace {

using mqa::DecodePlan;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(int d) { return d == MQA_DTYPE_F32 || d == MQA_DTYPE_BF16 || d == MQA_DTYPE_F16; }

bool is16(int d) { return d == MQA_DTYPE_BF16 || d == MQA_DTYPE_F16; }

// 16-bit inputs give their own type or fp32; fp32 inputs give fp32
bool valid_out(int in, int out) { return out == MQA_DTYPE_F32 || (is16(in) && out == in); }

thread_local hipError_t g_last_hip_error = hipSuccess;

// HIP keeps the last error of ANY runtime call made on this thread (by any
// library) until someone reads it.  Read and drop such a stale error before
// launching, so that the check after the launch reports only our launches.
void clear_stale_error() { (void)hipGetLastError(); }

int hip_status(hipError_t e) {
    g_last_hip_error = e;
    return e == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

// Prefill widths / group size the kernels cover (bf16: rows per workgroup
// must hold at least one full head group).
bool prefill_supported(int d_qk, int d_v, int G, bool bf) {
    const mqa::PrefillPlan p = mqa::prefill_plan(d_qk, d_v, bf ? 1 : 0);
    return G >= 1 && G <= p.rows_per_wg;
}

size_t decode_ws_bytes(int B, int Hq, int D, const DecodePlan& p) {
    return (size_t)B * Hq * p.n_split * ((size_t)D + 2) * sizeof(float);
}

// Fixed device scratch of mqa_decode_noalloc (its split partials), one copy
// per device, held until the process ends.  In host code `scratch` only
// names the symbol: its device address is looked up once per device with
// hipGetSymbolAddress and kept in scratch_ptr; that pointer, never the
// array's name, is what the kernels receive.
static __device__ __align__(256) char scratch[MQA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call made with that device current).
int current_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = e;
        return MQA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return MQA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            g_last_hip_error = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return MQA_ERR_HIP;
        }
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return MQA_OK;
}

// Validation, plan and launch shared by mqa_decode and mqa_decode_noalloc.
// get_ws(need, &ws, &bytes) is called only once every argument has been
// accepted; it supplies the workspace (the caller's, or the device's fixed
// scratch) or a status that ends the call.
template <typename GetWs>
int decode_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                       float* lse, int B, int Hq, int Hkv, int max_len, int head_dim, float scale, int dtype,
                       int out_dtype, GetWs get_ws, void* stream) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || max_len < 0 || head_dim <= 0) return MQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return MQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return MQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return MQA_ERR_INVALID_ARG;
    if (B == 0) return MQA_OK;
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return MQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        ((uintptr_t)seq_lens & 3u) || (lse && ((uintptr_t)lse & 3u)))
        return MQA_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    if (!is16(dtype) || !valid_out(dtype, out_dtype)) return MQA_ERR_UNSUPPORTED;
    if (head_dim != 128 && head_dim != 512) return MQA_ERR_UNSUPPORTED;
    if (G > 16) return MQA_ERR_UNSUPPORTED;
    if (max_len == 0) return MQA_ERR_INVALID_ARG;  // a cache with no rows cannot hold the current token
    const DecodePlan plan = mqa::decode_plan(B, Hkv, max_len, head_dim);
    const size_t need = decode_ws_bytes(B, Hq, head_dim, plan);
    void* workspace = nullptr;
    size_t workspace_bytes = 0;
    const int st = get_ws(need, &workspace, &workspace_bytes);
    if (st != MQA_OK) return st;
    if (!workspace || workspace_bytes < need) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_INVALID_ARG;
    mqa::DecodeArgs a;
    a.q = q; a.k = k_cache; a.v = v_cache; a.seq_lens = seq_lens; a.out = out; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.max_len = max_len; a.D = head_dim; a.G = G;
    a.scale = scale; a.f16 = dtype == MQA_DTYPE_F16; a.out_f32 = out_dtype == MQA_DTYPE_F32;
    a.part_o = (float*)workspace;
    a.part_ml = (float*)workspace + (size_t)B * Hq * plan.n_split * head_dim;
    a.plan = plan; a.stream = (hipStream_t)stream;
    clear_stale_error();
    return hip_status(mqa::decode_launch(a));
}

}  // namespace

extern "C" {

int mqa_attn_abi_version(void) { return MQA_ATTN_ABI_VERSION; }

const char* mqa_last_hip_error_name(void) { return hipGetErrorName(g_last_hip_error); }

const char* mqa_status_string(int status) {
    switch (status) {
        case MQA_OK: return "ok";
        case MQA_ERR_INVALID_ARG: return "invalid argument";
        case MQA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case MQA_ERR_WORKSPACE: return "workspace missing or too small";
        case MQA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

size_t mqa_prefill_ex_workspace_size(int B, int Hq, int Hkv, int T_q, int T_kv, int d_qk, int d_v, int in_dtype) {
    (void)Hq;
    (void)T_q;
    if (!is16(in_dtype) || B <= 0 || Hkv <= 0 || T_kv <= 0 || d_qk <= 0 || d_v <= 0) return 0;
    const mqa::PrefillPlan p = mqa::prefill_plan(d_qk, d_v, 1);
    if (p.kt <= 0) return 0;
    const size_t tiles = ((size_t)T_kv + p.kt - 1) / p.kt;
    // V^T tile, 16-bit elements, and at d_qk = 512 the padded K tile
    // (narrower K rows are copied from K itself)
    const size_t k_tile = d_qk == 512 ? (size_t)mqa::layout::prefill_k_tile_bytes(p.kt, d_qk) : 0;
    return (size_t)B * Hkv * tiles * (k_tile + (size_t)p.kt * d_v * 2);
}

size_t mqa_prefill_workspace_size(int B, int Hq, int Hkv, int T, int head_dim, int in_dtype) {
    return mqa_prefill_ex_workspace_size(B, Hq, Hkv, T, T, head_dim, head_dim, in_dtype);
}

int mqa_prefill_ex(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                   int T_q, int T_kv, int d_qk, int d_v, float scale, int causal, int in_dtype, int out_dtype,
                   void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || T_q < 0 || T_kv < 0 || d_qk <= 0 || d_v <= 0) return MQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return MQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return MQA_ERR_INVALID_ARG;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return MQA_ERR_INVALID_ARG;
    // causal queries are the last T_q of T_kv tokens: more queries than keys
    // would leave a query with no visible key
    if (causal && T_q > T_kv) return MQA_ERR_INVALID_ARG;
    if (B == 0 || T_q == 0) return MQA_OK;
    if (T_kv == 0) return MQA_ERR_INVALID_ARG;   // queries with no key at all
    if (!q || !k || !v || !out) return MQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (lse && ((uintptr_t)lse & 3u)))
        return MQA_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    const bool bf = is16(in_dtype);
    if (!valid_out(in_dtype, out_dtype)) return MQA_ERR_UNSUPPORTED;
    if (!prefill_supported(d_qk, d_v, G, bf)) return MQA_ERR_UNSUPPORTED;
    // the bf16 kernels address one (batch, KV head) tile stream with 32-bit
    // byte offsets
    if (bf && ((size_t)T_kv + 31) * ((size_t)d_qk + d_v) * 2 > 0xFFFFFFFFull) return MQA_ERR_UNSUPPORTED;
    // the fp32 kernel deals the T_q x G rows of a (batch, KV head) in blocks
    // of 16 over the grid's x dimension
    if (!bf && ((long long)T_q * G + 15) / 16 > 0x7FFFFFFFLL) return MQA_ERR_UNSUPPORTED;
    const size_t need = mqa_prefill_ex_workspace_size(B, Hq, Hkv, T_q, T_kv, d_qk, d_v, in_dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return MQA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return MQA_ERR_INVALID_ARG;
    }
    mqa::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = T_q; a.Tkv = T_kv; a.DK = d_qk; a.DV = d_v; a.G = G;
    a.scale = scale; a.causal = causal != 0; a.in16 = bf; a.f16 = in_dtype == MQA_DTYPE_F16;
    a.out_f32 = out_dtype == MQA_DTYPE_F32;
    a.workspace = workspace; a.stream = (hipStream_t)stream;
    clear_stale_error();
    return hip_status(mqa::prefill_launch(a));
}

int mqa_prefill(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int T,
                int head_dim, float scale, int causal, int in_dtype, int out_dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
    return mqa_prefill_ex(q, k, v, out, lse, B, Hq, Hkv, T, T, head_dim, head_dim, scale, causal, in_dtype,
                          out_dtype, workspace, workspace_bytes, stream);
}

size_t mqa_decode_workspace_size(int B, int Hq, int Hkv, int max_len, int head_dim) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_len <= 0 || head_dim <= 0) return 0;
    return decode_ws_bytes(B, Hq, head_dim, mqa::decode_plan(B, Hkv, max_len, head_dim));
}

int mqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
               float* lse, int B, int Hq, int Hkv, int max_len, int head_dim, float scale, int dtype, int out_dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(q, k_cache, v_cache, seq_lens, out, lse, B, Hq, Hkv, max_len, head_dim, scale, dtype, out_dtype,
                       [&](size_t, void** ws, size_t* bytes) {
                           *ws = workspace;
                           *bytes = workspace_bytes;
                           return (int)MQA_OK;
                       },
                       stream);
}

int mqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                       float* lse, int B, int Hq, int Hkv, int max_len, int head_dim, float scale, int dtype,
                       int out_dtype, void* stream) {
    return decode_impl(q, k_cache, v_cache, seq_lens, out, lse, B, Hq, Hkv, max_len, head_dim, scale, dtype, out_dtype,
                       [](size_t need, void** ws, size_t* bytes) {
                           // too large for the fixed scratch: rejected before
                           // anything touches the device
                           if (need > MQA_DECODE_NOALLOC_SCRATCH_BYTES) return (int)MQA_ERR_WORKSPACE;
                           *bytes = MQA_DECODE_NOALLOC_SCRATCH_BYTES;
                           return current_scratch(ws);
                       },
                       stream);
}

size_t mla_decode_workspace_size(int B, int H, int max_len) {
    if (B <= 0 || H <= 0 || max_len <= 0) return 0;
    return decode_ws_bytes(B, H, 512, mqa::mla_plan(B, max_len));
}

int mla_decode_absorbed(const void* q_abs, const void* kv_cache, const int32_t* seq_lens, void* out, float* lse,
                        int B, int H, int max_len, float scale, int dtype, int out_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
    if (B < 0 || H <= 0 || max_len < 0) return MQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return MQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return MQA_ERR_INVALID_ARG;
    if (B == 0) return MQA_OK;
    if (!q_abs || !kv_cache || !seq_lens || !out) return MQA_ERR_INVALID_ARG;
    if (!aligned16(q_abs) || !aligned16(kv_cache) || !aligned16(out) || ((uintptr_t)seq_lens & 3u) ||
        (lse && ((uintptr_t)lse & 3u)))
        return MQA_ERR_INVALID_ARG;
    if (!is16(dtype) || !valid_out(dtype, out_dtype)) return MQA_ERR_UNSUPPORTED;
    if (H % 16 != 0 || H > 128) return MQA_ERR_UNSUPPORTED;
    if (max_len == 0) return MQA_ERR_INVALID_ARG;
    // one sequence's latent cache is addressed with 32-bit byte offsets
    if ((size_t)max_len * 576 * 2 > 0xFFFFFFFFull) return MQA_ERR_UNSUPPORTED;
    const DecodePlan plan = mqa::mla_plan(B, max_len);
    const size_t need = decode_ws_bytes(B, H, 512, plan);
    if (!workspace || workspace_bytes < need) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_INVALID_ARG;
    mqa::MlaArgs a;
    a.q = q_abs; a.kv = kv_cache; a.seq_lens = seq_lens; a.indices = nullptr; a.topk = 0; a.out = out; a.lse = lse;
    a.B = B; a.H = H; a.max_len = max_len; a.scale = scale; a.out_f32 = out_dtype == MQA_DTYPE_F32;
    a.f16 = dtype == MQA_DTYPE_F16;
    a.part_o = (float*)workspace;
    a.part_ml = (float*)workspace + (size_t)B * H * plan.n_split * 512;
    a.plan = plan; a.stream = (hipStream_t)stream;
    clear_stale_error();
    return hip_status(mqa::mla_launch(a));
}

size_t mla_decode_sparse_workspace_size(int B, int H, int topk) {
    if (B <= 0 || H <= 0 || topk <= 0) return 0;
    return decode_ws_bytes(B, H, 512, mqa::mla_sparse_plan(B, topk));
}

int mla_decode_sparse(const void* q_abs, const void* kv_cache, const int32_t* indices, void* out, float* lse,
                      int B, int H, int max_len, int topk, float scale, int dtype, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
    if (B < 0 || H <= 0 || max_len <= 0 || topk <= 0) return MQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return MQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return MQA_ERR_INVALID_ARG;
    if (B == 0) return MQA_OK;
    if (!q_abs || !kv_cache || !indices || !out) return MQA_ERR_INVALID_ARG;
    if (!aligned16(q_abs) || !aligned16(kv_cache) || !aligned16(out) || ((uintptr_t)indices & 3u) ||
        (lse && ((uintptr_t)lse & 3u)))
        return MQA_ERR_INVALID_ARG;
    if (!is16(dtype) || !valid_out(dtype, out_dtype)) return MQA_ERR_UNSUPPORTED;
    if (H % 16 != 0 || H > 128) return MQA_ERR_UNSUPPORTED;
    // one sequence's latent cache is addressed with 32-bit byte offsets
    if ((size_t)max_len * 576 * 2 > 0xFFFFFFFFull) return MQA_ERR_UNSUPPORTED;
    const DecodePlan plan = mqa::mla_sparse_plan(B, topk);
    const size_t need = decode_ws_bytes(B, H, 512, plan);
    if (!workspace || workspace_bytes < need) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_INVALID_ARG;
    mqa::MlaArgs a;
    a.q = q_abs; a.kv = kv_cache; a.seq_lens = nullptr; a.indices = indices; a.topk = topk; a.out = out; a.lse = lse;
    a.B = B; a.H = H; a.max_len = max_len; a.scale = scale; a.out_f32 = out_dtype == MQA_DTYPE_F32;
    a.f16 = dtype == MQA_DTYPE_F16;
    a.part_o = (float*)workspace;
    a.part_ml = (float*)workspace + (size_t)B * H * plan.n_split * 512;
    a.plan = plan; a.stream = (hipStream_t)stream;
    clear_stale_error();
    return hip_status(mqa::mla_launch(a));
}

int mla_absorb_query(const void* q_nope, const void* q_rope, const void* w_uk, const float* cos_t, const float* sin_t,
                     void* q_abs, int B, int H, int dtype, void* stream) {
    if (B < 0 || H <= 0) return MQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return MQA_ERR_INVALID_ARG;
    if (B == 0) return MQA_OK;
    if (!q_nope || !q_rope || !w_uk || !cos_t || !sin_t || !q_abs) return MQA_ERR_INVALID_ARG;
    if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(q_abs) ||
        ((uintptr_t)cos_t & 3u) || ((uintptr_t)sin_t & 3u))
        return MQA_ERR_INVALID_ARG;
    if (!is16(dtype)) return MQA_ERR_UNSUPPORTED;
    clear_stale_error();
    return hip_status(mqa::mla_absorb_launch(q_nope, q_rope, w_uk, cos_t, sin_t, q_abs, B, H, dtype == MQA_DTYPE_F16,
                                             (hipStream_t)stream));
}

int mla_cache_append(const void* c_kv, const void* k_pe, const float* cos_t, const float* sin_t,
                     const int32_t* positions, void* kv_cache, int B, int max_len, int dtype, void* stream) {
    if (B < 0 || max_len <= 0) return MQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return MQA_ERR_INVALID_ARG;
    if (B == 0) return MQA_OK;
    if (!c_kv || !k_pe || !cos_t || !sin_t || !positions || !kv_cache) return MQA_ERR_INVALID_ARG;
    if (!aligned16(c_kv) || !aligned16(k_pe) || !aligned16(kv_cache) || ((uintptr_t)cos_t & 3u) ||
        ((uintptr_t)sin_t & 3u) || ((uintptr_t)positions & 3u))
        return MQA_ERR_INVALID_ARG;
    if (!is16(dtype)) return MQA_ERR_UNSUPPORTED;
    clear_stale_error();
    return hip_status(mqa::mla_cache_append_launch(c_kv, k_pe, cos_t, sin_t, positions, kv_cache, B, max_len,
                                                   dtype == MQA_DTYPE_F16, (hipStream_t)stream));
}

int mla_output_project(const void* o_lat, const void* w_uv, void* out, int B, int H, int dtype, int out_dtype,
                       void* stream) {
    if (B < 0 || H <= 0) return MQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return MQA_ERR_INVALID_ARG;
    if (B == 0) return MQA_OK;
    if (!o_lat || !w_uv || !out) return MQA_ERR_INVALID_ARG;
    if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MQA_ERR_INVALID_ARG;
    if (!is16(dtype) || !valid_out(dtype, out_dtype)) return MQA_ERR_UNSUPPORTED;
    clear_stale_error();
    return hip_status(mqa::mla_out_proj_launch(o_lat, w_uv, out, B, H, out_dtype == MQA_DTYPE_F32,
                                               dtype == MQA_DTYPE_F16, (hipStream_t)stream));
}

}  // extern "C"
