// Internal interface between the C ABI (api.hip) and the kernel files.
// Arguments reaching these launchers have been validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mqa {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    int B, Hq, Hkv;
    int Tq, Tkv;      // query tokens, key tokens (causal: Tq <= Tkv, bottom-right)
    int DK, DV;       // query/key width, value width
    int G;
    float scale;
    bool causal;
    bool in16;        // 16-bit inputs (MFMA path); false: fp32 inputs
    bool f16;         // 16-bit type is fp16 (else bf16); also the 16-bit output type
    bool out_f32;
    void* workspace;
    hipStream_t stream;
};

struct PrefillPlan {
    int rows_per_wg;  // query rows (heads x tokens) per workgroup; 0 = widths unsupported
    int kt;           // keys per K/V tile, bf16 path
};

PrefillPlan prefill_plan(int d_qk, int d_v, int in16);
hipError_t prefill_launch(const PrefillArgs& a);

// Split-KV decode plan shared by the workspace query and the launch.
struct DecodePlan {
    int chunk;    // cache rows per workgroup (per split)
    int n_split;  // splits per sequence
};

DecodePlan decode_plan(int B, int Hkv, int max_len, int head_dim);
DecodePlan mla_plan(int B, int max_len);
DecodePlan mla_sparse_plan(int B, int topk);

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* seq_lens;
    void* out;
    float* lse;
    int B, Hq, Hkv, max_len, D, G;
    float scale;
    bool f16;        // fp16 inputs and 16-bit output (else bf16)
    bool out_f32;
    float* part_o;   // [B*Hq*n_split, D]
    float* part_ml;  // [B*Hq*n_split, 2]
    DecodePlan plan;
    hipStream_t stream;
};

hipError_t decode_launch(const DecodeArgs& a);

struct MlaArgs {
    const void* q;
    const void* kv;
    const int32_t* seq_lens;   // dense: rows 0 .. seq_lens[b]-1
    const int32_t* indices;    // sparse (non-null): rows indices[b, 0 .. topk-1]
    int topk;
    void* out;
    float* lse;
    int B, H, max_len;
    float scale;
    bool out_f32;
    bool f16;        // fp16 inputs (and fp16 output unless out_f32); else bf16
    float* part_o;   // [B*H*n_split, 512]
    float* part_ml;  // [B*H*n_split, 2]
    DecodePlan plan;
    hipStream_t stream;
};

hipError_t mla_launch(const MlaArgs& a);

// The steps either side of absorbed MLA decode (d_c 512, d_nope 128, d_R 64, d_v 128).
// f16: fp16 tensors (else bf16); out_f32: fp32 output (else the input type)
hipError_t mla_absorb_launch(const void* q_nope, const void* q_rope, const void* w_uk, const float* cosv,
                             const float* sinv, void* q_abs, int B, int H, bool f16, hipStream_t stream);
hipError_t mla_cache_append_launch(const void* c_kv, const void* k_pe, const float* cosv, const float* sinv,
                                   const int32_t* positions, void* kv_cache, int B, int max_len, bool f16,
                                   hipStream_t stream);
hipError_t mla_out_proj_launch(const void* o_lat, const void* w_uv, void* out, int B, int H, bool out_f32, bool f16,
                               hipStream_t stream);

// LSE merge of split partials (shared by both decode paths).
hipError_t merge_launch(const float* part_o, const float* part_ml, const int32_t* seq_lens, void* out,
                        float* lse, int B, int H, int max_len, int D, int chunk, int n_split, bool out_f32,
                        bool out_f16, hipStream_t stream);

}  // namespace mqa
