/*
 * mqa_attn.h -- C ABI of the MI355X (gfx950) attention library for query
 * heads that share few key/value heads: MQA, GQA and the absorbed form of
 * MLA.  Library: libmqa_attn.so (built from attention_mqa_gqa_amd/csrc).
 *
 * What is computed (source pages, by title and section):
 *   out = softmax(scale * Q K^T  [+ causal mask]) V, per query head, where a
 *   query head h reads key/value head h / (Hq / Hkv)
 *     - single-head definition: "带你了解Attention,从MHA到DeepSeek"
 *       (api.makesence.top) §1.2; causal mask and prefill/decode phases:
 *       "GQA和MLA详解" (lzwjava.github.io) §1;
 *     - head sharing (repeat_interleave on the head axis, done here by
 *       indexing, never by copying): lzwjava §2, makesence §3.1-3.2,
 *       "Full 路线：保留 softmax，压缩 K/V 表示" (walkerchi.com) §三;
 *     - MQA with head_dim 512 and 16 query heads over one KV head: zdabc.icu
 *       article on DeepSeek V4.1's MQA operator, sections
 *       "head_dim = 512 为什么值得注意" and the MQA benchmark baseline;
 *     - MLA decode on the cached latent after folding W_UK into the query and
 *       W_UV into the output (matrix absorption) with a decoupled 64-d RoPE
 *       key: lzwjava §3, makesence §4.3 and §4.5, walkerchi §四 4.2-4.3.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, owned by the caller, row-major
 *     with the last dimension contiguous, and 16-byte aligned.  The library
 *     allocates nothing, keeps no state between calls (beyond a once-per-
 *     process query of the device's CU count and a kernel's occupancy),
 *     never synchronises, and enqueues its kernels on `stream` (a
 *     hipStream_t; NULL = the default stream).  Inputs are read-only; outputs and workspace are overwritten.
 *   - Element types: MQA_DTYPE_F32 (IEEE float), MQA_DTYPE_BF16 (bfloat16)
 *     or MQA_DTYPE_F16 (IEEE half; the zdabc.icu benchmark runs its MQA
 *     operator in float16 on the GPU).  Products accumulate in fp32.
 *     Probabilities are rounded to the input's 16-bit type before the P.V
 *     product when the inputs are 16-bit; fp32 inputs stay fp32 end to end.
 *     A 16-bit input gives a result of the same type or fp32 (out_dtype).
 *     Conversions to 16 bits round to nearest even.
 *   - `lse` (optional, may be NULL) receives the natural-log log-sum-exp of
 *     the scaled, masked scores of each query row, in fp32.
 *   - Every argument is validated on the host before any HIP call; a rejected
 *     call returns a negative status and enqueues nothing.  A zero batch or
 *     zero sequence length is a valid empty call (returns MQA_OK, enqueues
 *     nothing).  The library never aborts; kernel-launch failures are
 *     reported as MQA_ERR_HIP.
 *   - Calls on different streams may overlap only if their outputs and
 *     workspaces do not alias.
 */
#ifndef MQA_ATTN_H
#define MQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MQA_ATTN_ABI_VERSION 3

typedef enum {
    MQA_DTYPE_F32 = 0,
    MQA_DTYPE_BF16 = 1,
    MQA_DTYPE_F16 = 2          /* IEEE half */
} mqa_dtype;

typedef enum {
    MQA_OK = 0,
    MQA_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or scale   */
    MQA_ERR_UNSUPPORTED = -2,  /* valid request outside what the kernels cover */
    MQA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required   */
    MQA_ERR_HIP = -4           /* the HIP runtime reported a launch error      */
} mqa_status;

/* Version of this ABI (MQA_ATTN_ABI_VERSION of the built library). */
int mqa_attn_abi_version(void);

/* Static description of a status code; never NULL. */
const char* mqa_status_string(int status);

/* Name of the HIP error behind the most recent MQA_ERR_HIP (or "hipSuccess")
 * returned on the calling thread; never NULL.  Each entry point discards any
 * error left pending by earlier, unrelated HIP calls on the thread before it
 * launches, so MQA_ERR_HIP always refers to this library's own launches. */
const char* mqa_last_hip_error_name(void);

/* ---------------------------------------------------------------- prefill
 * Causal (or full) attention over a whole sequence.
 *   q   [B, Hq,  T, D]      k, v [B, Hkv, T, D]      out [B, Hq, T, D]
 *   lse [B, Hq, T] fp32 or NULL
 *   causal != 0: key j is visible to query i iff j <= i (square, top-left
 *   aligned: query i is the token at position i).
 *   scale: the factor on Q.K^T, normally 1/sqrt(D).  Must be finite and > 0.
 * Supported: Hq % Hkv == 0;
 *   in_dtype BF16 or F16 -> out_dtype the same or F32, D in {128, 512}, and the group
 *     size G = Hq/Hkv <= 128 (D=512) or G <= 256 (D=128) (any G: a
 *     workgroup takes floor(rows / G) tokens of all G heads);
 *   in_dtype F32 -> out_dtype F32, D a multiple of 64 up to 512, any G, and
 *     T * G < 2^35 (the query rows are dealt in blocks of 16).
 * Workspace: 16-bit inputs need `mqa_prefill_workspace_size()` bytes, where the
 * library first writes a transposed V, and at D = 512 also K with padded
 * rows, as one stream of 32-key tiles (B * Hkv * ceil(T/32) * 32 * (D + k)
 * * 2 bytes, k = D + 8 when D = 512, else 0: narrower K rows are read from K
 * itself); F32 needs none (workspace may be NULL with workspace_bytes 0).
 */
size_t mqa_prefill_workspace_size(int B, int Hq, int Hkv, int T, int head_dim,
                                  int in_dtype);

int mqa_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                int B, int Hq, int Hkv, int T, int head_dim, float scale, int causal,
                int in_dtype, int out_dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------ general prefill
 * The same attention with separate query / key lengths and separate
 * query-key / value widths:
 *   q [B, Hq, T_q, d_qk]   k [B, Hkv, T_kv, d_qk]   v [B, Hkv, T_kv, d_v]
 *   out [B, Hq, T_q, d_v]  lse [B, Hq, T_q] fp32 or NULL
 *   causal != 0: the T_q queries are the LAST T_q tokens of the T_kv-token
 *   sequence (bottom-right alignment): query i sits at position
 *   T_kv - T_q + i and sees key j iff j <= T_kv - T_q + i.  T_q == T_kv is
 *   the square mask of mqa_prefill; T_q < T_kv is a block of new tokens
 *   after T_kv - T_q earlier ones whose keys and values are in k / v
 *   (chunked prefill, several decode tokens at once).  The pages show only
 *   the square case ("GQA和MLA详解" (lzwjava.github.io) §1); this alignment
 *   is the reading that keeps a chunk's rows equal to the matching rows of
 *   the whole sequence's prefill.  causal with T_q > T_kv is rejected
 *   (MQA_ERR_INVALID_ARG: a query would see no key).
 *   d_qk != d_v is the expanded (MHA-mode) MLA prefill: per-head keys
 *   [c_kv W_UK[h] | k_pe] of 128 + 64 = 192 values, per-head values
 *   c_kv W_UV[h] of 128, Hq = Hkv = 128, scale 1/sqrt(192)
 *   ("带你了解Attention,从MHA到DeepSeek" (api.makesence.top) §4.4, prefill
 *   expanded and decode absorbed; dimensions as in walkerchi.com "Full 路线"
 *   §四 4.2).
 * Supported: everything mqa_prefill supports (d_qk == d_v, as listed there),
 *   plus (d_qk, d_v) = (192, 128) with any G <= 128 (16-bit) or any G (fp32;
 *   T_q * G < 2^35 as for mqa_prefill).
 *   T_q == 0 or B == 0 is an empty call; T_kv == 0 with T_q > 0 is rejected.
 * Workspace (16-bit inputs): `mqa_prefill_ex_workspace_size()` bytes =
 *   B * Hkv * ceil(T_kv/32) * 32 * (k + d_v) * 2, k = d_qk + 8 when
 *   d_qk = 512 (padded 1 KB key rows), else 0; F32 needs none.
 * mqa_prefill(..., T, head_dim, ...) is exactly
 * mqa_prefill_ex(..., T, T, head_dim, head_dim, ...).
 */
size_t mqa_prefill_ex_workspace_size(int B, int Hq, int Hkv, int T_q, int T_kv,
                                     int d_qk, int d_v, int in_dtype);

int mqa_prefill_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int Hq, int Hkv, int T_q, int T_kv, int d_qk, int d_v,
                   float scale, int causal, int in_dtype, int out_dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------- decode
 * One new query token per sequence against a KV cache (split-KV: the valid
 * cache of each sequence is cut into chunks processed in parallel, then the
 * chunk results are merged by log-sum-exp in a fixed order, so the result is
 * deterministic run to run).
 *   q [B, Hq, D]     k_cache, v_cache [B, Hkv, max_len, D]    out [B, Hq, D]
 *   seq_lens int32[B] on the DEVICE: sequence b attends to cache rows
 *   0 .. seq_lens[b]-1 (the cache already holds the current token).  Values
 *   above max_len are treated as max_len; a sequence with seq_lens[b] <= 0
 *   gets out = 0 and lse = -inf.  Rows at or beyond seq_lens[b] are never
 *   read.
 *   lse [B, Hq] fp32 or NULL.
 * Supported: dtype BF16 or F16, out_dtype the same or F32, D in {128, 512},
 *   G = Hq/Hkv <= 16.
 * Workspace: `mqa_decode_workspace_size()` bytes (chunk partials).
 */
size_t mqa_decode_workspace_size(int B, int Hq, int Hkv, int max_len, int head_dim);

int mqa_decode(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* seq_lens, void* out, float* lse,
               int B, int Hq, int Hkv, int max_len, int head_dim, float scale,
               int dtype, int out_dtype,
               void* workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------- decode without allocation
 * mqa_decode for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, semantics, kernels and results
 * as mqa_decode (bit for bit), minus the workspace: the chunk partials go
 * to a fixed scratch array of MQA_DECODE_NOALLOC_SCRATCH_BYTES (64 MiB) in
 * the library's device memory, one per device, resolved on the first call
 * made with that device current and held until the process ends.  The call
 * allocates nothing (no hipMalloc / hipFree, no allocating library call).
 * A call whose partials would exceed the scratch, i.e.
 * mqa_decode_workspace_size(B, Hq, Hkv, max_len, head_dim) >
 * MQA_DECODE_NOALLOC_SCRATCH_BYTES, returns MQA_ERR_WORKSPACE and enqueues
 * nothing.  For scale: MQA batch 64 x 16 heads at d 512 needs 8 MiB with an
 * 8192-row cache and 32 MiB with a 65536-row one; GQA batch 128 x 64 heads
 * at d 128 with a 16384-row cache needs 4 MiB; MQA batch 2048 x 16 heads at
 * d 512 (64.25 MiB) is refused.
 * Every call on one device shares that device's scratch: calls that can run
 * at the same time on one device (different streams, or graphs replayed
 * concurrently) race on it and must be serialised by the caller.  Nothing
 * in the scratch needs to start at any particular value (each partial is
 * written before it is read).
 */
#define MQA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int mqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, void* out, float* lse,
                       int B, int Hq, int Hkv, int max_len, int head_dim, float scale,
                       int dtype, int out_dtype, void* stream);

/* ----------------------------------------------------- MLA absorbed decode
 * Decode for multi-head latent attention in the absorbed form.  Every cached
 * token is one row [c_kv (512) | k_pe (64)] = 576 values shared by all heads.
 * The caller passes the absorbed query of each head,
 *   q_abs[b,h] = [W_UK[h] q_nope (512) | RoPE(q_rope) (64)],
 * and applies W_UV[h] to the returned latent output itself.  The whole
 * 576-wide row is the key; its first 512 values are the value.
 *   q_abs [B, H, 576]   kv_cache [B, max_len, 576]   out [B, H, 512]
 *   seq_lens int32[B] on the device, as for mqa_decode.
 *   lse [B, H] fp32 or NULL.
 *   scale: normally 1/sqrt(128 + 64), the original per-head q.k width;
 *          finite and > 0.
 * Supported: dtype BF16 or F16, out_dtype the same or F32, H a multiple of 16, H <= 128.
 * Workspace: `mla_decode_workspace_size()` bytes.
 */
size_t mla_decode_workspace_size(int B, int H, int max_len);

int mla_decode_absorbed(const void* q_abs, const void* kv_cache, const int32_t* seq_lens,
                        void* out, float* lse, int B, int H, int max_len, float scale,
                        int dtype, int out_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------- MLA sparse (top-k) decode
 * Absorbed MLA decode over a selected subset of each sequence's cached rows:
 * DeepSeek sparse attention keeps the MLA latent cache and lets each query
 * attend only to the k positions an indexer selected (k = 2048 in V3.2;
 * "带你了解Attention,从MHA到DeepSeek" (api.makesence.top) §5.1).  The
 * selection is an input here (the indexer is not part of this library).
 *   q_abs [B, H, 576]   kv_cache [B, max_len, 576]   out [B, H, 512]
 *   indices int32 [B, topk] on the DEVICE: sequence b attends to the rows
 *   kv_cache[b, indices[b, j]], j = 0 .. topk-1.  Entries outside
 *   [0, max_len) are skipped (use -1 to pad sequences with fewer than topk
 *   selected rows); they are never read.  The list normally names distinct
 *   rows; a row listed twice enters the softmax twice.  A sequence with no
 *   valid entry gets out = 0 and lse = -inf.
 *   lse [B, H] fp32 or NULL.  scale as for mla_decode_absorbed.
 * Supported: dtype BF16 or F16, out_dtype the same or F32, H a multiple of 16, H <= 128,
 *   topk >= 1 (topk <= 0 is MQA_ERR_INVALID_ARG).
 * Workspace: `mla_decode_sparse_workspace_size()` bytes (chunk partials of
 *   the index list).
 */
size_t mla_decode_sparse_workspace_size(int B, int H, int topk);

int mla_decode_sparse(const void* q_abs, const void* kv_cache, const int32_t* indices,
                      void* out, float* lse, int B, int H, int max_len, int topk, float scale,
                      int dtype, int out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------- MLA decode: the steps around it
 * The pieces of one MLA decode step that surround mla_decode_absorbed, for
 * the DeepSeek-V3 shapes (walkerchi.com "Full 路线" §四 4.2: latent d_c =
 * 512, nope part 128, RoPE part d_R = 64, value 128 per head).  A step is
 *   mla_absorb_query -> mla_cache_append -> mla_decode_absorbed
 *   -> mla_output_project.
 * Matrix absorption ("GQA和MLA详解" (lzwjava.github.io) §3; walkerchi §四
 * 4.3): the per-head key up-projection folds into the query and the value
 * up-projection is applied to the latent output.  The 64-d RoPE part is
 * rotated by position and never absorbed ("带你了解Attention,从MHA到DeepSeek"
 * (api.makesence.top) §4.5); the rotation is the apply_rotary_pos_emb(q, k,
 * cos, sin) call of walkerchi §四 4.2 in rotate-half form:
 *   RoPE(x) = x * cos + [-x[32:64] | x[0:32]] * sin,
 * with cos, sin fp32 [B, 64] the rotary factors of each sequence's position
 * (the caller builds them, as a model's position embeddings).
 * dtype BF16 or F16 for every 16-bit tensor of the call (MQA_ERR_UNSUPPORTED
 * otherwise); every pointer a device pointer, 16-byte aligned (cos / sin /
 * positions 4-byte aligned).
 *
 * mla_absorb_query: q_nope [B, H, 128], q_rope [B, H, 64],
 *   w_uk [H, 512, 128] (per head: latent x nope) ->
 *   q_abs [B, H, 576] = [W_UK[h] q_nope (512) | RoPE(q_rope) (64)].
 * mla_cache_append: writes the new token of each sequence,
 *   kv_cache[b, positions[b]] = [c_kv[b] (512) | RoPE(k_pe[b]) (64)],
 *   c_kv [B, 512], k_pe [B, 64] (before rotation), positions int32 [B] on the
 *   device; a position outside [0, max_len) writes nothing.
 * mla_output_project: o_lat [B, H, 512] (mla_decode_absorbed's output),
 *   w_uv [H, 512, 128] (per head: latent x value) ->
 *   out [B, H, 128] = o_lat[b, h] W_UV[h]; out_dtype = dtype or F32.
 */
int mla_absorb_query(const void* q_nope, const void* q_rope, const void* w_uk,
                     const float* cos_t, const float* sin_t, void* q_abs,
                     int B, int H, int dtype, void* stream);

int mla_cache_append(const void* c_kv, const void* k_pe, const float* cos_t,
                     const float* sin_t, const int32_t* positions, void* kv_cache,
                     int B, int max_len, int dtype, void* stream);

int mla_output_project(const void* o_lat, const void* w_uv, void* out,
                       int B, int H, int dtype, int out_dtype, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* MQA_ATTN_H */
