// The steps either side of absorbed MLA decode: the query absorption, the
// rotary embedding of the decoupled RoPE parts with the cache append, and
// the output up-projection.
//
// After absorption ("GQA和MLA详解" (lzwjava.github.io) §3; walkerchi.com "Full
// 路线" §四 4.3) head h's query over the latent is W_UK[h] q_nope and its
// latent output o_lat is mapped back by W_UV[h]; the 64-d RoPE part of query
// and key is rotated by position and never absorbed (makesence §4.5; the
// rotation is the apply_rotary_pos_emb(q_rope, k_pe, cos, sin) call of
// walkerchi §四 4.2, rotate-half form).  Shapes (DeepSeek-V3, walkerchi §四
// 4.2): d_c = 512, d_nope = 128, d_R = 64, d_v = 128.
//
//   * absorption: per head a [B x 128] . [128 x 512] product.  W_UK[h] rows
//     (latent dims) are the A operand of v_mfma_f32_32x32x16_bf16 loaded
//     straight from HBM (each row contiguous along the contraction), q_nope
//     rows the B operand; a wave keeps its 32 weight rows in registers and
//     sweeps the batch 32 sequences at a time.
//   * up-projection: per head a [B x 512] . [512 x 128] product, contraction
//     over the latent = the rows of W_UV[h].  As in the decode kernel's P.V,
//     four weight rows load 16 bytes at a time and are transposed in
//     registers with byte permutes into A operands of
//     v_mfma_f32_16x16x16_bf16 (M = value dims 8m + t, K = latent dims); the
//     four waves split the latent and add their partial sums through LDS.
// All three take bf16 or (F16) fp16 tensors; fp32 accumulation.
#include "common.hpp"
#include "kernels.hpp"

namespace mqa {

namespace {
constexpr int kDc = 512;    // latent
constexpr int kDn = 128;    // nope part of q / k
constexpr int kDr = 64;     // RoPE part
constexpr int kDv = 128;    // value head dim
constexpr int kDq = kDc + kDr;

// One 16-bit element (bf16, or fp16 if F16; bf16 is the bit container) to
// fp32, and back with round to nearest even.
template <bool F16>
__device__ __forceinline__ float ld16f(const bf16* p) {
    if constexpr (F16) return (float)__builtin_bit_cast(_Float16, *(const uint16_t*)p);
    else return (float)*p;
}
template <bool F16>
__device__ __forceinline__ bf16 st16f(float v) {
    if constexpr (F16) return __builtin_bit_cast(bf16, (_Float16)v);
    else return (bf16)v;
}

// RoPE of one element: x d (of kDr) rotated by (cos, sin) of its position,
// rotate-half form: partner -x[d + 32] for the first half, x[d - 32] after.
template <bool F16>
__device__ __forceinline__ float rope_elem(const bf16* x, int d, const float* cs, const float* sn) {
    const float xv = ld16f<F16>(x + d);
    const float partner = d < kDr / 2 ? -ld16f<F16>(x + d + kDr / 2) : ld16f<F16>(x + d - kDr / 2);
    return xv * cs[d] + partner * sn[d];
}
}  // namespace

// grid (H, kDc / 128): workgroup = one head, 128 latent dims (32 per wave).
template <bool F16>
__global__ __launch_bounds__(256) void mla_absorb_kernel(const bf16* __restrict__ q_nope,
                                                         const bf16* __restrict__ q_rope,
                                                         const bf16* __restrict__ w_uk,
                                                         const float* __restrict__ cosv,
                                                         const float* __restrict__ sinv, bf16* __restrict__ q_abs,
                                                         int B, int H) {
    constexpr int KS = kDn / 16;     // 8 contraction steps
    // the 32 sequences x 128 latent dims of one sweep step, staged so that
    // each sequence's 256 bytes leave in 16-byte stores
    __shared__ __attribute__((aligned(16))) bf16 stage[32][128 + 8];
    const int h = blockIdx.x;
    const int lane = lane_id();
    const int w = wave_id();
    const int h2 = lane >> 5;
    const int n = lane & 31;
    const int c0 = blockIdx.y * 128 + 32 * w;          // latent rows of this wave

    // A operands: W_UK[h] row c0 + n, nope dims 16 ks + 8 h2 .. +7
    bf16x8 wa[KS];
    const bf16* wrow = w_uk + ((size_t)h * kDc + c0 + n) * kDn + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wa[ks] = __builtin_bit_cast(bf16x8, ldg16(wrow + 16 * ks));

    // RoPE part of q_abs (latent block y rotates dims 16 y .. 16 y + 15),
    // while the weight rows are in flight
    constexpr int kRd = kDr / (kDc / 128);
#pragma unroll 2
    for (int e = (int)threadIdx.x; e < B * kRd; e += 256) {
        const int b = e / kRd, d = kRd * blockIdx.y + e % kRd;
        const float y = rope_elem<F16>(q_rope + ((size_t)b * H + h) * kDr, d, cosv + (size_t)b * kDr,
                                       sinv + (size_t)b * kDr);
        q_abs[((size_t)b * H + h) * kDq + kDc + d] = st16f<F16>(y);
    }

    for (int b0 = 0; b0 < B; b0 += 32) {
        const int b = b0 + n;
        const bool ok = b < B;
        const bf16* qrow = q_nope + ((size_t)(ok ? b : 0) * H + h) * kDn + 8 * h2;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = ldg16(qrow + 16 * ks);
            acc = mfma_32x32x16_t<F16>(wa[ks], __builtin_bit_cast(bf16x8, ok ? v : u32x4{0, 0, 0, 0}), acc);
        }
        // accumulator i: latent row c0 + 8(i/4) + 4 h2 + i%4, sequence b
        __syncthreads();                         // the previous step's stores have read the stage
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x2 pk;
            pk.x = pack2_t<F16>(acc[4 * q + 0], acc[4 * q + 1]);
            pk.y = pack2_t<F16>(acc[4 * q + 2], acc[4 * q + 3]);
            *(u32x2*)&stage[n][32 * w + 8 * q + 4 * h2] = pk;
        }
        __syncthreads();
        // 32 rows x 16 chunks of 16 bytes, 256 threads: two chunks each
        for (int e = (int)threadIdx.x; e < 32 * 16; e += 256) {
            const int r = e >> 4, ch = e & 15;
            if (b0 + r < B)
                *(u32x4*)(q_abs + ((size_t)(b0 + r) * H + h) * kDq + blockIdx.y * 128 + 8 * ch) =
                    *(const u32x4*)&stage[r][8 * ch];
        }
    }

}

// grid (B): row positions[b] of sequence b's cache = [c_kv | RoPE(k_pe)].
template <bool F16>
__global__ __launch_bounds__(64) void mla_cache_append_kernel(const bf16* __restrict__ c_kv,
                                                              const bf16* __restrict__ k_pe,
                                                              const float* __restrict__ cosv,
                                                              const float* __restrict__ sinv,
                                                              const int32_t* __restrict__ positions,
                                                              bf16* __restrict__ kv_cache, int max_len) {
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    // every load goes out before the position is known (one memory round
    // trip for the whole kernel)
    const int pos = positions[b];
    const u32x4 lat = ldg16(c_kv + (size_t)b * kDc + 8 * t);             // 64 lanes x 8 = 512
    const float rot = rope_elem<F16>(k_pe + (size_t)b * kDr, t, cosv + (size_t)b * kDr, sinv + (size_t)b * kDr);
    if (pos < 0 || pos >= max_len) return;
    bf16* row = kv_cache + ((size_t)b * max_len + pos) * kDq;
    *(u32x4*)(row + 8 * t) = lat;
    row[kDc + t] = st16f<F16>(rot);
}

// grid (H, ceil(B / 16)): workgroup = one head, 16 sequences, all 128 value
// dims; wave w sums latent dims 128 w .. 128 w + 127.
template <bool OUT_F32, bool F16>
__global__ __launch_bounds__(256) void mla_out_proj_kernel(const bf16* __restrict__ o_lat,
                                                           const bf16* __restrict__ w_uv, void* __restrict__ out,
                                                           int B, int H) {
    constexpr int NSTEP = kDc / 4 / 16;    // 8 steps of 16 latent dims per wave
    __shared__ __attribute__((aligned(16))) float red[4][16][kDv + 4];
    const int h = blockIdx.x;
    const int b0 = blockIdx.y * 16;
    const int lane = lane_id();
    const int w = wave_id();
    const int g = lane >> 4;
    const int m = lane & 15;
    const int b = b0 + m;
    const bool ok = b < B;

    f32x4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16* wh = w_uv + (size_t)h * kDc * kDv;
    const bf16* orow = o_lat + ((size_t)(ok ? b : 0) * H + h) * kDc;
    // every load of the wave is issued before the first product: 32 KB of
    // W_UV[h] per wave in flight at once
    u32x4 r[NSTEP][4];
    u32x2 bop[NSTEP];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
        const int c = 128 * w + 16 * st + 4 * g;     // latent dims c .. c+3 of this lane group
#pragma unroll
        for (int j = 0; j < 4; ++j) r[st][j] = ldg16(wh + (size_t)(c + j) * kDv + 8 * m);   // W_UV[h][c+j][8m..8m+7]
        bop[st] = ok ? *(const u32x2*)(orow + c) : u32x2{0, 0};
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            // A operand of M-tile t: row m <-> value dim 8m + t, slot j <-> latent dim c + j
            const uint32_t sel = (t & 1) ? kSelHiHalves : kSelLoHalves;
            const int wd = t >> 1;
            u32x2 a;
            a.x = perm(r[st][1][wd], r[st][0][wd], sel);
            a.y = perm(r[st][3][wd], r[st][2][wd], sel);
            acc[t] = mfma_16x16x16_t<F16>(a, bop[st], acc[t]);
        }
    }
    // acc[t][i]: value dim 8(4g + i) + t, sequence b0 + m
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][m][8 * (4 * g + i) + t] = acc[t][i];
    __syncthreads();
    for (int e = (int)threadIdx.x; e < 16 * kDv; e += 256) {
        const int bb = e / kDv, d = e % kDv;
        if (b0 + bb >= B) continue;
        const float y = red[0][bb][d] + red[1][bb][d] + red[2][bb][d] + red[3][bb][d];
        const size_t o = ((size_t)(b0 + bb) * H + h) * kDv + d;
        if constexpr (OUT_F32) ((float*)out)[o] = y;
        else ((bf16*)out)[o] = st16f<F16>(y);
    }
}

hipError_t mla_absorb_launch(const void* q_nope, const void* q_rope, const void* w_uk, const float* cosv,
                             const float* sinv, void* q_abs, int B, int H, bool f16, hipStream_t stream) {
    const dim3 grid(H, kDc / 128);
    if (f16)
        hipLaunchKernelGGL(mla_absorb_kernel<true>, grid, dim3(256), 0, stream, (const bf16*)q_nope,
                           (const bf16*)q_rope, (const bf16*)w_uk, cosv, sinv, (bf16*)q_abs, B, H);
    else
        hipLaunchKernelGGL(mla_absorb_kernel<false>, grid, dim3(256), 0, stream, (const bf16*)q_nope,
                           (const bf16*)q_rope, (const bf16*)w_uk, cosv, sinv, (bf16*)q_abs, B, H);
    return hipGetLastError();
}

hipError_t mla_cache_append_launch(const void* c_kv, const void* k_pe, const float* cosv, const float* sinv,
                                   const int32_t* positions, void* kv_cache, int B, int max_len, bool f16,
                                   hipStream_t stream) {
    if (f16)
        hipLaunchKernelGGL(mla_cache_append_kernel<true>, dim3(B), dim3(64), 0, stream, (const bf16*)c_kv,
                           (const bf16*)k_pe, cosv, sinv, positions, (bf16*)kv_cache, max_len);
    else
        hipLaunchKernelGGL(mla_cache_append_kernel<false>, dim3(B), dim3(64), 0, stream, (const bf16*)c_kv,
                           (const bf16*)k_pe, cosv, sinv, positions, (bf16*)kv_cache, max_len);
    return hipGetLastError();
}

hipError_t mla_out_proj_launch(const void* o_lat, const void* w_uv, void* out, int B, int H, bool out_f32, bool f16,
                               hipStream_t stream) {
    const dim3 grid(H, (B + 15) / 16);
#define MQA_OUT_PROJ(O, F) \
    hipLaunchKernelGGL((mla_out_proj_kernel<O, F>), grid, dim3(256), 0, stream, (const bf16*)o_lat, (const bf16*)w_uv, \
                       out, B, H)
    if (f16) {
        if (out_f32) MQA_OUT_PROJ(true, true); else MQA_OUT_PROJ(false, true);
    } else {
        if (out_f32) MQA_OUT_PROJ(true, false); else MQA_OUT_PROJ(false, false);
    }
#undef MQA_OUT_PROJ
    return hipGetLastError();
}

}  // namespace mqa
