// MLA decode in the absorbed form: attention of H query heads directly over
// the cached latent rows [c_kv (512) | k_pe (64)].
//
// After folding W_UK into the query and W_UV into the output (matrix
// absorption, "GQA和MLA详解" (lzwjava.github.io) §3; "带你了解Attention,从MHA到
// DeepSeek" §4.3) every head attends over the same 576-wide rows: the whole
// row is the key, its first 512 values (the latent) are the value, and the
// 64-d RoPE key is the part that cannot be absorbed (makesence §4.5;
// walkerchi "Full 路线" §四 4.2).  Each cached row is read from HBM once per
// step and used by all heads:
//   * one workgroup (8 waves) = one (sequence, chunk of rows), all heads;
//     wave w owns heads 16w .. 16w+15;
//   * 32-row tiles are copied global -> LDS with asynchronous direct-to-LDS
//     loads (double buffered, swizzled); the latent part of each tile is then
//     transposed once in LDS for the P.V operand;
//   * S^T = KV q_abs^T (K = 576 = 18 steps of 32) and O^T += V^T P^T
//     (V^T = first 512 columns) on v_mfma_f32_16x16x32_bf16, fp32
//     accumulation, online softmax in registers;
//   * partials per (head, split) are merged by the shared log-sum-exp kernel.
#include "common.hpp"
#include "layout.hpp"
#include "kernels.hpp"

namespace mqa {

namespace {
constexpr int kDK = 576;   // key width: latent + RoPE part
constexpr int kDC = 512;   // latent width (= value width)
constexpr int kDR = 64;    // RoPE part
constexpr int kKT = 32;    // rows per tile
constexpr int kNW = 8;     // waves per workgroup
}  // namespace

__global__ __launch_bounds__(kNW * 64, 1) void mla_split_kernel(
    const bf16* __restrict__ Qa, const bf16* __restrict__ KV, const int32_t* __restrict__ seq_lens,
    float* __restrict__ part_o, float* __restrict__ part_ml, int H, int max_len, int chunk, int n_split,
    float scale_log2) {
    constexpr int KS_LAT = kDC / 32;        // 16
    constexpr int KS_ROPE = kDR / 32;       // 2
    constexpr int KS = KS_LAT + KS_ROPE;    // 18
    constexpr int MT_S = kKT / 16;          // 2
    constexpr int MT_O = kDC / 16;          // 32
    constexpr int LAT_TILE = kKT * kDC;     // elements
    constexpr int ROPE_TILE = kKT * kDR;
    constexpr int RL = kKT / 8;             // chunks per V^T row (4)

    __shared__ __attribute__((aligned(16))) bf16 lat[2][LAT_TILE];
    __shared__ __attribute__((aligned(16))) bf16 rope[2][ROPE_TILE];
    __shared__ __attribute__((aligned(16))) bf16 vt[LAT_TILE];

    const int s_idx = blockIdx.x;
    const int b = blockIdx.y;
    const int L = min(max(seq_lens[b], 0), max_len);
    const int begin = s_idx * chunk;
    if (begin >= L) return;
    const int end = min(begin + chunk, L);
    const int n_tiles = (end - begin + kKT - 1) / kKT;

    const int lane = lane_id();
    const int w = wave_id();
    const int g = lane >> 4;
    const int n = lane & 15;
    const int tid = threadIdx.x;
    const bool active = 16 * w < H;
    const int head = 16 * w + n;

    const bf16* KVb = KV + (size_t)b * max_len * kDK;

    bf16x8 qb[KS];
    {
        const bf16* qrow = Qa + ((size_t)b * H + (active ? head : 0)) * kDK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks < KS_LAT ? 32 * ks + 8 * g : kDC + 32 * (ks - KS_LAT) + 8 * g;
            qb[ks] = ldg_bf16x8(qrow + c);
        }
    }

    // 36 one-KB copies per tile: 32 latent rows (one row each) + 4 for the RoPE block.
    auto issue = [&](int tile, int stage) {
#pragma unroll
        for (int r = 0; r < 5; ++r) {
            const int u = r * kNW + w;          // wave-uniform
            if (u < 32) {
                const int kk = u;
                const int key = min(begin + tile * kKT + kk, end - 1);
                const int c = lane ^ layout::kswz(kk);
                copy16_to_lds_off(KVb + (size_t)key * kDK, (uint32_t)c * 16u, &lat[stage][kk * kDC]);
            } else if (u < 36) {
                const int q = (u - 32) * 64 + lane;
                const int kk = q >> 3;
                const int c = (q & 7) ^ layout::swz8(kk);
                const int key = min(begin + tile * kKT + kk, end - 1);
                copy16_to_lds_off(KVb, (uint32_t)(key * kDK + kDC + c * 8) * 2u, &rope[stage][(u - 32) * 512]);
            }
        }
    };

    f32x4 o[MT_O];
#pragma unroll
    for (int mt = 0; mt < MT_O; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    issue(0, 0);
    for (int it = 0; it < n_tiles; ++it) {
        const int stage = it & 1;
        wait_vmcnt<0>();
        __syncthreads();
        // transpose the latent tile: thread (kb, db) moves an 8x8 block, in
        // two 4-row halves (each half gives 4 keys = 8 bytes per head dim)
        if (tid < 256) {
            const int kb = tid & 3;
            const int db = tid >> 2;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                u32x4 r[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kk = 8 * kb + 4 * half + j;
                    r[j] = *(const u32x4*)&lat[stage][kk * kDC + (db ^ layout::kswz(kk)) * 8];
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int d = 8 * db + t;
                    const uint32_t sel = (t & 1) ? kSelHiHalves : kSelLoHalves;
                    const int wd = t >> 1;
                    u32x2 ov;
                    ov.x = perm(r[1][wd], r[0][wd], sel);
                    ov.y = perm(r[3][wd], r[2][wd], sel);
                    *(u32x2*)&vt[(d * RL + (kb ^ layout::swz4(d))) * 8 + 4 * half] = ov;
                }
            }
        }
        __syncthreads();
        if (it + 1 < n_tiles) issue(it + 1, stage ^ 1);
        if (!active) continue;

        // ---- S^T = KV q^T ----------------------------------------------------
        f32x4 s[MT_S];
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt) s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt) {
                const int kk = layout::st_row_key(mt, n);
                bf16x8 a;
                if (ks < KS_LAT) {
                    const int pos = (4 * ks + g) ^ layout::kswz(kk);
                    a = *(const bf16x8*)&lat[stage][kk * kDC + pos * 8];
                } else {
                    const int pos = (4 * (ks - KS_LAT) + g) ^ layout::swz8(kk);
                    a = *(const bf16x8*)&rope[stage][kk * kDR + pos * 8];
                }
                s[mt] = mfma_16x16x32(a, qb[ks], s[mt]);
            }
        }
        // ---- mask + online softmax ---------------------------------------------
        const int j0 = begin + it * kKT;
        float mloc = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = j0 + layout::st_c_key(mt, g, i);
                const float v = key < end ? s[mt][i] * scale_log2 : -INFINITY;
                s[mt][i] = v;
                mloc = fmaxf(mloc, v);
            }
        }
        const float mx = max_over_groups(mloc);
        if (__any(mx > m_run + kRescaleSlack)) {
            const float mnew = fmaxf(m_run, mx);
            const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - mnew);
            m_run = mnew;
            l_run *= alpha;
#pragma unroll
            for (int mt = 0; mt < MT_O; ++mt) o[mt] *= alpha;
        }
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(s[mt][i] - m_run);
                s[mt][i] = p;
                l_run += p;
            }
        }
        const bf16x8 pb = pack_bf16x8(s[0], s[1]);
        // ---- O^T += V^T P^T -----------------------------------------------------
#pragma unroll
        for (int mt = 0; mt < MT_O; ++mt) {
            const int d = layout::pv_row_d(mt, n);
            const bf16x8 a = *(const bf16x8*)&vt[(d * RL + (g ^ layout::swz4(d))) * 8];
            o[mt] = mfma_16x16x32(a, pb, o[mt]);
        }
    }

    if (!active) return;
    const float l_tot = sum_over_groups(l_run);
    const size_t prow = ((size_t)b * H + head) * n_split + s_idx;
#pragma unroll
    for (int bq = 0; bq < kDC / 32; ++bq) {
        float* dst = part_o + prow * kDC + 32 * bq + 8 * g;
        *(f32x4*)dst = o[2 * bq];
        *(f32x4*)(dst + 4) = o[2 * bq + 1];
    }
    if (g == 0) { part_ml[2 * prow] = m_run; part_ml[2 * prow + 1] = l_tot; }
}

DecodePlan mla_plan(int B, int max_len) {
    const int target_wgs = 256;
    int splits = (target_wgs + B - 1) / B;
    int chunk = (max_len + splits - 1) / splits;
    if (chunk < 1024) chunk = 1024;
    chunk = (chunk + kKT - 1) / kKT * kKT;
    DecodePlan p;
    p.chunk = chunk;
    p.n_split = (max_len + chunk - 1) / chunk;
    if (p.n_split < 1) p.n_split = 1;
    return p;
}

hipError_t mla_launch(const MlaArgs& a) {
    const dim3 grid(a.plan.n_split, a.B);
    hipLaunchKernelGGL(mla_split_kernel, grid, dim3(kNW * 64), 0, a.stream, (const bf16*)a.q, (const bf16*)a.kv,
                       a.seq_lens, a.part_o, a.part_ml, a.H, a.max_len, a.plan.chunk, a.plan.n_split,
                       a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return merge_launch(a.part_o, a.part_ml, a.seq_lens, a.out, a.lse, a.B, a.H, a.max_len, kDC, a.plan.chunk,
                        a.plan.n_split, a.out_f32, a.stream);
}

}  // namespace mqa
