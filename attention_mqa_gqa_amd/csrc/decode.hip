// Split-KV decode for one new query token per sequence (MQA / GQA).
//
// Decode reads the whole KV cache once per step and is bound by memory
// bandwidth ("GQA和MLA详解" (lzwjava.github.io) §1, decode phase).  The design
// therefore streams the cache straight from HBM into registers:
//   * one workgroup = one (sequence, KV head, chunk of cache rows); its NW
//     waves take consecutive sub-ranges of the chunk;
//   * the G query heads sharing the KV head form the 16 MFMA columns (heads
//     indexed, not copied; lzwjava §2), zero-padded up to 16;
//   * K rows load with 16-byte loads directly in the A-operand layout of
//     v_mfma_f32_16x16x32_bf16 (S^T = K q^T, no LDS);
//   * V rows load 16 bytes at a time (256 contiguous bytes per row per
//     instruction) and are transposed in registers with byte permutes into
//     the A operand of v_mfma_f32_16x16x16_bf16 (O^T += V^T P^T);
//   * per-wave online softmax, then the waves of a workgroup merge through
//     LDS and write one (m, l, unnormalised O) partial per (head, split);
//   * a second kernel merges the splits of each row by log-sum-exp in a fixed
//     order, so the result is deterministic (no float atomics; lzwjava §4
//     on ordering and determinism).
// The cache streams with non-temporal loads (each row is read once).
// F16: fp16 inputs (the _f16 MFMAs, P rounded to fp16); else bf16.
// Cache rows at or beyond seq_lens[b] are never read.
#include "common.hpp"
#include "layout.hpp"
#include "kernels.hpp"

namespace mqa {

// Sequences are taken longest first: workgroup z works on the sequence whose
// rank by (clamped length descending, index ascending) is z.  With ragged
// lengths the workgroups of the longest sequences then start in the first
// round of resident workgroups instead of forming the tail.  Batches above
// kSortMax keep the identity order, and so does a grid that is resident
// all at once (sort = false: the order cannot matter there).  Returns the
// sequence; its clamped length goes to *len.
constexpr int kSortMax = 256;
template <int NT>
__device__ __forceinline__ int longest_first(const int32_t* __restrict__ seq_lens, int B, int max_len, int z,
                                             bool sort, int* sl, int* pick, int* len) {
    static_assert(NT >= kSortMax, "one thread per sequence");
    if (!sort || B <= 1 || B > kSortMax) {
        *len = min(max(seq_lens[z], 0), max_len);
        return z;
    }
    const int t = (int)threadIdx.x;
    if (t < B) sl[t] = min(max(seq_lens[t], 0), max_len);
    __syncthreads();
    if (t < B) {
        const int lt = sl[t];
        int r = 0;
#pragma unroll 8
        for (int u = 0; u < B; ++u) {
            const int lu = sl[u];
            r += (lu > lt) | ((lu == lt) & (u < t));
        }
        if (r == z) *pick = t;
    }
    __syncthreads();
    const int b = *pick;
    *len = sl[b];
    return b;
}

template <int D, int KSUB, int NW, bool F16>
__global__ __launch_bounds__(NW * 64, 1) void decode_split_kernel(
    const bf16* __restrict__ Qp, const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_o, float* __restrict__ part_ml, int Hq,
    int Hkv, int max_len, int G, int chunk, int n_split, float scale_log2, int sort) {
    constexpr int KS = D / 32;     // QK^T contraction steps (16x16x32)
    constexpr int NSL = D / 128;   // V slices of 128 head dims
    constexpr int MT_O = D / 16;   // O^T M-tiles
    constexpr int STEP = 16 * KSUB;
    constexpr int PAD = D + 4;     // LDS row stride (floats) for the merge

    __shared__ float sm_m[NW][16];
    __shared__ float sm_l[NW][16];
    __shared__ __attribute__((aligned(16))) float sm_o[NW][16][PAD];

    __shared__ int sm_len[kSortMax];
    __shared__ int sm_pick;

    const int s_idx = blockIdx.x;
    const int hk = blockIdx.y;
    int L;
    const int b = longest_first<NW * 64>(seq_lens, (int)gridDim.z, max_len, (int)blockIdx.z, sort != 0, sm_len,
                                         &sm_pick, &L);
    const int wg_begin = s_idx * chunk;
    if (wg_begin >= L) return;                       // whole workgroup: uniform exit
    const int wg_end = min(wg_begin + chunk, L);

    const int lane = lane_id();
    const int w = wave_id();
    const int g = lane >> 4;
    const int n = lane & 15;
    // the rows this workgroup really has (fewer than chunk at the end of a
    // sequence) split evenly over its waves, 16-row aligned; a wave whose
    // share starts past wg_end idles
    const int per_wave = ((wg_end - wg_begin + NW - 1) / NW + 15) / 16 * 16;
    const int k_begin = wg_begin + w * per_wave;
    const int k_end = min(k_begin + per_wave, wg_end);

    const size_t bh = (size_t)b * Hkv + hk;
    const bf16* Kbh = Kc + bh * (size_t)max_len * D;
    const bf16* Vbh = Vc + bh * (size_t)max_len * D;

    // q^T operand: column n = head hk*G + n (zero for n >= G).
    bf16x8 qb[KS];
    {
        const bool ok = n < G;
        const bf16* qrow = Qp + ((size_t)b * Hq + hk * G + (ok ? n : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ks] = ok ? ldg_bf16x8(qrow + 32 * ks + 8 * g) : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }

    f32x4 o[MT_O];
#pragma unroll
    for (int mt = 0; mt < MT_O; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // K rows of a step land directly in the A-operand layout of the S^T
    // MFMA; V rows 16 bytes at a time.  Rows past k_end are clamped to the
    // last valid row (and masked below).
    bf16x8 ka[KSUB][KS];
    u32x4 vr[KSUB][NSL][4];
    auto load_k = [&](int k0) {
#pragma unroll
        for (int sub = 0; sub < KSUB; ++sub) {
            const int kr = min(k0 + 16 * sub + n, k_end - 1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16* src = Kbh + (size_t)kr * D + 32 * ks + 8 * g;
                // streaming hint: faster for 1 KB rows, slower for 256-byte
                // rows (two loads share each 128-byte line here)
                ka[sub][ks] = (D >= 512) ? ldg_bf16x8_stream(src) : ldg_bf16x8(src);
            }
        }
    };
    auto load_v = [&](int k0) {
#pragma unroll
        for (int sub = 0; sub < KSUB; ++sub)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int vrow = min(k0 + 16 * sub + 4 * g + j, k_end - 1);
#pragma unroll
                for (int sl = 0; sl < NSL; ++sl) vr[sub][sl][j] = ldg16_stream(Vbh + (size_t)vrow * D + (16 * sl + n) * 8);
            }
    };
    // Software pipeline: the K rows of the next step load while this step's
    // softmax and P.V run, and its V rows while the next scores run, so the
    // wave always has one of the two streams in flight.
    if (k_begin < k_end) {
        load_k(k_begin);
        load_v(k_begin);
    }
    for (int k0 = k_begin; k0 < k_end; k0 += STEP) {
        const bool more = k0 + STEP < k_end;
        // S^T: lane group g holds keys k0 + 16 sub + 4g + i for head n
        f32x4 s[KSUB];
#pragma unroll
        for (int sub = 0; sub < KSUB; ++sub) {
            s[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s[sub] = mfma_16x16x32_t<F16>(ka[sub][ks], qb[ks], s[sub]);
        }
        if (more) load_k(k0 + STEP);
        float mloc = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < KSUB; ++sub) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = k0 + 16 * sub + 4 * g + i;
                const float v = key < k_end ? s[sub][i] * scale_log2 : -INFINITY;
                s[sub][i] = v;
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
        for (int sub = 0; sub < KSUB; ++sub) {
            u32x2 pb;
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(s[sub][i] - m_run);
                l_run += p[i];
            }
            pb.x = pack2_t<F16>(p[0], p[1]);
            pb.y = pack2_t<F16>(p[2], p[3]);
            // V^T operands: M-tile (sl, t): row n <-> head dim 128 sl + 8 n + t,
            // slot j <-> key 4g + j.
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const uint32_t sel = (t & 1) ? kSelHiHalves : kSelLoHalves;
                    const int wd = t >> 1;
                    u32x2 a;
                    a.x = perm(vr[sub][sl][1][wd], vr[sub][sl][0][wd], sel);
                    a.y = perm(vr[sub][sl][3][wd], vr[sub][sl][2][wd], sel);
                    o[sl * 8 + t] = mfma_16x16x16_t<F16>(a, pb, o[sl * 8 + t]);
                }
            }
        }
        if (more) load_v(k0 + STEP);
    }

    // ---- merge the waves of this workgroup through LDS ------------------------
    const float l_tot = sum_over_groups(l_run);
    if (g == 0) { sm_m[w][n] = m_run; sm_l[w][n] = l_tot; }
    // accumulator element i of M-tile (sl, t) is head dim 128 sl + 32 g + 8 i + t
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float* dst = &sm_o[w][n][128 * sl + 32 * g + 8 * i];
            *(f32x4*)dst = f32x4{o[sl * 8 + 0][i], o[sl * 8 + 1][i], o[sl * 8 + 2][i], o[sl * 8 + 3][i]};
            *(f32x4*)(dst + 4) = f32x4{o[sl * 8 + 4][i], o[sl * 8 + 5][i], o[sl * 8 + 6][i], o[sl * 8 + 7][i]};
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * (D / 4); idx += NW * 64) {
        const int hn = idx / (D / 4);
        const int d4 = (idx % (D / 4)) * 4;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][hn]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = sm_m[ww][hn];
            const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            acc += *(const f32x4*)&sm_o[ww][hn][d4] * f;
            lsum += sm_l[ww][hn] * f;
        }
        const size_t prow = ((size_t)b * Hq + hk * G + hn) * n_split + s_idx;
        *(f32x4*)(part_o + prow * D + d4) = acc;
        if (d4 == 0) { part_ml[2 * prow] = M; part_ml[2 * prow + 1] = lsum; }
    }
}

// ---------------------------------------------------------------------------
// LSE merge: out[b,h] = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// lse = M ln2 + ln(sum).  Splits are visited in index order.  One block per
// (head, sequence); DV/4 threads with four head dims each.  Output fp32, or
// 16-bit (fp16 if OUT_F16, else bf16).
// ---------------------------------------------------------------------------
template <int DV, bool OUT_F32, bool OUT_F16>
__global__ __launch_bounds__(DV / 4) void lse_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           const int32_t* __restrict__ seq_lens, void* __restrict__ Out,
                                                           float* __restrict__ Lse, int H, int max_len, int chunk,
                                                           int n_split) {
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int d4 = threadIdx.x * 4;
    // seq_lens null: all n_split partials are present (some may be empty:
    // m = -inf, l = 0, O = 0, which contribute nothing)
    int ns = n_split;
    if (seq_lens != nullptr) {
        const int L = min(max(seq_lens[b], 0), max_len);
        ns = L > 0 ? (L + chunk - 1) / chunk : 0;
    }
    const size_t row = (size_t)b * H + h;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float M = -INFINITY, lsum = 0.f;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[2 * (row * n_split + s)]);
    for (int s = 0; s < ns; ++s) {
        const size_t pr = row * n_split + s;
        const float ms = part_ml[2 * pr];
        const float f = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
        lsum += part_ml[2 * pr + 1] * f;
        acc += *(const f32x4*)(part_o + pr * DV + d4) * f;
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    acc *= inv;
    if constexpr (OUT_F32) {
        *(f32x4*)((float*)Out + row * DV + d4) = acc;
    } else {
        u32x2 pk;
        pk.x = pack2_t<OUT_F16>(acc.x, acc.y);
        pk.y = pack2_t<OUT_F16>(acc.z, acc.w);
        *(u32x2*)((bf16*)Out + row * DV + d4) = pk;
    }
    if (Lse != nullptr && threadIdx.x == 0) Lse[row] = lsum > 0.f ? M * kLn2 + __logf(lsum) : -INFINITY;
}

hipError_t merge_launch(const float* part_o, const float* part_ml, const int32_t* seq_lens, void* out, float* lse,
                        int B, int H, int max_len, int D, int chunk, int n_split, bool out_f32, bool out_f16,
                        hipStream_t stream) {
    const dim3 grid(H, B);
#define MQA_MERGE_ONE(DV, F32, F16)                                                                        \
    hipLaunchKernelGGL((lse_merge_kernel<DV, F32, F16>), grid, dim3(DV / 4), 0, stream, part_o, part_ml,   \
                       seq_lens, out, lse, H, max_len, chunk, n_split)
#define MQA_MERGE(DV)                                                                                      \
    do {                                                                                                    \
        if (out_f32) MQA_MERGE_ONE(DV, true, false);                                                        \
        else if (out_f16) MQA_MERGE_ONE(DV, false, true);                                                   \
        else MQA_MERGE_ONE(DV, false, false);                                                               \
    } while (0)
    if (D == 512) MQA_MERGE(512);
    else if (D == 128) MQA_MERGE(128);
    else return hipErrorInvalidValue;
#undef MQA_MERGE
#undef MQA_MERGE_ONE
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan: chunk = cache rows per workgroup.  About 1024 workgroups of the
// longest sequence in total (fewer, longer chunks measured faster than more
// splits: each workgroup pays a load latency before its first step and a
// partial write), never under min_chunk rows.
// ---------------------------------------------------------------------------
// 64-bit throughout: the planners also answer workspace queries for sizes
// the launch itself would reject.
static long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

DecodePlan decode_plan(int B, int Hkv, int max_len, int head_dim) {
    const long long units = (long long)B * Hkv;
    const long long step = head_dim == 512 ? 4 * 16 : 4 * 64;      // NW * STEP
    const long long min_chunk = head_dim == 512 ? 2048 : 1024;
    const long long target_wgs = 1024;
    const long long want = ((long long)max_len * units + target_wgs - 1) / target_wgs;
    long long chunk = want > max_len ? (long long)max_len : want;
    if (chunk < min_chunk) chunk = min_chunk;
    chunk = round_up(chunk, step);
    long long n_split = ((long long)max_len + chunk - 1) / chunk;
    if (n_split < 1) n_split = 1;
    DecodePlan p;
    p.chunk = (int)(chunk > 0x7FFFFFC0LL ? 0x7FFFFFC0LL : chunk);
    p.n_split = (int)n_split;
    return p;
}

// Workgroups of one decode kernel that the device holds at once (queried
// once per kernel); 0 if the query fails.
template <int D, int KSUB, bool F16>
static long resident_wgs() {
    static const long n = [] {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<D, KSUB, 4, F16>, 256, 0) !=
                hipSuccess)
            return 0L;
        return (long)cus * per_cu;
    }();
    return n;
}

hipError_t decode_launch(const DecodeArgs& a) {
    const float sl2 = a.scale * kLog2e;
    const dim3 grid(a.plan.n_split, a.Hkv, a.B);
    const long wgs = (long)a.plan.n_split * a.Hkv * a.B;
#define MQA_DECODE(D, KSUB, F16)                                                                              \
    hipLaunchKernelGGL((decode_split_kernel<D, KSUB, 4, F16>), grid, dim3(256), 0, a.stream, (const bf16*)a.q,    \
                       (const bf16*)a.k, (const bf16*)a.v, a.seq_lens, a.part_o, a.part_ml, a.Hq, a.Hkv, a.max_len, \
                       a.G, a.plan.chunk, a.plan.n_split, sl2, (int)(wgs > resident_wgs<D, KSUB, F16>()))
    if (a.D == 512) {
        if (a.f16) MQA_DECODE(512, 1, true); else MQA_DECODE(512, 1, false);
    } else if (a.D == 128) {
        if (a.f16) MQA_DECODE(128, 4, true); else MQA_DECODE(128, 4, false);
    } else {
        return hipErrorInvalidValue;
    }
#undef MQA_DECODE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return merge_launch(a.part_o, a.part_ml, a.seq_lens, a.out, a.lse, a.B, a.Hq, a.max_len, a.D, a.plan.chunk,
                        a.plan.n_split, a.out_f32, a.f16, a.stream);
}

}  // namespace mqa
