// Causal / full prefill attention for query heads sharing key/value heads.
//
// bf16 path (flash-style, one pass over K/V, scores never materialised --
// the tiling idea of "GQA和MLA详解" (lzwjava.github.io) §4 applied to the
// (T,T) score matrix as that page's §1 describes):
//   * one workgroup = one (batch, KV head) and a block of query tokens for
//     ALL G query heads of that KV head, so every K/V tile staged in LDS is
//     reused by the whole head group (the MQA/GQA saving; heads are indexed,
//     never copied -- lzwjava §2);
//   * per wave: 16*NT query rows; S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_f32_16x16x32_bf16 with fp32 accumulation; Q stays in VGPRs,
//     the O^T accumulator for the full head dim stays in (A)VGPRs;
//   * online softmax per row in registers (exp2 domain, lazy rescale);
//   * K tiles and pre-transposed V tiles are copied global->LDS with
//     asynchronous direct-to-LDS loads, double buffered;
//   * causal: key tiles past the block's last token are never visited, the
//     diagonal tile is masked per element, and the heaviest blocks start
//     first.
// fp32 path: a plain fp32 VALU kernel (no reduced-precision operands).
#include "common.hpp"
#include "layout.hpp"
#include "kernels.hpp"

namespace mqa {

// ---------------------------------------------------------------------------
// V [B*Hkv, T, D] -> Vt tiles [B*Hkv, n_tiles, D rows of KT keys] in exactly
// the swizzled order the prefill kernel keeps in LDS (zero past T).
// ---------------------------------------------------------------------------
template <int D, int KT>
__global__ __launch_bounds__(256) void vt_pack_kernel(const bf16* __restrict__ V, bf16* __restrict__ Vt,
                                                      int T, int n_tiles) {
    constexpr int RL = KT / 8;           // 16-byte chunks per V^T row
    constexpr int NB = RL * (D / 8);     // 8x8 blocks per tile
    const int tile = blockIdx.x;
    const size_t bh = blockIdx.y;
    const bf16* src = V + bh * (size_t)T * D;
    bf16* dst = Vt + (bh * n_tiles + tile) * (size_t)(KT * D);
    for (int blk = threadIdx.x; blk < NB; blk += 256) {
        const int kb = blk % RL;
        const int db = blk / RL;
        u32x4 r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = tile * KT + kb * 8 + j;
            if (key < T) r[j] = ldg16(src + (size_t)key * D + db * 8);
            else r[j] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int d = db * 8 + t;
            const uint32_t sel = (t & 1) ? kSelHiHalves : kSelLoHalves;
            const int w = t >> 1;
            u32x4 o;
            o.x = perm(r[1][w], r[0][w], sel);
            o.y = perm(r[3][w], r[2][w], sel);
            o.z = perm(r[5][w], r[4][w], sel);
            o.w = perm(r[7][w], r[6][w], sel);
            const int pos = kb ^ layout::vswz(d, RL);
            *(u32x4*)(dst + (size_t)(d * RL + pos) * 8) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 flash prefill.
//   D      head dim (128 or 512)          NT  16-row N-tiles per row block
//   NW     waves per workgroup            KT  keys per tile (multiple of 32)
//   SPLIT  waves sharing one row block; each owns D/SPLIT head dims of both
//          the Q.K^T contraction (fp32 partial scores are summed through
//          LDS) and of the output accumulator, which halves the registers a
//          wave needs at D = 512 without changing the LDS traffic per row.
// Rows of a workgroup: r = 0 .. (NW/SPLIT)*16*NT-1, head = r % G,
// token = t0 + r / G.
// ---------------------------------------------------------------------------
template <int D, int NT, int NW, int KT, int SPLIT, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ Vt,
    void* __restrict__ Out, float* __restrict__ Lse, int Hq, int Hkv, int T, int G,
    int tok_per_wg, int n_tok_blocks, int n_kv_tiles, float scale_log2) {
    constexpr int RW = 16 * NT;
    constexpr int DS = D / SPLIT;         // head dims owned by one wave
    constexpr int KS = DS / 32;           // QK^T contraction steps per wave
    constexpr int MT_S = KT / 16;         // S^T M-tiles (keys)
    constexpr int MT_O = DS / 16;         // O^T M-tiles (head dims)
    constexpr int KS_P = KT / 32;         // P.V contraction steps
    constexpr int RL = KT / 8;            // chunks per V^T row
    constexpr int TILE = KT * D;          // elements per K tile (and per V^T tile)
    constexpr int CHUNKS = TILE / 8;
    constexpr int LOADS = CHUNKS / (NW * 64);
    constexpr int ROW_CHUNKS = D / 8;
    constexpr int NSX = MT_S * NT;        // f32x4 partial-score registers per lane
    static_assert(CHUNKS % (NW * 64) == 0, "tile must split evenly over the waves");
    static_assert(DS % 128 == 0 || DS == D, "split head dim");
    static_assert(KT % 32 == 0 && (RL == 4 || RL == 8), "key tile");
    static_assert(SPLIT == 1 || NW * 64 * NSX * 16 <= TILE * 2, "score exchange must fit in a K tile");

    __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * TILE];

    const int lane = lane_id();
    const int w = wave_id();
    const int g = lane >> 4;
    const int n = lane & 15;
    const int rb = w / SPLIT;             // row block of this wave
    const int hd = w % SPLIT;             // head-dim part of this wave
    const int dbase = hd * DS;
    const int tb = CAUSAL ? (n_tok_blocks - 1 - (int)blockIdx.x) : (int)blockIdx.x;
    const int hk = blockIdx.y;
    const int b = blockIdx.z;
    const int t0 = tb * tok_per_wg;
    const int rows_used = tok_per_wg * G;

    int row_tok[NT];
    int row_head[NT];
    bool row_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = rb * RW + 16 * nt + n;
        row_tok[nt] = t0 + r / G;
        row_head[nt] = hk * G + r % G;
        row_ok[nt] = (r < rows_used) && (row_tok[nt] < T);
    }

    // Q^T operands (B of S^T): lane group g holds head dims dbase + 32ks + 8g .. +7.
    bf16x8 qb[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const bf16* qrow = Q + (((size_t)b * Hq + row_head[nt]) * T + (row_ok[nt] ? row_tok[nt] : 0)) * D + dbase;
        const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = ldg16(qrow + 32 * ks + 8 * g);
            qb[nt][ks] = __builtin_bit_cast(bf16x8, row_ok[nt] ? v : zero);
        }
    }

    const size_t bh = (size_t)b * Hkv + hk;
    const bf16* Kbh = K + bh * (size_t)T * D;
    const bf16* Vtbh = Vt + bh * (size_t)n_kv_tiles * TILE;

    const int t_last = min(T, t0 + tok_per_wg) - 1;
    const int n_tiles = CAUSAL ? (t_last / KT + 1) : n_kv_tiles;

    auto issue = [&](int tile, int stage) {
        bf16* ks_lds = smem + stage * 2 * TILE;
        bf16* vs_lds = ks_lds + TILE;
        const bf16* Vtile = Vtbh + (size_t)tile * TILE;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int inst = i * NW + w;               // wave-uniform
            const int q = inst * 64 + lane;            // chunk index inside the tile
            const int kk = q / ROW_CHUNKS;
            const int pos = q % ROW_CHUNKS;
            const int c = pos ^ layout::kswz(kk);
            const int key = min(tile * KT + kk, T - 1);   // past T: any valid row, masked later
            copy16_to_lds_off(Kbh, (uint32_t)(key * D + c * 8) * 2u, ks_lds + inst * 64 * 8);
            copy16_to_lds_off(Vtile, (uint32_t)q * 16u, vs_lds + inst * 64 * 8);
        }
    };

    f32x4 o[MT_O][NT];
#pragma unroll
    for (int mt = 0; mt < MT_O; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[NT], l_run[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) { m_run[nt] = -INFINITY; l_run[nt] = 0.f; }

    issue(0, 0);
    for (int it = 0; it < n_tiles; ++it) {
        const int stage = it & 1;
        wait_vmcnt<0>();            // this wave's copies of tile `it` have landed
        __syncthreads();            // ... and everyone's; all waves are done with tile it-1
        if (it + 1 < n_tiles) issue(it + 1, stage ^ 1);
        bf16* ks_lds = smem + stage * 2 * TILE;
        const bf16* vs_lds = ks_lds + TILE;

        // ---- S^T = K Q^T (this wave's head dims) --------------------------
        f32x4 s[MT_S][NT];
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) s[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt) {
                const int kk = layout::st_row_key(mt, n);
                const int pos = (dbase / 8 + 4 * ks + g) ^ layout::kswz(kk);
                const bf16x8 a = *(const bf16x8*)(ks_lds + kk * D + pos * 8);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) s[mt][nt] = mfma_16x16x32(a, qb[nt][ks], s[mt][nt]);
            }
        }
        if constexpr (SPLIT == 2) {
            // Sum the two halves of the contraction: every wave parks its
            // partial scores in the (now idle) K tile and adds its partner's.
            f32x4* xs = (f32x4*)ks_lds;
            __syncthreads();
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) xs[(w * NSX + mt * NT + nt) * 64 + lane] = s[mt][nt];
            __syncthreads();
            const int pw = w ^ 1;
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const f32x4 other = xs[(pw * NSX + mt * NT + nt) * 64 + lane];
                    // fixed summation order (lower head dims first) in both waves
                    s[mt][nt] = hd == 0 ? s[mt][nt] + other : other + s[mt][nt];
                }
        }

        // ---- mask + online softmax ----------------------------------------
        const int j0 = it * KT;
        float mx[NT];
        bool need = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float mloc = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = j0 + layout::st_c_key(mt, g, i);
                    const bool vis = CAUSAL ? (key <= row_tok[nt]) : (key < T);
                    const float v = vis ? s[mt][nt][i] * scale_log2 : -INFINITY;
                    s[mt][nt][i] = v;
                    mloc = fmaxf(mloc, v);
                }
            }
            mx[nt] = max_over_groups(mloc);
            need |= mx[nt] > m_run[nt] + kRescaleSlack;
        }
        if (__any(need)) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float mnew = fmaxf(m_run[nt], mx[nt]);
                const float alpha = (m_run[nt] == -INFINITY) ? 0.f : fast_exp2(m_run[nt] - mnew);
                m_run[nt] = mnew;
                l_run[nt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT_O; ++mt) o[mt][nt] *= alpha;
            }
        }
        bf16x8 pb[NT][KS_P];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float lsum = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = fast_exp2(s[mt][nt][i] - m_run[nt]);
                    s[mt][nt][i] = p;
                    lsum += p;
                }
            }
            l_run[nt] += lsum;
#pragma unroll
            for (int kp = 0; kp < KS_P; ++kp) pb[nt][kp] = pack_bf16x8(s[2 * kp][nt], s[2 * kp + 1][nt]);
        }

        // ---- O^T += V^T P^T (this wave's head dims) ---------------------------
#pragma unroll
        for (int kp = 0; kp < KS_P; ++kp) {
#pragma unroll
            for (int mt = 0; mt < MT_O; ++mt) {
                const int d = dbase + layout::pv_row_d(mt, n);
                const int pos = (4 * kp + g) ^ layout::vswz(d, RL);
                const bf16x8 a = *(const bf16x8*)(vs_lds + (d * RL + pos) * 8);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) o[mt][nt] = mfma_16x16x32(a, pb[nt][kp], o[mt][nt]);
            }
        }
    }

    // ---- epilogue: normalise, store ------------------------------------------
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const float l = sum_over_groups(l_run[nt]);
        const float inv = 1.f / l;
        if (!row_ok[nt]) continue;
        const size_t row = ((size_t)b * Hq + row_head[nt]) * T + row_tok[nt];
#pragma unroll
        for (int bq = 0; bq < DS / 32; ++bq) {
            const f32x4 lo = o[2 * bq][nt] * inv;
            const f32x4 hi = o[2 * bq + 1][nt] * inv;
            const int d0 = dbase + 32 * bq + 8 * g;     // = dbase + pv_c_d(2bq, g, 0)
            if constexpr (OUT_F32) {
                float* dst = (float*)Out + row * D + d0;
                *(f32x4*)dst = lo;
                *(f32x4*)(dst + 4) = hi;
            } else {
                bf16* dst = (bf16*)Out + row * D + d0;
                *(bf16x8*)dst = pack_bf16x8(lo, hi);
            }
        }
        if (Lse != nullptr && g == 0 && hd == 0) Lse[row] = m_run[nt] * kLn2 + __logf(l);
    }
}

// ---------------------------------------------------------------------------
// fp32 prefill: genuine fp32 end to end (fp32 FMA, fp32 exp2).  One wave
// handles four consecutive query tokens of one head; lanes split the head
// dim (E = D/64 consecutive elements per lane).  Online softmax per row.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void prefill_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                          const float* __restrict__ V, float* __restrict__ Out,
                                                          float* __restrict__ Lse, int Hq, int Hkv, int T, int G,
                                                          float scale_log2) {
    constexpr int E = D / 64;
    constexpr int RPW = 4;
    const int lane = lane_id();
    const int w = wave_id();
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int hk = h / G;
    const int tb = CAUSAL ? ((int)gridDim.x - 1 - (int)blockIdx.x) : (int)blockIdx.x;
    const int tbase = tb * (4 * RPW) + w * RPW;
    if (tbase >= T) return;

    const float* Kbh = K + ((size_t)b * Hkv + hk) * (size_t)T * D;
    const float* Vbh = V + ((size_t)b * Hkv + hk) * (size_t)T * D;
    float q[RPW][E], o[RPW][E], m[RPW], l[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int t = min(tbase + r, T - 1);
        const float* qrow = Q + (((size_t)b * Hq + h) * T + t) * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) { q[r][e] = qrow[e]; o[r][e] = 0.f; }
        m[r] = -INFINITY;
        l[r] = 0.f;
    }
    const int jmax = CAUSAL ? min(tbase + RPW - 1, T - 1) : T - 1;
    for (int j = 0; j <= jmax; ++j) {
        float kv[E], vv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) { kv[e] = Kbh[(size_t)j * D + lane * E + e]; vv[e] = Vbh[(size_t)j * D + lane * E + e]; }
        float dot[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) acc = fmaf(q[r][e], kv[e], acc);
            dot[r] = acc;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
            for (int r = 0; r < RPW; ++r) dot[r] += __shfl_xor(dot[r], off);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            if (CAUSAL && j > tbase + r) continue;
            const float sc = dot[r] * scale_log2;
            const float mnew = fmaxf(m[r], sc);
            const float alpha = fast_exp2(m[r] - mnew);
            const float p = fast_exp2(sc - mnew);
            l[r] = l[r] * alpha + p;
#pragma unroll
            for (int e = 0; e < E; ++e) o[r][e] = fmaf(p, vv[e], o[r][e] * alpha);
            m[r] = mnew;
        }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int t = tbase + r;
        if (t >= T) continue;
        const size_t row = ((size_t)b * Hq + h) * T + t;
        const float inv = 1.f / l[r];
#pragma unroll
        for (int e = 0; e < E; ++e) Out[row * D + lane * E + e] = o[r][e] * inv;
        if (Lse != nullptr && lane == 0) Lse[row] = m[r] * kLn2 + logf(l[r]);
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers (validated arguments only).
// ---------------------------------------------------------------------------
template <int D, int NT, int NW, int KT, int SPLIT>
static hipError_t launch_bf16(const PrefillArgs& a) {
    const int R = (NW / SPLIT) * 16 * NT;
    const int tok = R / a.G;
    const int n_tok_blocks = (a.T + tok - 1) / tok;
    const int n_kv_tiles = (a.T + KT - 1) / KT;
    bf16* vt = (bf16*)a.workspace;
    hipLaunchKernelGGL((vt_pack_kernel<D, KT>), dim3(n_kv_tiles, a.B * a.Hkv), dim3(256), 0, a.stream,
                       (const bf16*)a.v, vt, a.T, n_kv_tiles);
    const dim3 grid(n_tok_blocks, a.Hkv, a.B);
    const float sl2 = a.scale * kLog2e;
#define MQA_PREFILL_LAUNCH(C, F)                                                                      \
    hipLaunchKernelGGL((prefill_bf16_kernel<D, NT, NW, KT, SPLIT, C, F>), grid, dim3(NW * 64), 0, a.stream, \
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)vt, a.out, a.lse, a.Hq, a.Hkv, a.T, \
                       a.G, tok, n_tok_blocks, n_kv_tiles, sl2)
    if (a.causal) {
        if (a.out_f32) MQA_PREFILL_LAUNCH(true, true); else MQA_PREFILL_LAUNCH(true, false);
    } else {
        if (a.out_f32) MQA_PREFILL_LAUNCH(false, true); else MQA_PREFILL_LAUNCH(false, false);
    }
#undef MQA_PREFILL_LAUNCH
    return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(const PrefillArgs& a) {
    const int n_blocks = (a.T + 15) / 16;
    const dim3 grid(n_blocks, a.Hq, a.B);
    const float sl2 = a.scale * kLog2e;
    if (a.causal)
        hipLaunchKernelGGL((prefill_f32_kernel<D, true>), grid, dim3(256), 0, a.stream, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (float*)a.out, a.lse, a.Hq, a.Hkv, a.T, a.G, sl2);
    else
        hipLaunchKernelGGL((prefill_f32_kernel<D, false>), grid, dim3(256), 0, a.stream, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (float*)a.out, a.lse, a.Hq, a.Hkv, a.T, a.G, sl2);
    return hipGetLastError();
}

PrefillPlan prefill_plan(int head_dim, int in_bf16) {
    PrefillPlan p{};
    if (!in_bf16) { p.rows_per_wg = 1 << 30; p.kt = 0; return p; }
    if (head_dim == 512) { p.rows_per_wg = (8 / 2) * 16 * 2; p.kt = 32; }
    else if (head_dim == 128) { p.rows_per_wg = 4 * 16 * 2; p.kt = 32; }
    return p;
}

hipError_t prefill_launch(const PrefillArgs& a) {
    if (!a.in_bf16) {
        switch (a.D) {
            case 64: return launch_f32<64>(a);
            case 128: return launch_f32<128>(a);
            case 192: return launch_f32<192>(a);
            case 256: return launch_f32<256>(a);
            case 320: return launch_f32<320>(a);
            case 384: return launch_f32<384>(a);
            case 448: return launch_f32<448>(a);
            case 512: return launch_f32<512>(a);
            default: return hipErrorInvalidValue;
        }
    }
    if (a.D == 512) return launch_bf16<512, 2, 8, 32, 2>(a);
    if (a.D == 128) return launch_bf16<128, 2, 4, 32, 1>(a);
    return hipErrorInvalidValue;
}

}  // namespace mqa
