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
//   * one workgroup (4 waves, one per SIMD) = one (sequence, chunk of rows)
//     and all (up to 128) heads;
//   * 32-row tiles are copied global -> LDS with asynchronous direct-to-LDS
//     loads (non-temporal: each cached row is read once), three stages deep
//     (two tiles in flight);
//   * scores: wave w computes S^T = KV q_abs^T for heads 32w..32w+31 on
//     v_mfma_f32_32x32x16_bf16 (or _f16; 36 contraction steps over the 576-wide
//     row), then the online softmax of those heads;
//   * P (bf16) of every head goes to LDS, and each wave accumulates
//     O^T += V^T P^T for ITS quarter of the 512 value dims and all heads:
//     every V^T operand then feeds four MFMAs, so LDS traffic per MFMA is a
//     quarter of a full-width split.  V^T operands come straight from the
//     row-major latent tile through transposing LDS reads;
//   * partials per (head, split) are merged by the shared log-sum-exp kernel.
// Sparse variant (top-k attention over the same cache, makesence §5.1): the
// rows of sequence b are kv[b, indices[b, j]] instead of kv[b, 0 .. L-1];
// each workgroup stages its chunk of the index list in LDS, every copy
// fetches the listed row (the direct-to-LDS copy takes any per-lane source
// address), and list entries outside [0, max_len) are masked.
// F16: fp16 queries and cache (the _f16 MFMAs, P rounded to fp16); else bf16.
#include "common.hpp"
#include "layout.hpp"
#include "kernels.hpp"

namespace mqa {

typedef float f32x2 __attribute__((ext_vector_type(2)));

namespace {
constexpr int kDK = 576;    // key width: latent + RoPE part
constexpr int kDC = 512;    // latent width (= value width)
constexpr int kDR = 64;     // RoPE part
constexpr int kKT = 32;     // cache rows per tile
constexpr int kNW = 4;      // waves per workgroup
constexpr int kHW = 32;     // heads per wave (scores and softmax)
constexpr int kHMAX = kNW * kHW;                                 // 128
constexpr int kDW = kDC / kNW;                                   // value dims per wave (128)
constexpr int kNS = 3;                                           // tile stages
constexpr int kLatRowB = layout::padded_row_bytes(2 * kDC);      // 1040
constexpr int kLatB = kKT * kLatRowB;                            // 33280
constexpr int kRopeB = kKT * kDR * 2;                            // 4096
constexpr int kStageB = kLatB + kRopeB;                          // 37376
constexpr int kPB = kHMAX * kKT * 2;                             // P tile: 8192
constexpr int kLdsB = kNS * kStageB + 2 * kPB + 2 * kHMAX * 4;
constexpr int kMaxSparseChunk = 2048;                            // list entries staged per workgroup
}  // namespace

// SPARSE = false: sequence b's rows are 0 .. seq_lens[b]-1 (indices unused).
// SPARSE = true:  its rows are indices[b, 0 .. topk-1] (seq_lens unused).
template <bool SPARSE, bool F16, int NT>
__global__ __launch_bounds__(kNW * 64, 1) void mla_decode_kernel(
    const bf16* __restrict__ Qa, const bf16* __restrict__ KV, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ indices, float* __restrict__ part_o, float* __restrict__ part_ml, int H,
    int max_len, int topk, int chunk, int n_split, float scale_log2) {
    constexpr int KS = kDK / 16;         // 36 score steps
    constexpr int KS_LAT = kDC / 16;     // 32 of them over the latent
    constexpr int MT = kDW / 32;         // 4 O^T M-tiles (value dims) per wave
    static_assert(NT >= 1 && NT <= kNW, "32-head blocks: 1 .. 4");
    constexpr int PF = 4;                // operand read-ahead

    __shared__ __attribute__((aligned(16))) char smem[kLdsB];
    __shared__ int sidx[SPARSE ? kMaxSparseChunk : 1];          // this chunk's rows (-1: skipped)
    char* const pbuf = smem + kNS * kStageB;                    // [2][kPB]
    float* const alpha_buf = (float*)(pbuf + 2 * kPB);          // [2][kHMAX]

    // Workgroups are dealt to the XCDs round-robin by flat index; when the
    // batch splits evenly over the XCDs, all splits of one sequence go to
    // one XCD, so its q_abs rows are fetched once into that XCD's L2.
    int s_idx = blockIdx.x, b = blockIdx.y;
    if (gridDim.y % kNumXcd == 0) {
        const int f = (int)(blockIdx.x + gridDim.x * blockIdx.y);
        const int x = f % kNumXcd, slot = f / kNumXcd;
        b = (slot / (int)gridDim.x) * kNumXcd + x;
        s_idx = slot % (int)gridDim.x;
    }
    // positions begin .. end-1 of the row list (cache rows, or list entries)
    const int L = SPARSE ? topk : min(max(seq_lens[b], 0), max_len);
    const int begin = s_idx * chunk;
    if (begin >= L) return;
    const int end = min(begin + chunk, L);
    const int n_tiles = (end - begin + kKT - 1) / kKT;
    if constexpr (SPARSE) {
        const int32_t* ib = indices + (size_t)b * topk + begin;
        for (int r = (int)threadIdx.x; r < end - begin; r += kNW * 64) {
            const int v = ib[r];
            sidx[r] = (v >= 0 && v < max_len) ? v : -1;
        }
        __syncthreads();
    }
    // cache row behind list position pos (begin <= pos < end); skipped
    // entries read row 0 and are masked
    auto cache_row = [&](int pos) -> int {
        if constexpr (SPARSE) {
            const int v = sidx[pos - begin];
            return v < 0 ? 0 : v;
        } else {
            return pos;
        }
    };

    const int lane = lane_id();
    const int w = wave_id();
    const int h2 = lane >> 5;
    const int n = lane & 31;
    const int head = kHW * w + n;                // head whose scores this lane holds
    const bool head_ok = head < H;
    // NT blocks of 32 heads (H <= 32 NT): waves 0 .. NT-1 compute the scores
    // and softmax of one block each; the others only copy and accumulate
    // O^T, so a small H does not pay for 128 heads' MFMAs
    const bool scorer = NT == kNW || w < NT;

    // q_abs^T operands: lane half h2 holds dims 16ks + 8h2 .. +7 of `head`
    bf16x8 qb[KS];
    {
        const bf16* qrow = Qa + ((size_t)b * H + (head_ok ? head : 0)) * kDK;
        const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = ldg16(qrow + 16 * ks + 8 * h2);
            qb[ks] = __builtin_bit_cast(bf16x8, head_ok ? v : zero);
        }
    }

    const bf16* KVb = KV + (size_t)b * max_len * kDK;
    const uint32_t lds_base = lds_addr(smem);
    const uint32_t lane16 = (uint32_t)lane * 16u;
    // One tile = 32 latent rows (one 1 KB copy each, padded positions) + the
    // 32 RoPE parts (4 copies, swizzled through the per-lane source offset):
    // 9 copies per wave.  Rows past the chunk end re-read the last row and
    // are masked.
    constexpr int kCopiesPerWave = (kKT + kRopeB / 1024) / kNW;
    static_assert(kCopiesPerWave * kNW == kKT + kRopeB / 1024, "copies must split evenly over the waves");
    // copy i (0 .. 8) of this wave for tile `tile`
    auto issue_one = [&](int tile, int i) {
        const uint32_t st = lds_base + (uint32_t)((tile % kNS) * kStageB);
        const int row0 = begin + tile * kKT;
        if (i < kKT / kNW) {
            const int u = i * kNW + w;               // wave-uniform latent row
            const int key = cache_row(min(row0 + u, end - 1));
            const uint32_t dst = st + (uint32_t)(layout::mla_lat_pos(u) * kLatRowB);
            if constexpr (SPARSE) copy16_to_lds_async_stream(KVb, (uint32_t)key * (kDK * 2u) + lane16, dst);
            else copy16_to_lds_async_stream(KVb + (size_t)key * kDK, lane16, dst);
        } else {
            const int r = 8 * w + (lane >> 3);       // RoPE row of this lane
            const int c = (lane & 7) ^ layout::mla_rope_swz(r);
            const int key = cache_row(min(row0 + r, end - 1));
            copy16_to_lds_async_stream(KVb, (uint32_t)key * (kDK * 2u) + (uint32_t)(kDC * 2 + c * 16), st + (uint32_t)(kLatB + w * 1024));
        }
    };
    auto issue = [&](int tile) {
#pragma unroll
        for (int i = 0; i < kCopiesPerWave; ++i) issue_one(tile, i);
    };

    // score operand offsets (bytes within a stage)
    const uint32_t lat_off = (uint32_t)(layout::mla_lat_pos(n) * kLatRowB + h2 * 16);
    uint32_t rope_off[KS - KS_LAT];
#pragma unroll
    for (int j = 0; j < KS - KS_LAT; ++j)
        rope_off[j] = (uint32_t)(kLatB + n * 128 + (((2 * j + h2) ^ layout::mla_rope_swz(n)) * 16));
    // A read pattern's per-lane base within the current stage, held in one
    // VGPR the compiler cannot split again: left to itself it keeps one
    // loop-invariant offset per read and adds the stage offset to each of
    // them every tile (two VALU per read); pinned, each read adds only an
    // immediate offset
    auto pinned = [&](const char* p) -> const char* {
        uint32_t off = (uint32_t)(p - smem);
        asm volatile("" : "+v"(off));
        return smem + off;
    };
    // klat = pinned(stage + lat_off)
    auto kread = [&](const char* klat, const char* st, int ks) {
        if (ks < KS_LAT) return *(const bf16x8*)(klat + ks * 32);
        return *(const bf16x8*)(st + rope_off[ks - KS_LAT]);
    };
    // transposing V^T reads: 16-lane group q = lane / 16, lane j = 4s + a in
    // it reads latent row 16kp + 8h2 + 4r + s, value dims 128w + 32mt +
    // 16(q%2) + 4a .. +3; the result is the A operand for value dims
    // 128w + 32mt + (lane % 32), keys 16kp + 8h2 .. +7 (r = 0, 1).
    const int tj = lane & 15;
    const uint32_t tr_off = (uint32_t)((8 * h2 + 2 * (tj >> 2)) * kLatRowB +
                                       2 * (kDW * w + 16 * ((lane >> 4) & 1) + 4 * (tj & 3)));
    // vb = pinned(stage + tr_off)
    auto vread = [&](const char* vb, int kp, int mt) {
        const char* p = vb + kp * 16 * kLatRowB + mt * 64;
        const s16x4 lo = lds_read_tr16(p);
        const s16x4 hi = lds_read_tr16(p + kLatRowB);
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    };

    f32x16 o[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[mt][nt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // ---- scores of one tile: S^T = KV q_abs^T (heads 32w + n, keys
    // 8(i/4) + 4h2 + i%4) ------------------------------------------------------
    // between(ks) runs before step ks's MFMA (work spread over the phase)
    auto scores = [&](const char* st, auto&& between) {
        f32x16 sc = f32x16{};
        const char* klat = pinned(st + lat_off);
        bf16x8 abuf[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) abuf[j] = kread(klat, st, j);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            between(ks);
            const bf16x8 a = abuf[ks % PF];
            if (ks + PF < KS) abuf[ks % PF] = kread(klat, st, ks + PF);
            sc = mfma_32x32x16_t<F16>(a, qb[ks], sc);
        }
        sched_reads_ahead<PF, KS - PF>();
        return sc;
    };
    auto nothing = [](int) {};

    // ---- online softmax, in three pieces so that it can sit between MFMAs --
    // (1) mask, row max, lazy rescale: returns the exponent reference.  The
    // scale is > 0, so the row max is taken on the raw scores and the scale
    // folds into the exponent: p = 2^(s * c - m).  A tile past the chunk end
    // is all masked: it changes nothing and writes P = 0.
    float alpha_t = 1.f;
    auto sm_max = [&](f32x16& sc, int tile) {
        const int row0 = begin + tile * kKT;
        if constexpr (SPARSE) {
            // one validity bit per list entry of the tile (lane n: entry n)
            const bool ok = row0 + n < end && sidx[min(row0 + n, end - 1) - begin] >= 0;
            const uint32_t vm = (uint32_t)__ballot(ok);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (!((vm >> (8 * (i >> 2) + 4 * h2 + (i & 3))) & 1u)) sc[i] = -INFINITY;
        } else if (row0 + kKT > end) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = row0 + 8 * (i >> 2) + 4 * h2 + (i & 3);
                if (key >= end) sc[i] = -INFINITY;
            }
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) mloc = max3f(mloc, sc[2 * i], sc[2 * i + 1]);
        const float mx = max_over_halves(mloc) * scale_log2;
        alpha_t = 1.f;
        if (mx > m_run + kRescaleSlack) {
            const float mnew = fmaxf(m_run, mx);
            alpha_t = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - mnew);
            m_run = mnew;
            l_run *= alpha_t;
        }
    };
    // (2) exponentials of accumulators 4c .. 4c+3, packed, to P(tile) in LDS.
    // A sparse chunk can start with tiles of skipped entries only: then
    // m_run is still -inf and every p must be 0 (2^(-inf - 0)).
    auto sm_exp = [&](f32x16& sc, int tile, int c) {
        const float m_use = (SPARSE && m_run == -INFINITY) ? 0.f : m_run;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sc[4 * c + i], scale_log2, -m_use));
        u32x2 pk;
        pk.x = pack2_t<F16>(p[0], p[1]);
        pk.y = pack2_t<F16>(p[2], p[3]);
        // the row sum takes the packed 16-bit probabilities (the values the
        // P.V MFMAs use), a pair per v_dot2c: half the VALU of adding the
        // fp32 ones (1.8 % faster)
        l_run = add_pair_t<F16>(pk.x, l_run);
        l_run = add_pair_t<F16>(pk.y, l_run);
        char* pl = pbuf + (tile & 1) * kPB + head * 64 + 8 * h2;
        *(u32x2*)(pl + ((c ^ layout::ptile_swz(head)) * 16)) = pk;
    };
    // (3) the per-head rescale factor of the tile
    auto sm_alpha = [&](int tile) {
        if (h2 == 0) alpha_buf[(tile & 1) * kHMAX + head] = alpha_t;
    };

    // ---- O^T += V^T P^T for value dims 128w .. 128w+127, all heads ------------
    // 8 steps (kp, mt), each one V^T operand x 4 P^T operands; between(stp)
    // runs after step stp's MFMAs (work placed between them).  The MFMAs are
    // opaque to the scheduler, so the software pipeline is pinned with
    // scheduling fences: V^T reads run two steps ahead and the P^T operands
    // of kp = 1 are read during kp = 0.
    auto pv_tile = [&](int it, auto&& between) {
        const char* st = smem + (it % kNS) * kStageB;
        const char* vb = pinned(st + tr_off);
        const char* pl = pbuf + (it & 1) * kPB;
        auto pread = [&](int kp, int nt) {
            const int hh = 32 * nt + n;
            return *(const bf16x8*)(pl + hh * 64 + (((2 * kp + h2) ^ layout::ptile_swz(hh)) * 16));
        };
        constexpr int NSTEP = 2 * MT;
        bf16x8 pb[2][NT];
        bf16x8 va[3];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pb[0][nt] = pread(0, nt);
        va[0] = vread(vb, 0, 0);
        va[1] = vread(vb, 0, 1);
        const float* al = alpha_buf + (it & 1) * kHMAX;
        float a4[NT];
        bool need = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            a4[nt] = al[32 * nt + n];
            need |= a4[nt] != 1.f;
        }
        between(-1);
        if (__any(need)) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) scale_acc(o[mt][nt], a4[nt]);
        }
#pragma unroll
        for (int stp = 0; stp < NSTEP; ++stp) {
            if (stp + 2 < NSTEP) va[(stp + 2) % 3] = vread(vb, (stp + 2) / MT, (stp + 2) % MT);
            if (stp == 1) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) pb[1][nt] = pread(1, nt);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) mfma_32x32x16_acc_t<F16>(va[stp % 3], pb[stp / MT][nt], o[stp % MT][nt]);
            between(stp);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Tile t lives in stage t % 3.
    issue(0);
    if (n_tiles > 1) issue(1);
    if (n_tiles > 1) wait_vmcnt<kCopiesPerWave>(); else wait_vmcnt<0>();
    __syncthreads();
    if constexpr (!SPARSE) {
        // Iteration t (entered with tile t+1 landed and P(t) in LDS): copies
        // of tile t+2 (into the stage of tile t-1, whose P.V every wave
        // finished before the barrier), the scores of tile t+1, then
        // P(t).V(t) with the softmax of tile t+1 and the writes of P(t+1)
        // between its MFMAs, and a barrier once tile t+2 has landed.  On the
        // last iteration the scores of the (absent) next tile read a stale
        // stage and are masked away.
        if (scorer) {
            f32x16 s0 = scores(smem, nothing);
            sm_max(s0, 0);
#pragma unroll
            for (int c = 0; c < 4; ++c) sm_exp(s0, 0, c);
            sm_alpha(0);
        }
        wait_vmcnt<0>();
        __syncthreads();
        for (int it = 0; it < n_tiles; ++it) {
            // copies of tile t+2 spread over the score MFMAs, one every
            // four steps.  They are issued on every iteration, also past the
            // last tile (their rows clamp to the chunk's last row and land in
            // a stage nothing reads again): a branch here would split the
            // MFMA chain into short scheduling regions, and the K operand
            // reads would then go out only one or two MFMAs ahead of use
            // (3 % slower)
            f32x16 sn = f32x16{};
            if (scorer) {
                sn = scores(smem + ((it + 1) % kNS) * kStageB, [&](int ks) {
                    if (ks % 4 == 0 && ks / 4 < kCopiesPerWave) issue_one(it + 2, ks / 4);
                });
            } else {
#pragma unroll
                for (int i = 0; i < kCopiesPerWave; ++i) issue_one(it + 2, i);
            }
            // P(t).V(t) as in pv_tile (written out: the register allocator
            // fits this loop without spills only in this form), with the
            // softmax of the next tile: max after step 1, exponentials and P
            // writes over steps 2..5, the rescale factor at 6
            {
                const char* st = smem + (it % kNS) * kStageB;
                const char* vb = pinned(st + tr_off);
                const char* pl = pbuf + (it & 1) * kPB;
                auto pread = [&](int kp, int nt) {
                    const int hh = 32 * nt + n;
                    return *(const bf16x8*)(pl + hh * 64 + (((2 * kp + h2) ^ layout::ptile_swz(hh)) * 16));
                };
                constexpr int NSTEP = 2 * MT;
                bf16x8 pb[2][NT];
                bf16x8 va[3];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) pb[0][nt] = pread(0, nt);
                va[0] = vread(vb, 0, 0);
                va[1] = vread(vb, 0, 1);
                const float* al = alpha_buf + (it & 1) * kHMAX;
                float a4[NT];
                bool need = false;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    a4[nt] = al[32 * nt + n];
                    need |= a4[nt] != 1.f;
                }
                if (__any(need)) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) scale_acc(o[mt][nt], a4[nt]);
                }
#pragma unroll
                for (int stp = 0; stp < NSTEP; ++stp) {
                    if (stp + 2 < NSTEP) va[(stp + 2) % 3] = vread(vb, (stp + 2) / MT, (stp + 2) % MT);
                    if (stp == 1) {
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) pb[1][nt] = pread(1, nt);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) mfma_32x32x16_acc_t<F16>(va[stp % 3], pb[stp / MT][nt], o[stp % MT][nt]);
                    if (scorer) {
                        if (stp == 1) sm_max(sn, it + 1);
                        if (stp >= 2 && stp < 6) sm_exp(sn, it + 1, stp - 2);
                        if (stp == 6) sm_alpha(it + 1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            wait_vmcnt<0>();
            __syncthreads();
        }
    } else {
        // Sparse chunks are short (a few tiles), so they keep two tiles in
        // flight instead: iteration t computes the scores and softmax of t,
        // barrier, then copies of tile t+2 and P(t).V(t).
        for (int it = 0; it < n_tiles; ++it) {
            if (scorer) {
                f32x16 sc = scores(smem + (it % kNS) * kStageB, nothing);
                sm_max(sc, it);
#pragma unroll
                for (int c = 0; c < 4; ++c) sm_exp(sc, it, c);
                sm_alpha(it);
            }
            // tile it+1 has landed (nothing later was issued yet)
            wait_vmcnt<0>();
            __syncthreads();
            pv_tile(it, [&](int stp) {
                if (stp == -1 && it + 2 < n_tiles) issue(it + 2);
            });
        }
    }

    // ---- partials: unnormalised O^T slices, (m, l) per head ---------------------
    mfma_acc_drain();
    const float l_tot = sum_over_halves(l_run);
    // (m, l) per head, split-major: ((b * n_split + s_idx) * H + head)
    if (head_ok && h2 == 0) {
        const size_t prow = ((size_t)b * n_split + s_idx) * H + head;
        *(f32x2*)(part_ml + 2 * prow) = f32x2{m_run, l_tot};
    }
    // O^T partials chunk-major: the 8 value dims 8c .. 8c+7 of head h lie at
    // ((b * n_split + s_idx) * 64 + c) * H + h (8 floats each), so each store
    // instruction writes 32 heads' chunk c, 1 KB contiguous (stores of 32
    // bytes of each of 32 head rows were 2 % slower)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int hh = 32 * nt + n;
        if (hh >= H) continue;
        float* dst = part_o + ((size_t)(b * n_split + s_idx) * (kDC / 8) + (kDW / 8) * w) * H * 8 + (size_t)hh * 8 + 4 * h2;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x16& acc = o[mt][nt];
                *(f32x4*)(dst + (size_t)(4 * mt + q) * H * 8) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
            }
    }
}

// ---------------------------------------------------------------------------
// Merge of the MLA split partials (the same arithmetic as the decode merge:
// splits summed in index order, weights 2^(m_s - M), one division), reading
// the chunk-major layout above: a workgroup takes 32 heads and 4 chunks (32
// value dims) of one sequence; lane (n, h2) of wave w sums head 32 hg + n,
// floats 4 h2 .. 4 h2 + 3 of chunk 4 cg + w, so every load instruction
// reads 1 KB contiguous; the results leave through LDS as row pieces.
// ---------------------------------------------------------------------------
template <bool OUT_F32, bool OUT_F16>
__global__ __launch_bounds__(256) void mla_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        const int32_t* __restrict__ seq_lens, void* __restrict__ Out,
                                                        float* __restrict__ Lse, int H, int max_len, int chunk,
                                                        int n_split) {
    constexpr int EB = OUT_F32 ? 4 : 2;              // output element bytes
    constexpr int TROW_B = 32 * EB + 16;             // LDS row: 32 dims + padding
    __shared__ __attribute__((aligned(16))) char tile[32 * TROW_B];
    const int cg = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, h2 = lane >> 5;
    const int h = 32 * hg + n;
    const bool h_ok = h < H;
    // seq_lens null: all n_split partials are present (some may be empty:
    // m = -inf, l = 0, O = 0, which contribute nothing)
    int ns = n_split;
    if (seq_lens != nullptr) {
        const int L = min(max(seq_lens[b], 0), max_len);
        ns = L > 0 ? (L + chunk - 1) / chunk : 0;
    }
    if (!h_ok) ns = 0;
    const size_t row = (size_t)b * H + (h_ok ? h : 0);
    // (m, l) of split s: ((b * n_split + s) * H + h), 32 heads' pairs contiguous
    const float* ml = part_ml + 2 * ((size_t)b * n_split * H + (h_ok ? h : 0));
    const size_t ml_stride = 2 * (size_t)H;
    const float* src = part_o + ((size_t)b * n_split * (kDC / 8) + 4 * cg + w) * H * 8 + (size_t)h * 8 + 4 * h2;
    const size_t split_stride = (size_t)(kDC / 8) * H * 8;
    // the first NC splits' (m, l) and partials are loaded once, all at once
    // (splits past this sequence's count are loaded while inside the
    // workspace and then ignored, never multiplied)
    constexpr int NC = 8;
    f32x2 mlc[NC];
    f32x4 pc[NC];
#pragma unroll
    for (int s = 0; s < NC; ++s) {
        const bool in = s < ns;
        mlc[s] = in ? *(const f32x2*)(ml + s * ml_stride) : f32x2{-INFINITY, 0.f};
        pc[s] = (s < n_split && h_ok) ? *(const f32x4*)(src + s * split_stride) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float M = -INFINITY, lsum = 0.f;
#pragma unroll
    for (int s = 0; s < NC; ++s) M = fmaxf(M, mlc[s].x);
    for (int s = NC; s < ns; ++s) M = fmaxf(M, ml[s * ml_stride]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NC; ++s) {
        if (s < ns) {
            const float f = mlc[s].x == -INFINITY ? 0.f : fast_exp2(mlc[s].x - M);
            lsum += mlc[s].y * f;
            acc += pc[s] * f;
        }
    }
    for (int s = NC; s < ns; ++s) {
        const f32x2 msl = *(const f32x2*)(ml + s * ml_stride);
        const float f = msl.x == -INFINITY ? 0.f : fast_exp2(msl.x - M);
        lsum += msl.y * f;
        acc += *(const f32x4*)(src + s * split_stride) * f;
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const f32x4 v = acc * inv;
    // dims of chunk 4 cg + w within this workgroup's 32: 8 w + 4 h2
    char* dst = tile + n * TROW_B + (8 * w + 4 * h2) * EB;
    if constexpr (OUT_F32) {
        *(f32x4*)dst = v;
    } else {
        u32x2 pk;
        pk.x = pack2_t<OUT_F16>(v.x, v.y);
        pk.y = pack2_t<OUT_F16>(v.z, v.w);
        *(u32x2*)dst = pk;
    }
    if (Lse != nullptr && cg == 0 && w == 0 && h2 == 0 && h_ok) Lse[row] = lsum > 0.f ? M * kLn2 + __logf(lsum) : -INFINITY;
    __syncthreads();
    // 32 row pieces of 32 * EB bytes, 16 bytes per thread
    constexpr int CPR = 32 * EB / 16;                // 16-byte chunks per row piece
    if ((int)threadIdx.x < 32 * CPR) {
        const int r = (int)threadIdx.x / CPR, q = (int)threadIdx.x % CPR;
        if (32 * hg + r < H) {
            char* out = (char*)Out + (((size_t)b * H + 32 * hg + r) * kDC + 32 * cg) * EB + 16 * q;
            *(u32x4*)out = *(const u32x4*)(tile + r * TROW_B + 16 * q);
        }
    }
}

// 64-bit arithmetic: the planners also answer workspace queries for sizes
// the launch itself would reject.
DecodePlan mla_plan(int B, int max_len) {
    // one workgroup per CU (LDS-bound): about 256 workgroups in total
    const long long target_wgs = 256;
    const long long splits = (target_wgs + B - 1) / B;
    long long chunk = ((long long)max_len + splits - 1) / splits;
    if (chunk < 512) chunk = 512;
    chunk = (chunk + kKT - 1) / kKT * kKT;
    long long n_split = ((long long)max_len + chunk - 1) / chunk;
    if (n_split < 1) n_split = 1;
    DecodePlan p;
    p.chunk = (int)chunk;
    p.n_split = (int)n_split;
    return p;
}

DecodePlan mla_sparse_plan(int B, int topk) {
    // about 256 workgroups; 128 .. kMaxSparseChunk list entries each
    const long long target_wgs = 256;
    const long long splits = (target_wgs + B - 1) / B;
    long long chunk = ((long long)topk + splits - 1) / splits;
    if (chunk < 128) chunk = 128;
    chunk = (chunk + kKT - 1) / kKT * kKT;
    if (chunk > kMaxSparseChunk) chunk = kMaxSparseChunk;
    long long n_split = ((long long)topk + chunk - 1) / chunk;
    if (n_split < 1) n_split = 1;
    DecodePlan p;
    p.chunk = (int)chunk;
    p.n_split = (int)n_split;
    return p;
}

template <bool SPARSE, bool F16, int NT>
static void mla_kernel_launch_nt(const MlaArgs& a) {
    const dim3 grid(a.plan.n_split, a.B);
    hipLaunchKernelGGL((mla_decode_kernel<SPARSE, F16, NT>), grid, dim3(kNW * 64), 0, a.stream, (const bf16*)a.q,
                       (const bf16*)a.kv, SPARSE ? (const int32_t*)nullptr : a.seq_lens,
                       SPARSE ? a.indices : (const int32_t*)nullptr, a.part_o, a.part_ml, a.H, a.max_len,
                       SPARSE ? a.topk : 0, a.plan.chunk, a.plan.n_split, a.scale * kLog2e);
}

// 32-head blocks: 1 for H <= 32, 2 for H <= 64, else 4
template <bool SPARSE, bool F16>
static void mla_kernel_launch(const MlaArgs& a) {
    if (a.H <= 32) mla_kernel_launch_nt<SPARSE, F16, 1>(a);
    else if (a.H <= 64) mla_kernel_launch_nt<SPARSE, F16, 2>(a);
    else mla_kernel_launch_nt<SPARSE, F16, 4>(a);
}

hipError_t mla_launch(const MlaArgs& a) {
    const bool sparse = a.indices != nullptr;
    if (sparse) {
        if (a.f16) mla_kernel_launch<true, true>(a); else mla_kernel_launch<true, false>(a);
    } else {
        if (a.f16) mla_kernel_launch<false, true>(a); else mla_kernel_launch<false, false>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // sparse: every split of every sequence wrote a partial (seq_lens = null)
    const dim3 grid(kDC / 32, (a.H + 31) / 32, a.B);
    const int32_t* sl = sparse ? nullptr : a.seq_lens;
#define MQA_MLA_MERGE(F32, F16)                                                                          \
    hipLaunchKernelGGL((mla_merge_kernel<F32, F16>), grid, dim3(256), 0, a.stream, a.part_o, a.part_ml, sl, \
                       a.out, a.lse, a.H, a.max_len, a.plan.chunk, a.plan.n_split)
    if (a.out_f32) MQA_MLA_MERGE(true, false);
    else if (a.f16) MQA_MLA_MERGE(false, true);
    else MQA_MLA_MERGE(false, false);
#undef MQA_MLA_MERGE
    return hipGetLastError();
}

}  // namespace mqa
